"""Python binding of the MLRA decode C ABI (argument marshalling only).

torch supplies device memory and the current HIP stream; every step of the
computation runs in libmlra.so's kernels. Tensor layouts are those of
include/mlra.h:

  q_latent      [S][Q][H][NB][DC]      bf16 or fp32
  q_rope        [S][Q][H][DR]          same dtype, shared by all branches
  latent_cache  [blocks][64][NB][DC]   same dtype (any strides with DC contiguous)
  rope_cache    [blocks][64][DR]       same dtype (any strides with DR contiguous)
  block_table   [S][max_blocks]        int32
  seq_lens      [S]                    int32, on the device
Returns (out, lse): out [S][Q][H][DC] for reduce="sum", [S][Q][H][NB][DC] for
"concat"; lse [S][Q][H][NB] float32.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.MLRA_BF16, torch.float32: _lib.MLRA_FP32}
_REDUCE = {"sum": _lib.MLRA_BRANCH_SUM, "concat": _lib.MLRA_BRANCH_CONCAT}

_workspaces: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A per-device scratch buffer that only grows (torch owns the memory)."""
    key = (device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        # zero-filled once: the library keeps its counter words at zero
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def make_dims(q_latent, q_rope, latent_cache, rope_cache, block_table, *, max_seq_len: int,
              reduce: str = "sum", causal: bool = True, num_splits: int = 0,
              sum_seq_lens: int = 0) -> _lib.DecodeDims:
    S, Q, H, NB, DC = q_latent.shape
    if latent_cache.dim() != 4 or latent_cache.shape[2] != NB or latent_cache.shape[3] != DC:
        raise ValueError(f"latent_cache shape {tuple(latent_cache.shape)} does not match "
                         f"q_latent {tuple(q_latent.shape)}")
    if rope_cache.dim() != 3 or q_rope.shape[:3] != (S, Q, H):
        raise ValueError("rope_cache must be [blocks][64][DR] and q_rope [S][Q][H][DR]")
    if latent_cache.stride(3) != 1 or rope_cache.stride(2) != 1:
        raise ValueError("the feature dimension of each cache must be contiguous")
    if q_latent.dtype not in _DTYPES or any(
            t.dtype != q_latent.dtype for t in (q_rope, latent_cache, rope_cache)):
        raise TypeError("q_latent, q_rope and both caches must share dtype bf16 or fp32")
    if block_table.dtype != torch.int32 or block_table.dim() != 2:
        raise TypeError("block_table must be a 2-D int32 tensor")
    d = _lib.DecodeDims()
    d.num_seqs, d.q_len, d.num_heads, d.d_latent = S, Q, H, DC
    d.d_rope = q_rope.shape[3]
    d.block_size = latent_cache.shape[1]
    d.max_blocks_per_seq = block_table.shape[1]
    d.num_blocks = latent_cache.shape[0]
    d.max_seq_len = int(max_seq_len)
    d.causal = 1 if causal else 0
    d.num_splits = int(num_splits)
    d.dtype = _DTYPES[q_latent.dtype]
    d.reduce = _REDUCE[reduce]
    d.latent_stride_block, d.latent_stride_token, d.latent_stride_branch = (
        latent_cache.stride(0), latent_cache.stride(1), latent_cache.stride(2))
    d.rope_stride_block, d.rope_stride_token = rope_cache.stride(0), rope_cache.stride(1)
    d.sum_seq_lens = int(sum_seq_lens)
    return d


def make_plan(dims: _lib.DecodeDims, n_branch: int, num_cus: int = 0) -> _lib.DecodePlan:
    lib = _lib.load()
    plan = _lib.DecodePlan()
    _lib.check(lib.mlra_decode_make_plan(dims, n_branch, num_cus, plan), "mlra_decode_make_plan")
    return plan


def _call(entry: str, q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
          n_branch, scale, out_rescale, max_seq_len, reduce, causal, num_splits, sum_seq_lens,
          out, lse, workspace, stream):
    lib = _lib.load()
    tensors = (q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens)
    dev = q_latent.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must be on the same GPU")
    for name, t in (("q_latent", q_latent), ("q_rope", q_rope), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (q_latent.shape[0],):
        raise TypeError("seq_lens must be an int32 tensor of shape [S]")
    dims = make_dims(q_latent, q_rope, latent_cache, rope_cache, block_table,
                     max_seq_len=max_seq_len, reduce=reduce, causal=causal,
                     num_splits=num_splits, sum_seq_lens=sum_seq_lens)
    S, Q, H, NB, DC = q_latent.shape
    oshape = (S, Q, H, DC) if reduce == "sum" else (S, Q, H, NB, DC)
    if out is None:
        out = torch.empty(oshape, dtype=q_latent.dtype, device=dev)
    if lse is None:
        lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device=dev)
    if tuple(out.shape) != oshape or out.dtype != q_latent.dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {q_latent.dtype} tensor of shape {oshape}")
    if tuple(lse.shape) != (S, Q, H, NB) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [S][Q][H][NB]")
    need = make_plan(dims, NB).workspace_bytes
    if workspace is None:
        workspace = _workspace(dev, need)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    if entry == "mla":
        status = lib.mla_decode_attention(
            q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
            rope_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), float(scale),
            out.data_ptr(), lse.data_ptr(), dims, workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), stream)
    else:
        status = lib.mlra_decode_attention(
            q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
            rope_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), int(n_branch),
            float(scale), float(out_rescale), out.data_ptr(), lse.data_ptr(), dims,
            workspace.data_ptr(), workspace.numel() * workspace.element_size(), stream)
    _lib.check(status, f"{entry}_decode_attention")
    return out, lse


def mlra_decode_attention(q_latent: torch.Tensor, q_rope: torch.Tensor,
                          latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor, n_branch: int,
                          scale: float, out_rescale: float, *, max_seq_len: int,
                          reduce: str = "sum", causal: bool = True, num_splits: int = 0,
                          sum_seq_lens: int = 0, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          stream: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLRA decode attention; see include/mlra.h for the definition."""
    if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
        raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
    return _call("mlra", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 n_branch, scale, out_rescale, max_seq_len, reduce, causal, num_splits,
                 sum_seq_lens, out, lse, workspace, stream)


def mla_decode_attention(q_latent: torch.Tensor, q_rope: torch.Tensor,
                         latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, *,
                         max_seq_len: int, causal: bool = True, num_splits: int = 0,
                         sum_seq_lens: int = 0, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLA-shaped single-latent call (n_branch = 1, out_rescale = 1).

    q_latent may be [S][Q][H][DC] or [S][Q][H][1][DC]; latent_cache may be
    [blocks][64][DC] or [blocks][64][1][DC]. Returns out [S][Q][H][DC] and
    lse [S][Q][H]."""
    if q_latent.dim() == 4:
        q_latent = q_latent.unsqueeze(3)
    if latent_cache.dim() == 3:
        latent_cache = latent_cache.unsqueeze(2)
    if lse is not None and lse.dim() == 3:
        lse = lse.unsqueeze(3)
    out, lse = _call("mla", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                     1, scale, 1.0, max_seq_len, "sum", causal, num_splits, sum_seq_lens, out,
                     lse, workspace, stream)
    return out, lse[..., 0]
