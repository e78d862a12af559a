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

Calls that do not pass a workspace share one per device; such calls must not
run concurrently on different streams, and they are refused while a stream is
being captured into a HIP graph (the shared buffer is replaced when a later
call needs more bytes, so a replayed graph would write freed memory): captured
calls pass their own workspace, or use PreparedDecode, which owns one.
PreparedDecode validates and marshals once, for loops that repeat the same call.
"""
from __future__ import annotations

from typing import Optional, Tuple

import ctypes

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.MLRA_BF16, torch.float32: _lib.MLRA_FP32}
_REDUCE = {"sum": _lib.MLRA_BRANCH_SUM, "concat": _lib.MLRA_BRANCH_CONCAT}

_workspaces: dict = {}


def _workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A per-device scratch buffer that only grows (torch owns the memory).

    Refused under stream capture: a graph would keep the pointer of a buffer
    that a later, larger call frees."""
    if torch.cuda.is_current_stream_capturing():
        raise RuntimeError("a call captured into a HIP graph must pass its own workspace "
                           "(or use PreparedDecode): the shared per-device workspace can be "
                           "replaced by a later call")
    key = (device.type, device.index)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = new_workspace(device, nbytes)
        _workspaces[key] = ws
    return ws


def new_workspace(device, nbytes: int) -> torch.Tensor:
    """A decode workspace of at least nbytes, zero-filled: its header (status
    word and in-kernel merge counters) must start at zero; every call leaves
    it ready for the next."""
    return torch.zeros(max(int(nbytes), _lib.MLRA_DECODE_WS_HEADER_BYTES), dtype=torch.uint8,
                       device=device)


def read_status(workspace: torch.Tensor, clear: bool = False, stream=None) -> int:
    """MLRA_DEVSTATUS_* bits set by calls on this workspace (0: none).
    Waits for the stream."""
    lib = _lib.load()
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
    bits = ctypes.c_uint32(0)
    _lib.check(lib.mlra_decode_read_status(workspace.data_ptr(), ctypes.byref(bits),
                                           1 if clear else 0, stream), "mlra_decode_read_status")
    return int(bits.value)


def default_workspace(device) -> Optional[torch.Tensor]:
    """The shared per-device workspace of calls that pass none (or None)."""
    dev = torch.device(device)
    return _workspaces.get((dev.type, dev.index))


def make_dims(q_latent, q_rope, latent_cache, rope_cache, block_table, *, max_seq_len: int,
              reduce: str = "sum", causal: bool = True, num_splits: int = 0,
              sum_seq_lens: int = 0, fused_merge: bool = False) -> _lib.DecodeDims:
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
    d.flags = _lib.MLRA_DECODE_FLAG_FUSED_MERGE if fused_merge else 0
    return d


def make_plan(dims: _lib.DecodeDims, n_branch: int, num_cus: int = 0) -> _lib.DecodePlan:
    lib = _lib.load()
    plan = _lib.DecodePlan()
    _lib.check(lib.mlra_decode_make_plan(dims, n_branch, num_cus, plan), "mlra_decode_make_plan")
    return plan


def make_prefill_plan(dims: _lib.DecodeDims, n_branch: int, num_cus: int = 0) -> _lib.DecodePlan:
    lib = _lib.load()
    plan = _lib.DecodePlan()
    _lib.check(lib.mlra_prefill_make_plan(dims, n_branch, num_cus, plan), "mlra_prefill_make_plan")
    return plan


def _call(entry: str, q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
          n_branch, scale, out_rescale, max_seq_len, reduce, causal, num_splits, sum_seq_lens,
          out, lse, workspace, stream, fused_merge=False):
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
                     num_splits=num_splits, sum_seq_lens=sum_seq_lens, fused_merge=fused_merge)
    S, Q, H, NB, DC = q_latent.shape
    oshape = (S, Q, H, DC) if reduce == "sum" else (S, Q, H, NB, DC)
    if entry == "partials":
        pass
    elif out is None:
        out = torch.empty(oshape, dtype=q_latent.dtype, device=dev)
    if entry != "partials":
        if lse is None:
            lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device=dev)
        if tuple(out.shape) != oshape or out.dtype != q_latent.dtype or not out.is_contiguous():
            raise ValueError(f"out must be a contiguous {q_latent.dtype} tensor of shape {oshape}")
        if (tuple(lse.shape) != (S, Q, H, NB) or lse.dtype != torch.float32
                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 tensor [S][Q][H][NB]")
    if workspace is None:
        if entry == "combine":
            raise ValueError("mlra_decode_combine needs the workspace of its partials call")
        plan = make_prefill_plan(dims, NB) if entry == "prefill" else make_plan(dims, NB)
        workspace = _workspace(dev, plan.workspace_bytes)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    wsb = workspace.numel() * workspace.element_size()
    if entry == "partials":
        status = lib.mlra_decode_partials(
            q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
            rope_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), int(n_branch),
            float(scale), dims, workspace.data_ptr(), wsb, stream)
        _lib.check(status, "mlra_decode_partials")
        return workspace
    if entry == "combine":
        status = lib.mlra_decode_combine(
            seq_lens.data_ptr(), int(n_branch), float(out_rescale), out.data_ptr(),
            lse.data_ptr(), dims, workspace.data_ptr(), wsb, stream)
    elif entry == "prefill":
        status = lib.mlra_prefill_attention(
            q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
            rope_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), int(n_branch),
            float(scale), float(out_rescale), out.data_ptr(), lse.data_ptr(), dims,
            workspace.data_ptr(), wsb, stream)
    elif entry == "mla":
        status = lib.mla_decode_attention(
            q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
            rope_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), float(scale),
            out.data_ptr(), lse.data_ptr(), dims, workspace.data_ptr(), wsb, stream)
    else:
        status = lib.mlra_decode_attention(
            q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
            rope_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(), int(n_branch),
            float(scale), float(out_rescale), out.data_ptr(), lse.data_ptr(), dims,
            workspace.data_ptr(), wsb, stream)
    _lib.check(status, {"combine": "mlra_decode_combine", "prefill": "mlra_prefill_attention"}
               .get(entry, f"{entry}_decode_attention"))
    return out, lse


def mlra_cache_append(latent_new: torch.Tensor, rope_new: torch.Tensor,
                      latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                      block_table: torch.Tensor, seq_lens: torch.Tensor, latent_scale: float,
                      rope_base: float = 10000.0, *, stream=None) -> None:
    """Write the Q new tokens of every sequence into the paged caches, in place.

    latent_new [S][Q][NB][DC] and rope_new [S][Q][DR] are float32 (projected;
    the key not yet rotated); the caches are laid out as for the decode call.
    Token j of sequence s lands at position seq_lens[s] - Q + j (include/mlra.h).
    """
    lib = _lib.load()
    tensors = (latent_new, rope_new, latent_cache, rope_cache, block_table, seq_lens)
    dev = latent_new.device
    if dev.type != "cuda" or any(t.device != dev for t in tensors):
        raise ValueError("all tensors must be on the same GPU")
    if latent_new.dtype != torch.float32 or rope_new.dtype != torch.float32:
        raise TypeError("latent_new and rope_new must be float32")
    if latent_new.dim() != 4 or rope_new.dim() != 3 or rope_new.shape[:2] != latent_new.shape[:2]:
        raise ValueError("latent_new must be [S][Q][NB][DC] and rope_new [S][Q][DR]")
    for name, t in (("latent_new", latent_new), ("rope_new", rope_new),
                    ("block_table", block_table), ("seq_lens", seq_lens)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    S, Q, NB, DC = latent_new.shape
    if seq_lens.dtype != torch.int32 or seq_lens.shape != (S,):
        raise TypeError("seq_lens must be an int32 tensor of shape [S]")
    # dims as the decode call sees these caches (one head: only the layout matters here)
    dims = make_dims(torch.empty((S, Q, 1, NB, DC), dtype=latent_cache.dtype, device="meta"),
                     torch.empty((S, Q, 1, rope_new.shape[2]), dtype=latent_cache.dtype,
                                 device="meta"),
                     latent_cache, rope_cache, block_table,
                     max_seq_len=block_table.shape[1] * latent_cache.shape[1])
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    status = lib.mlra_cache_append(latent_new.data_ptr(), rope_new.data_ptr(),
                                   latent_cache.data_ptr(), rope_cache.data_ptr(),
                                   block_table.data_ptr(), seq_lens.data_ptr(), int(NB),
                                   float(latent_scale), float(rope_base), dims, stream)
    _lib.check(status, "mlra_cache_append")


def pack_out_projection_weight(w: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Rewrite the absorbed weight w [D][K] (bf16) into the order
    mlra_out_projection loads (include/mlra.h). Done once per weight."""
    lib = _lib.load()
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_contiguous() or w.device.type != "cuda":
        raise ValueError("w must be a contiguous bf16 [D][K] tensor on the GPU")
    packed = torch.empty_like(w)
    if stream is None:
        stream = torch.cuda.current_stream(w.device).cuda_stream
    _lib.check(lib.mlra_out_projection_pack(w.data_ptr(), packed.data_ptr(), w.shape[1],
                                            w.shape[0], stream), "mlra_out_projection_pack")
    return packed


def out_projection_workspace_bytes(m: int, k: int, d: int) -> int:
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    _lib.check(lib.mlra_out_projection_workspace_size(int(m), int(k), int(d), ctypes.byref(n)),
               "mlra_out_projection_workspace_size")
    return int(n.value)


def mlra_out_projection(x: torch.Tensor, w_packed: torch.Tensor, *,
                        out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """y = x . W^T in bf16 (float32 accumulation): x is the decode call's CONCAT
    output [S][Q][H][NB][DC] (or already [M][K]); w_packed the absorbed weight
    [D][K] after pack_out_projection_weight. Returns y [M][D] (or [S][Q][D]
    for a 5-D x)."""
    lib = _lib.load()
    if x.dtype != torch.bfloat16 or w_packed.dtype != torch.bfloat16:
        raise TypeError("x and w_packed must be bfloat16")
    if not x.is_contiguous() or not w_packed.is_contiguous():
        raise ValueError("x and w_packed must be contiguous")
    lead = tuple(x.shape[:2]) if x.dim() == 5 else None
    x2 = x.reshape(-1, x.shape[2] * x.shape[3] * x.shape[4]) if x.dim() == 5 else x
    if x2.dim() != 2 or w_packed.dim() != 2 or w_packed.shape[1] != x2.shape[1]:
        raise ValueError("x must be [M][K] (or [S][Q][H][NB][DC]) and w_packed [D][K]")
    if x.device != w_packed.device or x.device.type != "cuda":
        raise ValueError("x and w_packed must be on the same GPU")
    M, K = x2.shape
    D = w_packed.shape[0]
    if out is None:
        out = torch.empty((M, D), dtype=torch.bfloat16, device=x.device)
    if out.numel() != M * D or out.dtype != torch.bfloat16 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous bf16 tensor of {M}x{D} elements")
    need = out_projection_workspace_bytes(M, K, D)
    if workspace is None and need > 0:
        workspace = _workspace(x.device, need)
    wsp = workspace.data_ptr() if workspace is not None else None
    wsb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _lib.check(lib.mlra_out_projection(x2.data_ptr(), w_packed.data_ptr(), out.data_ptr(), M, K, D,
                                       wsp, wsb, stream), "mlra_out_projection")
    return out.view(lead + (D,)) if lead else out.view(M, D)


def mlra_decode_attention(q_latent: torch.Tensor, q_rope: torch.Tensor,
                          latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                          block_table: torch.Tensor, seq_lens: torch.Tensor, n_branch: int,
                          scale: float, out_rescale: float, *, max_seq_len: int,
                          reduce: str = "sum", causal: bool = True, num_splits: int = 0,
                          sum_seq_lens: int = 0, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None,
                          stream: Optional[int] = None,
                          fused_merge: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """MLRA decode attention; see include/mlra.h for the definition.
    fused_merge=True lets the split kernel merge the splits itself where it
    can (MLRA_DECODE_FLAG_FUSED_MERGE)."""
    if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
        raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
    return _call("mlra", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 n_branch, scale, out_rescale, max_seq_len, reduce, causal, num_splits,
                 sum_seq_lens, out, lse, workspace, stream, fused_merge)


def mlra_decode_attention_static(q_latent: torch.Tensor, q_rope: torch.Tensor,
                                 latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                                 block_table: torch.Tensor, seq_lens: torch.Tensor, n_branch: int,
                                 scale: float, out_rescale: float, *, out: torch.Tensor,
                                 lse: torch.Tensor, max_seq_len: int, reduce: str = "sum",
                                 causal: bool = True, num_splits: int = 0, sum_seq_lens: int = 0,
                                 stream: Optional[int] = None,
                                 fused_merge: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """mlra_decode_attention on the library's own device scratch: no
    workspace, and nothing allocated (out and lse are the caller's), e.g. for
    code under graph capture; calls on one GPU must not overlap
    (include/mlra.h)."""
    lib = _lib.load()
    if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
        raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
    dims = make_dims(q_latent, q_rope, latent_cache, rope_cache, block_table,
                     max_seq_len=max_seq_len, reduce=reduce, causal=causal,
                     num_splits=num_splits, sum_seq_lens=sum_seq_lens, fused_merge=fused_merge)
    if stream is None:
        stream = torch.cuda.current_stream(q_latent.device).cuda_stream
    _lib.check(lib.mlra_decode_attention_static(
        q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(), rope_cache.data_ptr(),
        block_table.data_ptr(), seq_lens.data_ptr(), int(n_branch), float(scale),
        float(out_rescale), out.data_ptr(), lse.data_ptr(), dims, stream),
        "mlra_decode_attention_static")
    return out, lse


def mlra_prefill_attention(q_latent: torch.Tensor, q_rope: torch.Tensor,
                           latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                           block_table: torch.Tensor, seq_lens: torch.Tensor, n_branch: int,
                           scale: float, out_rescale: float, *, max_seq_len: int,
                           reduce: str = "sum", causal: bool = True, num_splits: int = 0,
                           sum_seq_lens: int = 0,
                           out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           stream: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked-prefill MLRA attention (many query tokens per sequence, bf16);
    see include/mlra.h. Same tensors and results as mlra_decode_attention.
    sum_seq_lens (optional) is the host-side sum of seq_lens: when it shows
    every sequence at max_seq_len the kernel skips ranking its work items."""
    if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
        raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
    return _call("prefill", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 n_branch, scale, out_rescale, max_seq_len, reduce, causal, num_splits,
                 sum_seq_lens, out, lse, workspace, stream)


def mla_decode_attention(q_latent: torch.Tensor, q_rope: torch.Tensor,
                         latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, scale: float, *,
                         max_seq_len: int, causal: bool = True, num_splits: int = 0,
                         sum_seq_lens: int = 0, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[int] = None,
                         fused_merge: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
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
                     lse, workspace, stream, fused_merge)
    return out, lse[..., 0]


def mlra_decode_partials(q_latent: torch.Tensor, q_rope: torch.Tensor,
                         latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                         block_table: torch.Tensor, seq_lens: torch.Tensor, n_branch: int,
                         scale: float, *, max_seq_len: int, reduce: str = "sum",
                         causal: bool = True, num_splits: int = 0, sum_seq_lens: int = 0,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[int] = None) -> torch.Tensor:
    """First half of mlra_decode_attention: per-split partial results into the
    workspace (layout in include/mlra.h). Returns the workspace tensor."""
    if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
        raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
    return _call("partials", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 n_branch, scale, 1.0, max_seq_len, reduce, causal, num_splits, sum_seq_lens,
                 None, None, workspace, stream)


def mlra_decode_combine(q_latent: torch.Tensor, q_rope: torch.Tensor,
                        latent_cache: torch.Tensor, rope_cache: torch.Tensor,
                        block_table: torch.Tensor, seq_lens: torch.Tensor, n_branch: int,
                        out_rescale: float, *, workspace: torch.Tensor, max_seq_len: int,
                        reduce: str = "sum", causal: bool = True, num_splits: int = 0,
                        sum_seq_lens: int = 0, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None,
                        stream: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Second half of mlra_decode_attention. The tensors other than seq_lens
    only give the shapes (the same as the partials call); their data is not
    read."""
    if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
        raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
    return _call("combine", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 n_branch, 1.0, out_rescale, max_seq_len, reduce, causal, num_splits,
                 sum_seq_lens, out, lse, workspace, stream)


class PreparedDecode:
    """One decode call with its arguments validated and marshalled once.

    run() / partials() / combine() enqueue the same call again on the stream
    captured at construction (the current stream by default; run() also takes
    another stream handle, e.g. a capturing one); a different
    block table of the same shape (e.g. another copy of the cache) may be
    passed per call. Tensors must stay alive and keep their storage.
    """

    def __init__(self, q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
                 n_branch: int, scale: float, out_rescale: float, *, max_seq_len: int,
                 reduce: str = "sum", causal: bool = True, num_splits: int = 0,
                 sum_seq_lens: int = 0, out=None, lse=None, workspace=None, stream=None,
                 fused_merge: bool = False):
        if q_latent.dim() != 5 or q_latent.shape[3] != n_branch:
            raise ValueError("q_latent must be [S][Q][H][n_branch][DC]")
        # one validated functional-path setup; its checks and shapes are reused
        self.dims = make_dims(q_latent, q_rope, latent_cache, rope_cache, block_table,
                              max_seq_len=max_seq_len, reduce=reduce, causal=causal,
                              num_splits=num_splits, sum_seq_lens=sum_seq_lens,
                              fused_merge=fused_merge)
        self.plan = make_plan(self.dims, n_branch)
        dev = q_latent.device
        S, Q, H, NB, DC = q_latent.shape
        oshape = (S, Q, H, DC) if reduce == "sum" else (S, Q, H, NB, DC)
        self.out = out if out is not None else torch.empty(oshape, dtype=q_latent.dtype,
                                                           device=dev)
        self.lse = lse if lse is not None else torch.empty((S, Q, H, NB), dtype=torch.float32,
                                                           device=dev)
        self.workspace = workspace if workspace is not None else new_workspace(
            dev, self.plan.workspace_bytes)
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
        # run the functional path once: validates every tensor and pointer rule
        _call("mlra", q_latent, q_rope, latent_cache, rope_cache, block_table, seq_lens,
              n_branch, scale, out_rescale, max_seq_len, reduce, causal, num_splits,
              sum_seq_lens, self.out, self.lse, self.workspace, self.stream, fused_merge)
        self._table_shape = tuple(block_table.shape)
        self._table_dev = block_table.device
        self._lib = _lib.load()
        self._ptrs = (q_latent.data_ptr(), q_rope.data_ptr(), latent_cache.data_ptr(),
                      rope_cache.data_ptr())
        self._table = block_table.data_ptr()
        self._lens = seq_lens.data_ptr()
        self._nb, self._scale, self._rescale = int(n_branch), float(scale), float(out_rescale)
        self._wsb = self.workspace.numel() * self.workspace.element_size()

    def _table_ptr(self, block_table):
        if block_table is None:
            return self._table
        if (tuple(block_table.shape) != self._table_shape or block_table.dtype != torch.int32
                or block_table.device != self._table_dev or not block_table.is_contiguous()):
            raise ValueError("block_table must match the prepared table's shape and device")
        return block_table.data_ptr()

    def run(self, block_table=None, stream=None):
        """Both kernels (mlra_decode_attention); returns (out, lse)."""
        q, qr, lc, rc = self._ptrs
        _lib.check(self._lib.mlra_decode_attention(
            q, qr, lc, rc, self._table_ptr(block_table), self._lens, self._nb, self._scale,
            self._rescale, self.out.data_ptr(), self.lse.data_ptr(), self.dims,
            self.workspace.data_ptr(), self._wsb, self.stream if stream is None else stream),
            "mlra_decode_attention")
        return self.out, self.lse

    def partials(self, block_table=None):
        """The split kernel only (mlra_decode_partials; never the in-kernel
        merge, so partials() + combine() is the two-kernel form of run())."""
        q, qr, lc, rc = self._ptrs
        _lib.check(self._lib.mlra_decode_partials(
            q, qr, lc, rc, self._table_ptr(block_table), self._lens, self._nb, self._scale,
            self.dims, self.workspace.data_ptr(), self._wsb, self.stream),
            "mlra_decode_partials")

    def combine(self):
        """The combine kernel only (mlra_decode_combine); returns (out, lse)."""
        _lib.check(self._lib.mlra_decode_combine(
            self._lens, self._nb, self._rescale, self.out.data_ptr(), self.lse.data_ptr(),
            self.dims, self.workspace.data_ptr(), self._wsb, self.stream), "mlra_decode_combine")
        return self.out, self.lse
