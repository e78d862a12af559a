"""Benchmark: MLRA decode attention over a paged latent KV cache on one MI355X.

Headline workload: one 4-way tensor-parallel rank's share of MLRA-4 decode
(one latent branch of 128 plus the shared 64-wide RoPE key, 1.5*dh per token),
batch 16, context 8192, 32 query heads, bf16, 64-token blocks placed by a
shuffled block table. A step is one full decode-attention call (split-K
kernel + log-sum-exp combine) over the batch.

Timing: the caches are replicated into enough copies (each with its own
block table) that consecutive steps never find their data in the 256 MB
Infinity Cache; HIP events on the launch stream bracket the K timed steps.
With --graph the timed steps are replayed from a HIP graph holding one call
per cache copy (as a serving loop would capture its decode step), and the
same K steps issued as individual launches are reported as eager_ms_per_step
(on one box graph replay saved 1.5 us per step, on another it cost 0.4 us,
so the default stays with individual launches).
value = algorithmic HBM bytes per step / time per step (GB/s); algorithmic
bytes = cache rows read + queries + block-table entries + seq_lens + outputs.
Two more passes issue K launches of each kernel alone (split kernel, then
combine kernel), bracketed by events: roofline.achieved is the split kernel's
algorithmic bytes (everything above but the outputs) over its average
per-launch time.

With --outproj it measures the output side (mlra_out_projection: the decode
call's concatenated output times the absorbed W_O . W_UV weight, model width
4096) for the workload's rows, next to torch.matmul on the same operands.
With --append the line instead measures the cache append (mlra_cache_append:
the new tokens' calibrated latents and rotated position keys written into the
paged caches) on the workload's layout, default mlra4_append_b4096_q2.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 20]
                       [--workload NAME] [--no-cpu-baseline] [--graph] [--append]
                       [--outproj] [--prefill]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 << 20      # Infinity Cache


def algorithmic_bytes(inp) -> dict:
    c = inp.cfg
    el = 2 if c.dtype == "bf16" else 4
    L = inp.seq_lens.astype(np.int64)
    cache = int(L.sum()) * (c.n_branch * c.d_latent + c.d_rope) * el
    q = c.num_seqs * c.q_len * c.num_heads * (c.n_branch * c.d_latent + c.d_rope) * el
    table = int(((L + c.block_size - 1) // c.block_size).sum()) * 4
    lens = c.num_seqs * 4
    out = c.num_seqs * c.q_len * c.num_heads * c.d_latent * el
    lse = c.num_seqs * c.q_len * c.num_heads * c.n_branch * 4
    total = cache + q + table + lens + out + lse
    return dict(total=total, cache=cache, out=out, lse=lse, kv_tokens=int(L.sum()))


KERNEL_SOURCES = {
    "decode": ("mlra_kernels.hip", "mlra_internal.h", "mlra_device.h"),
    "step": ("mlra_step_kernels.hip", "mlra_internal.h", "mlra_device.h"),
    "prefill": ("mlra_prefill_kernels.hip", "mlra_internal.h", "mlra_device.h"),
}


def kernel_source_digest(kernel: str = "mlra_split_pc") -> str:
    """sha256 over the sources that define a kernel (the decode kernels, or
    the append and output-projection kernels), to tell whether a stored
    counter measurement still describes the kernel that runs."""
    family = ("step" if kernel.startswith(("mlra_append", "mlra_outproj"))
              else "prefill" if kernel.startswith("mlra_prefill") else "decode")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, "latent_kv_cache_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# Split kernel that serves each plan.kernel_variant (include/mlra.h).
SPLIT_KERNELS = {1: "mlra_split_valu", 4: "mlra_split_pc"}


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per split-kernel launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None
    when there is none for this workload or the kernel source has changed."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256") != kernel_source_digest(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def flops(inp) -> int:
    c = inp.cfg
    L = inp.seq_lens.astype(np.int64)
    per = 2 * (c.n_branch * c.d_latent + c.d_rope) + 2 * c.n_branch * c.d_latent
    return int(L.sum()) * c.q_len * c.num_heads * per


def append_bytes(cfg) -> int:
    """Algorithmic bytes of one append call: the float32 new values read, the
    cache rows written, one block-table entry per token and seq_lens."""
    el = 2 if cfg.dtype == "bf16" else 4
    tokens = cfg.num_seqs * cfg.q_len
    row = cfg.n_branch * cfg.d_latent + cfg.d_rope
    return tokens * (row * 4 + row * el + 4) + cfg.num_seqs * 4


def bench_append(torch, args) -> int:
    from latent_kv_cache_amd import api, configs
    from latent_kv_cache_amd.inputs import make_append_inputs, make_inputs, to_device

    name = args.workload or "mlra4_append_b4096_q2"
    cfg = configs.BY_NAME[name]
    inp = make_inputs(cfg)
    lat_new, rope_new = make_append_inputs(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = to_device(inp, dev)
    nbytes = append_bytes(cfg)
    cache_bytes = d["latent_cache"].numel() * d["latent_cache"].element_size()
    # copies of the caches and of the new values, so that consecutive calls
    # touch memory the Infinity Cache does not hold
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / max(nbytes, 1)))
    copies = min(copies, max(2, int(40e9 // max(cache_bytes, 1))))
    nb = inp.num_blocks
    lat_all = d["latent_cache"].repeat(copies, 1, 1, 1)
    rope_all = d["rope_cache"].repeat(copies, 1, 1)
    tables = [(d["block_table"] + k * nb).contiguous() for k in range(copies)]
    lat_in = [torch.from_numpy(lat_new).to(dev) for _ in range(copies)]
    rope_in = [torch.from_numpy(rope_new).to(dev) for _ in range(copies)]
    scale = 1.0 / math.sqrt(2.0)

    def step(i):
        k = i % copies
        api.mlra_cache_append(lat_in[k], rope_in[k], lat_all, rope_all, tables[k],
                              d["seq_lens"], scale)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        step(i)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "cache append HBM GB/s (% of peak) + new tokens/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) float32 new tokens, shuffled paged blocks)",
        "config": {"workload": cfg.name, "batch": cfg.num_seqs, "new_tokens": cfg.q_len,
                   "n_branch": cfg.n_branch, "d_latent": cfg.d_latent, "d_rope": cfg.d_rope,
                   "block_size": cfg.block_size, "copies": copies},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(cfg.num_seqs * cfg.q_len / (ms * 1e-3), 1),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "hbm", "kernel": "mlra_append", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("mlra_append", cfg.name)},
    }
    if not args.no_cpu_baseline:
        from oracle import cache_append
        reps, t_total = 0, 0.0
        while t_total < 12.0 and reps < 100:
            t0 = time.perf_counter()
            cache_append(lat_new, rope_new, inp.latent_cache, inp.rope_cache, inp.block_table,
                         inp.seq_lens, scale, 10000.0, cfg.block_size)
            t_total += time.perf_counter() - t0
            reps += 1
        per = t_total / reps
        res["cpu_baseline"] = {
            "value": round(nbytes / per / 1e9, 4), "unit": "GB/s", **cpu_fields(1), "kind": "oracle",
            "sample": f"{reps} full passes of the {cfg.name} batch through the float64 oracle "
                      f"(single-threaded Python loop over tokens; {per * 1e3:.1f} ms per pass, "
                      f"{cfg.num_seqs * cfg.q_len / per:.0f} new tokens/s)"}
    print(json.dumps(res), flush=True)
    return 0


OUTPROJ_D = 4096  # model width: H * dv with dv = 128 (not on the pages)


def bench_outproj(torch, args) -> int:
    from latent_kv_cache_amd import api, configs
    from latent_kv_cache_amd.inputs import make_out_proj_inputs

    cfg = configs.BY_NAME[args.workload or DEFAULT_WORKLOAD]
    M = cfg.num_seqs * cfg.q_len
    K = cfg.num_heads * cfg.n_branch * cfg.d_latent
    D = OUTPROJ_D
    x, w = make_out_proj_inputs(M, K, D, seed=cfg.seed)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wbytes = D * K * 2
    nbytes = wbytes + M * K * 2 + M * D * 2
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / wbytes))
    xd = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    w0 = torch.from_numpy(w).to(dev).to(torch.bfloat16)
    wps = [api.pack_out_projection_weight(w0) for _ in range(copies)]   # packed once per weight
    wts = [w0.clone() for _ in range(copies)]                            # for torch.matmul
    y = torch.empty((M, D), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        torch.cuda._sleep(50_000_000)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms = timed(lambda i: api.mlra_out_projection(xd, wps[i % copies], out=y))
    ms_lib = timed(lambda i: torch.matmul(xd, wts[i % copies].t()))
    gbs = nbytes / (ms * 1e-3) / 1e9
    res = {
        "metric": "decode output projection HBM GB/s (% of peak)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) decode output, N(0,1/K) absorbed weight)",
        "config": {"workload": cfg.name, "rows": M, "k": K, "d_model": D, "weight_copies": copies},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "algorithmic_bytes_per_step": nbytes,
        "torch_matmul_us": round(ms_lib * 1e3, 3),
        "roofline": {"bound": "hbm", "kernel": "mlra_outproj", "achieved": round(gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("mlra_outproj", cfg.name)},
    }
    if not args.no_cpu_baseline:
        from oracle import out_projection
        x3 = x.astype(np.float64)[:, None, None, None, :]
        reps, t_total = 0, 0.0
        while t_total < 10.0 and reps < 200:
            t0 = time.perf_counter()
            out_projection(x3, w)
            t_total += time.perf_counter() - t0
            reps += 1
        per = t_total / reps
        res["cpu_baseline"] = {
            "value": round(nbytes / per / 1e9, 3), "unit": "GB/s", **cpu_fields(_blas_threads()),
            "kind": "oracle",
            "sample": f"{reps} passes of the float64 oracle (NumPy matmul, float64 copy of the "
                      f"weight included) over the same operands, {per * 1e3:.1f} ms per pass"}
    print(json.dumps(res), flush=True)
    return 0


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def prefill_visible_tokens(inp) -> int:
    """Sum over query tokens of the tokens each one sees (causal chunk rule)."""
    c = inp.cfg
    L = inp.seq_lens.astype(np.int64)[:, None]
    j = np.arange(c.q_len, dtype=np.int64)[None, :]
    V = L - (c.q_len - 1 - j) if c.causal else np.broadcast_to(L, (len(L), c.q_len))
    return int(np.clip(V, 0, None).sum())


def prefill_flops(inp) -> int:
    """Algorithmic flops of one prefill call: per query row, branch and visible
    token, 2*(DC + DR) for the score and 2*DC for the output."""
    c = inp.cfg
    per = 2 * (c.d_latent + c.d_rope) + 2 * c.d_latent
    return prefill_visible_tokens(inp) * c.num_heads * c.n_branch * per


def _sdpa_whole_prefill_ms(torch, inp, d, timed):
    """torch's scaled_dot_product_attention (its own causal flag) on the same
    whole-sequence prefill with keys and values materialised per branch, or
    None when the shape has cached context before the chunk or SDPA fails."""
    c = inp.cfg
    if not c.causal or any(int(L) != c.q_len for L in inp.seq_lens):
        return None
    try:
        S, Q, H, NB, DC = c.num_seqs, c.q_len, c.num_heads, c.n_branch, c.d_latent
        nblk = -(-Q // c.block_size)
        tab = d["block_table"][:, :nblk].long()
        lat = d["latent_cache"][tab].reshape(S, nblk * c.block_size, NB, DC)[:, :Q]
        kr = d["rope_cache"][tab].reshape(S, nblk * c.block_size, -1)[:, :Q]
        qs, ks, vs = [], [], []
        for b in range(NB):
            qs.append(torch.cat([d["q_latent"][:, :, :, b], d["q_rope"]], -1).transpose(1, 2)
                      .contiguous())
            ks.append(torch.cat([lat[:, :, b], kr], -1)[:, None].expand(S, H, Q, -1).contiguous())
            v = torch.nn.functional.pad(lat[:, :, b], (0, c.d_rope))  # v padded to the qk width
            vs.append(v[:, None].expand(S, H, Q, -1).contiguous())
        f = torch.nn.functional.scaled_dot_product_attention

        def run(i):
            for b in range(NB):
                f(qs[b], ks[b], vs[b], is_causal=True, scale=c.scale)
        return timed(run)
    except Exception:
        return None


def bench_prefill(torch, args) -> int:
    from latent_kv_cache_amd import api, configs
    from latent_kv_cache_amd.inputs import make_inputs, to_device

    cfg = configs.BY_NAME[args.workload or "mlra4_tp_share_prefill_b4_c2048_t8192"]
    inp = make_inputs(cfg)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = to_device(inp, dev)
    S, Q, H, NB, DC = inp.q_latent.shape
    out = torch.empty((S, Q, H, DC), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device=dev)
    dims = api.make_dims(d["q_latent"], d["q_rope"], d["latent_cache"], d["rope_cache"],
                         d["block_table"], max_seq_len=inp.max_seq_len, causal=cfg.causal)
    plan = api.make_prefill_plan(dims, NB)
    ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    fl = prefill_flops(inp)

    def step(i):
        api.mlra_prefill_attention(d["q_latent"], d["q_rope"], d["latent_cache"],
                                   d["rope_cache"], d["block_table"], d["seq_lens"], NB,
                                   cfg.scale, cfg.out_rescale, max_seq_len=inp.max_seq_len,
                                   causal=cfg.causal, sum_seq_lens=int(inp.seq_lens.sum()),
                                   out=out, lse=lse, workspace=ws)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(args.steps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms = timed(step)
    tfs = fl / (ms * 1e-3) / 1e12
    sdpa_ms = _sdpa_whole_prefill_ms(torch, inp, d, timed)
    res = {
        "metric": "chunked-prefill attention TFLOP/s (% of bf16 MFMA peak)",
        "value": round(tfs, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 latents, keys and queries, shuffled paged blocks)",
        "config": {"workload": cfg.name, "batch": S, "chunk_tokens": Q, "heads": H,
                   "n_branch": NB, "d_latent": DC, "d_rope": cfg.d_rope,
                   "context": int(inp.max_seq_len), "causal": bool(cfg.causal),
                   "splits": plan.splits_per_seq, "workgroups": plan.target_groups},
        "pct_of_mfma_peak": round(100 * tfs / MFMA_BF16_PEAK_TFLOPS, 2),
        "algorithmic_flops_per_step": fl,
        "query_tokens_per_s": round(S * Q / (ms * 1e-3), 1),
        "torch_sdpa_ms": None if sdpa_ms is None else round(sdpa_ms, 4),
        "roofline": {"bound": "mfma", "kernel": "mlra_prefill", "achieved": round(tfs, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("mlra_prefill", cfg.name)},
    }
    if not args.no_cpu_baseline:
        from oracle import mlra_decode
        # query tokens of sequence 0, from its last one backwards, one oracle
        # call per token (its visible length as the sequence length)
        per_tok = 2 * (DC + cfg.d_rope) + 2 * DC
        L0 = int(inp.seq_lens[0])
        done, t_total, ntok = 0, 0.0, 0
        for j in range(Q - 1, -1, -1):
            if t_total >= 10.0:
                break
            V = L0 - (Q - 1 - j) if cfg.causal else L0
            t0 = time.perf_counter()
            mlra_decode(inp.q_latent[:1, j:j + 1], inp.q_rope[:1, j:j + 1], inp.latent_cache,
                        inp.rope_cache, inp.block_table[:1], np.array([V], dtype=np.int32),
                        cfg.scale, cfg.out_rescale, "sum", False, cfg.block_size)
            t_total += time.perf_counter() - t0
            done += max(V, 0) * H * NB * per_tok
            ntok += 1
        res["cpu_baseline"] = {
            "value": round(done / t_total / 1e12, 6), "unit": "TFLOP/s",
            **cpu_fields(_blas_threads()), "kind": "oracle",
            "sample": f"{ntok} query tokens of sequence 0 (all {H} heads, the last ones of the "
                      f"chunk) through the float64 NumPy oracle, {t_total:.1f} s"}
    print(json.dumps(res), flush=True)
    return 0


def _blas_info() -> dict:
    """BLAS library NumPy calls into: vendor (internal_api) and thread count."""
    try:
        from threadpoolctl import threadpool_info
        blas = [t for t in threadpool_info() if t.get("user_api") == "blas"]
        if blas:
            return {"vendor": str(blas[0].get("internal_api", "unknown")),
                    "threads": int(max(t.get("num_threads", 1) for t in blas))}
    except Exception:  # pragma: no cover
        pass
    return {"vendor": "unknown", "threads": 1}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_fields(threads_used: int) -> dict:
    """What the CPU baseline ran on: `cores` is the threads the oracle used
    (BLAS threads, never more than the cores this process may run on); the
    affinity count, CPU model and BLAS vendor/threads are reported beside it."""
    affinity = len(os.sched_getaffinity(0))
    return {"cores": int(min(threads_used, affinity)), "affinity_cores": affinity,
            "cpu_model": _cpu_model(), "blas": _blas_info()}


def _blas_threads() -> int:
    return _blas_info()["threads"]


def cpu_baseline(inp, budget_s: float = 12.0) -> dict:
    """Time the float64 oracle on the host over repeated passes of the batch."""
    from oracle import mlra_decode
    threads = _blas_threads()
    c = inp.cfg
    nbytes = algorithmic_bytes(inp)["total"]
    reps, t_total = 0, 0.0
    while t_total < budget_s and reps < 1000:
        t0 = time.perf_counter()
        mlra_decode(inp.q_latent, inp.q_rope, inp.latent_cache, inp.rope_cache,
                    inp.block_table, inp.seq_lens, c.scale, c.out_rescale, "sum", c.causal,
                    c.block_size)
        t_total += time.perf_counter() - t0
        reps += 1
    per = t_total / reps
    return {"value": round(nbytes / per / 1e9, 3), "unit": "GB/s", **cpu_fields(threads),
            "kind": "oracle",
            "sample": f"{reps} full passes of the {c.name} batch through the float64 NumPy "
                      f"oracle ({per * 1e3:.1f} ms per pass, {c.num_seqs * c.q_len / per:.1f} "
                      f"decode tokens/s)"}


def copy_calibration(torch, mib: int, steps: int, warmup: int) -> int:
    """K copies of a MIB-MiB buffer: each reads and writes exactly MIB MiB."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "ms_per_copy": round(ms, 5),
                      "gbs_read_plus_write": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


DEFAULT_WORKLOAD = "mlra4_tp_share_b16_t8192"

CEILING_BUFFER = 2 << 30  # bytes streamed by the 2 GB read, and rotated through by the small one


def read_ceiling(torch, lib, nbytes: int, workgroups: int, steps: int, timed) -> dict:
    """Streaming-read ceiling in the same run (mlra_stream_read, a plain HIP
    read kernel): nbytes per launch with `workgroups` workgroups of 512
    threads, launches rotating through a 2 GB buffer so that none finds its
    bytes in the 256 MB Infinity Cache (a read larger than the buffer gets a
    buffer of its own size); then one 2 GB read per launch."""
    dev = torch.device("cuda:0")
    unit = 16 * workgroups
    n = max(unit, nbytes // unit * unit)
    size = max(CEILING_BUFFER, n)
    buf = torch.empty(size, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(max(workgroups, 2048), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    slots = size // n

    def small(i):
        _check_status(lib.mlra_stream_read(buf.data_ptr() + (i % slots) * n, n, workgroups,
                                           sink.data_ptr(), stream))

    def big(i):
        _check_status(lib.mlra_stream_read(buf.data_ptr(), CEILING_BUFFER, 2048, sink.data_ptr(),
                                           stream))

    ms_small = timed(small)
    ms_big = timed(big, min(steps, 20))
    del buf
    return {"at_split_shape_gbs": round(n / (ms_small * 1e-3) / 1e9, 1), "workgroups": workgroups,
            "bytes": n, "us": round(ms_small * 1e3, 3),
            "gbs_2gb": round(CEILING_BUFFER / (ms_big * 1e-3) / 1e9, 1)}


def _check_status(st: int) -> None:
    if st != 0:
        raise RuntimeError(f"mlra_stream_read failed with status {st}")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help=f"workload name (default {DEFAULT_WORKLOAD}; with --append "
                         "mlra4_append_b4096_q2)")
    ap.add_argument("--append", action="store_true",
                    help="measure the cache append instead of decode attention")
    ap.add_argument("--outproj", action="store_true",
                    help="measure the output projection instead of decode attention")
    ap.add_argument("--prefill", action="store_true",
                    help="measure chunked-prefill attention (default workload "
                         "mlra4_tp_share_prefill_b4_c2048_t8192) instead of decode attention")
    ap.add_argument("--copies", type=int, default=0, help="cache copies (0: enough to exceed 2x MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-merge", action="store_true",
                    help="let the split kernel merge the splits itself where it can "
                         "(MLRA_DECODE_FLAG_FUSED_MERGE) instead of a second kernel")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from a HIP graph (the individual-launch time is "
                         "reported beside as eager_ms_per_step)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run K plain device-to-device copies of MIB MiB (the known-size "
                         "reference for scaling HBM byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this decode path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        return copy_calibration(torch, args.copy_calibration, args.steps, args.warmup)
    if args.append:
        return bench_append(torch, args)
    if args.outproj:
        return bench_outproj(torch, args)
    if args.prefill:
        return bench_prefill(torch, args)
    from latent_kv_cache_amd import api, configs
    from latent_kv_cache_amd.inputs import make_inputs, to_device

    cfg = configs.BY_NAME[args.workload or DEFAULT_WORKLOAD]
    inp = make_inputs(cfg)
    ab = algorithmic_bytes(inp)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = to_device(inp, dev)

    # Replicate the caches so that consecutive steps touch disjoint memory.
    copies = args.copies or max(2, math.ceil(2 * MALL_BYTES / ab["cache"]))
    nb = inp.num_blocks
    lat_all = d["latent_cache"].repeat(copies, 1, 1, 1)
    rope_all = d["rope_cache"].repeat(copies, 1, 1)
    tables = [(d["block_table"] + k * nb).contiguous() for k in range(copies)]
    del d["latent_cache"], d["rope_cache"]
    reduce = "sum"
    S, Q, H, NB, DC = inp.q_latent.shape
    out = torch.empty((S, Q, H, DC), dtype=d["q_latent"].dtype, device=dev)
    lse = torch.empty((S, Q, H, NB), dtype=torch.float32, device=dev)
    kw = dict(max_seq_len=inp.max_seq_len, reduce=reduce, causal=cfg.causal,
              sum_seq_lens=int(inp.seq_lens.sum()))
    prep = api.PreparedDecode(d["q_latent"], d["q_rope"], lat_all, rope_all, tables[0],
                              d["seq_lens"], NB, cfg.scale, cfg.out_rescale, out=out, lse=lse,
                              fused_merge=args.fused_merge, **kw)
    plan = prep.plan

    def step(i):
        prep.run(tables[i % copies])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cs = torch.cuda.current_stream().cuda_stream
            for i in range(copies):
                prep.run(tables[i], stream=cs)
        graph.replay()
        torch.cuda.synchronize()

    def head_start():
        # A short spin kernel ahead of the timed work lets the host enqueue the
        # steps before the GPU reaches them, so host-side call overhead never
        # leaves the GPU idle between kernels inside the timed region.
        torch.cuda._sleep(50_000_000)

    # Timed region: K steps between two events on the launch stream (torch's
    # current stream, which the prepared call enqueues on).
    def timed_steps(use_graph):
        torch.cuda.synchronize()
        head_start()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        if use_graph:
            reps = max(1, args.steps // copies)
            for _ in range(reps):
                graph.replay()
            n = reps * copies
        else:
            for i in range(args.steps):
                step(i)
            n = args.steps
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / n, n

    eager_ms, steps = timed_steps(False)
    ms = eager_ms
    if graph is not None:
        ms, steps = timed_steps(True)

    # Kernel passes: the same K steps issued as one half of the call at a time
    # (K split-kernel launches, then K combine launches over the last
    # partials), each run bracketed by two events on the launch stream; an
    # event between every two kernels would itself add about 1.5 us per event.
    def timed(fn, n=None):
        n = n or args.steps
        torch.cuda.synchronize()
        head_start()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    split_avg = timed(lambda i: prep.partials(tables[i % copies]))
    comb_avg = timed(lambda i: prep.combine())
    split_bytes = ab["total"] - ab["out"] - ab["lse"]
    split_gbs = split_bytes / (split_avg * 1e-3) / 1e9
    # the same-run ceiling: a plain read of the split kernel's bytes with one
    # 512-thread workgroup per CU (its launch shape), and a 2 GB read
    ceiling = read_ceiling(torch, api._lib.load(), split_bytes, plan.num_cus, args.steps, timed)

    # per-step events (a separate pass) for the median step time
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(args.steps, 200))]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in evs)
    med_ms = per_step[len(per_step) // 2]
    split_kernel = SPLIT_KERNELS.get(plan.kernel_variant, f"variant{plan.kernel_variant}")
    traffic = measured_traffic(split_kernel, cfg.name)

    gbs = ab["total"] / (ms * 1e-3) / 1e9
    res = {
        "metric": "decode attention latent-cache HBM GB/s (% of peak) + tokens/s at B=16, T=8k",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) latents and queries, shuffled paged blocks)",
        "config": {"workload": cfg.name, "batch": cfg.num_seqs, "context": inp.max_seq_len,
                   "q_len": cfg.q_len, "heads": cfg.num_heads, "n_branch": cfg.n_branch,
                   "d_latent": cfg.d_latent, "d_rope": cfg.d_rope, "block_size": cfg.block_size,
                   "cache_copies": copies, "tiles_per_split": plan.tiles_per_split,
                   "splits_per_seq": plan.splits_per_seq, "fused_merge": bool(plan.fused_merge),
                   "graph": bool(graph)},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(cfg.num_seqs * cfg.q_len / (ms * 1e-3), 1),
        "kv_tokens_per_s": round(ab["kv_tokens"] / (ms * 1e-3), 1),
        "median_step_ms": round(med_ms, 5),
        "eager_ms_per_step": round(eager_ms, 5),
        "algorithmic_bytes_per_step": ab["total"],
        "kernels": {"split_avg_us": round(split_avg * 1e3, 3),
                    "combine_avg_us": round(comb_avg * 1e3, 3),
                    "split_algorithmic_bytes": split_bytes},
        "read_ceiling": ceiling,
        "pct_of_read_ceiling": round(100 * gbs / ceiling["at_split_shape_gbs"], 2),
        "split_pct_of_read_ceiling": round(100 * split_gbs / ceiling["at_split_shape_gbs"], 2),
        "roofline": {"bound": "hbm", "kernel": split_kernel, "achieved": round(split_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(split_gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
