"""C-ABI checks that need no GPU: the library loads, exports what the header
declares, validates arguments and plans split-K on the host."""
import ctypes
import math
import os
import re

import pytest

from latent_kv_cache_amd import _lib, configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlra.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _dims(cfg, **kw):
    d = _lib.DecodeDims()
    d.num_seqs, d.q_len, d.num_heads = cfg.num_seqs, cfg.q_len, cfg.num_heads
    d.d_latent, d.d_rope, d.block_size = cfg.d_latent, cfg.d_rope, 64
    L = cfg.context if cfg.context is not None else cfg.context_range[1]
    d.max_blocks_per_seq = -(-L // 64)
    d.num_blocks = d.max_blocks_per_seq * cfg.num_seqs + 1
    d.max_seq_len = L
    d.causal = 1
    d.dtype = _lib.MLRA_BF16 if cfg.dtype == "bf16" else _lib.MLRA_FP32
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _plan(lib, d, nb, cus=256):
    p = _lib.DecodePlan()
    st = lib.mlra_decode_make_plan(ctypes.byref(d), nb, cus, ctypes.byref(p))
    return st, p


def test_header_declarations_are_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:mlra_status|const char\*|int32_t)\s+(\w+)\s*\(", text,
                              re.M))
    assert declared == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_struct_layouts_match_header():
    # int32 x 14 then int64 x 6; the plan ends with a size_t.
    assert ctypes.sizeof(_lib.DecodeDims) == 14 * 4 + 6 * 8
    assert _lib.DecodeDims.latent_stride_block.offset == 56
    assert ctypes.sizeof(_lib.DecodePlan) == 10 * 4 + 8


def test_status_strings_and_version(lib):
    for code in range(7):
        assert lib.mlra_status_string(code)
    assert lib.mlra_status_string(99) == b"unknown status"
    assert lib.mlra_version() >= 100


@pytest.mark.parametrize("cfg", configs.ALL + [configs.MLA_COMPARE] + configs.EXTRA,
                         ids=lambda c: c.name)
def test_plan_covers_every_tile(lib, cfg):
    d = _dims(cfg)
    st, p = _plan(lib, d, cfg.n_branch)
    assert st == 0
    max_tiles = -(-d.max_seq_len // 64)
    assert p.splits_per_seq * p.tiles_per_split >= max_tiles
    assert (p.splits_per_seq - 1) * p.tiles_per_split < max(max_tiles, 1)
    if cfg.dtype == "bf16":  # block ids of a split fit the LDS table
        assert p.tiles_per_split <= 1024
    rows = cfg.num_heads * cfg.q_len
    slots = cfg.num_seqs * p.splits_per_seq * cfg.n_branch * rows
    assert p.workspace_bytes >= slots * (cfg.d_latent + 1) * 4
    # 1: fp32 vector ALU; 4: bf16 (loader and compute waves)
    expect = 1 if cfg.dtype != "bf16" else 4
    assert p.kernel_variant == expect
    assert p.lds_bytes <= 160 * 1024


# (branches, latent, heads, q_len) -> workgroups per split. A workgroup's
# four compute waves take (branch, 32-row tile, 128-column slice) triples:
# with up to 32 rows one workgroup holds every branch; with more it holds
# the power of two of row tiles that covers them (as far as the slices leave
# waves) for as many branches as fit, and further branches and row tiles
# take more workgroups (branch groups x row groups, at most 4).
@pytest.mark.parametrize("nb,dc,h,q,groups", [
    (1, 128, 32, 1, 1), (1, 128, 24, 2, 1), (2, 64, 32, 2, 1), (4, 128, 16, 1, 1),
    (4, 128, 32, 1, 1), (4, 128, 17, 2, 2), (4, 64, 32, 2, 2), (1, 256, 32, 1, 1),
    (1, 256, 32, 2, 1), (2, 256, 16, 1, 1), (2, 256, 24, 2, 2), (1, 512, 32, 1, 1),
    (1, 512, 32, 2, 2), (1, 128, 32, 4, 1), (1, 64, 24, 4, 1), (2, 128, 32, 3, 2),
    (4, 128, 32, 4, 4), (4, 64, 20, 4, 4), (1, 256, 32, 4, 2), (2, 256, 32, 4, 4),
    (1, 512, 24, 4, 3), (1, 512, 32, 4, 4)])
def test_workgroups_per_split(lib, nb, dc, h, q, groups):
    cfg = configs.MLRA4_FUSED.with_(n_branch=nb, d_latent=dc, num_heads=h, q_len=q)
    st, p = _plan(lib, _dims(cfg), nb)
    assert st == 0
    assert p.row_groups == groups
    assert p.kernel_variant == 4 and p.waves_per_group == 8
    assert p.lds_bytes <= 160 * 1024


def test_plan_fills_the_gpu_for_the_single_branch_share(lib):
    d = _dims(configs.MLRA4_TP_SHARE)
    st, p = _plan(lib, d, 1)
    groups = d.num_seqs * p.splits_per_seq
    assert st == 0 and groups >= 256


def test_ragged_hint_balances_splits(lib):
    cfg = configs.RAGGED_Q2
    d = _dims(cfg)
    _, p_worst = _plan(lib, d, 4)
    d.sum_seq_lens = cfg.num_seqs * 16896
    _, p_hint = _plan(lib, d, 4)
    assert p_hint.tiles_per_split < p_worst.tiles_per_split
    d.num_splits = 3
    _, p_forced = _plan(lib, d, 4)
    assert p_forced.splits_per_seq <= 3


@pytest.mark.parametrize("field,value,status", [
    ("num_seqs", 0, 2), ("q_len", 5, 3), ("num_heads", 65, 3), ("d_latent", 96, 3),
    ("d_rope", 48, 3), ("block_size", 32, 3), ("block_size", 0, 2), ("max_blocks_per_seq", 0, 2),
    ("max_seq_len", 10 ** 6, 2), ("max_seq_len", -1, 2), ("num_splits", -2, 2), ("dtype", 7, 2),
    ("reduce", 2, 2), ("flags", 2, 2), ("flags", -1, 2), ("latent_stride_block", 1000, 2),
    ("latent_stride_token", 516, 5), ("rope_stride_block", 60, 2), ("sum_seq_lens", -1, 2),
    ("num_seqs", 70000, 3),
])
def test_validation_errors(lib, field, value, status):
    d = _dims(configs.MLRA4_FUSED)
    if field == "num_heads":
        d.q_len = 2
    setattr(d, field, value)
    st, _ = _plan(lib, d, 4)
    assert st == status, (field, value, st)


def test_branch_and_width_rules(lib):
    d = _dims(configs.MLA_COMPARE)
    assert _plan(lib, d, 1)[0] == 0
    assert _plan(lib, d, 2)[0] == 3        # bf16 512-wide latent only as a single head
    assert _plan(lib, d, 3)[0] == 3
    assert _plan(lib, d, 0)[0] == 2
    d.dtype = _lib.MLRA_FP32
    assert _plan(lib, d, 2)[0] == 0
    d = _dims(configs.MLRA2_FUSED)             # bf16 256-wide latent: up to two branches, RoPE 64
    assert _plan(lib, d, 2)[0] == 0 and _plan(lib, d, 1)[0] == 0
    assert _plan(lib, d, 4)[0] == 3
    d.d_rope = 32
    assert _plan(lib, d, 2)[0] == 3


def test_pointer_and_alignment_errors_before_any_device_call(lib):
    cfg = configs.MLRA4_TP_SHARE
    d = _dims(cfg)
    ok = ctypes.c_void_p(4096)
    args = [ok] * 6 + [1, 0.1, 0.5, ok, ok, ctypes.byref(d), ok, 1 << 30, None]
    a = list(args)
    a[0] = None
    assert lib.mlra_decode_attention(*a) == 1
    a = list(args)
    a[10] = None
    assert lib.mlra_decode_attention(*a) == 1
    a = list(args)
    a[2] = ctypes.c_void_p(4096 + 8)
    assert lib.mlra_decode_attention(*a) == 5
    a = list(args)
    a[7] = math.inf
    assert lib.mlra_decode_attention(*a) == 2
    a = list(args)
    a[6] = 3
    assert lib.mlra_decode_attention(*a) == 3
    assert lib.mla_decode_attention(None, ok, ok, ok, ok, ok, 0.1, ok, ok, ctypes.byref(d), ok,
                                    1 << 30, None) == 1


def test_two_phase_entry_points_check_only_their_own_pointers(lib):
    d = _dims(configs.MLRA4_TP_SHARE)
    ok = ctypes.c_void_p(4096)
    part = [ok] * 6 + [1, 0.1, ctypes.byref(d), ok, 1 << 30, None]
    for i in range(6):
        a = list(part)
        a[i] = None
        assert lib.mlra_decode_partials(*a) == 1, i
    a = list(part)
    a[7] = -1.0
    assert lib.mlra_decode_partials(*a) == 2
    a = list(part)
    a[4] = ctypes.c_void_p(4098)          # block table must be 4-byte aligned
    assert lib.mlra_decode_partials(*a) == 5
    a = list(part)
    a[9] = None                           # workspace
    assert lib.mlra_decode_partials(*a) == 4
    comb = [ok, 1, 0.5, ok, ok, ctypes.byref(d), ok, 1 << 30, None]
    for i in (0, 3, 4):
        a = list(comb)
        a[i] = None
        assert lib.mlra_decode_combine(*a) == 1, i
    a = list(comb)
    a[2] = math.nan
    assert lib.mlra_decode_combine(*a) == 2
    a = list(comb)
    a[3] = ctypes.c_void_p(4096 + 4)      # out must be 16-byte aligned
    assert lib.mlra_decode_combine(*a) == 5


def test_cache_append_validates_before_touching_memory(lib):
    # statuses come from host checks alone: no pointer is dereferenced
    d = _dims(configs.MLRA4_FUSED)
    fake = [256 * (i + 1) for i in range(6)]   # aligned, never read
    ok_args = lambda: fake + [4, 0.5, 10000.0, ctypes.byref(d), None]
    args = ok_args()
    args[0] = None
    assert lib.mlra_cache_append(*args) == 1                     # NULL latent_new
    for k, v in ((7, float("nan")), (8, 0.0), (8, -1.0), (8, float("inf"))):
        args = ok_args()
        args[k] = v
        assert lib.mlra_cache_append(*args) == 2, (k, v)         # bad scale / base
    args = ok_args()
    args[2] = 256 + 8
    assert lib.mlra_cache_append(*args) == 5                     # misaligned cache
    args = ok_args()
    args[6] = 3
    assert lib.mlra_cache_append(*args) == 3                     # unsupported n_branch


def test_out_projection_validation(lib):
    n = ctypes.c_size_t(123)
    assert lib.mlra_out_projection_workspace_size(16, 4096, 4096, ctypes.byref(n)) == 0
    # the header every workspace starts with, then eight K-chunks of float32 partials
    assert n.value == _lib.MLRA_DECODE_WS_HEADER_BYTES + 8 * 16 * 4096 * 4
    assert lib.mlra_out_projection_workspace_size(0, 512, 128, ctypes.byref(n)) == 2
    for m, k, d in ((129, 512, 128), (16, 768, 128), (16, 512, 96)):  # M, K or D off the grid
        assert lib.mlra_out_projection_workspace_size(m, k, d, ctypes.byref(n)) == 3
    fake = 4096
    assert lib.mlra_out_projection(None, fake, fake, 16, 4096, 4096, fake, 1 << 22, None) == 1
    assert lib.mlra_out_projection(fake, fake, fake, 16, 4096, 4096, fake, 16, None) == 4
    assert lib.mlra_out_projection(fake + 2, fake, fake, 16, 4096, 4096, fake, 1 << 22, None) == 5
    assert lib.mlra_out_projection_pack(fake, None, 4096, 4096, None) == 1
    assert lib.mlra_out_projection_pack(fake, fake, 100, 4096, None) == 3
    assert lib.mlra_out_projection_pack(fake, fake + 8, 4096, 4096, None) == 5


# --------------------------------------------------------------------------- prefill

def _pplan(lib, d, nb, cus=256):
    p = _lib.DecodePlan()
    st = lib.mlra_prefill_make_plan(ctypes.byref(d), nb, cus, ctypes.byref(p))
    return st, p


@pytest.mark.parametrize("cfg", configs.PREFILL, ids=lambda c: c.name)
def test_prefill_plan_covers_rows_and_tiles(lib, cfg):
    d = _dims(cfg)
    st, p = _pplan(lib, d, cfg.n_branch)
    assert st == 0 and p.kernel_variant == 8 and p.waves_per_group == 8
    rows = cfg.num_heads * cfg.q_len
    assert p.row_groups == -(-rows // 256)
    max_tiles = -(-d.max_seq_len // 64)
    assert p.splits_per_seq * p.tiles_per_split >= max_tiles
    assert (p.splits_per_seq - 1) * p.tiles_per_split < max_tiles
    assert p.target_groups == p.row_groups * cfg.num_seqs * cfg.n_branch * p.splits_per_seq
    assert p.tiles_per_split <= 1024  # a split's block ids are staged in LDS
    assert p.lds_bytes <= 160 * 1024
    direct = p.splits_per_seq == 1 and cfg.n_branch == 1
    if direct:
        assert p.workspace_bytes == 0
    else:
        slots = cfg.num_seqs * p.splits_per_seq * cfg.n_branch * rows
        assert p.workspace_bytes >= slots * (cfg.d_latent + 1) * 4


def test_prefill_plan_splits_only_when_rows_leave_cus_idle(lib):
    cfg = configs.MLRA4_TP_PREFILL
    st, p = _pplan(lib, _dims(cfg), 1)
    assert st == 0 and p.splits_per_seq == 1 and p.target_groups >= 256
    # a 16-token chunk: 2 row groups per sequence, so the context is split
    small = cfg.with_(q_len=16)
    st, p = _pplan(lib, _dims(small), 1)
    assert st == 0 and p.splits_per_seq > 1 and p.tiles_per_split >= 2
    assert p.target_groups >= 128
    d = _dims(small, num_splits=3)
    st, p = _pplan(lib, d, 1)
    assert st == 0 and p.splits_per_seq == 3
    # a split covers at most 1024 tiles even when the rows alone fill the GPU
    d = _dims(cfg.with_(context=2_000_000))
    st, p = _pplan(lib, d, 1)
    assert st == 0 and p.tiles_per_split <= 1024 and p.splits_per_seq == 31
    # CONCAT with one split needs no workspace even with four branches
    d = _dims(cfg.with_(n_branch=4), reduce=_lib.MLRA_BRANCH_CONCAT)
    st, p = _pplan(lib, d, 4)
    assert st == 0 and p.splits_per_seq == 1 and p.workspace_bytes == 0
    size = ctypes.c_size_t(7)
    assert lib.mlra_prefill_workspace_size(ctypes.byref(_dims(cfg)), 1, ctypes.byref(size)) in (0, 6)


@pytest.mark.parametrize("field,value,status", [
    ("q_len", 0, 2), ("num_heads", 0, 2), ("dtype", _lib.MLRA_FP32, 3), ("d_latent", 256, 3),
    ("d_latent", 96, 3), ("d_rope", 48, 3), ("block_size", 32, 3), ("num_seqs", 0, 2),
    ("max_seq_len", -1, 2), ("flags", 2, 2),
])
def test_prefill_rejects_bad_dims(lib, field, value, status):
    d = _dims(configs.MLRA4_TP_PREFILL, **{field: value})
    st, _ = _pplan(lib, d, 1)
    assert st == status, (field, value, st)


def test_prefill_rejects_a_merge_grid_past_the_launch_limit(lib):
    # 1024 sequences x 2^24 rows: 2^27 attention workgroups per branch fit the
    # grid, but a branch sum needs 2^31 merge workgroups (rows x 32 feature
    # groups / 256); one branch writes directly, with no merge, and is planned
    d = _dims(configs.MLRA4_TP_PREFILL, num_seqs=1024, num_heads=1 << 10, q_len=1 << 14)
    st, _ = _pplan(lib, d, 2)
    assert st == 3
    st, p = _pplan(lib, d, 1)
    assert st == 0 and p.workspace_bytes == 0


def test_prefill_rejects_too_many_rows_and_bad_pointers(lib):
    d = _dims(configs.MLRA4_TP_PREFILL, num_heads=1 << 13, q_len=1 << 14)
    st, _ = _pplan(lib, d, 1)
    assert st == 3
    d = _dims(configs.MLRA4_TP_PREFILL)
    # pointer checks come before any device query
    st = lib.mlra_prefill_attention(None, None, None, None, None, None, 1, 0.1, 0.5, None,
                                    None, ctypes.byref(d), None, 0, None)
    assert st == 1
    st = lib.mlra_prefill_attention(16, 16, 16, 16, 16, 16, 1, float("nan"), 0.5, 16, 16,
                                    ctypes.byref(d), None, 0, None)
    assert st == 2
    st = lib.mlra_prefill_attention(16, 16, 16, 16, 16, 16, 1, 0.1, 0.5, 24, 16,
                                    ctypes.byref(d), None, 0, None)
    assert st == 5


@pytest.mark.parametrize("cfg,nb,kw,fused", [
    (configs.MLRA4_TP_SHARE, 1, {"flags": 1}, 1),             # B=16, T=8192: 16 splits x 16
    (configs.MLRA4_FUSED, 4, {"flags": 1}, 1),                # B=32, four branches
    (configs.MLA_COMPARE, 1, {"flags": 1}, 1),
    (configs.MLRA4_TP_SHARE, 1, {}, 0),                       # not asked for
    (configs.MLRA4_TP_SHARE.with_(num_seqs=12), 1, {"flags": 1}, 0),    # not a multiple of 8
    (configs.LONG_CONTEXT, 4, {"flags": 1}, 0),                         # 4 sequences
    (configs.RAGGED_Q2, 4, {"flags": 1, "sum_seq_lens": 64 * 16896}, 0),  # ragged hint
    (configs.MLRA4_TP_SHARE.with_(num_seqs=128, context=512), 1, {"flags": 1}, 0),  # > 64 seqs
])
def test_plan_chooses_the_in_kernel_merge(lib, cfg, nb, kw, fused):
    d = _dims(cfg, **kw)
    st, p = _plan(lib, d, nb)
    assert st == 0
    assert p.fused_merge == fused
    if fused:  # one round of one workgroup per CU, a sequence's workgroups on one XCD
        per = p.splits_per_seq * p.row_groups
        assert cfg.num_seqs % 8 == 0 and cfg.num_seqs * per <= 256 and per <= 32
    rows = cfg.num_heads * cfg.q_len
    slots = cfg.num_seqs * p.splits_per_seq * nb * rows
    assert p.workspace_bytes >= _lib.MLRA_DECODE_WS_HEADER_BYTES + slots * (cfg.d_latent + 1) * 4


def test_status_and_workspace_init_validate_without_a_gpu(lib):
    bits = ctypes.c_uint32(0)
    assert lib.mlra_decode_read_status(None, ctypes.byref(bits), 0, None) == 1
    assert lib.mlra_decode_read_status(24, ctypes.byref(bits), 0, None) == 5
    assert lib.mlra_decode_workspace_init(None, 1 << 20, None) == 1
    assert lib.mlra_decode_workspace_init(16, 100, None) == 4
    assert lib.mlra_decode_workspace_init(24, 1 << 20, None) == 5
    assert lib.mlra_testing_set_wait_limit(-1) == 0
