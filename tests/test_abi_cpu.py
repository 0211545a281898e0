"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, matches the binding's struct layout, and rejects bad arguments on the
host before launching anything."""

import ctypes
import os
import re

import numpy as np
import pytest

from long_context_sparse_block_amd import _lib as L
from long_context_sparse_block_amd import api
from oracle import offsets as oo

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sparse_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built")
    return L.lib()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared_functions()
    assert {"sparse_attn_build_mask", "sparse_attn_fwd", "offset_attn_fwd"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, n


def test_mask_desc_layout_matches_binding(lib):
    fields = [f[0] for f in L.MaskDesc._fields_]
    n = lib.sa_mask_desc_layout(None, 0)
    assert n == len(fields) + 1
    out = (ctypes.c_int64 * n)()
    assert lib.sa_mask_desc_layout(out, n) == n
    assert out[0] == ctypes.sizeof(L.MaskDesc)
    for n, name in enumerate(fields):
        assert out[n + 1] == getattr(L.MaskDesc, name).offset, name


def test_status_strings(lib):
    for st in (L.SA_OK, L.SA_ERR_NULL, L.SA_ERR_INVALID, L.SA_ERR_UNSUPPORTED, L.SA_ERR_CAPACITY, L.SA_ERR_HIP):
        assert L.status_string(st)
    assert lib.sa_version() >= 1


def _spec(**kw):
    s = dict(num_blocks=8, num_groups=1, causal=True, win_before=1, win_after=0, win_clamp=False,
             global_blocks=[0], num_random=1, literal_mode="none", literal_p=0.0, seed=1)
    s.update(kw)
    return s


@pytest.mark.parametrize("over,status", [
    (dict(num_blocks=0), L.SA_ERR_INVALID),
    (dict(num_blocks=L.SA_MAX_BLOCKS + 1), L.SA_ERR_INVALID),
    (dict(num_groups=0), L.SA_ERR_INVALID),
    (dict(win_before=-1), L.SA_ERR_INVALID),
    (dict(win_after=1), L.SA_ERR_INVALID),              # causal window may not look ahead
    (dict(global_blocks=[3, 2]), L.SA_ERR_INVALID),     # not ascending
    (dict(global_blocks=[0, 0]), L.SA_ERR_INVALID),     # repeated
    (dict(global_blocks=[8]), L.SA_ERR_INVALID),        # out of range
    (dict(num_random=L.SA_MAX_RANDOM + 1), L.SA_ERR_INVALID),
    (dict(literal_mode="pair", literal_p=1.5), L.SA_ERR_INVALID),
    (dict(causal=False, num_blocks=16384, num_groups=16), L.SA_ERR_UNSUPPORTED),
])
def test_mask_desc_errors(lib, over, status):
    assert api.sparse_attn_check_mask_desc(_spec(**over)) == status


def test_mask_capacity(lib):
    # the largest possible CSR plus one scratch entry per row (row lengths)
    assert api.sparse_attn_mask_capacity(_spec()) == 8 * 9 // 2 + 8
    assert api.sparse_attn_mask_capacity(_spec(causal=False, num_groups=3)) == 3 * 64 + 3 * 8
    assert api.sparse_attn_check_mask_desc(_spec()) == L.SA_OK


def test_build_mask_host_errors(lib):
    d = L.MaskDesc()
    keep = []
    d = api._mask_desc(_spec(), "cpu", keep)
    fake = ctypes.c_void_p(1 << 20)
    # NULL outputs
    assert lib.sparse_attn_build_mask(ctypes.byref(d), None, fake, 100, None, None) == L.SA_ERR_NULL
    # capacity below the bound
    assert lib.sparse_attn_build_mask(ctypes.byref(d), fake, fake, 35, None, None) == L.SA_ERR_CAPACITY
    assert lib.sparse_attn_build_mask(None, fake, fake, 100, None, None) == L.SA_ERR_NULL


def _fwd(lib, **kw):
    fake = ctypes.c_void_p(1 << 20)
    a = dict(dtype=L.SA_BF16, q=fake, k=fake, v=fake, o=fake, lse=fake, B=1, H=2, H_kv=2, N=512,
             d=64, block=64, strides=None, row_ptr=fake, col_idx=fake, cap=100, sched=None, G=1,
             mbs=0, mhs=0, causal=1, scale=0.125, row_split=1, split_rows=0, split_ways=2, ws=None,
             ws_bytes=0)
    a.update(kw)
    return lib.sparse_attn_fwd(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                               a["H_kv"], a["N"], a["d"], a["block"], a["strides"], a["row_ptr"],
                               a["col_idx"], a["cap"], a["sched"], a["G"], a["mbs"], a["mhs"],
                               a["causal"], a["scale"], a["row_split"], a["split_rows"], a["split_ways"],
                               a["ws"], a["ws_bytes"], None)


def _fwd_ws_bytes(B, H, d, block, split_rows, ways):
    """Split-row workspace size: a fixed area of SA_SPLIT_COUNTERS int32
    counters (the same for every split shape), then one partial state per part
    of each split row (per wave of 32 queries and lane: d/2 O^T values, m, l as
    fp32), rounded up to 256 bytes."""
    up = lambda x: (x + 255) // 256 * 256
    if split_rows == 0:
        return 0
    return 4 * L.SA_SPLIT_COUNTERS + up(B * H * split_rows * ways * (block // 32) * 64 * (d // 2 + 2) * 4)


@pytest.mark.parametrize("over,status", [
    (dict(q=None), L.SA_ERR_NULL),
    (dict(row_ptr=None), L.SA_ERR_NULL),
    (dict(dtype=7), L.SA_ERR_INVALID),
    (dict(N=500), L.SA_ERR_INVALID),                 # N % block != 0
    (dict(H=3, H_kv=2), L.SA_ERR_INVALID),
    (dict(d=96), L.SA_ERR_UNSUPPORTED),
    (dict(block=32), L.SA_ERR_UNSUPPORTED),
    (dict(G=1, mhs=1), L.SA_ERR_INVALID),            # head group index out of range
    (dict(causal=2), L.SA_ERR_INVALID),
    (dict(scale=float("nan")), L.SA_ERR_INVALID),
    (dict(row_split=0), L.SA_ERR_INVALID),
    (dict(row_split=3), L.SA_ERR_INVALID),
    (dict(split_rows=-1), L.SA_ERR_INVALID),
    (dict(split_rows=9), L.SA_ERR_INVALID),          # more than N_b = 8 rows
    (dict(split_rows=2, row_split=2), L.SA_ERR_INVALID),
    (dict(split_rows=2), L.SA_ERR_NULL),             # no workspace
    (dict(split_rows=2, ws=ctypes.c_void_p((1 << 20) + 8), ws_bytes=1 << 20), L.SA_ERR_INVALID),
    (dict(split_rows=2, ws=ctypes.c_void_p(1 << 20), ws_bytes=_fwd_ws_bytes(1, 2, 64, 64, 2, 2) - 1),
     L.SA_ERR_CAPACITY),
    (dict(split_rows=2, split_ways=1, ws=ctypes.c_void_p(1 << 20), ws_bytes=1 << 20), L.SA_ERR_INVALID),
    (dict(split_rows=2, split_ways=17, ws=ctypes.c_void_p(1 << 20), ws_bytes=1 << 20), L.SA_ERR_INVALID),
    (dict(cap=-1), L.SA_ERR_INVALID),
    (dict(q=ctypes.c_void_p((1 << 20) + 2)), L.SA_ERR_INVALID),  # misaligned
    (dict(strides=(ctypes.c_int64 * 12)(*([8192 * 64, 8192 * 64, 60] * 4))), L.SA_ERR_INVALID),
    (dict(strides=(ctypes.c_int64 * 12)(*([8192 * 64, 8192 * 64, 68] * 4))), L.SA_ERR_INVALID),
])
def test_fwd_host_errors(lib, over, status):
    assert _fwd(lib, **over) == status


@pytest.mark.parametrize("B,H,d,block,sr,ways", [(1, 2, 64, 64, 0, 2), (1, 2, 64, 64, 2, 2), (4, 8, 64, 64, 16, 3),
                                                (2, 3, 128, 128, 5, 8), (1, 16, 128, 64, 64, 16),
                                                (3, 1, 64, 128, 1, 2)])
def test_fwd_workspace_bytes(lib, B, H, d, block, sr, ways):
    assert lib.sparse_attn_fwd_workspace_bytes(B, H, d, block, sr, ways) == _fwd_ws_bytes(B, H, d, block, sr, ways)


def test_fwd_workspace_bytes_errors(lib):
    assert lib.sparse_attn_fwd_workspace_bytes(0, 1, 64, 64, 1, 2) == L.SA_ERR_INVALID
    assert lib.sparse_attn_fwd_workspace_bytes(1, 1, 64, 64, -1, 2) == L.SA_ERR_INVALID
    assert lib.sparse_attn_fwd_workspace_bytes(1, 1, 64, 64, 1, 1) == L.SA_ERR_INVALID
    assert lib.sparse_attn_fwd_workspace_bytes(1, 1, 64, 64, 1, 17) == L.SA_ERR_INVALID
    assert lib.sparse_attn_fwd_workspace_bytes(1, 1, 96, 64, 1, 2) == L.SA_ERR_UNSUPPORTED
    assert lib.sparse_attn_fwd_workspace_bytes(1, 1, 64, 32, 1, 2) == L.SA_ERR_UNSUPPORTED
    # more split rows than the fixed counter area holds
    assert lib.sparse_attn_fwd_workspace_bytes(4, 8, 64, 64, L.SA_SPLIT_COUNTERS // 32, 2) > 0
    assert lib.sparse_attn_fwd_workspace_bytes(4, 8, 64, 64, L.SA_SPLIT_COUNTERS // 32 + 1, 2) == \
        L.SA_ERR_UNSUPPORTED



def _off(lib, offsets, **kw):
    fake = ctypes.c_void_p(1 << 20)
    a = dict(dtype=L.SA_BF16, B=1, H=1, H_kv=1, N=64, d=64)
    a.update(kw)
    arr = (ctypes.c_int32 * max(1, len(offsets)))(*offsets)
    return lib.offset_attn_fwd(a["dtype"], fake, fake, fake, fake, fake, a["B"], a["H"], a["H_kv"],
                               a["N"], a["d"], None, arr, len(offsets), 0.125, None)


@pytest.mark.parametrize("offsets,over,status", [
    ([], {}, L.SA_ERR_INVALID),
    ([0, 2, 1], {}, L.SA_ERR_INVALID),
    ([0, 1, 1], {}, L.SA_ERR_INVALID),
    ([0, 64], {}, L.SA_ERR_INVALID),
    ([-1, 0], {}, L.SA_ERR_INVALID),
    (list(range(L.SA_MAX_OFFSETS + 1)), dict(N=4096), L.SA_ERR_INVALID),
    ([0, 1], dict(d=32), L.SA_ERR_UNSUPPORTED),
    ([0, 1], dict(H=2, H_kv=3), L.SA_ERR_INVALID),
])
def test_offset_host_errors(lib, offsets, over, status):
    assert _off(lib, offsets, **over) == status


def test_offset_table_matches_oracle(lib):
    for N in (64, 1000, 2048, 8192):
        base = oo.fibonacci_base(N)
        assert api.fibonacci_base(N) == base
        for l in range(16):
            a = 1.0 + l / 15.0
            assert api.offset_attn_make_table(8, a, base, N) == oo.offset_table(8, a, base, N)
    assert api.offset_attn_make_table(0, 0.5, [1, 3], 10) == [0, 1, 2]
    assert api.offset_attn_make_table(3, 1.0, [100], 50) == [0, 1, 2, 3]


def test_offset_table_capacity_error(lib):
    out = (ctypes.c_int32 * 2)()
    cnt = ctypes.c_int32()
    b = (ctypes.c_int64 * 1)(5)
    assert lib.offset_attn_make_table(3, 1.0, b, 1, 100, out, 2, ctypes.byref(cnt)) == L.SA_ERR_CAPACITY


def _off_interp(lib, offsets, rungs, **kw):
    fake = ctypes.c_void_p(1 << 20)
    a = dict(dtype=L.SA_BF16, B=1, H=1, H_kv=1, N=64, d=64)
    a.update(kw)
    arr = (ctypes.c_int32 * max(1, len(offsets)))(*offsets)
    rf = (ctypes.c_int32 * max(1, len(rungs)))(*[r[0] for r in rungs])
    rw = (ctypes.c_float * max(1, len(rungs)))(*[r[1] for r in rungs])
    return lib.offset_attn_fwd_interp(a["dtype"], fake, fake, fake, fake, fake, a["B"], a["H"], a["H_kv"],
                                      a["N"], a["d"], None, arr, len(offsets), rf, rw, len(rungs), 0.125, None)


@pytest.mark.parametrize("offsets,rungs,over,status", [
    ([], [], {}, L.SA_ERR_INVALID),                       # no key at all
    ([0], [(63, 0.5)], {}, L.SA_ERR_INVALID),             # a + 1 > N - 1
    ([0], [(-1, 0.5)], {}, L.SA_ERR_INVALID),
    ([0], [(3, 1.5)], {}, L.SA_ERR_INVALID),              # weight outside [0, 1]
    ([0], [(3, -0.1)], {}, L.SA_ERR_INVALID),
    ([0], [(3, float("nan"))], {}, L.SA_ERR_INVALID),
    ([0], [(1, 0.5)] * (L.SA_MAX_RUNGS + 1), {}, L.SA_ERR_INVALID),
    ([0, 0], [(1, 0.5)], {}, L.SA_ERR_INVALID),
    ([0], [(1, 0.5)], dict(d=32), L.SA_ERR_UNSUPPORTED),
])
def test_offset_interp_host_errors(lib, offsets, rungs, over, status):
    assert _off_interp(lib, offsets, rungs, **over) == status


def test_offset_ratio_table_matches_oracle(lib):
    fib15 = oo.fibonacci_base(1000)
    for N in (64, 1024, 4096):
        for l in range(16):
            num, den = 15 + 2 * l, 30
            assert api.offset_attn_make_table_ratio(8, num, den, fib15, N) == oo.offset_table_ratio(8, num, den, fib15, N)
        for base in (oo.fibonacci_base(N), oo.power2_base(N)):
            assert api.offset_attn_make_table_ratio(8, 7, 5, base, N) == oo.offset_table_ratio(8, 7, 5, base, N)
    assert api.power2_base(1024) == oo.power2_base(1024)
    b = (ctypes.c_int64 * 1)(5)
    out = (ctypes.c_int32 * 8)()
    cnt = ctypes.c_int32()
    assert lib.offset_attn_make_table_ratio(3, 1, 0, b, 1, 100, out, 8, ctypes.byref(cnt)) == L.SA_ERR_INVALID
    assert lib.offset_attn_make_table_ratio(3, -1, 2, b, 1, 100, out, 8, ctypes.byref(cnt)) == L.SA_ERR_INVALID
    assert lib.offset_attn_make_table_ratio(3, 1, 1, b, 1, 100, out, 2, ctypes.byref(cnt)) == L.SA_ERR_CAPACITY


def test_offset_interp_split_matches_oracle(lib):
    for N in (64, 300, 2048):
        for base in (oo.fibonacci_base(N), oo.power2_base(N)):
            for alpha in (0.5, 0.73, 1.0, 1.0 + 1e-3, 1.37, 2.0, -1.0):
                ints, rungs = api.offset_attn_make_interp(8, alpha, base, N)
                oi, orr = oo.interp_split(8, alpha, base, N)
                assert ints == oi
                assert [a for a, _ in rungs] == [a for a, _ in orr]
                assert [w for _, w in rungs] == [float(np.float32(w)) for _, w in orr]
                if alpha == int(alpha) and alpha > 0:
                    assert rungs == [] and ints == api.offset_attn_make_table(8, alpha, base, N)
    b = (ctypes.c_int64 * 2)(3, 5)
    out = (ctypes.c_int32 * 8)()
    rf = (ctypes.c_int32 * 1)()
    rw = (ctypes.c_float * 1)()
    cnt, rc = ctypes.c_int32(), ctypes.c_int32()
    assert lib.offset_attn_make_interp(1, 1.5, b, 2, 100, out, 8, ctypes.byref(cnt), rf, rw, 1,
                                       ctypes.byref(rc)) == L.SA_ERR_CAPACITY


def _bwd(lib, **kw):
    fake = ctypes.c_void_p(1 << 20)
    a = dict(dtype=L.SA_BF16, ws=fake, ws_bytes=1 << 40, B=1, H=2, H_kv=2, N=512, d=64, block=64,
             strides=None, G=1, mbs=0, mhs=0, causal=1, scale=0.125)
    a.update(kw)
    return lib.sparse_attn_bwd(a["dtype"], fake, fake, fake, fake, fake, fake, fake, fake, fake, a["ws"],
                               a["ws_bytes"], a["B"], a["H"], a["H_kv"], a["N"], a["d"], a["block"],
                               a["strides"], fake, fake, 100, None, fake, fake, 100, a["G"], a["mbs"], a["mhs"],
                               a["causal"], a["scale"], None)


def _bwd_strides(seq_q):
    """Per-tensor (batch, head, sequence) strides of q, k, v, o, dout, dq, dk, dv."""
    s = []
    for t in range(8):
        ss = seq_q if t == 0 else 64
        s += [2 * 512 * ss, 512 * ss, ss]
    return (ctypes.c_int64 * 24)(*s)


@pytest.mark.parametrize("over,status", [
    (dict(ws=None), L.SA_ERR_NULL),
    (dict(ws_bytes=0), L.SA_ERR_CAPACITY),
    (dict(ws=ctypes.c_void_p((1 << 20) + 4)), L.SA_ERR_INVALID),  # misaligned workspace
    (dict(d=96), L.SA_ERR_UNSUPPORTED),
    (dict(block=32), L.SA_ERR_UNSUPPORTED),
    (dict(N=500), L.SA_ERR_INVALID),
    (dict(causal=2), L.SA_ERR_INVALID),
    (dict(G=1, mhs=1), L.SA_ERR_INVALID),
    # bf16: row byte offsets of a 64-row tile are kept in 32 bits
    (dict(strides=_bwd_strides(1 << 24)), L.SA_ERR_UNSUPPORTED),
])
def test_bwd_host_errors(lib, over, status):
    assert _bwd(lib, **over) == status


def test_bwd_workspace_bytes(lib):
    # {lse log2(e), D} per row | work-item prefix and chunk size | fp32 partial dK, dV;
    # parts 256-byte aligned
    up = lambda x: (x + 255) // 256 * 256
    for B, H, Hkv, N, d, blk in ((1, 2, 2, 512, 64, 64), (2, 8, 2, 4096, 128, 128), (3, 3, 1, 192, 64, 64)):
        want = up(8 * B * H * N) + up(4 * (B * Hkv * (N // blk) + 2)) + up(2 * 4 * B * Hkv * N * d)
        assert lib.sparse_attn_bwd_workspace_bytes(B, H, Hkv, N, d, blk) == want
    assert lib.sparse_attn_bwd_workspace_bytes(0, 1, 1, 64, 64, 64) < 0


def test_plan_picks_row_split():
    """Whole rows per workgroup everywhere (long rows are split across
    workgroups instead, see test_plan_picks_split_rows)."""
    from long_context_sparse_block_amd import api
    from long_context_sparse_block_amd import workloads as wl
    for name in ("bigbird", "compression-guided", "long-context", "gzip-guided", "tiny-fp32"):
        assert api.row_split_for(wl.mask_spec(wl.BLOCK_WORKLOADS[name])) == 1


def test_plan_picks_split_rows():
    """The global rows of non-causal masks with global blocks are split into
    parts about as long as an ordinary row; nothing is split otherwise."""
    from long_context_sparse_block_amd import api
    from long_context_sparse_block_amd import workloads as wl
    spec = lambda n: wl.mask_spec(wl.BLOCK_WORKLOADS[n])
    assert api.split_rows_for(spec("bigbird")) == (2, 8)        # 64 blocks, 3 + 2 + 3 per ordinary row
    assert api.split_rows_for(spec("bigbird"), row_split=2) == (0, 2)
    for name in ("compression-guided", "long-context", "gzip-guided"):
        assert api.split_rows_for(spec(name)) == (0, 2)
    assert api.split_rows_for(api.mask_preset("local-only", 64, causal=False)) == (0, 2)
    # 8 global blocks, +-4 window: ordinary rows 9 + 8 blocks -> ceil(64 / 17) = 4 parts
    assert api.split_rows_for(api.mask_preset("longformer", 64, causal=False)) == (8, 4)
    # 64 global blocks: ordinary rows 9 + 64 -> ceil(512 / 73) = 8 parts
    assert api.split_rows_for(api.mask_preset("longformer", 512, causal=False)) == (64, 8)


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus above 1 prints one JSON line that says
    so and exits with status 2 before touching a device."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], cwd=root,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_library_rng_known_answer_vectors(lib):
    """The library's draws, run on the host by the same inline code the mask
    kernels run (sa_rng_*), reproduce the frozen vectors written from the
    oracle."""
    from tests.test_oracle_masks import read_rng_vectors
    keys, lits, draws = read_rng_vectors()
    for (s, t, a, b, c), want in keys:
        assert lib.sa_rng_key(s, t, a, b, c) == want
    for (s, g, j, p), want in lits:
        assert lib.sa_rng_literal(s, g, j, p) == want
    for (s, g, i, n, r), want in draws:
        out = (ctypes.c_int32 * max(1, r))()
        cnt = lib.sa_rng_random_blocks(s, g, i, n, r, out)
        assert cnt == len(want) and list(out[:cnt]) == want


def test_library_rng_matches_oracle_on_workloads(lib):
    """Every drawn literal flag of the compression-guided and long-context
    masks and every random draw of the BigBird mask, library host path vs
    oracle; argument errors of the draw entry point."""
    from long_context_sparse_block_amd import workloads as wl
    from oracle import rng
    for name in ("compression-guided", "long-context"):
        w = wl.BLOCK_WORKLOADS[name]
        G = w["B"] if w["groups"] == "per-sequence" else 1
        nb = w["N"] // w["block"]
        for g in range(G):
            got = [lib.sa_rng_literal(w["mask_seed"], g, j, w["literal_p"]) for j in range(nb)]
            assert got == [rng.literal_flag(w["mask_seed"], g, j, w["literal_p"]) for j in range(nb)], name
    w = wl.BLOCK_WORKLOADS["bigbird"]
    nb, r = w["N"] // w["block"], w["num_random"]
    out = (ctypes.c_int32 * r)()
    for i in range(nb):
        cnt = lib.sa_rng_random_blocks(w["mask_seed"], 0, i, nb, r, out)
        assert list(out[:cnt]) == rng.random_blocks(w["mask_seed"], 0, i, nb, r)
    assert lib.sa_rng_random_blocks(1, 0, 0, 4, 2, None) == L.SA_ERR_NULL
    assert lib.sa_rng_random_blocks(1, 0, 0, -1, 2, out) == L.SA_ERR_INVALID
    assert lib.sa_rng_random_blocks(1, 0, 0, 4, L.SA_MAX_RANDOM + 1, out) == L.SA_ERR_INVALID


def test_noalloc_rejects_oversized_split_before_anything(lib):
    """sparse_attn_fwd_noalloc refuses a split whose workspace exceeds its
    static scratch with SA_ERR_CAPACITY, and bad arguments as sparse_attn_fwd
    does, on the host (fake device pointers are never touched)."""
    fake = ctypes.c_void_p(1 << 20)
    def call(**kw):
        a = dict(dtype=L.SA_BF16, B=1, H=16, N=8192, d=128, block=128, split_rows=64, split_ways=16, causal=1)
        a.update(kw)
        return lib.sparse_attn_fwd_noalloc(a["dtype"], fake, fake, fake, fake, fake, a["B"], a["H"], a["H"], a["N"],
                                           a["d"], a["block"], None, fake, fake, 1 << 20, None, 1, 0, 0, a["causal"],
                                           0.1, 1, a["split_rows"], a["split_ways"], None)
    assert lib.sparse_attn_fwd_workspace_bytes(1, 16, 128, 128, 64, 16) > L.SA_NOALLOC_SCRATCH_BYTES
    assert call() == L.SA_ERR_CAPACITY
    assert call(split_ways=1) == L.SA_ERR_INVALID
    assert call(causal=2, split_rows=0) == L.SA_ERR_INVALID
    assert call(d=96, split_rows=0) == L.SA_ERR_UNSUPPORTED
