"""GPU block-sparse attention vs the oracle, element by element at reduced
sizes and on sampled rows at the full workload sizes, plus edge cases and
invariants that need no oracle."""

import math
import random

import numpy as np
import pytest
import torch

from long_context_sparse_block_amd import _lib as L
from long_context_sparse_block_amd import api
from long_context_sparse_block_amd import workloads as wl
from oracle import attention as oa
from oracle import block_mask as bm
from tests.gpu_util import announce, compare, f64, require_gpu, workload_spec

pytestmark = pytest.mark.gpu


def _run(w, spec, B=None, H=None, samples=None, use_schedule=True, seed=None, row_split=1, split_rows=0,
         split_ways=2):
    """Run the GPU path for workload dict w (optionally fewer batch / heads) and
    compare against the oracle (all rows, or the given samples)."""
    B = w["B"] if B is None else B
    H = w["H"] if H is None else H
    dt = wl.torch_dtype(w["dtype"])
    q, k, v = wl.make_qkv(B, H, w["N"], w["d"], dt, w["qkv_seed"] if seed is None else seed)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    mask = api.sparse_attn_build_mask(spec)
    scale = 1.0 / math.sqrt(w["d"])
    mbs, mhs = spec["mask_batch_stride"], spec["mask_head_stride"]
    o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, scale, mbs, mhs, use_schedule=use_schedule,
                                 row_split=row_split, split_rows=split_rows, split_ways=split_ways)
    torch.cuda.synchronize()
    rp, ci, _ = bm.build(spec)
    q64, k64, v64 = f64(q), f64(k), f64(v)
    if samples is None:
        o_ref, l_ref = oa.csr_attention(q64, k64, v64, rp, ci, w["block"], w["causal"], scale, mbs, mhs)
        return compare(o, lse, o_ref, l_ref, dt, w.get("name", ""))
    o_ref, l_ref = oa.csr_attention_rows(q64, k64, v64, rp, ci, w["block"], w["causal"], scale,
                                         samples, mbs, mhs)
    og = torch.stack([o[b, h, t] for b, h, t in samples])
    lg = torch.stack([lse[b, h, t] for b, h, t in samples])
    return compare(og, lg, o_ref, l_ref, dt, "sampled")


def test_tiny_fp32_full_parity():
    require_gpu()
    w = wl.BLOCK_WORKLOADS["tiny-fp32"]
    announce("[bsa] tiny-fp32 [1,1,512,64] fp32")
    _run(w, wl.mask_spec(w))


@pytest.mark.parametrize("name,B,H", [("compression-guided", 4, 2), ("bigbird", 2, 3), ("gzip-guided", 4, 2),
                                      ("gzip-head-groups", 2, 12)])
def test_bf16_reduced_heads_full_parity(name, B, H):
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS[name], name=name)
    announce(f"[bsa] {name} reduced B={B} H={H} N={w['N']}")
    _run(w, workload_spec(dict(w, B=B, H=H)), B=B, H=H)


def test_long_context_reduced_length_full_parity():
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS["long-context"], N=8192, H=2, name="long-context-8k")
    announce("[bsa] long-context d=128 blk=128 reduced N=8192 H=2")
    _run(w, wl.mask_spec(w))


def _samples(B, H, N, block, n, seed):
    R = random.Random(seed)
    out = {(0, 0, 0), (B - 1, H - 1, N - 1), (0, H - 1, block - 1), (B - 1, 0, block)}
    while len(out) < n:
        out.add((R.randrange(B), R.randrange(H), R.randrange(N)))
    return sorted(out)


@pytest.mark.parametrize("name", ["compression-guided", "bigbird", "gzip-guided", "gzip-head-groups",
                                  "long-context"])
def test_full_size_sampled_rows(name):
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS[name], name=name)
    announce(f"[bsa] {name} full size {w['B']}x{w['H']}x{w['N']}x{w['d']} sampled")
    samples = _samples(w["B"], w["H"], w["N"], w["block"], 96, 7)
    _run(w, workload_spec(w), samples=samples)


@pytest.mark.parametrize("name", ["compression-guided"])
def test_anyq_reduced_full_parity(name):
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS[name], name=name + "/anyq")
    announce(f"[bsa] {name} anyq reduced")
    _run(w, wl.mask_spec(dict(w, B=2), literal_mode="anyq"), B=2, H=2)


@pytest.mark.parametrize("d,block,dtype", [(64, 128, "bf16"), (128, 64, "bf16"), (128, 128, "f32"),
                                           (64, 128, "f32"), (128, 64, "f32")])
def test_other_tile_shapes(d, block, dtype):
    require_gpu()
    w = dict(B=2, H=2, N=1024, d=d, block=block, dtype=dtype, causal=True, win_before=1, win_after=0,
             win_clamp=False, global_blocks=[0], num_random=2, literal_mode="pair", literal_p=0.3,
             mask_seed=11, groups="per-sequence", qkv_seed=77, name=f"d{d}b{block}{dtype}")
    announce(f"[bsa] tile d={d} block={block} {dtype}")
    _run(w, wl.mask_spec(w))


def test_noncausal_other_shapes():
    require_gpu()
    for d, block in [(128, 128), (64, 64)]:
        w = dict(B=1, H=2, N=1024, d=d, block=block, dtype="bf16", causal=False, win_before=1,
                 win_after=2, win_clamp=False, global_blocks=[1], num_random=1, literal_mode="anyq",
                 literal_p=0.2, mask_seed=12, groups="shared", qkv_seed=78, name=f"nc d{d}")
        announce(f"[bsa] noncausal d={d} block={block}")
        _run(w, wl.mask_spec(w))


def _hand_mask(rows, nb, causal, device="cuda"):
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.array([c for r in rows for c in r] or [0], dtype=np.int32)
    return api.BlockMask(torch.from_numpy(row_ptr).to(device), torch.from_numpy(col_idx).to(device),
                         None, 1, nb, causal), row_ptr, col_idx[:row_ptr[-1]]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_hand_masks_empty_rows_and_ignored_blocks(dtype):
    """Empty rows give o = 0 and lse = -inf; under causal, listed blocks after the
    query block contribute nothing."""
    require_gpu()
    nb, block, d = 6, 64, 64
    rows = [[], [0, 1, 3, 5], [2], [], [0, 4], [1, 2, 3, 4, 5]]
    for causal in (True, False):
        announce(f"[bsa] hand mask causal={causal} {dtype}")
        mask, rp, ci = _hand_mask(rows, nb, causal)
        q, k, v = wl.make_qkv(1, 2, nb * block, d, dtype, 91)
        o, lse = api.sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask, 0.125)
        torch.cuda.synchronize()
        o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, block, causal, 0.125)
        compare(o, lse, o_ref, l_ref, dtype, f"hand causal={causal}")


def test_out_of_range_columns_are_skipped():
    require_gpu()
    nb, block, d = 4, 64, 64
    rows_bad = [[-3, 0], [0, 1, 99], [2], [0, 3, 7]]
    rows_ok = [[0], [0, 1], [2], [0, 3]]
    mask_bad, _, _ = _hand_mask(rows_bad, nb, True)
    mask_ok, rp, ci = _hand_mask(rows_ok, nb, True)
    q, k, v = [t.cuda() for t in wl.make_qkv(1, 1, nb * block, d, torch.bfloat16, 92)]
    o1, l1 = api.sparse_attn_fwd(q, k, v, mask_bad)
    o2, l2 = api.sparse_attn_fwd(q, k, v, mask_ok)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("row_split,split_rows", [(1, 0), (2, 0), (1, 3)])
def test_gqa_and_strided_inputs(row_split, split_rows):
    """Grouped K/V heads and [B, N, H, d] storage, with and without split rows
    (three parts each)."""
    require_gpu()
    B, H, Hkv, N, d, block = 2, 4, 2, 1024, 64, 64
    spec = dict(num_blocks=N // block, num_groups=1, causal=True, win_before=2, win_after=0,
                win_clamp=False, global_blocks=[0], num_random=1, random_blocks=None,
                literal_mode="pair", literal_flags=None, literal_p=0.3, seed=4,
                mask_batch_stride=0, mask_head_stride=0)
    mask = api.sparse_attn_build_mask(spec)
    q, k, v = wl.make_qkv(B, H, N, d, torch.bfloat16, 93, H_kv=Hkv)
    # strided views: [B, N, H, d] storage seen as [B, H, N, d]
    qs = q.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    ks = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vs = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    announce(f"[bsa] gqa + strided row_split={row_split} split_rows={split_rows}")
    o, lse = api.sparse_attn_fwd(qs, ks, vs, mask, row_split=row_split, split_rows=split_rows, split_ways=3)
    torch.cuda.synchronize()
    rp, ci, _ = bm.build(spec)
    o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, block, True, 1 / math.sqrt(d))
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "gqa strided")


def test_determinism_and_schedule_invariance():
    require_gpu()
    w = wl.BLOCK_WORKLOADS["compression-guided"]
    spec = wl.mask_spec(w)
    mask = api.sparse_attn_build_mask(spec)
    q, k, v = [t.cuda() for t in wl.make_qkv(w["B"], w["H"], w["N"], w["d"], torch.bfloat16, 5)]
    announce("[bsa] determinism / schedule invariance")
    o1, l1 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0)
    o2, l2 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0)
    o3, l3 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0, use_schedule=False)
    # split rows: deterministic as well (a fixed merge order of the two groups)
    o4, l4 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0, row_split=2)
    o5, l5 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0, row_split=2, use_schedule=False)
    # rows split over two workgroups: the same from launch to launch (the two
    # halves merge in a fixed order whichever finishes last)
    ws = api.fwd_workspace(w["B"], w["H"], w["d"], w["block"], 32, 3, q.device)
    o6, l6 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0, split_rows=32, split_ways=3, workspace=ws)
    o7, l7 = api.sparse_attn_fwd(q, k, v, mask, None, 1, 0, split_rows=32, split_ways=3, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(o4, o5) and torch.equal(l4, l5)
    assert torch.equal(o6, o7) and torch.equal(l6, l7)


def test_zero_query_counts_keys():
    """q = 0: lse = ln |K(t)| exactly, which checks the mask cardinality end to end."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["bigbird"]
    spec = wl.mask_spec(w)
    mask = api.sparse_attn_build_mask(spec)
    _, k, v = wl.make_qkv(1, 1, w["N"], w["d"], torch.bfloat16, 6)
    q = torch.zeros_like(k)
    announce("[bsa] zero query")
    o, lse = api.sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask)
    torch.cuda.synchronize()
    rp, ci, _ = bm.build(spec)
    nb, block = spec["num_blocks"], w["block"]
    counts = np.repeat(np.diff(rp).astype(np.float64) * block, block)
    np.testing.assert_allclose(lse[0, 0].cpu().double().numpy(), np.log(counts), atol=1e-6, rtol=0)


def test_unreferenced_blocks_poisoned():
    """Key / value blocks a query block does not list are filled with NaN: that
    query block's outputs stay bitwise unchanged (zero weight outside the mask)."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["compression-guided"]
    spec = wl.mask_spec(dict(w, B=1))
    mask = api.sparse_attn_build_mask(spec)
    rp, ci, _ = bm.build(spec)
    q, k, v = [t.cuda() for t in wl.make_qkv(1, 2, w["N"], w["d"], torch.bfloat16, 7)]
    o1, l1 = api.sparse_attn_fwd(q, k, v, mask)
    nb = spec["num_blocks"]
    for row in (5, 70, nb - 1):
        listed = set(ci[rp[row]:rp[row + 1]].tolist())
        k2, v2 = k.clone(), v.clone()
        for j in range(nb):
            if j not in listed:
                k2[:, :, j * 64:(j + 1) * 64] = float("nan")
                v2[:, :, j * 64:(j + 1) * 64] = float("nan")
        announce(f"[bsa] poison all blocks outside row {row} ({nb - len(listed)} blocks)")
        o2, l2 = api.sparse_attn_fwd(q, k2, v2, mask)
        torch.cuda.synchronize()
        sl = slice(row * 64, (row + 1) * 64)
        assert torch.equal(o1[:, :, sl], o2[:, :, sl]) and torch.equal(l1[:, :, sl], l2[:, :, sl])


@pytest.mark.parametrize("name,B,H", [("bigbird", 2, 3), ("compression-guided", 2, 2), ("gzip-head-groups", 1, 12)])
def test_row_split_reduced_full_parity(name, B, H):
    """Every row's tiles split over two wave groups, merged at the end."""
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS[name], name=name + "/split")
    announce(f"[bsa] row split {name} B={B} H={H}")
    _run(w, workload_spec(dict(w, B=B, H=H)), B=B, H=H, row_split=2)


@pytest.mark.parametrize("d,block", [(64, 128), (128, 64), (128, 128)])
def test_row_split_other_tile_shapes(d, block):
    require_gpu()
    for causal in (True, False):
        w = dict(B=2, H=2, N=1024, d=d, block=block, dtype="bf16", causal=causal, win_before=1,
                 win_after=0 if causal else 1, win_clamp=False, global_blocks=[0], num_random=2,
                 literal_mode="pair", literal_p=0.3, mask_seed=13, groups="per-sequence", qkv_seed=79,
                 name=f"split d{d}b{block} causal={causal}")
        announce(f"[bsa] row split d={d} block={block} causal={causal}")
        _run(w, wl.mask_spec(w), row_split=2)


def test_row_split_hand_masks():
    """Rows of 0, 1 and several tiles (one group then has no tile) and the
    bigbird full size on sampled rows, split over two groups."""
    require_gpu()
    nb, block, d = 6, 64, 64
    rows = [[], [0, 1, 3, 5], [2], [], [0, 4], [1, 2, 3, 4, 5]]
    for causal in (True, False):
        announce(f"[bsa] row split hand mask causal={causal}")
        mask, rp, ci = _hand_mask(rows, nb, causal)
        q, k, v = wl.make_qkv(1, 2, nb * block, d, torch.bfloat16, 93)
        o, lse = api.sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask, 0.125, row_split=2)
        torch.cuda.synchronize()
        o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, block, causal, 0.125)
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"split hand causal={causal}")
    w = dict(wl.BLOCK_WORKLOADS["bigbird"], name="bigbird/split")
    _run(w, workload_spec(w), samples=_samples(w["B"], w["H"], w["N"], w["block"], 64, 8), row_split=2)


# ---- rows split over several workgroups (split_rows, split_ways) ----

def test_split_rows_bigbird_reduced_full_parity():
    """The plan's split of BigBird's global rows (two rows per head, eight
    parts each), every output against the oracle."""
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS["bigbird"], name="bigbird/split-rows")
    spec = workload_spec(dict(w, B=2, H=3))
    sr, ways = api.split_rows_for(spec)
    assert (sr, ways) == (2, 8)
    announce(f"[bsa] split rows bigbird B=2 H=3 split_rows={sr} ways={ways}")
    _run(w, spec, B=2, H=3, split_rows=sr, split_ways=ways)


@pytest.mark.parametrize("name,B,H,ways", [("compression-guided", 4, 2, 2), ("gzip-guided", 4, 2, 3),
                                           ("gzip-head-groups", 2, 12, 4)])
def test_split_rows_causal_reduced_full_parity(name, B, H, ways):
    """Causal masks with their longest eighth of the rows split."""
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS[name], name=name + "/split-rows")
    spec = workload_spec(dict(w, B=B, H=H))
    sr = (spec["num_blocks"] + 7) // 8
    announce(f"[bsa] split rows {name} B={B} H={H} split_rows={sr} ways={ways}")
    _run(w, spec, B=B, H=H, split_rows=sr, split_ways=ways)


def test_split_rows_long_context_reduced_length():
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS["long-context"], N=8192, H=2, name="long-context-8k/split-rows")
    announce("[bsa] split rows long-context N=8192 H=2 split_rows=8 ways=5")
    _run(w, wl.mask_spec(w), split_rows=8, split_ways=5)


@pytest.mark.parametrize("d,block", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_split_rows_tile_shapes(d, block):
    """One split row and every row split, in 2 and 5 parts, causal and not, at
    every tile shape."""
    require_gpu()
    N = 1024
    for causal in (True, False):
        for sr, ways in ((1, 2), (N // block, 5)):
            w = dict(B=2, H=2, N=N, d=d, block=block, dtype="bf16", causal=causal, win_before=1,
                     win_after=0 if causal else 1, win_clamp=False, global_blocks=[0], num_random=2,
                     literal_mode="pair", literal_p=0.3, mask_seed=14, groups="per-sequence", qkv_seed=80,
                     name=f"split-rows d{d}b{block} causal={causal} sr={sr} ways={ways}")
            announce(f"[bsa] split rows d={d} block={block} causal={causal} split_rows={sr} ways={ways}")
            _run(w, wl.mask_spec(w), split_rows=sr, split_ways=ways)


def test_split_rows_hand_masks():
    """Split rows without a launch order (positions are row ids), with rows of
    0, 1 and several tiles: parts may have no tile, or only fully masked ones."""
    require_gpu()
    nb, block, d = 6, 64, 64
    rows = [[], [0, 1, 3, 5], [2], [], [0, 4], [1, 2, 3, 4, 5]]
    for causal in (True, False):
        for sr, ways in ((1, 2), (3, 4), (nb, 2), (nb, 16)):
            announce(f"[bsa] split rows hand mask causal={causal} split_rows={sr} ways={ways}")
            mask, rp, ci = _hand_mask(rows, nb, causal)
            q, k, v = wl.make_qkv(1, 2, nb * block, d, torch.bfloat16, 94)
            o, lse = api.sparse_attn_fwd(q.cuda(), k.cuda(), v.cuda(), mask, 0.125, split_rows=sr, split_ways=ways)
            torch.cuda.synchronize()
            o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, block, causal, 0.125)
            compare(o, lse, o_ref, l_ref, torch.bfloat16, f"split-rows hand causal={causal} sr={sr} ways={ways}")


def test_split_rows_workspace_reuse_and_counters():
    """One workspace over several launches: bit-identical results, every
    counter back at 0 after each launch, and later launches with other split
    shapes on the same workspace still match the oracle."""
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS["bigbird"], name="split-rows reuse")
    B, H = 2, 2
    spec = wl.mask_spec(dict(w, B=B))
    mask = api.sparse_attn_build_mask(spec)
    q, k, v = wl.make_qkv(B, H, w["N"], w["d"], torch.bfloat16, 95)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = api.fwd_workspace(B, H, w["d"], w["block"], 16, 8, qd.device)
    mbs, mhs = spec["mask_batch_stride"], spec["mask_head_stride"]
    announce("[bsa] split rows workspace reuse")
    outs = [api.sparse_attn_fwd(qd, kd, vd, mask, None, mbs, mhs, split_rows=2, split_ways=8, workspace=ws)
            for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    assert torch.all(ws[: B * H * 16 * 4] == 0)
    rp, ci, _ = bm.build(spec)
    o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, w["block"], False, 1 / math.sqrt(w["d"]),
                                    mbs, mhs)
    compare(outs[0][0], outs[0][1], o_ref, l_ref, torch.bfloat16, "split-rows reuse 2x8")
    for sr, ways in ((16, 3), (5, 8)):
        o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, None, mbs, mhs, split_rows=sr, split_ways=ways, workspace=ws)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"split-rows reuse {sr}x{ways}")
        assert torch.all(ws[: B * H * 16 * 4] == 0)


def test_split_rows_workspace_reuse_other_counter_layout():
    """A workspace sized and zeroed for (split_rows 2, 16 ways) reused by a
    launch with more split rows and fewer ways (16 x 2: more counters, as many
    partial states, the same byte count): the counter area has a fixed size,
    so the second launch's counters are not the first launch's partial states,
    and every launch matches the oracle."""
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS["bigbird"], name="split-rows reuse other layout")
    B, H = 2, 3
    spec = wl.mask_spec(dict(w, B=B))
    mask = api.sparse_attn_build_mask(spec)
    q, k, v = wl.make_qkv(B, H, w["N"], w["d"], torch.bfloat16, 96)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    ws = api.fwd_workspace(B, H, w["d"], w["block"], 2, 16, qd.device)
    need = L.lib().sparse_attn_fwd_workspace_bytes(B, H, w["d"], w["block"], 16, 2)
    assert 0 < need <= ws.numel()
    mbs, mhs = spec["mask_batch_stride"], spec["mask_head_stride"]
    rp, ci, _ = bm.build(spec)
    o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, w["block"], False, 1 / math.sqrt(w["d"]),
                                    mbs, mhs)
    for sr, ways in ((2, 16), (16, 2), (2, 16), (16, 2)):
        announce(f"[bsa] split rows workspace {sr}x{ways} after other layouts")
        o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, None, mbs, mhs, split_rows=sr, split_ways=ways, workspace=ws)
        torch.cuda.synchronize()
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"split-rows reuse {sr}x{ways}")
        assert torch.all(ws[: 4 * L.SA_SPLIT_COUNTERS] == 0)


@pytest.mark.parametrize("name", ["bigbird", "compression-guided", "long-context"])
def test_split_rows_full_size_sampled(name):
    """Full workload sizes with split rows (the plan's split for BigBird, the
    longest eighth in two parts otherwise), on sampled rows with the longest
    rows -- the split ones -- included."""
    require_gpu()
    w = dict(wl.BLOCK_WORKLOADS[name], name=name + "/split-rows")
    spec = workload_spec(w)
    sr, ways = api.split_rows_for(spec)
    if sr == 0:
        sr, ways = (spec["num_blocks"] + 7) // 8, 2
    rp, _, sched = bm.build(spec)
    nb = spec["num_blocks"]
    lens = np.diff(np.asarray(rp[: nb + 1]))
    longest = int(np.argmax(lens))
    samples = set(_samples(w["B"], w["H"], w["N"], w["block"], 64, 9))
    samples |= {(0, 0, longest * w["block"]), (0, 0, longest * w["block"] + w["block"] - 1)}
    announce(f"[bsa] split rows {name} full size sampled split_rows={sr} ways={ways}")
    _run(w, spec, samples=sorted(samples), split_rows=sr, split_ways=ways)


def test_bigbird_step_as_captured_graph():
    """The BigBird step (mask build + forward with split rows) captured into a
    HIP graph and replayed several times, with eager work of the library and of
    torch between the replays: every replay equals the eager result bit for
    bit, and the eager result matches the oracle."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["bigbird"]
    B, H = 1, 4
    spec = wl.mask_spec(dict(w, B=B))
    q, k, v = wl.make_qkv(B, H, w["N"], w["d"], torch.bfloat16, 97)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    announce("[bsa] bigbird step as a captured graph")
    plan = api.BlockSparsePlan(spec, qd, kd, vd)
    assert plan.split_rows > 0
    plan()
    torch.cuda.synchronize()
    o_eager, l_eager = plan.o.clone(), plan.lse.clone()
    rp, ci, _ = bm.build(spec)
    o_ref, l_ref = oa.csr_attention(f64(q), f64(k), f64(v), rp, ci, w["block"], False, 1 / math.sqrt(w["d"]))
    compare(o_eager, l_eager, o_ref, l_ref, torch.bfloat16, "bigbird eager")
    g = api.capture_graph(plan)
    other = api.BlockSparsePlan(spec, kd, qd, vd)  # eager work in between, other inputs
    for rep in range(4):
        plan.o.zero_()
        plan.lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.o, o_eager) and torch.equal(plan.lse, l_eager), f"replay {rep}"
        other()
        _ = (qd.float() * 2).sum()
        torch.cuda.synchronize()
