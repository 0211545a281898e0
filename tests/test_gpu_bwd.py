"""GPU backward passes vs the fp64 oracle gradients: the block-mask transpose
(bit-exact), block-sparse dq / dk / dv (fp32 and bf16, GQA, per-head mask
groups, strided layouts, reduced and full-size workloads) and offset dq / dk /
dv.

Bars for gradients (derived from the arithmetic).  Each gradient entry is a
sum of terms; M is the same sum with every factor taken in absolute value
(oracle term magnitudes, D_t counted as sum |dO_tx| |o_tx|).  bf16 path: the
forward's lse is accurate to 2^-9 (its normaliser sums bf16-rounded weights),
so every recomputed weight p is off by up to 2^-9 relative; P and dS enter the
MFMAs rounded to bf16 (2^-9); D_t is formed from the stored bf16 o (2^-9 of
its magnitude); the output is rounded to bf16 (2^-9 of the entry).  Hence
|g - ref| <= 2^-7 M + 2^-8 |ref| per entry, and the mean error stays below
2^-8 mean(M).  fp32 path: |g - ref| <= 1e-5 (M + |ref|) + 1e-7 (fp32 rounding
of the exp2 argument, about 1e-6 of every weight)."""

import math
import random

import numpy as np
import pytest
import torch

from long_context_sparse_block_amd import api
from long_context_sparse_block_amd import workloads as wl
from oracle import backward as ob
from oracle import block_mask as bm
from oracle import offsets as oo
from tests.gpu_util import announce, f64, require_gpu, workload_spec

pytestmark = pytest.mark.gpu


def compare_grads(gpu, ref, mag, dtype, what):
    g = f64(gpu)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    diff = np.abs(g - ref)
    if dtype == torch.bfloat16:
        lim = 2.0 ** -7 * mag + 2.0 ** -8 * np.abs(ref) + 1e-6
        assert diff.mean() <= 2.0 ** -8 * mag.mean() + 1e-7, f"{what}: mean-abs {diff.mean():.3e} vs mean M {mag.mean():.3e}"
    else:
        lim = 1e-5 * (mag + np.abs(ref)) + 1e-7
    bad = int(np.argmax(diff - lim))
    assert np.all(diff <= lim), (f"{what}: |err| {diff.flat[bad]:.3e} > bar {lim.flat[bad]:.3e} "
                                 f"(|ref| {abs(ref.flat[bad]):.3e}, index {np.unravel_index(bad, ref.shape)})")
    return float(np.max(diff / lim))


def _dout(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def _bsa_case(spec, B, H, Hkv, N, d, dtype, seed, scale=None, heads=None, layout=None):
    block = N // spec["num_blocks"]
    q, k, v = wl.make_qkv(B, H, N, d, dtype, seed, H_kv=Hkv)
    do = _dout(q.shape, dtype, seed + 1)
    if layout == "bnhd":  # [B, N, H, d] storage viewed as [B, H, N, d]
        q, k, v, do = [t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v, do)]
    qd, kd, vd, dod = [t.cuda() for t in (q, k, v, do)]
    mask = api.sparse_attn_build_mask(spec)
    mbs, mhs = spec["mask_batch_stride"], spec["mask_head_stride"]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, scale, mbs, mhs)
    dq, dk, dv = api.sparse_attn_bwd(qd, kd, vd, o, lse, dod, mask, None, scale, mbs, mhs)
    torch.cuda.synchronize()
    rp, ci, _ = bm.build(spec)
    ref = ob.csr_attention_bwd(f64(q), f64(k), f64(v), f64(do), rp, ci, block, spec["causal"], scale, mbs, mhs,
                               heads=heads, mags=True)
    return (dq, dk, dv), ref


def _check_all(got, ref, dtype, what, heads=None):
    (gq, gk, gv), (mq, mk, mv) = ref
    for n, gt, rf, mg in zip(("dq", "dk", "dv"), got, (gq, gk, gv), (mq, mk, mv)):
        if heads is not None:
            gt = torch.stack([gt[b, h] for b, h in heads])
            rf = np.stack([rf[b, h] for b, h in heads])
            mg = np.stack([mg[b, h] for b, h in heads])
        compare_grads(gt, rf, mg, dtype, f"{what} {n}")


def _specs():
    out = []
    for name in ("compression-guided", "bigbird", "long-context", "gzip-head-groups"):
        w = wl.BLOCK_WORKLOADS[name]
        out.append((name, workload_spec(dict(w, B=min(w["B"], 2)))))
    R = random.Random(3)
    for s in range(4):
        nb = R.randint(1, 40)
        causal = s % 2 == 0
        out.append((f"random{s}", dict(num_blocks=nb, num_groups=3, causal=causal, win_before=R.randint(0, 3),
                                       win_after=0 if causal else 1, win_clamp=True,
                                       global_blocks=[0] if nb > 1 else [], num_random=2, random_blocks=None,
                                       literal_mode="pair", literal_flags=None, literal_p=0.3, seed=s,
                                       mask_batch_stride=1, mask_head_stride=0)))
    return out


def test_mask_transpose_bitexact():
    require_gpu()
    for name, spec in _specs():
        announce(f"[bwd] transpose {name}")
        mask = api.sparse_attn_build_mask(spec)
        col_ptr, row_idx = api.sparse_attn_mask_transpose(mask)
        torch.cuda.synchronize()
        m = bm.block_mask(spec)
        cp_ref, ri_ref = bm.to_csr(np.transpose(m, (0, 2, 1)))
        assert np.array_equal(col_ptr.cpu().numpy(), cp_ref), name
        n = int(cp_ref[-1])
        assert np.array_equal(row_idx[:n].cpu().numpy(), ri_ref), name


def test_bsa_bwd_fp32_tiny_workload():
    require_gpu()
    w = wl.BLOCK_WORKLOADS["tiny-fp32"]
    announce("[bwd] bsa fp32 tiny workload")
    got, ref = _bsa_case(wl.mask_spec(w), w["B"], w["H"], w["H"], w["N"], w["d"], torch.float32, w["qkv_seed"])
    _check_all(got, ref, torch.float32, "tiny")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,block", [(64, 64), (64, 128), (128, 64), (128, 128)])
def test_bsa_bwd_gqa_head_groups(dtype, d, block):
    """GQA (4 q heads on 2 K/V heads) with one mask group per q head, causal
    and non-causal, rows whose only entries lie in the future."""
    require_gpu()
    N = 8 * block
    for causal in (True, False):
        spec = dict(num_blocks=N // block, num_groups=4, causal=causal, win_before=1, win_after=0 if causal else 1,
                    win_clamp=True, global_blocks=[0], num_random=2, random_blocks=None, literal_mode="anyq",
                    literal_flags=None, literal_p=0.3, seed=11, mask_batch_stride=0, mask_head_stride=1)
        announce(f"[bwd] bsa gqa {dtype} d={d} block={block} causal={causal}")
        got, ref = _bsa_case(spec, 2, 4, 2, N, d, dtype, 40 + d + block)
        _check_all(got, ref, dtype, f"gqa d={d} b={block} causal={causal}")


@pytest.mark.parametrize("name,B,H", [("compression-guided", 2, 2), ("bigbird", 1, 3), ("long-context", 1, 2),
                                      ("gzip-head-groups", 1, 12)])
def test_bsa_bwd_bf16_reduced_workloads(name, B, H):
    require_gpu()
    w = wl.BLOCK_WORKLOADS[name]
    N = w["N"] if name != "long-context" else 8192
    w = dict(w, B=B, H=H, N=N)
    spec = workload_spec(w)
    announce(f"[bwd] bsa {name} B={B} H={H} N={N}")
    got, ref = _bsa_case(spec, B, H, H, N, w["d"], torch.bfloat16, w["qkv_seed"])
    _check_all(got, ref, torch.bfloat16, name)


def test_bsa_bwd_bf16_launch_order():
    """The dQ rows run in the mask's longest-first order or in ascending
    order (sched NULL): each dq row is one workgroup's sum in a fixed order, so
    dq agrees bit for bit; dk / dv come from the same kernel either way and
    both results meet the oracle's bar."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["compression-guided"]
    w = dict(w, B=2, H=4)
    spec = workload_spec(w)
    announce("[bwd] bsa launch order, compression-guided B=2 H=4")
    q, k, v = wl.make_qkv(2, 4, w["N"], w["d"], torch.bfloat16, 31)
    do = _dout(q.shape, torch.bfloat16, 32)
    qd, kd, vd, dod = [t.cuda() for t in (q, k, v, do)]
    mask = api.sparse_attn_build_mask(spec)
    mbs, mhs = spec["mask_batch_stride"], spec["mask_head_stride"]
    scale = 1.0 / math.sqrt(w["d"])
    o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, scale, mbs, mhs)
    got = [api.sparse_attn_bwd(qd, kd, vd, o, lse, dod, mask, None, scale, mbs, mhs, use_schedule=u)
           for u in (True, False)]
    torch.cuda.synchronize()
    assert torch.equal(got[0][0], got[1][0]), "dq depends on the launch order"
    rp, ci, _ = bm.build(spec)
    ref = ob.csr_attention_bwd(f64(q), f64(k), f64(v), f64(do), rp, ci, w["N"] // spec["num_blocks"],
                               spec["causal"], scale, mbs, mhs, mags=True)
    for n, g in zip(("sched", "ascending"), got):
        _check_all(g, ref, torch.bfloat16, f"launch order {n}")


def test_bsa_bwd_bf16_strided_negative_scale():
    require_gpu()
    w = wl.BLOCK_WORKLOADS["bigbird"]
    spec = workload_spec(dict(w, B=1))
    announce("[bwd] bsa strided [B,N,H,d], scale -0.1")
    got, ref = _bsa_case(spec, 1, 4, 4, w["N"], 64, torch.bfloat16, 77, scale=-0.1, layout="bnhd")
    _check_all(got, ref, torch.bfloat16, "strided")


def test_bsa_bwd_bf16_full_size_sampled_heads():
    """The headline workload at full size; whole (batch, head) slices checked."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["compression-guided"]
    heads = [(0, 0), (w["B"] - 1, w["H"] - 1), (2, 5)]
    announce(f"[bwd] bsa compression-guided full {w['B']}x{w['H']}x{w['N']}")
    got, ref = _bsa_case(workload_spec(w), w["B"], w["H"], w["H"], w["N"], w["d"], torch.bfloat16, w["qkv_seed"],
                         heads=heads)
    _check_all(got, ref, torch.bfloat16, "full", heads=heads)


def _off_case(offs, B, H, Hkv, N, d, dtype, seed, scale, offs_ref=None):
    """Offset backward on the GPU over ``offs`` and the oracle's gradients over
    ``offs_ref`` (the oracle's own table; default ``offs``)."""
    offs_ref = offs if offs_ref is None else offs_ref
    q, k, v = wl.make_qkv(B, H, N, d, dtype, seed, H_kv=Hkv)
    do = _dout(q.shape, dtype, seed + 1)
    qd, kd, vd, dod = [t.cuda() for t in (q, k, v, do)]
    o, lse = api.offset_attn_fwd(qd, kd, vd, offs, scale)
    got = api.offset_attn_bwd(qd, kd, vd, o, lse, dod, offs, scale)
    torch.cuda.synchronize()
    ref = ob.offset_attention_bwd(f64(q), f64(k), f64(v), f64(do), offs_ref, scale, mags=True)
    return got, ref


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
def test_offset_bwd_ragged_gqa(dtype, d):
    require_gpu()
    for N, Hkv in ((1, 2), (63, 1), (300, 2), (1000, 1)):
        offs = api.offset_attn_make_table(5, 1.3, api.fibonacci_base(N), N)
        offs_ref = oo.offset_table(5, 1.3, oo.fibonacci_base(N), N)
        announce(f"[bwd] offsets N={N} d={d} {dtype} H_kv={Hkv}")
        got, ref = _off_case(offs, 2, 2, Hkv, N, d, dtype, 600 + N, 0.2, offs_ref)
        _check_all(got, ref, dtype, f"offsets N={N}")


def test_offset_bwd_no_self_distance():
    """Table without distance 0: the first queries have no key (lse = -inf)."""
    require_gpu()
    got, ref = _off_case([3, 7, 20], 1, 2, 2, 200, 64, torch.bfloat16, 650, 0.3)
    _check_all(got, ref, torch.bfloat16, "no self")


def test_offset_bwd_workload_reduced_batch():
    require_gpu()
    ow = wl.OFFSET_WORKLOAD
    for N in ow["lengths"]:
        offs = api.offset_attn_make_table(ow["W"], ow["alphas"][7], api.fibonacci_base(N), N)
        offs_ref = oo.offset_table(ow["W"], ow["alphas"][7], oo.fibonacci_base(N), N)
        announce(f"[bwd] offsets workload N={N} B=1 H=2")
        got, ref = _off_case(offs, 1, 2, 2, N, ow["d"], torch.bfloat16, ow["qkv_seed_base"][N] + 7,
                             1 / math.sqrt(ow["d"]), offs_ref)
        _check_all(got, ref, torch.bfloat16, f"offsets workload N={N}")


def _hand_mask(rows, nb, causal):
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.array([c for r in rows for c in r] or [0], dtype=np.int32)
    return api.BlockMask(torch.from_numpy(row_ptr).cuda(), torch.from_numpy(col_idx).cuda(), None, 1, nb,
                         causal), row_ptr, col_idx[:row_ptr[-1]]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_bsa_bwd_hand_masks_empty_and_ignored(dtype):
    """Empty rows and empty columns give zero gradients; entries out of range or
    (causal) after the query block are skipped: the gradients equal those of
    the clean mask bit for bit, and the oracle's for it."""
    require_gpu()
    nb, block, d, scale = 6, 64, 64, 0.125
    rows_ok = [[], [0, 1, 3, 5], [2], [], [0, 4], [1, 2, 4, 5]]
    rows_bad = [[-2], [0, 1, 3, 5, 9], [2, 4], [], [0, 4, 5], [1, 2, 4, 5, 77]]
    for causal in (True, False):
        announce(f"[bwd] hand masks causal={causal} {dtype}")
        # non-causal: every in-range entry counts, only the out-of-range ones go
        bad = rows_bad
        ok = rows_ok if causal else [[c for c in r if 0 <= c < nb] for r in rows_bad]
        q, k, v = wl.make_qkv(1, 2, nb * block, d, dtype, 95)
        do = _dout(q.shape, dtype, 96)
        qd, kd, vd, dod = [t.cuda() for t in (q, k, v, do)]
        grads = []
        for rows in (bad, ok):
            mask, rp, ci = _hand_mask(rows, nb, causal)
            o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, scale)
            grads.append(api.sparse_attn_bwd(qd, kd, vd, o, lse, dod, mask, None, scale))
        torch.cuda.synchronize()
        for x, y, n in zip(grads[0], grads[1], ("dq", "dk", "dv")):
            assert torch.equal(x, y), f"{n}: skipped entries changed the result"
        _, rp, ci = _hand_mask(ok, nb, causal)
        (gq, gk, gv), mags = ob.csr_attention_bwd(f64(q), f64(k), f64(v), f64(do), rp, ci, block, causal, scale,
                                                   mags=True)
        _check_all(grads[1], ((gq, gk, gv), mags), dtype, f"hand causal={causal}")
        # query block 3 lists nothing: its dq rows are zero; key block 3 is listed
        # by no usable row when causal
        assert torch.count_nonzero(grads[1][0][:, :, 3 * block:4 * block]) == 0
        if causal:
            assert torch.count_nonzero(grads[1][1][:, :, 3 * block:4 * block]) == 0


@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1)])
def test_bsa_bwd_bf16_split_columns_block64(H, Hkv):
    """Key block 0 is global: listed by all 70 query blocks (of every q head of a
    K/V head), more than one work item holds at block 64, so its dK / dV rows
    are summed from several workgroups' fp32 partials."""
    require_gpu()
    nb, block, d = 70, 64, 64
    spec = dict(num_blocks=nb, num_groups=1, causal=True, win_before=1, win_after=0, win_clamp=False,
                global_blocks=[0], num_random=0, random_blocks=None, literal_mode="none", literal_flags=None,
                literal_p=0.0, seed=0, mask_batch_stride=0, mask_head_stride=0)
    announce(f"[bwd] split columns H={H} Hkv={Hkv}")
    got, ref = _bsa_case(spec, 1, H, Hkv, nb * block, d, torch.bfloat16, 97)
    _check_all(got, ref, torch.bfloat16, f"split columns H={H} Hkv={Hkv}")


def _long_rows(nb, causal, lo, seed, every=1):
    """Hand CSR rows: every ``every``-th row lists between ``lo`` and all of its
    allowed key blocks (more than one 64-entry pass of the dQ walk), the other
    rows 1 to 4; entries ascending and unique, at random positions."""
    R = np.random.default_rng(seed)
    rows = []
    for i in range(nb):
        n_allowed = i + 1 if causal else nb
        want = int(R.integers(lo, nb + 1)) if i % every == 0 else int(R.integers(1, 5))
        k = min(n_allowed, want)
        rows.append(sorted(int(c) for c in R.choice(n_allowed, size=k, replace=False)))
    return rows


@pytest.mark.parametrize("dtype,d,block,nb,H,Hkv", [
    (torch.bfloat16, 64, 64, 140, 2, 1),
    (torch.bfloat16, 128, 64, 140, 1, 1),
    (torch.bfloat16, 64, 128, 80, 2, 1),
    (torch.bfloat16, 128, 128, 80, 1, 1),
    (torch.float32, 64, 64, 140, 1, 1),
    (torch.float32, 128, 128, 80, 1, 1),
])
def test_bsa_bwd_rows_longer_than_one_pass(dtype, d, block, nb, H, Hkv):
    """Rows of 65 to nb key blocks: the dQ walk takes a row's list in passes of
    64 entries (two passes above 64, three above 128 at 140 blocks), and the
    transposed columns, listed by up to nb query blocks of each q head, are
    split into several dK / dV work items.  Causal and non-causal, element by
    element against the oracle's gradients."""
    require_gpu()
    N = nb * block
    for causal in (False, True):
        rows = _long_rows(nb, causal, 65, 500 + nb + d + block, every=1 if block == 64 else 4)
        longest = max(len(r) for r in rows)
        assert longest > 64
        announce(f"[bwd] long rows {dtype} d={d} block={block} nb={nb} H={H}/{Hkv} causal={causal} "
                 f"longest={longest}")
        q, k, v = wl.make_qkv(1, H, N, d, dtype, 900 + d + block, H_kv=Hkv)
        do = _dout(q.shape, dtype, 901 + d + block)
        qd, kd, vd, dod = [t.cuda() for t in (q, k, v, do)]
        mask, rp, ci = _hand_mask(rows, nb, causal)
        scale = 1.0 / math.sqrt(d)
        o, lse = api.sparse_attn_fwd(qd, kd, vd, mask, scale)
        got = api.sparse_attn_bwd(qd, kd, vd, o, lse, dod, mask, None, scale)
        torch.cuda.synchronize()
        ref = ob.csr_attention_bwd(f64(q), f64(k), f64(v), f64(do), rp, ci, block, causal, scale, mags=True)
        _check_all(got, ref, dtype, f"long rows d={d} b={block} causal={causal}")


def test_bsa_bwd_long_context_full_size_sampled_heads():
    """The long-context workload at full size ([1, 16, 65536, 128], block 128),
    run as the bench runs it; whole heads 0 and 15 checked against the oracle.
    19 of its 512 rows list 65 to 83 key blocks (a second dQ pass) and the four
    global key blocks are listed by every later query block (split over eight
    dK / dV work items each: this size gets 64 entries per item)."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["long-context"]
    spec = workload_spec(w)
    rp, ci, _ = bm.build(spec)
    assert int(np.diff(rp).max()) > 64
    sel = [0, w["H"] - 1]
    announce(f"[bwd] long-context full size {w['B']}x{w['H']}x{w['N']}x{w['d']}, heads {sel}")
    q, k, v = wl.make_qkv(w["B"], w["H"], w["N"], w["d"], torch.bfloat16, w["qkv_seed"])
    do = _dout(q.shape, torch.bfloat16, w["qkv_seed"] + 1)
    plan = api.BlockSparsePlan(spec, q.cuda(), k.cuda(), v.cuda())
    plan()
    bp = api.BlockSparseBwdPlan(plan, do.cuda())
    got = bp()
    torch.cuda.synchronize()
    assert np.array_equal(plan.mask.row_ptr.cpu().numpy(), rp)
    got = [t[:, sel] for t in got]
    scale = 1.0 / math.sqrt(w["d"])
    qs, ks, vs, ds = [f64(t[:, sel]) for t in (q, k, v, do)]
    ref = ob.csr_attention_bwd(qs, ks, vs, ds, rp, ci, w["block"], True, scale, mags=True)
    _check_all(got, ref, torch.bfloat16, "long-context full size")


def test_bsa_bwd_bigbird_full_size_sampled_heads():
    """The BigBird workload at full size ([2, 12, 4096, 64], non-causal, block
    64), run as the bench runs it: the two global key blocks are listed by all
    64 query blocks of a head, so their columns are split over four dK / dV
    work items (16 entries each at this size) whose fp32 partials meet in the
    workspace; three whole (batch, head) slices checked against the oracle."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["bigbird"]
    spec = workload_spec(w)
    rp, ci, _ = bm.build(spec)
    assert spec["mask_batch_stride"] == 0 and spec["mask_head_stride"] == 0  # one mask for every head
    heads = [(0, 0), (1, 5), (w["B"] - 1, w["H"] - 1)]
    announce(f"[bwd] bigbird full size {w['B']}x{w['H']}x{w['N']}x{w['d']}, heads {heads}")
    q, k, v = wl.make_qkv(w["B"], w["H"], w["N"], w["d"], torch.bfloat16, w["qkv_seed"])
    do = _dout(q.shape, torch.bfloat16, w["qkv_seed"] + 1)
    plan = api.BlockSparsePlan(spec, q.cuda(), k.cuda(), v.cuda())
    plan()
    bp = api.BlockSparseBwdPlan(plan, do.cuda())
    got = bp()
    torch.cuda.synchronize()
    assert np.array_equal(plan.mask.row_ptr.cpu().numpy(), rp)
    scale = 1.0 / math.sqrt(w["d"])
    got = [torch.stack([t[b, h] for b, h in heads])[None] for t in got]
    qs, ks, vs, ds = [f64(torch.stack([t[b, h] for b, h in heads])[None]) for t in (q, k, v, do)]
    ref = ob.csr_attention_bwd(qs, ks, vs, ds, rp, ci, w["block"], False, scale, mags=True)
    _check_all(got, ref, torch.bfloat16, "bigbird full size")
