"""Pins of the fp64 attention gradients (oracle.backward): central finite
differences of the forward oracle, two independent derivations (dense-masked
and CSR-gather), the full mask against torch autograd, and the invariants
that softmax attention fixes (key shift, value sums, keys outside the mask)."""

import math
import random

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import backward as ob
from oracle import block_mask as bm
from oracle import offsets as oo
from long_context_sparse_block_amd import workloads as wl


def _qkv(B, H, N, d, seed, Hkv=None):
    q, k, v = wl.make_qkv(B, H, N, d, torch.float64, seed, H_kv=Hkv)
    return q.numpy(), k.numpy(), v.numpy()


def _csr(rows):
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.array([c for r in rows for c in r], dtype=np.int32)
    return row_ptr, col_idx


def _numgrad(f, x, eps=1e-6):
    """Central differences of the scalar f() with respect to every entry of x."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_block_sparse_finite_differences():
    # two mask groups (one per q head), GQA (2 q heads on 1 K/V head), causal,
    # a query block whose only listed block lies in its future (empty rows)
    B, H, N, d, block = 1, 2, 12, 3, 3
    q, k, v = _qkv(B, H, N, d, 5, Hkv=1)
    do = np.random.default_rng(6).standard_normal(q.shape)
    rows = [[0], [0, 1], [1, 3], [0, 2, 3],      # group 0 (row 2 lists block 3 > 2)
            [0], [1], [0, 2], [1, 3]]            # group 1
    row_ptr, col_idx = _csr(rows)
    scale = 0.7

    def loss():
        o, _ = oa.csr_attention(q, k, v, row_ptr, col_idx, block, True, scale, 0, 1)
        return float(np.sum(o * do))
    dq, dk, dv = ob.csr_attention_bwd(q, k, v, do, row_ptr, col_idx, block, True, scale, 0, 1)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        np.testing.assert_allclose(g, _numgrad(loss, x), atol=1e-7, rtol=0)


def test_offsets_finite_differences():
    B, H, N, d = 1, 2, 14, 3
    q, k, v = _qkv(B, H, N, d, 7, Hkv=1)
    do = np.random.default_rng(8).standard_normal(q.shape)
    offs = [1, 3, 4, 9]  # no distance 0: the first query has no key

    def loss():
        o, _ = oo.offset_attention(q, k, v, offs, 0.6)
        return float(np.sum(o * do))
    dq, dk, dv = ob.offset_attention_bwd(q, k, v, do, offs, 0.6)
    for x, g in ((q, dq), (k, dk), (v, dv)):
        np.testing.assert_allclose(g, _numgrad(loss, x), atol=1e-7, rtol=0)


@pytest.mark.parametrize("seed", range(6))
def test_dense_masked_equals_csr_gather(seed):
    R = random.Random(100 + seed)
    block = R.choice([2, 4, 8])
    nb = R.randint(1, 7)
    causal = R.random() < 0.5
    spec = dict(num_blocks=nb, num_groups=2, causal=causal, win_before=R.randint(0, 2),
                win_after=0 if causal else R.randint(0, 2), win_clamp=R.random() < 0.5,
                global_blocks=sorted(R.sample(range(nb), R.randint(0, min(2, nb)))),
                num_random=R.randint(0, 2), random_blocks=None,
                literal_mode=R.choice(["none", "pair", "anyq"]), literal_flags=None,
                literal_p=0.4, seed=seed)
    N = nb * block
    q, k, v = _qkv(2, 4, N, 8, 200 + seed, Hkv=2)
    do = np.random.default_rng(seed).standard_normal(q.shape)
    masks = bm.block_mask(spec)
    row_ptr, col_idx = bm.to_csr(masks)
    a = ob.dense_masked_attention_bwd(q, k, v, do, masks, block, causal, 0.3, 1, 0)
    b = ob.csr_attention_bwd(q, k, v, do, row_ptr, col_idx, block, causal, 0.3, 1, 0)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)


@pytest.mark.parametrize("causal", [True, False])
def test_full_mask_equals_autograd(causal):
    B, H, N, d, block = 2, 2, 32, 8, 8
    q, k, v = _qkv(B, H, N, d, 9)
    do = np.random.default_rng(10).standard_normal(q.shape)
    nb = N // block
    rows = [list(range(i + 1)) if causal else list(range(nb)) for i in range(nb)]
    row_ptr, col_idx = _csr(rows)
    dq, dk, dv = ob.csr_attention_bwd(q, k, v, do, row_ptr, col_idx, block, causal, 0.25)
    qt, kt, vt = [torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v)]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=causal, scale=0.25)
    o.backward(torch.from_numpy(do))
    for g, t in ((dq, qt), (dk, kt), (dv, vt)):
        np.testing.assert_allclose(g, t.grad.numpy(), atol=1e-12, rtol=0)


def test_invariants_key_shift_value_sum_and_outside_mask():
    B, H, N, d, block = 1, 4, 40, 6, 4
    q, k, v = _qkv(B, H, N, d, 11, Hkv=2)
    do = np.random.default_rng(12).standard_normal(q.shape)
    nb = N // block
    # causal; key block 7 is listed by no row, query block 5 lists nothing
    rows = [[c for c in range(i + 1) if c != 7 and (i * 3 + c) % 4 != 1] if i != 5 else [] for i in range(nb)]
    rows = [r if (i == 5 or r) else [i] for i, r in enumerate(rows)]
    row_ptr, col_idx = _csr(rows)
    dq, dk, dv = ob.csr_attention_bwd(q, k, v, do, row_ptr, col_idx, block, True, 0.4)
    # shifting every key by one vector leaves each softmax row unchanged:
    # the key gradients of each K/V head sum to zero
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    # the weights of a non-empty row sum to one: value gradients add up to the
    # upstream gradients of the non-empty rows of the heads sharing the K/V head
    nonempty = np.array([i != 5 for i in range(nb) for _ in range(block)])
    want = do[:, :, nonempty].reshape(B, 2, 2, -1, d).sum(axis=(2, 3))
    np.testing.assert_allclose(dv.sum(axis=2), want, atol=1e-12)
    # no query attends key block 7: zero gradient there, and changing those
    # keys / values changes nothing
    np.testing.assert_array_equal(dk[:, :, 28:32], 0.0)
    np.testing.assert_array_equal(dv[:, :, 28:32], 0.0)
    np.testing.assert_array_equal(dq[:, :, 20:24], 0.0)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 28:32] += 5.0
    v2[:, :, 28:32] -= 3.0
    for x, y in zip((dq, dk, dv), ob.csr_attention_bwd(q, k2, v2, do, row_ptr, col_idx, block, True, 0.4)):
        np.testing.assert_array_equal(x, y)


def test_offsets_bwd_special_cases():
    N, d = 24, 5
    q, k, v = _qkv(1, 2, N, d, 13)
    do = np.random.default_rng(14).standard_normal(q.shape)
    # the full table is dense causal attention
    a = ob.offset_attention_bwd(q, k, v, do, list(range(N)), 0.5)
    rows = [list(range(t + 1)) for t in range(N)]
    b = ob.csr_attention_bwd(q, k, v, do, *_csr(rows), 1, True, 0.5)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)
    # the table {0}: o = v, so dq = dk = 0 (up to rounding of dp - D) and dv = dO
    dq, dk, dv = ob.offset_attention_bwd(q, k, v, do, [0], 0.5)
    np.testing.assert_allclose(dq, 0.0, atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv, do, atol=0)
    # any table equals the token-level CSR form with block 1
    offs = [0, 2, 3, 7, 13]
    a = ob.offset_attention_bwd(q, k, v, do, offs, 0.5)
    rows = [[t - x for x in reversed(offs) if t - x >= 0] for t in range(N)]
    b = ob.csr_attention_bwd(q, k, v, do, *_csr(rows), 1, True, 0.5)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12, rtol=0)


def test_term_magnitudes_bound_the_gradients():
    # |gradient entry| <= its term magnitude (triangle inequality), and with
    # non-negative dO the value-gradient magnitudes are the value gradients
    B, H, N, d, block = 1, 2, 24, 4, 4
    q, k, v = _qkv(B, H, N, d, 21)
    do = np.random.default_rng(22).standard_normal(q.shape)
    nb = N // block
    rows = [list(range(i + 1)) for i in range(nb)]
    rp, ci = _csr(rows)
    g, m = ob.csr_attention_bwd(q, k, v, do, rp, ci, block, True, 0.5, mags=True)
    for x, y in zip(g, m):
        assert np.all(np.abs(x) <= y + 1e-12)
    g, m = ob.csr_attention_bwd(q, k, v, np.abs(do), rp, ci, block, True, 0.5, mags=True)
    np.testing.assert_allclose(g[2], m[2], atol=1e-12)
    g, m = ob.offset_attention_bwd(q, k, v, do, [0, 1, 5], 0.5, mags=True)
    g2 = ob.offset_attention_bwd(q, k, v, do, [0, 1, 5], 0.5)
    for x, y, z in zip(g, m, g2):
        assert np.all(np.abs(x) <= y + 1e-12)
        np.testing.assert_array_equal(x, z)
