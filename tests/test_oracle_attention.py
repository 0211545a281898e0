"""Pins of the oracle's attention forms (no GPU): special cases that reduce to
textbook / library attention, closed forms, invariants and tiny brute force."""

import math
import random

import numpy as np
import pytest
import torch

from oracle import attention as oa
from oracle import block_mask as bm
from oracle import offsets as oo
from oracle import tiny
from long_context_sparse_block_amd import workloads as wl
from tests.conftest import golden_path


def _qkv(B, H, N, d, seed, Hkv=None):
    q, k, v = wl.make_qkv(B, H, N, d, torch.float64, seed, H_kv=Hkv)
    return q.numpy(), k.numpy(), v.numpy()


def _full_csr(nb, causal, G=1):
    rows = []
    for _ in range(G):
        for i in range(nb):
            rows.append(list(range(i + 1)) if causal else list(range(nb)))
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.array([c for r in rows for c in r], dtype=np.int32)
    return row_ptr, col_idx


def _sdpa(q, k, v, causal, scale):
    o = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        is_causal=causal, scale=scale)
    return o.numpy()


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("block", [4, 16])
def test_full_mask_equals_library_attention(causal, block):
    B, H, N, d = 2, 3, 64, 16
    q, k, v = _qkv(B, H, N, d, 1)
    row_ptr, col_idx = _full_csr(N // block, causal)
    scale = 1 / math.sqrt(d)
    o, lse = oa.csr_attention(q, k, v, row_ptr, col_idx, block, causal, scale)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal, scale), atol=1e-12, rtol=0)
    # lse against a direct log-sum-exp over the causal / full score rows
    s = scale * np.einsum("bhtd,bhsd->bhts", q, k)
    if causal:
        s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
    ref = np.log(np.exp(s - s.max(-1, keepdims=True)).sum(-1)) + s.max(-1)
    np.testing.assert_allclose(lse, ref, atol=1e-12, rtol=0)


def _random_block_case(seed):
    R = random.Random(seed)
    block = R.choice([2, 4, 8])
    nb = R.randint(1, 9)
    causal = R.random() < 0.5
    spec = dict(num_blocks=nb, num_groups=2, causal=causal, win_before=R.randint(0, 2),
                win_after=0 if causal else R.randint(0, 2), win_clamp=R.random() < 0.5,
                global_blocks=sorted(R.sample(range(nb), R.randint(0, min(2, nb)))),
                num_random=R.randint(0, 2), random_blocks=None,
                literal_mode=R.choice(["none", "pair", "anyq"]), literal_flags=None,
                literal_p=0.4, seed=seed)
    return spec, block


@pytest.mark.parametrize("seed", range(12))
def test_dense_masked_equals_csr_gather(seed):
    spec, block = _random_block_case(seed)
    nb = spec["num_blocks"]
    B, H, d = 2, 2, 8
    q, k, v = _qkv(B, H, nb * block, d, 10 + seed)
    mask = bm.block_mask(spec)
    row_ptr, col_idx = bm.to_csr(mask)
    scale = 0.37
    o1, l1 = oa.csr_attention(q, k, v, row_ptr, col_idx, block, spec["causal"], scale, 1, 0)
    o2, l2 = oa.dense_masked_attention(q, k, v, mask, block, spec["causal"], scale, 1, 0)
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_array_equal(np.isinf(l1), np.isinf(l2))
    fin = np.isfinite(l1)
    np.testing.assert_allclose(l1[fin], l2[fin], atol=1e-12, rtol=0)


def _key_sets(row_ptr, col_idx, nb, block, causal, g=0):
    N = nb * block
    sets = []
    for t in range(N):
        r = g * nb + t // block
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        ks = [c * block + j for c in cols for j in range(block)]
        if causal:
            ks = [s for s in ks if s <= t]
        sets.append(ks)
    return sets


@pytest.mark.parametrize("seed", range(4))
def test_zero_query_closed_form(seed):
    """q = 0: every allowed logit is 0, so lse = ln |K(t)| and o = mean of v over K(t)."""
    spec, block = _random_block_case(100 + seed)
    nb = spec["num_blocks"]
    _, k, v = _qkv(1, 1, nb * block, 8, 20 + seed)
    q = np.zeros_like(k)
    row_ptr, col_idx, _ = bm.build(spec)
    o, lse = oa.csr_attention(q, k, v, row_ptr, col_idx, block, spec["causal"], 0.5)
    for t, ks in enumerate(_key_sets(row_ptr, col_idx, nb, block, spec["causal"])):
        if not ks:
            assert lse[0, 0, t] == -np.inf and np.all(o[0, 0, t] == 0)
            continue
        assert abs(lse[0, 0, t] - math.log(len(ks))) < 1e-13
        np.testing.assert_allclose(o[0, 0, t], v[0, 0, ks].mean(axis=0), atol=1e-13)


def test_softmax_rows_sum_to_one_and_zero_outside():
    spec = wl.mask_spec(wl.BLOCK_WORKLOADS["tiny-fp32"])
    block, nb = 64, spec["num_blocks"]
    q, k, v = _qkv(1, 1, nb * block, 64, 5)
    row_ptr, col_idx, _ = bm.build(spec)
    scale = 0.125
    o, lse = oa.csr_attention(q, k, v, row_ptr, col_idx, block, True, scale)
    sets = _key_sets(row_ptr, col_idx, nb, block, True)
    for t in range(0, nb * block, 7):
        s = scale * (k[0, 0, sets[t]] @ q[0, 0, t])
        assert abs(np.exp(s - lse[0, 0, t]).sum() - 1.0) < 1e-12
    # keys outside K(t) may change arbitrarily without changing o or lse bitwise
    inside = np.zeros(nb * block, dtype=bool)
    t0 = 300
    inside[sets[t0]] = True
    k2, v2 = k.copy(), v.copy()
    k2[0, 0, ~inside] = 1e3
    v2[0, 0, ~inside] = -7.0
    o2, lse2 = oa.csr_attention_rows(q, k2, v2, row_ptr, col_idx, block, True, scale, [(0, 0, t0)])
    o1, lse1 = oa.csr_attention_rows(q, k, v, row_ptr, col_idx, block, True, scale, [(0, 0, t0)])
    assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2)
    np.testing.assert_allclose(o1[0], o[0, 0, t0], atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_tiny_brute_force_hand_masks(seed):
    """N <= 32, b in {2,4,8}, hand-built rows including empty ones."""
    R = random.Random(seed)
    block = [2, 4, 8][seed % 3]
    nb = 32 // block
    causal = seed % 2 == 0
    rows = []
    for i in range(nb):
        if R.random() < 0.2:
            rows.append(set())  # empty row
        else:
            rows.append(set(R.sample(range(nb), R.randint(1, nb))))
    if causal:
        rows[nb - 1] = {nb - 1}
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.array([c for r in rows for c in sorted(r)], dtype=np.int32)
    q, k, v = _qkv(1, 1, 32, 4, 30 + seed)
    o, lse = oa.csr_attention(q, k, v, row_ptr, col_idx, block, causal, 0.7)
    ot, lt = tiny.masked_softmax_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                           tiny.block_rows_allowed(rows, block, causal), 0.7)
    np.testing.assert_allclose(o[0, 0], np.array(ot), atol=1e-12)
    lt = np.array(lt)
    assert np.array_equal(np.isinf(lt), np.isinf(lse[0, 0]))
    np.testing.assert_allclose(lse[0, 0][np.isfinite(lt)], lt[np.isfinite(lt)], atol=1e-12)


def test_gqa_equals_repeated_heads():
    B, H, Hkv, N, d, block = 1, 4, 2, 32, 8, 8
    q, k, v = _qkv(B, H, N, d, 3, Hkv=Hkv)
    row_ptr, col_idx = _full_csr(N // block, True)
    o1, l1 = oa.csr_attention(q, k, v, row_ptr, col_idx, block, True, 0.3)
    kr, vr = np.repeat(k, H // Hkv, axis=1), np.repeat(v, H // Hkv, axis=1)
    o2, l2 = oa.csr_attention(q, kr, vr, row_ptr, col_idx, block, True, 0.3)
    np.testing.assert_array_equal(o1, o2)


# ------------------------------------------------------------ offsets ----

def _read_fib():
    lines = [x.strip() for x in open(golden_path("fibonacci_base.txt")) if x.strip() and not x.startswith("#")]
    base = [int(x) for x in lines[0].split()]
    count = int(lines[1].split()[1])
    return base, count


def test_fibonacci_base_matches_page():
    base, _ = _read_fib()
    assert oo.fibonacci_base(1000) == base
    assert oo.fibonacci_base(988) == base and oo.fibonacci_base(987) == base[:-1]


def test_distinct_distance_count_matches_page():
    base, count = _read_fib()
    assert len(oo.offset_table(8, 1.0, base, 1024)) == count


def test_offset_tables_of_the_workload():
    w = wl.OFFSET_WORKLOAD
    for N in w["lengths"]:
        base = oo.fibonacci_base(N)
        sizes = set()
        for a in w["alphas"]:
            t = oo.offset_table(w["W"], a, base, N)
            assert t == sorted(set(t)) and t[0] == 0 and t[-1] < N
            assert set(range(9)) <= set(t)
            # no ties: alpha * f = (15 + l) f / 15 never has fractional part 1/2
            for f in base:
                frac = (a * f) % 1.0
                assert abs(frac - 0.5) > 1e-6
            sizes.add(len(t))
        assert sizes == ({20, 21} if N == 2048 else {23, 24})


def test_offset_rounding_is_half_up():
    # alpha * f = 0.5 and 1.5: half-up gives 1 and 2; half-to-even would give 0 and 2
    assert oo.offset_table(0, 0.5, [1, 3], 10) == [0, 1, 2]


def test_offsets_full_table_is_dense_causal():
    B, H, N, d = 1, 2, 48, 8
    q, k, v = _qkv(B, H, N, d, 8)
    o, lse = oo.offset_attention(q, k, v, list(range(N)), 0.4)
    np.testing.assert_allclose(o, _sdpa(q, k, v, True, 0.4), atol=1e-12)


def test_offsets_zero_table_is_identity():
    q, k, v = _qkv(1, 1, 40, 8, 9)
    o, lse = oo.offset_attention(q, k, v, [0], 0.4)
    assert np.array_equal(o, v)
    np.testing.assert_allclose(lse[0, 0], 0.4 * np.einsum("td,td->t", q[0, 0], k[0, 0]), atol=1e-13)


def test_offsets_equal_token_level_csr():
    """Offset attention = block-sparse attention with block 1 and row t = {t - delta}."""
    N, d = 64, 8
    q, k, v = _qkv(2, 2, N, d, 11)
    offs = oo.offset_table(3, 1.5, oo.fibonacci_base(N), N)
    rows = [[t - x for x in reversed(offs) if t - x >= 0] for t in range(N)]
    row_ptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    col_idx = np.array([c for r in rows for c in r], dtype=np.int32)
    o1, l1 = oo.offset_attention(q, k, v, offs, 0.3)
    o2, l2 = oa.csr_attention(q, k, v, row_ptr, col_idx, 1, True, 0.3)
    np.testing.assert_allclose(o1, o2, atol=1e-12)
    np.testing.assert_allclose(l1, l2, atol=1e-12)


def test_offsets_tiny_brute_force():
    N = 30
    q, k, v = _qkv(1, 1, N, 4, 12)
    offs = [0, 1, 2, 5, 9, 17]
    o, lse = oo.offset_attention(q, k, v, offs, 0.9)
    ot, lt = tiny.masked_softmax_attention(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(),
                                           tiny.offsets_allowed(offs), 0.9)
    np.testing.assert_allclose(o[0, 0], np.array(ot), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(lt), atol=1e-12)
    rows = oo.offset_attention_rows(q, k, v, offs, 0.9, [(0, 0, 0), (0, 0, 29)])
    np.testing.assert_allclose(rows[0], o[0, 0, [0, 29]], atol=1e-13)
