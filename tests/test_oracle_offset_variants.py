"""Oracle pins for the offset-attention variants of "Depth-Staggered Fibonacci
Spacing for Sparse Attention", Sec. 2: the power-of-2 control base, alpha as
an exact ratio on the linear-stagger grid (rungs that land on a half), and the
interpolated gather for continuous distances."""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import offsets as oo
from oracle import tiny

FIB15 = [1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 233, 377, 610, 987]


def test_power2_base_reach_and_count():
    # powers of two below the limit: 1..512 below 1024, ceil(log2 N) rungs
    assert oo.power2_base(1024) == [2 ** i for i in range(10)]
    assert oo.power2_base(1025) == [2 ** i for i in range(11)]
    assert oo.power2_base(1) == [] and oo.power2_base(2) == [1]
    for N in (2, 3, 100, 2048, 8193):
        assert len(oo.power2_base(N)) == math.ceil(math.log2(N))
    # W = 8, alpha = 1, N = 1024: the window plus 16, 32, ..., 512
    assert oo.offset_table(8, 1.0, oo.power2_base(1024), 1024) == list(range(9)) + [16, 32, 64, 128, 256, 512]

def test_ratio_table_is_exact_half_up():
    # every rung equals floor(alpha f + 1/2) in exact rational arithmetic
    for l in range(16):
        num, den = 15 + 2 * l, 30  # alpha = 0.5 + l/15
        alpha = Fraction(num, den)
        tab = oo.offset_table_ratio(8, num, den, FIB15, 4096)
        want = sorted(set(range(9)) | {math.floor(alpha * f + Fraction(1, 2)) for f in FIB15})
        assert tab == want

def test_stagger_grid_has_34_ties_and_they_round_up():
    # alpha = 0.5 + l/15 over l = 0..15 and the 15-rung base: alpha f has a
    # fractional part that is a multiple of 1/30; exactly 34 (l, f) pairs land
    # on a half (l = 0 and 15: the 10 odd rungs each; l = 5, 10: f in {3, 21,
    # 987}; l = 3, 6, 9, 12: f in {5, 55})
    ties = [(l, f) for l in range(16) for f in FIB15 if (Fraction(15 + 2 * l, 30) * f).denominator == 2]
    assert len(ties) == 34
    by_l = {}
    for l, f in ties:
        by_l.setdefault(l, []).append(f)
    assert by_l[0] == by_l[15] == [1, 3, 5, 13, 21, 55, 89, 233, 377, 987]
    assert by_l[5] == by_l[10] == [3, 21, 987]
    assert all(by_l[l] == [5, 55] for l in (3, 6, 9, 12))
    # half up: alpha = 1/2 sends rungs 1, 3, 5 to 1, 2, 3
    assert oo.offset_table_ratio(0, 1, 2, [1, 3, 5], 100) == [0, 1, 2, 3]
    assert oo.offset_table_ratio(0, 3, 2, [1, 3], 100) == [0, 2, 5]

def test_ratio_table_matches_double_table_off_ties():
    # where no rung is a tie the exact and the double-precision tables agree
    for l in (1, 2, 4, 7, 8, 11, 13, 14):
        a = 0.5 + l / 15
        assert oo.offset_table_ratio(8, 15 + 2 * l, 30, FIB15, 4096) == oo.offset_table(8, a, FIB15, 4096)

def test_interp_split_integer_alpha_reduces_to_table():
    for N in (64, 1024, 2048):
        base = oo.fibonacci_base(N)
        for alpha in (1.0, 2.0, 3.0):
            ints, rungs = oo.interp_split(8, alpha, base, N)
            assert rungs == []
            assert ints == oo.offset_table(8, alpha, base, N)

def test_interp_split_rungs():
    ints, rungs = oo.interp_split(2, 1.25, [1, 2, 4, 8, 100], 50)
    # 1.25 -> (1, .25); 2.5 -> (2, .5); 5 integer; 10 integer; 125 beyond N
    assert ints == [0, 1, 2, 5, 10]
    assert rungs == [(1, 0.25), (2, 0.5)]
    # a rung whose upper row is N - 1 is kept, one row further is dropped
    assert oo.interp_split(0, 1.5, [1, 3], 5)[1] == [(1, 0.5), (4, 0.5)][:1]
    assert oo.interp_split(0, 1.5, [1, 3], 6)[1] == [(1, 0.5), (4, 0.5)]

def _qkv(B, H, N, d, seed, Hkv=None):
    r = np.random.default_rng(seed)
    Hkv = Hkv or H
    return r.standard_normal((B, H, N, d)), r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hkv, N, d))

def test_interp_without_rungs_is_offset_attention():
    q, k, v = _qkv(2, 2, 40, 8, 1)
    offs = [0, 1, 2, 5, 13]
    o1, l1 = oo.interp_offset_attention(q, k, v, offs, [], 0.3)
    o2, l2 = oo.offset_attention(q, k, v, offs, 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)

def test_interp_brute_force_explicit_keys():
    # every query against its key list built by hand, pure-Python softmax
    q, k, v = _qkv(1, 2, 24, 4, 2, Hkv=1)
    offs = [0, 1, 3]
    rungs = [(2, 0.25), (6, 0.75), (11, 0.5)]
    o, lse = oo.interp_offset_attention(q, k, v, offs, rungs, 0.7)
    for h in range(2):
        for t in range(24):
            keys, vals = [], []
            for dl in offs:
                if t - dl >= 0:
                    keys.append(list(k[0, 0, t - dl]))
                    vals.append(list(v[0, 0, t - dl]))
            for a, w in rungs:
                if t - a - 1 >= 0:
                    keys.append([(1 - w) * x + w * y for x, y in zip(k[0, 0, t - a], k[0, 0, t - a - 1])])
                    vals.append([(1 - w) * x + w * y for x, y in zip(v[0, 0, t - a], v[0, 0, t - a - 1])])
            ob, lb = tiny.explicit_keys_attention(list(q[0, h, t]), keys, vals, 0.7)
            assert np.allclose(o[0, h, t], ob, atol=1e-12) and abs(lse[0, h, t] - lb) < 1e-12

def test_interp_closed_forms():
    B, H, N, d = 1, 1, 30, 6
    q, k, v = _qkv(B, H, N, d, 3)
    offs = [0, 2]
    rungs = [(3, 0.4), (7, 0.9)]
    # q = 0: uniform weights, lse = ln |keys|, o = mean of the (interpolated) values
    o, lse = oo.interp_offset_attention(np.zeros_like(q), k, v, offs, rungs, 1.0)
    for t in (0, 3, 4, 8, 29):
        vals = [v[0, 0, t - x] for x in offs if t - x >= 0]
        vals += [(1 - w) * v[0, 0, t - a] + w * v[0, 0, t - a - 1] for a, w in rungs if t - a - 1 >= 0]
        assert abs(lse[0, 0, t] - math.log(len(vals))) < 1e-12
        assert np.allclose(o[0, 0, t], np.mean(vals, axis=0), atol=1e-12)
    # constant value rows: every convex combination returns the constant
    vc = np.broadcast_to(np.arange(d, dtype=float), v.shape).copy()
    o, _ = oo.interp_offset_attention(q, k, vc, offs, rungs, 0.5)
    assert np.allclose(o, vc, atol=1e-12)

def test_interp_weight_limits_are_plain_rows():
    # w -> 0 approaches a second copy of the row at distance a, w = 1 is the row
    # at distance a + 1 taken twice (the interpolated key is its own key)
    q, k, v = _qkv(1, 1, 20, 4, 4)
    o_dup, l_dup = tiny.explicit_keys_attention(list(q[0, 0, 15]), [list(k[0, 0, 15]), list(k[0, 0, 10]), list(k[0, 0, 10])],
                                                [list(v[0, 0, 15]), list(v[0, 0, 10]), list(v[0, 0, 10])], 0.5)
    o, l = oo.interp_offset_attention(q, k, v, [0, 5], [(5, 1e-12)], 0.5)
    assert np.allclose(o[0, 0, 15], o_dup, atol=1e-9) and abs(l[0, 0, 15] - l_dup) < 1e-9
    o, l = oo.interp_offset_attention(q, k, v, [0, 5], [(4, 1.0)], 0.5)
    assert np.allclose(o[0, 0, 15], o_dup, atol=1e-12) and abs(l[0, 0, 15] - l_dup) < 1e-12
