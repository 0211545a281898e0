"""Token-level offset attention (Fibonacci offsets), fp64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"Depth-Staggered Fibonacci Spacing for Sparse Attention", Sec. 2 ("Attended
set"): query i attends the dense window of distances {0, 1, ..., W} (the self
position included, so no query has an empty key set) plus the rungs
d_k = alpha * f_k of the Fibonacci base; the distances are shared by all
queries (shifted gathers).  Integer distances are taken as floor(alpha*f + 1/2)
(round half up), rungs are the base values below N, repeated distances count
once (the attended set is a set) and distances >= N are dropped.

The same section's variants: the reach-matched power-of-2 base ("Control
base"), alpha as an exact ratio (the linear stagger alpha = 0.5 + l/(L - 1)
puts some rungs exactly on a half), and the interpolated gather for a
continuous d_k = alpha f_k ("Attended set"; "Implementation note"): the
gathered key and value are the linear interpolation between the rows at
distances floor(d_k) and floor(d_k) + 1.
"""

import math

import numpy as np


def fibonacci_base(limit):
    """Fibonacci base 1, 2, 3, 5, 8, ... of all values below ``limit``.

    Sec. 2 lists fib = [1, 2, 3, 5, 8, ..., 987] (K = 15 rungs for length 1024).
    """
    out = []
    a, b = 1, 2
    while a < limit:
        out.append(a)
        a, b = b, a + b
    return out


def offset_table(W, alpha, base, N):
    """Sorted distinct distances {0..W} U {floor(alpha*f + 1/2) : f in base},
    restricted to [0, N - 1]."""
    d = set(range(0, W + 1))
    for f in base:
        d.add(int(math.floor(float(alpha) * float(f) + 0.5)))
    return sorted(x for x in d if 0 <= x < N)


def offset_attention(q, k, v, offsets, scale):
    """o, lse for every query: keys {t - delta : delta in offsets, t - delta >= 0}.

    q [B, H, N, d], k, v [B, H_kv, N, d] float64.  Returns (o, lse) float64.
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    rep = H // Hkv
    offs = list(offsets)
    D = len(offs)
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    t = np.arange(N)
    for b in range(B):
        for h in range(H):
            kh = h // rep
            s = np.full((N, D), -np.inf)
            for n, delta in enumerate(offs):
                src = t - delta
                ok = (src >= 0) & (src < N)
                s[ok, n] = scale * np.einsum("ij,ij->i", q[b, h, t[ok]], k[b, kh, src[ok]])
            m = s.max(axis=1)
            empty = ~np.isfinite(m)
            m_safe = np.where(empty, 0.0, m)
            e = np.where(np.isfinite(s), np.exp(s - m_safe[:, None]), 0.0)
            l = e.sum(axis=1)
            acc = np.zeros((N, d))
            for n, delta in enumerate(offs):
                src = t - delta
                ok = (src >= 0) & (src < N)
                acc[ok] += e[ok, n][:, None] * v[b, kh, src[ok]]
            nz = l > 0
            o[b, h, nz] = acc[nz] / l[nz][:, None]
            lse[b, h, nz] = m_safe[nz] + np.log(l[nz])
    return o, lse


def offset_attention_rows(q, k, v, offsets, scale, samples):
    """Same for single queries; samples = [(b, h, t)].  Returns (o, lse)."""
    H = q.shape[1]
    rep = H // k.shape[1]
    N = q.shape[2]
    o = np.zeros((len(samples), q.shape[3]))
    lse = np.full(len(samples), -np.inf)
    for n, (b, h, t) in enumerate(samples):
        src = np.array([t - x for x in offsets if 0 <= t - x < N], dtype=np.int64)
        if src.size == 0:
            continue
        kh = h // rep
        s = scale * (k[b, kh, src] @ q[b, h, t])
        m = s.max()
        e = np.exp(s - m)
        o[n] = (e @ v[b, kh, src]) / e.sum()
        lse[n] = m + np.log(e.sum())
    return o, lse


def power2_base(limit):
    """Powers of two 1, 2, 4, ... below ``limit`` (Sec. 2, "Control base": the
    log-sparse base that reaches as far as the Fibonacci one with fewer rungs)."""
    out = []
    x = 1
    while x < limit:
        out.append(x)
        x *= 2
    return out


def offset_table_ratio(W, num, den, base, N):
    """offset_table for alpha = num / den held exactly: floor(num f / den + 1/2)
    evaluated in integers, so a rung that lands exactly on a half rounds up."""
    d = set(range(0, W + 1))
    for f in base:
        d.add((2 * num * f + den) // (2 * den))
    return sorted(x for x in d if 0 <= x < N)


def interp_split(W, alpha, base, N):
    """Key set of the interpolated gather (Sec. 2, "Attended set"): the window
    {0..W}, every rung whose alpha*f (double) is an integer as an ordinary
    distance (so integer alpha*f gives exactly offset_table), and every other
    rung as (a, w) = (floor(alpha f), alpha f - floor(alpha f)): the key and
    value are (1 - w) row[t - a] + w row[t - a - 1], used by queries t >= a + 1.
    Rungs with a + 1 > N - 1 reach no query and are dropped."""
    ints = set(range(0, W + 1))
    rungs = []
    for f in base:
        x = float(alpha) * float(f)
        if x < 0:
            continue  # a negative distance reaches no key
        a = math.floor(x)
        if x == a:
            ints.add(int(a))
        elif a + 1 <= N - 1:
            rungs.append((int(a), x - a))
    return sorted(i for i in ints if 0 <= i < N), rungs


def interp_offset_attention(q, k, v, offsets, rungs, scale):
    """o, lse for every query over the integer distances ``offsets`` and the
    interpolated rungs ``rungs`` [(a, w)] (one key each, valid for t >= a + 1).

    q [B, H, N, d], k, v [B, H_kv, N, d] float64.  Returns (o, lse) float64.
    """
    B, H, N, d = q.shape
    rep = H // k.shape[1]
    offs = list(offsets)
    R = len(rungs)
    D = len(offs) + R
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    t = np.arange(N)

    def key_rows(kv, b, kh, n):
        # rows of key n for every query (index arrays ok), as float64 [n_ok, d]
        if n < len(offs):
            src = t - offs[n]
            ok = src >= 0
            return ok, kv[b, kh, src[ok]]
        a, w = rungs[n - len(offs)]
        ok = t - a - 1 >= 0
        return ok, (1.0 - w) * kv[b, kh, (t - a)[ok]] + w * kv[b, kh, (t - a - 1)[ok]]

    for b in range(B):
        for h in range(H):
            kh = h // rep
            s = np.full((N, D), -np.inf)
            for n in range(D):
                ok, kr = key_rows(k, b, kh, n)
                s[ok, n] = scale * np.einsum("ij,ij->i", q[b, h, t[ok]], kr)
            m = s.max(axis=1)
            empty = ~np.isfinite(m)
            m_safe = np.where(empty, 0.0, m)
            e = np.where(np.isfinite(s), np.exp(s - m_safe[:, None]), 0.0)
            l = e.sum(axis=1)
            acc = np.zeros((N, d))
            for n in range(D):
                ok, vr = key_rows(v, b, kh, n)
                acc[ok] += e[ok, n][:, None] * vr
            nz = l > 0
            o[b, h, nz] = acc[nz] / l[nz][:, None]
            lse[b, h, nz] = m_safe[nz] + np.log(l[nz])
    return o, lse
