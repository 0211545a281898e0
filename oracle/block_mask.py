"""Block-level attention masks, their CSR form and a longest-first schedule.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

A mask spec is a plain dict with the keys
  num_blocks   N_b = N / b                  (compression paper, Sec. 3.1: B = N/b)
  num_groups   G, number of independent masks (one per sequence, or shared)
  causal       bool
  win_before, win_after   local window in blocks before / after the row
  win_clamp    non-causal only: shift the window at the edges so that every
               row keeps exactly win_before + win_after + 1 blocks
  global_blocks   list of global block ids
  num_random   r random blocks per row
  random_blocks   optional explicit draws, int array [G, N_b, r] (-1 = none)
  literal_mode "none" | "pair" | "anyq"
  literal_flags   optional explicit flags, uint8 array [G, N_b]
  literal_p    Bernoulli rate used when literal_flags is None
  seed         key of every draw
  exclude_parts   optional list of component names left out of the union
               ("window", "global", "random", "literal"); the identity stays
  period_exclude  optional list of P such lists: group g also leaves out
               period_exclude[g % P] and reads literal flags of group g // P

Each component is built as a dense N_b x N_b boolean matrix per group, the way
the pages write them, and the mask is their union (Eq. 3 of "Parameter-free
Adaptive Sparse Attention", extended with the BigBird global and random graphs
of "BigBird" Sec. 2), intersected with the block-causal triangle when causal.
"""

import numpy as np

from . import rng

LITERAL_MODES = ("none", "pair", "anyq")


def _get(spec, key, default):
    v = spec.get(key, default)
    return default if v is None else v


def period(spec):
    """P: with P > 0, group g has the extra exclusions period_exclude[g % P] and
    the literal flags of flag group g // P (e.g. one group per (sequence, head)
    with P = H: every head of a sequence shares that sequence's flags)."""
    return len(_get(spec, "period_exclude", []))


def flag_group(spec, g):
    P = period(spec)
    return g // P if P else g


def literal_flags(spec):
    """uint8 [F, N_b] literal flags per flag group (F = G, or ceil(G / P) with a
    period): the explicit ones, else Bernoulli draws.

    Compression paper, Sec. 3.1 Eq. 2 defines l_i = 1[r_i > mean r] from gzip
    ratios (see ``literal``); the synthetic workloads may replace the ratios
    with seeded Bernoulli(p) flags (rng.literal_flag).
    """
    G, nb = spec["num_groups"], spec["num_blocks"]
    F = flag_group(spec, G - 1) + 1
    explicit = spec.get("literal_flags")
    if explicit is not None:
        f = np.asarray(explicit, dtype=np.uint8).reshape(-1, nb)[:F]
        return (f != 0).astype(np.uint8)
    p = float(_get(spec, "literal_p", 0.0))
    seed = int(_get(spec, "seed", 0))
    out = np.zeros((F, nb), dtype=np.uint8)
    for f in range(F):
        for j in range(nb):
            out[f, j] = rng.literal_flag(seed, f, j, p)
    return out


def identity_component(nb):
    """I: every block attends itself (compression paper, Eq. 3; Algorithm 1 step 3)."""
    return np.eye(nb, dtype=bool)


def window_component(nb, causal, win_before, win_after, clamp):
    """Local window M^local / G_W.

    Compression paper Sec. 3.2: M^local_ij = 1 iff |i - j| <= w (symmetric w).
    BigBird Sec. 2: w consecutive keys centred on the query, left-windowed when
    causal, |G_W| = N * w.  Here the band is [i - win_before, i + win_after];
    causal rows keep only j <= i.  Non-causal with ``clamp`` shifts the band
    inside [0, N_b) so that each row has exactly win_before + win_after + 1
    blocks (this is what makes |G_W| = N_b * w exact); without it the band is
    clipped at the edges.
    """
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    if causal:
        return (j >= i - win_before) & (j <= i)
    width = win_before + win_after + 1
    if clamp:
        if width >= nb:
            return np.ones((nb, nb), dtype=bool)
        start = np.clip(np.arange(nb) - win_before, 0, nb - width)[:, None]
        return (j >= start) & (j < start + width)
    return (j >= i - win_before) & (j <= i + win_after)


def global_component(nb, causal, global_blocks):
    """Global graph G_G (BigBird Sec. 2): every row attends every global block
    and every global row attends all blocks; |G_G| = 2 g N - g^2 when not causal.
    Causal rows keep only j <= i."""
    m = np.zeros((nb, nb), dtype=bool)
    gl = np.asarray(sorted(set(int(x) for x in global_blocks)), dtype=np.int64)
    if gl.size:
        m[:, gl] = True
        m[gl, :] = True
    if causal:
        m &= np.tril(np.ones((nb, nb), dtype=bool))
    return m


def random_component(spec, g):
    """Random graph G_R (BigBird Sec. 2): r distinct uniform draws per row.

    Causal rows draw only from earlier blocks [0, i), since a later key would
    break causality (BigBird Sec. 4, "Random pattern in causal/decoder
    settings"); non-causal rows draw from [0, N_b).  Explicit draws, when given,
    are used as they are (entries outside the allowed range are ignored).
    """
    nb = spec["num_blocks"]
    causal = bool(spec["causal"])
    r = int(_get(spec, "num_random", 0))
    seed = int(_get(spec, "seed", 0))
    m = np.zeros((nb, nb), dtype=bool)
    if r <= 0:
        return m
    explicit = spec.get("random_blocks")
    if explicit is not None:
        draws = np.asarray(explicit, dtype=np.int64).reshape(spec["num_groups"], nb, r)[g]
    for i in range(nb):
        n = i if causal else nb
        if explicit is not None:
            picks = [int(x) for x in draws[i] if 0 <= int(x) < n]
        else:
            picks = rng.random_blocks(seed, g, i, n, r)
        for c in picks:
            m[i, c] = True
    return m


def literal_component(nb, causal, win_before, win_after, flags, mode):
    """Literal-to-literal graph M^lit (compression paper Sec. 3.2; Algorithm 1
    step 3): M^lit_ij = 1 iff l_i = l_j = 1 and j lies outside the local band.

    mode "pair" is that definition; "anyq" drops the condition on the query
    block (every row attends every literal block outside its band).  Causal
    rows keep only j <= i.
    """
    m = np.zeros((nb, nb), dtype=bool)
    if mode == "none":
        return m
    lit = np.asarray(flags, dtype=bool)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    outside = (j < i - win_before) | (j > i + win_after)
    if mode == "pair":
        m = lit[:, None] & lit[None, :] & outside
    elif mode == "anyq":
        m = np.broadcast_to(lit[None, :], (nb, nb)) & outside
    else:
        raise ValueError(mode)
    if causal:
        m &= np.tril(np.ones((nb, nb), dtype=bool))
    return m


def components(spec, g, flags=None):
    """Dict of the boolean [N_b, N_b] components of group g."""
    nb = spec["num_blocks"]
    causal = bool(spec["causal"])
    wb = int(_get(spec, "win_before", 0))
    wa = int(_get(spec, "win_after", 0))
    clamp = bool(_get(spec, "win_clamp", False))
    mode = _get(spec, "literal_mode", "none")
    if flags is None:
        flags = literal_flags(spec)
    return {
        "identity": identity_component(nb),
        "window": window_component(nb, causal, wb, wa, clamp),
        "global": global_component(nb, causal, _get(spec, "global_blocks", [])),
        "random": random_component(spec, g),
        "literal": literal_component(nb, causal, wb, wa, flags[flag_group(spec, g)], mode),
    }


def block_mask(spec):
    """bool [G, N_b, N_b]: union of all components, block-causal when causal.

    Compression paper Eq. 3 (M = M^lit U M^local U I) with BigBird's G_G and G_R
    added; causal masks keep j <= i (Algorithm 1 step 4 at block level).
    """
    G, nb = spec["num_groups"], spec["num_blocks"]
    flags = literal_flags(spec)
    # components a head group leaves out (compression paper, Sec. 3.3: local
    # heads use M^local U I, long-range heads M^lit U I); I is always kept
    excluded_all = set(_get(spec, "exclude_parts", None) or [])
    pe, P = _get(spec, "period_exclude", []), period(spec)
    out = np.zeros((G, nb, nb), dtype=bool)
    for g in range(G):
        excluded = excluded_all | (set(pe[g % P]) if P else set())
        comp = components(spec, g, flags)
        m = np.zeros((nb, nb), dtype=bool)
        for name, c in comp.items():
            if name not in excluded:
                m |= c
        if spec["causal"]:
            m &= np.tril(np.ones((nb, nb), dtype=bool))
        out[g] = m
    return out


def to_csr(mask):
    """CSR of a [G, N_b, N_b] mask: rows in (g, i) order, columns ascending.

    Returns (row_ptr int32 [G*N_b + 1], col_idx int32 [nnz]).
    """
    G, nb, _ = mask.shape
    flat = mask.reshape(G * nb, nb)
    counts = flat.sum(axis=1).astype(np.int64)
    row_ptr = np.zeros(G * nb + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(flat)[1]  # row-major order: per row, ascending columns
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


def longest_first_schedule(row_ptr, num_groups, num_blocks):
    """int32 [G, N_b]: per group, row ids ordered by (-nnz, row id).

    A longest-first (LPT) order of the independent query-block rows; ties keep
    ascending row order so the schedule is unique.
    """
    counts = np.diff(np.asarray(row_ptr, dtype=np.int64)).reshape(num_groups, num_blocks)
    out = np.zeros((num_groups, num_blocks), dtype=np.int32)
    for g in range(num_groups):
        out[g] = np.array(sorted(range(num_blocks), key=lambda i: (-counts[g, i], i)), dtype=np.int32)
    return out


def build(spec):
    """(row_ptr, col_idx, sched) for a spec: the full oracle mask build."""
    m = block_mask(spec)
    row_ptr, col_idx = to_csr(m)
    sched = longest_first_schedule(row_ptr, spec["num_groups"], spec["num_blocks"])
    return row_ptr, col_idx, sched


def bigbird_edge_count(nb, w, g, r):
    """|G_BB| = N (w + r) + 2 g N - g^2 (BigBird Sec. 2), at block granularity."""
    return nb * (w + r) + 2 * g * nb - g * g
