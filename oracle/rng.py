"""Counter-based random draws for mask construction (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

The pages draw random blocks (BigBird, Sec. 2: r key indices per query, drawn
uniformly and independently; Sec. 3 sketch: a prefix of a random permutation
per row) and the synthetic workloads draw Bernoulli literal flags.  Neither page fixes a
generator, so both sides of the parity check implement the same published
counter-based generator, SplitMix64 (G. L. Steele, D. Lea, C. H. Flood, "Fast
Splittable Pseudorandom Number Generators", OOPSLA 2014), independently, and
derive every draw from a key that names what is drawn.  The key chain, the
Bernoulli threshold and the multiply-shift range reduction are this library's
convention, written out in the functions below, not the pages'.

All arithmetic is on Python integers reduced modulo 2**64.
"""

MASK64 = (1 << 64) - 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15
TAG_LITERAL = 1
TAG_RANDOM = 2


def splitmix64(state):
    """SplitMix64 output for generator state ``state`` (Steele et al. 2014).

    The state is advanced by the golden-ratio increment and the advanced value
    is passed through the 64-bit finaliser (xor-shift 30, multiply, xor-shift
    27, multiply, xor-shift 31).  ``splitmix64(0)`` is the first output of a
    generator seeded with 0.
    """
    z = (state + GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def draw_key(seed, tag, a, b, c):
    """Key of one draw: SplitMix64 chained over (seed, tag, a, b, c).

    key = sm(sm(sm(sm(sm(seed) ^ tag) ^ a) ^ b) ^ c), every operand taken
    modulo 2**64.
    """
    h = splitmix64(seed & MASK64)
    for word in (tag, a, b, c):
        h = splitmix64(h ^ (word & MASK64))
    return h


def bernoulli_threshold(p):
    """32-bit threshold for Bernoulli(p): floor(p * 2**32), clamped to [0, 2**32]."""
    if not (p > 0.0):
        return 0
    t = int(float(p) * 4294967296.0)  # float multiply in double, then floor (p >= 0)
    return min(t, 1 << 32)


def literal_flag(seed, group, block, p):
    """Bernoulli(p) literal flag of block ``block`` in group ``group``.

    Stands in for the per-sequence mean-threshold flag of Eq. 2 ("Parameter-free
    Adaptive Sparse Attention", Sec. 3.1) in the synthetic workloads: the high 32
    bits of the key are compared against floor(p * 2**32).
    """
    h = draw_key(seed, TAG_LITERAL, group, block, 0)
    return 1 if (h >> 32) < bernoulli_threshold(p) else 0


def uniform_below(h, n):
    """Map the high 32 bits of ``h`` onto [0, n) by multiply-shift (n < 2**31)."""
    return ((h >> 32) * n) >> 32


def random_blocks(seed, group, row, n, r):
    """The ``min(r, n)`` distinct uniform draws from [0, n) for one mask row.

    BigBird (Sec. 2, "Random attention G_R") samples r key indices per query;
    its sketch (Sec. 3) takes a prefix of a random permutation, so the draws of
    one row are distinct.  Candidate k is uniform_below(key(seed, RANDOM, group,
    row, k), n); a candidate equal to an earlier one is skipped.  Drawing stops
    once min(r, n) values are accepted or after 64 * r candidates.
    Returns the accepted values in draw order.
    """
    want = min(r, n)
    out = []
    if want <= 0:
        return out
    for k in range(64 * r):
        if len(out) == want:
            break
        c = uniform_below(draw_key(seed, TAG_RANDOM, group, row, k), n)
        if c not in out:
            out.append(c)
    return out
