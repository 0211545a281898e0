"""Write rng_vectors.txt: known-answer vectors of the draw-key chain, the
Bernoulli literal draw and the distinct random-block draws.

Run from the repository root:  python tests/golden/make_rng_vectors.py

The values come from the oracle alone (oracle/rng.py, written from the stated
convention: SplitMix64 of Steele, Lea & Flood, OOPSLA 2014, chained over
(seed, tag, a, b, c); Bernoulli threshold floor(p 2^32); multiply-shift range
reduction; repeats skipped, at most 64 r candidates).  They freeze that
convention so that a later change to either side shows up as a failing test.
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import rng  # noqa: E402

M = (1 << 64) - 1
KEYS = [(0, 0, 0, 0, 0), (0, 1, 0, 0, 0), (0, 2, 0, 0, 0), (1, 1, 0, 0, 0), (2, 1, 3, 17, 0),
        (5, 1, 0, 511, 0), (3, 2, 0, 63, 2), (12345, 2, 7, 100, 191), (M, 1, M, M, M),
        (0x9E3779B97F4A7C15, 2, 1 << 40, 1 << 33, 5)]
LITERALS = [(2, 0, j, 0.25) for j in range(16)] + [(5, 0, j, 0.15) for j in range(16)] + \
           [(9, 3, 7, 0.0), (9, 3, 7, 1.0), (9, 3, 7, 0.5), (M, M, M, 0.999999)]
DRAWS = [(1, 0, 5, 5, 1), (3, 0, 10, 64, 3), (3, 0, 63, 64, 3), (7, 2, 4, 4, 3), (7, 2, 4, 4, 4),
         (7, 2, 3, 3, 32), (11, 1, 0, 1, 2), (11, 1, 9, 0, 2), (13, 0, 1000, 16384, 32), (0, 5, 2, 2, 2)]


def main():
    lines = ["# Known-answer vectors of the library's counter-based draws (written by",
             "# tests/golden/make_rng_vectors.py from oracle/rng.py alone).",
             "# key  seed tag a b c -> key(seed, tag, a, b, c)",
             "# lit  seed group block p -> Bernoulli(p) literal flag",
             "# draw seed group row n r -> the distinct draws from [0, n) in draw order"]
    for s, t, a, b, c in KEYS:
        lines.append(f"key {s:#x} {t} {a:#x} {b:#x} {c:#x} {rng.draw_key(s, t, a, b, c):#018x}")
    for s, g, j, p in LITERALS:
        lines.append(f"lit {s:#x} {g:#x} {j:#x} {p!r} {rng.literal_flag(s, g, j, p)}")
    for s, g, i, n, r in DRAWS:
        d = rng.random_blocks(s, g, i, n, r)
        lines.append(f"draw {s:#x} {g} {i} {n} {r} " + (",".join(str(x) for x in d) or "-"))
    with open(os.path.join(HERE, "rng_vectors.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
