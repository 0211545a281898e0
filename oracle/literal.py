"""Literal flags from byte content by per-block gzip size.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

"Parameter-free Adaptive Sparse Attention via Compression-Based Content
Selection", Sec. 3.1: a sequence of N bytes is cut into B = N / b blocks, block
i has compression ratio r_i = |gzip(block_i)| / b with gzip at level 1 (Eq. 1),
and it is literal iff r_i is above the mean ratio of the sequence (Eq. 2);
Appendix B, Algorithm 1 steps 1-2 take the same two steps.  Python's ``gzip``
module is the compressor (a library primitive).
"""

import gzip

import numpy as np


def gzip_block_sizes(seq, b, level=1):
    """Compressed size |gzip(block)| of every b-byte block of ``seq`` (Eq. 1 numerators)."""
    seq = bytes(seq)
    if len(seq) % b != 0:
        raise ValueError("sequence length must be a multiple of the block size")
    return [len(gzip.compress(seq[i:i + b], compresslevel=level, mtime=0)) for i in range(0, len(seq), b)]


def ratios(sizes, b):
    """r_i = |gzip(block_i)| / b (Eq. 1)."""
    return [s / b for s in sizes]


def flags_from_sizes(sizes):
    """Eq. 2: l_i = 1 iff r_i > mean_j r_j.

    With r_i = c_i / b and mean = (sum_j c_j) / (B b), the comparison is taken
    exactly in integers: c_i * B > sum_j c_j.
    """
    B = len(sizes)
    total = sum(int(c) for c in sizes)
    return np.array([1 if int(c) * B > total else 0 for c in sizes], dtype=np.uint8)


def literal_flags(seq, b, level=1):
    """Steps 1-2 of Algorithm 1 for one sequence: flags uint8 [B]."""
    return flags_from_sizes(gzip_block_sizes(seq, b, level))


def literal_flags_batch(data, b, level=1):
    """Flags for each row of a uint8 array [G, n]: uint8 [G, n / b]."""
    data = np.asarray(data, dtype=np.uint8)
    return np.stack([literal_flags(row.tobytes(), b, level) for row in data])
