"""Pins of the gzip-derived literal flags (compression paper, Sec. 3.1, Eq. 1-2;
Appendix B, Algorithm 1 steps 1-2) and the library's host implementation of
them, bit for bit.  No GPU needed."""

import gzip
import os

import numpy as np
import pytest

from oracle import literal

B128 = 128


def test_mean_threshold_closed_form():
    # Eq. 2: literal iff r_i > mean r (strict)
    assert literal.flags_from_sizes([10, 20, 30]).tolist() == [0, 0, 1]
    assert literal.flags_from_sizes([1, 3]).tolist() == [0, 1]
    assert literal.flags_from_sizes([5, 5, 5, 5]).tolist() == [0, 0, 0, 0]
    # mean exactly equal to one entry: that entry is not literal
    assert literal.flags_from_sizes([2, 4, 6]).tolist() == [0, 0, 1]
    # integer form is exact where a float mean of ratios could round: sum 7 over 3
    assert literal.flags_from_sizes([2, 2, 3]).tolist() == [0, 0, 1]
    assert literal.ratios([64, 128], 128) == [0.5, 1.0]


def test_threshold_ignores_constant_overhead_and_scale():
    # a constant per-block overhead (e.g. a container header) or a common scale
    # of the sizes leaves r_i > mean r unchanged
    rng = np.random.default_rng(3)
    for _ in range(50):
        sizes = rng.integers(10, 200, size=rng.integers(1, 70)).tolist()
        base = literal.flags_from_sizes(sizes)
        assert np.array_equal(literal.flags_from_sizes([c + 18 for c in sizes]), base)
        assert np.array_equal(literal.flags_from_sizes([3 * c for c in sizes]), base)


def test_at_least_one_block_below_mean_unless_all_equal():
    rng = np.random.default_rng(4)
    for _ in range(50):
        sizes = rng.integers(1, 100, size=rng.integers(2, 40)).tolist()
        f = literal.flags_from_sizes(sizes)
        if len(set(sizes)) == 1:
            assert f.sum() == 0
        else:
            assert 0 < f.sum() < len(sizes)


def test_incompressible_blocks_are_literal_repetitive_are_not():
    # gzip cannot shrink uniform random bytes (its size exceeds the block) and
    # shrinks a constant block far below half: in a sequence alternating the
    # two, exactly the random blocks are literal
    rng = np.random.default_rng(5)
    blocks, expect = [], []
    for i in range(16):
        if i % 3 == 0:
            blocks.append(bytes(rng.integers(0, 256, B128, dtype=np.uint8)))
            expect.append(1)
        else:
            blocks.append(bytes([65 + i]) * B128)
            expect.append(0)
    seq = b"".join(blocks)
    sizes = literal.gzip_block_sizes(seq, B128)
    for c, e in zip(sizes, expect):
        assert (c > B128) if e else (c < B128 // 2)
    assert literal.literal_flags(seq, B128).tolist() == expect


def test_block_sizes_are_per_block():
    # each block is compressed on its own: a block's size does not depend on
    # the blocks around it
    rng = np.random.default_rng(6)
    a = bytes(rng.integers(0, 256, B128, dtype=np.uint8))
    b = b"xyz" * 42 + b"xy"
    assert literal.gzip_block_sizes(a + b, B128) == literal.gzip_block_sizes(b + a, B128)[::-1]
    with pytest.raises(ValueError):
        literal.gzip_block_sizes(a + b[:5], B128)


def test_sizes_follow_gzip_format():
    # gzip container: 10-byte header and 8-byte trailer around the deflate data
    assert literal.gzip_block_sizes(bytes(B128), B128)[0] >= 18
    blk = bytes(range(B128))
    assert literal.gzip_block_sizes(blk, B128)[0] == len(gzip.compress(blk, compresslevel=1, mtime=0))


# ---- the library's host implementation, bit for bit ------------------------

def _lib_available():
    from long_context_sparse_block_amd import _lib
    return os.path.exists(_lib.LIB_PATH)


@pytest.mark.skipif(not _lib_available(), reason="library not built")
@pytest.mark.parametrize("block,seed", [(128, 7), (64, 2), (128, 11), (256, 3)])
def test_library_flags_equal_oracle(block, seed):
    from long_context_sparse_block_amd import api
    from long_context_sparse_block_amd import workloads as wl
    data = wl.synthetic_bytes(3, 8192, block, seed)
    flags, sizes = api.sparse_attn_literal_flags(data, block)
    for g in range(3):
        row = data[g].tobytes()
        assert sizes[g].tolist() == literal.gzip_block_sizes(row, block)
        assert flags[g].tolist() == literal.literal_flags(row, block).tolist()


@pytest.mark.skipif(not _lib_available(), reason="library not built")
@pytest.mark.parametrize("level", [1, 6, 9])
def test_library_levels_and_edge_blocks(level):
    from long_context_sparse_block_amd import api
    rng = np.random.default_rng(level)
    data = np.stack([rng.integers(0, 256, 1024, dtype=np.uint8), np.zeros(1024, np.uint8)])
    flags, sizes = api.sparse_attn_literal_flags(data, 128, level)
    assert sizes[0].tolist() == literal.gzip_block_sizes(data[0].tobytes(), 128, level)
    assert sizes[1].tolist() == literal.gzip_block_sizes(data[1].tobytes(), 128, level)
    assert flags[1].sum() == 0  # identical blocks: none above the mean
    # a single block is never above its own mean
    f1, _ = api.sparse_attn_literal_flags(data[:1, :128], 128, level)
    assert f1.tolist() == [[0]]


@pytest.mark.skipif(not _lib_available(), reason="library not built")
def test_library_literal_flags_errors():
    import ctypes
    from long_context_sparse_block_amd import _lib as L
    lib = L.lib()
    buf = (ctypes.c_uint8 * 256)()
    out = (ctypes.c_uint8 * 4)()
    assert lib.sparse_attn_literal_flags(None, 1, 256, 64, 1, out, None) == L.SA_ERR_NULL
    assert lib.sparse_attn_literal_flags(buf, 1, 256, 64, 1, None, None) == L.SA_ERR_NULL
    assert lib.sparse_attn_literal_flags(buf, 1, 250, 64, 1, out, None) == L.SA_ERR_INVALID
    assert lib.sparse_attn_literal_flags(buf, 0, 256, 64, 1, out, None) == L.SA_ERR_INVALID
    assert lib.sparse_attn_literal_flags(buf, 1, 256, 64, 0, out, None) == L.SA_ERR_INVALID
    assert lib.sparse_attn_literal_flags(buf, 1, 256, 64, 10, out, None) == L.SA_ERR_INVALID
    assert lib.sparse_attn_literal_flags(buf, 1, 256, 0, 1, out, None) == L.SA_ERR_INVALID
    assert lib.sparse_attn_literal_flags(buf, 1, 256, 64, 1, out, None) == L.SA_OK
