"""GPU offset attention vs the oracle: all 16 staggered calls at reduced batch,
sampled rows at full size, special tables and ragged lengths."""

import math
import random

import numpy as np
import pytest
import torch

from long_context_sparse_block_amd import api
from long_context_sparse_block_amd import workloads as wl
from oracle import offsets as oo
from tests.gpu_util import announce, compare, f64, require_gpu

pytestmark = pytest.mark.gpu

W = wl.OFFSET_WORKLOAD


def _tables(Wn, alpha, N):
    """(table the kernel gets, table the oracle uses): the product's own table
    builder feeds the kernel, as in the bench; the reference output is computed
    over the oracle's table, so a difference between the two shows up as a
    parity failure."""
    return (api.offset_attn_make_table(Wn, alpha, api.fibonacci_base(N), N),
            oo.offset_table(Wn, alpha, oo.fibonacci_base(N), N))


def _table(alpha, N):
    return _tables(W["W"], alpha, N)


@pytest.mark.parametrize("N", W["lengths"])
def test_all_alphas_reduced_batch(N):
    require_gpu()
    B, H = 1, 2
    for l, alpha in enumerate(W["alphas"]):
        offs, offs_ref = _table(alpha, N)
        q, k, v = wl.make_qkv(B, H, N, W["d"], torch.bfloat16, W["qkv_seed_base"][N] + l)
        announce(f"[offset] N={N} alpha={alpha:.4f} |D|={len(offs)}")
        o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), offs)
        torch.cuda.synchronize()
        o_ref, l_ref = oo.offset_attention(f64(q), f64(k), f64(v), offs_ref, 1 / math.sqrt(W["d"]))
        compare(o, lse, o_ref, l_ref, torch.bfloat16, f"N={N} l={l}")


@pytest.mark.parametrize("N", W["lengths"])
def test_full_size_sampled(N):
    require_gpu()
    B, H, d = W["B"], W["H"], W["d"]
    R = random.Random(N)
    samples = sorted({(0, 0, 0), (B - 1, H - 1, N - 1)} |
                     {(R.randrange(B), R.randrange(H), R.randrange(N)) for _ in range(94)})
    for l in (0, 7, 15):
        alpha = W["alphas"][l]
        offs, offs_ref = _table(alpha, N)
        q, k, v = wl.make_qkv(B, H, N, d, torch.bfloat16, W["qkv_seed_base"][N] + l)
        announce(f"[offset] full {B}x{H}x{N}x{d} l={l}")
        o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), offs)
        torch.cuda.synchronize()
        o_ref, l_ref = oo.offset_attention_rows(f64(q), f64(k), f64(v), offs_ref, 1 / math.sqrt(d), samples)
        og = torch.stack([o[b, h, t] for b, h, t in samples])
        lg = torch.stack([lse[b, h, t] for b, h, t in samples])
        compare(og, lg, o_ref, l_ref, torch.bfloat16, f"full N={N} l={l}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_lengths_and_dtypes(dtype, d):
    require_gpu()
    for N in (1, 63, 257, 1000):
        offs, offs_ref = _tables(5, 1.3, N)
        q, k, v = wl.make_qkv(2, 2, N, d, dtype, 500 + N)
        announce(f"[offset] ragged N={N} d={d} {dtype}")
        o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), offs, 0.2)
        torch.cuda.synchronize()
        o_ref, l_ref = oo.offset_attention(f64(q), f64(k), f64(v), offs_ref, 0.2)
        compare(o, lse, o_ref, l_ref, dtype, f"ragged N={N}")


def test_zero_table_is_identity_fp32():
    require_gpu()
    q, k, v = [t.cuda() for t in wl.make_qkv(1, 2, 300, 64, torch.float32, 8)]
    announce("[offset] table {0}")
    o, lse = api.offset_attn_fwd(q, k, v, [0], 0.3)
    torch.cuda.synchronize()
    assert torch.equal(o, v)


def test_full_table_is_dense_causal():
    require_gpu()
    N = 128
    q, k, v = wl.make_qkv(1, 2, N, 64, torch.float32, 9)
    announce("[offset] table {0..N-1}")
    o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), list(range(N)), 0.125)
    torch.cuda.synchronize()
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                                           is_causal=True, scale=0.125)
    assert (o.cpu().double() - ref).abs().max() < 1e-5


def test_gqa_offsets():
    require_gpu()
    q, k, v = wl.make_qkv(2, 4, 512, 64, torch.bfloat16, 10, H_kv=1)
    offs, offs_ref = _table(1.5, 512)
    announce("[offset] gqa")
    o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), offs)
    torch.cuda.synchronize()
    o_ref, l_ref = oo.offset_attention(f64(q), f64(k), f64(v), offs_ref, 0.125)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "gqa")


# Tables that exercise each part of the bf16 kernel on their own: only far
# rungs (> 64, no staged band), only near distances, distance 64 at the band's
# edge, a dense table whose 60+ far rungs take many register batches, and rows
# that stay empty (smallest distance > 0).
TABLE_CASES = {
    "far-only": [65, 100, 299],
    "near-only": list(range(9)),
    "edge-64": [64],
    "near-far-edge": [0, 63, 64, 65],
    "dense": list(range(120)),
    "sparse-near": [1, 7, 30, 57],
}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("name", sorted(TABLE_CASES))
def test_table_shapes_bf16(name, d):
    require_gpu()
    N = 300
    offs = TABLE_CASES[name]
    q, k, v = wl.make_qkv(2, 3, N, d, torch.bfloat16, 700 + len(offs) + d)
    announce(f"[offset] table {name} d={d}")
    o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), offs, 0.1)
    torch.cuda.synchronize()
    o_ref, l_ref = oo.offset_attention(f64(q), f64(k), f64(v), offs, 0.1)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, f"table {name} d={d}")


def test_strided_layout_and_negative_scale():
    """Q / K / V / O as [B, N, H, d] storage viewed as [B, H, N, d]."""
    require_gpu()
    B, H, N, d = 2, 4, 700, 64
    g = torch.Generator().manual_seed(77)
    store = [torch.randn(B, N, H, d, generator=g).to(torch.bfloat16) for _ in range(3)]
    q, k, v = [t.cuda().permute(0, 2, 1, 3) for t in store]
    offs, offs_ref = _table(1.7, N)
    announce("[offset] strided [B,N,H,d] layout, scale -0.125")
    o, lse = api.offset_attn_fwd(q, k, v, offs, -0.125)
    torch.cuda.synchronize()
    o_ref, l_ref = oo.offset_attention(f64(q.cpu()), f64(k.cpu()), f64(v.cpu()), offs_ref, -0.125)
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "strided")


def test_multi_tile_walk_ragged():
    """Enough (batch, head, tile) work that each workgroup walks several
    64-query tiles through the staged ring; N is not a multiple of 64, so the
    last walk of every head is shorter."""
    require_gpu()
    B, H, N, d = 4, 24, 4100, 64
    offs, offs_ref = _table(1.25, N)
    q, k, v = wl.make_qkv(B, H, N, d, torch.bfloat16, 4100)
    announce(f"[offset] multi-tile walk {B}x{H}x{N}x{d}")
    o, lse = api.offset_attn_fwd(q.cuda(), k.cuda(), v.cuda(), offs)
    torch.cuda.synchronize()
    o_ref, l_ref = oo.offset_attention(f64(q), f64(k), f64(v), offs_ref, 1 / math.sqrt(d))
    compare(o, lse, o_ref, l_ref, torch.bfloat16, "walk")
