"""The allocation-free forward entry point (sparse_attn_fwd_noalloc) against
sparse_attn_fwd with a caller workspace: two calls in a row, the second with a
smaller input, on the same static scratch; results equal bit for bit (the
split rows merge their parts in a fixed order) and within the bf16 bars."""

import math

import pytest
import torch

from long_context_sparse_block_amd import _lib as L
from long_context_sparse_block_amd import api
from long_context_sparse_block_amd import workloads as wl
from tests.gpu_util import announce, compare, f64, require_gpu

pytestmark = pytest.mark.gpu


def _pair(w, B, H, N, seed, split_rows, split_ways):
    spec = wl.mask_spec(dict(w, B=B, H=H, N=N))
    mask = api.sparse_attn_build_mask(spec)
    q, k, v = [t.cuda() for t in wl.make_qkv(B, H, N, w["d"], torch.bfloat16, seed)]
    mbs, mhs = spec["mask_batch_stride"], spec["mask_head_stride"]
    ref = api.sparse_attn_fwd(q, k, v, mask, None, mbs, mhs, split_rows=split_rows, split_ways=split_ways)
    got = api.sparse_attn_fwd_noalloc(q, k, v, mask, None, mbs, mhs, split_rows=split_rows, split_ways=split_ways)
    torch.cuda.synchronize()
    return got, ref


def test_noalloc_matches_workspace_entry_point_two_calls():
    require_gpu()
    w = wl.BLOCK_WORKLOADS["bigbird"]
    sr, ways = api.split_rows_for(wl.mask_spec(w))
    assert sr > 0
    cases = [(w["B"], w["H"], w["N"], w["qkv_seed"], sr, ways),   # full size, the plan's split
             (1, 3, w["N"], 77, 2, 4)]                             # then a smaller input
    for B, H, N, seed, r, ways_ in cases:
        announce(f"[noalloc] bigbird B={B} H={H} N={N} split {r}x{ways_}")
        (o, lse), (o_ref, lse_ref) = _pair(w, B, H, N, seed, r, ways_)
        compare(o, lse, f64(o_ref), f64(lse_ref), torch.bfloat16, f"noalloc B={B} H={H} N={N}")
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_without_split_rows_and_capacity_error():
    """No split rows (nothing of the scratch used) gives the plain forward's
    result; a split whose workspace exceeds the scratch is refused with
    SA_ERR_CAPACITY before anything is launched (the outputs keep their fill)."""
    require_gpu()
    w = wl.BLOCK_WORKLOADS["compression-guided"]
    announce("[noalloc] compression-guided B=1 H=2, no split rows")
    (o, lse), (o_ref, lse_ref) = _pair(w, 1, 2, w["N"], 78, 0, 2)
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    lc = wl.BLOCK_WORKLOADS["long-context"]
    need = L.lib().sparse_attn_fwd_workspace_bytes(1, 16, 128, 128, 512, 16)
    assert need > L.SA_NOALLOC_SCRATCH_BYTES
    spec = wl.mask_spec(dict(lc, N=8192))
    mask = api.sparse_attn_build_mask(spec)
    q, k, v = [t.cuda() for t in wl.make_qkv(1, 16, 8192, 128, torch.bfloat16, 79)]
    o = torch.full_like(q, 7.0)
    with pytest.raises(api.SparseAttnError) as e:
        api.sparse_attn_fwd_noalloc(q, k, v, mask, None, 0, 0, out=o, split_rows=64, split_ways=16)
    assert e.value.status == L.SA_ERR_CAPACITY
    torch.cuda.synchronize()
    assert torch.all(o == 7.0)
