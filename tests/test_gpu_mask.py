"""GPU mask builder vs the oracle: row_ptr, col_idx and the schedule must be
bit-exact."""

import random

import numpy as np
import pytest
import torch

from long_context_sparse_block_amd import api
from long_context_sparse_block_amd import workloads as wl
from oracle import block_mask as bm
from tests.gpu_util import announce, require_gpu, workload_spec

pytestmark = pytest.mark.gpu


def _check_csr(spec, what):
    announce(f"[mask] {what}: G={spec['num_groups']} nb={spec['num_blocks']}")
    m = api.sparse_attn_build_mask(spec)
    torch.cuda.synchronize()
    rp, ci, sc = bm.build(spec)
    g_rp = m.row_ptr.cpu().numpy()
    assert np.array_equal(g_rp, rp), f"{what}: row_ptr differs"
    nnz = int(rp[-1])
    assert np.array_equal(m.col_idx[:nnz].cpu().numpy(), ci), f"{what}: col_idx differs"
    assert np.array_equal(m.sched.cpu().numpy(), sc), f"{what}: schedule differs"
    return nnz


@pytest.mark.parametrize("name", list(wl.BLOCK_WORKLOADS))
def test_workload_masks_bitexact(name):
    require_gpu()
    spec = workload_spec(wl.BLOCK_WORKLOADS[name])
    nnz = _check_csr(spec, name)
    assert nnz > 0


@pytest.mark.parametrize("name", ["compression-guided", "long-context"])
def test_workload_masks_anyq_bitexact(name):
    require_gpu()
    spec = wl.mask_spec(wl.BLOCK_WORKLOADS[name], literal_mode="anyq")
    _check_csr(spec, name + "/anyq")


def test_bigbird_union_size_and_components():
    require_gpu()
    spec = wl.mask_spec(wl.BLOCK_WORKLOADS["bigbird"])
    nnz = _check_csr(spec, "bigbird")
    comp = bm.components(spec, 0)
    assert comp["window"].sum() + comp["global"].sum() + comp["random"].sum() == \
        bm.bigbird_edge_count(64, 3, 2, 3)
    assert nnz <= 636


@pytest.mark.parametrize("G", [16, 17])
def test_row_count_both_build_paths(G):
    """8192 rows (prefix sum folded into the fill) and 8704 rows (separate
    prefix-sum kernel): both bit-exact."""
    require_gpu()
    spec = dict(num_blocks=512, num_groups=G, causal=True, win_before=3, win_after=0, win_clamp=False,
                global_blocks=[0], num_random=2, random_blocks=None, literal_mode="pair",
                literal_flags=None, literal_p=0.2, seed=31)
    _check_csr(spec, f"rows={G * 512}")


def test_explicit_flags_and_draws_bitexact():
    require_gpu()
    G, nb, r = 3, 77, 4
    for causal in (True, False):
        spec = dict(num_blocks=nb, num_groups=G, causal=causal, win_before=2,
                    win_after=0 if causal else 1, win_clamp=not causal, global_blocks=[0, 40],
                    num_random=r, random_blocks=wl.random_draws(G, nb, r, causal, 5).numpy(),
                    literal_mode="pair", literal_flags=wl.random_flags(G, nb, 0.3, 6).numpy(),
                    literal_p=0.0, seed=0)
        _check_csr(spec, f"explicit causal={causal}")


def _fuzz_spec(seed):
    R = random.Random(seed)
    nb = R.choice([1, 2, 3, 63, 64, 65, 127, 200, 513])
    causal = R.random() < 0.5
    return dict(num_blocks=nb, num_groups=R.randint(1, 4), causal=causal,
                win_before=R.randint(0, 5), win_after=0 if causal else R.randint(0, 4),
                win_clamp=R.random() < 0.5,
                global_blocks=sorted(R.sample(range(nb), R.randint(0, min(4, nb)))),
                num_random=R.randint(0, 6), random_blocks=None,
                literal_mode=R.choice(["none", "pair", "anyq"]), literal_flags=None,
                literal_p=R.random(), seed=R.randint(0, 2**63))


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_masks_bitexact(seed):
    require_gpu()
    _check_csr(_fuzz_spec(seed), f"fuzz {seed}")


@pytest.mark.parametrize("causal", [True, False])
def test_presets_and_head_groups_bitexact(causal):
    require_gpu()
    G, nb = 3, 64
    flags = wl.random_flags(G, nb, 0.45, 21).numpy()
    for name in ("dense", "local-only", "longformer", "literal-pure", "gzip-guided"):
        spec = api.mask_preset(name, nb, G, causal, literal_flags=flags,
                               mask_batch_stride=1, mask_head_stride=0)
        _check_csr(spec, f"preset {name} causal={causal}")
    base = api.mask_preset("gzip-guided", nb, G, causal, literal_flags=flags,
                           mask_batch_stride=1, mask_head_stride=0)
    _check_csr(api.head_group_spec(base, 12), f"head groups causal={causal}")
    # drawn flags with a period: every head of a sequence draws the same flags
    drawn = dict(base, literal_flags=None, literal_p=0.3, seed=77)
    _check_csr(api.head_group_spec(drawn, 8), f"head groups drawn causal={causal}")
    # a period with every component on, and exclusions of globals / randoms
    bb = dict(base, global_blocks=[0, 31], num_random=2, period_exclude=[["global"], ["random"], []],
              num_groups=3 * G)
    _check_csr(bb, f"period over globals/randoms causal={causal}")


def test_exclusion_and_period_errors():
    require_gpu()
    base = api.mask_preset("local-only", 16)
    with pytest.raises(api.SparseAttnError):
        api.sparse_attn_build_mask(dict(base, exclude_parts=99))
    with pytest.raises((api.SparseAttnError, ValueError)):
        api.sparse_attn_build_mask(dict(base, period_exclude=[[]] * 65))
