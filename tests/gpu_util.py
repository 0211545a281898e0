"""Helpers shared by the GPU parity tests (comparison bars and input plumbing)."""

import numpy as np
import pytest
import torch

from long_context_sparse_block_amd import _lib as L
from tests.conftest import announce

# Parity bars.  bf16 outputs: max-abs 2e-2 and mean-abs 1e-3 on O; the LSE is
# fp32 arithmetic on exact bf16 inputs and is held to 2e-3 (one bf16 unit
# roundoff, 2^-9, of the normaliser).  fp32 path: 1e-5 on both.
BF16_O_MAX = 2e-2
BF16_O_MEAN = 1e-3
BF16_LSE = 2e-3
F32_TOL = 1e-5


def workload_spec(w, **over):
    """Mask spec of a workload dict.  For gzip-sourced workloads the literal
    flags come from the library's host implementation (the product path), and
    they must equal the oracle's flags for the same bytes, bit for bit."""
    from long_context_sparse_block_amd import api
    from long_context_sparse_block_amd import workloads as wl
    from oracle import literal
    if w.get("literal_source") == "gzip" and "literal_flags" not in over:
        data = wl.synthetic_bytes(w["B"], w["N"], w["block"], w["text_seed"])
        flags, _ = api.sparse_attn_literal_flags(data, w["block"])
        ref = literal.literal_flags_batch(data, w["block"])
        assert np.array_equal(flags, ref), "gzip literal flags differ from the oracle"
        over = dict(over, literal_flags=flags)
    spec = wl.mask_spec(w, **over)
    if w.get("head_groups"):
        spec = api.head_group_spec(spec, w["H"])
    return spec


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.lib()  # raises if the HIP library is missing: no silent fallback


def to_dev(*ts):
    return [t.cuda() for t in ts]


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Assert the bars; o_ref / lse_ref are float64 numpy arrays of the same shape."""
    o = f64(o_gpu)
    lse = f64(lse_gpu)
    diff = np.abs(o - o_ref)
    inf_g, inf_r = np.isinf(lse), np.isinf(lse_ref)
    assert np.array_equal(inf_g, inf_r), f"{what}: -inf rows differ"
    if inf_r.any():
        assert np.all(lse[inf_r] < 0) and np.all(o[inf_r] == 0), f"{what}: empty rows must give o = 0"
    ld = np.abs(lse[~inf_r] - lse_ref[~inf_r]) if (~inf_r).any() else np.zeros(1)
    if dtype == torch.bfloat16:
        assert diff.max() <= BF16_O_MAX, f"{what}: O max-abs {diff.max():.3e}"
        assert diff.mean() <= BF16_O_MEAN, f"{what}: O mean-abs {diff.mean():.3e}"
        assert ld.max() <= BF16_LSE, f"{what}: LSE max-abs {ld.max():.3e}"
    else:
        assert diff.max() <= F32_TOL, f"{what}: O max-abs {diff.max():.3e}"
        assert ld.max() <= F32_TOL, f"{what}: LSE max-abs {ld.max():.3e}"
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    return diff.max(), diff.mean(), ld.max()


__all__ = ["announce", "require_gpu", "to_dev", "f64", "compare"]
