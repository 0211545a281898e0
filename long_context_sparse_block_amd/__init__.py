"""MI355X (gfx950) sparse block / offset attention: HIP kernels behind a C ABI.

The library (lib/libsparse_attn.so, built by ``build.py``) exports the mask
builder, the block-sparse and offset forwards and their backward passes (see
include/sparse_attn.h); ``api`` binds them for PyTorch tensors.  ``workloads``
holds the seeded synthetic inputs.
"""

from .api import (  # noqa: F401
    BlockMask,
    SparseAttnError,
    fibonacci_base,
    head_group_spec,
    mask_preset,
    alpha_schedule,
    offset_attn_bwd,
    offset_attn_fwd,
    offset_attn_fwd_interp,
    offset_attn_make_interp,
    offset_attn_make_table,
    offset_attn_make_table_ratio,
    power2_base,
    fwd_workspace,
    row_split_for,
    split_rows_for,
    sparse_attn_bwd,
    sparse_attn_build_mask,
    sparse_attn_check_mask_desc,
    sparse_attn_fwd,
    sparse_attn_literal_flags,
    sparse_attn_mask_capacity,
    sparse_attn_mask_transpose,
)
