"""ctypes view of the C ABI declared in include/sparse_attn.h.

Loads lib/libsparse_attn.so (built in-tree by ``build.py``).  There is no
fallback: if the library is missing or cannot be loaded, every entry point
raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libsparse_attn.so")

SA_OK = 0
SA_ERR_NULL = -1
SA_ERR_INVALID = -2
SA_ERR_UNSUPPORTED = -3
SA_ERR_CAPACITY = -4
SA_ERR_HIP = -5

SA_F32 = 0
SA_BF16 = 1

SA_LIT_NONE = 0
SA_LIT_PAIR = 1
SA_LIT_ANYQ = 2

SA_PART_WINDOW = 1
SA_PART_GLOBAL = 2
SA_PART_RANDOM = 4
SA_PART_LITERAL = 8

SA_MAX_GLOBAL = 64
SA_MAX_RANDOM = 32
SA_MAX_BLOCKS = 16384
SA_MAX_OFFSETS = 128
SA_MAX_PERIOD = 64
SA_MAX_RUNGS = 64
SA_MAX_SPLIT_WAYS = 16
SA_SPLIT_COUNTERS = 16384
SA_NOALLOC_SCRATCH_BYTES = 16 << 20

# every function the header declares, with (restype, argtypes)
_i32, _i64, _f32, _f64, _u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_uint64
_p = ctypes.c_void_p


class MaskDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", _i32),
        ("num_groups", _i32),
        ("causal", _i32),
        ("win_before", _i32),
        ("win_after", _i32),
        ("win_clamp", _i32),
        ("global_blocks", ctypes.POINTER(_i32)),
        ("num_global", _i32),
        ("num_random", _i32),
        ("random_blocks", _p),
        ("literal_mode", _i32),
        ("literal_flags", _p),
        ("literal_p", _f64),
        ("seed", _u64),
        ("exclude_parts", _i32),
        ("group_period", _i32),
        ("period_exclude", _i32 * 64),
    ]


SIGNATURES = {
    "sparse_attn_mask_capacity": (_i64, [ctypes.POINTER(MaskDesc)]),
    "sparse_attn_check_mask_desc": (_i32, [ctypes.POINTER(MaskDesc)]),
    "sparse_attn_build_mask": (_i32, [ctypes.POINTER(MaskDesc), _p, _p, _i64, _p, _p]),
    "sparse_attn_fwd": (_i32, [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(_i64), _p, _p, _i64, _p, _i32, _i64, _i64, _i32,
                               _f32, _i32, _i32, _i32, _p, _i64, _p]),
    "sparse_attn_fwd_workspace_bytes": (_i64, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "sparse_attn_fwd_noalloc": (_i32, [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                       ctypes.POINTER(_i64), _p, _p, _i64, _p, _i32, _i64, _i64, _i32,
                                       _f32, _i32, _i32, _i32, _p]),
    "sparse_attn_literal_flags": (_i32, [_p, _i32, _i64, _i32, _i32, _p, _p]),
    "offset_attn_make_table": (_i32, [_i32, _f64, ctypes.POINTER(_i64), _i32, _i32,
                                      ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32)]),
    "offset_attn_fwd": (_i32, [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(_i64), ctypes.POINTER(_i32), _i32, _f32, _p]),
    "offset_attn_make_table_ratio": (_i32, [_i32, _i64, _i64, ctypes.POINTER(_i64), _i32, _i32,
                                            ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32)]),
    "offset_attn_make_interp": (_i32, [_i32, _f64, ctypes.POINTER(_i64), _i32, _i32, ctypes.POINTER(_i32), _i32,
                                       ctypes.POINTER(_i32), ctypes.POINTER(_i32), ctypes.POINTER(_f32), _i32,
                                       ctypes.POINTER(_i32)]),
    "offset_attn_fwd_interp": (_i32, [_i32, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                      ctypes.POINTER(_i64), ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32),
                                      ctypes.POINTER(_f32), _i32, _f32, _p]),
    "sparse_attn_mask_transpose": (_i32, [_i32, _i32, _p, _p, _i64, _p, _p, _i64, _p]),
    "sparse_attn_bwd_workspace_bytes": (_i64, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "sparse_attn_bwd": (_i32, [_i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(_i64), _p, _p, _i64, _p, _p, _p, _i64, _i32, _i64, _i64, _i32,
                               _f32, _p]),
    "offset_attn_bwd": (_i32, [_i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                               ctypes.POINTER(_i64), ctypes.POINTER(_i32), _i32, _f32, _p]),
    "sa_rng_key": (_u64, [_u64, _u64, _u64, _u64, _u64]),
    "sa_rng_literal": (_i32, [_u64, _u64, _u64, _f64]),
    "sa_rng_random_blocks": (_i32, [_u64, _u64, _u64, _i32, _i32, ctypes.POINTER(_i32)]),
    "sa_clock_probe": (_i32, [_p, _i64, _p]),
    "sa_status_string": (ctypes.c_char_p, [_i32]),
    "sa_last_hip_error": (ctypes.c_char_p, []),
    "sa_version": (_i32, []),
    "sa_mask_desc_layout": (_i32, [ctypes.POINTER(_i64), _i32]),
}

_lib = None


class LibraryNotBuilt(RuntimeError):
    pass


def lib():
    """The loaded library (loaded once); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_block_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(st):
    return lib().sa_status_string(st).decode()


def last_hip_error():
    return lib().sa_last_hip_error().decode()
