"""Python binding of the C ABI: argument marshalling only.

Tensors come from PyTorch (device memory and the current HIP stream); every
step of the computation runs in the library's HIP kernels.  The functions keep
the names of the C entry points.
"""

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib as L

_LIT_MODES = {"none": L.SA_LIT_NONE, "pair": L.SA_LIT_PAIR, "anyq": L.SA_LIT_ANYQ}


class SparseAttnError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        text = L.status_string(status)
        if status == L.SA_ERR_HIP:
            text += ": " + L.last_hip_error()
        super().__init__(f"{what}: {text} ({status})")


def _check(status, what):
    if status != L.SA_OK:
        raise SparseAttnError(status, what)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


@dataclass
class BlockMask:
    """CSR key-block lists on the device (see sparse_attn_build_mask)."""
    row_ptr: torch.Tensor   # int32 [G * N_b + 1]
    col_idx: torch.Tensor   # int32 [capacity]
    sched: torch.Tensor     # int32 [G, N_b] or None
    num_groups: int
    num_blocks: int
    causal: bool


def _mask_desc(spec, device, keep):
    """sa_mask_desc from a plain-dict mask spec; device inputs are appended to keep."""
    d = L.MaskDesc()
    d.num_blocks = int(spec["num_blocks"])
    d.num_groups = int(spec["num_groups"])
    d.causal = int(bool(spec["causal"]))
    d.win_before = int(spec.get("win_before") or 0)
    d.win_after = int(spec.get("win_after") or 0)
    d.win_clamp = int(bool(spec.get("win_clamp")))
    gl = [int(x) for x in (spec.get("global_blocks") or [])]
    arr = (ctypes.c_int32 * max(1, len(gl)))(*gl)
    keep.append(arr)
    d.global_blocks = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    d.num_global = len(gl)
    d.num_random = int(spec.get("num_random") or 0)
    rb = spec.get("random_blocks")
    if rb is not None:
        t = torch.as_tensor(rb).to(device=device, dtype=torch.int32).contiguous()
        keep.append(t)
        d.random_blocks = t.data_ptr()
    d.literal_mode = _LIT_MODES[spec.get("literal_mode") or "none"]
    lf = spec.get("literal_flags")
    if lf is not None:
        t = torch.as_tensor(lf).to(device=device, dtype=torch.uint8).contiguous()
        keep.append(t)
        d.literal_flags = t.data_ptr()
    d.literal_p = float(spec.get("literal_p") or 0.0)
    d.seed = int(spec.get("seed") or 0) & ((1 << 64) - 1)
    d.exclude_parts = _parts(spec.get("exclude_parts"))
    pe = spec.get("period_exclude") or []
    if len(pe) > L.SA_MAX_PERIOD:
        raise ValueError("period_exclude longer than SA_MAX_PERIOD")
    d.group_period = len(pe)
    for n, parts in enumerate(pe):
        d.period_exclude[n] = _parts(parts)
    return d


_PARTS = {"window": L.SA_PART_WINDOW, "global": L.SA_PART_GLOBAL, "random": L.SA_PART_RANDOM,
          "literal": L.SA_PART_LITERAL}


def _parts(names):
    """SA_PART_* bits of a list of component names (or an int)."""
    if names is None:
        return 0
    if isinstance(names, int):
        return names
    bits = 0
    for n in names:
        bits |= _PARTS[n]
    return bits


def mask_preset(name, num_blocks, num_groups=1, causal=True, **over):
    """Mask spec of an attention variant the compression paper compares (Sec. 4.2).

    "dense" (every earlier block), "local-only" (+-1-block window),
    "longformer" (+-4-block window, a global block every 8 blocks),
    "literal-pure" (literal-to-literal pairs and the identity, no window: the
    band |i - j| <= w of M^lit is then empty), "gzip-guided" (literal pairs and
    a +-1-block window).  Literal flags go in ``literal_flags`` (e.g. from
    sparse_attn_literal_flags) or are drawn with ``literal_p``.
    """
    w = {"dense": num_blocks, "local-only": 1, "longformer": 4, "literal-pure": 0, "gzip-guided": 1}
    if name not in w:
        raise ValueError(f"unknown preset {name!r}")
    spec = dict(num_blocks=num_blocks, num_groups=num_groups, causal=causal, win_before=w[name],
                win_after=0 if causal else w[name], win_clamp=False, global_blocks=[], num_random=0,
                random_blocks=None, literal_mode="none", literal_flags=None, literal_p=0.0, seed=0)
    if name == "longformer":
        spec["global_blocks"] = list(range(0, num_blocks, 8))
    if name in ("literal-pure", "gzip-guided"):
        spec["literal_mode"] = "pair"
    spec.update(over)
    return spec


def head_group_spec(spec, H, local=0.5, long_range=0.25):
    """Per-head masks of the compression paper's head groups (Sec. 3.3).

    Heads [0, L) are local (window U I), [L, L + R) long-range (literal U I),
    the rest hybrid (the full mask), with L = floor(local H), R = floor(long_range
    H) (12 heads: 6, 3, 3).  The result has one mask group per (group of
    ``spec``, head): G' = G H, group g = g0 H + h, and every head of a group
    shares its literal flags.  Pass its mask_batch_stride / mask_head_stride to
    sparse_attn_fwd.
    """
    L_, R_ = int(local * H), int(long_range * H)
    pe = [["literal"]] * L_ + [["window"]] * R_ + [[]] * (H - L_ - R_)
    out = dict(spec, num_groups=spec["num_groups"] * H, period_exclude=pe)
    out["mask_batch_stride"] = int(spec.get("mask_batch_stride") or 0) * H
    out["mask_head_stride"] = 1
    return out


def sparse_attn_mask_capacity(spec):
    keep = []
    d = _mask_desc(spec, "cpu", keep)
    cap = L.lib().sparse_attn_mask_capacity(ctypes.byref(d))
    if cap < 0:
        raise SparseAttnError(int(cap), "sparse_attn_mask_capacity")
    return int(cap)


def sparse_attn_check_mask_desc(spec):
    keep = []
    d = _mask_desc(spec, "cpu", keep)
    return int(L.lib().sparse_attn_check_mask_desc(ctypes.byref(d)))


def sparse_attn_build_mask(spec, device=None, schedule=True):
    """Build the CSR block mask of ``spec`` on ``device`` (default: current GPU)."""
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    keep = []
    d = _mask_desc(spec, device, keep)
    cap = L.lib().sparse_attn_mask_capacity(ctypes.byref(d))
    if cap < 0:
        raise SparseAttnError(int(cap), "sparse_attn_build_mask")
    R = d.num_groups * d.num_blocks
    row_ptr = torch.empty(R + 1, dtype=torch.int32, device=device)
    col_idx = torch.empty(max(1, cap), dtype=torch.int32, device=device)
    sched = torch.empty((d.num_groups, d.num_blocks), dtype=torch.int32, device=device) if schedule else None
    st = L.lib().sparse_attn_build_mask(ctypes.byref(d), _ptr(row_ptr), _ptr(col_idx), cap,
                                        _ptr(sched), _stream(device))
    _check(st, "sparse_attn_build_mask")
    return BlockMask(row_ptr, col_idx, sched, d.num_groups, d.num_blocks, bool(d.causal))


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return L.SA_BF16
    if t.dtype == torch.float32:
        return L.SA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check_qkv(q, k, v):
    for t in (q, k, v):
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if t.dim() != 4 or t.stride(-1) != 1:
            raise ValueError("tensors must be [B, H, N, d] with d contiguous")
        if t.device != q.device or t.dtype != q.dtype:
            raise ValueError("q, k, v must share device and dtype")
    B, H, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k, v must be [B, H_kv, N, d]")
    return B, H, k.shape[1], N, d


def _strides(*ts):
    vals = []
    for t in ts:
        vals += [t.stride(0), t.stride(1), t.stride(2)]
    return (ctypes.c_int64 * len(vals))(*vals)


def row_split_for(spec):
    """Wave groups per mask row for the bf16 forward: 1.  Rows much longer than
    the rest (the global rows of a non-causal mask) are split over several
    workgroups instead (split_rows_for), which measured faster than splitting
    every row over two wave groups (row_split = 2, still available)."""
    return 1


def split_rows_for(spec, row_split=1):
    """(split_rows, split_ways) for the bf16 forward: the rows at the first
    split_rows launch positions of every head (the longest ones) are each run
    by split_ways workgroups.  Used for non-causal masks with global blocks,
    whose global rows list every block while the other rows list about
    window + globals + random ones: those rows are split into as many parts
    (2 .. 16) as make a part about as long as an ordinary row.  (0, 2)
    otherwise, and with row_split = 2."""
    glob = len(spec.get("global_blocks") or [])
    if row_split != 1 or spec.get("causal", True) or glob == 0:
        return 0, 2
    nb = int(spec["num_blocks"])
    ordinary = int(spec.get("win_before") or 0) + int(spec.get("win_after") or 0) + 1 + glob + \
        int(spec.get("num_random") or 0)
    ways = max(2, min(L.SA_MAX_SPLIT_WAYS, -(-nb // max(1, ordinary))))
    return min(glob, nb), ways


def fwd_workspace(B, H, d, block, split_rows, split_ways, device):
    """Zero-filled uint8 workspace for sparse_attn_fwd's split rows (None when
    split_rows is 0).  Its counter area has a fixed size and every launch
    leaves it zero, so it can be reused by later launches of any split shape
    whose sparse_attn_fwd_workspace_bytes it covers (one launch at a time)."""
    n = L.lib().sparse_attn_fwd_workspace_bytes(B, H, d, block, int(split_rows), int(split_ways))
    if n < 0:
        raise SparseAttnError(int(n), "sparse_attn_fwd_workspace_bytes")
    return torch.zeros(n, dtype=torch.uint8, device=device) if n > 0 else None


def sparse_attn_fwd(q, k, v, mask, scale=None, mask_batch_stride=0, mask_head_stride=0,
                    use_schedule=True, out=None, lse=None, row_split=1, split_rows=0, split_ways=2,
                    workspace=None):
    """Block-sparse attention; returns (o, lse).  ``mask`` is a BlockMask;
    ``row_split`` (1 or 2), ``split_rows`` and ``split_ways`` as for the C entry
    point (see row_split_for, split_rows_for).  A zero-filled workspace is
    allocated when split_rows > 0 and none is given."""
    B, H, Hkv, N, d = _check_qkv(q, k, v)
    if N % mask.num_blocks:
        raise ValueError("N must be a multiple of the number of mask blocks")
    block = N // mask.num_blocks
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    sched = mask.sched if use_schedule else None
    if split_rows > 0 and workspace is None and q.dtype == torch.bfloat16:
        workspace = fwd_workspace(B, H, d, block, split_rows, split_ways, q.device)
    st = L.lib().sparse_attn_fwd(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, d, block,
        _strides(q, k, v, o), _ptr(mask.row_ptr), _ptr(mask.col_idx), mask.col_idx.numel(),
        _ptr(sched), mask.num_groups, mask_batch_stride, mask_head_stride, int(mask.causal),
        scale, int(row_split), int(split_rows), int(split_ways), _ptr(workspace),
        workspace.numel() if workspace is not None else 0, _stream(q.device))
    _check(st, "sparse_attn_fwd")
    return o, lse_t


def sparse_attn_fwd_noalloc(q, k, v, mask, scale=None, mask_batch_stride=0, mask_head_stride=0,
                            use_schedule=True, out=None, lse=None, row_split=1, split_rows=0, split_ways=2):
    """sparse_attn_fwd through the entry point that allocates nothing on the
    device (its split-row workspace is the library's static scratch);
    returns (o, lse).  Pass ``out`` and ``lse`` to allocate nothing here
    either."""
    B, H, Hkv, N, d = _check_qkv(q, k, v)
    if N % mask.num_blocks:
        raise ValueError("N must be a multiple of the number of mask blocks")
    block = N // mask.num_blocks
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    sched = mask.sched if use_schedule else None
    st = L.lib().sparse_attn_fwd_noalloc(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t), B, H, Hkv, N, d, block,
        _strides(q, k, v, o), _ptr(mask.row_ptr), _ptr(mask.col_idx), mask.col_idx.numel(),
        _ptr(sched), mask.num_groups, mask_batch_stride, mask_head_stride, int(mask.causal),
        scale, int(row_split), int(split_rows), int(split_ways), _stream(q.device))
    _check(st, "sparse_attn_fwd_noalloc")
    return o, lse_t


def sparse_attn_mask_transpose(mask):
    """(col_ptr int32 [G*N_b+1], row_idx int32 [capacity]) device tensors: for
    each key block the ascending query blocks whose row lists it."""
    G, nb = mask.num_groups, mask.num_blocks
    col_ptr = torch.empty(G * nb + 1, dtype=torch.int32, device=mask.row_ptr.device)
    row_idx = torch.empty(mask.col_idx.numel(), dtype=torch.int32, device=mask.row_ptr.device)
    st = L.lib().sparse_attn_mask_transpose(G, nb, _ptr(mask.row_ptr), _ptr(mask.col_idx), mask.col_idx.numel(),
                                            _ptr(col_ptr), _ptr(row_idx), row_idx.numel(),
                                            _stream(mask.row_ptr.device))
    _check(st, "sparse_attn_mask_transpose")
    return col_ptr, row_idx


def _grad_outputs(q, k):
    return (torch.empty_like(q, memory_format=torch.contiguous_format),
            torch.empty_like(k, memory_format=torch.contiguous_format),
            torch.empty_like(k, memory_format=torch.contiguous_format),
            torch.empty(q.shape[:3], dtype=torch.float32, device=q.device))


def _bwd_workspace(B, H, Hkv, N, d, block, device):
    n = L.lib().sparse_attn_bwd_workspace_bytes(B, H, Hkv, N, d, block)
    if n < 0:
        raise SparseAttnError(int(n), "sparse_attn_bwd_workspace_bytes")
    return torch.empty(int(n), dtype=torch.uint8, device=device)


def sparse_attn_bwd(q, k, v, o, lse, dout, mask, transpose=None, scale=None, mask_batch_stride=0,
                    mask_head_stride=0, use_schedule=True):
    """Gradients (dq, dk, dv) of block-sparse attention; ``transpose`` is the
    result of sparse_attn_mask_transpose(mask) (computed when omitted); the
    dQ rows run in the mask's launch order when it has one and
    ``use_schedule``."""
    B, H, Hkv, N, d = _check_qkv(q, k, v)
    block = N // mask.num_blocks
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    col_ptr, row_idx = transpose if transpose is not None else sparse_attn_mask_transpose(mask)
    dq, dk, dv, _ = _grad_outputs(q, k)
    ws = _bwd_workspace(B, H, Hkv, N, d, block, q.device)
    st = L.lib().sparse_attn_bwd(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(ws), ws.numel(), B, H, Hkv, N, d, block, _strides(q, k, v, o, dout, dq, dk, dv), _ptr(mask.row_ptr),
        _ptr(mask.col_idx), mask.col_idx.numel(), _ptr(mask.sched if use_schedule else None), _ptr(col_ptr),
        _ptr(row_idx), row_idx.numel(), mask.num_groups, mask_batch_stride, mask_head_stride, int(mask.causal),
        scale, _stream(q.device))
    _check(st, "sparse_attn_bwd")
    return dq, dk, dv


def offset_attn_bwd(q, k, v, o, lse, dout, offsets, scale=None):
    """Gradients (dq, dk, dv) of offset attention over ``offsets``."""
    B, H, Hkv, N, d = _check_qkv(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    offs = [int(x) for x in offsets]
    arr = (ctypes.c_int32 * max(1, len(offs)))(*offs)
    dq, dk, dv, delta = _grad_outputs(q, k)
    st = L.lib().offset_attn_bwd(
        _dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(delta), B, H, Hkv, N, d, _strides(q, k, v, o, dout, dq, dk, dv), arr, len(offs), scale,
        _stream(q.device))
    _check(st, "offset_attn_bwd")
    return dq, dk, dv


def sparse_attn_literal_flags(data, block_bytes, level=1):
    """Literal flags of byte sequences by per-block gzip size (C, host only).

    ``data``: bytes (one sequence) or a uint8 numpy array [G, n_bytes].
    Returns (flags uint8 [G, B], sizes int32 [G, B]) as numpy arrays.
    """
    import numpy as np
    arr = np.frombuffer(data, dtype=np.uint8)[None, :] if isinstance(data, (bytes, bytearray)) else np.asarray(data)
    if arr.dtype != np.uint8 or arr.ndim != 2:
        raise ValueError("data must be bytes or a uint8 array [G, n_bytes]")
    arr = np.ascontiguousarray(arr)
    G, n = arr.shape
    nb = n // int(block_bytes) if block_bytes > 0 else 0
    flags = np.zeros((G, max(nb, 1)), dtype=np.uint8)
    sizes = np.zeros((G, max(nb, 1)), dtype=np.int32)
    st = L.lib().sparse_attn_literal_flags(arr.ctypes.data_as(ctypes.c_void_p), G, n, int(block_bytes),
                                           int(level), flags.ctypes.data_as(ctypes.c_void_p),
                                           sizes.ctypes.data_as(ctypes.c_void_p))
    _check(st, "sparse_attn_literal_flags")
    return flags[:, :nb], sizes[:, :nb]


def fibonacci_base(limit):
    """1, 2, 3, 5, 8, ... below ``limit`` (the rung base of the offset pattern)."""
    out, a, b = [], 1, 2
    while a < limit:
        out.append(a)
        a, b = b, a + b
    return out


def offset_attn_make_table(W, alpha, base, N):
    """Sorted distinct distances {0..W} U {floor(alpha f + 1/2)} below N (C helper)."""
    K = len(base)
    b = (ctypes.c_int64 * max(1, K))(*[int(x) for x in base])
    cap = W + 1 + K
    out = (ctypes.c_int32 * max(1, cap))()
    cnt = ctypes.c_int32(0)
    st = L.lib().offset_attn_make_table(int(W), float(alpha), b, K, int(N), out, cap, ctypes.byref(cnt))
    _check(st, "offset_attn_make_table")
    return [out[i] for i in range(cnt.value)]


def power2_base(limit):
    """1, 2, 4, 8, ... below ``limit`` (the reach-matched power-of-2 control base)."""
    out, x = [], 1
    while x < limit:
        out.append(x)
        x *= 2
    return out


def alpha_schedule(kind, L=16, S=7):
    """Per-layer alpha of the offset pattern: "fixed" (1 everywhere), "linear"
    (0.5 + l/(L - 1)) or "coprime" (layer l takes the linear value of index
    S*l mod L)."""
    lin = [0.5 + l / (L - 1) for l in range(L)]
    if kind == "fixed":
        return [1.0] * L
    if kind == "linear":
        return lin
    if kind == "coprime":
        return [lin[(S * l) % L] for l in range(L)]
    raise ValueError(kind)


def offset_attn_make_table_ratio(W, num, den, base, N):
    """offset_attn_make_table for alpha = num/den held exactly (C helper)."""
    K = len(base)
    b = (ctypes.c_int64 * max(1, K))(*[int(x) for x in base])
    cap = W + 1 + K
    out = (ctypes.c_int32 * max(1, cap))()
    cnt = ctypes.c_int32(0)
    st = L.lib().offset_attn_make_table_ratio(int(W), int(num), int(den), b, K, int(N), out, cap,
                                              ctypes.byref(cnt))
    _check(st, "offset_attn_make_table_ratio")
    return [out[i] for i in range(cnt.value)]


def offset_attn_make_interp(W, alpha, base, N):
    """(integer distances, [(floor, weight)]) for continuous rungs alpha*f (C helper)."""
    K = len(base)
    b = (ctypes.c_int64 * max(1, K))(*[int(x) for x in base])
    cap = W + 1 + K
    out = (ctypes.c_int32 * max(1, cap))()
    rf = (ctypes.c_int32 * max(1, K))()
    rw = (ctypes.c_float * max(1, K))()
    cnt, rc = ctypes.c_int32(0), ctypes.c_int32(0)
    st = L.lib().offset_attn_make_interp(int(W), float(alpha), b, K, int(N), out, cap, ctypes.byref(cnt),
                                         rf, rw, K, ctypes.byref(rc))
    _check(st, "offset_attn_make_interp")
    return [out[i] for i in range(cnt.value)], [(rf[i], rw[i]) for i in range(rc.value)]


def offset_attn_fwd_interp(q, k, v, offsets, rungs, scale=None, out=None, lse=None):
    """Offset attention with interpolated rungs ``rungs`` = [(floor, weight)]."""
    B, H, Hkv, N, d = _check_qkv(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    offs = [int(x) for x in offsets]
    arr = (ctypes.c_int32 * max(1, len(offs)))(*offs)
    rf = (ctypes.c_int32 * max(1, len(rungs)))(*[int(a) for a, _ in rungs])
    rw = (ctypes.c_float * max(1, len(rungs)))(*[float(w) for _, w in rungs])
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = L.lib().offset_attn_fwd_interp(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                        B, H, Hkv, N, d, _strides(q, k, v, o), arr, len(offs), rf, rw, len(rungs),
                                        scale, _stream(q.device))
    _check(st, "offset_attn_fwd_interp")
    return o, lse_t


def offset_attn_fwd(q, k, v, offsets, scale=None, out=None, lse=None):
    """Offset attention; ``offsets`` a host list of ascending distances."""
    B, H, Hkv, N, d = _check_qkv(q, k, v)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    offs = [int(x) for x in offsets]
    arr = (ctypes.c_int32 * max(1, len(offs)))(*offs)
    o = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    lse_t = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = L.lib().offset_attn_fwd(_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse_t),
                                 B, H, Hkv, N, d, _strides(q, k, v, o), arr, len(offs), scale,
                                 _stream(q.device))
    _check(st, "offset_attn_fwd")
    return o, lse_t


def capture_graph(fn):
    """Record the launches fn() makes on the current device into a HIP graph
    (torch.cuda.CUDAGraph; replay() re-issues them).  fn runs once eagerly on a
    side stream first, so one-time set-up happens outside the capture.  The
    library's launches contain no memset or allocation, so a plan's calls can
    be captured as they are."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


class BlockSparsePlan:
    """Preallocated buffers and pre-marshalled arguments for repeated
    (mask build, block-sparse forward) steps on fixed shapes.

    ``build_mask()`` and ``forward()`` each make one C call and allocate
    nothing; outputs land in ``self.mask``, ``self.o`` and ``self.lse``.
    ``row_split`` defaults to ``row_split_for(spec)``, (``split_rows``,
    ``split_ways``) to ``split_rows_for(spec, row_split)`` (no split rows
    without a launch schedule or for fp32); the split-row workspace is
    allocated once, zero-filled.
    """

    def __init__(self, spec, q, k, v, scale=None, use_schedule=True, row_split=None, split_rows=None,
                 split_ways=None):
        B, H, Hkv, N, d = _check_qkv(q, k, v)
        self.device = q.device
        self._keep = []
        self._desc = _mask_desc(spec, q.device, self._keep)
        cap = L.lib().sparse_attn_mask_capacity(ctypes.byref(self._desc))
        if cap < 0:
            raise SparseAttnError(int(cap), "BlockSparsePlan")
        G, nb = self._desc.num_groups, self._desc.num_blocks
        if N % nb:
            raise ValueError("N must be a multiple of the number of mask blocks")
        self.mask = BlockMask(torch.empty(G * nb + 1, dtype=torch.int32, device=q.device),
                              torch.empty(max(1, cap), dtype=torch.int32, device=q.device),
                              torch.empty((G, nb), dtype=torch.int32, device=q.device) if use_schedule else None,
                              G, nb, bool(self._desc.causal))
        self.q, self.k, self.v = q, k, v
        self.o = torch.empty_like(q, memory_format=torch.contiguous_format)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        self.scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self.mbs = int(spec.get("mask_batch_stride", 0))
        self.mhs = int(spec.get("mask_head_stride", 0))
        self.row_split = row_split_for(spec) if row_split is None else int(row_split)
        auto_rows, auto_ways = split_rows_for(spec, self.row_split) if use_schedule else (0, 2)
        self.split_rows = int(auto_rows if split_rows is None else split_rows) if q.dtype == torch.bfloat16 else 0
        self.split_ways = int(auto_ways if split_ways is None else split_ways)
        self.workspace = fwd_workspace(B, H, d, N // nb, self.split_rows, self.split_ways, q.device)
        self._fwd_args = (_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(self.o), _ptr(self.lse), B, H,
                          Hkv, N, d, N // nb, _strides(q, k, v, self.o), _ptr(self.mask.row_ptr),
                          _ptr(self.mask.col_idx), self.mask.col_idx.numel(), _ptr(self.mask.sched),
                          G, self.mbs, self.mhs, int(self._desc.causal), self.scale,
                          self.row_split, self.split_rows, self.split_ways, _ptr(self.workspace),
                          self.workspace.numel() if self.workspace is not None else 0)
        self._mask_args = (ctypes.byref(self._desc), _ptr(self.mask.row_ptr), _ptr(self.mask.col_idx),
                           self.mask.col_idx.numel(), _ptr(self.mask.sched))
        self._lib = L.lib()

    def build_mask(self):
        _check(self._lib.sparse_attn_build_mask(*self._mask_args, _stream(self.device)), "sparse_attn_build_mask")

    def forward(self):
        _check(self._lib.sparse_attn_fwd(*self._fwd_args, _stream(self.device)), "sparse_attn_fwd")

    def __call__(self):
        self.build_mask()
        self.forward()
        return self.o, self.lse


class BlockSparseBwdPlan:
    """Pre-marshalled sparse_attn_bwd call on the buffers of a BlockSparsePlan
    (its forward outputs o, lse) and an upstream gradient ``dout``; the mask
    transpose is built once (``transpose()`` rebuilds it after a new mask)."""

    def __init__(self, plan, dout):
        B, H, Hkv, N, d = _check_qkv(plan.q, plan.k, plan.v)
        self.device, self.plan, self.dout = plan.device, plan, dout
        m = plan.mask
        self.col_ptr = torch.empty(m.num_groups * m.num_blocks + 1, dtype=torch.int32, device=self.device)
        self.row_idx = torch.empty(m.col_idx.numel(), dtype=torch.int32, device=self.device)
        self.dq, self.dk, self.dv, _ = _grad_outputs(plan.q, plan.k)
        self.ws = _bwd_workspace(B, H, Hkv, N, d, N // m.num_blocks, self.device)
        self._lib = L.lib()
        self._tr_args = (m.num_groups, m.num_blocks, _ptr(m.row_ptr), _ptr(m.col_idx), m.col_idx.numel(),
                         _ptr(self.col_ptr), _ptr(self.row_idx), self.row_idx.numel())
        q, k, v = plan.q, plan.k, plan.v
        self._args = (_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(plan.o), _ptr(plan.lse), _ptr(dout),
                      _ptr(self.dq), _ptr(self.dk), _ptr(self.dv), _ptr(self.ws), self.ws.numel(), B, H, Hkv, N, d,
                      N // m.num_blocks, _strides(q, k, v, plan.o, dout, self.dq, self.dk, self.dv),
                      _ptr(m.row_ptr), _ptr(m.col_idx), m.col_idx.numel(), _ptr(m.sched), _ptr(self.col_ptr),
                      _ptr(self.row_idx),
                      self.row_idx.numel(), m.num_groups, plan.mbs, plan.mhs, int(m.causal), plan.scale)
        self.transpose()

    def transpose(self):
        _check(self._lib.sparse_attn_mask_transpose(*self._tr_args, _stream(self.device)),
               "sparse_attn_mask_transpose")

    def __call__(self):
        _check(self._lib.sparse_attn_bwd(*self._args, _stream(self.device)), "sparse_attn_bwd")
        return self.dq, self.dk, self.dv


class OffsetBwdPlan:
    """Pre-marshalled offset_attn_bwd call on the buffers of an OffsetPlan."""

    def __init__(self, plan, offsets, dout, scale=None):
        q, k, v = plan.q, plan.k, plan.v
        B, H, Hkv, N, d = _check_qkv(q, k, v)
        self.device = plan.device
        offs = [int(x) for x in offsets]
        self._arr = (ctypes.c_int32 * max(1, len(offs)))(*offs)
        self.dq, self.dk, self.dv, self.delta = _grad_outputs(q, k)
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        self._args = (_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(plan.o), _ptr(plan.lse), _ptr(dout),
                      _ptr(self.dq), _ptr(self.dk), _ptr(self.dv), _ptr(self.delta), B, H, Hkv, N, d,
                      _strides(q, k, v, plan.o, dout, self.dq, self.dk, self.dv), self._arr, len(offs), scale)
        self._lib = L.lib()

    def __call__(self):
        _check(self._lib.offset_attn_bwd(*self._args, _stream(self.device)), "offset_attn_bwd")
        return self.dq, self.dk, self.dv


class OffsetPlan:
    """Pre-marshalled offset_attn_fwd call on fixed tensors (allocates nothing per call)."""

    def __init__(self, q, k, v, offsets, scale=None, rungs=None):
        B, H, Hkv, N, d = _check_qkv(q, k, v)
        self.device = q.device
        self.q, self.k, self.v = q, k, v
        offs = [int(x) for x in offsets]
        self._arr = (ctypes.c_int32 * max(1, len(offs)))(*offs)
        self.o = torch.empty_like(q, memory_format=torch.contiguous_format)
        self.lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
        head = (_dtype_code(q), _ptr(q), _ptr(k), _ptr(v), _ptr(self.o), _ptr(self.lse), B, H, Hkv,
                N, d, _strides(q, k, v, self.o), self._arr, len(offs))
        self._lib = L.lib()
        if rungs is None:
            self._fn, self._name = self._lib.offset_attn_fwd, "offset_attn_fwd"
            self._args = head + (scale,)
        else:
            self._rf = (ctypes.c_int32 * max(1, len(rungs)))(*[int(a) for a, _ in rungs])
            self._rw = (ctypes.c_float * max(1, len(rungs)))(*[float(w) for _, w in rungs])
            self._fn, self._name = self._lib.offset_attn_fwd_interp, "offset_attn_fwd_interp"
            self._args = head + (self._rf, self._rw, len(rungs), scale)

    def __call__(self):
        _check(self._fn(*self._args, _stream(self.device)), self._name)
        return self.o, self.lse
