"""Benchmark of the sparse-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--trials T]
                    [--no-secondary] [--no-cpu-baseline]

One step = the whole hot path on one batch of the long-context workload (the
largest configuration that fits one GPU): block mask built on the device into
CSR (causal, own + 2 previous blocks, 4 global prefix blocks, literal-pair
blocks Bernoulli(0.15) shared by all heads), then the block-sparse attention
forward, bf16, B=1 H=16 N=65536 d=128, block 128.  Inputs are resident in HBM
before timing starts.  The value is algorithmic TFLOP/s: 4 * d * (unmasked
query/key pairs) per step / step time (a diagonal block counts b(b+1)/2 pairs,
blocks after the query block none).

W untimed warm-up steps, then exactly K timed steps between two device
synchronisations (HIP events on the launch stream).  The roofline figure is the
forward kernel alone: the median over T trials of back-to-back launches.

Prints ONE JSON line.  The other workloads (compression-guided with both
readings of the literal rule, BigBird with and without a captured graph, the
tiny fp32 case, gzip-guided with and without head groups, the long-context
literal variant, both backward passes, the Fibonacci offsets at both lengths
and their variants) are measured in the same run, each with the fp64 CPU
oracle timed on a bounded sample of the same workload, under "secondary".
"""

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from long_context_sparse_block_amd import _lib as L  # noqa: E402
from long_context_sparse_block_amd import api  # noqa: E402
from long_context_sparse_block_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "effective TFLOP/s on unmasked blocks (% of bf16 MFMA peak); offset-attn GB/s"
HEADLINE = "long-context"
PROFILE_DIR = os.path.join(ROOT, "profiles")
WALL_CLOCK_MHZ = 100.0      # s_memrealtime rate on MI355X (hipDeviceAttributeWallClockRate)


# ----------------------------------------------------------------- helpers --

def unmasked_pairs_per_group(row_ptr, col_idx, nb, block, causal):
    """Unmasked (query, key) token pairs of every mask group, from the CSR."""
    rp = np.asarray(row_ptr, dtype=np.int64)
    ci = np.asarray(col_idx[: int(rp[-1])], dtype=np.int64)
    G = (len(rp) - 1) // nb
    out = []
    full, diag = block * block, block * (block + 1) // 2
    for g in range(G):
        tot = 0
        for i in range(nb):
            cols = ci[rp[g * nb + i]: rp[g * nb + i + 1]]
            cols = cols[(cols >= 0) & (cols < nb)]
            if causal:
                tot += full * int((cols < i).sum()) + diag * int((cols == i).sum())
            else:
                tot += full * cols.size
        out.append(tot)
    return out


def events_ms(fn, iters):
    """Average ms of fn() over iters back-to-back calls (HIP events on the current stream,
    the stream every launch of this library goes to)."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def median_ms(fn, iters, trials):
    """Median over `trials` of the per-call ms of `iters` back-to-back calls."""
    return statistics.median(events_ms(fn, iters) for _ in range(trials))


def read_profile_record(kernel_tag, kind):
    """A stored rocprofv3 figure (profiles/<tag>_<kind>.txt, last JSON line) if it
    still matches the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"{kernel_tag}_{kind}.txt")
    if not os.path.exists(path):
        return None
    rec = None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            rec = json.loads(line)
    if not rec:
        return None
    src = os.path.join(ROOT, "long_context_sparse_block_amd", "csrc", rec.get("source", ""))
    if not os.path.exists(src):
        return None
    import hashlib
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec.get("source_sha256"):
        return None
    return rec


def host_info():
    """What the CPU baseline ran on."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)), "blas_threads": blas,
            "torch_threads": torch.get_num_threads()}


class ClockProbe:
    """Shader clock measured beside a workload: one probe wave on a second stream
    counts shader cycles while a given wall time passes (sa_clock_probe)."""

    def __init__(self):
        self.buf = torch.zeros(2, dtype=torch.int64, device="cuda")
        self.stream = torch.cuda.Stream()

    def start(self, seconds):
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            st = L.lib().sa_clock_probe(ctypes.c_void_p(self.buf.data_ptr()), int(seconds * WALL_CLOCK_MHZ * 1e6),
                                        ctypes.c_void_p(self.stream.cuda_stream))
        if st != L.SA_OK:
            raise RuntimeError(f"sa_clock_probe: {L.status_string(st)}")

    def mhz(self):
        self.stream.synchronize()
        cyc, ticks = [int(x) for x in self.buf.cpu()]
        return round(cyc / ticks * WALL_CLOCK_MHZ, 1) if ticks > 0 else None


def gemm_reference(n=8192, iters=50):
    """Dense bf16 GEMM rate of the vendor library (torch.matmul -> hipBLASLt)
    on this GPU, with iid N(0, 1) operands (the distribution of every workload
    here) and with all-ones operands.  The same GEMM runs markedly faster on
    constant operands, so the random-data rate is the practical ceiling that
    random-data MFMA work meets on this GPU; it is context for the roofline
    fractions, not part of the attention path."""
    g = torch.Generator(device="cuda").manual_seed(7)
    out = {"n": n}
    for name, mk in (("normal", lambda: torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)),
                     ("ones", lambda: torch.ones(n, n, device="cuda", dtype=torch.bfloat16))):
        a, b = mk(), mk().t().contiguous().t()  # B column-major: the library's faster layout here
        for _ in range(5):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        out[f"tflops_{name}"] = round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b
    out["frac_of_peak_normal"] = round(out["tflops_normal"] / PEAK_BF16_TFLOPS, 3)
    torch.cuda.empty_cache()
    return out


# -------------------------------------------------------- oracle baselines --

def _sample_rows(rp, nb, G, stride):
    """CSR with only every `stride`-th row of each group kept (the others empty)."""
    rp = np.asarray(rp, dtype=np.int64)
    keep = np.zeros(G * nb, dtype=bool)
    keep[::stride] = True
    lens = np.diff(rp) * keep
    new_rp = np.concatenate([[0], np.cumsum(lens)])
    return new_rp, keep


def cpu_block_forward(res, budget_s):
    """fp64 CSR-gather oracle on whole (batch, head) slices of a block workload,
    as many as fit in the budget (at least one)."""
    from oracle import attention as oa
    w, spec = res["w"], res["spec"]
    rp, ci, pairs = res["rp"], res["ci"], res["pairs_g"]
    q64, k64, v64 = (res[x].double().cpu().numpy() for x in ("q", "k", "v"))
    scale = 1.0 / math.sqrt(w["d"])
    done, flops = 0, 0.0
    t0 = time.perf_counter()
    for b in range(w["B"]):
        for h in range(w["H"]):
            oa.csr_attention(q64, k64, v64, rp, ci, w["block"], w["causal"], scale,
                             spec["mask_batch_stride"], spec["mask_head_stride"], heads=[(b, h)])
            done += 1
            flops += 4.0 * w["d"] * pairs[b * spec["mask_batch_stride"] + h * spec["mask_head_stride"]]
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return flops / el / 1e12, "TFLOP/s", f"fp64 CSR-gather oracle forward over {done} of {w['B'] * w['H']} " \
                                         f"(batch, head) slices ({el:.1f} s, {flops / 1e9:.2f} GFLOP)"


def cpu_block_backward(res, budget_s):
    """fp64 oracle gradients of head (0, 0) over every stride-th query block of
    its mask (stride chosen so the sample stays within about the budget)."""
    from oracle import backward as ob
    w, spec = res["w"], res["spec"]
    nb, G = spec["num_blocks"], res["G"]
    rp, ci = res["rp"], res["ci"]
    pairs0 = res["pairs_g"][0]
    # forward FLOPs of head (0, 0) and the measured oracle rate give the stride
    est_rate = 6e9  # fp64 FLOP/s of the gradient oracle, a first guess refined below
    stride = max(1, int(math.ceil(2.5 * 4.0 * w["d"] * pairs0 / (est_rate * budget_s))))
    new_rp, keep = _sample_rows(rp, nb, G, stride)
    new_ci = np.concatenate([ci[rp[r]:rp[r + 1]] for r in range(G * nb) if keep[r]] or [np.zeros(0, np.int64)])
    pairs = unmasked_pairs_per_group(new_rp, new_ci, nb, w["block"], w["causal"])[0]
    sel = (slice(0, 1), slice(0, 1))
    q64, k64, v64, do64 = (t[sel].double().cpu().numpy() for t in (res["q"], res["k"], res["v"], res["dout"]))
    t0 = time.perf_counter()
    ob.csr_attention_bwd(q64, k64, v64, do64, new_rp[: nb + 1], new_ci, w["block"], w["causal"],
                         1.0 / math.sqrt(w["d"]))
    el = time.perf_counter() - t0
    flops = 2.5 * 4.0 * w["d"] * pairs
    return flops / el / 1e12, "TFLOP/s", f"fp64 oracle gradients (dq, dk, dv) of head (0, 0) over every " \
                                         f"{stride}-th query block ({int(keep[:nb].sum())} of {nb} rows; " \
                                         f"{el:.1f} s, {flops / 1e9:.2f} GFLOP)"


def cpu_offsets(tensors, offs, budget_s, backward=False, dout=None, interp=None):
    """fp64 offset oracle on whole (batch, head) slices of one call, as many as fit."""
    from oracle import backward as ob
    from oracle import offsets as oo
    q, k, v = tensors
    B, H, N, d = q.shape
    scale = 1.0 / math.sqrt(d)
    done = 0
    t0 = time.perf_counter()
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(h, h + 1))
            qs, ks, vs = (t[sl].double().cpu().numpy() for t in (q, k, v))
            if backward:
                ob.offset_attention_bwd(qs, ks, vs, dout[sl].double().cpu().numpy(), offs, scale)
            elif interp is not None:
                oo.interp_offset_attention(qs, ks, vs, offs, interp, scale)
            else:
                oo.offset_attention(qs, ks, vs, offs, scale)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    per_head = N * ((8 * d * 2 + 12) if backward else (4 * d * 2 + 4))
    what = "gradients" if backward else "forward"
    return done * per_head / el / 1e9, "GB/s", f"fp64 offset oracle {what} over {done} of {B * H} (batch, head) " \
                                             f"slices of one call ({el:.1f} s)"


def cpu_line(fn, *args, **kw):
    value, unit, sample = fn(*args, **kw)
    return {"value": round(value, 6), "unit": unit, "cores": HOST["blas_threads"] or HOST["affinity_cores"],
            "kind": "oracle", "sample": sample}


# ---------------------------------------------------------- GPU workloads --

def block_workload(name, steps, warmup, trials, spec_over=None, qkv=None, kernel_iters=None):
    """Mask build + forward of a block workload: step time over `steps`, forward
    and mask build alone as medians of `trials`."""
    w = wl.BLOCK_WORKLOADS[name]
    flags_ms = None
    if w.get("literal_source") == "gzip":
        data = wl.synthetic_bytes(w["B"], w["N"], w["block"], w["text_seed"])
        api.sparse_attn_literal_flags(data, w["block"])  # warm
        t0 = time.perf_counter()
        for _ in range(5):
            flags, _ = api.sparse_attn_literal_flags(data, w["block"])
        flags_ms = (time.perf_counter() - t0) / 5 * 1e3
        spec = wl.mask_spec(w, literal_flags=flags)
    else:
        spec = wl.mask_spec(w)
    spec.update(spec_over or {})
    if w.get("head_groups"):
        spec = api.head_group_spec(spec, w["H"])
    dt = wl.torch_dtype(w["dtype"])
    if qkv is None:
        qkv = [t.cuda() for t in wl.make_qkv(w["B"], w["H"], w["N"], w["d"], dt, w["qkv_seed"])]
    q, k, v = qkv
    plan = api.BlockSparsePlan(spec, q, k, v)
    for _ in range(max(1, warmup)):
        plan()
    torch.cuda.synchronize()
    rp = plan.mask.row_ptr.cpu().numpy()
    ci = plan.mask.col_idx[: int(rp[-1])].cpu().numpy()
    pairs_g = unmasked_pairs_per_group(rp, ci, spec["num_blocks"], w["block"], w["causal"])
    pairs = sum(pairs_g[b * spec["mask_batch_stride"] + h * spec["mask_head_stride"]]
                for b in range(w["B"]) for h in range(w["H"]))
    flops = 4.0 * w["d"] * pairs
    step_ms = events_ms(plan, steps)
    ki = kernel_iters or steps
    fwd_ms = median_ms(plan.forward, ki, trials)
    mask_ms = median_ms(plan.build_mask, ki, trials)
    return dict(w=w, spec=spec, flops=flops, pairs=pairs, pairs_g=pairs_g, rp=rp, ci=ci, G=plan.mask.num_groups,
                step_ms=step_ms, fwd_ms=fwd_ms, mask_ms=mask_ms, nnz=int(rp[-1]), plan=plan, q=q, k=k, v=v,
                flags_ms=flags_ms)


def roofline_mfma(flops, ms, kernel, traffic=None):
    ach = flops / (ms * 1e-3) / 1e12
    out = {"bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
           "frac": round(ach / PEAK_BF16_TFLOPS, 4), "kernel": kernel}
    if traffic is not None:
        out["traffic"] = traffic
    return out


def roofline_hbm(byts, ms, kernel):
    gbs = byts / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel": kernel}


def fwd_kernel_name(w, row_split=1):
    return f"bsa_fwd_bf16_kernel<{w['d']},{w['block']},{row_split},1,false>" if w["dtype"] == "bf16" else \
        f"bsa_fwd_f32_kernel<{w['d']},{w['block']}>"


def block_line(name, r, label=None, cpu_budget=None):
    w = r["w"]
    line = {"workload": label or name, "value": round(r["flops"] / (r["step_ms"] * 1e-3) / 1e12, 3),
            "unit": "TFLOP/s", "ms_per_step": round(r["step_ms"], 5), "fwd_ms": round(r["fwd_ms"], 5),
            "mask_build_ms": round(r["mask_ms"], 5), "alg_gflop": round(r["flops"] / 1e9, 3), "nnz_blocks": r["nnz"],
            "roofline": roofline_mfma(r["flops"], r["fwd_ms"], fwd_kernel_name(w))}
    if r["flags_ms"] is not None:
        line["gzip_flags_host_ms"] = round(r["flags_ms"], 4)
        line["literal_fraction"] = round(float(np.mean(r["spec"]["literal_flags"])), 4)
    if cpu_budget:
        line["cpu_baseline"] = cpu_line(cpu_block_forward, r, cpu_budget)
    return line


def block_backward(r, reps, trials, cpu_budget=None):
    """sparse_attn_bwd on a block workload's forward outputs (seeded dO)."""
    plan = r["plan"]
    plan()
    g = torch.Generator().manual_seed(4242)
    r["dout"] = torch.randn(plan.q.shape, generator=g).to(plan.q.dtype).cuda()
    bp = api.BlockSparseBwdPlan(plan, r["dout"])
    bp()
    torch.cuda.synchronize()
    ms = median_ms(bp, reps, trials)
    tr_ms = median_ms(bp.transpose, reps, trials)
    # five products per tile (dV, dP, dQ, dK from dS, and S recomputed): 2.5x
    # the forward's two, as algorithmic FLOPs
    flops = 2.5 * r["flops"]
    line = {"workload": f"{r['w_name']} backward (dq, dk, dv; mask transpose timed apart)",
            "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "bwd_ms": round(ms, 5),
            "mask_transpose_ms": round(tr_ms, 5), "alg_gflop": round(flops / 1e9, 3),
            "roofline": roofline_mfma(flops, ms, "bsa_bwd_dq_bf16 + bsa_bwd_dkdv_bf16 (+ plan / convert)")}
    if cpu_budget:
        line["cpu_baseline"] = cpu_line(cpu_block_backward, r, cpu_budget)
    del bp
    return line


def graph_line(r, reps, trials, label):
    """The step (mask build + forward) captured once into a HIP graph and replayed."""
    plan = r["plan"]
    g = api.capture_graph(plan)
    g.replay()
    torch.cuda.synchronize()
    ms = median_ms(g.replay, reps, trials)
    return {"workload": label, "value": round(r["flops"] / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "ms_per_step": round(ms, 5), "alg_gflop": round(r["flops"] / 1e9, 3),
            "roofline": roofline_mfma(r["flops"], ms, "mask build + " + fwd_kernel_name(r["w"]) + " (graph)")}


def offset_workload(N, reps, trials, cpu_budget=None):
    ow = wl.OFFSET_WORKLOAD
    B, H, d = ow["B"], ow["H"], ow["d"]
    plans, tables = [], []
    for l, alpha in enumerate(ow["alphas"]):
        offs = api.offset_attn_make_table(ow["W"], alpha, api.fibonacci_base(N), N)
        q, k, v = [t.cuda() for t in wl.make_qkv(B, H, N, d, torch.bfloat16, ow["qkv_seed_base"][N] + l)]
        plans.append(api.OffsetPlan(q, k, v, offs))
        tables.append(offs)

    def all_calls():
        for p in plans:
            p()
    all_calls()
    ms = median_ms(all_calls, reps, trials) / len(plans)
    byt = B * H * N * (4 * d * 2 + 4)
    line = {"workload": f"fibonacci-offsets N={N} (16 staggered calls, distinct buffers)",
            "value": round(byt / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "call_ms": round(ms, 5),
            "alg_bytes_per_call": byt, "distances_per_call": [len(t) for t in tables],
            "roofline": roofline_hbm(byt, ms, "offset_mfma_kernel")}
    if cpu_budget:
        p = plans[7]
        line["cpu_baseline"] = cpu_line(cpu_offsets, (p.q, p.k, p.v), tables[7], cpu_budget)
    return line


def offset_backward(N, reps, trials, cpu_budget=None):
    ow = wl.OFFSET_WORKLOAD
    B, H, d = ow["B"], ow["H"], ow["d"]
    offs = api.offset_attn_make_table(ow["W"], ow["alphas"][7], api.fibonacci_base(N), N)
    q, k, v = [t.cuda() for t in wl.make_qkv(B, H, N, d, torch.bfloat16, ow["qkv_seed_base"][N] + 7)]
    fp = api.OffsetPlan(q, k, v, offs)
    fp()
    g = torch.Generator().manual_seed(4343)
    dout = torch.randn(q.shape, generator=g).to(q.dtype).cuda()
    bp = api.OffsetBwdPlan(fp, offs, dout)
    bp()
    torch.cuda.synchronize()
    ms = median_ms(bp, reps, trials)
    # q, k, v, o, dO read once, dq, dk, dv written once, lse read, D written and read
    byt = B * H * N * (8 * d * 2 + 12)
    line = {"workload": f"fibonacci-offsets backward N={N} (alpha = 1 + 7/15)",
            "value": round(byt / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "call_ms": round(ms, 5),
            "alg_bytes_per_call": byt, "roofline": roofline_hbm(byt, ms, "offset backward kernels")}
    if cpu_budget:
        line["cpu_baseline"] = cpu_line(cpu_offsets, (q, k, v), offs, cpu_budget, backward=True, dout=dout)
    return line


def offset_variant(name, reps, trials, N=2048, cpu_budget=None):
    """16 calls of an offset variant (distinct buffers per call)."""
    ow, v = wl.OFFSET_WORKLOAD, wl.OFFSET_VARIANTS[name]
    B, H, d = ow["B"], ow["H"], ow["d"]
    base = api.fibonacci_base(N) if v["base"] == "fibonacci" else api.power2_base(N)
    plans, nkeys, specs = [], [], []
    for l in range(16):
        q, k, v_ = [t.cuda() for t in wl.make_qkv(B, H, N, d, torch.bfloat16, v["qkv_seed_base"] + l)]
        if "ratios" in v:
            num, den = v["ratios"][l]
            offs = api.offset_attn_make_table_ratio(ow["W"], num, den, base, N)
            plans.append(api.OffsetPlan(q, k, v_, offs))
            nkeys.append(len(offs))
            specs.append((offs, None))
        else:
            offs, rungs = api.offset_attn_make_interp(ow["W"], wl.interp_alphas(v)[l], base, N)
            plans.append(api.OffsetPlan(q, k, v_, offs, rungs=rungs))
            nkeys.append(len(offs) + len(rungs))
            specs.append((offs, rungs))

    def all_calls():
        for p in plans:
            p()
    all_calls()
    ms = median_ms(all_calls, reps, trials) / len(plans)
    byt = B * H * N * (4 * d * 2 + 4)
    kern = "offset_mfma_kernel" if "ratios" in v else "offset_mfma_kernel (interpolated rungs)"
    line = {"workload": f"offsets {name} N={N} (16 calls, distinct buffers)",
            "value": round(byt / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "call_ms": round(ms, 5),
            "keys_per_query_mean": float(np.mean(nkeys)), "alg_bytes_per_call": byt,
            "roofline": roofline_hbm(byt, ms, kern)}
    if cpu_budget:
        p = plans[7]
        offs, rungs = specs[7]
        line["cpu_baseline"] = cpu_line(cpu_offsets, (p.q, p.k, p.v), offs, cpu_budget, interp=rungs)
    return line


# -------------------------------------------------------------------- main --

HOST = {}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernel",
                    choices=sorted(wl.BLOCK_WORKLOADS) + ["offsets-2048", "offsets-8192"]
                    + [n + "-bwd" for n in sorted(wl.BLOCK_WORKLOADS) if wl.BLOCK_WORKLOADS[n]["dtype"] == wl.BF16],
                    help="run only the given workload's kernels (for counter collection), then exit")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB",
                    help="run a plain device copy of MIB MiB (traffic-counter calibration), then exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    HOST.update(host_info())
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": n, "dispatches": args.steps}))
        return
    if args.profile_kernel:
        pk = args.profile_kernel
        if pk.startswith("offsets"):
            line = offset_workload(int(pk.split("-")[1]), reps=args.steps, trials=1)
        elif pk.endswith("-bwd"):
            name = pk[: -len("-bwd")]
            r = block_workload(name, steps=1, warmup=0, trials=1, kernel_iters=1)
            r["w_name"] = name
            line = block_backward(r, reps=args.steps, trials=1)
        else:
            r = block_workload(pk, steps=1, warmup=0, trials=1, kernel_iters=args.steps)
            line = block_line(pk, r)
        print(json.dumps(line), flush=True)
        return

    cpu = None if args.no_cpu_baseline else True
    probe = ClockProbe()
    w = wl.BLOCK_WORKLOADS[HEADLINE]
    qkv = [t.cuda() for t in wl.make_qkv(w["B"], w["H"], w["N"], w["d"], torch.bfloat16, w["qkv_seed"])]
    head = block_workload(HEADLINE, args.steps, args.warmup, args.trials, qkv=qkv, kernel_iters=max(20, args.steps))
    head["w_name"] = HEADLINE
    # clock during back-to-back forwards of the headline
    probe.start(0.25)
    events_ms(head["plan"].forward, int(250 / max(head["fwd_ms"], 1e-3)) + 1)
    clock = probe.mhz()
    value = head["flops"] / (head["step_ms"] * 1e-3) / 1e12
    traffic = read_profile_record("bsa_fwd_bf16_d128_b128_long-context", "traffic")
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1) Q/K/V; seeded Bernoulli literal flags)",
        "config": {"workload": "long-context block-sparse attention: bf16, B=1 H=16 N=65536 d=128, block 128, "
                               "causal, window own+2 previous blocks, global blocks 0-3, literal-pair blocks "
                               "Bernoulli(0.15) shared by all heads; step = device mask build + forward",
                   "global_batch": w["B"], "seq_len": w["N"], "heads": w["H"], "head_dim": w["d"],
                   "block": w["block"], "nnz_blocks": head["nnz"], "alg_gflop_per_step": round(head["flops"] / 1e9, 4),
                   "mask_build_ms": round(head["mask_ms"], 5), "fwd_ms": round(head["fwd_ms"], 5),
                   "kernel_trials": args.trials, "kernel_stat": "median"},
        "roofline": roofline_mfma(head["flops"], head["fwd_ms"], fwd_kernel_name(w),
                                  traffic=(traffic or {}).get("bytes_per_launch")),
        "system": {"shader_clock_mhz_measured": clock, "device": torch.cuda.get_device_name(0), "host": HOST,
                   "dense_bf16_gemm_reference": gemm_reference()},
    }
    if cpu:
        out["cpu_baseline"] = cpu_line(cpu_block_forward, head, 12.0)
    if not args.no_secondary:
        sec = []
        budget = 3.0 if cpu else None
        # the other reading of the literal rule on the same inputs
        r = block_workload(HEADLINE, 20, 3, args.trials, spec_over={"literal_mode": "anyq"}, qkv=qkv)
        sec.append(block_line(HEADLINE, r, "long-context, literal rule ANYQ (every earlier literal block)",
                              cpu_budget=budget))
        del r
        sec.append(block_backward(head, reps=5, trials=args.trials, cpu_budget=budget))
        del head["plan"], head["dout"]
        del qkv
        torch.cuda.empty_cache()
        for name, label, over in (("compression-guided", None, None),
                                  ("compression-guided", "compression-guided, literal rule ANYQ", {"literal_mode": "anyq"}),
                                  ("bigbird", None, None), ("tiny-fp32", None, None),
                                  ("gzip-guided", None, None), ("gzip-head-groups", None, None)):
            r = block_workload(name, 200, 10, args.trials, spec_over=over)
            r["w_name"] = name
            sec.append(block_line(name, r, label, cpu_budget=budget))
            if name == "bigbird":
                sec.append(graph_line(r, 200, args.trials, "bigbird step (mask build + forward) as one captured graph"))
            if name == "compression-guided" and over is None:
                sec.append(block_backward(r, reps=50, trials=args.trials, cpu_budget=budget))
            del r
            torch.cuda.empty_cache()
        for N in wl.OFFSET_WORKLOAD["lengths"]:
            sec.append(offset_workload(N, reps=5, trials=args.trials, cpu_budget=budget))
            torch.cuda.empty_cache()
        for N in wl.OFFSET_WORKLOAD["lengths"]:
            sec.append(offset_backward(N, reps=10, trials=args.trials, cpu_budget=budget))
            torch.cuda.empty_cache()
        for name in wl.OFFSET_VARIANTS:
            sec.append(offset_variant(name, reps=5, trials=args.trials, cpu_budget=budget))
            torch.cuda.empty_cache()
        out["secondary"] = sec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
