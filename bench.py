"""Benchmark of the sparse-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-secondary] [--no-cpu-baseline]

One step = the whole hot path on one batch of the headline workload
(compression-guided block mask, bf16, B=4 H=8 N=8192 d=64 block 64, causal,
literal rate 0.25): build the CSR mask on the device, then the block-sparse
attention forward.  Inputs are resident in HBM before timing starts.  The value
is algorithmic TFLOP/s: 4 * d * (unmasked query/key pairs) per step / step time
(the diagonal block counts b(b+1)/2 pairs; blocks after the query block none).

Prints ONE JSON line.  Secondary workloads (BigBird, gzip-guided with and
without head groups, long-context, Fibonacci offsets) are measured in the same
run and reported under "secondary".
The gzip-guided line takes its literal flags from per-block gzip sizes of
synthetic byte streams, computed on the host by the library; their host time is
reported beside the device step (mask build + forward), which it is not part of.
"""

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from long_context_sparse_block_amd import api  # noqa: E402
from long_context_sparse_block_amd import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "effective TFLOP/s on unmasked blocks (% of bf16 MFMA peak); offset-attn GB/s"
HEADLINE = "compression-guided"
PROFILE_DIR = os.path.join(ROOT, "profiles")


def unmasked_pairs_per_group(row_ptr, col_idx, nb, block, causal):
    """Unmasked (query, key) token pairs of every mask group, from the CSR."""
    rp = row_ptr.cpu().numpy().astype(np.int64)
    ci = col_idx[: int(rp[-1])].cpu().numpy().astype(np.int64)
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


def alg_flops(w, spec, mask):
    pairs = unmasked_pairs_per_group(mask.row_ptr, mask.col_idx, spec["num_blocks"], w["block"], w["causal"])
    tot = 0
    for b in range(w["B"]):
        for h in range(w["H"]):
            tot += pairs[b * spec["mask_batch_stride"] + h * spec["mask_head_stride"]]
    return 4.0 * w["d"] * tot, tot


def time_events(fn, iters):
    """Average ms of fn() over iters back-to-back calls, HIP events on the current stream."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def read_traffic(kernel_tag):
    """HBM traffic per launch from a stored rocprofv3 counter summary, if it still
    matches the current kernel source; else None."""
    path = os.path.join(PROFILE_DIR, f"{kernel_tag}_traffic.txt")
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
    return rec.get("bytes_per_launch")


def gzip_flags(w):
    """Literal flags of a gzip-sourced workload: per-block gzip sizes of its
    synthetic byte streams (host, in the library), and the host time they take."""
    data = wl.synthetic_bytes(w["B"], w["N"], w["block"], w["text_seed"])
    api.sparse_attn_literal_flags(data, w["block"])  # warm
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        flags, _ = api.sparse_attn_literal_flags(data, w["block"])
    return flags, (time.perf_counter() - t0) / reps * 1e3


def block_workload(name, steps, warmup, kernel_iters):
    w = wl.BLOCK_WORKLOADS[name]
    flags_ms = None
    if w.get("literal_source") == "gzip":
        flags, flags_ms = gzip_flags(w)
        spec = wl.mask_spec(w, literal_flags=flags)
    else:
        spec = wl.mask_spec(w)
    if w.get("head_groups"):
        spec = api.head_group_spec(spec, w["H"])
    dt = wl.torch_dtype(w["dtype"])
    q, k, v = [t.cuda() for t in wl.make_qkv(w["B"], w["H"], w["N"], w["d"], dt, w["qkv_seed"])]
    plan = api.BlockSparsePlan(spec, q, k, v)
    for _ in range(warmup):
        plan()
    torch.cuda.synchronize()
    flops, pairs = alg_flops(w, spec, plan.mask)
    # whole step (mask build + forward)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step_ms = time_events(plan, steps)
    wall = time.perf_counter() - t0
    # forward kernel alone, and the mask build alone
    fwd_ms = time_events(plan.forward, kernel_iters)
    mask_ms = time_events(plan.build_mask, kernel_iters)
    nnz = int(plan.mask.row_ptr[-1].item())
    return dict(w=w, spec=spec, flops=flops, pairs=pairs, step_ms=step_ms, fwd_ms=fwd_ms,
                mask_ms=mask_ms, wall_s=wall, nnz=nnz, plan=plan, q=q, k=k, v=v, flags_ms=flags_ms)


def block_backward(res, reps):
    """sparse_attn_bwd on a block workload's forward outputs (seeded dO)."""
    plan = res["plan"]
    plan()
    g = torch.Generator().manual_seed(4242)
    dout = torch.randn(plan.q.shape, generator=g).to(plan.q.dtype).cuda()
    bp = api.BlockSparseBwdPlan(plan, dout)
    bp()
    torch.cuda.synchronize()
    bwd_ms = time_events(bp, reps)
    tr_ms = time_events(bp.transpose, reps)
    # five products per tile (dV, dP, dS-based dQ and dK, and S recomputed):
    # 2.5x the forward's two, as algorithmic FLOPs
    flops = 2.5 * res["flops"]
    return dict(bwd_ms=bwd_ms, transpose_ms=tr_ms, flops=flops, tflops=flops / (bwd_ms * 1e-3) / 1e12)


def backward_line(name, r):
    return {"workload": f"{name} backward (dq, dk, dv; mask transpose timed apart)",
            "value": round(r["tflops"], 3), "unit": "TFLOP/s", "bwd_ms": round(r["bwd_ms"], 5),
            "mask_transpose_ms": round(r["transpose_ms"], 5), "alg_gflop": round(r["flops"] / 1e9, 3),
            "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 3), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(r["tflops"] / PEAK_BF16_TFLOPS, 4)}}


def offset_backward(N, reps):
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
    ms = time_events(bp, reps)
    # q, k, v, o, dO read once, dq, dk, dv written once, lse read, D written and read
    byt = B * H * N * (8 * d * 2 + 12)
    return dict(ms=ms, bytes=byt, gbs=byt / (ms * 1e-3) / 1e9)


def offset_workload(N, reps, warmup):
    ow = wl.OFFSET_WORKLOAD
    B, H, d = ow["B"], ow["H"], ow["d"]
    plans = []
    for l, alpha in enumerate(ow["alphas"]):
        offs = api.offset_attn_make_table(ow["W"], alpha, api.fibonacci_base(N), N)
        q, k, v = [t.cuda() for t in wl.make_qkv(B, H, N, d, torch.bfloat16, ow["qkv_seed_base"][N] + l)]
        plans.append(api.OffsetPlan(q, k, v, offs))

    def all_calls():
        for p in plans:
            p()
    for _ in range(warmup):
        all_calls()
    ms16 = time_events(all_calls, reps)
    call_ms = ms16 / len(plans)
    bytes_per_call = B * H * N * (4 * d * 2 + 4)
    return dict(N=N, call_ms=call_ms, bytes=bytes_per_call, gbs=bytes_per_call / (call_ms * 1e-3) / 1e9)


def offset_variant_workload(name, reps, warmup, N=2048):
    """16 calls of an offset variant (distinct buffers per call)."""
    ow, v = wl.OFFSET_WORKLOAD, wl.OFFSET_VARIANTS[name]
    B, H, d = ow["B"], ow["H"], ow["d"]
    base = api.fibonacci_base(N) if v["base"] == "fibonacci" else api.power2_base(N)
    plans, nkeys = [], []
    for l in range(16):
        q, k, v_ = [t.cuda() for t in wl.make_qkv(B, H, N, d, torch.bfloat16, v["qkv_seed_base"] + l)]
        if "ratios" in v:
            num, den = v["ratios"][l]
            offs = api.offset_attn_make_table_ratio(ow["W"], num, den, base, N)
            plans.append(api.OffsetPlan(q, k, v_, offs))
            nkeys.append(len(offs))
        else:
            offs, rungs = api.offset_attn_make_interp(ow["W"], wl.interp_alphas(v)[l], base, N)
            plans.append(api.OffsetPlan(q, k, v_, offs, rungs=rungs))
            nkeys.append(len(offs) + len(rungs))

    def all_calls():
        for p in plans:
            p()
    for _ in range(warmup):
        all_calls()
    ms16 = time_events(all_calls, reps)
    call_ms = ms16 / len(plans)
    bytes_per_call = B * H * N * (4 * d * 2 + 4)
    return dict(N=N, call_ms=call_ms, bytes=bytes_per_call, gbs=bytes_per_call / (call_ms * 1e-3) / 1e9,
                keys=float(np.mean(nkeys)))


def cpu_baseline(res, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the headline workload:
    whole (batch, head) slices, as many as fit in the time budget."""
    from oracle import attention as oa
    try:
        from threadpoolctl import threadpool_info
        threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    w, spec, mask = res["w"], res["spec"], res["plan"].mask
    rp = mask.row_ptr.cpu().numpy()
    ci = mask.col_idx[: int(rp[-1])].cpu().numpy()
    pairs = unmasked_pairs_per_group(mask.row_ptr, mask.col_idx, spec["num_blocks"], w["block"], w["causal"])
    q64 = res["q"].double().cpu().numpy()
    k64 = res["k"].double().cpu().numpy()
    v64 = res["v"].double().cpu().numpy()
    scale = 1.0 / math.sqrt(w["d"])
    done, flops = [], 0.0
    t0 = time.perf_counter()
    for b in range(w["B"]):
        for h in range(w["H"]):
            oa.csr_attention(q64, k64, v64, rp, ci, w["block"], w["causal"], scale,
                             spec["mask_batch_stride"], spec["mask_head_stride"], heads=[(b, h)])
            done.append((b, h))
            flops += 4.0 * w["d"] * pairs[b * spec["mask_batch_stride"] + h * spec["mask_head_stride"]]
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 CSR-gather oracle over {len(done)} of {w['B'] * w['H']} (batch, head) slices "
                      f"of the {HEADLINE} workload ({el:.1f} s, {flops / 1e9:.2f} GFLOP); "
                      f"host {platform.processor() or platform.machine()}, os.cpu_count={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-kernel", choices=sorted(wl.BLOCK_WORKLOADS) + ["offsets-2048", "offsets-8192"],
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
        if args.profile_kernel.startswith("offsets"):
            r = offset_workload(int(args.profile_kernel.split("-")[1]), reps=args.steps, warmup=0)
            print(json.dumps({"workload": args.profile_kernel, "call_ms": r["call_ms"], "gbs": r["gbs"]}))
        else:
            r = block_workload(args.profile_kernel, steps=1, warmup=0, kernel_iters=args.steps)
            print(json.dumps({"workload": args.profile_kernel, "fwd_ms": r["fwd_ms"],
                              "tflops": r["flops"] / (r["fwd_ms"] * 1e-3) / 1e12}))
        return

    head = block_workload(HEADLINE, args.steps, args.warmup, kernel_iters=max(50, args.steps))
    w = head["w"]
    value = head["flops"] / (head["step_ms"] * 1e-3) / 1e12
    achieved = head["flops"] / (head["fwd_ms"] * 1e-3) / 1e12
    traffic = read_traffic("bsa_fwd_bf16_d64_b64_compression-guided")
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
        "config": {"workload": "compression-guided block-sparse attention: bf16, B=4 H=8 N=8192 d=64, "
                               "block 64, causal, window own+3 previous blocks, literal-pair blocks "
                               "Bernoulli(0.25) per sequence; step = device mask build + forward",
                   "global_batch": w["B"], "seq_len": w["N"], "heads": w["H"], "head_dim": w["d"],
                   "block": w["block"], "nnz_blocks": head["nnz"], "alg_gflop_per_step": round(head["flops"] / 1e9, 4),
                   "mask_build_ms": round(head["mask_ms"], 5), "fwd_ms": round(head["fwd_ms"], 5)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "bsa_fwd_bf16_kernel<64,64>"},
    }
    if not args.no_secondary:
        sec = []
        for name, iters in (("bigbird", 200), ("gzip-guided", 200), ("gzip-head-groups", 200),
                            ("long-context", 20)):
            r = block_workload(name, steps=iters, warmup=3, kernel_iters=iters)
            ach = r["flops"] / (r["fwd_ms"] * 1e-3) / 1e12
            line = {"workload": name, "value": round(r["flops"] / (r["step_ms"] * 1e-3) / 1e12, 3),
                    "unit": "TFLOP/s", "ms_per_step": round(r["step_ms"], 5), "fwd_ms": round(r["fwd_ms"], 5),
                    "mask_build_ms": round(r["mask_ms"], 5), "alg_gflop": round(r["flops"] / 1e9, 3),
                    "roofline": {"bound": "mfma", "achieved": round(ach, 3), "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}}
            if r["flags_ms"] is not None:
                line["gzip_flags_host_ms"] = round(r["flags_ms"], 4)
                line["literal_fraction"] = round(float(np.mean(r["spec"]["literal_flags"])), 4)
            sec.append(line)
            if name == "long-context":
                sec.append(backward_line(name, block_backward(r, reps=5)))
            del r
            torch.cuda.empty_cache()
        sec.append(backward_line(HEADLINE, block_backward(head, reps=50)))
        torch.cuda.empty_cache()
        for N in wl.OFFSET_WORKLOAD["lengths"]:
            r = offset_workload(N, reps=5, warmup=1)
            sec.append({"workload": f"fibonacci-offsets N={N} (16 staggered calls, distinct buffers)",
                        "value": round(r["gbs"], 2), "unit": "GB/s", "call_ms": round(r["call_ms"], 5),
                        "alg_bytes_per_call": r["bytes"],
                        "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 2), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(r["gbs"] / PEAK_HBM_GBS, 4)}})
            torch.cuda.empty_cache()
        for N in wl.OFFSET_WORKLOAD["lengths"]:
            r = offset_backward(N, reps=10)
            sec.append({"workload": f"fibonacci-offsets backward N={N} (alpha = 1 + 7/15)", "value": round(r["gbs"], 2),
                        "unit": "GB/s", "call_ms": round(r["ms"], 5), "alg_bytes_per_call": r["bytes"],
                        "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 2), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(r["gbs"] / PEAK_HBM_GBS, 4)}})
            torch.cuda.empty_cache()
        for name in wl.OFFSET_VARIANTS:
            r = offset_variant_workload(name, reps=5, warmup=1)
            sec.append({"workload": f"offsets {name} N=2048 (16 calls, distinct buffers)",
                        "value": round(r["gbs"], 2), "unit": "GB/s", "call_ms": round(r["call_ms"], 5),
                        "keys_per_query_mean": r["keys"], "alg_bytes_per_call": r["bytes"],
                        "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 2), "peak": PEAK_HBM_GBS,
                                     "unit": "GB/s", "frac": round(r["gbs"] / PEAK_HBM_GBS, 4)}})
            torch.cuda.empty_cache()
        out["secondary"] = sec
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(head)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
