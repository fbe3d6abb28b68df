"""Benchmark of the shifted-window attention forward pass on one MI355X.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one swa_forward call over the whole workload (gather, window
attention with bias and mask, softmax, PV and scatter), inputs already in HBM.
With --pass backward a step is one swa_backward call (dq, dk, dv and the
bias-table gradient of the same workload); with --from-forward it is one
swa_backward_lse call, which takes the softmax statistics and the output that
swa_forward_lse produced (once per input set, before the timed steps).
With --pass layer a step is one swa_layer_forward call: the
query/key/value projection of the token embeddings, the window attention
and the output projection.
Default workload: bf16, B=1, 540x1080 grid (1/12 degree field at patch 4),
8 heads x 64, window 12x12, shift 6.  Prints one JSON line.

The CPU-baseline leg times the fp64 oracle on the host cores over a bounded
sample of the same workload (whole latitude rows) and reports the GPU's
relative max-abs error on that sample.
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shifted-window attention fwd TFLOP/s + tokens/s, % of bf16 MFMA peak"
METRIC_BWD = "shifted-window attention bwd TFLOP/s + tokens/s, % of bf16 MFMA peak"
BWD_SOURCES = ["shifted_window_attention_cyclic_amd/csrc/swa_backward.hip",
               "shifted_window_attention_cyclic_amd/csrc/swa_backward.h",
               "shifted_window_attention_cyclic_amd/csrc/swa_device.h",
               "shifted_window_attention_cyclic_amd/csrc/swa_geometry.h"]
METRIC_LAYER = ("shifted-window attention layer fwd (QKV projection + attention + output projection) "
                "TFLOP/s, % of bf16 MFMA peak")
PROJ_SOURCES = ["shifted_window_attention_cyclic_amd/csrc/swa_projection.hip",
                "shifted_window_attention_cyclic_amd/csrc/swa_projection.h",
                "shifted_window_attention_cyclic_amd/csrc/swa_device.h",
                "shifted_window_attention_cyclic_amd/csrc/swa_geometry.h"]
LAYER_SOURCES = ["shifted_window_attention_cyclic_amd/csrc/swa_layer.hip",
                 "shifted_window_attention_cyclic_amd/csrc/swa_layer.h",
                 "shifted_window_attention_cyclic_amd/csrc/swa_stream.h",
                 "shifted_window_attention_cyclic_amd/csrc/swa_device.h",
                 "shifted_window_attention_cyclic_amd/csrc/swa_geometry.h"]
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
MALL_BYTES = 256 << 20     # Infinity Cache; rotate inputs until the working set is 3x this
KERNEL_SOURCES = ["shifted_window_attention_cyclic_amd/csrc/swa_kernels.hip",
                  "shifted_window_attention_cyclic_amd/csrc/swa_stream.h",
                  "shifted_window_attention_cyclic_amd/csrc/swa_device.h",
                  "shifted_window_attention_cyclic_amd/csrc/swa_geometry.h"]
SCHEDULE_STREAM, SCHEDULE_BLOCK, SCHEDULE_KEYBLOCK = 1, 2, 3  # swa_info.schedule
CPU_SAMPLE_FLOPS = 4e11  # nominal FLOPs of the CPU-baseline sample (about 10 s of fp64 on 16 cores)


def kernel_name(p, info) -> str:
    if p.dtype == "f32":
        return "attn_f32_kernel"
    return {SCHEDULE_STREAM: "attn_bf16_stream_kernel", SCHEDULE_KEYBLOCK: "attn_bf16_kblock_kernel"}.get(
        info.schedule, "attn_bf16_kernel")


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(workload: str, backward: bool = False, tag: str = None, sources=None):
    """HBM bytes per launch measured by rocprofv3 counters, if the summary in
    profiles/ was taken on the current kernel sources; else None."""
    tag = tag if tag is not None else ("bwd_" if backward else "")
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}{workload}.md")
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic_json:\s*(\{.*\})\s*$", open(path).read(), flags=re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("kernel_source_sha256_16") != kernel_source_hash(sources or (BWD_SOURCES if backward else None)):
        return None
    return rec.get("bytes_per_launch")


def useful_pairs(p) -> int:
    """Visible (query, key) pairs summed over real queries: per axis, the key
    segment sizes multiply, so the sum factorises over the three axes."""
    total = p.batch
    for a in range(3):
        E, P, w, s, cyc = p.extent[a], p.padded[a], p.window[a], p.shift[a], p.cyclic[a]

        def label(c):
            if cyc:
                return ((c - s) % E) // w
            return -1 if c < s else (c - s) // w

        counts = {}
        for c in range(E):
            counts[label(c)] = counts.get(label(c), 0) + 1
        total *= sum(n * n for n in counts.values())
    return total


def cpu_baseline(p, x, out_gpu, rows):
    import numpy as np

    import oracle

    T, H, W = p.extent
    # whole latitude rows, as many as keep the sample near CPU_SAMPLE_FLOPS
    per_row = 4.0 * p.window_tokens * p.head_dim * p.heads * p.batch * T * W
    rows = max(1, min(rows, H, int(CPU_SAMPLE_FLOPS // per_row)))
    idx = np.array([((b * T + t) * H + y) * W + xx for b in range(p.batch) for t in range(T)
                    for y in range(rows) for xx in range(W)], dtype=np.int64)
    host = {n: x[n].float().numpy() for n in ("q", "k", "v", "table")}
    t0 = time.perf_counter()
    ref, used = oracle.direct_forward(p, host["q"], host["k"], host["v"], host["table"],
                                      query_index=idx)
    dt = time.perf_counter() - t0
    flops = 4.0 * p.window_tokens * p.head_dim * p.heads * len(idx)  # nominal, per query
    got = out_gpu.float().cpu().numpy().reshape(p.tokens, p.heads, p.head_dim)[idx]
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(used), "kind": "oracle",
        "sample": (f"fp64 direct-form oracle over latitude rows 0..{rows - 1} of every time step "
                   f"and batch item ({len(idx)} of {p.tokens} query tokens, all {p.heads} heads)"),
        "seconds": dt, "tokens_per_s": len(idx) / dt,
        "gpu_rel_max_abs_err_on_sample": err,
    }


def cpu_baseline_backward(p, x, dout, grads_gpu, windows):
    import numpy as np

    import oracle

    host = {n: x[n].float().numpy() for n in ("q", "k", "v", "table")}
    t0 = time.perf_counter()
    ref = oracle.literal_backward(p, host["q"], host["k"], host["v"], host["table"], dout.float().numpy(),
                                  windows=windows)
    dt = time.perf_counter() - t0
    mine = np.isin(oracle.token_windows(p), [w % (p.windows // p.batch) for w in windows])
    err = 0.0
    for g, r in zip(grads_gpu[:3], ref[:3]):
        got = g.float().cpu().numpy()[0][mine]
        err = max(err, float(np.abs(got - r[0][mine]).max() / np.abs(r[0][mine]).max()))
    flops = 10.0 * p.window_tokens ** 2 * p.head_dim * p.heads * len(windows)
    return {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
        "sample": (f"fp64 per-window oracle backward (numpy) over {len(windows)} of {p.windows} windows "
                   f"of batch item 0, all {p.heads} heads"),
        "seconds": dt, "gpu_rel_max_abs_err_on_sample": err,
    }


def warm_up(step, steps, min_ms):
    """Untimed warm-up: `steps` calls, then batches of 10 more until `min_ms`
    of wall time (GPU work included) have passed.  Returns (calls, ms)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    for _ in range(steps):
        step(n)
        n += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(10):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def launch_stats(launch_ms):
    """Mean, median, p10 and p90 of sorted per-launch times (ms)."""
    n = len(launch_ms)
    med = launch_ms[n // 2] if n % 2 else 0.5 * (launch_ms[n // 2 - 1] + launch_ms[n // 2])
    return {"avg_launch_ms": round(sum(launch_ms) / n, 5), "median_ms": round(med, 5),
            "p10_ms": round(launch_ms[n // 10], 5), "p90_ms": round(launch_ms[(9 * n) // 10], 5)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=200.0,
                    help="after the --warmup steps, keep warming up (untimed) until this much wall time has "
                         "passed, so that clocks have settled before the timed steps")
    ap.add_argument("--workload", default="c3_bf16_540x1080")
    ap.add_argument("--variant", default="fused", choices=["fused", "staged"])
    ap.add_argument("--schedule", default="auto", choices=["auto", "stream", "block", "keyblock"],
                    help="the bf16 attention schedule (forward and backward passes)")
    ap.add_argument("--cpu-rows", type=int, default=1 << 30,
                    help="latitude rows in the CPU-baseline sample (default: all that keep it "
                         "near 4e11 nominal FLOPs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--from-forward", action="store_true",
                    help="--pass backward: time swa_backward_lse from swa_forward_lse's output and statistics")
    ap.add_argument("--pass", dest="which", default="forward", choices=["forward", "backward", "layer"],
                    help="time swa_forward (default), swa_backward or swa_layer_forward")
    ap.add_argument("--layer", default="auto", choices=["auto", "fused", "unfused"],
                    help="the path of swa_layer_forward (--pass layer)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the forward pass is measured "
                                   "on one MI355X; multi-GPU sharding is not implemented",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    from shifted_window_attention_cyclic_amd import (WindowAttention, swa_backward, swa_backward_lse, swa_forward,
                                                     swa_forward_lse)
    from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.which == "layer":
        return run_layer(args)
    p = WORKLOADS[args.workload]
    x = make_inputs(p)
    att = WindowAttention(p, args.variant, args.schedule)
    info = att.info
    set_bytes = info.algorithmic_bytes
    nsets = max(1, min(8, math.ceil(3 * MALL_BYTES / set_bytes)))
    sets = []
    for i in range(nsets):
        xi = x if i == 0 else make_inputs(p, seed=p.seed + 7919 * i)
        d = {n: t.cuda() for n, t in xi.items()}
        d["out"] = torch.empty_like(d["q"])
        sets.append(d)

    backward = args.which == "backward"
    if backward:
        if info.backward_workspace_bytes == 0:
            sys.exit("the backward kernels do not take this workload's window")
        g = torch.Generator().manual_seed(p.seed + 17)
        dout_host = torch.randn(tuple(x["q"].shape), generator=g).to(x["q"].dtype)
        ws = torch.empty((info.backward_workspace_bytes + 15) // 16 * 4, dtype=torch.float32, device="cuda")
        for s in sets:
            s["dout"] = dout_host.cuda()
            s["dq"], s["dk"], s["dv"] = (torch.empty_like(s["q"]) for _ in range(3))
            s["dtable"] = torch.empty_like(s["table"])
            if args.from_forward:
                s["lse"] = torch.empty(att.io_shape[:-1], dtype=torch.float32, device="cuda")
                swa_forward_lse(att.handle, s["q"], s["k"], s["v"], s["table"], s["out"], s["lse"])
        torch.cuda.synchronize()

    def step(i):
        s = sets[i % nsets]
        if backward and args.from_forward:
            swa_backward_lse(att.handle, s["q"], s["k"], s["v"], s["table"], s["out"], s["lse"], s["dout"], s["dq"],
                             s["dk"], s["dv"], s["dtable"], ws)
        elif backward:
            swa_backward(att.handle, s["q"], s["k"], s["v"], s["table"], s["dout"], s["dq"], s["dk"], s["dv"],
                         s["dtable"], ws)
        else:
            swa_forward(att.handle, s["q"], s["k"], s["v"], s["table"], s["out"])

    warm_steps, warm_ms = warm_up(step, args.warmup, args.warmup_ms)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record()
        step(i)
        ends[i].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    launch_ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # forward: 4 N^2 d per unit (Q K^T, P V); backward: 10 N^2 d (Q K^T again, dO V^T,
    # dS K, dS^T Q, P^T dO).  Bytes: forward q, k, v read and out written; backward
    # q, k, v, dout read and dq, dk, dv written; the table once each way.
    flop_mul = 2.5 if backward else 1.0
    nominal_flops = info.nominal_flops * flop_mul
    table_bytes = 4.0 * math.prod(p.table_shape)
    tensor_bytes = (info.algorithmic_bytes - table_bytes) / 4
    # from the forward's statistics the backward also reads out and lse (one float per token and head)
    lse_bytes = 4.0 * info.tokens * p.heads
    alg_bytes = ((8 * tensor_bytes + lse_bytes if args.from_forward else 7 * tensor_bytes) + 2 * table_bytes
                 if backward else info.algorithmic_bytes)
    tflops = nominal_flops / (ms_per_step * 1e-3) / 1e12
    useful = 4.0 * useful_pairs(p) * p.head_dim * p.heads * flop_mul
    achieved_gbs = alg_bytes / (avg_launch_ms * 1e-3) / 1e9
    kernel_tflops = nominal_flops / (avg_launch_ms * 1e-3) / 1e12
    peak_tf = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = (traffic_from_profiles(p.name, backward, tag="bwdlse_" if args.from_forward else None)
               if args.variant == "fused" else None)
    # the roof that binds: HBM below the ridge (peak FLOP/s over peak bytes/s), MFMA above it
    intensity = nominal_flops / alg_bytes
    mfma_bound = intensity > peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": round(kernel_tflops, 1), "peak": peak_tf, "unit": "TFLOP/s",
             "frac": round(kernel_tflops / peak_tf, 4)} if mfma_bound else
            {"bound": "hbm", "achieved": round(achieved_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(achieved_gbs / PEAK_HBM_GBS, 4)})
    result = {
        "metric": METRIC_BWD if backward else METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, N(0,0.02^2) bias table)",
        "config": {
            "workload": p.name, "batch": p.batch, "grid_thw": list(p.extent),
            "padded_thw": list(p.padded), "window": list(p.window), "shift": list(p.shift),
            "heads": p.heads, "head_dim": p.head_dim, "variant": args.variant, "pass": args.which,
            **({"statistics": "forward" if args.from_forward else "recomputed"} if backward else {}),
            "input_sets_rotated": nsets,
        },
        "tokens_per_s": round(info.tokens / (ms_per_step * 1e-3), 1),
        "mfma_peak_frac": round(tflops / peak_tf, 5),
        "useful_tflops": round(useful / (ms_per_step * 1e-3) / 1e12, 3),
        "kernel": {"name": (("attn_f32_bwd_kernel" if p.dtype == "f32" else
                             ("attn_bf16_bwd_pkernel" if info.backward_workgroups > 0 else "attn_bf16_bwd_kernel")
                             if info.backward_schedule == 1 else
                             ("attn_bf16_bwd_q_kernel+attn_bf16_bwd_kvp_kernel" if info.backward_workgroups > 0
                              else "attn_bf16_bwd_q_kernel+attn_bf16_bwd_kv_kernel")) if backward
                            else kernel_name(p, info) if args.variant == "fused" else "gather+attn+scatter"),
                   "workgroups": info.backward_workgroups if backward else info.workgroups,
                   **launch_stats(launch_ms),
                   "source_sha256_16": kernel_source_hash(BWD_SOURCES if backward else None)},
        "warmup_calls": warm_steps,
        "warmup_ms": round(warm_ms, 1),
        "roofline": {
            **roof,
            "traffic": traffic,
            "algorithmic_gbs": round(achieved_gbs, 1),
            "intensity_flop_per_byte": round(intensity, 2),
            "algorithmic_bytes_per_launch": alg_bytes,
            "nominal_flops_per_launch": nominal_flops,
            "mfma_ceiling_frac_at_hbm_roof": round(
                min(1.0, nominal_flops / alg_bytes * PEAK_HBM_GBS * 1e9 / (peak_tf * 1e12)), 4),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        if backward:
            s0 = sets[0]
            step(0)
            torch.cuda.synchronize()
            per_b = p.windows // p.batch
            count = max(1, min(per_b, int(CPU_SAMPLE_FLOPS / 40 // (10.0 * p.window_tokens ** 2 * p.head_dim
                                                                     * p.heads))))
            wins = [int(w) for w in range(0, per_b, max(1, per_b // count))][:count]
            result["cpu_baseline"] = cpu_baseline_backward(p, x, s0["dout"].cpu(),
                                                           (s0["dq"], s0["dk"], s0["dv"]), wins)
        else:
            result["cpu_baseline"] = cpu_baseline(p, x, sets[0]["out"], args.cpu_rows)
    att.close()
    print(json.dumps(result), flush=True)


def timed(fn, steps):
    """Average milliseconds of fn() over `steps` calls, from HIP events recorded
    on torch's current stream (the stream the binding launches on)."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    return sorted(s.elapsed_time(e) for s, e in zip(starts, ends))


def cpu_baseline_layer(p, x, y_gpu, rows):
    import numpy as np

    import oracle

    T, H, W = p.extent
    C = p.heads * p.head_dim
    per_query = 8.0 * C * C + 4.0 * p.window_tokens * C
    per_row = per_query * p.batch * T * W
    # the projections run as numpy matrix products, several times faster than the C
    # attention per FLOP, so the sample is sized to 8x the attention sample's FLOPs
    rows = max(1, min(rows, H, int(8 * CPU_SAMPLE_FLOPS // per_row)))
    idx = np.array([((b * T + t) * H + y) * W + xx for b in range(p.batch) for t in range(T)
                    for y in range(rows) for xx in range(W)], dtype=np.int64)
    host = {n: t.float().numpy() for n, t in x.items()}
    # numpy's BLAS and the C oracle's OpenMP both take OMP_NUM_THREADS threads
    cores = min(os.cpu_count() or 1, int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    t0 = time.perf_counter()
    ref = oracle.layer_forward(p, host["x"], host["w_qkv"], host["b_qkv"], host["table"], host["w_o"], host["b_o"],
                               query_index=idx)
    dt = time.perf_counter() - t0
    got = y_gpu.float().cpu().numpy().reshape(p.tokens, C)[idx]
    err = float(np.abs(got - ref).max() / np.abs(ref).max())
    return {
        "value": per_query * len(idx) / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": (f"fp64 oracle layer (numpy projections of the windows the sample sees, C direct-form attention) "
                   f"for latitude rows 0..{rows - 1} of every time step and batch item ({len(idx)} of "
                   f"{p.tokens} tokens)"),
        "seconds": dt, "tokens_per_s": len(idx) / dt, "gpu_rel_max_abs_err_on_sample": err,
    }


def run_layer(args):
    import torch

    from shifted_window_attention_cyclic_amd import (WindowAttention, swa_forward, swa_layer_attention,
                                                      swa_layer_forward, swa_projection)
    from shifted_window_attention_cyclic_amd.inputs import WORKLOADS, make_layer_inputs

    p = WORKLOADS[args.workload]
    att = WindowAttention(p, args.variant, layer=args.layer)
    info = att.info
    fused = info.layer_path == 1  # SWA_LAYER_FUSED
    C = att.channels
    M = info.tokens
    eb = p.elem_bytes
    x = make_layer_inputs(p)
    set_bytes = 2.0 * M * C * eb
    nsets = max(1, min(8, math.ceil(3 * MALL_BYTES / set_bytes)))
    sets = []
    for i in range(nsets):
        xi = x if i == 0 else make_layer_inputs(p, seed=p.seed + 7919 * i)
        d = {n: t.cuda() for n, t in xi.items()}
        d["y"] = torch.empty_like(d["x"])
        sets.append(d)
    ws = att.layer_workspace()
    if fused:
        o = ws[:M * C]
        q = k = v = None
    else:
        q, k, v, o = (ws[i * M * C:(i + 1) * M * C] for i in range(4))

    def step(i):
        s = sets[i % nsets]
        swa_layer_forward(att.handle, s["x"], s["w_qkv"], s["b_qkv"], s["table"], s["w_o"], s["b_o"], s["y"], ws)

    warm_steps, warm_ms = warm_up(step, args.warmup, args.warmup_ms)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the kernels of a step, each timed alone through its own entry point
    # on the same inputs and stream
    def proj_qkv(i):
        s = sets[i % nsets]
        swa_projection(s["x"].view(M, C), s["w_qkv"], s["b_qkv"], [q, k, v], split=C)

    def attention(i):
        swa_forward(att.handle, q.view(att.io_shape), k.view(att.io_shape), v.view(att.io_shape),
                    sets[i % nsets]["table"], o.view(att.io_shape))

    def proj_out(i):
        s = sets[i % nsets]
        swa_projection(o.view(M, C), s["w_o"], s["b_o"], [s["y"].view(-1)])

    def qkv_attention(i):
        s = sets[i % nsets]
        swa_layer_attention(att.handle, s["x"], s["w_qkv"], s["b_qkv"], s["table"], o.view(att.io_shape))

    proj_flops_qkv = 2.0 * M * C * 3 * C
    proj_flops_out = 2.0 * M * C * C
    proj_name = "proj_bf16_kernel" if p.dtype == "bf16" else "proj_f32_kernel"
    # name: (call, kernel, flops, algorithmic bytes, kernel sources); projection
    # bytes: x and the weights read, the outputs written, the fp32 bias read;
    # the fused kernel reads x and the weights and writes the attention output
    if fused:
        kernels = {
            "qkv_attention": (qkv_attention, "layer_qkv_attn_kernel", proj_flops_qkv + info.nominal_flops,
                              (2 * M * C + 3 * C * C) * eb + 12.0 * C + 4.0 * math.prod(p.table_shape),
                              LAYER_SOURCES),
            "proj_out": (proj_out, proj_name, proj_flops_out, (2 * M * C + C * C) * eb + 4.0 * C, PROJ_SOURCES),
        }
    else:
        kernels = {
            "proj_qkv": (proj_qkv, proj_name, proj_flops_qkv, (M * C + 3 * C * C + 3 * M * C) * eb + 12.0 * C,
                         PROJ_SOURCES),
            "attention": (attention, kernel_name(p, info), info.nominal_flops, info.algorithmic_bytes,
                          KERNEL_SOURCES),
            "proj_out": (proj_out, proj_name, proj_flops_out, (2 * M * C + C * C) * eb + 4.0 * C, PROJ_SOURCES),
        }
    per_kernel = {}
    for name, (fn, kname, flops, nbytes, _) in kernels.items():
        warm_up(fn, args.warmup, args.warmup_ms / 3)
        ms = timed(fn, args.steps)
        st = launch_stats(ms)
        per_kernel[name] = {"kernel": kname, "avg_ms": st["avg_launch_ms"], "median_ms": st["median_ms"],
                            "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
                            "flops": flops, "algorithmic_bytes": nbytes}
    dom = max(per_kernel, key=lambda n: per_kernel[n]["avg_ms"])
    kd = per_kernel[dom]
    peak_tf = PEAK_BF16_TFLOPS if p.dtype == "bf16" else PEAK_F32_TFLOPS
    intensity = kd["flops"] / kd["algorithmic_bytes"]
    tf = kd["flops"] / (kd["avg_ms"] * 1e-3) / 1e12
    gbs = kd["algorithmic_bytes"] / (kd["avg_ms"] * 1e-3) / 1e9
    mfma_bound = intensity > peak_tf * 1e12 / (PEAK_HBM_GBS * 1e9)
    roof = ({"bound": "mfma", "achieved": round(tf, 1), "peak": peak_tf, "unit": "TFLOP/s",
             "frac": round(tf / peak_tf, 4)} if mfma_bound else
            {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4)})
    dom_sources = kernels[dom][4]
    traffic = (traffic_from_profiles(p.name, tag=f"layer_{dom}_", sources=dom_sources)
               if args.variant == "fused" else None)
    tflops = info.layer_flops / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": METRIC_LAYER,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": ("synthetic (seeded N(0,1) token embeddings, N(0,1/C) weights, N(0,0.02^2) biases and bias "
                 "table)"),
        "config": {
            "workload": p.name, "batch": p.batch, "grid_thw": list(p.extent), "padded_thw": list(p.padded),
            "window": list(p.window), "shift": list(p.shift), "heads": p.heads, "head_dim": p.head_dim,
            "channels": C, "variant": args.variant, "pass": "layer", "input_sets_rotated": nsets,
            "layer_path": "fused" if fused else "unfused",
        },
        "tokens_per_s": round(M / (ms_per_step * 1e-3), 1),
        "mfma_peak_frac": round(tflops / peak_tf, 5),
        "layer_flops_per_step": info.layer_flops,
        "kernels": per_kernel,
        "kernel": {"name": kd["kernel"], "step": dom, "avg_launch_ms": kd["avg_ms"], "median_ms": kd["median_ms"],
                   "p10_ms": kd["p10_ms"], "p90_ms": kd["p90_ms"], "source_sha256_16": kernel_source_hash(dom_sources)},
        "warmup_calls": warm_steps,
        "warmup_ms": round(warm_ms, 1),
        "roofline": {
            **roof,
            "traffic": traffic,
            "algorithmic_gbs": round(gbs, 1),
            "intensity_flop_per_byte": round(intensity, 2),
            "algorithmic_bytes_per_launch": kd["algorithmic_bytes"],
            "nominal_flops_per_launch": kd["flops"],
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        step(0)
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline_layer(p, x, sets[0]["y"], args.cpu_rows)
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    att.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
