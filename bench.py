#!/usr/bin/env python3
"""Throughput of the ternary linear layer path on one MI355X.

Default workload: BitNet-2B-shaped decode, one token (M = 1) streamed through 30
layers of {q, k, v, o: 2560->2560 / 2560->640, gate, up: 2560->6912, down:
6912->2560} with the per-token int8 activation quantisation fused into the
layers (bf16 activations between layers).  Chain per layer: q, k, v from the
layer input; o from q; gate and up from o; down from up; down is the next
layer's input.  One step = one token through the whole stack, replayed from a
HIP graph.  Weights are synthetic N(0, 0.02^2), seeded, ternarised on the GPU;
the stack is replicated so that the footprint cycled per step pair exceeds
1 GB (4x the 256 MB Infinity Cache) and weights really stream from HBM.

Printed: one JSON line with the packed-weight GB/s of the whole step (value),
the decode kernel's roofline (kernel durations from events stamped by the
kernel dispatch itself), the prefill kernel's int8 TOPS on the same layer
shapes at M = 512 and 4096, and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix peak (no sparsity)
CACHE_CYCLE_BYTES = 1 << 30      # cycle at least 1 GiB of weights between reuses


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="bitnet2b-decode-m1-30L")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this size (PMC calibration)")
    return p.parse_args()


def build_stack(torch, N, I, layer_shapes, layers, replicas):
    """Packed weights + scales on the GPU for replicas x layers x matrices."""
    stack = []
    for r in range(replicas):
        reps = []
        for l in range(layers):
            mats = {}
            for i, (nm, k, n) in enumerate(layer_shapes):
                g = torch.Generator(device="cuda").manual_seed(I.weight_seed(l, i) + 1_000_003 * r)
                w = torch.randn((n, k), generator=g, device="cuda", dtype=torch.float32)
                w.mul_(I.WEIGHT_SIGMA)
                mats[nm] = N.bitnet_quantize_weights(w)
                del w
            reps.append(mats)
        stack.append(reps)
    torch.cuda.synchronize()
    return stack


def decode_step_fn(torch, N, shapes, layers_mats, h0, bufs):
    """Enqueue one token through every layer (the chain described above)."""
    def step():
        h = bufs["h"]
        h.copy_(h0)
        for mats in layers_mats:
            N.bitnet_quant_linear(*mats["q"], h, x_q=bufs["xq_h"], x_scale=bufs["xs_h"], y=bufs["q"])
            N.bitnet_ternary_linear(*mats["k"], bufs["xq_h"], bufs["xs_h"], y=bufs["k"])
            N.bitnet_ternary_linear(*mats["v"], bufs["xq_h"], bufs["xs_h"], y=bufs["v"])
            N.bitnet_quant_linear(*mats["o"], bufs["q"], x_q=bufs["xq_q"], x_scale=bufs["xs_q"],
                                  y=bufs["o"])
            N.bitnet_quant_linear(*mats["gate"], bufs["o"], x_q=bufs["xq_o"], x_scale=bufs["xs_o"],
                                  y=bufs["gate"])
            N.bitnet_ternary_linear(*mats["up"], bufs["xq_o"], bufs["xs_o"], y=bufs["up"])
            N.bitnet_quant_linear(*mats["down"], bufs["up"], x_q=bufs["xq_u"], x_scale=bufs["xs_u"],
                                  y=h)
    return step


def time_decode_kernels(torch, N, layers_mats, xq_by_k, xs1, reps):
    """Per-launch durations of the decode kernel for every matrix of the stack,
    from events recorded by the kernel dispatch itself."""
    launches = []
    for mats in layers_mats:
        for nm, (p, s) in mats.items():
            launches.append((p, s))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in launches]
    for a, b in ev:
        a.record()
        b.record()
    outs = {p.shape[0]: torch.empty((1, p.shape[0]), dtype=torch.bfloat16, device="cuda")
            for p, _ in launches}
    durs, nbytes = [], []
    torch.cuda.synchronize()
    for _ in range(reps):
        for (p, s), (a, b) in zip(launches, ev):
            k = p.shape[1] * 4
            N.bitnet_ternary_linear_timed(p, s, xq_by_k[k], xs1, outs[p.shape[0]], a, b)
        torch.cuda.synchronize()
        for (p, _), (a, b) in zip(launches, ev):
            durs.append(a.elapsed_time(b) * 1e-3)
            nbytes.append(p.numel())
    return durs, nbytes


def prefill(torch, N, I, layer_shapes, mats, ms, steps):
    """int8 TOPS of the prefill kernel on one layer's matrices at M tokens."""
    res = {}
    for m in ms:
        xq = {}
        for _, k, _ in layer_shapes:
            if k not in xq:
                x = torch.randn((m, k), generator=torch.Generator(device="cuda").manual_seed(I.ACT_SEED),
                                device="cuda").to(torch.bfloat16)
                xq[k] = N.bitnet_quantize_acts(x)
        ys = {nm: torch.empty((m, n), dtype=torch.bfloat16, device="cuda") for nm, _, n in layer_shapes}
        ops = sum(2 * m * n * k for _, k, n in layer_shapes)

        def run():
            for nm, k, _ in layer_shapes:
                N.bitnet_ternary_linear(*mats[nm], *xq[k], y=ys[nm])
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        for _ in range(3):
            g.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3 / steps
        # kernel-own durations of the largest matrix
        nm, k, n = max(layer_shapes, key=lambda t: t[1] * t[2])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.record()
        kd = []
        for _ in range(5):
            N.bitnet_ternary_linear_timed(*mats[nm], *xq[k], ys[nm], a, b)
            torch.cuda.synchronize()
            kd.append(a.elapsed_time(b) * 1e-3)
        kd = sorted(kd)[len(kd) // 2]
        kop = 2 * m * n * k
        res[str(m)] = {"tops": round(ops / sec / 1e12, 2),
                       "frac_of_int8_peak": round(ops / sec / 1e12 / INT8_MFMA_PEAK_TOPS, 4),
                       "layer_ms": round(sec * 1e3, 4),
                       "largest_matrix": f"{k}->{n}",
                       "largest_matrix_kernel_us": round(kd * 1e6, 2),
                       "largest_matrix_kernel_tops": round(kop / kd / 1e12, 2)}
    return res


def cpu_baseline(I, layer_shapes, seconds):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole 2B-shaped layers at M = 1 (act-quant + layer per matrix)."""
    import numpy as np
    from oracle import bitnet_oracle as O
    mats = {}
    for i, (nm, k, n) in enumerate(layer_shapes):
        mats[nm] = O.quantize_weights(I.master_weights(n, k, I.weight_seed(0, i)))
    hk = layer_shapes[0][1]
    x0 = I.activations(1, hk)
    nbytes = 0
    layers_done = 0
    t0 = time.perf_counter()
    while True:
        h = x0
        qv = O.quant_linear(*mats["q"], h)[3]
        O.quant_linear(*mats["k"], h)
        O.quant_linear(*mats["v"], h)
        o = O.quant_linear(*mats["o"], qv)[3]
        O.quant_linear(*mats["gate"], o)
        u = O.quant_linear(*mats["up"], o)[3]
        O.quant_linear(*mats["down"], u)
        nbytes += sum(p.nbytes for p, _ in mats.values())
        layers_done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    _ = np
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{layers_done} x one 2B-shaped layer (7 matrices, "
                      f"{sum(p.nbytes for p, _ in mats.values())} packed bytes) at M=1, "
                      f"act-quant + unpack + int64 contraction + rescale, {el:.1f} s",
            "host": platform.processor() or platform.machine(), "host_threads": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    from ternary_weight_linear_bit_amd import _native as N
    from ternary_weight_linear_bit_amd import inputs as I

    wl = I.WORKLOADS[args.workload]
    shapes, layers = wl["layer"], wl["layers"]
    if wl["m"] != (1,) or len(shapes) != 7:
        raise SystemExit("bench.py times the layer-stack decode workloads")
    torch.cuda.set_device(0)
    N.lib()
    per_stack = I.packed_bytes(shapes) * layers
    replicas = max(1, math.ceil(CACHE_CYCLE_BYTES / per_stack))
    log(f"workload {args.workload}: {layers} layers, {per_stack / 1e6:.1f} MB packed per token, "
        f"{replicas} replicas")
    t0 = time.time()
    stack = build_stack(torch, N, I, shapes, layers, replicas)
    log(f"weights quantised on GPU in {time.time() - t0:.1f} s")

    act_dt = torch.bfloat16 if wl["act"] == "bf16" else torch.float32
    hidden = shapes[0][1]
    g = torch.Generator(device="cuda").manual_seed(I.ACT_SEED)
    h0 = torch.randn((1, hidden), generator=g, device="cuda").to(act_dt)
    sz = {nm: n for nm, _, n in shapes}
    kin = {nm: k for nm, k, _ in shapes}
    bufs = {nm: torch.empty((1, n), dtype=act_dt, device="cuda") for nm, n in sz.items()}
    bufs["h"] = torch.empty((1, hidden), dtype=act_dt, device="cuda")
    for tag, k in (("h", kin["q"]), ("q", kin["o"]), ("o", kin["gate"]), ("u", kin["down"])):
        bufs["xq_" + tag] = torch.empty((1, k), dtype=torch.int8, device="cuda")
        bufs["xs_" + tag] = torch.empty((1,), dtype=torch.float32, device="cuda")

    graphs = []
    for r in range(replicas):
        step = decode_step_fn(torch, N, shapes, stack[r], h0, bufs)
        step()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        graphs.append(gr)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        graphs[i % replicas].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    value = per_stack / (ms * 1e-3) / 1e9
    log(f"decode: {ms * 1e3:.1f} us/token, {value:.1f} GB/s packed")

    # decode kernel roofline: kernel-own durations over every matrix of one stack
    xq_by_k = {}
    for k in sorted(set(kin.values())):
        x = torch.randn((1, k), generator=g, device="cuda").to(act_dt)
        xq_by_k[k], xs1 = N.bitnet_quantize_acts(x)
    durs, nb = time_decode_kernels(torch, N, stack[0], xq_by_k, xs1, reps=min(5, max(1, args.steps)))
    avg_dur = sum(durs) / len(durs)
    avg_bytes = sum(nb) / len(nb)
    achieved = avg_bytes / avg_dur / 1e9
    log(f"decode kernel: {len(durs)} launches, avg {avg_dur * 1e6:.2f} us, "
        f"avg {avg_bytes / 1e6:.2f} MB -> {achieved:.0f} GB/s")

    result = {
        "metric": "decode GEMV packed-weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens_per_step": 1, "layers": layers,
                   "matrices_per_layer": len(shapes), "packed_bytes_per_step": per_stack,
                   "activations": wl["act"], "weight_replicas_cycled": replicas,
                   "launches_per_step": layers * len(shapes) + 1, "graph": "hip"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "gemv_kernel (decode, pre-quantised input)",
                     "launches_timed": len(durs), "avg_launch_us": round(avg_dur * 1e6, 3),
                     "avg_bytes_per_launch": int(avg_bytes)},
    }
    if not args.no_prefill:
        result["prefill"] = prefill(torch, N, I, shapes, stack[0][0], (512, 4096), steps=10)
        log(f"prefill: {result['prefill']}")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = 2 * a.numel() * 4
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(I, shapes, args.cpu_seconds)
        log(f"cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
