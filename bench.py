#!/usr/bin/env python3
"""Throughput of the ternary linear layer path on one MI355X.

Default workload (`bitnet2b-decode-m1-30L`): BitNet-2B-shaped decode, one token
(M = 1) streamed through 30 layers of {q, k, v: 2560->2560/640/640, o:
2560->2560, gate, up: 2560->6912, down: 6912->2560}, bf16 activations between
layers, the per-token int8 activation quantisation fused into the layers.
Chain per layer: q, k, v from the layer input (one launch); o from q; gate and up
from o (one launch); down from up; down is the next layer's input: 4 launches
per layer.  One step = one token through the whole stack, replayed from a HIP
graph.  Weights are synthetic N(0, 0.02^2), seeded, ternarised on the GPU by
the library; the stack is replicated so that more than 1 GiB of weights is cycled
between reuses (4x the 256 MB Infinity Cache) and weights stream from HBM.

Printed: one JSON line.  value = packed weight bytes per step / step time.
roofline = the decode kernel (the only kernel in the step): achieved = mean
packed bytes per launch / mean launch time, where the mean launch time is the
graph replay time over the timed steps divided by the number of launches (so it
includes the gap between dependent launches); traffic = HBM bytes per launch from
the PMC summary in profiles/, when it was taken on the current kernel sources.
Also: the same 2B chain as full layers (RMS norms and squared-ReLU gating fused
into the launches), the 8B-shaped stack (32 layers) at M = 1 and M = 16, the
100B-class decode stack (96 layers, 23.35 GB packed, fp32 activations), the
prefill kernel's int8 TOPS on the 2B layer shapes at M = 512 and 4096 and on the
8B shapes at M = 2048, the 2B and 100B chains with weights packed five per byte
(T1 layout, 1.6 bits per weight), single matrices at M = 1 through the
matrix-core kernel (2-bit and T1 weights) and the lookup-table path, the
standalone weight and activation quantisers against HBM, and the CPU oracle
timed on a bounded sample of the same decode workload (one core and all cores).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, vendor figure
INT8_MFMA_PEAK_TOPS = 5000.0     # MI355X dense int8 matrix peak (no sparsity)
CACHE_CYCLE_BYTES = 1 << 30      # cycle at least 1 GiB of weights between reuses


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def recorded_traffic():
    """HBM bytes per decode launch from the committed PMC summary, or None when the
    decode kernel's sources differ from the ones the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_bitnet2b_decode_chain.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-record:"):
            csrc = os.path.join(ROOT, "ternary_weight_linear_bit_amd", "csrc")
            for name, digest in re.findall(r"(\S+) sha256=([0-9a-f]{64})", line):
                data = open(os.path.join(csrc, name), "rb").read()
                if hashlib.sha256(data).hexdigest() != digest:
                    return None
            return int(re.search(r"bytes_per_launch=(\d+)", line).group(1))
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="bitnet2b-decode-m1-30L")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-100b", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the full-layer 2B chain and the 8B-shaped chains")
    p.add_argument("--no-t1", action="store_true",
                   help="skip the legs with weights packed five per byte")
    p.add_argument("--no-quant", action="store_true",
                   help="skip the standalone quantiser leg")
    p.add_argument("--no-compare", action="store_true",
                   help="skip the single-matrix comparison of the decode kernels")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this size (PMC calibration)")
    return p.parse_args()


def build_stack(torch, N, I, layer_shapes, layers, replicas, fmt="2bit"):
    """Packed weights + scales on the GPU for replicas x layers x matrices (2 bits
    per weight, or five weights per byte for fmt "t1")."""
    quantize = N.bitnet_quantize_weights_t1 if fmt == "t1" else N.bitnet_quantize_weights
    stack = []
    for r in range(replicas):
        reps = []
        for l in range(layers):
            mats = {}
            for i, (nm, k, n) in enumerate(layer_shapes):
                g = torch.Generator(device="cuda").manual_seed(I.weight_seed(l, i) + 1_000_003 * r)
                w = torch.randn((n, k), generator=g, device="cuda", dtype=torch.float32)
                w.mul_(I.WEIGHT_SIGMA)
                mats[nm] = quantize(w)
                del w
            reps.append(mats)
        stack.append(reps)
    torch.cuda.synchronize()
    return stack


def chain_fn(torch, N, layers_mats, h0, bufs, norms=None, eps=1e-5, fmt="2bit"):
    """Enqueue one step (M tokens) through every layer; returns the number of
    launches.  Plain chain: q, k, v from the layer input; o from q (attention is
    out of scope); gate and up from o; down from up.  Full layer (``norms``): an
    RMS norm in front of q/k/v and of gate/up, the sub-layer norm in front of o
    and of down, and down consumes ReLU(gate)^2 * up (the layer's neighbours as
    the BitNet b1.58 2B4T architecture names them), all fused into the launches."""
    m = h0.shape[0]
    per_multi = 1 if m <= 4 else 2   # fused act-quant, or act-quant + linear launches
    if fmt == "t1":
        def qlm(mats, x, **kw):
            return N.bitnet_quant_linear_t1(mats, x, **kw)
    else:
        def qlm(mats, x, **kw):
            return N.bitnet_quant_linear_multi(mats, x, **kw)

    def step():
        h = h0
        for li, mats in enumerate(layers_mats):
            nw = norms[li] if norms else None

            def pro(key, up=None):
                if nw is None:
                    return {}
                return dict(norm_weight=nw[key], eps=eps, up=up)
            qlm(
                [(*mats["q"], bufs["q"]), (*mats["k"], bufs["k"]), (*mats["v"], bufs["v"])], h,
                x_q=bufs["xq_h"], x_scale=bufs["xs_h"], **pro("in"))
            qlm([(*mats["o"], bufs["o"])], bufs["q"], x_q=bufs["xq_q"],
                                        x_scale=bufs["xs_q"], **pro("attn_sub"))
            qlm(
                [(*mats["gate"], bufs["gate"]), (*mats["up"], bufs["up"])], bufs["o"],
                x_q=bufs["xq_o"], x_scale=bufs["xs_o"], **pro("ffn_in"))
            if nw is None:
                qlm([(*mats["down"], bufs["h"])], bufs["up"],
                                            x_q=bufs["xq_u"], x_scale=bufs["xs_u"])
            else:
                qlm([(*mats["down"], bufs["h"])], bufs["gate"],
                                            x_q=bufs["xq_u"], x_scale=bufs["xs_u"],
                                            **pro("ffn_sub", up=bufs["up"]))
            h = bufs["h"]
        return 4 * per_multi * len(layers_mats)
    return step


def decode_leg(torch, N, I, name, steps, warmup, m=1, full_layer=False, min_cycle=None,
               fmt="2bit"):
    """M tokens at a time through a whole layer stack, replayed from HIP graphs."""
    wl = I.WORKLOADS[name]
    shapes, layers = wl["layer"], wl["layers"]
    per_stack = I.packed_bytes(shapes, fmt) * layers
    replicas = max(1, math.ceil((min_cycle or CACHE_CYCLE_BYTES) / per_stack))
    t0 = time.time()
    stack = build_stack(torch, N, I, shapes, layers, replicas, fmt)
    log(f"{name} ({fmt}): {layers} layers, {per_stack / 1e6:.1f} MB packed per step, "
        f"{replicas} replicas, weights ternarised on the GPU in {time.time() - t0:.1f} s")
    act_dt = torch.bfloat16 if wl["act"] == "bf16" else torch.float32
    hidden = shapes[0][1]
    g = torch.Generator(device="cuda").manual_seed(I.ACT_SEED)
    h0 = torch.randn((m, hidden), generator=g, device="cuda").to(act_dt)
    kin = {nm: k for nm, k, _ in shapes}
    bufs = {nm: torch.empty((m, n), dtype=act_dt, device="cuda") for nm, _, n in shapes}
    bufs["h"] = torch.empty((m, hidden), dtype=act_dt, device="cuda")
    for tag, k in (("h", kin["q"]), ("q", kin["o"]), ("o", kin["gate"]), ("u", kin["down"])):
        bufs["xq_" + tag] = torch.empty((m, k), dtype=torch.int8, device="cuda")
        bufs["xs_" + tag] = torch.empty((m,), dtype=torch.float32, device="cuda")
    norms = None
    if full_layer:
        norms = []
        for l in range(layers):
            norms.append({key: torch.from_numpy(I.norm_weight(kin[src], 50 + 4 * l + j)).cuda()
                          for j, (key, src) in enumerate((("in", "q"), ("attn_sub", "o"),
                                                          ("ffn_in", "gate"), ("ffn_sub", "down")))})
    graphs = []
    launches = 0
    for r in range(replicas):
        step = chain_fn(torch, N, stack[r], h0, bufs, norms, fmt=fmt)
        step()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            launches = step()
        graphs.append(gr)
    torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % replicas].replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        graphs[i % replicas].replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    pct = {q: per[min(steps - 1, int(q / 100 * steps))] for q in (10, 50, 90)}
    gbs = per_stack / (ms * 1e-3) / 1e9
    log(f"{name} ({fmt}, M={m}{', full layer' if full_layer else ''}): {ms * 1e3:.1f} us/step, "
        f"{gbs:.1f} GB/s packed, {ms * 1e3 / launches:.2f} us per launch")
    res = dict(ms=ms, gbs=gbs, per_stack=per_stack, replicas=replicas, launches=launches,
               weights=sum(n * k for _, k, n in shapes) * layers,
               layers=layers, shapes=shapes, act=wl["act"],
               ms_p10=pct[10], ms_median=pct[50], ms_p90=pct[90])
    del graphs, stack
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def leg_summary(d, m):
    return {"gbs": round(d["gbs"], 1), "frac_of_hbm_peak": round(d["gbs"] / HBM_PEAK_GBS, 4),
            "weights_per_s_G": round(d["weights"] / d["ms"] / 1e6, 1),
            "ms_per_step": round(d["ms"], 4), "tokens_per_s": round(m * 1e3 / d["ms"], 1),
            "packed_bytes_per_step": d["per_stack"], "launches_per_step": d["launches"],
            "avg_launch_us": round(d["ms"] * 1e3 / d["launches"], 3)}


def prefill(torch, N, I, layer_shapes, ms, steps):
    """int8 TOPS of the prefill kernel on one layer's matrices at M tokens (q, k, v
    in one launch, o, gate and up in one launch, down), and of its largest matrix
    alone."""
    names = [nm for nm, _, _ in layer_shapes]
    groups = [g for g in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
              if all(nm in names for nm in g)]
    assert sorted(sum(groups, ())) == sorted(names), "layer with an unknown matrix set"
    mats = {}
    for i, (nm, k, n) in enumerate(layer_shapes):
        g = torch.Generator(device="cuda").manual_seed(I.weight_seed(0, i))
        w = torch.randn((n, k), generator=g, device="cuda").mul_(I.WEIGHT_SIGMA)
        mats[nm] = N.bitnet_quantize_weights(w)
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

        kin = {nm: k for nm, k, _ in layer_shapes}

        def run(only=None, reps=1):
            for _ in range(reps):
                if only is not None:
                    N.bitnet_ternary_linear(*mats[only], *xq[kin[only]], y=ys[only])
                    continue
                # matrices that share an input run in one launch (q, k, v; gate, up)
                for grp in groups:
                    N.bitnet_ternary_linear_multi([(*mats[nm], ys[nm]) for nm in grp],
                                                  *xq[kin[grp[0]]])

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                fn()
            gr.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / steps

        sec = timed(run)
        nm, k, n = max(layer_shapes, key=lambda t: t[1] * t[2])
        ksec = timed(lambda: run(only=nm, reps=10)) / 10
        res[str(m)] = {"tops": round(ops / sec / 1e12, 2),
                       "frac_of_int8_peak": round(ops / sec / 1e12 / INT8_MFMA_PEAK_TOPS, 4),
                       "layer_ms": round(sec * 1e3, 4),
                       "largest_matrix": f"{k}->{n}",
                       "largest_matrix_us": round(ksec * 1e6, 2),
                       "largest_matrix_tops": round(2 * m * n * k / ksec / 1e12, 2)}
    return res


def kernel_compare(torch, N, I, shapes, steps):
    """Single matrices at M = 1: the matrix-core decode kernel on 2-bit weights,
    on T1 weights (five per byte), and the lookup-table path (three launches per
    token), each replayed from a HIP graph over >= 1 GiB of weight copies."""
    res = {}
    for k, n in shapes:
        g = torch.Generator(device="cuda").manual_seed(I.weight_seed(0, 0))
        w = torch.randn((n, k), generator=g, device="cuda").mul_(I.WEIGHT_SIGMA)
        p2, sc = N.bitnet_quantize_weights(w)
        del w
        x = torch.randn((1, k), generator=torch.Generator(device="cuda").manual_seed(I.ACT_SEED),
                        device="cuda").to(torch.bfloat16)
        xq, xs = N.bitnet_quantize_acts(x)
        y = torch.empty((1, n), device="cuda")
        ws = torch.empty(N.lib().bitnet_lut_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
        row = {}
        for path in ("mfma_2bit", "mfma_t1", "lut_2bit"):
            base = N.bitnet_repack_t1(p2) if path == "mfma_t1" else p2
            nbytes = base.numel()
            copies = max(2, math.ceil(CACHE_CYCLE_BYTES / nbytes))
            mats = [base.clone() for _ in range(copies)]

            def run():
                for c in range(copies):
                    if path == "mfma_2bit":
                        N.bitnet_ternary_linear(mats[c], sc, xq, xs, y=y)
                    elif path == "mfma_t1":
                        N.bitnet_ternary_linear_t1([(mats[c], sc, y)], xq, xs)
                    else:
                        N.bitnet_ternary_linear_lut(mats[c], sc, xq, xs, y=y, workspace=ws)
            run()
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                run()
            gr.replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(steps):
                gr.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (steps * copies)
            row[path] = {"us": round(us, 2), "packed_gbs": round(nbytes / us / 1e3, 1),
                         "weights_per_s_G": round(n * k / us / 1e3, 1)}
            del gr, mats
            torch.cuda.empty_cache()
        res[f"{k}->{n}"] = row
        log(f"compare {k}->{n}: {row}")
    return res


def quantisers(torch, N, I, steps):
    """The standalone quantisers against HBM: bitnet_quantize_weights (absmean
    scale + ternary 2-bit pack; two passes over the master weights, 2 x (2|4) B
    in + 0.25 B out per weight) and bitnet_quantize_acts (per-token absmax int8;
    M K (2|4) B in, M K + 4 M B out).  Each shape runs over >= 1 GiB of input
    copies, replayed from a HIP graph, so inputs stream from HBM."""
    res = {}
    for n, k, dt in ((6912, 2560, torch.float32), (6912, 2560, torch.bfloat16),
                     (28672, 8192, torch.float32)):
        es = 2 if dt == torch.bfloat16 else 4
        copies = max(2, math.ceil(CACHE_CYCLE_BYTES / (n * k * es)))
        g = torch.Generator(device="cuda").manual_seed(I.weight_seed(0, 0))
        ws = [torch.randn((n, k), generator=g, device="cuda").mul_(I.WEIGHT_SIGMA).to(dt)
              for _ in range(copies)]
        packed = torch.empty((n, k // 4), dtype=torch.uint8, device="cuda")
        scale = torch.empty(1, dtype=torch.float32, device="cuda")
        work = torch.empty(N.lib().bitnet_quantize_weights_workspace_bytes(n, k),
                           dtype=torch.uint8, device="cuda")
        us = _graph_time(torch, lambda: [N.bitnet_quantize_weights(w, packed, scale, work)
                                         for w in ws], steps) / copies
        nbytes = n * k * (2 * es) + n * k // 4
        res[f"weights {n}x{k} {'bf16' if es == 2 else 'f32'}"] = {
            "us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
            "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del ws, packed, scale, work
        torch.cuda.empty_cache()
    for m, k in ((4096, 6912), (4096, 2560), (2048, 14336)):
        copies = max(2, math.ceil(CACHE_CYCLE_BYTES / (m * k * 2)))
        g = torch.Generator(device="cuda").manual_seed(I.ACT_SEED)
        xs = [torch.randn((m, k), generator=g, device="cuda").to(torch.bfloat16) for _ in range(copies)]
        x_q = torch.empty((m, k), dtype=torch.int8, device="cuda")
        x_s = torch.empty(m, dtype=torch.float32, device="cuda")
        us = _graph_time(torch, lambda: [N.bitnet_quantize_acts(x, x_q, x_s) for x in xs],
                         steps) / copies
        nbytes = m * k * 2 + m * k + 4 * m
        res[f"acts {m}x{k} bf16"] = {"us": round(us, 2), "gbs": round(nbytes / us / 1e3, 1),
                                     "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        del xs, x_q, x_s
        torch.cuda.empty_cache()
    log(f"quantisers: {res}")
    return res


def mfma_ceiling(torch, N):
    """The chip's int8 matrix-core rate (bitnet_probe_mfma_i8, two waves per SIMD,
    ten launches of ~2 ms per operand kind, before the prefill legs): all-zero
    operands (the issue rate: no data switching), all-ones, and random int8
    activations against random ternary codes {0, 1, 2} (the prefill kernel's
    operands).  The rate falls as more operand bits switch: the chip's power
    management lowers the clock."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters, launches = 2 * cus, 2000, 10
    res = {"waves_per_simd": 2}
    for kind in ("zero", "ones", "random_int8_x_ternary"):
        ops = torch.full((wgs * 256, 16, 16), 1 if kind == "ones" else 0, dtype=torch.uint8,
                         device="cuda")
        if kind == "random_int8_x_ternary":
            g = torch.Generator(device="cuda").manual_seed(11)
            ops[:, :8] = torch.randint(0, 256, (wgs * 256, 8, 16), generator=g, device="cuda",
                                       dtype=torch.uint8)
            ops[:, 8:] = torch.randint(0, 3, (wgs * 256, 8, 16), generator=g, device="cuda",
                                       dtype=torch.uint8)
        out = torch.empty((wgs * 256, 64), dtype=torch.uint8, device="cuda")
        N.bitnet_probe_mfma_i8(ops, wgs, iters, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            N.bitnet_probe_mfma_i8(ops, wgs, iters, out)
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3
        res[f"{kind}_tops"] = round(launches * wgs * 4 * iters * 32 * 65536 / sec / 1e12, 1)
        del ops, out
    res["frac_of_peak"] = {k: round(v / INT8_MFMA_PEAK_TOPS, 4) for k, v in res.items()
                           if k.endswith("_tops")}
    log(f"mfma ceiling: {res}")
    return res


def _graph_time(torch, fn, steps):
    """Mean microseconds of one replay of fn captured in a HIP graph."""
    fn()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fn()
    gr.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    del gr
    return us


_ORACLE_LAYER = None   # (mats, x0) shared with forked workers


def _oracle_layers(seconds):
    """Whole 2B-shaped layers at M = 1 through the oracle for `seconds`:
    (packed bytes streamed, layers, elapsed)."""
    from oracle import bitnet_oracle as O
    mats, x0 = _ORACLE_LAYER
    per_layer = sum(p.nbytes for p, _ in mats.values())
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
        layers_done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return per_layer * layers_done, layers_done, el


def cpu_baseline(I, layer_shapes, seconds, workers):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole 2B-shaped layers at M = 1 (act-quant + layer per matrix), on one core
    and on `workers` processes at once (each runs its own layers; numpy's integer
    contraction is single-threaded).  Runs before the GPU is touched, so the
    worker processes are plain forks."""
    global _ORACLE_LAYER
    from oracle import bitnet_oracle as O
    mats = {}
    for i, (nm, k, n) in enumerate(layer_shapes):
        mats[nm] = O.quantize_weights(I.master_weights(n, k, I.weight_seed(0, i)))
    _ORACLE_LAYER = (mats, I.activations(1, layer_shapes[0][1]))
    per_layer = sum(p.nbytes for p, _ in mats.values())
    nbytes, layers_done, el = _oracle_layers(seconds)
    res = {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{layers_done} x one 2B-shaped layer (7 matrices, {per_layer} packed bytes) "
                     f"at M=1, act-quant + unpack + int64 contraction + rescale, {el:.1f} s",
           "host": platform.processor() or platform.machine(), "host_threads": os.cpu_count()}
    if workers > 1:
        import multiprocessing
        with multiprocessing.get_context("fork").Pool(workers) as pool:
            parts = pool.map(_oracle_layers, [seconds] * workers)
        total = sum(b for b, _, _ in parts)
        wall = max(e for _, _, e in parts)
        res["all_cores"] = {"value": round(total / wall / 1e9, 4), "unit": "GB/s", "cores": workers,
                            "sample": f"{sum(n for _, n, _ in parts)} layers over {workers} processes, "
                                      f"{wall:.1f} s"}
    _ORACLE_LAYER = None
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    import torch
    from ternary_weight_linear_bit_amd import _native as N
    from ternary_weight_linear_bit_amd import inputs as I

    wl = I.WORKLOADS[args.workload]
    if wl["m"] != (1,) or len(wl["layer"]) != 7:
        raise SystemExit("bench.py times the layer-stack decode workloads")
    cpu = None
    if not args.no_cpu_baseline:
        # before the GPU is initialised: the all-cores leg forks worker processes
        workers = min(16, os.cpu_count() or 1)
        cpu = cpu_baseline(I, wl["layer"], args.cpu_seconds, workers)
        log(f"cpu baseline: {cpu}")
    torch.cuda.set_device(0)
    N.lib()
    d = decode_leg(torch, N, I, args.workload, args.steps, args.warmup)
    avg_launch = d["ms"] * 1e-3 / d["launches"]
    avg_bytes = d["per_stack"] / d["launches"]
    achieved = avg_bytes / avg_launch / 1e9
    result = {
        "metric": "decode GEMV packed-weight GB/s (% HBM peak); prefill int8 TOPS (% MFMA peak)",
        "value": round(d["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens_per_step": 1, "layers": d["layers"],
                   "matrices_per_layer": len(d["shapes"]), "packed_bytes_per_step": d["per_stack"],
                   "activations": d["act"], "weight_replicas_cycled": d["replicas"],
                   "launches_per_step": d["launches"], "graph": "hip"},
        "ms_per_step_p10_median_p90": [round(d["ms_p10"], 5), round(d["ms_median"], 5),
                                       round(d["ms_p90"], 5)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(),
                     "kernel": "gemv_kernel (decode, fused int8 activation quantisation)",
                     "avg_launch_us": round(avg_launch * 1e6, 3),
                     "avg_bytes_per_launch": int(avg_bytes),
                     "launch_time": "graph replay time / launches in the timed steps"},
    }
    if not args.no_extra:
        df = decode_leg(torch, N, I, args.workload, args.steps, args.warmup, full_layer=True)
        result["decode_full_layer"] = dict(
            workload=args.workload + " with RMS norms and squared-ReLU gating fused in",
            **leg_summary(df, 1))
        for m in (1, 16):
            d8 = decode_leg(torch, N, I, "llama8b-ternary", max(5, args.steps // 3), 2, m=m)
            result[f"decode_8b_m{m}"] = dict(workload="llama8b-ternary (32 layers)",
                                             **leg_summary(d8, m))
    if not args.no_t1:
        dt = decode_leg(torch, N, I, args.workload, args.steps, args.warmup, fmt="t1")
        result["decode_t1"] = dict(workload=args.workload + ", weights five per byte (T1 layout)",
                                   **leg_summary(dt, 1))
    if not args.no_100b:
        d5 = decode_leg(torch, N, I, "ternary100b-decode-m1-96L", max(5, args.steps // 5), 2)
        result["decode_100b"] = dict(workload="ternary100b-decode-m1-96L", **leg_summary(d5, 1))
        if not args.no_t1:
            d6 = decode_leg(torch, N, I, "ternary100b-decode-m1-96L", max(5, args.steps // 5), 2,
                            fmt="t1")
            result["decode_100b_t1"] = dict(
                workload="ternary100b-decode-m1-96L, weights five per byte (T1 layout)",
                **leg_summary(d6, 1))
    if not args.no_quant:
        result["quantisers"] = quantisers(torch, N, I, steps=3)
    if not args.no_compare:
        result["kernel_compare_m1"] = kernel_compare(
            torch, N, I, ((2560, 2560), (2560, 6912), (6912, 2560), (8192, 28672), (28672, 8192)),
            steps=4)
    if not args.no_prefill:
        result["mfma_ceiling"] = mfma_ceiling(torch, N)
        result["prefill"] = prefill(torch, N, I, wl["layer"], (512, 4096), steps=10)
        result["prefill_8b"] = prefill(torch, N, I, I.LAYER_8B, (2048,), steps=5)
        log(f"prefill: {result['prefill']} {result['prefill_8b']}")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 18
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        result["calib_copy_bytes"] = 2 * a.numel() * 4
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
