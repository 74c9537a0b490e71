#!/usr/bin/env python3
"""Throughput of the ternary linear layer path on one MI355X.

Default workload (`ternary100b-decode-m1-96L`): the ~100B-class ternary decode
stack, one token (M = 1) streamed through 96 layers of {q, k, v, o: 8192->8192,
gate, up: 8192->28672, down: 28672->8192} with fp32 activations between layers
and the per-token int8 activation quantisation fused into every layer (23.35 GB
of packed weights per token, resident in HBM).  Chain per layer: q, k, v from
the layer input (one launch); o from q (attention is out of scope); gate and up
from o (one launch); down from up; down is the next layer's input: 4 launches per
layer, 384 per token, replayed from a HIP graph.  Weights are synthetic
N(0, 0.02^2), seeded, ternarised on the GPU by the library.

Printed: one JSON line.  value = packed weight bytes per token / token time.
roofline = the decode kernel (the only kernel in the step): achieved = packed
bytes per launch / mean launch time, the graph replay time of the timed steps
(HIP events on the stream the kernels run on) over the launches; traffic = HBM
bytes per launch from the PMC summary in profiles/, when it was taken on the
current kernel sources.  Also: the BitNet-2B-shaped decode stack (30 layers,
bf16 activations; plain and with RMS norms and squared-ReLU gating fused), the
8B-shaped stack at M = 1 and 16, the same 2B and 100B stacks through the
one-launch decode chain and with weights packed five per byte (T1), the prefill
kernel's int8 TOPS on the 2B shapes at M = 512 and 4096 and on the 8B shapes at
M = 2048 (with its own roofline block), single matrices at M = 1 through the
matrix-core kernel, T1 and the lookup-table path, the standalone quantisers
against HBM, and the CPU oracle timed on bounded samples of the decode and
prefill workloads (one core and all cores); the 100B-class stack again with bf16
activations between layers.
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


def recorded_traffic(profile="gemv_100b_decode_stack.md", workload=None):
    """HBM bytes per decode launch from the committed PMC summary, or None when the
    decode kernel's sources differ from the ones the counters were taken on, or the
    record names another workload than `workload`."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-record:"):
            csrc = os.path.join(ROOT, "ternary_weight_linear_bit_amd", "csrc")
            for name, digest in re.findall(r"(\S+) sha256=([0-9a-f]{64})", line):
                data = open(os.path.join(csrc, name), "rb").read()
                if hashlib.sha256(data).hexdigest() != digest:
                    return None
            wl = re.search(r"workload=(\S+)", line)
            if workload is not None and wl is not None and wl.group(1) != workload:
                return None
            return int(re.search(r"bytes_per_launch=(\d+)", line).group(1))
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="ternary100b-decode-m1-96L")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-prefill", action="store_true")
    p.add_argument("--no-2b", action="store_true", help="skip the 2B-shaped decode stacks")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the full-layer 2B stack and the 8B-shaped stacks")
    p.add_argument("--no-chain", action="store_true",
                   help="skip the one-launch decode chain legs")
    p.add_argument("--no-t1", action="store_true",
                   help="skip the legs with weights packed five per byte")
    p.add_argument("--no-quant", action="store_true",
                   help="skip the standalone quantiser leg")
    p.add_argument("--no-compare", action="store_true",
                   help="skip the single-matrix comparison of the decode kernels")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--sustain-seconds", type=float, default=8.0,
                   help="after every other leg, run the headline stack for this long "
                        "(reported as decode_sustained; 0: skip)")
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
               fmt="2bit", sustain_s=0.0):
    """M tokens at a time through a whole layer stack, replayed from HIP graphs.
    With sustain_s > 0, the stack then runs on for about that many seconds, timed
    on its own (the sustained rate: clocks and temperature under continuous load)."""
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
    if sustain_s > 0:
        n_sus = max(1, int(sustain_s * 1e3 / ms))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_sus):
            graphs[i % replicas].replay()
        e1.record()
        torch.cuda.synchronize()
        ms_sus = e0.elapsed_time(e1) / n_sus
        res["sustained"] = {"steps": n_sus, "seconds": round(ms_sus * n_sus * 1e-3, 2),
                            "ms_per_step": round(ms_sus, 5),
                            "gbs": round(per_stack / (ms_sus * 1e-3) / 1e9, 1)}
        log(f"{name}: sustained {n_sus} steps, {ms_sus * 1e3:.1f} us/step")
    del graphs, stack
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def chain_leg(torch, N, I, name, steps, warmup, m=1, min_cycle=None, ring=None):
    """The same stack through the decode chain: one cooperative launch per token
    runs every layer's four fused act-quant + linear stages with grid barriers
    between them (bitnet_chain_plan / bitnet_chain_run)."""
    wl = I.WORKLOADS[name]
    shapes, layers = wl["layer"], wl["layers"]
    per_stack = I.packed_bytes(shapes) * layers
    replicas = max(1, math.ceil((min_cycle or CACHE_CYCLE_BYTES) / per_stack))
    t0 = time.time()
    stack = build_stack(torch, N, I, shapes, layers, replicas)
    log(f"{name} (chain): {layers} layers, {per_stack / 1e6:.1f} MB packed per step, "
        f"{replicas} replicas, weights ternarised on the GPU in {time.time() - t0:.1f} s")
    act_dt = torch.bfloat16 if wl["act"] == "bf16" else torch.float32
    hidden = shapes[0][1]
    g = torch.Generator(device="cuda").manual_seed(I.ACT_SEED)
    h0 = torch.randn((m, hidden), generator=g, device="cuda").to(act_dt)
    kin = {nm: k for nm, k, _ in shapes}
    bufs = {nm: torch.empty((m, n), dtype=act_dt, device="cuda") for nm, _, n in shapes}
    for tag, k in (("h", kin["q"]), ("q", kin["o"]), ("o", kin["gate"]), ("u", kin["down"])):
        bufs["xq_" + tag] = torch.empty((m, k), dtype=torch.int8, device="cuda")
        bufs["xs_" + tag] = torch.empty((m,), dtype=torch.float32, device="cuda")
    chains = []
    for r in range(replicas):
        st = []
        h = h0
        for mats in stack[r]:
            st.append(dict(x=h, x_q=bufs["xq_h"], x_scale=bufs["xs_h"],
                           mats=[(*mats["q"], bufs["q"]), (*mats["k"], bufs["k"]),
                                 (*mats["v"], bufs["v"])]))
            st.append(dict(x=bufs["q"], x_q=bufs["xq_q"], x_scale=bufs["xs_q"],
                           mats=[(*mats["o"], bufs["o"])]))
            st.append(dict(x=bufs["o"], x_q=bufs["xq_o"], x_scale=bufs["xs_o"],
                           mats=[(*mats["gate"], bufs["gate"]), (*mats["up"], bufs["up"])]))
            st.append(dict(x=bufs["up"], x_q=bufs["xq_u"], x_scale=bufs["xs_u"],
                           mats=[(*mats["down"], bufs["down"])]))
            h = bufs["down"]
        c = N.bitnet_chain_plan(st, m)
        if ring:
            c.handle.ring = ring
        chains.append(c)
    for i in range(max(warmup, replicas)):
        N.bitnet_chain_run(chains[i % replicas])
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        N.bitnet_chain_run(chains[i % replicas])
        evs[i + 1].record()
    torch.cuda.synchronize()
    err = max(N.bitnet_chain_error(c) for c in chains)
    if err:
        raise RuntimeError(f"decode chain abandoned a barrier (error word {err})")
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    pct = {q: per[min(steps - 1, int(q / 100 * steps))] for q in (10, 50, 90)}
    gbs = per_stack / (ms * 1e-3) / 1e9
    log(f"{name} (chain, M={m}, ring {chains[0].handle.ring}, grid {chains[0].handle.grid}): "
        f"{ms * 1e3:.1f} us/step, {gbs:.1f} GB/s packed")
    res = dict(ms=ms, gbs=gbs, per_stack=per_stack, replicas=replicas, launches=1,
               weights=sum(n * k for _, k, n in shapes) * layers, layers=layers, shapes=shapes,
               act=wl["act"], ms_p10=pct[10], ms_median=pct[50], ms_p90=pct[90],
               ring=chains[0].handle.ring, grid=chains[0].handle.grid)
    del chains, stack
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
    alone: with the weights in the prefill layout (repacked once from the 2-bit
    rows, outside the timed region), the headline, and in the 2-bit row layout."""
    names = [nm for nm, _, _ in layer_shapes]
    groups = [g for g in (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
              if all(nm in names for nm in g)]
    assert sorted(sum(groups, ())) == sorted(names), "layer with an unknown matrix set"
    mats, pre = {}, {}
    for i, (nm, k, n) in enumerate(layer_shapes):
        g = torch.Generator(device="cuda").manual_seed(I.weight_seed(0, i))
        w = torch.randn((n, k), generator=g, device="cuda").mul_(I.WEIGHT_SIGMA)
        mats[nm] = N.bitnet_quantize_weights(w)
        pre[nm] = (N.bitnet_repack_prefill(mats[nm][0]), mats[nm][1], n)
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

        def run(only=None, reps=1, layout="prefill"):
            for _ in range(reps):
                # matrices that share an input run in one launch (q, k, v; gate, up)
                for grp in ((only,),) if only is not None else groups:
                    if layout == "prefill":
                        N.bitnet_ternary_linear_prefill([(*pre[nm], ys[nm]) for nm in grp],
                                                        *xq[kin[grp[0]]])
                    else:
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
        sec_rows = timed(lambda: run(layout="rows"))
        nm, k, n = max(layer_shapes, key=lambda t: t[1] * t[2])
        ksec = timed(lambda: run(only=nm, reps=10)) / 10
        tops = ops / sec / 1e12
        res[str(m)] = {"tops": round(tops, 2),
                       "frac_of_int8_peak": round(tops / INT8_MFMA_PEAK_TOPS, 4),
                       "layer_ms": round(sec * 1e3, 4),
                       "weights": "prefill layout (repacked once from the 2-bit rows)",
                       "row_layout_tops": round(ops / sec_rows / 1e12, 2),
                       "row_layout_layer_ms": round(sec_rows * 1e3, 4),
                       "largest_matrix": f"{k}->{n}",
                       "largest_matrix_us": round(ksec * 1e6, 2),
                       "largest_matrix_tops": round(2 * m * n * k / ksec / 1e12, 2),
                       "roofline": {"bound": "mfma", "achieved": round(tops, 1),
                                    "peak": INT8_MFMA_PEAK_TOPS, "unit": "TOPS (int8)",
                                    "frac": round(tops / INT8_MFMA_PEAK_TOPS, 4), "traffic": None,
                                    "kernel": "gemm_kernel (prefill, int8 MFMA, prefill layout)",
                                    "ops": "2 M N K per launch, zero weights counted (the "
                                           "sum_pos - sum_neg form needs ~0.69 M N K add/subs)",
                                    "launches_per_layer": 4,
                                    "avg_launch_us": round(sec * 1e6 / 4, 2)}}
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


def mfma_ceiling(torch):
    """The chip's int8 matrix-core rate (a bench-only probe library, two waves per
    SIMD, ten launches of ~2 ms per operand kind, before the prefill legs):
    all-zero operands (the issue rate: no data switching), all-ones, and random
    int8 activations against random ternary codes {0, 1, 2} (the prefill kernel's
    operands); with the shader clock the probe's waves saw under that load and
    the rate per clock and SIMD (2048 int8 ops is the matrix core's full rate).
    Context only: the roofline peak stays the published 5.0 POPS."""
    import ctypes
    path = os.path.join(ROOT, "ternary_weight_linear_bit_amd", "libbitnet_bench_probe.so")
    probe = ctypes.CDLL(path).bitnet_bench_probe_mfma_i8
    probe.restype = ctypes.c_int
    probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
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
        clk = torch.zeros((wgs * 4, 2), dtype=torch.int64, device="cuda")

        def run():
            if probe(ops.data_ptr(), wgs, iters, out.data_ptr(), clk.data_ptr(), stream) != 0:
                raise RuntimeError("matrix-core probe launch failed")
        run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            run()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) * 1e-3
        tops = launches * wgs * 4 * iters * 32 * 65536 / sec / 1e12
        c = clk.double()
        ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
        simds = 4 * cus
        res[f"{kind}_tops"] = round(tops, 1)
        res[f"{kind}_clock_ghz"] = round(ghz, 3)
        res[f"{kind}_ops_per_clock_per_simd"] = round(tops * 1e12 / (ghz * 1e9) / simds, 1)
        del ops, out, clk
    res["frac_of_peak"] = {k: round(v / INT8_MFMA_PEAK_TOPS, 4) for k, v in res.items()
                           if k.endswith("_tops")}
    log(f"mfma ceiling: {res}")
    return res


def _probe_lib():
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "ternary_weight_linear_bit_amd", "libbitnet_bench_probe.so"))
    lib.bitnet_bench_probe_read.restype = ctypes.c_int
    lib.bitnet_bench_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                            ctypes.c_void_p]
    lib.bitnet_bench_probe_empty.restype = ctypes.c_int
    lib.bitnet_bench_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    return lib


def hbm_read_ceiling(torch, gib=4, launches=5):
    """HBM read rate of this chip (bench-only probe library), the context for the
    decode kernel's roofline: a 4 GiB buffer (larger than the 256 MB Infinity
    Cache) read once per launch, streamed with 16-byte loads (1 KiB per wave
    load) at 1, 2 and 8 workgroups per CU, and in the decode kernel's pattern
    (16 rows x 64 bytes per wave load over 8192-weight rows) at 2 and 3 per CU.
    The roofline peak stays the published 8 TB/s."""
    lib = _probe_lib()
    stream = torch.cuda.current_stream().cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = gib << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    res = {"bytes_per_launch": nbytes}
    for name, pattern, rowb, per_cu in (("stream_16B_loads", 0, 0, (1, 2, 8)),
                                        ("decode_pattern_rows_2048B", 1, 2048, (2, 3))):
        res[name] = {}
        for k in per_cu:
            wgs = k * cus
            out = torch.empty(wgs * 4096, dtype=torch.uint8, device="cuda")

            def run():
                if lib.bitnet_bench_probe_read(buf.data_ptr(), nbytes, pattern, rowb, wgs,
                                               out.data_ptr(), stream) != 0:
                    raise RuntimeError("read probe launch failed")
            run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(launches):
                run()
            e1.record()
            torch.cuda.synchronize()
            res[name][f"gbs_{wgs}_workgroups"] = round(
                launches * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
            del out
    best = max(v for name in ("stream_16B_loads", "decode_pattern_rows_2048B")
               for v in res[name].values())
    res["best_gbs"] = best
    res["best_frac_of_hbm_peak"] = round(best / HBM_PEAK_GBS, 4)
    del buf
    log(f"hbm read ceiling: {res}")
    return res


def launch_gap(torch, launches=400):
    """Cost of a dependent launch: an empty kernel replayed from a HIP graph
    (one workgroup, and two workgroups per CU like the decode kernel)."""
    lib = _probe_lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for wgs in (1, 2 * cus):
        def run():
            for _ in range(launches):
                if lib.bitnet_bench_probe_empty(wgs, torch.cuda.current_stream().cuda_stream) != 0:
                    raise RuntimeError("empty probe launch failed")
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[f"us_per_empty_launch_{wgs}_workgroups"] = round(e0.elapsed_time(e1) * 1e3 / (5 * launches), 3)
        del g
    log(f"launch gap: {res}")
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


_ORACLE = None   # the CPU sample's matrices and inputs, shared with forked workers


def _random_packed(I, n, k, seed):
    """Packed ternary codes [N, K/4] with the value distribution of absmean-quantised
    N(0, sigma) weights: P(0) = 0.31, P(+1) = P(-1) = 0.345 (the CPU sample needs
    only valid codes of that mix; generating and quantising fp32 masters of the
    100B-class shapes on the host would take minutes)."""
    from oracle import bitnet_oracle as O
    import numpy as np
    u = np.random.Generator(np.random.PCG64(seed)).random((n, k), dtype=np.float32)
    q = (u > np.float32(0.655)).astype(np.int8) - (u < np.float32(0.345)).astype(np.int8)
    return O.pack_codes(q)


def _oracle_decode(seconds):
    """100B-class layers at M = 1 through the oracle for `seconds`: act-quant +
    unpack + integer contraction + rescale per matrix, with the stack's data flow
    (q, k, v from h; o from q; gate, up from o; down from up; h <- down).
    Returns (packed bytes streamed, matrices, elapsed)."""
    from oracle import bitnet_oracle as O
    mats, x0 = _ORACLE["decode"]
    nbytes = done = 0
    t0 = time.perf_counter()
    h = x0

    def lin(nm, x):
        nonlocal nbytes, done
        p, g = mats[nm]
        y = O.quant_linear(p, g, x)[3]
        nbytes += p.nbytes
        done += 1
        return y
    while True:
        q = lin("qkv", h)
        lin("qkv", h)
        lin("qkv", h)
        o = lin("o", q)
        lin("gu", o)
        up = lin("gu", o)
        h = lin("down", up)
        el = time.perf_counter() - t0
        if el >= seconds:
            return nbytes, done, el


def _oracle_prefill(seconds):
    """The 2B-shaped layer's matrices at M tokens through the oracle's integer
    contraction (plus act-quant and rescale) for `seconds`: (int8 ops, elapsed)."""
    from oracle import bitnet_oracle as O
    mats, xs = _ORACLE["prefill"]
    ops = 0
    t0 = time.perf_counter()
    while True:
        for p, g in mats:
            x = xs[p.shape[1] * 4]
            O.quant_linear(p, g, x)
            ops += 2 * x.shape[0] * p.shape[0] * p.shape[1] * 4
            el = time.perf_counter() - t0
            if el >= seconds:
                return ops, el


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(I, seconds, workers, prefill_m=64):
    """The CPU oracle, as it stands, on bounded samples of the same workloads, on one
    core and on `workers` processes at once (each runs its own sample; numpy's
    integer contraction is single-threaded).  Decode: the 100B-class layer's three
    matrix shapes at M = 1 in the stack's order, scaled to packed-weight GB/s.
    Prefill: the 2B-shaped layer's matrices at `prefill_m` tokens (a slice of the
    M = 512 batch), scaled to int8 TOPS (2 M N K).  Runs before the GPU is touched,
    so the worker processes are plain forks."""
    global _ORACLE
    import numpy as np
    from oracle import bitnet_oracle as O
    shapes = {nm: (k, n) for nm, k, n in I.LAYER_100B}
    dec = {"qkv": (_random_packed(I, 8192, 8192, 1), np.float32(0.0159)),
           "o": (_random_packed(I, 8192, 8192, 2), np.float32(0.0159)),
           "gu": (_random_packed(I, 28672, 8192, 3), np.float32(0.0159)),
           "down": (_random_packed(I, 8192, 28672, 4), np.float32(0.0159))}
    assert shapes["down"] == (28672, 8192) and shapes["gate"] == (8192, 28672)
    pre = []
    for i, (nm, k, n) in enumerate(I.LAYER_2B):
        pre.append(O.quantize_weights(I.master_weights(n, k, I.weight_seed(0, i))))
    xs = {k: I.activations(prefill_m, k) for k in {k for _, k, _ in I.LAYER_2B}}
    _ORACLE = {"decode": (dec, I.activations(1, 8192)), "prefill": (pre, xs)}
    nbytes, mats_done, el = _oracle_decode(seconds)
    res = {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{mats_done} matrices of the 100B-class layer (8192->8192, 8192->28672, "
                     f"28672->8192 in the stack's order) at M=1, act-quant + unpack + int64 "
                     f"contraction + rescale, {nbytes / 1e6:.0f} MB packed in {el:.1f} s",
           "host_cpu": _cpu_model(), "host_threads": os.cpu_count()}
    ops, el2 = _oracle_prefill(seconds)
    res["prefill"] = {"value": round(ops / el2 / 1e12, 6), "unit": "TOPS", "cores": 1,
                      "kind": "oracle",
                      "sample": f"2B-shaped layer matrices at M={prefill_m} tokens, "
                                f"{ops / 1e9:.1f} G int8 ops in {el2:.1f} s"}
    if workers > 1:
        import multiprocessing
        with multiprocessing.get_context("fork").Pool(workers) as pool:
            parts = pool.map(_oracle_decode, [seconds] * workers)
        total = sum(b for b, _, _ in parts)
        wall = max(e for _, _, e in parts)
        res["all_cores"] = {"value": round(total / wall / 1e9, 4), "unit": "GB/s", "cores": workers,
                            "sample": f"{sum(n for _, n, _ in parts)} matrices over {workers} "
                                      f"processes, {wall:.1f} s"}
    _ORACLE = None
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
        cpu = cpu_baseline(I, args.cpu_seconds, workers)
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
        "tokens_per_s": round(1e3 / d["ms"], 1),
        "decode_sustained": None,   # filled in last
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(workload=args.workload),
                     "kernel": "gemv_kernel (decode, fused int8 activation quantisation)",
                     "avg_launch_us": round(avg_launch * 1e6, 3),
                     "avg_bytes_per_launch": int(avg_bytes),
                     "launch_time": "graph replay time / launches in the timed steps (HIP "
                                    "events on the kernels' stream)"},
    }
    two_b = "bitnet2b-decode-m1-30L"
    if not args.no_2b:
        d2 = decode_leg(torch, N, I, two_b, args.steps, args.warmup)
        result["decode_2b"] = dict(workload=two_b, **leg_summary(d2, 1),
                                   traffic_per_launch=recorded_traffic(
                                       "gemv_bitnet2b_decode_chain.md", two_b))
    if not args.no_extra:
        if not args.no_2b:
            df = decode_leg(torch, N, I, two_b, args.steps, args.warmup, full_layer=True)
            result["decode_2b_full_layer"] = dict(
                workload=two_b + " with RMS norms and squared-ReLU gating fused in",
                **leg_summary(df, 1))
        if args.workload == "ternary100b-decode-m1-96L":
            b16 = args.workload + "-bf16"
            d16 = decode_leg(torch, N, I, b16, max(10, args.steps // 2), 5)
            result["decode_100b_bf16"] = dict(
                workload=b16 + " (bf16 activations between layers)", **leg_summary(d16, 1))
        for m in (1, 16):
            d8 = decode_leg(torch, N, I, "llama8b-ternary", max(5, args.steps // 3), 2, m=m)
            result[f"decode_8b_m{m}"] = dict(workload="llama8b-ternary (32 layers)",
                                             **leg_summary(d8, m))
    if not args.no_chain:
        dc = chain_leg(torch, N, I, args.workload, max(5, args.steps // 5), 2)
        result["decode_chain"] = dict(
            workload=args.workload + ", one cooperative launch per token (decode chain)",
            **leg_summary(dc, 1))
        if not args.no_2b:
            dc2 = chain_leg(torch, N, I, two_b, args.steps, args.warmup)
            result["decode_2b_chain"] = dict(
                workload=two_b + ", one cooperative launch per token (decode chain)",
                **leg_summary(dc2, 1))
    if not args.no_t1:
        dt = decode_leg(torch, N, I, args.workload, max(5, args.steps // 5), 2, fmt="t1")
        result["decode_t1"] = dict(workload=args.workload + ", weights five per byte (T1 layout)",
                                   **leg_summary(dt, 1))
        if not args.no_2b:
            dt2 = decode_leg(torch, N, I, two_b, args.steps, args.warmup, fmt="t1")
            result["decode_2b_t1"] = dict(workload=two_b + ", weights five per byte (T1 layout)",
                                          **leg_summary(dt2, 1))
    if not args.no_quant:
        result["quantisers"] = quantisers(torch, N, I, steps=3)
    if not args.no_compare:
        result["hbm_read_ceiling"] = hbm_read_ceiling(torch)
        result["launch_gap"] = launch_gap(torch)
        result["kernel_compare_m1"] = kernel_compare(
            torch, N, I, ((2560, 2560), (2560, 6912), (6912, 2560), (8192, 28672), (28672, 8192)),
            steps=4)
    if not args.no_prefill:
        result["mfma_ceiling"] = mfma_ceiling(torch)
        result["prefill"] = prefill(torch, N, I, I.LAYER_2B, (512, 4096), steps=10)
        result["prefill_8b"] = prefill(torch, N, I, I.LAYER_8B, (2048,), steps=5)
        log(f"prefill: {result['prefill']} {result['prefill_8b']}")
    if args.sustain_seconds > 0:
        # last, so that the continuous load does not warm the chip for the other legs
        ds = decode_leg(torch, N, I, args.workload, 3, 2, sustain_s=args.sustain_seconds)
        result["decode_sustained"] = ds["sustained"]
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
