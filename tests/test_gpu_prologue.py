"""The layer's input prologue (squared-ReLU gating, RMS norm) on the HIP path vs
the oracle (readings N1-N3), through the C ABI.

Bar: bit-exact everywhere (int8 codes, token scales, int32 accumulators and
the outputs).  With a norm the mean of squares is the exactly rounded one on
both sides; the rows built below put it on a rounding midpoint, just above one,
and at the extremes of the exponent range, so that the GPU's exact path (taken
when its float64 sum cannot decide the rounding) is exercised and decides the
codes.
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, acts, dev, f32_bits, host
from golden_util import norm_example_arrays

pytestmark = pytest.mark.gpu
EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


def _inputs(m, k, seed, dt, glu, norm):
    xt, x = acts(m, k, seed, dt)
    ut, u = acts(m, k, seed + 1, dt) if glu else (None, None)
    w = I.norm_weight(k, seed + 2) if norm else None
    return xt, x, ut, u, (dev(w) if norm else None), w


def _check_scale(got, want, norm=True):
    np.testing.assert_array_equal(f32_bits(got), f32_bits(want))


@pytest.mark.parametrize("m,k,dt,glu,norm", [
    (1, 2560, "bf16", True, True), (1, 6912, "bf16", True, True), (3, 100, "f32", True, True),
    (4, 1024, "f32", False, True), (2, 512, "bf16", True, False), (7, 4096, "bf16", True, True),
    (2, 28672, "f32", False, True), (5, 20, "f32", True, False)])
def test_quantize_acts_prologue(m, k, dt, glu, norm):
    xt, x, ut, u, wt, w = _inputs(m, k, 500 + m + k, dt, glu, norm)
    xq, xs = N.bitnet_quantize_acts(xt, up=ut, norm_weight=wt, eps=EPS)
    want_q, want_d = O.prologue_quantize_acts(x, up=u, norm_weight=w, eps=EPS)
    np.testing.assert_array_equal(host(xq), want_q)
    _check_scale(host(xs), want_d, norm)


# fused into the decode kernel (M <= 4), and the separate quantisation followed
# by the decode (M = 5) or prefill (M = 40) kernel
@pytest.mark.parametrize("m,k,ns,dt,glu,norm", [
    (1, 2560, (2560, 640, 640), "bf16", False, True),
    (1, 6912, (2560,), "bf16", True, True),
    (1, 2560, (6912, 6912), "f32", False, True),
    (2, 512, (100, 37), "bf16", True, False),
    (3, 1024, (48,), "f32", True, True),
    (1, 28672, (130,), "f32", True, True),
    (5, 256, (64, 33), "bf16", True, True),
    (40, 512, (100,), "f32", True, True)])
def test_quant_linear_prologue(m, k, ns, dt, glu, norm):
    xt, x, ut, u, wt, w = _inputs(m, k, 600 + m + k, dt, glu, norm)
    mats = [O.quantize_weights(I.master_weights(n, k, 610 + i)) for i, n in enumerate(ns)]
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for n in ns]
    dm = [(dev(p), dev(np.array([g], np.float32)), None, a) for (p, g), a in zip(mats, accs)]
    ys, xq, xs = N.bitnet_quant_linear_multi(dm, xt, up=ut, norm_weight=wt, eps=EPS)
    want_q, want_d = O.prologue_quantize_acts(x, up=u, norm_weight=w, eps=EPS)
    np.testing.assert_array_equal(host(xq), want_q)
    _check_scale(host(xs), want_d, norm)
    for (p, g), y, acc in zip(mats, ys, accs):
        acc_w, y_w = O.ternary_linear(p, g, want_q, want_d)
        np.testing.assert_array_equal(host(acc), acc_w)
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


def test_full_layer_chain():
    """Two BitNet-2B-shaped layers at M = 1 with the neighbours fused in: an RMS
    norm in front of q/k/v and of gate/up, the sub-layer norm in front of o, and
    squared-ReLU gating plus the sub-layer norm in front of down (o consumes q:
    attention is out of scope).  Activations stay fp32 between layers, so every
    step is compared bit for bit."""
    k_model = 2560
    layers = []
    for l in range(2):
        mats = {nm: O.quantize_weights(I.master_weights(n, k, I.weight_seed(l, i)))
                for i, (nm, k, n) in enumerate(I.LAYER_2B)}
        norms = {"in": I.norm_weight(2560, 50 + 4 * l), "attn_sub": I.norm_weight(2560, 51 + 4 * l),
                 "ffn_in": I.norm_weight(2560, 52 + 4 * l), "ffn_sub": I.norm_weight(6912, 53 + 4 * l)}
        layers.append((mats, norms))
    h = I.activations(1, k_model, 7)
    hd = dev(h)
    ref = h
    for mats, norms in layers:
        dm = {nm: (dev(p), dev(np.array([g], np.float32))) for nm, (p, g) in mats.items()}
        dn = {nm: dev(v) for nm, v in norms.items()}
        # GPU
        (q, _, _), xq1, xs1 = N.bitnet_quant_linear_multi([dm["q"], dm["k"], dm["v"]], hd,
                                                          norm_weight=dn["in"], eps=EPS)
        (o,), xq2, xs2 = N.bitnet_quant_linear_multi([dm["o"]], q, norm_weight=dn["attn_sub"],
                                                     eps=EPS)
        (gate, up), xq3, xs3 = N.bitnet_quant_linear_multi([dm["gate"], dm["up"]], o,
                                                           norm_weight=dn["ffn_in"], eps=EPS)
        (hd,), xq4, xs4 = N.bitnet_quant_linear_multi([dm["down"]], gate, up=up,
                                                      norm_weight=dn["ffn_sub"], eps=EPS)
        # oracle, fed with the GPU's fp32 layer outputs so that each step is
        # compared on identical inputs
        steps = [(ref, None, norms["in"], ["q"], xq1, xs1),
                 (host(q), None, norms["attn_sub"], ["o"], xq2, xs2),
                 (host(o), None, norms["ffn_in"], ["gate", "up"], xq3, xs3),
                 (host(gate), host(up), norms["ffn_sub"], ["down"], xq4, xs4)]
        outs = {"q": q, "o": o, "gate": gate, "up": up, "down": hd}
        for x_in, u_in, w, names, xq_g, xs_g in steps:
            want_q, want_d = O.prologue_quantize_acts(x_in, up=u_in, norm_weight=w, eps=EPS)
            np.testing.assert_array_equal(host(xq_g), want_q)
            _check_scale(host(xs_g), want_d, True)
            for nm in names:
                _, y_w = O.ternary_linear(*mats[nm], want_q, want_d)
                np.testing.assert_array_equal(f32_bits(host(outs[nm])), f32_bits(y_w))
        ref = host(hd)


# --- rows whose mean of squares the float64 sum cannot round -----------------
#
# v0 = 1 + t 2^-12 (t odd, t < 2^11) and v2 = 1/4 in a row of K = 2^j inputs,
# the rest 0: v0^2 + v2^2 = 1 + 2^-4 + t 2^-11 + t^2 2^-24 needs one bit more
# than fp32 holds in [1, 2), so the exact mean lies on a rounding midpoint (ties
# to even).  (v2 keeps the largest normalised value away from sqrt(K), which it
# would equal, whatever the rounding of r, for a single non-zero input.)  Adding
# v1 = 2^-40 puts the exact mean 2^-80 / K above the midpoint, which a float64
# sum loses.  Scaled by 2^60 the mean stays a midpoint near 2^114; scaled by
# 2^-66 it is sub-normal (below 2^-132 / K).

def _row(k, pos, t, kind):
    v = np.zeros(k, np.float32)
    v[pos] = np.float32(1 + t * 2.0 ** -12)
    v[(pos + 2) % k] = np.float32(0.25)
    if kind == "above":
        v[(pos + 1) % k] = np.float32(2.0 ** -40)
    elif kind == "big":
        v *= np.float32(2.0 ** 60)
    elif kind == "tiny":
        v *= np.float32(2.0 ** -66)
    return v


def _sensitive_t(k, pos):
    """An odd t whose midpoint row and just-above row get different token scales
    from the oracle (eps = 0): the exact rounding of the mean decides the output."""
    for t in range(1, 2048, 2):
        rows = np.stack([_row(k, pos, t, "mid"), _row(k, pos, t, "above")])
        _, d = O.prologue_quantize_acts(rows, norm_weight=np.ones(k, np.float32), eps=0.0)
        if d[0] != d[1]:
            return t
    raise AssertionError("no sensitive t")


def _exact_path_inputs(m, k, pos, kinds, seed):
    t = _sensitive_t(k, pos)
    rows = [_row(k, pos, t, kinds[i % len(kinds)]) for i in range(m)]
    v = np.stack(rows).astype(np.float32)
    w = np.ones(k, np.float32)
    w[pos] = np.float32(1.25)   # the norm weight scales the surviving value
    return v, w


@pytest.mark.parametrize("m,k,pos,kinds,glu", [
    (4, 64, 5, ("mid", "above", "big", "tiny"), False),
    (4, 64, 63, ("above", "mid", "tiny", "big"), True),
    (1, 32768, 30001, ("mid",), False),
    (1, 32768, 30001, ("above",), True),
    (1, 32768, 7, ("tiny",), False),
    (2, 8192, 8000, ("above", "big"), False),
    (3, 4096, 1000, ("big", "above", "mid"), True),
    (6, 64, 0, ("mid", "above", "big", "tiny"), False),
    (5, 32768, 30001, ("above", "mid", "tiny"), False)])
def test_norm_exact_mean_path(m, k, pos, kinds, glu):
    """Codes, scales and outputs bit-exact on rows whose mean of squares needs the
    exact path: through the standalone quantisation, and fused into the decode
    kernel (M <= 4) or the separate quantisation in front of the decode (M > 4).
    With gating the gate is 1 and the up projection carries the row, so the gated
    input is the row itself."""
    v, w = _exact_path_inputs(m, k, pos, kinds, 700 + m + k)
    x, u = (np.ones_like(v), v) if glu else (v, None)
    want_q, want_d = O.prologue_quantize_acts(x, up=u, norm_weight=w, eps=0.0)
    xt, ut, wt = dev(x), (dev(u) if glu else None), dev(w)
    xq, xs = N.bitnet_quantize_acts(xt, up=ut, norm_weight=wt, eps=0.0)
    np.testing.assert_array_equal(host(xq), want_q)
    _check_scale(host(xs), want_d)
    p, g = O.quantize_weights(I.master_weights(48, k, 710 + m))
    acc = torch.empty((m, 48), dtype=torch.int32, device=DEV)
    (y,), xq2, xs2 = N.bitnet_quant_linear_multi([(dev(p), dev(np.array([g], np.float32)), None, acc)],
                                                 xt, up=ut, norm_weight=wt, eps=0.0)
    np.testing.assert_array_equal(host(xq2), want_q)
    _check_scale(host(xs2), want_d)
    acc_w, y_w = O.ternary_linear(p, g, want_q, want_d)
    np.testing.assert_array_equal(host(acc), acc_w)
    np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


def test_norm_golden_example_on_gpu(golden):
    """The hand-worked normalise-then-quantise example: codes and token scale equal
    the values worked out by hand, on the standalone and the fused path."""
    for ex in golden["norm_examples"]:
        v, w = norm_example_arrays(ex)
        want = np.zeros((1, ex["K"]), np.int8)
        for i, q in ex["xq_entries"]:
            want[0, i] = q
        xt, wt = dev(v), dev(w)
        xq, xs = N.bitnet_quantize_acts(xt, norm_weight=wt, eps=ex["eps"])
        np.testing.assert_array_equal(host(xq), want)
        assert f32_bits(host(xs))[0] == int(ex["d_bits"], 16)
        p, g = O.quantize_weights(I.master_weights(32, ex["K"], 720))
        acc = torch.empty((1, 32), dtype=torch.int32, device=DEV)
        _, xq2, xs2 = N.bitnet_quant_linear_multi([(dev(p), dev(np.array([g], np.float32)), None, acc)],
                                                  xt, norm_weight=wt, eps=ex["eps"])
        np.testing.assert_array_equal(host(xq2), want)
        assert f32_bits(host(xs2))[0] == int(ex["d_bits"], 16)
        np.testing.assert_array_equal(host(acc), O.ternary_linear(p, g, want, host(xs2))[0])
