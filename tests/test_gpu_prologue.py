"""The layer's input prologue (squared-ReLU gating, RMS norm) on the HIP path vs
the oracle (readings N1-N3), through the C ABI.

Bar: the int8 activations and the int32 accumulators are bit-exact.  The token
scale with a norm carries the factor r, whose mean of squares the GPU sums in
float64 (the oracle exactly): it is compared to 4e-7 relative (two fp32 ulps),
and so are the fp32 outputs that use it; without a norm everything is bit-exact.
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, acts, dev, f32_bits, host

pytestmark = pytest.mark.gpu
EPS = 1e-5
SCALE_RTOL = 4e-7


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


def _check_scale(got, want, norm):
    if norm:
        assert np.all(np.abs(got / want - 1.0) <= SCALE_RTOL), (got, want)
    else:
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
        got = host(y)
        if norm:
            np.testing.assert_allclose(got, y_w, rtol=2 * SCALE_RTOL, atol=0)
        else:
            np.testing.assert_array_equal(f32_bits(got), f32_bits(y_w))


def test_full_layer_chain():
    """Two BitNet-2B-shaped layers at M = 1 with the neighbours fused in: an RMS
    norm in front of q/k/v and of gate/up, the sub-layer norm in front of o, and
    squared-ReLU gating plus the sub-layer norm in front of down (o consumes q:
    attention is out of scope).  Activations stay fp32 between layers, so every
    step is compared: int8 codes exactly, scales and outputs to 2 ulps."""
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
                np.testing.assert_allclose(host(outs[nm]), y_w, rtol=2 * SCALE_RTOL, atol=0)
        ref = host(hd)
