"""Five-weights-per-byte layout (reading T1) on the HIP path vs the oracle,
through the C ABI: packing from master weights and from the 2-bit layout, the
decode kernel on T1 weights, and the fused act-quant (with the layer prologue).

Bar: packed bytes, gamma*, int8 activations and int32 accumulators bit-exact;
fp32/bf16 outputs bit-exact under the rescale order, with and without the
layer prologue.
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, acts, bf16_bits, dev, f32_bits, host, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


@pytest.mark.parametrize("n,k,dt", [(37, 80, "f32"), (5, 1, "f32"), (64, 100, "bf16"),
                                    (130, 6912, "bf16"), (33, 2560, "f32"), (7, 333, "f32"),
                                    (300, 4096, "f32")])
def test_quantize_weights_t1(n, k, dt):
    wt, w = weights(n, k, 900 + n + k, dt)
    p, g = N.bitnet_quantize_weights_t1(wt)
    want_p, want_g = O.quantize_weights_t1(w)
    assert host(g)[0].view(np.uint32) == np.float32(want_g).view(np.uint32)
    np.testing.assert_array_equal(host(p), want_p)


@pytest.mark.parametrize("n,k", [(19, 160), (3, 100), (64, 36), (257, 6912), (40, 4)])
def test_repack_t1(n, k):
    w = I.master_weights(n, k, 950 + n)
    p2, _ = O.quantize_weights(w)
    got = host(N.bitnet_repack_t1(dev(p2)))
    np.testing.assert_array_equal(got, O.pack_t1(O.unpack_codes(p2)))


def _t1_mats(ns, k, seed):
    return [O.quantize_weights_t1(I.master_weights(n, k, seed + i)) for i, n in enumerate(ns)]


def _check_outputs(mats, ys, accs, xq, d, k, ydt):
    for (p, g), y, acc in zip(mats, ys, accs):
        acc_w, y_w = O.ternary_linear_t1(p, g, xq, d)
        np.testing.assert_array_equal(host(acc), acc_w)
        if ydt == "bf16":
            np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_w))
        else:
            np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


# decode kernel on T1 weights: single and grouped matrices (5 = two launches),
# ragged N, K with and without a partial last block, M up to 16 and beyond
# (groups of 16 tokens), a multi-phase staging case (M = 16, K = 6912)
@pytest.mark.parametrize("m,k,ns,ydt", [
    (1, 80, (16,), "f32"), (1, 16, (5,), "f32"), (1, 2560, (2560, 640, 640), "f32"),
    (1, 6912, (2560,), "bf16"), (3, 96, (33, 17), "f32"), (4, 1296, (100,), "bf16"),
    (16, 6912, (130, 48), "f32"), (17, 512, (64,), "f32"), (40, 160, (7, 9, 11, 13, 15), "f32"),
    (2, 28672, (70,), "f32")])
def test_ternary_linear_t1(m, k, ns, ydt):
    mats = _t1_mats(ns, k, 1100 + m + k)
    xt, x = acts(m, k, 1200 + k, "f32")
    xq, d = O.quantize_acts(x)
    ytd = torch.bfloat16 if ydt == "bf16" else torch.float32
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for n in ns]
    dm = [(dev(p), dev(np.array([g], np.float32)), None, a) for (p, g), a in zip(mats, accs)]
    ys = N.bitnet_ternary_linear_t1(dm, dev(xq), dev(d), y_dtype=ytd)
    _check_outputs(mats, ys, accs, xq, d, k, ydt)


# act-quant fused into the T1 decode launch (M <= 4) or separate (M = 5, and a
# K too large for one phase at M = 4), with and without the layer prologue
@pytest.mark.parametrize("m,k,ns,dt,glu,norm", [
    (1, 2560, (2560, 640, 640), "bf16", False, False), (1, 6912, (2560,), "bf16", True, True),
    (2, 2560, (6912, 6912), "f32", False, True), (3, 100 * 16, (48,), "f32", True, False),
    (5, 256, (64, 33), "bf16", True, True), (4, 28672, (40,), "f32", False, False),
    # three input groups per thread at M = 1: two held, the third read again
    (1, 8192, (48, 20), "f32", False, False), (1, 8192, (33,), "bf16", False, False)])
def test_quant_linear_t1(m, k, ns, dt, glu, norm):
    mats = _t1_mats(ns, k, 1300 + m + k)
    xt, x = acts(m, k, 1400 + k, dt)
    ut, u = acts(m, k, 1401 + k, dt) if glu else (None, None)
    w = I.norm_weight(k, 1402 + k) if norm else None
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for n in ns]
    dm = [(dev(p), dev(np.array([g], np.float32)), None, a) for (p, g), a in zip(mats, accs)]
    ys, xq, xs = N.bitnet_quant_linear_t1(dm, xt, up=ut, norm_weight=None if w is None else dev(w),
                                          eps=1e-5)
    want_q, want_d = O.prologue_quantize_acts(x, up=u, norm_weight=w, eps=1e-5)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))
    _check_outputs(mats, ys, accs, want_q, want_d, k, "f32")


def test_t1_matches_two_bit_path_on_the_same_weights():
    """The same ternary matrices through both layouts give identical integers."""
    k, ns = 6912, (2560, 130)
    p2 = [O.quantize_weights(I.master_weights(n, k, 1500 + i)) for i, n in enumerate(ns)]
    xt, x = acts(1, k, 1501, "bf16")
    d2 = [(dev(p), dev(np.array([g], np.float32)), None,
           torch.empty((1, n), dtype=torch.int32, device=DEV)) for (p, g), n in zip(p2, ns)]
    d5 = [(N.bitnet_repack_t1(t[0]), t[1], None,
           torch.empty((1, n), dtype=torch.int32, device=DEV)) for t, n in zip(d2, ns)]
    y2, _, _ = N.bitnet_quant_linear_multi(d2, xt)
    y5, _, _ = N.bitnet_quant_linear_t1(d5, xt)
    for a, b, u, v in zip(d2, d5, y2, y5):
        np.testing.assert_array_equal(host(a[3]), host(b[3]))
        np.testing.assert_array_equal(f32_bits(host(u)), f32_bits(host(v)))
