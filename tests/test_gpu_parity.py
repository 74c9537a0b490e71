"""HIP path vs the CPU oracle, element by element, through the C ABI.

Bar: bit-exact packed bytes, gamma*, int8 activations, token scales and int32
accumulators; fp32 outputs bit-exact as well (the rescale order is fixed, so no
tolerance is needed; the contract floor would be 1e-6 relative) and bf16 outputs
bit-exact (floor: 1 ulp).  Shapes span several tiles of every kernel and ragged
tails in M, N and K.
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from golden_util import f32_from_hex, golden_arrays, hex_bits
from gpu_helpers import DEV, acts, bf16_bits, dev, f32_bits, host, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


def check_linear(packed, gamma, xq, d, m, n, k, y_dtype=torch.float32, x_q_dev=None):
    acc_want, y_want = O.ternary_linear(packed, gamma, xq, d)
    acc = torch.empty((m, n), dtype=torch.int32, device=DEV)
    xq_d = dev(xq) if x_q_dev is None else x_q_dev
    y = N.bitnet_ternary_linear(dev(packed), dev(np.array([gamma], np.float32)), xq_d, dev(d),
                                y_dtype=y_dtype, acc_out=acc)
    np.testing.assert_array_equal(host(acc), acc_want)
    if y_dtype == torch.float32:
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_want))
    else:
        np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_want))


# ---------------------------------------------------------------------------
# weight quantisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,k,dt,seed", [
    (256, 256, "f32", 1), (37, 100, "f32", 2), (64, 2560, "bf16", 3), (1, 4, "f32", 4),
    (999, 64, "f32", 5), (16, 4100, "bf16", 6), (300, 1028, "f32", 7)])
def test_quantize_weights_bit_exact(n, k, dt, seed):
    wt, w_or = weights(n, k, seed, dt)
    packed, scale = N.bitnet_quantize_weights(wt)
    want_p, want_g = O.quantize_weights(w_or)
    assert f32_bits(host(scale))[0] == f32_bits(want_g)
    np.testing.assert_array_equal(host(packed), want_p)


def test_quantize_weights_wide_exponents_and_subnormals():
    """Exact mean over magnitudes 2^-149 .. 2^100: an order-dependent float sum
    would differ from the oracle here."""
    rng = np.random.Generator(np.random.PCG64(40))
    w = (rng.standard_normal((128, 512)) * np.exp2(rng.integers(-140, 100, (128, 512)))).astype(np.float32)
    w[0, :8] = np.array([1e-45, -1e-45, 3e-42, 0.0, -0.0, 1e-38, 2.0 ** -126, 1e30], np.float32)
    packed, scale = N.bitnet_quantize_weights(dev(w))
    want_p, want_g = O.quantize_weights(w)
    assert f32_bits(host(scale))[0] == f32_bits(want_g)
    np.testing.assert_array_equal(host(packed), want_p)


def test_quantize_weights_degenerate():
    packed, scale = N.bitnet_quantize_weights(torch.zeros((8, 64), device=DEV))
    assert f32_bits(host(scale))[0] == f32_bits(np.float32(1e-5))
    assert np.all(host(packed) == 0x55)
    for bad in (np.nan, np.inf, -np.inf):
        w = I.master_weights(16, 64, 9)
        w[3, 7] = bad
        _, scale = N.bitnet_quantize_weights(dev(w))
        assert np.isnan(host(scale)[0])


def test_quantize_weights_unaligned_buffers():
    """Weights at a 4-byte (not 16-byte) offset and packed output at an odd byte
    offset take the scalar paths; results must not change."""
    n, k = 33, 96
    w = I.master_weights(n, k, 11)
    base = torch.zeros(n * k + 1, dtype=torch.float32, device=DEV)
    base[1:] = dev(w.reshape(-1))
    wv = base[1:].view(n, k)
    pbase = torch.zeros(n * k // 4 + 1, dtype=torch.uint8, device=DEV)
    pv = pbase[1:].view(n, k // 4)
    N.bitnet_quantize_weights(wv, packed=pv)
    want_p, _ = O.quantize_weights(w)
    np.testing.assert_array_equal(host(pv), want_p)


def test_golden_examples_on_gpu(golden):
    """The hand-worked examples through every kernel family: as given (decode kernel
    at K % 64 == 0, else the generic one), with the token tiled to 20 rows (the
    prefill kernel at K % 64 == 0), and through the fused act-quant + linear call."""
    for ex in golden["examples"]:
        w, x, _, want_xq = golden_arrays(ex)
        want_gamma = (f32_from_hex(ex["gamma_bits"]) if "gamma_bits" in ex
                      else np.float32(ex["gamma"]))
        packed, scale = N.bitnet_quantize_weights(dev(w))
        np.testing.assert_array_equal(host(packed), np.array(ex["packed"], np.uint8))
        assert f32_bits(host(scale))[0] == f32_bits(want_gamma), ex["name"]
        want_acc = np.array(ex["acc"], np.int32)
        want_y = hex_bits(ex["y_bits"])
        want_b = hex_bits(ex["y_bf16_bits"], np.uint16)
        want_d = np.array([int(h, 16) for h in ex["d_bits"]], np.uint32)
        for rep in (1, 20):
            xt = np.tile(x, (rep, 1))
            xq, xs = N.bitnet_quantize_acts(dev(xt))
            np.testing.assert_array_equal(host(xq), np.tile(want_xq, (rep, 1)))
            np.testing.assert_array_equal(f32_bits(host(xs)), np.tile(want_d, rep))
            acc = torch.empty((xt.shape[0], w.shape[0]), dtype=torch.int32, device=DEV)
            y = N.bitnet_ternary_linear(packed, scale, xq, xs, acc_out=acc)
            np.testing.assert_array_equal(host(acc), np.tile(want_acc, (rep, 1)), ex["name"])
            np.testing.assert_array_equal(f32_bits(host(y)), np.tile(want_y, (rep, 1)), ex["name"])
            yb = N.bitnet_ternary_linear(packed, scale, xq, xs, y_dtype=torch.bfloat16)
            np.testing.assert_array_equal(bf16_bits(yb), np.tile(want_b, (rep, 1)), ex["name"])
        xq, xs = (torch.empty(x.shape, dtype=torch.int8, device=DEV),
                  torch.empty(x.shape[0], dtype=torch.float32, device=DEV))
        acc = torch.empty((x.shape[0], w.shape[0]), dtype=torch.int32, device=DEV)
        y, _, _ = N.bitnet_quant_linear(packed, scale, dev(x), x_q=xq, x_scale=xs, acc_out=acc)
        np.testing.assert_array_equal(host(xq), want_xq)
        np.testing.assert_array_equal(f32_bits(host(xs)), want_d)
        np.testing.assert_array_equal(host(acc), want_acc, ex["name"])
        np.testing.assert_array_equal(f32_bits(host(y)), want_y, ex["name"])


# ---------------------------------------------------------------------------
# activation quantisation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,k,dt", [(4, 256, "f32"), (1, 2560, "bf16"), (3, 100, "f32"),
                                    (7, 6912, "bf16"), (33, 28672, "f32"), (5, 20, "bf16")])
def test_quantize_acts_bit_exact(m, k, dt):
    xt, x_or = acts(m, k, 7 + m, dt)
    xq, xs = N.bitnet_quantize_acts(xt)
    want_q, want_d = O.quantize_acts(x_or)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))


def test_quantize_acts_special_rows():
    x = np.zeros((4, 64), np.float32)
    x[1, :8] = [127.0, 2.5, -0.5, 3.5, 126.5, -1.5, 0.49, -127.0]
    x[2] = np.linspace(-3e-6, 3e-6, 64, dtype=np.float32)        # below the floor
    x[3] = np.linspace(-1e30, 1e30, 64, dtype=np.float32)
    xq, xs = N.bitnet_quantize_acts(dev(x))
    want_q, want_d = O.quantize_acts(x)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))


def test_quantize_acts_empty():
    xq, xs = N.bitnet_quantize_acts(torch.empty((0, 64), device=DEV))
    assert xq.shape == (0, 64) and xs.shape == (0,)
    xq, xs = N.bitnet_quantize_acts(torch.empty((3, 0), device=DEV))
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(O.quantize_acts(np.zeros((3, 0), np.float32))[1]))


# ---------------------------------------------------------------------------
# ternary linear: decode kernel (M <= 16), prefill kernel, generic kernel
# ---------------------------------------------------------------------------

LINEAR_SHAPES = [
    # decode kernel: several 16-row tiles, ragged N, K not a multiple of 256
    (1, 16, 64), (1, 37, 256), (1, 640, 2560), (1, 200, 320), (3, 100, 1024), (4, 256, 256),
    (16, 48, 2048), (5, 33, 6912), (2, 17, 28672), (1, 2560, 6912),
    # prefill kernel, 64 x 128 tiles (chosen when 128 x 128 tiles would not cover
    # the compute units once): ragged M and N
    (17, 100, 256), (100, 130, 2560), (300, 257, 192), (128, 128, 64), (513, 640, 512),
    (16, 50, 4096),
    # prefill kernel, 128 x 128 tiles: ragged M and N, K of one and a half steps
    (1000, 5000, 192), (900, 6000, 64),
    # prefill kernel, 128 x 256 tiles (chosen when they fill 80-100% of one round
    # of the chip's compute units): ragged M and N
    (2000, 4000, 64), (1920, 3900, 192), (700, 9000, 64),
    # prefill kernel, 256 x 256 tiles (chosen when they fill at least 80% of the
    # compute units over the launch's rounds): ragged M and N, K of one half step
    (2000, 6600, 64), (1100, 10400, 192),
    # decode kernel: several K phases, multi-tile workgroups, M = 16 at large K
    (16, 100, 14336), (1, 40, 28672), (3, 24, 65536), (1, 20, 131072), (2, 9000, 256),
    (1, 70000, 64), (16, 300, 1088),
    # decode kernel, bandwidth regime with two tiles per workgroup and two K phases
    # at M = 16, the second phase one 256-k super-chunk long (three of the four
    # waves have no loads in it): the weight ring runs on across tiles and phases
    (16, 9000, 4352),
]


@pytest.mark.parametrize("m,n,k", LINEAR_SHAPES)
def test_ternary_linear_bit_exact(m, n, k):
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 100 + n))
    xq, d = O.quantize_acts(I.activations(m, k, 200 + m))
    check_linear(packed, gamma, xq, d, m, n, k)


@pytest.mark.parametrize("m,n,k", [(1, 640, 2560), (300, 257, 192), (1000, 5000, 192),
                                   (2000, 4000, 64), (2000, 6600, 64)])
def test_ternary_linear_bf16_output(m, n, k):
    """bf16 output from the decode kernel and from each prefill tile shape (64 x 128,
    128 x 128, 128 x 256, 256 x 256)."""
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 300 + n))
    xq, d = O.quantize_acts(I.activations(m, k, 400 + m))
    check_linear(packed, gamma, xq, d, m, n, k, y_dtype=torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [(3, 40, 100), (1, 9, 4), (20, 31, 196)])
def test_ternary_linear_generic_k(m, n, k):
    """K % 64 != 0 takes the generic kernel."""
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 500 + k))
    xq, d = O.quantize_acts(I.activations(m, k, 600 + k))
    check_linear(packed, gamma, xq, d, m, n, k)


def test_ternary_linear_unaligned_activations():
    m, n, k = 3, 40, 256
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 12))
    xq, d = O.quantize_acts(I.activations(m, k, 13))
    base = torch.zeros(m * k + 1, dtype=torch.int8, device=DEV)
    base[1:] = dev(xq.reshape(-1))
    check_linear(packed, gamma, xq, d, m, n, k, x_q_dev=base[1:].view(m, k))


def test_extreme_activations_and_k_zero():
    """All activations at -128 / 127 and all weights +-1: the largest accumulators."""
    m, n, k = 2, 32, 4096
    q = np.ones((n, k), np.int8)
    q[1::2] = -1
    q[5, ::3] = 0
    packed = O.pack_codes(q)
    xq = np.full((m, k), 127, np.int8)
    xq[1] = -128
    d = np.array([0.5, 2.0 ** -20], np.float32)
    check_linear(packed, np.float32(0.013), xq, d, m, n, k)
    check_linear(packed, np.float32(0.013), np.repeat(xq, 20, axis=0),
                 np.repeat(d, 20), 40, n, k)
    y = N.bitnet_ternary_linear(torch.empty((4, 0), dtype=torch.uint8, device=DEV),
                                dev(np.array([1.0], np.float32)),
                                torch.empty((3, 0), dtype=torch.int8, device=DEV),
                                dev(np.ones(3, np.float32)))
    np.testing.assert_array_equal(host(y), np.zeros((3, 4), np.float32))


def test_decode_and_prefill_kernels_agree():
    n, k = 96, 2048
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 14))
    xq, d = O.quantize_acts(I.activations(40, k, 15))
    args = (dev(packed), dev(np.array([gamma], np.float32)))
    a16 = torch.empty((16, n), dtype=torch.int32, device=DEV)
    a40 = torch.empty((40, n), dtype=torch.int32, device=DEV)
    N.bitnet_ternary_linear(*args, dev(xq[:16]), dev(d[:16]), acc_out=a16)
    N.bitnet_ternary_linear(*args, dev(xq), dev(d), acc_out=a40)
    np.testing.assert_array_equal(host(a16), host(a40)[:16])


def test_end_to_end_gpu_quantisers():
    """GPU weight and activation quantisers feeding the GPU layer."""
    m, n, k = 4, 256, 2560
    wt, w_or = weights(n, k, 16, "bf16")
    xt, x_or = acts(m, k, 17, "bf16")
    packed, scale = N.bitnet_quantize_weights(wt)
    xq, xs = N.bitnet_quantize_acts(xt)
    y = N.bitnet_ternary_linear(packed, scale, xq, xs)
    want_p, want_g = O.quantize_weights(w_or)
    _, _, _, y_want = O.quant_linear(want_p, want_g, x_or)
    np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_want))


# ---------------------------------------------------------------------------
# activation quantisation fused into the layer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,n,k,dt", [(1, 2560, 2560, "bf16"), (1, 640, 6912, "f32"),
                                      (2, 100, 256, "f32"), (4, 48, 1024, "bf16"),
                                      (5, 64, 512, "f32"), (1, 20, 100, "f32"),
                                      (1, 130, 28672, "f32"), (300, 64, 256, "bf16"),
                                      (3, 50, 12288, "bf16"), (2, 70, 8192, "f32")])
def test_quant_linear_fused(m, n, k, dt):
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 700 + n))
    xt, x_or = acts(m, k, 800 + m, dt)
    acc = torch.empty((m, n), dtype=torch.int32, device=DEV)
    y, xq, xs = N.bitnet_quant_linear(dev(packed), dev(np.array([gamma], np.float32)), xt,
                                      acc_out=acc)
    want_q, want_d, want_acc, want_y = O.quant_linear(packed, gamma, x_or)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))
    np.testing.assert_array_equal(host(acc), want_acc)
    np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(want_y))


def test_chain_of_layers_fused():
    """Two 2B-shaped layers at M = 1 chained on the GPU without host round trips,
    against the oracle chain (reading: o consumes q, gate/up consume o, down
    consumes up; activations between layers are bf16)."""
    shapes = {nm: (k, n) for nm, k, n in I.LAYER_2B}
    layers = []
    for l in range(2):
        mats = {}
        for i, (nm, k, n) in enumerate(I.LAYER_2B):
            w = I.master_weights(n, k, I.weight_seed(l, i))
            mats[nm] = O.quantize_weights(w)
        layers.append(mats)
    h = I.to_bf16(I.activations(1, 2560, 7))
    # GPU
    hd = h.to(DEV)
    for mats in layers:
        dm = {nm: (dev(p), dev(np.array([g], np.float32))) for nm, (p, g) in mats.items()}
        q, xq, xs = N.bitnet_quant_linear(*dm["q"], hd, y_dtype=torch.bfloat16)
        N.bitnet_ternary_linear(*dm["k"], xq, xs, y_dtype=torch.bfloat16)
        N.bitnet_ternary_linear(*dm["v"], xq, xs, y_dtype=torch.bfloat16)
        o, _, _ = N.bitnet_quant_linear(*dm["o"], q, y_dtype=torch.bfloat16)
        _, xq2, xs2 = N.bitnet_quant_linear(*dm["gate"], o, y_dtype=torch.bfloat16)
        u = N.bitnet_ternary_linear(*dm["up"], xq2, xs2, y_dtype=torch.bfloat16)
        hd, _, _ = N.bitnet_quant_linear(*dm["down"], u, y_dtype=torch.bfloat16)
    got = bf16_bits(hd)
    # oracle
    hx = h.float().numpy()
    for mats in layers:
        def lin(nm, x):
            _, _, _, y = O.quant_linear(*mats[nm], x)
            return O.bf16_bits_to_f32(O.f32_to_bf16_bits(y))
        q = lin("q", hx)
        o = lin("o", q)
        u = lin("up", o)
        hx = lin("down", u)
    np.testing.assert_array_equal(got, O.f32_to_bf16_bits(hx))
    assert shapes["down"] == (6912, 2560)


def test_repeatable_and_stream_ordered():
    m, n, k = 1, 4096, 8192
    packed, gamma = O.quantize_weights(I.master_weights(n, k, 18))
    xq, d = O.quantize_acts(I.activations(m, k, 19))
    args = (dev(packed), dev(np.array([gamma], np.float32)), dev(xq), dev(d))
    y1 = host(N.bitnet_ternary_linear(*args))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y2 = N.bitnet_ternary_linear(*args)
    s.synchronize()
    np.testing.assert_array_equal(f32_bits(y1), f32_bits(y2.cpu().numpy()))
    _, want = O.ternary_linear(packed, gamma, xq, d)
    np.testing.assert_array_equal(f32_bits(y1), f32_bits(want))


def _group(ns, k, seed):
    # an empty matrix (N = 0) has no weights to take a scale from: any gamma will do
    return [O.quantize_weights(I.master_weights(n, k, seed + i)) if n else
            (np.zeros((0, k // 4), np.uint8), np.float32(1.0)) for i, n in enumerate(ns)]


@pytest.mark.parametrize("m,k,ns", [(1, 2560, (2560, 640, 640)), (5, 256, (100, 37, 16, 64, 200)),
                                    (16, 1024, (48, 33)), (40, 512, (100, 130, 17)),
                                    (1, 64, (30000, 20000, 7)),
                                    (300, 256, (100, 37, 260, 5, 129)), (129, 128, (0, 300, 64)),
                                    (2000, 64, (1990, 2000)), (800, 64, (9000, 4100, 300))])
def test_ternary_linear_multi(m, k, ns):
    """Grouped matrices sharing x_q, including more than 4 (split into launches),
    an empty matrix, and M beyond the decode kernel (up to four matrices per
    prefill launch; 2000 x (1990, 2000) selects the 128 x 256 tiles and
    800 x (9000, 4100, 300) the 256 x 256 tiles)."""
    mats = _group(ns, k, 900)
    xq, d = O.quantize_acts(I.activations(m, k, 901))
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for n in ns]
    dm = [(dev(p), dev(np.array([g], np.float32)), None, a) for (p, g), a in zip(mats, accs)]
    ys = N.bitnet_ternary_linear_multi(dm, dev(xq), dev(d))
    for (p, g), y, acc in zip(mats, ys, accs):
        acc_w, y_w = O.ternary_linear(p, g, xq, d)
        np.testing.assert_array_equal(host(acc), acc_w)
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


@pytest.mark.parametrize("m,k,ns,dt", [(1, 2560, (2560, 640, 640), "bf16"),
                                       (1, 2560, (6912, 6912), "bf16"),
                                       (3, 512, (100, 37, 16, 64, 200), "f32"),
                                       (1, 28672, (40, 24), "f32"), (8, 256, (16, 20), "f32"),
                                       (1, 10240, (40, 24), "f32"), (1, 12288, (17,), "bf16"),
                                       (600, 256, (300, 100, 700), "bf16")])
def test_quant_linear_multi(m, k, ns, dt):
    mats = _group(ns, k, 950)
    xt, x_or = acts(m, k, 951, dt)
    dm = [(dev(p), dev(np.array([g], np.float32))) for p, g in mats]
    ys, xq, xs = N.bitnet_quant_linear_multi(dm, xt, y_dtype=torch.bfloat16)
    want_q, want_d = O.quantize_acts(x_or)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))
    for (p, g), y in zip(mats, ys):
        _, y_w = O.ternary_linear(p, g, want_q, want_d)
        np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_w))
