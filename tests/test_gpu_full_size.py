"""Parity at the full benchmark shapes, through the same calls the bench times.

For every distinct (K, N) of the 2B-, 8B- and 100B-shaped layer sets: gamma* and
the packed bytes of the whole matrix (bit-exact), and the accumulators
and outputs at sampled (token, row) pairs plus one full output row, at the token
counts of each configuration (decode M = 1 / 16, prefill M = 512 / 2048 / 4096).
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, bf16_bits, f32_bits, host

pytestmark = pytest.mark.gpu

# (K, N, token counts) -- every distinct matrix shape of the configurations
FULL = [
    (2560, 2560, (1, 512, 4096)), (2560, 640, (1, 4096)), (2560, 6912, (1, 512, 4096)),
    (6912, 2560, (1, 4096)),
    (4096, 4096, (1, 16, 2048)), (4096, 1024, (1, 16)), (4096, 14336, (1, 16, 2048)),
    (14336, 4096, (1, 16, 2048)),
    (8192, 8192, (1,)), (8192, 28672, (1,)), (28672, 8192, (1,)),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


@pytest.mark.parametrize("k,n,ms", FULL, ids=[f"{k}x{n}" for k, n, _ in FULL])
def test_full_size(k, n, ms):
    print(f"full-size K={k} N={n} M={ms}", flush=True)
    seed = I.weight_seed(0, (k * 7 + n) % 7)
    w = I.master_weights(n, k, seed)
    w_d = torch.from_numpy(w).to(DEV)
    packed_d, scale_d = N.bitnet_quantize_weights(w_d)
    gamma = O.weight_scale(w)
    assert f32_bits(host(scale_d))[0] == f32_bits(gamma)
    rng = np.random.Generator(np.random.PCG64(k + n))
    packed_o = O.pack_codes(O.ternarize(w, gamma))
    del w, w_d
    np.testing.assert_array_equal(host(packed_d), packed_o)
    for m in ms:
        x = I.activations(m, k, I.ACT_SEED + m)
        xq_d, xs_d = N.bitnet_quantize_acts(torch.from_numpy(x).to(DEV))
        xq, d = O.quantize_acts(x)
        np.testing.assert_array_equal(host(xq_d), xq)
        np.testing.assert_array_equal(f32_bits(host(xs_d)), f32_bits(d))
        acc_d = torch.empty((m, n), dtype=torch.int32, device=DEV)
        y_d = N.bitnet_ternary_linear(packed_d, scale_d, xq_d, xs_d, acc_out=acc_d)
        acc_h, y_h = host(acc_d), host(y_d)
        mi = np.concatenate([rng.integers(0, m, 256), np.zeros(n, np.int64)])
        ni = np.concatenate([rng.integers(0, n, 256), np.arange(n)])
        acc_w, y_w = O.ternary_linear_at(packed_o, gamma, xq, d, mi, ni)
        np.testing.assert_array_equal(acc_h[mi, ni], acc_w)
        np.testing.assert_array_equal(f32_bits(y_h[mi, ni]), f32_bits(y_w))
    del packed_d
    torch.cuda.empty_cache()


# The T1 layout (five weights per byte) at the decode shapes of the bench's T1 legs,
# through the fused act-quant call the bench times (2B: bf16 input; 100B: fp32)
FULL_T1 = [(2560, 2560, "bf16"), (2560, 6912, "bf16"), (6912, 2560, "bf16"),
           (8192, 8192, "f32"), (8192, 28672, "f32"), (28672, 8192, "f32")]


@pytest.mark.parametrize("k,n,dt", FULL_T1, ids=[f"t1-{k}x{n}" for k, n, _ in FULL_T1])
def test_full_size_t1(k, n, dt):
    print(f"full-size T1 K={k} N={n}", flush=True)
    w = I.master_weights(n, k, I.weight_seed(1, (k * 7 + n) % 7))
    p_d, s_d = N.bitnet_quantize_weights_t1(torch.from_numpy(w).to(DEV))
    p_o, gamma = O.quantize_weights_t1(w)
    del w
    assert f32_bits(host(s_d))[0] == f32_bits(gamma)
    np.testing.assert_array_equal(host(p_d), p_o)
    x = I.activations(1, k, I.ACT_SEED + 1)
    if dt == "bf16":
        xt = I.to_bf16(x).to(DEV)
        x = xt.float().cpu().numpy()
    else:
        xt = torch.from_numpy(x).to(DEV)
    acc_d = torch.empty((1, n), dtype=torch.int32, device=DEV)
    (y_d,), xq_d, xs_d = N.bitnet_quant_linear_t1([(p_d, s_d, None, acc_d)], xt)
    xq, d = O.quantize_acts(x)
    np.testing.assert_array_equal(host(xq_d), xq)
    np.testing.assert_array_equal(f32_bits(host(xs_d)), f32_bits(d))
    ni = np.arange(n)
    acc_w, y_w = O.ternary_linear_t1_at(p_o, gamma, xq, d, np.zeros(n, np.int64), ni)
    np.testing.assert_array_equal(host(acc_d)[0], acc_w)
    np.testing.assert_array_equal(f32_bits(host(y_d)[0]), f32_bits(y_w))
    del p_d
    torch.cuda.empty_cache()


def test_full_size_gate_up_grouped():
    """Gate and up of the 2B layer at M = 4096 in one grouped prefill launch: 864
    tiles of 256 x 256 leave a last round under 40% full, so the launch splits at
    token 3584 into 256 x 256 tiles and a second launch for the last 512 tokens.
    Sampled outputs on both sides of the split (and the tokens at it), plus one
    full output row of each matrix."""
    k, n, m = 2560, 6912, 4096
    print(f"full-size grouped gate+up K={k} N={n} x 2 M={m}", flush=True)
    mats, mats_d = [], []
    for j in range(2):
        w = I.master_weights(n, k, I.weight_seed(0, 4 + j))
        p_d, s_d = N.bitnet_quantize_weights(torch.from_numpy(w).to(DEV))
        gamma = O.weight_scale(w)
        assert f32_bits(host(s_d))[0] == f32_bits(gamma)
        mats.append((O.pack_codes(O.ternarize(w, gamma)), gamma))
        mats_d.append((p_d, s_d))
        del w
    x = I.activations(m, k, I.ACT_SEED + 7)
    xq_d, xs_d = N.bitnet_quantize_acts(torch.from_numpy(x).to(DEV))
    xq, d = O.quantize_acts(x)
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for _ in range(2)]
    ys = N.bitnet_ternary_linear_multi([(p, s, None, a) for (p, s), a in zip(mats_d, accs)],
                                       xq_d, xs_d, y_dtype=torch.bfloat16)
    rng = np.random.Generator(np.random.PCG64(4096))
    edge = np.array([0, 255, 3583, 3584, 3585, 3839, 3840, 4095])
    for (packed_o, gamma), acc_d, y_d in zip(mats, accs, ys):
        acc_h, y_b = host(acc_d), bf16_bits(y_d)
        mi = np.concatenate([rng.integers(0, m, 256), np.repeat(edge, 32), np.full(n, 3584)])
        ni = np.concatenate([rng.integers(0, n, 256), rng.integers(0, n, 32 * len(edge)),
                             np.arange(n)])
        acc_w, y_w = O.ternary_linear_at(packed_o, gamma, xq, d, mi, ni)
        np.testing.assert_array_equal(acc_h[mi, ni], acc_w)
        np.testing.assert_array_equal(y_b[mi, ni], O.f32_to_bf16_bits(y_w))
    del mats_d, accs, ys
    torch.cuda.empty_cache()
