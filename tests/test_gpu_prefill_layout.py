"""Prefill weight layout (reading P1) on the HIP path vs the oracle, through the
C ABI: the repack from the 2-bit row layout, and the prefill kernel reading it.

Bar: packed bytes, int32 accumulators and fp32 / bf16 outputs bit-exact (the
layout changes where the codes sit, not the integers; dashen-tech.com,
"BitNet.cpp 深度解析", section 3.1: sum over +1 weights minus sum over -1).
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, bf16_bits, dev, f32_bits, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


@pytest.mark.parametrize("n,k", [(1, 64), (33, 192), (64, 256), (100, 2560), (257, 6912),
                                 (2560, 2560), (31, 320)])
def test_repack_prefill_bit_exact(n, k):
    packed, _ = O.quantize_weights(I.master_weights(n, k, 3100 + n + k))
    out = N.bitnet_repack_prefill(dev(packed))
    want = O.repack_prefill(packed, k)
    np.testing.assert_array_equal(host(out).reshape(-1), want)


# (M, rows of each matrix, K): every tile shape the prefill kernel picks, ragged
# M and N, K a half step past a multiple of 128, small M (the prefill kernel runs
# for any M on this layout), a long K, several matrices per launch
CASES = [
    (1, (64,), 64), (5, (33, 100), 192), (16, (300,), 2560), (17, (100,), 256),
    (300, (257,), 192), (513, (640,), 512), (1000, (5000,), 192), (2000, (4000,), 64),
    (1920, (3900,), 320), (2000, (6600,), 64), (1100, (10400,), 192),
    (4096, (2560, 640, 640), 2560), (512, (6912, 6912), 2560), (256, (2560,), 6912),
    (4000, (2500,), 192),
]


@pytest.mark.parametrize("m,ns,k", CASES)
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_prefill_layout_linear(m, ns, k, ydt):
    print(f"prefill layout M={m} N={ns} K={k} y={ydt}", flush=True)
    xq, d = O.quantize_acts(I.activations(m, k, 3200 + m))
    mats, wants, canon = [], [], []
    ytd = torch.bfloat16 if ydt == "bf16" else torch.float32
    for j, n in enumerate(ns):
        packed, g = O.quantize_weights(I.master_weights(n, k, 3300 + 7 * j + n))
        wp = N.bitnet_repack_prefill(dev(packed))
        acc = torch.empty((m, n), dtype=torch.int32, device=DEV) if j == 0 else None
        y = torch.empty((m, n), dtype=ytd, device=DEV)
        mats.append((wp, dev(np.array([g], np.float32)), n, y, acc))
        canon.append((dev(packed), dev(np.array([g], np.float32))))
        wants.append(O.ternary_linear(packed, g, xq, d))
    xq_t, d_t = dev(xq), dev(d)
    ys = N.bitnet_ternary_linear_prefill(mats, xq_t, d_t)
    ys_canon = N.bitnet_ternary_linear_multi(canon, xq_t, d_t, y_dtype=ytd)
    for j, ((acc_w, y_w), y, yc) in enumerate(zip(wants, ys, ys_canon)):
        if j == 0:
            np.testing.assert_array_equal(host(mats[0][4]), acc_w)
        if ydt == "bf16":
            np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_w))
            np.testing.assert_array_equal(bf16_bits(y), bf16_bits(yc))
        else:
            np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))
            np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(host(yc)))


def test_prefill_layout_rejects_bad_operands():
    """K not a multiple of 64, and a misaligned x_q, are refused before any launch."""
    m, n, k = 4, 32, 192
    packed, g = O.quantize_weights(I.master_weights(n, k, 3400))
    wp = N.bitnet_repack_prefill(dev(packed))
    xq = torch.zeros((m, k + 16), dtype=torch.int8, device=DEV)
    d = torch.ones(m, dtype=torch.float32, device=DEV)
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    arr = (N.BitnetMatrix * 1)(N.BitnetMatrix(wp.data_ptr(), dev(np.array([g], np.float32)).data_ptr(),
                                              n, y.data_ptr(), 0))
    lib = N.lib()
    code = {v: c for c, v in N.STATUS.items()}
    assert lib.bitnet_ternary_linear_prefill(arr, 1, xq.data_ptr(), d.data_ptr(), m, 160, 0,
                                             None) == code["BITNET_ERR_SHAPE"]
    assert lib.bitnet_ternary_linear_prefill(arr, 1, xq.data_ptr() + 4, d.data_ptr(), m, k, 0,
                                             None) == code["BITNET_ERR_ALIGN"]
