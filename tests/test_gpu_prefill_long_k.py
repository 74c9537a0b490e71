"""Prefill kernel at long K, every tile shape, every output compared.

For each of the prefill kernel's tile shapes (256 x 256, 192 x 256, 128 x 256,
128 x 128, 64 x 128 tokens x rows) and for the split launches (the tokens, or the
row tiles, that fill whole rounds of 256 x 256 tiles, then the rest with their own
tile), one shape at
K >= 2560 (at least 20 steps of 128 k, so the loads issued ahead run in their
steady state), with the tile the library picks asserted on a 256-CU MI355X, and
every int32 accumulator and fp32 output compared with the oracle.  The
dashen-tech.com page "BitNet.cpp 深度解析", section 3.1, defines the contraction
(sum over +1 weights minus sum over -1 weights).
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, acts, bf16_bits, dev, f32_bits, host

pytestmark = pytest.mark.gpu

CASES = {
    # name: (M, rows of each matrix, K, tile expected on 256 CUs, first launch tokens;
    #        with a row split: first launch rows, and the second launch's tile)
    "256x256": (4096, (4096,), 2560, (256, 256), 0),
    # one round of 256 x 256 tiles filling 75% of the compute units, taken at K >= 4096
    # (192 x 256 tiles would need a second round)
    "256x256 one round": (2048, (4096, 1024, 1024), 4096, (256, 256), 0),
    # one round of 192 x 256 tiles (210 of 256 compute units; the last token tile
    # holds 160 tokens)
    "192x256": (4000, (2560,), 2560, (192, 256), 0),
    "128x256": (512, (6912, 6912), 2560, (128, 256), 0),
    "128x128": (1280, (6912,), 2560, (128, 128), 0),
    "64x128": (512, (2560,), 6912, (64, 128), 0),
    "split": (4096, (6912, 6912), 2560, (256, 256), 3584),
    # 896 tiles of 256 x 256: three whole rounds of row tiles (the gate matrix and
    # the first 10240 rows of up), then the last 4096 rows of up in 128 x 256 tiles
    "row split": (2048, (14336, 14336), 4096, (256, 256), 0, 24576, (128, 256)),
    # the same split with ragged tokens and rows (the cut inside the second matrix)
    "row split ragged": (2000, (14000, 14336), 2560, (256, 256), 0, 24576, (128, 256)),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_long_k_every_output(name):
    m, ns, k, tile, first = CASES[name][:5]
    rows, rest_tile = CASES[name][5:] if len(CASES[name]) > 5 else (0, None)
    print(f"prefill long-K case {name}: M={m} N={ns} K={k}", flush=True)
    bm, bn, f, r = N.bitnet_prefill_tile(m, ns, k)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert (bm, bn, f, r) == (*tile, first, rows), (name, bm, bn, f, r)
        if first:
            # the rest of the tokens: a second launch with its own tile
            assert N.bitnet_prefill_tile(m - first, ns, k) == (128, 256, 0, 0)
        if rows:
            # the rest of the rows: the matrices cut at 256-row tiles taken in order
            rest, t0 = [], 0
            for n in ns:
                tj = -(-n // 256)
                if t0 + tj > rows // 256:
                    rest.append(n - (rows - 256 * t0 if t0 < rows // 256 else 0))
                t0 += tj
            assert N.bitnet_prefill_tile(m, rest, k)[:2] == rest_tile, (name, rest)
    xt, x = acts(m, k, 90 + m, "f32")
    xq_t, xs_t = N.bitnet_quantize_acts(xt)
    want_q, want_d = O.quantize_acts(x)
    np.testing.assert_array_equal(host(xq_t), want_q)
    mats, wants = [], []
    for j, n in enumerate(ns):
        w = I.master_weights(n, k, 7000 + 13 * j + m)
        p, g = N.bitnet_quantize_weights(dev(w))
        want_p, want_g = O.quantize_weights(w)
        np.testing.assert_array_equal(host(p), want_p)
        y = torch.empty((m, n), dtype=torch.float32, device=DEV)
        acc = torch.empty((m, n), dtype=torch.int32, device=DEV)
        mats.append((p, g, y, acc))
        wants.append((want_p, want_g))
    N.bitnet_ternary_linear_multi(mats, xq_t, xs_t)
    torch.cuda.synchronize()
    for j, ((p, g, y, acc), (want_p, want_g)) in enumerate(zip(mats, wants)):
        want_acc, want_y = O.ternary_linear(want_p, want_g, want_q, want_d)
        np.testing.assert_array_equal(host(acc), want_acc, f"{name} matrix {j} acc")
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(want_y), f"{name} matrix {j} y")
    if name == "split":
        # bf16 outputs through the same two launches
        p, g = mats[0][0], mats[0][1]
        yb = N.bitnet_ternary_linear(p, g, xq_t, xs_t, y_dtype=torch.bfloat16)
        _, want_y = O.ternary_linear(wants[0][0], wants[0][1], want_q, want_d)
        np.testing.assert_array_equal(bf16_bits(yb), O.f32_to_bf16_bits(want_y))
