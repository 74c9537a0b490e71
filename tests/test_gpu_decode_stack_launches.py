"""Decode launches of the bench's stacks at M <= 4 through the fused act-quant call
(the decode path the bench times), every output compared with the oracle.

The four launches of a 100B-class layer, q+k+v (3 x 8192 -> 8192), o (8192 ->
8192), gate+up (2 x 8192 -> 28672) and down (28672 -> 8192), take the
bandwidth-regime plans with several 16-row tiles per workgroup (list runs); the
8B-class down projection (14336 -> 4096, 256 tiles) and a ragged 12800 -> 3000
(188 tiles) take eight-wave workgroups of one tile each, and the 8B-class q+k+v
(4096 -> 4096 + 1024 + 1024, 384 tiles) one tile in each of 384 four-wave
workgroups, the second workgroup on a compute unit staging at a raised priority.  Each launch has its own
seeded input, bf16 and fp32 inputs; the small parity shapes reach none of these
plans.  Weights are seeded
ternary codes packed by the oracle (ternarising 235 M master weights on the host
would take minutes; the weight quantiser is checked at these sizes in
test_gpu_full_size.py).  Bar: bit-exact x_q, token scales and outputs.  The
contraction is the sum over +1 weights minus the sum over -1 weights
(dashen-tech.com, "BitNet.cpp 深度解析", section 3.1); the activations are quantised
per token (communeify.com page on BitNet b1.58 2B4T, quantisation details).
"""

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, acts, bf16_bits, dev, f32_bits, host

pytestmark = pytest.mark.gpu

GAMMA = np.float32(0.0159)
LAUNCHES = {"qkv": (8192, (8192, 8192, 8192)), "o": (8192, (8192,)),
            "gate+up": (8192, (28672, 28672)), "down": (28672, (8192,)),
            "8B down": (14336, (4096,)), "ragged": (12800, (3000,)),
            "8B qkv": (4096, (4096, 1024, 1024))}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


@pytest.fixture(scope="module")
def weights():
    """Packed codes per launch (host and device), generated once for the module."""
    out = {}
    for li, (name, (k, ns)) in enumerate(LAUNCHES.items()):
        out[name] = [O.pack_codes(I.ternary_codes(n, k, 9100 + 10 * li + j)) for j, n in enumerate(ns)]
    return out


@pytest.mark.parametrize("dt,m", [("bf16", 1), ("f32", 1), ("bf16", 3)])
@pytest.mark.parametrize("name", list(LAUNCHES))
def test_100b_launch_every_output(weights, name, dt, m):
    k, ns = LAUNCHES[name]
    print(f"decode launch {name}: K={k} N={ns} M={m} input {dt}", flush=True)
    xt, x = acts(m, k, 9200 + m + k, dt)
    g_d = dev(np.array([GAMMA], np.float32))
    mats = [(dev(p), g_d) for p in weights[name]]
    ydt = torch.bfloat16 if dt == "bf16" else torch.float32
    ys, xq, xs = N.bitnet_quant_linear_multi(mats, xt, y_dtype=ydt)
    want_q, want_d = O.quantize_acts(x)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))
    for j, (p, y) in enumerate(zip(weights[name], ys)):
        _, y_w = O.ternary_linear(p, GAMMA, want_q, want_d)
        if dt == "bf16":
            np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_w), f"matrix {j}")
        else:
            np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w), f"matrix {j}")
