"""Decode launches whose matrices' tiles are split as one list in balanced runs
(a workgroup's run may cross from one matrix into the next), vs the oracle,
element by element, through the C ABI.

The library takes balanced runs only where splitting each matrix on its own
would leave more workgroups than the compute units hold two at a time; the
shapes here (K = 1024, over 6 MB of packed weights, so the launch spreads its
tiles two workgroups per compute unit) are chosen so that this happens on a
256-CU device: with 3 tiles per run, the per-matrix split needs 513 workgroups
and the list split 511 or 512.  They cover three and four matrices (a fourth
matrix's pointer comes from the argument block), runs of equal length (rt = 0)
and of two lengths, rows that are not a multiple of 16, the int8-input kernel
at M = 1 and 16, and the fused quantisation (fp32 and bf16 input, with and
without the RMS-norm and gating prologue).  Bar: bit-exact.
"""

import math

import numpy as np
import pytest
import torch

from oracle import bitnet_oracle as O
from ternary_weight_linear_bit_amd import _native as N
from ternary_weight_linear_bit_amd import inputs as I

from gpu_helpers import DEV, acts, bf16_bits, dev, f32_bits, host

pytestmark = pytest.mark.gpu
K = 1024
EPS = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


def _split(ns, k, cus):
    """(per-matrix workgroups, list workgroups, slots) of a bandwidth-regime
    decode launch: runs of t tiles, t from two workgroups per compute unit."""
    tiles = [(n + 15) // 16 for n in ns]
    total = sum(tiles)
    assert total * 16 * (k // 4) > 6_000_000
    t = math.ceil(total / (2 * cus))
    return sum(math.ceil(x / t) for x in tiles), math.ceil(total / t), 2 * cus, min(tiles) >= t


def _require_balanced(ns):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    per_matrix, listed, slots, fits = _split(ns, K, cus)
    if not (per_matrix > slots >= listed and fits):
        pytest.skip(f"shape does not take balanced runs on {cus} compute units")


def _mats(ns, seed):
    return [O.quantize_weights(I.master_weights(n, K, seed + i)) for i, n in enumerate(ns)]


SHAPES = [(8192, 8192, 8192), (6629, 10561, 7300), (5782, 7106, 11617),
          (7009, 7330, 8066, 2080), (4135, 6198, 10291, 3842)]


@pytest.mark.parametrize("ns", SHAPES)
@pytest.mark.parametrize("m", [1, 16])
def test_balanced_runs_int8_input(ns, m):
    _require_balanced(ns)
    mats = _mats(ns, 1300 + m)
    xq, d = O.quantize_acts(I.activations(m, K, 1310 + m))
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for n in ns]
    dm = [(dev(p), dev(np.array([g], np.float32)), None, a) for (p, g), a in zip(mats, accs)]
    ys = N.bitnet_ternary_linear_multi(dm, dev(xq), dev(d))
    for (p, g), y, acc in zip(mats, ys, accs):
        acc_w, y_w = O.ternary_linear(p, g, xq, d)
        np.testing.assert_array_equal(host(acc), acc_w)
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


@pytest.mark.parametrize("ns,m,dt,glu,norm", [
    ((8192, 8192, 8192), 1, "f32", False, False),
    ((5782, 7106, 11617), 4, "bf16", False, False),
    ((4135, 6198, 10291, 3842), 1, "f32", False, True),
    ((7009, 7330, 8066, 2080), 2, "bf16", True, True)])
def test_balanced_runs_fused(ns, m, dt, glu, norm):
    _require_balanced(ns)
    mats = _mats(ns, 1400 + m)
    xt, x = acts(m, K, 1410 + m, dt)
    ut, u = acts(m, K, 1411 + m, dt) if glu else (None, None)
    w = I.norm_weight(K, 1412 + m) if norm else None
    dm = [(dev(p), dev(np.array([g], np.float32))) for p, g in mats]
    ys, xq, xs = N.bitnet_quant_linear_multi(dm, xt, up=ut, norm_weight=dev(w) if norm else None,
                                             eps=EPS, y_dtype=torch.bfloat16)
    want_q, want_d = O.prologue_quantize_acts(x, up=u, norm_weight=w, eps=EPS)
    np.testing.assert_array_equal(host(xq), want_q)
    np.testing.assert_array_equal(f32_bits(host(xs)), f32_bits(want_d))
    for (p, g), y in zip(mats, ys):
        _, y_w = O.ternary_linear(p, g, want_q, want_d)
        np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_w))
