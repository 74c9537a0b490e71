"""Decode launches whose matrices' tiles are split as one list ("list runs": a
workgroup's run may cross from one matrix into the next), vs the oracle,
element by element, through the C ABI.

The library takes list runs in two cases of a launch spread two workgroups per
compute unit (over 6 MB of packed weights; K = 1024 here): when the tiles come
to S = total / CUs per compute unit with S >= 5, the workgroups dispatched first
(b < CUs) take S / 2 + 1 tiles and the others the rest (skewed runs; fused 2-bit
launches with an even S on a 256-CU device take S / 2 each instead, the second
workgroup of each compute unit staging its input at a raised priority); else, when
splitting each matrix on its own would leave more workgroups than the compute
units hold two at a time, runs of equal length to within one tile (with 3
tiles per run, 513 per-matrix workgroups against 511 or 512).  The shapes cover
both on a 256-CU device: one to four matrices (a fourth matrix's pointer comes
from the argument block), S = 6, 7 and 14, rows that are not a multiple of 16,
the int8-input kernel at M = 1 and 16, and the fused quantisation (fp32 and
bf16 input, with and without the RMS-norm and gating prologue).  Bar:
bit-exact.
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


def _list_runs(ns, k, cus):
    """Whether a bandwidth-regime decode launch of these matrices takes list
    runs: 'skewed' (S = total / cus >= 5 tiles per compute unit, every matrix at
    least S // 2 + 1 tiles), 'balanced' (per-matrix runs of t tiles would need
    more than 2 * cus workgroups, the list fewer), else None."""
    tiles = [(n + 15) // 16 for n in ns]
    total = sum(tiles)
    assert total * 16 * (k // 4) > 6_000_000
    if total % cus == 0 and total // cus >= 5 and min(tiles) >= total // cus // 2 + 1:
        return "skewed"
    t = math.ceil(total / (2 * cus))
    per_matrix = sum(math.ceil(x / t) for x in tiles)
    if len(ns) > 1 and per_matrix > 2 * cus >= math.ceil(total / t) and min(tiles) >= t:
        return "balanced"
    return None


def _require_list_runs(ns, kind):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if _list_runs(ns, K, cus) != kind:
        pytest.skip(f"shape does not take {kind} list runs on {cus} compute units")


def _mats(ns, seed):
    return [O.quantize_weights(I.master_weights(n, K, seed + i)) for i, n in enumerate(ns)]


SHAPES = [((8192, 8192, 8192), "skewed"), ((28657,), "skewed"), ((18705, 9937), "skewed"),
          ((8145, 18641, 30513), "skewed"), ((13121, 7681, 1873, 1841), "skewed"),
          ((6629, 10561, 7300), "balanced"), ((5782, 7106, 11617), "balanced"),
          ((7009, 7330, 8066, 2080), "balanced"), ((4135, 6198, 10291, 3842), "balanced")]


@pytest.mark.parametrize("ns,kind", SHAPES)
@pytest.mark.parametrize("m", [1, 16])
def test_list_runs_int8_input(ns, kind, m):
    _require_list_runs(ns, kind)
    mats = _mats(ns, 1300 + m)
    xq, d = O.quantize_acts(I.activations(m, K, 1310 + m))
    accs = [torch.empty((m, n), dtype=torch.int32, device=DEV) for n in ns]
    dm = [(dev(p), dev(np.array([g], np.float32)), None, a) for (p, g), a in zip(mats, accs)]
    ys = N.bitnet_ternary_linear_multi(dm, dev(xq), dev(d))
    for (p, g), y, acc in zip(mats, ys, accs):
        acc_w, y_w = O.ternary_linear(p, g, xq, d)
        np.testing.assert_array_equal(host(acc), acc_w)
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


@pytest.mark.parametrize("ns,kind,m,dt,glu,norm", [
    ((8192, 8192, 8192), "skewed", 1, "f32", False, False),
    ((8145, 18641, 30513), "skewed", 3, "bf16", True, False),
    ((13121, 7681, 1873, 1841), "skewed", 1, "f32", False, True),
    ((5782, 7106, 11617), "balanced", 4, "bf16", False, False),
    ((4135, 6198, 10291, 3842), "balanced", 1, "f32", False, True),
    ((7009, 7330, 8066, 2080), "balanced", 2, "bf16", True, True)])
def test_list_runs_fused(ns, kind, m, dt, glu, norm):
    _require_list_runs(ns, kind)
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
