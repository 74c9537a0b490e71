"""Lookup-table contraction (reading L1) on the HIP path vs the oracle's table
method, through the C ABI.  Integer throughout: accumulators and outputs are
bit-exact (and equal to the matrix-core path on the same inputs)."""

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


# ragged N (row blocks of 64), K from one chunk to splits of several sizes, M up
# to 3 tokens, bf16 outputs
@pytest.mark.parametrize("m,n,k,ydt", [
    (1, 64, 64, "f32"), (1, 100, 2560, "f32"), (3, 257, 6912, "bf16"), (1, 2560, 2560, "f32"),
    (2, 130, 28672, "f32"), (1, 8192, 8192, "bf16"), (1, 1, 192, "f32")])
def test_ternary_linear_lut(m, n, k, ydt):
    p, g = O.quantize_weights(I.master_weights(n, k, 1600 + n))
    xq, d = O.quantize_acts(I.activations(m, k, 1601 + k))
    ytd = torch.bfloat16 if ydt == "bf16" else torch.float32
    acc = torch.empty((m, n), dtype=torch.int32, device=DEV)
    y = N.bitnet_ternary_linear_lut(dev(p), dev(np.array([g], np.float32)), dev(xq), dev(d),
                                    y_dtype=ytd, acc_out=acc)
    acc_w, y_w = O.lut_linear(p, g, xq, d)
    np.testing.assert_array_equal(host(acc), acc_w)
    if ydt == "bf16":
        np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(y_w))
    else:
        np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(y_w))


def test_lut_equals_matrix_core_path_and_reuses_workspace():
    """Same integers as the decode kernel; a workspace reused across calls of
    different shapes needs no clearing by the caller."""
    ws = torch.empty(N.lib().bitnet_lut_workspace_bytes(6912, 6912), dtype=torch.uint8, device=DEV)
    for n, k in ((6912, 2560), (2560, 6912), (640, 2560)):
        p, g = O.quantize_weights(I.master_weights(n, k, 1700 + n))
        xq, d = O.quantize_acts(I.activations(1, k, 1701))
        pd, gd, xd, dd = dev(p), dev(np.array([g], np.float32)), dev(xq), dev(d)
        a1 = torch.empty((1, n), dtype=torch.int32, device=DEV)
        a2 = torch.empty((1, n), dtype=torch.int32, device=DEV)
        y1 = N.bitnet_ternary_linear_lut(pd, gd, xd, dd, acc_out=a1, workspace=ws)
        y2 = N.bitnet_ternary_linear(pd, gd, xd, dd, acc_out=a2)
        np.testing.assert_array_equal(host(a1), host(a2))
        np.testing.assert_array_equal(f32_bits(host(y1)), f32_bits(host(y2)))
