"""The allocation-free weight quantiser against the workspace one, through the C ABI.

bitnet_quantize_weights_noalloc runs the same kernels with the library's own
per-device workspace.  Two calls in a row, the second on a smaller matrix (the
workspace keeps the first call's contents, so a missing clear would show), each
bit-exact against bitnet_quantize_weights on the same input.
"""

import numpy as np
import pytest
import torch

from ternary_weight_linear_bit_amd import _native as N

from gpu_helpers import DEV, f32_bits, host, weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    N.lib()


def test_noalloc_matches_workspace_call_twice():
    cases = [(3000, 2560, "f32", 1001), (37, 64, "bf16", 1002)]
    for n, k, dt, seed in cases:
        w, _ = weights(n, k, seed, dt)
        p0, s0 = N.bitnet_quantize_weights(w)
        p1 = torch.full((n, k // 4), 0xAA, dtype=torch.uint8, device=DEV)
        s1 = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
        N.bitnet_quantize_weights_noalloc(w, p1, s1)
        assert f32_bits(host(s1))[0] == f32_bits(host(s0))[0], (n, k, dt)
        np.testing.assert_array_equal(host(p1), host(p0))


def test_noalloc_rejects_bad_arguments():
    f = N.lib().bitnet_quantize_weights_noalloc
    w = torch.zeros((4, 8), dtype=torch.float32, device=DEV)
    p = torch.zeros((4, 2), dtype=torch.uint8, device=DEV)
    s = torch.zeros(1, dtype=torch.float32, device=DEV)
    assert f(None, 0, 4, 8, p.data_ptr(), s.data_ptr(), None) == 1
    assert f(w.data_ptr(), 0, 4, 6, p.data_ptr(), s.data_ptr(), None) == 2
    assert f(w.data_ptr(), 0, 1 << 20, 1 << 18, p.data_ptr(), s.data_ptr(), None) == 2
    assert f(w.data_ptr(), 9, 4, 8, p.data_ptr(), s.data_ptr(), None) == 3
