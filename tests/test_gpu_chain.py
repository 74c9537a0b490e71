"""The decode chain (every stage of a token in one launch) against the oracle run
stage by stage, and against the per-launch path, through the C ABI.

Bar: bit-exact x_q, token scales, int32 accumulators and fp32 / bf16 outputs of
every stage (the chain runs the same arithmetic as bitnet_quant_linear_multi).
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


def _as_f32(t):
    """An output tensor as the fp32 values the next stage reads (bf16 upcast exactly)."""
    return host(t.float()) if t.dtype == torch.bfloat16 else host(t)


def _make_matrix(n, k, seed):
    w = I.master_weights(n, k, seed)
    p, g = N.bitnet_quantize_weights(dev(w))
    return p, g, O.quantize_weights(w)


def _run_and_check(m, spec, x0_dtype, seed0):
    """spec: list of stages; each stage = (input: 'x0' or (stage, matrix), K,
    [(N, y_dtype, with_acc)]).  Builds the chain, runs it twice, and checks every
    stage against the oracle applied to the GPU's own stage inputs (the oracle
    chain itself is checked stage by stage, so a mismatch names its stage)."""
    k0 = spec[0][1]
    x0 = I.activations(m, k0, seed0)
    x0_t = dev(x0).to(x0_dtype)
    stages, outs, oracle_mats = [], [], []
    for si, (src, k, mats) in enumerate(spec):
        x = x0_t if src == "x0" else outs[src[0]][src[1]][0]
        assert x.shape == (m, k)
        row, omats = [], []
        for mi, (n, ydt, with_acc) in enumerate(mats):
            p, g, (want_p, want_g) = _make_matrix(n, k, 5000 + 10 * si + mi)
            y = torch.empty((m, n), dtype=ydt, device=DEV)
            acc = torch.empty((m, n), dtype=torch.int32, device=DEV) if with_acc else None
            row.append((y, acc, p, g))
            omats.append((want_p, want_g))
        outs.append(row)
        oracle_mats.append(omats)
        stages.append(dict(x=x, x_q=torch.empty((m, k), dtype=torch.int8, device=DEV),
                           x_scale=torch.empty(m, dtype=torch.float32, device=DEV),
                           mats=[(p, g, y, acc) for (y, acc, p, g) in row]))
    chain = N.bitnet_chain_plan(stages, m)
    for rep in range(2):
        for row in outs:
            for y, acc, _, _ in row:
                y.fill_(float("nan"))
                if acc is not None:
                    acc.fill_(-7)
        N.bitnet_chain_run(chain)
        torch.cuda.synchronize()
        assert N.bitnet_chain_error(chain) == 0
        for si, st in enumerate(stages):
            x_in = _as_f32(st["x"])
            want_q, want_d = O.quantize_acts(x_in)
            np.testing.assert_array_equal(host(st["x_q"]), want_q, f"stage {si} x_q")
            np.testing.assert_array_equal(f32_bits(host(st["x_scale"])), f32_bits(want_d),
                                          f"stage {si} x_scale")
            for mi, ((y, acc, _, _), (want_p, want_g)) in enumerate(zip(outs[si], oracle_mats[si])):
                want_acc, want_y = O.ternary_linear(want_p, want_g, want_q, want_d)
                tag = f"stage {si} matrix {mi} run {rep}"
                if acc is not None:
                    np.testing.assert_array_equal(host(acc), want_acc, tag)
                if y.dtype == torch.bfloat16:
                    np.testing.assert_array_equal(bf16_bits(y), O.f32_to_bf16_bits(want_y), tag)
                else:
                    np.testing.assert_array_equal(f32_bits(host(y)), f32_bits(want_y), tag)
    return chain


F32, BF16 = torch.float32, torch.bfloat16


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_chain_small_stack_bit_exact(m):
    spec = [
        ("x0", 256, [(320, F32, True), (64, F32, False)]),
        ((0, 0), 320, [(192, BF16, True)]),
        ((1, 0), 192, [(256, F32, False), (130, F32, True), (17, F32, False)]),
        ((2, 0), 256, [(256, F32, True), (64, F32, True), (64, F32, True), (48, F32, True)]),
        ((3, 1), 64, [(100, F32, True)]),    # input: matrix 1 of stage 3 (64 wide)
    ]
    _run_and_check(m, spec, F32, 31 + m)


def test_chain_bf16_input_long_k_and_many_tiles():
    spec = [
        ("x0", 2560, [(2560, BF16, True), (640, BF16, False), (640, BF16, False)]),
        ((0, 0), 2560, [(2560, BF16, True)]),
        ((1, 0), 2560, [(6912, BF16, False), (6912, BF16, True)]),
        ((2, 1), 6912, [(2560, BF16, True)]),
    ]
    _run_and_check(1, spec, BF16, 41)


def test_chain_equals_per_launch_path_100b_layer():
    """One 100B-class layer (8192 / 28672, fp32 between stages) through the chain and
    through bitnet_quant_linear_multi launches: identical bits everywhere."""
    shapes = {nm: (k, n) for nm, k, n in I.LAYER_100B}
    mats = {}
    for i, (nm, (k, n)) in enumerate(shapes.items()):
        g = torch.Generator(device=DEV).manual_seed(I.weight_seed(0, i))
        w = torch.randn((n, k), generator=g, device=DEV).mul_(I.WEIGHT_SIGMA)
        mats[nm] = N.bitnet_quantize_weights(w)
        del w
    h = torch.randn((1, 8192), generator=torch.Generator(device=DEV).manual_seed(7), device=DEV)

    def bufs():
        b = {nm: torch.empty((1, n), device=DEV) for nm, (k, n) in shapes.items()}
        for tag, k in (("h", 8192), ("q", 8192), ("o", 8192), ("u", 28672)):
            b["xq_" + tag] = torch.empty((1, k), dtype=torch.int8, device=DEV)
            b["xs_" + tag] = torch.empty((1,), dtype=torch.float32, device=DEV)
        return b
    a, c = bufs(), bufs()
    N.bitnet_quant_linear_multi([(*mats["q"], a["q"]), (*mats["k"], a["k"]), (*mats["v"], a["v"])],
                                h, x_q=a["xq_h"], x_scale=a["xs_h"])
    N.bitnet_quant_linear_multi([(*mats["o"], a["o"])], a["q"], x_q=a["xq_q"], x_scale=a["xs_q"])
    N.bitnet_quant_linear_multi([(*mats["gate"], a["gate"]), (*mats["up"], a["up"])], a["o"],
                                x_q=a["xq_o"], x_scale=a["xs_o"])
    N.bitnet_quant_linear_multi([(*mats["down"], a["down"])], a["up"], x_q=a["xq_u"],
                                x_scale=a["xs_u"])
    stages = [
        dict(x=h, x_q=c["xq_h"], x_scale=c["xs_h"],
             mats=[(*mats["q"], c["q"]), (*mats["k"], c["k"]), (*mats["v"], c["v"])]),
        dict(x=c["q"], x_q=c["xq_q"], x_scale=c["xs_q"], mats=[(*mats["o"], c["o"])]),
        dict(x=c["o"], x_q=c["xq_o"], x_scale=c["xs_o"],
             mats=[(*mats["gate"], c["gate"]), (*mats["up"], c["up"])]),
        dict(x=c["up"], x_q=c["xq_u"], x_scale=c["xs_u"], mats=[(*mats["down"], c["down"])]),
    ]
    chain = N.bitnet_chain_plan(stages, 1)
    N.bitnet_chain_run(chain)
    torch.cuda.synchronize()
    assert N.bitnet_chain_error(chain) == 0
    for key in a:
        if a[key].dtype == torch.int8:
            np.testing.assert_array_equal(host(c[key]), host(a[key]), key)
        else:
            np.testing.assert_array_equal(f32_bits(host(c[key])), f32_bits(host(a[key])), key)
