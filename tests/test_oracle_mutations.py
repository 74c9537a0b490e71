"""Planted mistakes in the oracle must fail its external pins.

Each case swaps one oracle step for a plausible wrong reading of the pages (a
different rounding order or formula that agrees with the chosen one on easy
inputs) and checks that the hand-worked examples in tests/golden/ reject it.
The mistakes live only inside this test (monkeypatch, CPU); nothing here calls
the HIP library.
"""

import numpy as np
import pytest

from oracle import bitnet_oracle as O

import test_oracle_pins as P

F32 = np.float32


def _acts_d_reciprocal(x):
    xq, d = ORIG_ACTS(x)
    a = np.maximum(np.abs(np.asarray(x, np.float32)).max(axis=1), O.EPS)
    return xq, (F32(1.0) / (O.QB / a).astype(np.float32)).astype(np.float32)


def _acts_d_times_inverse(x):
    xq, d = ORIG_ACTS(x)
    a = np.maximum(np.abs(np.asarray(x, np.float32)).max(axis=1), O.EPS)
    return xq, (a * (F32(1.0) / O.QB)).astype(np.float32)


def _dequant_acc_gamma_first(acc, gamma, d):
    a = (np.asarray(acc, np.int32).astype(np.float32) * F32(gamma)).astype(np.float32)
    return (a * np.asarray(d, np.float32)[:, None]).astype(np.float32)


def _dequant_acc_d_first(acc, gamma, d):
    a = (np.asarray(acc, np.int32).astype(np.float32) * np.asarray(d, np.float32)[:, None])
    return (a.astype(np.float32) * F32(gamma)).astype(np.float32)


def _ternarize_reciprocal(w, gamma):
    t = (np.asarray(w, np.float32) * (F32(1.0) / F32(gamma))).astype(np.float32)
    return np.clip(np.rint(t), -1.0, 1.0).astype(np.int8)


def _prologue_fused_order(x, up=None, norm_weight=None, eps=1e-5):
    v = np.asarray(x, np.float32)
    if up is not None:
        v = O.relu2_glu(v, up)
    if norm_weight is None:
        return O.quantize_acts(v)
    xq, d = O.quantize_acts((v * np.asarray(norm_weight, np.float32)[None, :]).astype(np.float32))
    return xq, (d * O.rms_factor(v, eps)).astype(np.float32)


def _rms_normalise_one_rounding(v, w, eps):
    r = O.rms_factor(v, eps).astype(np.float64)
    return (np.asarray(v, np.float64) * r[:, None] * np.asarray(w, np.float64)[None, :]).astype(np.float32)


ORIG_ACTS = O.quantize_acts

MUTATIONS = {
    "token scale as 1 / s": ("quantize_acts", _acts_d_reciprocal),
    "token scale as a* x RN32(1/127)": ("quantize_acts", _acts_d_times_inverse),
    "rescale RN32(RN32(acc gamma) d)": ("dequantize", _dequant_acc_gamma_first),
    "rescale RN32(RN32(acc d) gamma)": ("dequantize", _dequant_acc_d_first),
    "ternarise with a rounded reciprocal": ("ternarize", _ternarize_reciprocal),
}


NORM_MUTATIONS = {
    "norm: quantise v w and fold r into the scale": ("prologue_quantize_acts", _prologue_fused_order),
    "norm: v r w rounded once": ("rms_normalise", _rms_normalise_one_rounding),
}


@pytest.mark.parametrize("name", sorted(NORM_MUTATIONS))
def test_norm_golden_example_rejects_mutation(name, golden, monkeypatch):
    attr, fn = NORM_MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    with pytest.raises(AssertionError):
        P.test_norm_golden_example(golden)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_golden_examples_reject_mutation(name, golden, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    with pytest.raises(AssertionError):
        P.test_golden_worked_examples(golden)


def test_golden_examples_accept_the_oracle(golden):
    P.test_golden_worked_examples(golden)
