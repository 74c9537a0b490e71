"""Planted mistakes in the oracle must fail its external pins.

Each case swaps one oracle step for a plausible wrong reading of the pages or a
plausible slip (a different rounding order or formula that agrees with the
chosen one on easy inputs, a wrong bit order, a dropped term) and checks that
the named pin rejects it.  The mistakes live only inside this test (monkeypatch,
CPU); nothing here calls the HIP library.
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


# --- slips in every step, each with the pin that must reject it ---------------

def _ternarize_half_away(w, gamma):
    t = (np.asarray(w, np.float32) / F32(gamma)).astype(np.float32)
    return np.clip(np.sign(t) * np.floor(np.abs(t) + 0.5), -1.0, 1.0).astype(np.int8)


def _pack_msb_first(q):
    q = np.asarray(q, np.int8)
    n, k = q.shape
    codes = (q.astype(np.int16) + 1).astype(np.uint8).reshape(n, k // 4, 4)
    out = np.zeros((n, k // 4), np.uint8)
    for i in range(4):
        out |= codes[:, :, i] << np.uint8(6 - 2 * i)
    return out


def _unpack_reversed_fields(packed):
    p = np.asarray(packed, np.uint8)
    n, kb = p.shape
    codes = np.empty((n, kb, 4), np.uint8)
    for i in range(4):
        codes[:, :, i] = (p >> np.uint8(6 - 2 * i)) & np.uint8(3)
    return (codes.astype(np.int8) - 1).reshape(n, 4 * kb)


def _acts_qb_128(x):
    x = np.asarray(x, np.float32)
    a = np.maximum(np.abs(x).max(axis=1), O.EPS)
    s = (F32(128.0) / a).astype(np.float32)
    xq = np.clip(np.rint((x * s[:, None]).astype(np.float32)), -128, 127).astype(np.int8)
    return xq, (a / F32(128.0)).astype(np.float32)


def _acts_round_half_up(x):
    x = np.asarray(x, np.float32)
    a = np.maximum(np.abs(x).max(axis=1), O.EPS)
    s = (O.QB / a).astype(np.float32)
    xq = np.clip(np.floor((x * s[:, None]).astype(np.float32) + 0.5), -128, 127).astype(np.int8)
    return xq, (a / O.QB).astype(np.float32)


def _acts_per_tensor(x):
    x = np.asarray(x, np.float32)
    a = np.maximum(np.abs(x).max(), O.EPS)
    s = F32(O.QB / a)
    xq = np.clip(np.rint((x * s).astype(np.float32)), -128, 127).astype(np.int8)
    return xq, np.full(x.shape[0], F32(a / O.QB), np.float32)


def _weight_scale_fp32_sum(w):
    w = np.asarray(w, np.float32).reshape(-1)
    acc = F32(0.0)
    for v in np.abs(w):
        acc = F32(acc + v)
    g = F32(acc / F32(w.size))
    return g if g > O.EPS else O.EPS


def _abs_sum_no_subnormals(w):
    w = np.asarray(w, np.float32)
    bits = w.reshape(-1).view(np.uint32)
    keep = ((bits >> np.uint32(23)) & np.uint32(0xFF)) != 0
    return ORIG_ABS_SUM(np.where(keep, w.reshape(-1), F32(0.0)))


def _rn32_ties_away(num, den):
    got = ORIG_RN32(num, den)
    up = np.nextafter(got, F32(np.inf), dtype=np.float32)
    from fractions import Fraction
    r = Fraction(num, den)
    if abs(Fraction(float(up)) - r) == abs(r - Fraction(float(got))):
        return up
    return got


def _bf16_truncate(y):
    return (np.ascontiguousarray(y, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _matmul_sign_flipped(q, xq):
    return (-ORIG_MATMUL(q, xq).astype(np.int64)).astype(np.int32)


def _matmul_transposed_codes(q, xq):
    q = np.asarray(q)
    n, k = q.shape
    qt = q.reshape(n, k // 4, 4)[:, :, ::-1].reshape(n, k)
    return ORIG_MATMUL(qt, xq)


def _mean_sq_float64(v):
    v = np.asarray(v, np.float64)
    return (np.sum(v * v, axis=1) / v.shape[1]).astype(np.float32)


def _mean_sq_fp32(v):
    v = np.asarray(v, np.float32)
    return (np.sum(v * v, axis=1, dtype=np.float32) / F32(v.shape[1])).astype(np.float32)


def _glu_one_rounding(gate, up):
    g = np.maximum(np.asarray(gate, np.float64), 0.0)
    return (g * g * np.asarray(up, np.float64)).astype(np.float32)


def _pack_t1_digits_reversed(q):
    q = np.asarray(q, np.int8)
    n, k = q.shape
    blocks = (k + 79) // 80
    codes = np.ones((n, blocks * 80), np.int64)
    codes[:, :k] = q.astype(np.int64) + 1
    codes = codes.reshape(n, blocks, 5, 16)
    value = np.zeros((n, blocks, 16), np.int64)
    for j in range(5):
        value += codes[:, :, 4 - j, :] * 3 ** j
    return (-((-256 * value) // 243)).reshape(n, blocks * 16).astype(np.uint8)


def _lut_tables_swapped_roles(xq):
    x = np.asarray(xq, np.int64)
    idx = np.arange(16)
    q0 = (idx >> 2) - 1
    q1 = (idx & 3) - 1
    return q0[None, None, :] * x[:, 0::2, None] + q1[None, None, :] * x[:, 1::2, None]


def _pack_prefill_o3_pairs(q):
    q = np.asarray(q, np.int8)
    n, k = q.shape
    nb, sb = -(-n // 32), -(-k // 128)
    codes = np.ones((nb * 32, sb * 128), np.uint32)
    codes[:n, :k] = (q.astype(np.int16) + 1).astype(np.uint32)
    c = codes.reshape(nb, 32, sb, 2, 4, 16)
    words = np.zeros((nb, 32, sb, 2, 4), np.uint32)
    for t in range(16):
        words |= c[..., t] << np.uint32(2 * t)          # O3's order inside the dword
    return words.transpose(0, 2, 3, 1, 4).reshape(-1).astype("<u4").view(np.uint8)


ORIG_ABS_SUM = O.exact_abs_sum_units
ORIG_RN32 = O.rn32_ratio
ORIG_MATMUL = O.integer_matmul

# name -> (oracle attribute, replacement, pin(s) that must fail)
SLIPS = {
    "ternarise rounds half away from zero": ("ternarize", _ternarize_half_away,
                                             [P.test_ternarize_ties_and_clip]),
    "pack with the first weight in the top bits": ("pack_codes", _pack_msb_first,
                                                   [lambda g: P.test_golden_byte_layout(g)]),
    "unpack with the fields reversed": ("unpack_codes", _unpack_reversed_fields,
                                        [P.test_pack_roundtrip_all_valid_bytes]),
    "activations scaled to 128": ("quantize_acts", _acts_qb_128, [P.test_act_quant_invariants]),
    "activations rounded half up": ("quantize_acts", _acts_round_half_up,
                                    [P.test_act_quant_ties_and_zero_row]),
    "one activation scale per tensor": ("quantize_acts", _acts_per_tensor,
                                        [P.test_act_quant_invariants]),
    "weight scale from an fp32 running sum": ("weight_scale", _weight_scale_fp32_sum,
                                              [P.test_weight_scale_is_nearest_fp32_of_exact_mean]),
    "exact sum drops sub-normals": ("exact_abs_sum_units", _abs_sum_no_subnormals,
                                    [P.test_exact_abs_sum_equals_fraction_sum]),
    "fp32 rounding of a ratio ties away": ("rn32_ratio", _rn32_ties_away,
                                           [P.test_rn32_ratio_nearest_and_ties_to_even]),
    "bf16 by truncation": ("f32_to_bf16_bits", _bf16_truncate, [P.test_bf16_rounding_matches_torch]),
    "contraction with the sign flipped": ("integer_matmul", _matmul_sign_flipped,
                                          [lambda g: P.test_matmul_brute_force_every_ternary_row(4)]),
    "contraction pairs weights and inputs in the wrong order": (
        "integer_matmul", _matmul_transposed_codes, [P.test_matmul_equals_sum_pos_minus_sum_neg]),
    "mean of squares summed in float64": ("mean_of_squares", _mean_sq_float64,
                                          [P.test_norm_mean_of_squares_just_above_a_midpoint]),
    "mean of squares summed in fp32": ("mean_of_squares", _mean_sq_fp32,
                                       [P.test_norm_mean_of_squares_just_above_a_midpoint]),
    "gating rounded once": ("relu2_glu", _glu_one_rounding, [P.test_relu2_glu_hand_worked_rounding]),
    "five-per-byte digits in reverse order": ("pack_t1", _pack_t1_digits_reversed,
                                              [lambda g, t1=None: P.test_t1_golden_layout(t1)]),
    "prefill layout with O3's bit-pair order": (
        "pack_prefill", _pack_prefill_o3_pairs, [lambda g, pf=None: P.test_prefill_golden_layout(pf)]),
    "lookup-table index with the code roles swapped": (
        "lut_tables", _lut_tables_swapped_roles, [lambda g, lut=None: P.test_lut_golden_tables(lut)]),
}


def _call(pin, fixtures):
    import inspect
    params = list(inspect.signature(pin).parameters)
    if params[1:2] == ["t1"]:
        return pin(None, fixtures["t1"])
    if params[1:2] == ["lut"]:
        return pin(None, fixtures["lut"])
    if params[1:2] == ["pf"]:
        return pin(None, fixtures["pf"])
    return pin(fixtures["golden"]) if len(params) == 1 else pin()


@pytest.mark.parametrize("name", sorted(SLIPS))
def test_pins_reject_slip(name, golden, t1_golden, lut_golden, prefill_golden, monkeypatch):
    attr, fn, pins = SLIPS[name]
    fixtures = {"golden": golden, "t1": t1_golden, "lut": lut_golden, "pf": prefill_golden}
    for pin in pins:
        _call(pin, fixtures)          # the pin holds for the oracle as it stands
    monkeypatch.setattr(O, attr, fn)
    for pin in pins:
        with pytest.raises((AssertionError, ValueError, OverflowError)):
            _call(pin, fixtures)
