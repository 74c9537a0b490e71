"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the mistake it would catch.  None of them calls the HIP library.
"""

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import bitnet_oracle as O
from golden_util import golden_arrays, norm_example_arrays

F32 = np.float32


def f32_from_hex(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def frac_of(v):
    return Fraction(float(v))


# ---------------------------------------------------------------------------
# hand-worked examples (tests/golden/worked_examples.json)
# ---------------------------------------------------------------------------

def test_golden_worked_examples(golden):
    """Full layer on hand-derived examples: catches any wrong step end to end.

    The example with gamma and d both away from 1 fixes three readings that
    plainer examples leave open: the weight is divided by gamma (one correctly
    rounded division, not a product with a rounded reciprocal: one weight's
    quotient lands within 2^-25 of 0.5), the token scale is RN32(a*/127) (not
    the reciprocal of s, nor a* times RN32(1/127)), and the rescale multiplies
    acc by RN32(gamma * d) (the two other orders of the two products give
    different fp32 outputs)."""
    for ex in golden["examples"]:
        w, x, want_q, want_xq = golden_arrays(ex)
        packed, gamma = O.quantize_weights(w)
        want_gamma = f32_from_hex(ex["gamma_bits"]) if "gamma_bits" in ex else F32(ex["gamma"])
        assert gamma.view(np.uint32) == want_gamma.view(np.uint32), ex["name"]
        np.testing.assert_array_equal(O.ternarize(w, gamma), want_q)
        np.testing.assert_array_equal(packed, np.array(ex["packed"], dtype=np.uint8))
        xq, d = O.quantize_acts(x)
        np.testing.assert_array_equal(xq, want_xq)
        np.testing.assert_array_equal(d.view(np.uint32),
                                      np.array([int(h, 16) for h in ex["d_bits"]], dtype=np.uint32))
        acc, y = O.ternary_linear(packed, gamma, xq, d)
        np.testing.assert_array_equal(acc, np.array(ex["acc"], dtype=np.int32))
        want_y = np.array([[int(h, 16) for h in r] for r in ex["y_bits"]], dtype=np.uint32)
        np.testing.assert_array_equal(y.view(np.uint32), want_y)
        want_b = np.array([[int(h, 16) for h in r] for r in ex["y_bf16_bits"]], dtype=np.uint16)
        np.testing.assert_array_equal(O.f32_to_bf16_bits(y), want_b)


def test_golden_byte_layout(golden):
    """Bit order and code map: catches MSB-first packing, two's-complement codes."""
    for case in golden["byte_layout"]["cases"]:
        q = np.array([case["q"]], dtype=np.int8)
        assert int(O.pack_codes(q)[0, 0]) == case["byte"], case
        np.testing.assert_array_equal(O.unpack_codes(np.array([[case["byte"]]], np.uint8)), q)


def test_golden_size_arithmetic(golden):
    """Two bits per weight: eight weights in 16 bits, 100B weights in ~25 GB."""
    for n, k, nbytes in golden["size_arithmetic"]["cases"]:
        assert n * k // 4 == nbytes
        if n * k <= 1 << 20:
            assert O.pack_codes(np.zeros((n, k), np.int8)).nbytes == nbytes


# ---------------------------------------------------------------------------
# exact rounding of a rational to fp32
# ---------------------------------------------------------------------------

def test_rn32_ratio_matches_ieee_division():
    """numpy's fp32 division is correctly rounded: for fp32 operands the exact
    rational a/b must round to the same value.  Catches truncation, off-by-one
    exponent choice and wrong tie handling (sub-normal quotients included)."""
    rng = np.random.Generator(np.random.PCG64(11))
    a = (rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))).astype(np.float32)
    b = (rng.standard_normal(4000) * np.exp2(rng.integers(-60, 60, 4000))).astype(np.float32)
    a = np.abs(a)
    b = np.abs(b)
    # push a few quotients into the sub-normal range
    a[:200] = np.abs(rng.standard_normal(200)).astype(np.float32) * F32(2.0 ** -120)
    b[:200] = np.abs(rng.standard_normal(200)).astype(np.float32) * F32(2.0 ** 20)
    with np.errstate(under="ignore"):
        want = a / b
    for ai, bi, wi in zip(a, b, want):
        fa, fb = Fraction(float(ai)), Fraction(float(bi))
        r = fa / fb
        got = O.rn32_ratio(r.numerator, r.denominator)
        assert got.view(np.uint32) == wi.view(np.uint32), (ai, bi)


def test_rn32_ratio_nearest_and_ties_to_even():
    """Checks the defining property with exact Fractions on constructed ties and
    random large rationals (catches ties-away and double rounding)."""
    rng = np.random.Generator(np.random.PCG64(12))
    for _ in range(300):
        q = int(rng.integers(1 << 23, 1 << 24))
        e = int(rng.integers(-140, 90))
        tie = Fraction(2 * q + 1, 2) * Fraction(2) ** e
        got = O.rn32_ratio(tie.numerator, tie.denominator)
        want_q = q + (q & 1)
        assert Fraction(float(got)) == Fraction(want_q) * Fraction(2) ** e
    for _ in range(300):
        num = int(rng.integers(1, 1 << 62)) << int(rng.integers(0, 60))
        den = int(rng.integers(1, 1 << 40))
        r = Fraction(num, den)
        got = O.rn32_ratio(num, den)
        up = np.nextafter(got, F32(np.inf), dtype=np.float32)
        dn = np.nextafter(got, F32(0), dtype=np.float32)
        err = abs(r - frac_of(got))
        assert err <= abs(r - frac_of(up)) and err <= abs(r - frac_of(dn))


# ---------------------------------------------------------------------------
# O1: weight scale
# ---------------------------------------------------------------------------

def _mixed_weights(seed, n):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = (rng.standard_normal(n) * np.exp2(rng.integers(-30, 10, n))).astype(np.float32)
    w[:5] = np.array([0.0, -0.0, 1e-45, -3e-42, 2.0 ** -126], dtype=np.float32)
    return w


def test_exact_abs_sum_equals_fraction_sum():
    """Python Fractions hold every float exactly: catches dropped sub-normals,
    a wrong hidden bit or a wrong exponent offset in the integer decomposition."""
    for seed in range(6):
        w = _mixed_weights(seed, 3000)
        units = O.exact_abs_sum_units(w)
        want = sum((abs(Fraction(float(v))) for v in w), Fraction(0))
        assert Fraction(units) * Fraction(2) ** -149 == want


def test_exact_abs_sum_equals_plain_integer_sum():
    """Bucketed float64 sums against a plain per-element Python-integer sum on a
    wide exponent range (catches an inexact bucket sum or a wrong exponent shift)."""
    rng = np.random.Generator(np.random.PCG64(31))
    w = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)
    bits = w.view(np.uint32)
    want = 0
    for b in bits.tolist():
        e = (b >> 23) & 0xFF
        f = b & 0x7FFFFF
        want += ((f | (1 << 23)) << (e - 1)) if e else f
    assert O.exact_abs_sum_units(w) == want
    # many equal large significands in one exponent bucket
    w = np.full(1 << 21, np.nextafter(np.float32(2.0), np.float32(0)), dtype=np.float32)
    assert O.exact_abs_sum_units(w) == w.size * ((2 ** 24 - 1) << 126)   # biased exponent 127


def test_weight_scale_is_nearest_fp32_of_exact_mean():
    """gamma must be the fp32 nearest to the exact mean (checked against both
    neighbours with Fractions), including a case where a naive fp32 sum differs."""
    rng = np.random.Generator(np.random.PCG64(5))
    for n, k in [(3, 4), (17, 64), (64, 256)]:
        w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
        gamma = O.weight_scale(w)
        mean = sum((abs(Fraction(float(v))) for v in w.reshape(-1)), Fraction(0)) / (n * k)
        up = np.nextafter(gamma, F32(np.inf), dtype=np.float32)
        dn = np.nextafter(gamma, F32(0), dtype=np.float32)
        err = abs(mean - frac_of(gamma))
        assert err <= abs(mean - frac_of(up)) and err <= abs(mean - frac_of(dn))
    # one large value and many tiny ones: an fp32 running sum loses the tiny ones
    w = np.full(1 << 14, 2.0 ** -25, dtype=np.float32)
    w[0] = 1.0
    gamma = O.weight_scale(w)
    mean = (Fraction(1) + (w.size - 1) * Fraction(2) ** -25) / w.size
    assert abs(mean - frac_of(gamma)) <= abs(mean - frac_of(np.nextafter(gamma, F32(1))))
    naive = F32(np.float32(0))
    for v in w:
        naive = F32(naive + v)
    assert F32(naive / F32(w.size)) != gamma


def test_weight_scale_invariants():
    """Sign, order and power-of-two invariance; constant W; floor; non-finite."""
    rng = np.random.Generator(np.random.PCG64(8))
    w = (rng.standard_normal((32, 64)) * 0.02).astype(np.float32)
    g = O.weight_scale(w)
    assert O.weight_scale(-w) == g
    assert O.weight_scale(w[::-1, ::-1].copy()) == g
    assert O.weight_scale(rng.permutation(w.reshape(-1))) == g
    for j in (-3, 5):
        assert O.weight_scale(w * F32(2.0 ** j)) == g * F32(2.0 ** j)
    c = F32(0.0123)
    assert O.weight_scale(np.full((7, 12), c, np.float32)) == c
    assert O.weight_scale(np.full((3, 4), -c, np.float32)) == c
    assert O.weight_scale(np.zeros((4, 8), np.float32)) == F32(1e-5)
    assert O.weight_scale(np.full((4, 8), 1e-7, np.float32)) == F32(1e-5)
    for bad in (np.inf, -np.inf, np.nan):
        wb = w.copy()
        wb[3, 5] = bad
        assert np.isnan(O.weight_scale(wb))
        packed, gb = O.quantize_weights(wb)
        assert packed is None and np.isnan(gb)


# ---------------------------------------------------------------------------
# O2: ternarise
# ---------------------------------------------------------------------------

def test_ternarize_ties_and_clip():
    """t = +-0.5 -> 0 and t = +-1.5 -> +-1 (round half even, then clip): catches
    round-half-away-from-zero, floor/truncation and a missing clip."""
    w = np.array([[0.5, 1.5, -0.5, -1.5, 0.7, -0.3, 3.0, -9.0]], np.float32)
    gamma = F32(1.0)
    np.testing.assert_array_equal(O.ternarize(w, gamma), [[0, 1, 0, -1, 1, 0, 1, -1]])
    # just above / below the 0.5 threshold after the fp32 division
    g = F32(0.8125)
    half = F32(0.40625)                     # exactly g/2
    above = np.nextafter(half, F32(1), dtype=np.float32)
    below = np.nextafter(half, F32(0), dtype=np.float32)
    np.testing.assert_array_equal(O.ternarize(np.array([half, above, below, -above]), g),
                                  [0, 1, 0, -1])


def test_ternarize_gaussian_closed_form():
    """For W ~ N(0, s^2), gamma -> s*sqrt(2/pi) and q = 0 iff |W| < gamma/2, so
    P(q = 0) = erf(1/(2*sqrt(pi))) = 0.31006 and P(+1) = P(-1) = 0.34497.
    Catches dividing by absmax or RMS instead of the absolute mean."""
    w = np.random.Generator(np.random.PCG64(21)).standard_normal(1 << 22, dtype=np.float32)
    w *= F32(0.02)
    q = O.ternarize(w, O.weight_scale(w))
    p0 = math.erf(1.0 / (2.0 * math.sqrt(math.pi)))
    n = w.size
    sigma0 = math.sqrt(p0 * (1 - p0) / n)
    assert abs(np.mean(q == 0) - p0) < 5 * sigma0
    p1 = (1 - p0) / 2
    sigma1 = math.sqrt(p1 * (1 - p1) / n)
    assert abs(np.mean(q == 1) - p1) < 5 * sigma1
    assert abs(np.mean(q == -1) - p1) < 5 * sigma1
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}


def test_ternarize_symmetry_and_scale():
    rng = np.random.Generator(np.random.PCG64(3))
    w = (rng.standard_normal((16, 64)) * 0.02).astype(np.float32)
    g = O.weight_scale(w)
    q = O.ternarize(w, g)
    np.testing.assert_array_equal(O.ternarize(-w, O.weight_scale(-w)), -q)
    w2 = w * F32(8.0)
    np.testing.assert_array_equal(O.ternarize(w2, O.weight_scale(w2)), q)


# ---------------------------------------------------------------------------
# O3: pack / unpack
# ---------------------------------------------------------------------------

def test_pack_roundtrip_all_valid_bytes():
    """All 81 bytes built from codes {0,1,2} survive unpack->pack; code 3 is rejected."""
    valid = [c0 | c1 << 2 | c2 << 4 | c3 << 6
             for c0, c1, c2, c3 in itertools.product(range(3), repeat=4)]
    b = np.array([valid], dtype=np.uint8)
    np.testing.assert_array_equal(O.pack_codes(O.unpack_codes(b)), b)
    with pytest.raises(ValueError):
        O.unpack_codes(np.array([[0xFF]], np.uint8))
    rng = np.random.Generator(np.random.PCG64(4))
    q = rng.integers(-1, 2, (13, 40)).astype(np.int8)
    np.testing.assert_array_equal(O.unpack_codes(O.pack_codes(q)), q)
    assert O.pack_codes(q).shape == (13, 10)


# ---------------------------------------------------------------------------
# O4: activations
# ---------------------------------------------------------------------------

def test_act_quant_invariants():
    """Range, exact 127 at the row maximum, sign symmetry, power-of-two scaling,
    per-token independence and the half-step error bound."""
    rng = np.random.Generator(np.random.PCG64(9))
    x = rng.standard_normal((257, 96)).astype(np.float32)
    x[5] *= F32(1e4)
    x[6] *= F32(1e-3)
    xq, d = O.quantize_acts(x)
    assert xq.min() >= -127 and xq.max() <= 127
    np.testing.assert_array_equal(np.abs(xq.astype(np.int32)).max(axis=1), 127)
    xn, dn = O.quantize_acts(-x)
    np.testing.assert_array_equal(xn, -xq)
    np.testing.assert_array_equal(dn, d)
    for j in (-7, 4):
        xs, ds = O.quantize_acts(x * F32(2.0 ** j))
        np.testing.assert_array_equal(xs, xq)
        np.testing.assert_array_equal(ds, d * F32(2.0 ** j))
    # a row's result does not depend on the other rows (per-token, not per-tensor)
    xr, dr = O.quantize_acts(x[5:6])
    np.testing.assert_array_equal(xr[0], xq[5])
    assert dr[0] == d[5]
    # |xq*d - x| <= d/2 (plus fp32 slack) everywhere: catches d = a/128 or Qb = 128
    err = np.abs(xq.astype(np.float64) * d[:, None] - x.astype(np.float64))
    assert np.all(err <= d[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_act_quant_ties_and_zero_row():
    """Row with absmax 127 has s = 1 exactly, so xq = round-half-even(x)."""
    x = np.array([[127.0, 2.5, -0.5, 3.5, 126.5, -1.5, 0.49, -127.0],
                  [0.0] * 8], np.float32)
    xq, d = O.quantize_acts(x)
    np.testing.assert_array_equal(xq[0], [127, 2, 0, 4, 126, -2, 0, -127])
    assert d[0] == F32(1.0)
    np.testing.assert_array_equal(xq[1], 0)
    assert d[1].view(np.uint32) == 0x33A917DC          # RN32(RN32(1e-5)/127)


def test_act_quant_rounding_of_product_matches_fraction():
    """xq = rne(RN32(x*s)): compare with exact Fractions, rounding the product
    to fp32 by hand through rn32_ratio's independent check above."""
    rng = np.random.Generator(np.random.PCG64(10))
    x = rng.standard_normal((4, 33)).astype(np.float32)
    xq, d = O.quantize_acts(x)
    for m in range(4):
        a = max(abs(Fraction(float(v))) for v in x[m])
        s = F32(127.0) / F32(float(a))
        for k in range(33):
            prod = Fraction(float(x[m, k])) * Fraction(float(s))
            p32 = O.rn32_ratio(abs(prod.numerator), prod.denominator)
            p = Fraction(float(p32)) * (1 if prod >= 0 else -1)
            fl = math.floor(p)
            rem = p - fl
            r = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else 0)
            assert int(xq[m, k]) == max(-128, min(127, r))


# ---------------------------------------------------------------------------
# O5: integer contraction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("k", [4, 8])
def test_matmul_brute_force_every_ternary_row(k):
    """W enumerates all 3^K ternary rows; every output is checked against a
    pure-Python integer dot product.  Catches transposed operands, a wrong sign,
    a wrong unpack order and any dropped term."""
    rows = np.array(list(itertools.product((-1, 0, 1), repeat=k)), dtype=np.int8)
    rng = np.random.Generator(np.random.PCG64(k))
    xq = rng.integers(-128, 128, (3, k)).astype(np.int8)
    xq[0, 0] = -128
    xq[1, :] = 127
    packed = O.pack_codes(rows)
    acc, _ = O.ternary_linear(packed, F32(1.0), xq, np.ones(3, np.float32))
    for m in range(3):
        for n in range(rows.shape[0]):
            want = 0
            for j in range(k):
                want += int(rows[n, j]) * int(xq[m, j])
            assert int(acc[m, n]) == want


def test_matmul_equals_sum_pos_minus_sum_neg():
    """The pages' form (sum over +1 weights minus sum over -1 weights)."""
    rng = np.random.Generator(np.random.PCG64(13))
    q = rng.integers(-1, 2, (37, 100)).astype(np.int8)
    xq = rng.integers(-127, 128, (5, 100)).astype(np.int8)
    acc = O.integer_matmul(q, xq)
    for m in range(5):
        for n in range(37):
            assert int(acc[m, n]) == O.sum_pos_minus_sum_neg(q[n], xq[m])
    np.testing.assert_array_equal(O.integer_matmul(-q, xq), -acc)


def test_matmul_equals_int64_product_at_the_largest_k():
    """The contraction against numpy's int64 product (a different library routine
    and number type) at the largest K the linear calls accept, with the extreme
    values: all +1 weights against all 127 (or -128) activations reach
    |acc| = 128 K.  Catches a contraction that rounds once the sums grow."""
    k = 131072
    rng = np.random.Generator(np.random.PCG64(21))
    q = rng.integers(-1, 2, (6, k)).astype(np.int8)
    q[0] = 1
    q[1] = -1
    xq = rng.integers(-128, 128, (3, k)).astype(np.int8)
    xq[0] = 127
    xq[1] = -128
    acc = O.integer_matmul(q, xq)
    want = xq.astype(np.int64) @ q.astype(np.int64).T
    np.testing.assert_array_equal(acc.astype(np.int64), want)
    assert int(acc[0, 0]) == 127 * k and int(acc[1, 0]) == -128 * k and int(acc[1, 1]) == 128 * k


def test_identity_weights_reproduce_activations():
    """W = I: gamma = RN32(1/K), every diagonal t ~ K >= 1.5 -> q = I, acc = xq."""
    k = 64
    packed, gamma = O.quantize_weights(np.eye(k, dtype=np.float32))
    assert gamma == F32(1.0 / k)
    np.testing.assert_array_equal(O.unpack_codes(packed), np.eye(k, dtype=np.int8))
    x = np.random.Generator(np.random.PCG64(2)).standard_normal((3, k)).astype(np.float32)
    xq, d, acc, y = O.quant_linear(packed, gamma, x)
    np.testing.assert_array_equal(acc, xq.astype(np.int32))
    np.testing.assert_array_equal(y, xq.astype(np.float32) * (gamma * d)[:, None])


def test_sampled_outputs_match_full():
    rng = np.random.Generator(np.random.PCG64(14))
    w = (rng.standard_normal((40, 128)) * 0.02).astype(np.float32)
    x = rng.standard_normal((6, 128)).astype(np.float32)
    packed, gamma = O.quantize_weights(w)
    xq, d, acc, y = O.quant_linear(packed, gamma, x)
    mi = rng.integers(0, 6, 50)
    ni = rng.integers(0, 40, 50)
    a2, y2 = O.ternary_linear_at(packed, gamma, xq, d, mi, ni)
    np.testing.assert_array_equal(a2, acc[mi, ni])
    np.testing.assert_array_equal(y2.view(np.uint32), y[mi, ni].view(np.uint32))


# ---------------------------------------------------------------------------
# O6: rescale
# ---------------------------------------------------------------------------

def test_dequant_error_bound_and_zero():
    """y is within two fp32 roundings of acc*gamma*d (exact rationals), and acc=0 -> +0."""
    rng = np.random.Generator(np.random.PCG64(15))
    acc = rng.integers(-(1 << 20), 1 << 20, (7, 50)).astype(np.int32)
    acc[0, :3] = 0
    d = (np.abs(rng.standard_normal(7)) * 0.05).astype(np.float32)
    gamma = F32(0.0159587)
    y = O.dequantize(acc, gamma, d)
    assert np.all(y[0, :3] == 0) and not np.any(np.signbit(y[0, :3]))
    for m in range(7):
        for n in range(50):
            exact = Fraction(int(acc[m, n])) * Fraction(float(gamma)) * Fraction(float(d[m]))
            if exact == 0:
                continue
            rel = abs((Fraction(float(y[m, n])) - exact) / exact)
            assert rel <= Fraction(2 * 2 ** -24 + 2 ** -47)


def test_bf16_rounding_matches_torch():
    """The oracle's fp32->bf16 rounding against torch's conversion (RNE)."""
    torch = pytest.importorskip("torch")
    rng = np.random.Generator(np.random.PCG64(16))
    y = (rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))).astype(np.float32)
    ties = (rng.integers(0, 1 << 15, 2000).astype(np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    y = np.concatenate([y, ties.view(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40], np.float32)])
    y = y[np.isfinite(y) | np.isinf(y)]
    got = O.f32_to_bf16_bits(y)
    want = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, want)
    nan = O.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert (int(nan[0]) & 0x7F80) == 0x7F80 and (int(nan[0]) & 0x7F) != 0


def test_bf16_upcast_is_exact():
    torch = pytest.importorskip("torch")
    x = torch.randn(1000, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_bits_to_f32(bits), x.float().numpy())


# ---------------------------------------------------------------------------
# N1-N3: squared-ReLU gating and the sub-layer RMS norm in front of the layer
# ---------------------------------------------------------------------------

def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def test_relu2_glu_hand_worked_rounding():
    """Worked by hand: a = 1 + 2^-12, a^2 = 1 + 2^-11 + 2^-24 is a tie between
    1 + 2^-11 (even) and the next fp32, so RN32(a^2) = 1 + 2^-11 (0x3F801000);
    times up = 1 + 2^-23 the exact product 1 + 2^-11 + 2^-23 + 2^-34 rounds to
    0x3F801001.  Rounding once at the end instead would give 0x3F801002."""
    gate = np.array([_f32(0x3F800800), -2.0, 3.0, 0.0], dtype=np.float32)
    up = np.array([_f32(0x3F800001), 5.0, 0.5, -7.0], dtype=np.float32)
    u = O.relu2_glu(gate, up)
    assert u.view(np.uint32)[0] == 0x3F801001
    assert u[1] == 0.0 and u[2] == np.float32(4.5) and u[3] == 0.0


def test_relu2_glu_matches_exact_rational_steps():
    rng = np.random.default_rng(11)
    g = rng.standard_normal(2000).astype(np.float32)
    up = rng.standard_normal(2000).astype(np.float32)
    u = O.relu2_glu(g, up)
    for i in range(0, 2000, 7):
        a = max(Fraction(float(g[i])), Fraction(0))
        a2 = O.rn32_ratio((a * a).numerator, (a * a).denominator)
        prod = Fraction(float(a2)) * Fraction(float(up[i]))
        want = O.rn32_ratio(abs(prod).numerator, prod.denominator) if prod != 0 else np.float32(0)
        want = -want if prod < 0 else want
        assert np.float32(u[i]) == np.float32(want)


def test_exact_square_sum_equals_fraction_sum():
    rng = np.random.default_rng(12)
    v = (rng.standard_normal(3000) * np.exp(rng.uniform(-60, 60, 3000))).astype(np.float32)
    v[:5] = np.array([0x1, 0x7FFFFF, 0x00800000, 0x3F800000, 0x80000003], dtype=np.uint32).view(np.float32)
    exact = sum(Fraction(float(t)) ** 2 for t in v)
    assert Fraction(O.exact_square_sum_units(v), 1 << 298) == exact


def test_rms_factor_closed_form_integer_rows():
    """Rows 1..n (eps = 0): sum k^2 = n(n+1)(2n+1)/6, so mean = (n+1)(2n+1)/6."""
    for n in (1, 3, 64, 1000, 4096):
        v = np.arange(1, n + 1, dtype=np.float32)[None, :]
        mean = Fraction((n + 1) * (2 * n + 1), 6)
        ms = O.rn32_ratio(mean.numerator, mean.denominator)
        want = np.float32(1.0 / math.sqrt(float(ms)))
        assert O.rms_factor(v, 0.0)[0] == want


def test_rms_factor_power_of_two_scaling_and_float64():
    rng = np.random.default_rng(13)
    v = rng.standard_normal((6, 700)).astype(np.float32)
    r0 = O.rms_factor(v, 0.0)
    for j in (-5, 3, 9):
        rj = O.rms_factor((v * np.float32(2.0 ** j)).astype(np.float32), 0.0)
        np.testing.assert_array_equal(rj, (r0 * np.float32(2.0 ** -j)).astype(np.float32))
    r = O.rms_factor(v, 1e-5)
    ref = 1.0 / np.sqrt((v.astype(np.float64) ** 2).mean(axis=1) + 1e-5)
    assert np.all(np.abs(r / ref - 1.0) < 3e-7)


def test_norm_golden_example(golden):
    """Hand-worked normalise-then-quantise example (tests/golden/worked_examples.json,
    norm_examples): the exact mean of squares, r, the normalised and scaled values,
    and the codes and token scale.  Catches the fused order (quantising v * w and
    folding r into the token scale: another code and scale here), a rounding of
    v * w * r in one step, and a mean of squares summed in fp32."""
    for ex in golden["norm_examples"]:
        v, w = norm_example_arrays(ex)
        r = O.rms_factor(v, ex["eps"])
        assert r.view(np.uint32)[0] == int(ex["r_bits"], 16)
        u = O.rms_normalise(v, w, ex["eps"])
        np.testing.assert_array_equal(u[0, :4].view(np.uint32), [int(h, 16) for h in ex["u_bits"]])
        assert not np.any(u[0, 4:])
        xq, d = O.prologue_quantize_acts(v, norm_weight=w, eps=ex["eps"])
        want = np.zeros(ex["K"], np.int8)
        for i, q in ex["xq_entries"]:
            want[i] = q
        np.testing.assert_array_equal(xq[0], want)
        assert d.view(np.uint32)[0] == int(ex["d_bits"], 16)
        assert int(xq[0, 0]) != ex["fused_order_xq0"]


def test_norm_mean_of_squares_at_a_rounding_midpoint():
    """A row whose exact mean of squares lies exactly halfway between two fp32
    values: v0 = 1 + 2^-12, the other 63 inputs 0, so the mean is
    (1 + 2^-11 + 2^-24) / 64 = 2^-6 + 2^-17 + 2^-30, halfway between
    2^-6 + 2^-17 and the next fp32 (spacing 2^-29); ties go to the even
    significand 2^23 + 2^12, i.e. 2^-6 + 2^-17 (0x3c801000).  Catches a mean
    rounded half away from zero or rounded twice."""
    v = np.zeros((1, 64), np.float32)
    v[0, 0] = np.float32(1 + 2.0 ** -12)
    assert O.mean_of_squares(v).view(np.uint32)[0] == 0x3C801000
    # scaled by 2^60 the mean is 2^120 times as large: the same significand
    big = (v * np.float32(2.0 ** 60)).astype(np.float32)
    assert O.mean_of_squares(big).view(np.uint32)[0] == 0x3C801000 + (120 << 23)
    # scaled by 2^-70 the mean 2^-146 + 2^-157 + 2^-170 is sub-normal: 2^-149
    # spacing, 8 + 2^-8 + 2^-21 units, rounds to 8 units (bits 0x00000008)
    tiny = (v * np.float32(2.0 ** -70)).astype(np.float32)
    assert O.mean_of_squares(tiny).view(np.uint32)[0] == 8


def test_norm_mean_of_squares_just_above_a_midpoint():
    """The midpoint row above plus v1 = 2^-40: the exact mean exceeds the midpoint
    by 2^-86 and rounds up to 0x3c801001, while a float64 sum of the squares loses
    v1^2 = 2^-80 (below half an ulp of 1) and lands on the midpoint itself, which
    rounds to even (0x3c801000).  Catches a sum of squares that is not exact and a
    dropped sticky bit."""
    v = np.zeros((1, 64), np.float32)
    v[0, 0] = np.float32(1 + 2.0 ** -12)
    v[0, 1] = np.float32(2.0 ** -40)
    assert O.mean_of_squares(v).view(np.uint32)[0] == 0x3C801001
    ss = np.float64(v[0, 0]) ** 2 + np.float64(v[0, 1]) ** 2
    assert np.float32(ss / 64).view(np.uint32) == 0x3C801000


def test_norm_closed_forms():
    """A constant row c = 2^j (eps = 0): ms = 4^j, r = 2^-j exactly, every
    normalised value is +-1 and u is the norm weight itself, so the codes and
    scale are O4 of w, whatever j.  A zero row: u = 0, codes 0, the floor scale."""
    rng = np.random.default_rng(16)
    w = (1.0 + 0.3 * rng.standard_normal(256)).astype(np.float32)
    want_q, want_d = O.quantize_acts(w[None, :])
    for j in (-9, 0, 5):
        for sign in (1.0, -1.0):
            v = np.full((1, 256), sign * 2.0 ** j, np.float32)
            xq, d = O.prologue_quantize_acts(v, norm_weight=w, eps=0.0)
            np.testing.assert_array_equal(xq, (want_q * np.int8(sign)).astype(np.int8))
            np.testing.assert_array_equal(d, want_d)
    xq0, d0 = O.prologue_quantize_acts(np.zeros((2, 256), np.float32), norm_weight=w, eps=1e-5)
    assert not np.any(xq0)
    assert np.all(d0 == np.float32(O.EPS / O.QB))


def test_prologue_quantize_invariants():
    rng = np.random.default_rng(15)
    g = rng.standard_normal((5, 512)).astype(np.float32)
    up = rng.standard_normal((5, 512)).astype(np.float32)
    w = (1.0 + 0.2 * rng.standard_normal(512)).astype(np.float32)
    xq, d = O.prologue_quantize_acts(g, up=up, norm_weight=w, eps=0.0)
    # scaling the up projection of a row by 2^j leaves the normalised input, so
    # the codes and the token scale, unchanged (eps = 0)
    for j in (-7, 4):
        xq2, d2 = O.prologue_quantize_acts(g, up=(up * np.float32(2.0 ** j)).astype(np.float32),
                                           norm_weight=w, eps=0.0)
        np.testing.assert_array_equal(xq2, xq)
        np.testing.assert_array_equal(d2, d)
    # a gate that is negative everywhere zeroes the row: codes 0 and the floor
    # scale (the normalised row is 0)
    gz = -np.abs(g)
    xq0, d0 = O.prologue_quantize_acts(gz, up=up, norm_weight=w, eps=1e-5)
    assert not np.any(xq0)
    assert np.all(d0 == np.float32(O.EPS / O.QB))
    # without a norm the prologue is plain O4 of the gated input
    xq1, d1 = O.prologue_quantize_acts(g, up=up)
    xq2, d2 = O.quantize_acts(O.relu2_glu(g, up))
    np.testing.assert_array_equal(xq1, xq2)
    np.testing.assert_array_equal(d1, d2)


# ---------------------------------------------------------------------------
# T1: five ternary codes per byte (base 3)
# ---------------------------------------------------------------------------

def _t1_case_q(case):
    q = np.zeros((1, case["K"]), np.int8)
    for k, v in case["set"]:
        q[0, k] = v
    return q


def test_t1_golden_layout(t1_golden):
    """Hand-worked bytes: catches a transposed block, a reversed digit order, a
    wrong padding code."""
    for case in t1_golden["cases"]:
        q = _t1_case_q(case)
        want = np.full(O.t1_row_bytes(case["K"]), case["bytes"]["all"], np.uint8)
        for i, v in case["bytes"].items():
            if i != "all":
                want[int(i)] = v
        np.testing.assert_array_equal(O.pack_t1(q)[0], want, err_msg=case["name"])
        np.testing.assert_array_equal(O.unpack_t1(want[None, :], case["K"]), q)


def _fixed_point_digits(byte):
    """Base-3 digits of an 8-bit fixed-point fraction, most significant first:
    each is the integer part of three times the remaining fraction."""
    f, out = int(byte), []
    for _ in range(5):
        t = 3 * f
        out.append(t >> 8)
        f = t & 255
    return out


def test_t1_bytes_are_fixed_point_base3_fractions():
    """For every v in 0..242 (digits from Python's base-3 string, least
    significant = the block's first 16 weights): the byte is v/243 rounded up
    to a multiple of 1/256 (checked with Fraction), its fixed-point digits are
    the digits of v, and the decoder recovers them."""
    for v in range(243):
        digits = [int(c) for c in reversed(np.base_repr(v, 3).rjust(5, "0"))]
        q = np.zeros((1, 80), np.int8)
        for j in range(5):
            q[0, 16 * j] = digits[j] - 1
        byte = int(O.pack_t1(q)[0, 0])
        gap = Fraction(byte, 256) - Fraction(v, 243)
        assert 0 <= gap < Fraction(1, 256), (v, byte)
        assert _fixed_point_digits(byte) == digits[::-1], (v, byte)
        back = O.unpack_t1(np.full((1, 16), byte, np.uint8), 80)[0]
        for j in range(5):
            np.testing.assert_array_equal(back[16 * j:16 * j + 16], digits[j] - 1)


def test_t1_pack_matches_python_int_parse():
    """Independent packer: each byte from int(s, 3) of the codes picked by
    explicit index arithmetic, rounded up with Fraction, on ragged rows."""
    rng = np.random.Generator(np.random.PCG64(51))
    for k in (1, 7, 79, 80, 81, 173):
        q = rng.integers(-1, 2, (3, k)).astype(np.int8)
        got = O.pack_t1(q)
        nb = (k + 79) // 80
        assert got.shape == (3, 16 * nb)
        for n in range(3):
            for b in range(nb):
                for i in range(16):
                    codes = []
                    for j in range(5):
                        kk = 80 * b + 16 * j + i
                        codes.append(int(q[n, kk]) + 1 if kk < k else 1)
                    v = int("".join(str(c) for c in reversed(codes)), 3)
                    want = math.ceil(Fraction(256 * v, 243))
                    assert int(got[n, 16 * b + i]) == want, (k, n, b, i)


def test_t1_bijection_and_roundtrip():
    """The 3^5 digit tuples map one-to-one onto 243 bytes; the other 13 bytes,
    and non-zero padding, are rejected; pack/unpack round trips."""
    seen = set()
    for tup in itertools.product((-1, 0, 1), repeat=5):
        q = np.zeros((1, 80), np.int8)
        q[0, [0, 16, 32, 48, 64]] = tup
        seen.add(int(O.pack_t1(q)[0, 0]))
    assert len(seen) == 243 and max(seen) == 255 and min(seen) == 0
    for byte in set(range(256)) - seen:
        with pytest.raises(ValueError):
            O.unpack_t1(np.full((1, 16), byte, np.uint8), 80)
    rng = np.random.Generator(np.random.PCG64(52))
    for k in (1, 64, 80, 100, 160, 6912 // 8):
        q = rng.integers(-1, 2, (5, k)).astype(np.int8)
        np.testing.assert_array_equal(O.unpack_t1(O.pack_t1(q), k), q)
    b = O.pack_t1(rng.integers(-1, 2, (4, 160)).astype(np.int8))
    np.testing.assert_array_equal(O.pack_t1(O.unpack_t1(b, 160)), b)
    q80 = np.zeros((1, 80), np.int8)
    q80[0, 79] = 1                                     # weight k = 79 >= K = 70
    with pytest.raises(ValueError):
        O.unpack_t1(O.pack_t1(q80), 70)


def test_t1_linear_equals_two_bit_linear():
    """The same ternary matrix in both formats gives identical accumulators and
    outputs (the 2-bit contraction is pinned by brute force above)."""
    rng = np.random.Generator(np.random.PCG64(53))
    for k in (64, 160, 6912 // 16):
        q = rng.integers(-1, 2, (9, k)).astype(np.int8)
        xq = rng.integers(-127, 128, (3, k)).astype(np.int8)
        d = rng.uniform(0.001, 0.05, 3).astype(np.float32)
        gamma = np.float32(0.0173)
        acc2, y2 = O.ternary_linear(O.pack_codes(q), gamma, xq, d)
        acc5, y5 = O.ternary_linear_t1(O.pack_t1(q), gamma, xq, d)
        np.testing.assert_array_equal(acc5, acc2)
        np.testing.assert_array_equal(y5.view(np.uint32), y2.view(np.uint32))
        mi, ni = np.array([0, 2, 1]), np.array([8, 0, 4])
        acc_s, y_s = O.ternary_linear_t1_at(O.pack_t1(q), gamma, xq, d, mi, ni)
        np.testing.assert_array_equal(acc_s, acc5[mi, ni])
        np.testing.assert_array_equal(y_s.view(np.uint32), y5[mi, ni].view(np.uint32))


def test_t1_quantize_weights_is_ternarise_then_pack():
    rng = np.random.Generator(np.random.PCG64(54))
    w = (rng.standard_normal((6, 200)) * 0.02).astype(np.float32)
    p2, g2 = O.quantize_weights(w)
    p5, g5 = O.quantize_weights_t1(w)
    assert g5.view(np.uint32) == g2.view(np.uint32)
    np.testing.assert_array_equal(O.unpack_t1(p5, 200), O.unpack_codes(p2))
    wn = w.copy()
    wn[1, 3] = np.inf
    p, g = O.quantize_weights_t1(wn)
    assert p is None and np.isnan(g)


def test_t1_size_matches_page_figure(t1_golden):
    """The 2B-shaped stack: 0.42 GB at five trits per byte, which matches the
    0.4 GB the comparison table gives for the 2B model (the 2-bit layout's
    0.52 GB does not)."""
    s = t1_golden["size_2b_stack"]
    layer = [(2560, 2560), (2560, 640), (2560, 640), (2560, 2560), (2560, 6912),
             (2560, 6912), (6912, 2560)]
    per_layer = sum(n * O.t1_row_bytes(k) for k, n in layer)
    assert per_layer == s["layer_bytes"]
    assert 30 * per_layer == s["stack_bytes"]
    assert 30 * sum(n * k // 4 for k, n in layer) == s["stack_bytes_2bit"]
    assert round(s["stack_bytes"] / 1e9, 1) == s["page_figure_gb"]
    assert round(s["stack_bytes_2bit"] / 1e9, 1) != s["page_figure_gb"]
    assert O.pack_t1(np.zeros((2, 6912), np.int8)).shape == (2, O.t1_row_bytes(6912))


# ---------------------------------------------------------------------------
# L1: lookup-table contraction
# ---------------------------------------------------------------------------

def test_lut_golden_tables(lut_golden):
    """Hand-worked table entries (catches swapped code roles, a missing offset)."""
    for case in lut_golden["cases"]:
        t = O.lut_tables(np.array([case["x"]], np.int8))[0, 0]
        for i, v in case["entries"].items():
            assert int(t[int(i)]) == v, (case["x"], i)
    ex = lut_golden["row_example"]
    acc, _ = O.lut_linear(np.array([[ex["packed_byte"]]], np.uint8), np.float32(1.0),
                          np.array([ex["x"]], np.int8), np.ones(1, np.float32))
    assert int(acc[0, 0]) == ex["acc"]


def test_lut_entries_are_sum_pos_minus_sum_neg():
    """Every valid nibble of every random pair: the entry is the pages' form
    (sum under +1 weights minus sum under -1 weights) of the two weights."""
    rng = np.random.Generator(np.random.PCG64(61))
    x = rng.integers(-127, 128, (1, 64)).astype(np.int8)
    t = O.lut_tables(x)[0]
    for g in range(32):
        for c0 in range(3):
            for c1 in range(3):
                q = np.array([c0 - 1, c1 - 1])
                assert t[g, c0 + 4 * c1] == O.sum_pos_minus_sum_neg(q, x[0, 2 * g:2 * g + 2])


def test_lut_linear_equals_integer_matmul():
    """The table method reaches the pinned contraction exactly (acc and y)."""
    rng = np.random.Generator(np.random.PCG64(62))
    for m, n, k in ((1, 33, 64), (3, 17, 256), (2, 5, 8)):
        q = rng.integers(-1, 2, (n, k)).astype(np.int8)
        xq = rng.integers(-127, 128, (m, k)).astype(np.int8)
        d = rng.uniform(0.001, 0.05, m).astype(np.float32)
        p = O.pack_codes(q)
        acc, y = O.lut_linear(p, np.float32(0.021), xq, d)
        acc_w, y_w = O.ternary_linear(p, np.float32(0.021), xq, d)
        np.testing.assert_array_equal(acc, acc_w)
        np.testing.assert_array_equal(y.view(np.uint32), y_w.view(np.uint32))


# ---------------------------------------------------------------------------
# P1: prefill weight layout
# ---------------------------------------------------------------------------

def _prefill_case(case):
    n, k = case["N"], case["K"]
    q = np.zeros((n, k), np.int8)
    if "codes_row0" in case:
        q[0, :] = np.array(case["codes_row0"], np.int16) - 1
    for r, c, v in case.get("set", []):
        q[r, c] = v
    want = np.full(case["size"], case["other"], np.uint8)
    for off, v in case["bytes"].items():
        want[int(off)] = v
    return q, want


def test_prefill_golden_layout(prefill_golden):
    """Hand-worked bytes (tests/golden/prefill_layout.json): catches the bit pairs
    in O3's order, a wrong block order, a swapped chunk index (r + 32 h) and a
    wrong padding code."""
    for case in prefill_golden["cases"]:
        q, want = _prefill_case(case)
        assert O.prefill_layout_bytes(case["N"], case["K"]) == case["size"]
        np.testing.assert_array_equal(O.pack_prefill(q), want, err_msg=case["name"])
        np.testing.assert_array_equal(O.unpack_prefill(want, case["N"], case["K"]), q)


def test_prefill_layout_roundtrip_and_contraction():
    """Random ternary matrices (ragged N and K, K = 64 mod 128): the layout is a
    bijection onto valid codes, the O3 repack agrees with packing q directly, and
    the contraction on P1 weights equals the one on O3 weights (same integers)."""
    rng = np.random.default_rng(71)
    for n, k in ((1, 64), (33, 192), (64, 256), (70, 2560), (5, 6912)):
        q = rng.integers(-1, 2, (n, k)).astype(np.int8)
        p1 = O.pack_prefill(q)
        assert p1.size == O.prefill_layout_bytes(n, k)
        np.testing.assert_array_equal(O.unpack_prefill(p1, n, k), q)
        np.testing.assert_array_equal(O.repack_prefill(O.pack_codes(q), k), p1)
        xq = rng.integers(-128, 128, (3, k)).astype(np.int8)
        d = rng.random(3).astype(np.float32)
        acc_a, y_a = O.ternary_linear_prefill(p1, n, F32(0.5), xq, d)
        acc_b, y_b = O.ternary_linear(O.pack_codes(q), F32(0.5), xq, d)
        np.testing.assert_array_equal(acc_a, acc_b)
        np.testing.assert_array_equal(y_a, y_b)
    # a byte holding code 3, and a non-zero padding weight, are rejected
    p1 = O.pack_prefill(np.zeros((1, 64), np.int8))
    bad = p1.copy(); bad[0] = 0xFF
    with pytest.raises(ValueError):
        O.unpack_prefill(bad, 1, 64)
    bad = p1.copy(); bad[100] = 0x56          # row 6, inside the padding rows
    with pytest.raises(ValueError):
        O.unpack_prefill(bad, 1, 64)
