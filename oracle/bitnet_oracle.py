"""Plain CPU oracle for the BitNet b1.58 W1.58A8 ternary linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product
path (the HIP library and its Python binding) never touches it, and this module
imports nothing from the product package: the two share no code.

Every step is the plain definition written out with numpy (fp32 where the step
is a floating-point rounding, exact Python integers where the step is an exact
sum or an integer contraction).  Nothing is blocked, fused or reordered.

Sources (web pages, cited by title and section)
-----------------------------------------------
[OV]  onedollarvps.pages.dev, "如何在本地運行 BitNet B1.58（1-Bit LLM）"
      (How to run BitNet B1.58 locally), section 2 "技術背景" (technical
      background), sub-section on 1-bit vs 1.58-bit quantisation: weights are
      scaled by the reciprocal of their mean absolute value, then rounded and
      clipped to the three values -1, 0, +1.
[DT]  dashen-tech.com, "BitNet.cpp 深度解析：1-bit LLM 推論、CPU 上運行 100B
      模型速度提升 6 倍" (BitNet.cpp deep dive), section 2.3 "I2_S 格式" (2 bits
      per stored weight, eight weights in 16 bits) and section 3.1 "計算核心：
      整數矩陣乘法" (integer matmul; the product with ternary weights splits into
      the sum over +1 weights minus the sum over -1 weights).
[CM]  communeify.com, "微軟 BitNet b1.58 震撼登場：跑更快、更省電的 1 位元 AI
      模型來了？", section introducing BitNet b1.58 2B4T, item "量化細節"
      (quantisation details: W1.58A8, i.e. ternary weights, 8-bit integer
      activations).
[GN]  th.news.hada.io, "BitNet - เฟรมเวิร์กการอนุมานสำหรับ LLM แบบ 1 บิต"
      (GeekNews summary), Hacker News comments: the stored 2-bit field can hold
      the four values -1, 0, 1, 2.

Readings taken where the pages are silent
-----------------------------------------
O1  weight scale: one per-tensor scale; the mean |W| is taken exactly and
    rounded once to fp32 (RN32, ties to even); gamma* = max(gamma, RN32(1e-5)).
O2  ternarise: t = RN32(W / gamma*) (correctly rounded fp32 division), then
    round half to even, then clip to [-1, 1].
O3  pack: code = q + 1 in {0, 1, 2}; four codes per byte, least significant bit
    pair first; row n occupies bytes [n*K/4, (n+1)*K/4); K % 4 == 0.
O4  activations: per token (row) absmax a, a* = max(a, RN32(1e-5)),
    s = RN32(127 / a*), xq = clip(rne(RN32(x * s)), -128, 127), d = RN32(a* / 127).
O5  contraction: acc[m, n] = sum_k q[n, k] * xq[m, k] exactly (int32 range).
O6  rescale: y = RN32(float(acc) * RN32(gamma* * d[m])); bf16 output = RNE(y).

Neighbours of the layer ([CM], section introducing BitNet b1.58 2B4T, item
"架構" (architecture): squared-ReLU activation, sub-layer normalisation, no bias
terms anywhere):
N1  squared-ReLU gating: u = RN32(RN32(max(g, 0) * max(g, 0)) * up), elementwise,
    where g and up are the gate and up projections of the same input.
N2  sub-layer RMS normalisation (no bias) of the input v of a BitLinear layer:
    RMSNorm(v)[k] = v[k] * r * w[k] with r = 1 / sqrt(mean_k v[k]^2 + eps).
    ms = RN32(exact sum_k v^2 / K); r = RN32(1 / sqrt(RN32(ms + eps))) with the
    square root and the division taken in float64.
N3  normalise, then quantise: u[k] = RN32(RN32(v[k] * r) * w[k]) (the row scaled
    by r, then by the norm weight, each product rounded to fp32), and u is the
    layer's input: xq, d = O4(u).

Lookup-table contraction ([JJ] juejin.cn, "微软 BitNet：让百亿参数大模型在 CPU
上飞起来", technical principles, item 2 "查表法优化": bitnet.cpp's kernels use
T-MAC's lookup-table method, turning the matrix product into table lookups;
[DT] section 3.2 names the lookup-table kernel types TL1 and TL2):
L1  per token, every pair of activations (x[2g], x[2g+1]) gets a table of 16
    partial sums T[g][c0 + 4*c1] = (c0 - 1)*x[2g] + (c1 - 1)*x[2g+1] over the
    2-bit codes c0, c1 in 0..3, so a nibble of the 2-bit layout (two weights)
    is the index; acc[m, n] = sum_g T[m][g][nibble g of row n].  The method
    reaches the same integers as O5.

Denser packing ([OV] introduction and section 2: a ternary weight carries
log2(3) ~ 1.58 bits of information; [CM] comparison table: 0.4 GB of
non-embedding memory for the 2B model, i.e. about 1.6 bits per weight):
T1  five ternary codes per byte (3**5 = 243 <= 256, so 1.6 bits per weight).
    The codes c_j = q_j + 1 are the base-3 digits of b = sum_j c_j * 3**j, and
    the byte holds b / 243 = 0.c4 c3 c2 c1 c0 (base 3) as an 8-bit fixed-point
    fraction rounded up: byte = ceil(256 * b / 243) (so b = floor(243 * byte /
    256); 13 byte values are never written).  A row is padded with q = 0 to a
    multiple of 80 weights and cut into blocks of 80 weights in 16 bytes: byte i
    (0..15) of block b holds the weights k = 80*b + 16*j + i as digit j
    (j = 0..4).  Row n occupies bytes [n*R, (n+1)*R), R = 16*ceil(K/80).  The
    pages describe no such format; this layout is ours (each digit j of a
    block's 16 bytes covers 16 consecutive weights, and a digit falls out of
    the fixed-point fraction as the integer part of three times it).

Prefill weight layout (the same 2-bit codes as O3, rearranged once for the
matrix-core kernel; the pages describe only CPU layouts, [DT] section 2.3):
P1  rows are padded with q = 0 to a multiple of 32 and K to a multiple of 128.
    The matrix is cut into blocks of 32 rows x 128 k, 1024 bytes each, stored
    block-row-major: block (rb, s) at byte (rb * S + s) * 1024, S = K_pad / 128.
    In a block, 16-byte chunk L = r + 32 h (r = 0..31, h = 0, 1) holds row
    32 rb + r at k = 128 s + 64 h + 0..63; its dword j holds the 16 weights
    k = 128 s + 64 h + 16 j + t (t = 0..15), the code c = q + 1 of weight t at
    bits 8 (t mod 4) + 2 (t div 4) (byte t mod 4, bit pair t div 4: O3's byte
    and bit-pair roles swapped within each dword).

bf16 inputs are upcast to fp32 exactly (bit pattern shifted left by 16) before
any step, so every function here takes fp32 arrays.

Parity pins: every function below is checked in tests/test_oracle_pins.py
against values that do not come from this module (hand-worked examples in
tests/golden/, Python ``fractions`` exact arithmetic, numpy's IEEE fp32
division, torch's fp32->bf16 conversion, brute-force enumeration of all
ternary rows, the Gaussian closed form of the zero fraction, and invariants).
"""

from __future__ import annotations

import math

import numpy as np

F32 = np.float32
EPS = F32(1e-5)          # RN32(1e-5): the floor of both scales (readings O1, O4)
QB = F32(127.0)          # symmetric int8 activation range (reading O4)
_FLT_MAX_UNITS_EXP = 104  # largest finite fp32 = (2**24 - 1) * 2**104


# ---------------------------------------------------------------------------
# bf16 <-> fp32 bit helpers (bf16 held as uint16 bit patterns)
# ---------------------------------------------------------------------------

def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns (uint16) to fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_bf16_bits(y: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits.

    A finite value keeps its top 16 bits after adding half of the dropped
    field's range, with the kept field's lowest bit deciding exact ties.
    NaN stays a quiet NaN with its sign.
    """
    y = np.ascontiguousarray(y, dtype=np.float32)
    u = y.view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(y)
    if nan.any():
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint16)
        r = np.where(nan, sign | np.uint16(0x7FC0), r)
    return r


# ---------------------------------------------------------------------------
# O1: exact absolute-mean weight scale
# ---------------------------------------------------------------------------

def exact_abs_sum_units(w: np.ndarray):
    """Exact sum of |w| over fp32 ``w``, as an integer count of 2**-149 units.

    Every finite fp32 value is an integer multiple of 2**-149 (the subnormal
    spacing): a normal value with biased exponent e and fraction f equals
    (2**23 + f) * 2**(e - 1) units, a subnormal equals f units.  The 24-bit
    significands are summed per exponent, split into two 12-bit halves so that
    every partial sum is an integer below 4096 * 2**38 < 2**53; numpy's bincount
    adds them in float64, where such integers and their sums are exact.  The
    per-exponent sums are combined in Python integers, so no rounding occurs
    anywhere.  Needs fewer than 2**38 elements.  Returns None if any element is
    Inf or NaN.
    """
    bits = np.ascontiguousarray(w, dtype=np.float32).reshape(-1).view(np.uint32)
    if bits.size >= (1 << 38):
        raise ValueError("exact sum supports fewer than 2**38 elements")
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.intp)
    if np.any(e == 0xFF):
        return None
    frac = bits & np.uint32(0x7FFFFF)
    mant = np.where(e > 0, frac | np.uint32(1 << 23), frac)
    hi = np.bincount(e, weights=(mant >> np.uint32(12)).astype(np.float64), minlength=256)
    lo = np.bincount(e, weights=(mant & np.uint32(0xFFF)).astype(np.float64), minlength=256)
    total = 0
    for ex in range(255):
        part = (int(hi[ex]) << 12) + int(lo[ex])
        total += part << (ex - 1 if ex > 0 else 0)
    return total


def rn32_ratio(num: int, den: int) -> np.float32:
    """Round the non-negative rational num/den to fp32, ties to even.

    Exact integer arithmetic: choose the power of two 2**e that puts the
    quotient's integer part q in [2**23, 2**24) (or e = -149 in the subnormal
    range), then round q using the remainder.
    """
    if num < 0 or den <= 0:
        raise ValueError("rn32_ratio needs num >= 0 and den > 0")
    if num == 0:
        return F32(0.0)
    e = num.bit_length() - den.bit_length() - 24
    while True:
        n2, d2 = (num, den << e) if e >= 0 else (num << -e, den)
        q, r = divmod(n2, d2)
        if q >= (1 << 24):
            e += 1
        elif q < (1 << 23):
            e -= 1
        else:
            break
    if e < -149:                      # below 2**-126: fixed subnormal spacing
        e = -149
        n2, d2 = num << 149, den
        q, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and (q & 1)):
        q += 1
    if q == (1 << 24):                # rounding carried into the next binade
        q >>= 1
        e += 1
    if e > _FLT_MAX_UNITS_EXP:
        return F32(np.inf)
    return F32(math.ldexp(q, e))


def weight_scale(w: np.ndarray) -> np.float32:
    """gamma* per reading O1 ([OV] section 2: divide by the mean absolute value).

    gamma = RN32(exact sum|W| / (N*K)); gamma* = max(gamma, RN32(1e-5)).
    NaN if W holds any Inf or NaN.
    """
    count = int(np.asarray(w).size)
    if count == 0:
        raise ValueError("weight_scale needs at least one weight")
    units = exact_abs_sum_units(w)
    if units is None:
        return F32(np.nan)
    gamma = rn32_ratio(units, count << 149)
    return gamma if gamma > EPS else EPS


# ---------------------------------------------------------------------------
# O2 / O3: ternarise and pack
# ---------------------------------------------------------------------------

def ternarize(w: np.ndarray, gamma: np.float32) -> np.ndarray:
    """q = clip(rne(RN32(w / gamma)), -1, 1) as int8 ([OV] section 2: round, clip)."""
    t = np.ascontiguousarray(w, dtype=np.float32) / F32(gamma)
    return np.clip(np.rint(t), -1.0, 1.0).astype(np.int8)


def pack_codes(q: np.ndarray) -> np.ndarray:
    """Pack ternary q [N, K] into uint8 [N, K/4] per reading O3 ([DT] section 2.3).

    Byte j of row n holds codes q[n, 4j + i] + 1 at bits 2i..2i+1.
    """
    q = np.asarray(q, dtype=np.int8)
    n_rows, k = q.shape
    if k % 4:
        raise ValueError("K must be a multiple of 4")
    codes = (q.astype(np.int16) + 1).astype(np.uint8).reshape(n_rows, k // 4, 4)
    out = np.zeros((n_rows, k // 4), dtype=np.uint8)
    for i in range(4):
        out |= codes[:, :, i] << np.uint8(2 * i)
    return out


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_codes: uint8 [N, K/4] -> int8 q [N, K].  Code 3 is invalid."""
    p = np.asarray(packed, dtype=np.uint8)
    n_rows, kb = p.shape
    codes = np.empty((n_rows, kb, 4), dtype=np.uint8)
    for i in range(4):
        codes[:, :, i] = (p >> np.uint8(2 * i)) & np.uint8(3)
    if np.any(codes == 3):
        raise ValueError("packed weights hold the unused code 3")
    return (codes.astype(np.int8) - 1).reshape(n_rows, 4 * kb)


def quantize_weights(w: np.ndarray):
    """Readings O1-O3 in sequence: returns (packed uint8 [N, K/4], gamma*).

    If W holds a non-finite value, gamma* is NaN and packed is None.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    gamma = weight_scale(w)
    if not np.isfinite(gamma):
        return None, gamma
    return pack_codes(ternarize(w, gamma)), gamma


# ---------------------------------------------------------------------------
# O4: per-token absmax int8 activations ([CM] quantisation details: A8)
# ---------------------------------------------------------------------------

def quantize_acts(x: np.ndarray):
    """Per token m: a = max|x|, a* = max(a, eps), s = RN32(127/a*),
    xq = clip(rne(RN32(x*s)), -128, 127), d = RN32(a*/127).

    Returns (xq int8 [M, K], d fp32 [M]).  Activations must be finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    m_rows, k = x.shape
    a = np.abs(x).max(axis=1) if k > 0 else np.zeros(m_rows, dtype=np.float32)
    a_star = np.maximum(a, EPS)
    s = QB / a_star
    xq = np.clip(np.rint(x * s[:, None]), -128.0, 127.0).astype(np.int8)
    d = (a_star / QB).astype(np.float32)
    return xq, d


# ---------------------------------------------------------------------------
# O5: exact integer contraction ([DT] section 3.1)
# ---------------------------------------------------------------------------

def integer_matmul(q: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[n, k] * xq[m, k] in exact integers -> int32 [M, N].

    The product is taken by the float64 matrix product (a library routine): every
    term q * xq is an integer of magnitude <= 128 and every partial sum an integer
    of magnitude <= 128 K, so while 128 K < 2**53 each intermediate is an exactly
    representable integer and the result is the exact sum in any summation order.
    Beyond that bound (never reached by the layer's K), numpy's int64 product."""
    q = np.asarray(q)
    xq = np.asarray(xq)
    if 128 * q.shape[1] < 2 ** 53:
        acc = np.rint(xq.astype(np.float64) @ q.astype(np.float64).T).astype(np.int64)
    else:
        acc = xq.astype(np.int64) @ q.astype(np.int64).T
    if acc.size and np.abs(acc).max() >= 2 ** 31:
        raise OverflowError("accumulator leaves the int32 range")
    return acc.astype(np.int32)


def sum_pos_minus_sum_neg(q_row: np.ndarray, x_row: np.ndarray) -> int:
    """The pages' form of one output ([DT] section 3.1): the sum of the inputs
    met by +1 weights minus the sum of the inputs met by -1 weights."""
    q_row = np.asarray(q_row)
    x_row = np.asarray(x_row, dtype=np.int64)
    return int(x_row[q_row == 1].sum()) - int(x_row[q_row == -1].sum())


# ---------------------------------------------------------------------------
# O6: rescale to fp32 / bf16
# ---------------------------------------------------------------------------

def dequantize(acc: np.ndarray, gamma: np.float32, d: np.ndarray) -> np.ndarray:
    """y[m, n] = RN32(float(acc[m, n]) * RN32(gamma* * d[m])) as fp32 [M, N]."""
    scale = (F32(gamma) * np.asarray(d, dtype=np.float32)).astype(np.float32)
    return np.asarray(acc, dtype=np.int32).astype(np.float32) * scale[:, None]


def ternary_linear(packed: np.ndarray, gamma: np.float32, xq: np.ndarray,
                   d: np.ndarray):
    """Whole layer on pre-quantised inputs: returns (acc int32 [M, N], y fp32 [M, N])."""
    q = unpack_codes(packed)
    acc = integer_matmul(q, xq)
    return acc, dequantize(acc, gamma, d)


def ternary_linear_at(packed: np.ndarray, gamma: np.float32, xq: np.ndarray,
                      d: np.ndarray, m_idx, n_idx):
    """Selected outputs only: acc and y at the pairs (m_idx[i], n_idx[i])."""
    m_idx = np.asarray(m_idx, dtype=np.int64)
    n_idx = np.asarray(n_idx, dtype=np.int64)
    q_rows = unpack_codes(np.asarray(packed)[n_idx]).astype(np.int64)
    x_rows = np.asarray(xq)[m_idx].astype(np.int64)
    acc = (q_rows * x_rows).sum(axis=1)
    if acc.size and np.abs(acc).max() >= 2 ** 31:
        raise OverflowError("accumulator leaves the int32 range")
    acc = acc.astype(np.int32)
    scale = (F32(gamma) * np.asarray(d, dtype=np.float32)[m_idx]).astype(np.float32)
    return acc, acc.astype(np.float32) * scale


# ---------------------------------------------------------------------------
# N1-N3: the layer's neighbours fused into its input ([CM] architecture item)
# ---------------------------------------------------------------------------

def relu2_glu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """N1: u = RN32(RN32(a * a) * up) with a = max(gate, 0), all fp32."""
    a = np.maximum(np.asarray(gate, dtype=np.float32), F32(0.0))
    return ((a * a).astype(np.float32) * np.asarray(up, dtype=np.float32)).astype(np.float32)


def exact_square_sum_units(v: np.ndarray) -> int:
    """Exact sum of v**2 over fp32 ``v`` as an integer count of 2**-298 units.

    v = m * 2**(e - 150) for a normal value (m the 24-bit significand, e the
    biased exponent), m * 2**-149 for a subnormal, so v**2 = m**2 * 2**(2e - 300)
    (normal) or m**2 * 2**-298 (subnormal).  m**2 < 2**48 is split into two
    24-bit halves that numpy sums exactly in float64 per exponent; the
    per-exponent sums are combined in Python integers.  Needs fewer than 2**29
    elements and finite values.
    """
    bits = np.ascontiguousarray(v, dtype=np.float32).reshape(-1).view(np.uint32)
    if bits.size >= (1 << 29):
        raise ValueError("exact square sum supports fewer than 2**29 elements")
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.intp)
    if np.any(e == 0xFF):
        raise ValueError("exact square sum needs finite values")
    frac = (bits & np.uint32(0x7FFFFF)).astype(np.uint64)
    mant = np.where(e > 0, frac | np.uint64(1 << 23), frac)
    sq = mant * mant
    hi = np.bincount(e, weights=(sq >> np.uint64(24)).astype(np.float64), minlength=256)
    lo = np.bincount(e, weights=(sq & np.uint64(0xFFFFFF)).astype(np.float64), minlength=256)
    total = 0
    for ex in range(255):
        part = (int(hi[ex]) << 24) + int(lo[ex])
        total += part << (2 * ex - 2 if ex > 0 else 0)
    return total


def mean_of_squares(v: np.ndarray) -> np.ndarray:
    """N2: per row, ms = RN32(exact sum v^2 / K) (one rounding of the exact mean)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    m_rows, k = v.shape
    return np.array([rn32_ratio(exact_square_sum_units(v[m]), k << 298) for m in range(m_rows)],
                    dtype=np.float32)


def rms_factor(v: np.ndarray, eps: float) -> np.ndarray:
    """N2: per row, r = RN32(1 / sqrt(RN32(ms + eps))), the root and division in float64."""
    eps32 = F32(eps)
    ms = mean_of_squares(v)
    return np.array([F32(1.0 / math.sqrt(float(F32(m + eps32)))) for m in ms], dtype=np.float32)


def rms_normalise(v: np.ndarray, norm_weight: np.ndarray, eps: float) -> np.ndarray:
    """N2-N3: u = RN32(RN32(v * r) * w) per row, r = rms_factor(v, eps)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    r = rms_factor(v, eps)
    n = (v * r[:, None]).astype(np.float32)
    return (n * np.asarray(norm_weight, dtype=np.float32)[None, :]).astype(np.float32)


def prologue_quantize_acts(x: np.ndarray, up=None, norm_weight=None, eps: float = 1e-5):
    """The layer input after its neighbours, quantised (N1-N3, then O4).

    x is the layer input, or the gate projection when ``up`` is given (N1);
    with ``norm_weight`` the input is RMS-normalised and scaled by the weight
    (N2, N3) before the per-token quantisation.  Returns (xq int8 [M, K], d fp32 [M]).
    """
    v = np.ascontiguousarray(x, dtype=np.float32)
    if up is not None:
        v = relu2_glu(v, up)
    if norm_weight is not None:
        v = rms_normalise(v, norm_weight, eps)
    return quantize_acts(v)


# ---------------------------------------------------------------------------
# T1: five ternary codes per byte (base 3)
# ---------------------------------------------------------------------------

T1_BLOCK_WEIGHTS = 80   # weights per block
T1_BLOCK_BYTES = 16     # bytes per block
T1_DIGITS = 5           # base-3 digits per byte


def t1_row_bytes(k: int) -> int:
    """Bytes of one packed row of K weights: 16 * ceil(K / 80)."""
    return T1_BLOCK_BYTES * ((k + T1_BLOCK_WEIGHTS - 1) // T1_BLOCK_WEIGHTS)


def pack_t1(q: np.ndarray) -> np.ndarray:
    """Pack ternary q [N, K] into uint8 [N, 16*ceil(K/80)] per reading T1.

    Byte i of block b of row n = ceil(256 * v / 243) with
    v = sum_j (q[n, 80b + 16j + i] + 1) * 3**j and q = 0 for the padding
    weights k >= K.
    """
    q = np.asarray(q, dtype=np.int8)
    n_rows, k = q.shape
    blocks = (k + T1_BLOCK_WEIGHTS - 1) // T1_BLOCK_WEIGHTS
    codes = np.ones((n_rows, blocks * T1_BLOCK_WEIGHTS), dtype=np.int64)  # padding: code 1
    codes[:, :k] = q.astype(np.int64) + 1
    codes = codes.reshape(n_rows, blocks, T1_DIGITS, T1_BLOCK_BYTES)   # [n][b][j][i]
    value = np.zeros((n_rows, blocks, T1_BLOCK_BYTES), dtype=np.int64)
    for j in range(T1_DIGITS):
        value += codes[:, :, j, :] * 3 ** j
    byte = -((-256 * value) // 243)                          # ceil(256 v / 243)
    return byte.reshape(n_rows, blocks * T1_BLOCK_BYTES).astype(np.uint8)


def unpack_t1(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of pack_t1: uint8 [N, 16*ceil(K/80)] -> int8 q [N, K].

    The base-3 value of a byte is v = floor(243 * byte / 256); a byte that is
    not ceil(256 * v / 243) of its own v, and non-zero padding weights, are
    invalid.
    """
    p = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    n_rows, row_bytes = p.shape
    if row_bytes != t1_row_bytes(k):
        raise ValueError("row length does not match K")
    value = (243 * p) // 256
    if np.any(-((-256 * value) // 243) != p):
        raise ValueError("byte is not the encoding of a base-3 value")
    blocks = row_bytes // T1_BLOCK_BYTES
    rest = value.reshape(n_rows, blocks, T1_BLOCK_BYTES)
    codes = np.empty((n_rows, blocks, T1_DIGITS, T1_BLOCK_BYTES), dtype=np.int64)
    for j in range(T1_DIGITS):
        codes[:, :, j, :] = rest % 3
        rest = rest // 3
    q = (codes - 1).reshape(n_rows, blocks * T1_BLOCK_WEIGHTS)
    if np.any(q[:, k:] != 0):
        raise ValueError("padding weights must be zero")
    return q[:, :k].astype(np.int8)


def quantize_weights_t1(w: np.ndarray):
    """Readings O1, O2 and T1: returns (packed uint8 [N, 16*ceil(K/80)], gamma*).

    If W holds a non-finite value, gamma* is NaN and packed is None.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    gamma = weight_scale(w)
    if not np.isfinite(gamma):
        return None, gamma
    return pack_t1(ternarize(w, gamma)), gamma


def ternary_linear_t1(packed: np.ndarray, gamma: np.float32, xq: np.ndarray,
                      d: np.ndarray):
    """ternary_linear on T1-packed weights: returns (acc int32 [M, N], y fp32 [M, N])."""
    q = unpack_t1(packed, np.asarray(xq).shape[1])
    acc = integer_matmul(q, xq)
    return acc, dequantize(acc, gamma, d)


def ternary_linear_t1_at(packed: np.ndarray, gamma: np.float32, xq: np.ndarray,
                         d: np.ndarray, m_idx, n_idx):
    """Selected outputs of ternary_linear_t1: acc and y at the pairs (m_idx[i], n_idx[i])."""
    m_idx = np.asarray(m_idx, dtype=np.int64)
    n_idx = np.asarray(n_idx, dtype=np.int64)
    q_rows = unpack_t1(np.asarray(packed)[n_idx], np.asarray(xq).shape[1]).astype(np.int64)
    x_rows = np.asarray(xq)[m_idx].astype(np.int64)
    acc = (q_rows * x_rows).sum(axis=1).astype(np.int32)
    scale = (F32(gamma) * np.asarray(d, dtype=np.float32)[m_idx]).astype(np.float32)
    return acc, acc.astype(np.float32) * scale


# ---------------------------------------------------------------------------
# P1: prefill weight layout (32-row x 128-k blocks, bit pairs transposed per dword)
# ---------------------------------------------------------------------------

P1_ROWS = 32            # rows per block
P1_K = 128              # weights per block row
P1_BLOCK_BYTES = 1024   # bytes per block


def prefill_layout_bytes(n: int, k: int) -> int:
    """Bytes of an N x K matrix in the P1 layout: ceil(N/32) * ceil(K/128) * 1024."""
    return (-(-n // P1_ROWS)) * (-(-k // P1_K)) * P1_BLOCK_BYTES


def pack_prefill(q: np.ndarray) -> np.ndarray:
    """Ternary q [N, K] -> uint8 [prefill_layout_bytes(N, K)] per reading P1."""
    q = np.asarray(q, dtype=np.int8)
    n_rows, k = q.shape
    nb, sb = -(-n_rows // P1_ROWS), -(-k // P1_K)
    codes = np.ones((nb * P1_ROWS, sb * P1_K), dtype=np.uint32)     # padding: q = 0
    codes[:n_rows, :k] = (q.astype(np.int16) + 1).astype(np.uint32)
    # [rb][r][s][h][j][t]: block rb, row r, step s, half h, dword j, weight t
    c = codes.reshape(nb, P1_ROWS, sb, 2, 4, 16)
    words = np.zeros((nb, P1_ROWS, sb, 2, 4), dtype=np.uint32)
    for t in range(16):
        words |= c[..., t] << np.uint32(8 * (t % 4) + 2 * (t // 4))
    # chunk L = r + 32 h of block (rb, s): order [rb][s][h][r][j]
    out = words.transpose(0, 2, 3, 1, 4).reshape(-1)
    return out.astype("<u4").view(np.uint8)


def unpack_prefill(packed: np.ndarray, n: int, k: int) -> np.ndarray:
    """Inverse of pack_prefill: uint8 [prefill_layout_bytes(N, K)] -> q [N, K].
    Code 3 and non-zero padding weights are invalid."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    if p.size != prefill_layout_bytes(n, k):
        raise ValueError("size does not match N and K")
    nb, sb = -(-n // P1_ROWS), -(-k // P1_K)
    words = p.view("<u4").astype(np.uint32).reshape(nb, sb, 2, P1_ROWS, 4)
    words = words.transpose(0, 3, 1, 2, 4)                      # [rb][r][s][h][j]
    codes = np.empty(words.shape + (16,), dtype=np.uint32)
    for t in range(16):
        codes[..., t] = (words >> np.uint32(8 * (t % 4) + 2 * (t // 4))) & np.uint32(3)
    if np.any(codes == 3):
        raise ValueError("packed weights hold the unused code 3")
    q = (codes.astype(np.int16) - 1).reshape(nb * P1_ROWS, sb * P1_K)
    if np.any(q[n:, :]) or np.any(q[:, k:]):
        raise ValueError("padding weights must be zero")
    return q[:n, :k].astype(np.int8)


def repack_prefill(packed: np.ndarray, k: int) -> np.ndarray:
    """O3 layout [N, K/4] -> P1 layout (the same codes)."""
    return pack_prefill(unpack_codes(packed)[:, :k])


def ternary_linear_prefill(packed_p1: np.ndarray, n: int, gamma: np.float32, xq: np.ndarray,
                           d: np.ndarray):
    """ternary_linear on P1-laid-out weights: returns (acc int32 [M, N], y fp32 [M, N])."""
    q = unpack_prefill(packed_p1, n, np.asarray(xq).shape[1])
    acc = integer_matmul(q, xq)
    return acc, dequantize(acc, gamma, d)


# ---------------------------------------------------------------------------
# L1: lookup-table contraction
# ---------------------------------------------------------------------------

def lut_tables(xq: np.ndarray) -> np.ndarray:
    """L1 tables: int64 [M, K/2, 16], entry c0 + 4*c1 of pair g of token m is
    (c0 - 1) * xq[m, 2g] + (c1 - 1) * xq[m, 2g + 1].  K must be even."""
    x = np.asarray(xq, dtype=np.int64)
    if x.shape[1] % 2:
        raise ValueError("K must be even")
    idx = np.arange(16)
    q0 = (idx & 3) - 1
    q1 = (idx >> 2) - 1
    return q0[None, None, :] * x[:, 0::2, None] + q1[None, None, :] * x[:, 1::2, None]


def lut_linear(packed: np.ndarray, gamma: np.float32, xq: np.ndarray, d: np.ndarray):
    """The layer by table lookup (L1): one lookup per nibble (pair of weights) of
    the 2-bit layout.  Returns (acc int32 [M, N], y fp32 [M, N])."""
    p = np.asarray(packed, dtype=np.uint8)
    n_rows, kb = p.shape
    nib = np.empty((n_rows, 2 * kb), dtype=np.int64)
    nib[:, 0::2] = p & 15          # weights 4j, 4j+1 -> pair 2j
    nib[:, 1::2] = p >> 4          # weights 4j+2, 4j+3 -> pair 2j+1
    tables = lut_tables(xq)
    acc = np.empty((tables.shape[0], n_rows), dtype=np.int64)
    pairs = np.arange(2 * kb)
    for m in range(tables.shape[0]):
        acc[m] = tables[m][pairs[None, :], nib].sum(axis=1)
    if acc.size and np.abs(acc).max() >= 2 ** 31:
        raise OverflowError("accumulator leaves the int32 range")
    acc = acc.astype(np.int32)
    return acc, dequantize(acc, gamma, d)


def quant_linear(packed: np.ndarray, gamma: np.float32, x: np.ndarray):
    """Act-quant followed by the layer: returns (xq, d, acc, y)."""
    xq, d = quantize_acts(x)
    acc, y = ternary_linear(packed, gamma, xq, d)
    return xq, d, acc, y
