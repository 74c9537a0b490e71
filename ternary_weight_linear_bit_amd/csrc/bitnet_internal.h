// Internal declarations shared by the HIP translation units of libbitnet_mi355x.
// Not part of the public ABI (include/bitnet_mi355x.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr float kEps = 1e-5f;   // floor of both scales; the literal rounds to RN32(1e-5)
constexpr float kQb = 127.0f;   // symmetric int8 activation range

// Exact bf16 -> fp32 upcast.
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN -> quiet NaN with its sign.
__device__ __forceinline__ uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> bf16 (round to nearest, ties to even) in one gfx950 conversion
// (v_cvt_pk_bf16_f32): lo in bits 0-15, hi in bits 16-31.  Bit-identical to
// float_to_bf16_rne for every non-NaN input (all 2^32 fp32 bit patterns compared
// on gfx950); a NaN keeps payload bits instead of becoming sign | 0x7fc0.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Wave64 reductions (butterfly over all 64 lanes).
// Wave-wide reductions on DPP: quad permutes and the two row mirrors make every
// lane of a 16-lane row hold the row's result; row broadcasts 15 and 31 (rows
// 1 and 3, then rows 2 and 3) carry it into lane 63, which is read back as a
// wave-uniform scalar.  A few vector instructions, where a shuffle tree costs
// six round trips through the LDS crossbar.  Every lane must be active; lanes
// a broadcast does not reach keep the identity (zero) as their operand.
#define BITNET_DPP(old, v, ctrl, rows) __builtin_amdgcn_update_dpp((old), (v), (ctrl), (rows), 0xF, false)
// max over the wave of non-negative values
__device__ __forceinline__ float wave_max(float v) {
  int b = __float_as_int(v);
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(BITNET_DPP(0, b, 0xB1, 0xF))));   // lane ^ 1
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(BITNET_DPP(0, b, 0x4E, 0xF))));   // lane ^ 2
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(BITNET_DPP(0, b, 0x141, 0xF))));  // half-row mirror
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(BITNET_DPP(0, b, 0x140, 0xF))));  // row mirror
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(BITNET_DPP(0, b, 0x142, 0xA))));  // row bcast 15
  b = __float_as_int(fmaxf(__int_as_float(b), __int_as_float(BITNET_DPP(0, b, 0x143, 0xC))));  // row bcast 31
  return __int_as_float(__builtin_amdgcn_readlane(b, 63));
}
// sum over the wave (fp64, both halves moved by DPP)
__device__ __forceinline__ double wave_sum_f64(double v) {
  auto step = [](double x, double y) { return x + y; };
#define BITNET_DPP_F64(ctrl, rows)                                                        \
  {                                                                                       \
    const uint64_t u = (uint64_t)__double_as_longlong(v);                                 \
    const uint32_t lo = (uint32_t)BITNET_DPP(0, (int)(uint32_t)u, ctrl, rows);            \
    const uint32_t hi = (uint32_t)BITNET_DPP(0, (int)(uint32_t)(u >> 32), ctrl, rows);    \
    v = step(v, __longlong_as_double((long long)(((uint64_t)hi << 32) | lo)));            \
  }
  BITNET_DPP_F64(0xB1, 0xF)
  BITNET_DPP_F64(0x4E, 0xF)
  BITNET_DPP_F64(0x141, 0xF)
  BITNET_DPP_F64(0x140, 0xF)
  BITNET_DPP_F64(0x142, 0xA)
  BITNET_DPP_F64(0x143, 0xC)
#undef BITNET_DPP_F64
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
#undef BITNET_DPP
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 4x4 byte transpose of four dwords: out[i].byte[b] = in[b].byte[i], as eight
// byte permutes (v_perm: selector bytes 0-3 pick from the second operand, 4-7
// from the first).
__device__ __forceinline__ void transpose4x4_bytes(const uint32_t in[4], uint32_t out[4]) {
  const uint32_t t0 = __builtin_amdgcn_perm(in[1], in[0], 0x05010400u);  // in0.b0 in1.b0 in0.b1 in1.b1
  const uint32_t t1 = __builtin_amdgcn_perm(in[1], in[0], 0x07030602u);  // in0.b2 in1.b2 in0.b3 in1.b3
  const uint32_t t2 = __builtin_amdgcn_perm(in[3], in[2], 0x05010400u);
  const uint32_t t3 = __builtin_amdgcn_perm(in[3], in[2], 0x07030602u);
  out[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
  out[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
  out[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
  out[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
}

// One packed dword (codes of k-offsets 0..15, byte b holding 4b..4b+3) -> the
// 16-byte operand whose byte 4i + b is the weight q = c - 1 of k-offset 4b + i.
// Each field is isolated with a mask and mapped through a byte lookup (v_perm:
// selector byte c picks byte c of kCodeLut: 0 -> -1, 1 -> 0, 2 -> +1).
constexpr uint32_t kCodeLut = 0x000100ffu;
__device__ __forceinline__ v4i unpack_weights_transposed(uint32_t w) {
  v4i a;
  a.x = (int)__builtin_amdgcn_perm(0u, kCodeLut, w & 0x03030303u);
  a.y = (int)__builtin_amdgcn_perm(0u, kCodeLut, (w >> 2) & 0x03030303u);
  a.z = (int)__builtin_amdgcn_perm(0u, kCodeLut, (w >> 4) & 0x03030303u);
  a.w = (int)__builtin_amdgcn_perm(0u, kCodeLut, (w >> 6) & 0x03030303u);
  return a;
}

// Stage one 16-byte group of int8 activations in the unpacked weights' k order.
__device__ __forceinline__ void store_transposed(uint8_t* dst, uint4 v) {
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
  transpose4x4_bytes(in, o);
  *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
}

// The code clip(rne(RN32(x * s)), -128, 127) of activation x with the token's
// factor s = RN32(127 / a*), in the low byte of the bits of RN32(t + 1.5 * 2^23),
// t = RN32(x * s): the sum lies in [2^23, 2^24), where the floats are the
// integers, so the addition rounds t to the nearest integer, ties to even
// (1.5 * 2^23 is even), and the low mantissa byte is that integer mod 256, its
// int8 bit pattern.  For finite inputs |x| <= a*, so |t| <= 127 (1 + 2^-24)
// and the clip never acts.  (Two instructions per value; rounding, clamping
// and converting took four, and the packing two more.)
constexpr float kRneMagic = 12582912.0f;   // 1.5 * 2^23
__device__ __forceinline__ uint32_t rne_bits(float x, float s) {
  const float t = x * s;
  return __float_as_uint(t + kRneMagic);
}

// The low bytes of four dwords, a first, as one dword (three byte permutes)
__device__ __forceinline__ uint32_t low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);   // a.b0 b.b0 0 0
  const uint32_t hi = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);   // c.b0 d.b0 0 0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Quantise four activations (rne_bits), packed little-endian into one dword.
__device__ __forceinline__ uint32_t quant4(const float* v, float s) {
  return low_bytes(rne_bits(v[0], s), rne_bits(v[1], s), rne_bits(v[2], s), rne_bits(v[3], s));
}

// 16 consecutive fp32 or bf16 activations from a 16-byte aligned address
// (i16 counts groups of 16 elements).
template <bool BF16>
__device__ __forceinline__ void load16_act(const void* x, int64_t i16, float v[16]) {
  if (BF16) {
    const uint4* p = reinterpret_cast<const uint4*>(x) + 2 * i16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 a = p[h];
      const uint32_t d[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * h + 2 * j] = __uint_as_float(d[j] << 16);
        v[8 * h + 2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(x) + 4 * i16;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 a = p[h];
      v[4 * h] = a.x;
      v[4 * h + 1] = a.y;
      v[4 * h + 2] = a.z;
      v[4 * h + 3] = a.w;
    }
  }
}

// The 16 activations of one group from its raw 16-byte words (2 words of bf16 or
// 4 of fp32); bf16 -> fp32 is exact.
template <bool BF>
__device__ __forceinline__ void raw_to_f32(const uint4* w, float v[16]) {
  if (BF) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t d[4] = {w[h].x, w[h].y, w[h].z, w[h].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * h + 2 * j] = __uint_as_float(d[j] << 16);
        v[8 * h + 2 * j + 1] = __uint_as_float(d[j] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[4 * h] = __uint_as_float(w[h].x);
      v[4 * h + 1] = __uint_as_float(w[h].y);
      v[4 * h + 2] = __uint_as_float(w[h].z);
      v[4 * h + 3] = __uint_as_float(w[h].w);
    }
  }
}

// Raw buffer resource over [base, base + bytes).  Loads at offsets >= bytes
// return zeros (hardware range check), which pads ragged rows and tails without
// branches.  Word 3 selects 32-bit data format as gfx9 buffer loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
constexpr uint32_t kOob = 0x80000000u;  // an offset past every range used with make_rsrc

// make_rsrc for a base and size that are the same in every lane of the wave: the
// readfirstlanes keep the descriptor in scalar registers, so the loads need no
// per-lane legalisation loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_uniform_rsrc(const void* base,
                                                                    uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}
// The same, non-temporal (cache policy nt: data read once, first to be evicted).
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4i v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// A generic pointer as a global address-space pointer, so that accesses through
// it compile to global rather than flat instructions (flat ones also count as LDS
// traffic, which makes the compiler's waits conservative).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* as_global(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

// Wait for this wave's LDS operations, then workgroup barrier.  Unlike
// __syncthreads() this does not wait for outstanding global loads, so weight
// prefetches stay in flight across it; the "memory" clobber keeps the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Host-side launchers (one per kernel family); each returns a hipError_t from
// hipGetLastError() after its launches.
// Weight quantisation workspace: kWqCopies copies of the 256 exponent buckets
// (uint64) and the ternarisation threshold.
constexpr int kWqCopies = 8;
constexpr size_t kWqThresholdAt = (size_t)kWqCopies * 256 * 8;
constexpr size_t kWqWorkspaceBytes = kWqThresholdAt + 256;
hipError_t launch_wq(const void* w, bool w_bf16, int64_t n_weights, uint8_t* w_packed,
                     float* w_scale, void* workspace, hipStream_t s);
// The same with the library's own per-device workspace (a file-scope device array
// of kWqWorkspaceBytes): allocates nothing.
hipError_t launch_wq_noalloc(const void* w, bool w_bf16, int64_t n_weights, uint8_t* w_packed,
                             float* w_scale, hipStream_t s);
// The same scale with the T1 layout (five codes per byte, 16 * ceil(K / 80) bytes
// per row), and the exact conversion of a 2-bit packed matrix (K % 4 == 0) to it.
hipError_t launch_wq_t1(const void* w, bool w_bf16, int64_t N, int64_t K, uint8_t* w_t1,
                        float* w_scale, void* workspace, hipStream_t s);
hipError_t launch_repack_t1(const uint8_t* w_packed, int64_t N, int64_t K, uint8_t* w_t1,
                            hipStream_t s);
// Input prologue of a layer (squared-ReLU gating and RMS norm), already validated.
struct ActPrologue {
  const void* up;       // gating: up projection, same dtype and shape as x; else nullptr
  const float* w;       // RMS norm weight [K]; else nullptr
  float eps;
};

// Elementwise part of the prologue for one activation: the gated value
// v = RN32(RN32(a * a) * up) with a = max(x, 0) (or v = x), and the value that is
// quantised, RN32(v * w) (or v).  Two separate roundings; no fused multiply-add.
__device__ __forceinline__ float glu_value(float x, float up) {
  const float a = fmaxf(x, 0.0f);
  return __fmul_rn(__fmul_rn(a, a), up);
}

// --- RMS norm: the exactly rounded mean of squares ---------------------------
//
// ms = RN32(exact sum_k v_k^2 / K) for finite fp32 v (the reading of the norm:
// one rounding of the exact mean, so that it does not depend on the order in
// which a launch sums).  Fast path: the float64 sum ss of the squares (each
// square exact in float64), in any order, is within (K - 1) 2^-53 S of the exact
// sum S; when both ends of the widened interval [ss/K (1 - g), ss/K (1 + g)],
// g = (K + 4) 2^-52, round to the same fp32 value, that value is RN32(S / K)
// (rounding is monotonic).  Otherwise (the mean lies within about K 2^-53 of a
// rounding boundary: about one token in K^-1 2^28) the exact path below is
// taken.
__device__ __forceinline__ bool mean_sq_fast(double ss, int64_t K, float& ms) {
  const double m = ss / (double)K;
  const double g = (double)(K + 4) * 0x1p-52;
  const float lo = (float)(m * (1.0 - g));
  const float hi = (float)(m * (1.0 + g));
  ms = lo;
  return lo == hi;
}

// Exact path: S = sum v^2 as an integer count of 2^-298 units (v = m 2^(e-150)
// for a normal v with biased exponent e and 24-bit significand m, m 2^-149 for a
// sub-normal: v^2 = m^2 2^(P - 298), P = 2 (max(e, 1) - 1) in [0, 506]), kept in
// kSqLimbs carry-save limbs of 32-bit digits in LDS (limb i weighs 2^(32 i)).
// Every square adds three chunks of under 2^32 to three limbs, so a limb holds
// the chunks of up to 2^31 squares without overflow.
constexpr int kSqLimbs = 20;
__device__ __forceinline__ void sq_limbs_add(unsigned long long* limbs, float v) {
  const uint32_t b = __float_as_uint(v) & 0x7fffffffu;
  if (b == 0u) return;
  const uint32_t e = b >> 23;
  const uint64_t m = e ? ((b & 0x7fffffu) | 0x800000u) : (b & 0x7fffffu);
  const unsigned __int128 t = (unsigned __int128)(m * m) << ((2 * ((e ? e : 1u) - 1u)) & 31u);
  const int L = (int)((2 * ((e ? e : 1u) - 1u)) >> 5);
  atomicAdd(&limbs[L], (unsigned long long)(uint32_t)t);
  atomicAdd(&limbs[L + 1], (unsigned long long)(uint32_t)(t >> 32));
  atomicAdd(&limbs[L + 2], (unsigned long long)(t >> 64));
}

// RN32(S 2^-298 / K) from the limbs, by one thread, with kSqWork words of LDS as
// work space (kept out of private memory: indexed arrays there would give the
// kernel a scratch segment).  The limbs are normalised to 32-bit digits, shifted
// up by 64 bits (so the quotient has at least 47 bits) and divided by K from the
// top digit down; the quotient's leading 24 bits are rounded to nearest even with
// the next bit and a sticky bit (lower quotient bits or a nonzero remainder).
constexpr int kSqDigits = kSqLimbs + 2;   // digits of S * 2^64
constexpr int kSqWork = 2 * kSqDigits;
__device__ float sq_limbs_mean(const unsigned long long* limbs, int64_t K, uint32_t* work) {
  uint32_t* d = work;                // S * 2^64, little-endian 32-bit digits
  uint32_t* q = work + kSqDigits;    // the quotient
  d[0] = 0u;
  d[1] = 0u;
  unsigned long long carry = 0;
  for (int i = 0; i < kSqLimbs; ++i) {
    const unsigned long long v = limbs[i] + carry;
    d[i + 2] = (uint32_t)v;
    carry = v >> 32;
  }
  unsigned long long rem = 0;
  for (int i = kSqDigits - 1; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | d[i];
    q[i] = (uint32_t)(cur / (unsigned long long)K);
    rem = cur % (unsigned long long)K;
  }
  int top = kSqDigits - 1;
  while (top >= 0 && q[top] == 0u) --top;
  if (top < 0) return 0.0f;          // S / K below 2^-362: rounds to +0
  const int nq = 32 * top + (32 - __builtin_clz(q[top]));   // bits of the quotient
  auto bit = [&](int i) -> uint32_t { return i < 0 ? 0u : (q[i >> 5] >> (i & 31)) & 1u; };
  auto any_below = [&](int i) -> bool {   // any quotient bit below bit i
    if (i <= 0) return false;
    for (int w = 0; w < (i >> 5); ++w)
      if (q[w]) return true;
    return (i & 31) ? (q[i >> 5] & ((1u << (i & 31)) - 1u)) != 0u : false;
  };
  // value = q 2^-362 (+ a fraction below its last bit when rem != 0)
  int e2 = nq - 1 - 362;            // exponent of the leading bit
  const bool sub = e2 < -126;
  const int shift = sub ? 362 - 149 : nq - 24;   // sub-normal: fixed spacing 2^-149
  uint32_t sig = 0;
  for (int i = 23; i >= 0; --i) sig = (sig << 1) | bit(shift + i);
  const bool sticky = any_below(shift - 1) || rem != 0;
  if (bit(shift - 1) && (sticky || (sig & 1u))) ++sig;
  if (sub) return __uint_as_float(sig);   // sig <= 2^23: sub-normal or the least normal
  if (sig == (1u << 24)) {
    sig >>= 1;
    ++e2;
  }
  if (e2 > 127) return __uint_as_float(0x7f800000u);
  return __uint_as_float(((uint32_t)(e2 + 127) << 23) | (sig & 0x7fffffu));
}

// RMS norm factor from the exactly rounded mean of squares:
// r = RN32(1 / sqrt(RN32(ms + eps))), square root and division in float64.
__device__ __forceinline__ float rms_factor_of_mean(float ms, float eps) {
  const float t = __fadd_rn(ms, eps);
  return (float)(1.0 / sqrt((double)t));
}

// The value the layer quantises with a norm: RN32(RN32(v * r) * w).
__device__ __forceinline__ float norm_value(float v, float r, float w) {
  return __fmul_rn(__fmul_rn(v, r), w);
}

hipError_t launch_aq(const void* x, bool x_bf16, int64_t M, int64_t K, int8_t* x_q,
                     float* x_scale, const ActPrologue& pro, hipStream_t s);
// Decode kernel arguments: up to kMaxGroup weight matrices sharing K and the
// activations, passed by value.
constexpr int kMaxGroup = 4;
struct GemvArgs {
  const uint8_t* wp[kMaxGroup];
  const float* ws[kMaxGroup];
  void* y[kMaxGroup];
  int32_t* acc[kMaxGroup];
  int n[kMaxGroup];
  int wg0[kMaxGroup];        // first workgroup of each matrix (set by launch_gemv)
  const int8_t* xq;          // int8 activations (pre-quantised input)
  const float* xs;           // their token scales
  const void* xf;            // fp32/bf16 activations (fused quantisation) or nullptr
  int8_t* xq_out;            // fused: where x_q and x_scale are written
  float* xs_out;
  int count, unused0;
  int M, K;                  // pairs of ints are read as one 64-bit value each
  int y_bf16, tiles_per_wg;  // row tiles per workgroup (set by launch_gemv)
  int mdiv, unused1;         // ceil(65536 / M) (launch_gemv)
  const void* xup;           // fused prologue: up projection (gating) or nullptr
  const float* gnorm;        // fused prologue: RMS norm weight or nullptr
  float eps, unused2;
};

// Weight formats of the decode kernel: 2 bits per weight (K % 64 == 0), or five
// per byte (T1, K % 16 == 0, rows of 16 * ceil(K / 80) bytes).
constexpr int kFmt2 = 0, kFmtT1 = 1;
// Decode kernel: M <= 16 and K % 64 == 0 (fmt 0: 2-bit weights) or K % 16 == 0
// (fmt 1: T1 weights); the fused variant (a.xf != nullptr) also needs M <= 4 and
// the activations of all tokens in one LDS phase.
constexpr int kGemvMaxM = 16;
// K travels in 19 bits of a kernel argument (the linear calls accept K <= 2^17)
constexpr int64_t kGemvMaxK = (1 << 19) - 1;
bool gemv_fits(int64_t M, int64_t K, int fmt);
bool gemv_fused_fits(int64_t M, int64_t K, int fmt);
hipError_t launch_gemv(GemvArgs a, int xf_dtype, int fmt, hipStream_t s);
// Decode chain (one cooperative launch per token, chain.hip): the device-side
// descriptor of one stage, i.e. one fused act-quant + linear over up to
// kMaxGroup matrices that share the stage input.  Filled by bitnet_chain_plan.
struct ChainStage {
  const void* x;             // stage input [M][K], fp32 or bf16 (flags bit 0)
  int8_t* xq_out;            // the quantised input [M][K] and its token scales [M],
  float* xs_out;             //   written by workgroup 0
  const uint8_t* wp[kMaxGroup];
  const float* ws[kMaxGroup];
  void* y[kMaxGroup];        // outputs [M][N], fp32 or bf16 (flags bit 1)
  int32_t* acc[kMaxGroup];   // optional int32 accumulators [M][N]
  int n[kMaxGroup];
  int tc0[kMaxGroup + 1];    // first 16-row tile of each matrix in the stage's tile list;
                             //   tc0[count..] = all tiles (spread evenly over the grid)
  int K, count, flags;
};
constexpr int kChainMaxM = 4;
constexpr int kChainMaxTiles = 16;       // row tiles per workgroup and stage
constexpr int kChainThreads = 512;     // 4 streaming + 4 staging waves
constexpr size_t kChainHeaderBytes = 4096;  // barrier counters and the error word
constexpr int kChainGroups = 8;             // barrier groups (counter lines 0-7)
constexpr size_t kChainErrorAt = 256 * (kChainGroups + 2);  // byte offset of the error word
// LDS bytes of the chain kernel for M tokens, inputs up to kmax and up to tmax
// tiles per workgroup.
size_t chain_lds_bytes(int M, int kmax, int tmax);
// Bytes of a plan: header (counters), stage table.
size_t chain_plan_bytes(int n_stages);
// One token through every stage; grid = workgroups (all co-resident).
hipError_t launch_chain(const void* plan, int n_stages, int M, int grid, int kmax, int tmax,
                        int ring, hipStream_t s);
int chain_grid(int M, int kmax, int tmax, int ring);

// Prefill kernel arguments: up to kMaxGroup weight matrices sharing K and the
// int8 activations, passed by value.  launch_gemm fills nb0.
struct GemmArgs {
  const uint8_t* wp[kMaxGroup];
  const float* ws[kMaxGroup];
  void* y[kMaxGroup];
  int32_t* acc[kMaxGroup];
  int n[kMaxGroup];
  int ld[kMaxGroup];         // row stride of y and acc in elements (0: n)
  int nb0[kMaxGroup + 1];    // first row tile of each matrix; nb0[count] = all row tiles
  const int8_t* xq;          // int8 activations [M][K]
  const float* xs;           // their token scales
  int count, M, K, y_bf16;
  int layout;                // weights: 0 = rows of K/4 bytes, 1 = prefill layout
};
// Prefill kernel: K % 64 == 0, 16-byte aligned packed weights and activations.
hipError_t launch_gemm(GemmArgs a, hipStream_t s);
// Prefill layout: its size, and the conversion from rows of K/4 bytes (K % 64
// == 0, 16-byte aligned input and output).
int64_t prefill_layout_bytes(int64_t N, int64_t K);
hipError_t launch_repack_prefill(const uint8_t* w, int64_t N, int64_t K, uint8_t* out,
                                 hipStream_t s);
// The prefill launch's tile for M tokens over `count` matrices of n[j] rows on a
// device with `cus` compute units: bm tokens x bn rows per workgroup; when
// first_tokens > 0 the first first_tokens tokens run as one launch with this tile
// and the rest as a second launch planned on its own; when first_rows > 0, the
// first first_rows rows of the matrices taken in order (a multiple of bn) run as
// one launch with this tile and the remaining rows as a second launch planned on
// its own.
struct GemmPlan {
  int bm, bn;
  int64_t first_tokens;
  int64_t first_rows;
};
GemmPlan gemm_plan(int64_t M, const int* n, int count, int64_t K, int cus);
// Lookup-table decode: workspace bytes (tables 16 K + accumulators 4 N, each
// rounded up to 256) and the launches (three per token).  K % 64 == 0, 16-byte
// aligned packed weights and workspace.
size_t lut_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_lut(const uint8_t* wp, const float* w_scale, const int8_t* xq,
                      const float* x_scale, int64_t M, int64_t N, int64_t K, void* y,
                      bool y_bf16, int32_t* acc_out, void* workspace, int cus, hipStream_t s);
int device_cus();
hipError_t launch_generic_linear(const uint8_t* wp, const float* w_scale, const int8_t* xq,
                                 const float* x_scale, int64_t M, int64_t N, int64_t K,
                                 void* y, bool y_bf16, int32_t* acc_out, hipStream_t s);

}  // namespace bitnet
