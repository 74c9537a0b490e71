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

// Quantise four activations with the token's factor s = RN32(127 / a*):
// clip(rne(RN32(x * s)), -128, 127), packed little-endian into one dword.
__device__ __forceinline__ uint32_t quant4(const float* v, float s) {
  uint32_t out = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q = rintf(v[i] * s);
    q = fminf(fmaxf(q, -128.0f), 127.0f);
    out |= ((uint32_t)(int32_t)q & 0xffu) << (8 * i);
  }
  return out;
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

// RMS norm factor of a row from its float64 sum of squares ss over K values:
// r = RN32(1 / sqrt(RN32(RN32(ss / K) + eps))), square root and division in float64.
__device__ __forceinline__ float rms_factor(double ss, int64_t K, float eps) {
  const float ms = (float)(ss / (double)K);
  const float t = __fadd_rn(ms, eps);
  return (float)(1.0 / sqrt((double)t));
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
// Prefill kernel arguments: up to kMaxGroup weight matrices sharing K and the
// int8 activations, passed by value.  launch_gemm fills nb0.
struct GemmArgs {
  const uint8_t* wp[kMaxGroup];
  const float* ws[kMaxGroup];
  void* y[kMaxGroup];
  int32_t* acc[kMaxGroup];
  int n[kMaxGroup];
  int nb0[kMaxGroup + 1];    // first row tile of each matrix; nb0[count] = all row tiles
  const int8_t* xq;          // int8 activations [M][K]
  const float* xs;           // their token scales
  int count, M, K, y_bf16;
};
// Prefill kernel: K % 64 == 0, 16-byte aligned packed weights and activations.
hipError_t launch_gemm(GemmArgs a, hipStream_t s);
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
