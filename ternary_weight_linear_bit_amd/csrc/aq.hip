// Per-token absmax int8 activation quantisation, with the layer's optional input
// prologue (squared-ReLU gating, RMS norm).
//
// Method: communeify.com, "微軟 BitNet b1.58 震撼登場", section on BitNet b1.58
// 2B4T, quantisation details: activations are 8-bit integers (W1.58A8).  The pages
// give no scheme; the reading here is per token (row) absmax to the symmetric
// range [-127, 127]:  a* = max(max|x|, RN32(1e-5)), s = RN32(127/a*),
// xq = clip(rne(RN32(x*s)), -128, 127), d = RN32(a*/127).
// Prologue (same page, architecture item: ReLU^2 activation, subln norm, no
// biases): with gating the input is v = RN32(RN32(relu(x)^2) * up); with a norm
// weight w the row is normalised first, u = RN32(RN32(v * r) * w) with
// r = RN32(1/sqrt(RN32(ms + eps))) and ms = RN32(exact mean of v^2), and u is
// what is quantised (its own absmax and token scale).
//
// One workgroup per token row.  Pass 1 reduces max|v| (exact in any order) or,
// with the norm, the float64 sum of v^2 (each square exact), from which the
// exactly rounded mean follows (or, near a rounding boundary, from the exact
// integer sum in LDS); with the norm, pass 2 forms u and reduces max|u|; the last
// pass writes 16 int8 per 16-byte store.  Each thread's first H groups of 16 stay
// in registers between the passes, all loaded before any is used; H (1, 2 or 4)
// covers the row when it can (K <= 16 H kAqThreads) and no more, since the
// registers cost occupancy; groups past those are read again (from L1/L2).
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kAqThreads = 256;

template <bool BF16>
__device__ __forceinline__ float load_act(const void* x, int64_t i) {
  if (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[i]);
  return reinterpret_cast<const float*>(x)[i];
}

// 16 consecutive prologue inputs v of group c (the input, or the gated value).
template <bool BF16>
__device__ __forceinline__ void prologue16(const void* row, const void* urow, int64_t c,
                                           float v[16]) {
  load16_act<BF16>(row, c, v);
  if (urow) {
    float u[16];
    load16_act<BF16>(urow, c, u);
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = glu_value(v[j], u[j]);
  }
}

template <bool BF16>
__device__ __forceinline__ float prologue1(const void* row, const void* urow, int64_t i) {
  float v = load_act<BF16>(row, i);
  if (urow) v = glu_value(v, load_act<BF16>(urow, i));
  return v;
}

// The quantised values of group c with the norm applied: u = RN32(RN32(v r) w).
__device__ __forceinline__ void normalise16(float v[16], const float* w, int64_t c, float r) {
  const float4* wp = reinterpret_cast<const float4*>(w) + 4 * c;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const float4 g = wp[h];
    v[4 * h] = norm_value(v[4 * h], r, g.x);
    v[4 * h + 1] = norm_value(v[4 * h + 1], r, g.y);
    v[4 * h + 2] = norm_value(v[4 * h + 2], r, g.z);
    v[4 * h + 3] = norm_value(v[4 * h + 3], r, g.w);
  }
}

__device__ __forceinline__ uint4 quant16(const float v[16], float s) {
  return make_uint4(quant4(v, s), quant4(v + 4, s), quant4(v + 8, s), quant4(v + 12, s));
}

template <bool BF16, int H>
__global__ __launch_bounds__(kAqThreads) void aq_kernel(const void* __restrict__ x, int64_t K,
                                                       bool vec, int8_t* __restrict__ xq,
                                                       float* __restrict__ xs,
                                                       const ActPrologue pro) {
  __shared__ float wmax[kAqThreads / 64];
  __shared__ double wss[kAqThreads / 64];
  __shared__ unsigned long long limbs[kSqLimbs];
  __shared__ uint32_t sqwork[kSqWork];
  __shared__ float sh_ms;
  const int64_t m = blockIdx.x;
  const size_t esz = BF16 ? 2 : 4;
  const void* row = reinterpret_cast<const uint8_t*>(x) + (size_t)m * K * esz;
  const void* urow = pro.up ? reinterpret_cast<const uint8_t*>(pro.up) + (size_t)m * K * esz
                            : nullptr;
  const float* w = pro.w;
  int8_t* qrow = xq + m * K;
  const int tid = threadIdx.x;
  const int64_t n16 = vec ? K / 16 : 0;
  auto reduce_max = [&](float a) -> float {
    a = wave_max(a);
    if ((tid & 63) == 0) wmax[tid >> 6] = a;
    __syncthreads();
    a = wmax[0];
#pragma unroll
    for (int i = 1; i < kAqThreads / 64; ++i) a = fmaxf(a, wmax[i]);
    __syncthreads();   // wmax is reused
    return a;
  };

  // Pass 1: the prologue inputs v (held groups stay in registers).  Held groups
  // past the row read its last group again (valid memory) and are dropped.
  float hold[H][16];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int64_t c = tid + (int64_t)h * kAqThreads;
    if (n16 > 0) prologue16<BF16>(row, urow, c < n16 ? c : n16 - 1, hold[h]);
  }
  float a = 0.0f;
  if (!w) {
#pragma unroll
    for (int h = 0; h < H; ++h)
      if (tid + (int64_t)h * kAqThreads < n16)
#pragma unroll
        for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(hold[h][j]));
    for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
      float v[16];
      prologue16<BF16>(row, urow, c, v);
#pragma unroll
      for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
    }
    for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads)
      a = fmaxf(a, fabsf(prologue1<BF16>(row, urow, i)));
    a = reduce_max(a);
  } else {
    // the mean of v^2: float64 sum, then the exactly rounded mean
    double ss = 0.0;
#pragma unroll
    for (int h = 0; h < H; ++h)
      if (tid + (int64_t)h * kAqThreads < n16)
#pragma unroll
        for (int j = 0; j < 16; ++j) ss += (double)hold[h][j] * (double)hold[h][j];
    for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
      float v[16];
      prologue16<BF16>(row, urow, c, v);
#pragma unroll
      for (int j = 0; j < 16; ++j) ss += (double)v[j] * (double)v[j];
    }
    for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads) {
      const float v = prologue1<BF16>(row, urow, i);
      ss += (double)v * (double)v;
    }
    ss = wave_sum_f64(ss);
    if ((tid & 63) == 0) wss[tid >> 6] = ss;
    __syncthreads();
    ss = wss[0];
#pragma unroll
    for (int i = 1; i < kAqThreads / 64; ++i) ss += wss[i];
    float ms;
    if (!mean_sq_fast(ss, K, ms)) {
      // near a rounding boundary: the exact sum of the squares (uniform branch:
      // every thread holds the same ss)
      if (tid < kSqLimbs) limbs[tid] = 0ull;
      __syncthreads();
#pragma unroll
      for (int h = 0; h < H; ++h)
        if (tid + (int64_t)h * kAqThreads < n16)
#pragma unroll
          for (int j = 0; j < 16; ++j) sq_limbs_add(limbs, hold[h][j]);
      for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
        float v[16];
        prologue16<BF16>(row, urow, c, v);
#pragma unroll
        for (int j = 0; j < 16; ++j) sq_limbs_add(limbs, v[j]);
      }
      for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads)
        sq_limbs_add(limbs, prologue1<BF16>(row, urow, i));
      __syncthreads();
      if (tid == 0) sh_ms = sq_limbs_mean(limbs, K, sqwork);
      __syncthreads();
      ms = sh_ms;
    }
    const float r = rms_factor_of_mean(ms, pro.eps);
    // pass 2: u = RN32(RN32(v r) w) and its absmax
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t c = tid + (int64_t)h * kAqThreads;
      if (c < n16) {
        normalise16(hold[h], w, c, r);
#pragma unroll
        for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(hold[h][j]));
      }
    }
    for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
      float v[16];
      prologue16<BF16>(row, urow, c, v);
      normalise16(v, w, c, r);
#pragma unroll
      for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
    }
    for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads)
      a = fmaxf(a, fabsf(norm_value(prologue1<BF16>(row, urow, i), r, w[i])));
    a = reduce_max(a);
    // quantise (below) sees u: recompute it for the groups that are read again
    const float astar = fmaxf(a, kEps);
    const float s = kQb / astar;   // correctly rounded fp32 division
#pragma unroll
    for (int h = 0; h < H; ++h) {
      const int64_t c = tid + (int64_t)h * kAqThreads;
      if (c < n16) reinterpret_cast<uint4*>(qrow)[c] = quant16(hold[h], s);
    }
    for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
      float v[16];
      prologue16<BF16>(row, urow, c, v);
      normalise16(v, w, c, r);
      reinterpret_cast<uint4*>(qrow)[c] = quant16(v, s);
    }
    for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads) {
      const float q = rintf(norm_value(prologue1<BF16>(row, urow, i), r, w[i]) * s);
      qrow[i] = (int8_t)(int32_t)fminf(fmaxf(q, -128.0f), 127.0f);
    }
    if (tid == 0) xs[m] = astar / kQb;
    return;
  }

  const float astar = fmaxf(a, kEps);
  const float s = kQb / astar;   // correctly rounded fp32 division
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int64_t c = tid + (int64_t)h * kAqThreads;
    if (c < n16) reinterpret_cast<uint4*>(qrow)[c] = quant16(hold[h], s);
  }
  for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
    float v[16];
    prologue16<BF16>(row, urow, c, v);
    reinterpret_cast<uint4*>(qrow)[c] = quant16(v, s);
  }
  for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads) {
    const float q = rintf(prologue1<BF16>(row, urow, i) * s);
    qrow[i] = (int8_t)(int32_t)fminf(fmaxf(q, -128.0f), 127.0f);
  }
  if (tid == 0) xs[m] = astar / kQb;
}

}  // namespace

hipError_t launch_aq(const void* x, bool x_bf16, int64_t M, int64_t K, int8_t* x_q,
                     float* x_scale, const ActPrologue& pro, hipStream_t s) {
  // 16-element vectors need 16-byte aligned rows in the input, the output and
  // the prologue operands.
  const size_t esz = x_bf16 ? 2 : 4;
  const auto a16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  const bool vec = (K % 16 == 0) && a16(x) && a16(x_q) && a16(pro.up) && a16(pro.w) &&
                   ((K * esz) % 16 == 0);
  const int64_t per_thread = (K / 16 + kAqThreads - 1) / kAqThreads;   // groups per thread
  const int h = per_thread <= 1 ? 1 : per_thread <= 2 ? 2 : 4;
  const void* kern = x_bf16 ? (h == 1 ? (const void*)aq_kernel<true, 1>
                               : h == 2 ? (const void*)aq_kernel<true, 2> : (const void*)aq_kernel<true, 4>)
                            : (h == 1 ? (const void*)aq_kernel<false, 1>
                               : h == 2 ? (const void*)aq_kernel<false, 2> : (const void*)aq_kernel<false, 4>);
  void* args[] = {(void*)&x, (void*)&K, (void*)&vec, (void*)&x_q, (void*)&x_scale, (void*)&pro};
  return hipLaunchKernel(kern, dim3((unsigned)M), dim3(kAqThreads), args, 0, s);
}

}  // namespace bitnet
