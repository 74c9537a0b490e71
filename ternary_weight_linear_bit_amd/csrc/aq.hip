// Per-token absmax int8 activation quantisation.
//
// Method: communeify.com, "微軟 BitNet b1.58 震撼登場", section on BitNet b1.58
// 2B4T, quantisation details: activations are 8-bit integers (W1.58A8).  The pages
// give no scheme; the reading here is per token (row) absmax to the symmetric
// range [-127, 127]:  a* = max(max|x|, RN32(1e-5)), s = RN32(127/a*),
// xq = clip(rne(RN32(x*s)), -128, 127), d = RN32(a*/127).
//
// One workgroup per token row.  Pass 1 reduces max|x| (exact in any order) with
// wave butterflies and a cross-wave step in LDS; pass 2 re-reads the row (now in
// L1/L2) and writes 16 int8 per 16-byte store.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kAqThreads = 256;

template <bool BF16>
__device__ __forceinline__ float load_act(const void* x, int64_t i) {
  if (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[i]);
  return reinterpret_cast<const float*>(x)[i];
}

template <bool BF16>
__global__ __launch_bounds__(kAqThreads) void aq_kernel(const void* __restrict__ x, int64_t K,
                                                       bool vec, int8_t* __restrict__ xq,
                                                       float* __restrict__ xs) {
  __shared__ float wmax[kAqThreads / 64];
  const int64_t m = blockIdx.x;
  const void* row = BF16 ? (const void*)(reinterpret_cast<const uint16_t*>(x) + m * K)
                         : (const void*)(reinterpret_cast<const float*>(x) + m * K);
  int8_t* qrow = xq + m * K;
  const int tid = threadIdx.x;
  const int64_t n16 = vec ? K / 16 : 0;

  float a = 0.0f;
  for (int64_t c = tid; c < n16; c += kAqThreads) {
    float v[16];
    load16_act<BF16>(row, c, v);
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
  }
  for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads) a = fmaxf(a, fabsf(load_act<BF16>(row, i)));
  a = wave_max(a);
  if ((tid & 63) == 0) wmax[tid >> 6] = a;
  __syncthreads();
  a = wmax[0];
#pragma unroll
  for (int w = 1; w < kAqThreads / 64; ++w) a = fmaxf(a, wmax[w]);

  const float astar = fmaxf(a, kEps);
  const float s = kQb / astar;   // correctly rounded fp32 division
  for (int64_t c = tid; c < n16; c += kAqThreads) {
    float v[16];
    load16_act<BF16>(row, c, v);
    uint4 o;
    o.x = quant4(v, s);
    o.y = quant4(v + 4, s);
    o.z = quant4(v + 8, s);
    o.w = quant4(v + 12, s);
    reinterpret_cast<uint4*>(qrow)[c] = o;
  }
  for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads) {
    float q = rintf(load_act<BF16>(row, i) * s);
    qrow[i] = (int8_t)(int32_t)fminf(fmaxf(q, -128.0f), 127.0f);
  }
  if (tid == 0) xs[m] = astar / kQb;
}

}  // namespace

hipError_t launch_aq(const void* x, bool x_bf16, int64_t M, int64_t K, int8_t* x_q,
                     float* x_scale, hipStream_t s) {
  // 16-element vectors need 16-byte aligned rows in both the input and the output.
  const size_t esz = x_bf16 ? 2 : 4;
  const bool vec = (K % 16 == 0) && (((uintptr_t)x & 15u) == 0) && (((uintptr_t)x_q & 15u) == 0) &&
                   ((K * esz) % 16 == 0);
  if (x_bf16)
    hipLaunchKernelGGL(aq_kernel<true>, dim3((unsigned)M), dim3(kAqThreads), 0, s, x, K, vec, x_q,
                       x_scale);
  else
    hipLaunchKernelGGL(aq_kernel<false>, dim3((unsigned)M), dim3(kAqThreads), 0, s, x, K, vec, x_q,
                       x_scale);
  return hipGetLastError();
}

}  // namespace bitnet
