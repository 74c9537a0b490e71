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
// weight w the row is quantised as RN32(v * w) and the token scale becomes
// RN32(d * r), r = RN32(1/sqrt(RN32(RN32(mean v^2) + eps))) -- absmax
// quantisation is invariant under the positive per-token factor r.
//
// One workgroup per token row.  Pass 1 reduces max|v*w| (exact in any order) and
// sum v^2 (float64; the products are exact) with wave butterflies and a
// cross-wave step in LDS; pass 2 writes 16 int8 per 16-byte store.  Each thread's
// first H groups of 16 stay in registers between the passes, all loaded before
// any is used; H (1, 2 or 4) covers the row when it can (K <= 16 H kAqThreads)
// and no more, since the registers cost occupancy; groups past those are read
// again in pass 2 (from L1/L2).
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kAqThreads = 256;

template <bool BF16>
__device__ __forceinline__ float load_act(const void* x, int64_t i) {
  if (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(x)[i]);
  return reinterpret_cast<const float*>(x)[i];
}

// 16 consecutive prologue values (the quantised ones, q) of group c; adds v^2
// to ss when the norm is on.
template <bool BF16>
__device__ __forceinline__ void prologue16(const void* row, const void* urow, const float* w,
                                           int64_t c, float q[16], double& ss) {
  load16_act<BF16>(row, c, q);
  if (urow) {
    float u[16];
    load16_act<BF16>(urow, c, u);
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = glu_value(q[j], u[j]);
  }
  if (w) {
    const float4* wp = reinterpret_cast<const float4*>(w) + 4 * c;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float4 g = wp[h];
      const float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = q[4 * h + j];
        ss += (double)v * (double)v;
        q[4 * h + j] = __fmul_rn(v, gv[j]);
      }
    }
  }
}

template <bool BF16>
__device__ __forceinline__ float prologue1(const void* row, const void* urow, const float* w,
                                           int64_t i, double& ss) {
  float v = load_act<BF16>(row, i);
  if (urow) v = glu_value(v, load_act<BF16>(urow, i));
  if (w) {
    ss += (double)v * (double)v;
    v = __fmul_rn(v, w[i]);
  }
  return v;
}

template <bool BF16, int H>
__global__ __launch_bounds__(kAqThreads) void aq_kernel(const void* __restrict__ x, int64_t K,
                                                       bool vec, int8_t* __restrict__ xq,
                                                       float* __restrict__ xs,
                                                       const ActPrologue pro) {
  __shared__ float wmax[kAqThreads / 64];
  __shared__ double wss[kAqThreads / 64];
  const int64_t m = blockIdx.x;
  const size_t esz = BF16 ? 2 : 4;
  const void* row = reinterpret_cast<const uint8_t*>(x) + (size_t)m * K * esz;
  const void* urow = pro.up ? reinterpret_cast<const uint8_t*>(pro.up) + (size_t)m * K * esz
                            : nullptr;
  int8_t* qrow = xq + m * K;
  const int tid = threadIdx.x;
  const int64_t n16 = vec ? K / 16 : 0;

  float a = 0.0f;
  double ss = 0.0;
  // held groups: an index past the row reads its last group again (valid memory)
  // and is dropped from the max, the sum and the stores
  float hold[H][16];
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int64_t c = tid + (int64_t)h * kAqThreads;
    double s2 = 0.0;
    if (n16 > 0) prologue16<BF16>(row, urow, pro.w, c < n16 ? c : n16 - 1, hold[h], s2);
    if (c < n16) {
      ss += s2;
#pragma unroll
      for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(hold[h][j]));
    }
  }
  for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
    float v[16];
    prologue16<BF16>(row, urow, pro.w, c, v, ss);
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(v[j]));
  }
  for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads)
    a = fmaxf(a, fabsf(prologue1<BF16>(row, urow, pro.w, i, ss)));
  a = wave_max(a);
  ss = wave_sum_f64(ss);
  if ((tid & 63) == 0) {
    wmax[tid >> 6] = a;
    wss[tid >> 6] = ss;
  }
  __syncthreads();
  a = wmax[0];
  ss = wss[0];
#pragma unroll
  for (int w = 1; w < kAqThreads / 64; ++w) {
    a = fmaxf(a, wmax[w]);
    ss += wss[w];
  }

  const float astar = fmaxf(a, kEps);
  const float s = kQb / astar;   // correctly rounded fp32 division
#pragma unroll
  for (int h = 0; h < H; ++h) {
    const int64_t c = tid + (int64_t)h * kAqThreads;
    if (c < n16) {
      uint4 o;
      o.x = quant4(hold[h], s);
      o.y = quant4(hold[h] + 4, s);
      o.z = quant4(hold[h] + 8, s);
      o.w = quant4(hold[h] + 12, s);
      reinterpret_cast<uint4*>(qrow)[c] = o;
    }
  }
  for (int64_t c = tid + (int64_t)H * kAqThreads; c < n16; c += kAqThreads) {
    float v[16];
    double unused = 0.0;
    prologue16<BF16>(row, urow, pro.w, c, v, unused);
    uint4 o;
    o.x = quant4(v, s);
    o.y = quant4(v + 4, s);
    o.z = quant4(v + 8, s);
    o.w = quant4(v + 12, s);
    reinterpret_cast<uint4*>(qrow)[c] = o;
  }
  for (int64_t i = n16 * 16 + tid; i < K; i += kAqThreads) {
    double unused = 0.0;
    float q = rintf(prologue1<BF16>(row, urow, pro.w, i, unused) * s);
    qrow[i] = (int8_t)(int32_t)fminf(fmaxf(q, -128.0f), 127.0f);
  }
  if (tid == 0) {
    float d = astar / kQb;
    if (pro.w) d = __fmul_rn(d, rms_factor(ss, K, pro.eps));
    xs[m] = d;
  }
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
