// Prefill kernel (M > 16 tokens): dense int8 contraction on the matrix cores.
//
// Method: dashen-tech.com, "BitNet.cpp 深度解析", section 3.1: ternary weights turn
// the float matmul into an integer one.  At many tokens the contraction is
// compute-bound (hundreds of int8 ops per weight byte), so the ternary tiles are
// expanded to signed int8 in LDS and fed to v_mfma_i32_16x16x64_i8.
//
// Tile: 128 tokens x 128 output rows per workgroup, K step 64; 4 waves as 2 x 2,
// each owning a 64 x 64 sub-tile (4 x 4 instructions, 64 int32 accumulators per
// lane).  Per K step each thread loads 32 activation bytes and 8 packed weight
// bytes (32 codes) from global memory into registers one step ahead, expands the
// codes to signed int8 in natural k order and writes both tiles to LDS (row
// stride 80 bytes so the 16-byte operand reads of 8 consecutive rows hit distinct
// banks).  The rescale y = RN32(float(acc) * RN32(gamma * d[m])) is fused into the
// store.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int kThreads = 256;
constexpr int kLds = BK + 16;   // row stride in bytes

// One packed dword (codes of k-offsets 0..15) -> four dwords of signed int8 in
// natural order (dword b holds k-offsets 4b..4b+3).
__device__ __forceinline__ void unpack_signed_natural(uint32_t w, uint32_t out[4]) {
  uint32_t m[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = (w >> (2 * i)) & 0x03030303u;   // byte b = code(4b + i)
  transpose4x4_bytes(m, out);                                         // byte i = code(4b + i)
#pragma unroll
  for (int b = 0; b < 4; ++b) out[b] = (out[b] + 0x7f7f7f7fu) ^ 0x80808080u;  // c -> c - 1
}

__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const uint8_t* __restrict__ wp, const float* __restrict__ w_scale,
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int M, int N, int K,
    void* __restrict__ y, int y_bf16, int32_t* __restrict__ acc_out) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[BM * kLds];
  __shared__ __attribute__((aligned(16))) uint8_t ws[BN * kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;

  // global -> register assignment: row tid/2, half tid%2 of the K step
  const int lrow = tid >> 1, lhalf = tid & 1;
  const bool xrow_ok = m0 + lrow < M;
  const bool wrow_ok = n0 + lrow < N;
  const int8_t* xptr = xq + (size_t)(xrow_ok ? m0 + lrow : 0) * K + 32 * lhalf;
  const uint8_t* wptr = wp + (size_t)(wrow_ok ? n0 + lrow : 0) * (size_t)(K >> 2) + 8 * lhalf;
  uint4 xa = make_uint4(0u, 0u, 0u, 0u), xb = xa;
  uint2 wv = make_uint2(0u, 0u);
  auto gload = [&](int k0) {
    if (xrow_ok) {
      const uint4* p = reinterpret_cast<const uint4*>(xptr + k0);
      xa = p[0];
      xb = p[1];
    }
    if (wrow_ok) wv = *reinterpret_cast<const uint2*>(wptr + (k0 >> 2));
  };

  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4i){0, 0, 0, 0};

  const int orow = lane & 15, ocol = 16 * (lane >> 4);
  gload(0);
  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    {
      uint8_t* xd = xs + lrow * kLds + 32 * lhalf;
      *reinterpret_cast<uint4*>(xd) = xa;
      *reinterpret_cast<uint4*>(xd + 16) = xb;
      uint32_t o[8];
      unpack_signed_natural(wv.x, o);
      unpack_signed_natural(wv.y, o + 4);
      uint8_t* wd = ws + lrow * kLds + 32 * lhalf;
      *reinterpret_cast<uint4*>(wd) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(wd + 16) = make_uint4(o[4], o[5], o[6], o[7]);
    }
    __syncthreads();
    if (k0 + BK < K) gload(k0 + BK);
    v4i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *reinterpret_cast<const v4i*>(xs + (wm * 64 + i * 16 + orow) * kLds + ocol);
      bf[i] = *reinterpret_cast<const v4i*>(ws + (wn * 64 + i * 16 + orow) * kLds + ocol);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
  }

  // D layout: lane holds tokens 4*(lane/16) + v of each 16 x 16 block, row lane % 16
  const float gamma = *w_scale;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + v;
      if (m < M) {
        const float sc = gamma * x_scale[m];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + (lane & 15);
          if (n < N) {
            const int a = acc[i][j][v];
            const float yv = (float)a * sc;
            const size_t o = (size_t)m * N + n;
            if (acc_out) acc_out[o] = a;
            if (y_bf16)
              reinterpret_cast<uint16_t*>(y)[o] = float_to_bf16_rne(yv);
            else
              reinterpret_cast<float*>(y)[o] = yv;
          }
        }
      }
    }
  }
}

// Any K % 4 == 0, any alignment: one thread per output, plain byte loops.
__global__ __launch_bounds__(256) void generic_linear_kernel(
    const uint8_t* __restrict__ wp, const float* __restrict__ w_scale,
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int64_t M, int64_t N,
    int64_t K, void* __restrict__ y, int y_bf16, int32_t* __restrict__ acc_out) {
  const int64_t total = M * N;
  const float gamma = *w_scale;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t m = idx / N, n = idx - m * N;
    const uint8_t* wrow = wp + n * (K >> 2);
    const int8_t* xrow = xq + m * K;
    int a = 0;
    for (int64_t kb = 0; kb < (K >> 2); ++kb) {
      const uint32_t b = wrow[kb];
#pragma unroll
      for (int i = 0; i < 4; ++i) a += ((int)((b >> (2 * i)) & 3u) - 1) * (int)xrow[4 * kb + i];
    }
    const float yv = (float)a * (gamma * x_scale[m]);
    if (acc_out) acc_out[idx] = a;
    if (y_bf16)
      reinterpret_cast<uint16_t*>(y)[idx] = float_to_bf16_rne(yv);
    else
      reinterpret_cast<float*>(y)[idx] = yv;
  }
}

}  // namespace

hipError_t launch_gemm(const uint8_t* wp, const float* w_scale, const int8_t* xq,
                       const float* x_scale, int M, int N, int K, void* y, bool y_bf16,
                       int32_t* acc_out, hipStream_t s) {
  if (K % BK != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(kThreads), 0, s, wp, w_scale, xq, x_scale, M, N, K, y,
                     y_bf16 ? 1 : 0, acc_out);
  return hipGetLastError();
}

hipError_t launch_generic_linear(const uint8_t* wp, const float* w_scale, const int8_t* xq,
                                 const float* x_scale, int64_t M, int64_t N, int64_t K,
                                 void* y, bool y_bf16, int32_t* acc_out, hipStream_t s) {
  int64_t blocks = (M * N + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(generic_linear_kernel, dim3((unsigned)blocks), dim3(256), 0, s, wp, w_scale,
                     xq, x_scale, M, N, K, y, y_bf16 ? 1 : 0, acc_out);
  return hipGetLastError();
}

}  // namespace bitnet
