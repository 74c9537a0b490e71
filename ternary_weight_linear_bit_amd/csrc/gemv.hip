// Decode kernel (M <= 16 tokens): stream packed ternary weights from HBM and
// contract them with int8 activations on the int8 matrix cores.
//
// Method: dashen-tech.com, "BitNet.cpp 深度解析", section 3.1 (integer matmul):
// with weights in {-1, 0, +1} each output is the sum of the inputs under +1
// weights minus the sum under -1 weights.  Here every weight is carried as its
// 2-bit code c = q + 1 in {0, 1, 2} (section 2.3: two bits per weight), so
//     acc[m, n] = sum_k c[n, k] * x[m, k]  -  sum_k x[m, k],
// one unsigned-code contraction plus one per-token correction that every
// workgroup forms once from its staged activations.
//
// Design for gfx950 (not the pages' CPU kernels):
//  * Workgroup = 4 waves = one tile of 16 output rows; the waves split K in
//    interleaved 256-k super-chunks.  Each lane streams 16-byte chunks (64 codes)
//    of one row with raw buffer loads; one wave load instruction covers 16 rows x
//    64 contiguous bytes, and the four waves together read 256 contiguous bytes of
//    each row per step.  Rows past N and chunks past K read as zeros (buffer range
//    check), so the stream has no branches.
//  * kUnroll loads per lane are kept in flight; the first batch is issued before
//    the activations are staged, and the LDS-only barriers do not drain it.
//  * Unpack is 7 VALU ops per packed dword: (w >> 2i) & 0x03030303, i = 0..3,
//    yields 16 int8 codes in a k order that is a 4x4 byte transpose of the natural
//    one.  The activations are written to LDS with the same transpose, once per
//    workgroup, so the matrix-core operands agree without a per-weight shuffle.
//  * v_mfma_i32_16x16x64_i8: A = 16 weight rows x 64 k (codes), B = 64 k x 16
//    tokens (tokens >= M read a zero slot), int32 accumulate.  The four lane
//    groups of the instruction take four different 16-k blocks, so the matrix core
//    also performs the reduction along K inside a wave.
//  * The four waves' partial tiles are summed through LDS; wave 0 applies the
//    correction and the rescale y = RN32(float(acc) * RN32(gamma * d[m])).
//
// XMODE 1/2 (M <= kMaxFusedM) fuse the per-token absmax activation quantisation
// (fp32 / bf16 input) into the staging step: every workgroup quantises the
// activations with the same arithmetic as the standalone kernel, and workgroup 0
// also writes x_q and x_scale.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kRows = 16;      // output rows per workgroup (one MFMA tile)
constexpr int kUnroll = 8;     // 16-byte weight loads in flight per lane
constexpr int kStageBatch = 8; // 16-byte activation loads in flight per thread when staging
constexpr int kMaxM = 16;
constexpr int kMaxFusedM = 4;
constexpr int kLdsLimit = 64 * 1024;

// LDS layout after the activations (offsets from zero_off = M * (K + 16)):
constexpr int kZeroBytes = 64;                   // four zero 16-byte groups
constexpr int kSumxOff = kZeroBytes;             // int   sumx[16]
constexpr int kSclOff = kSumxOff + 64;           // float scl[16]
constexpr int kRedOff = kSclOff + 64;            // v4i   red[3][64]
constexpr int kWredOff = kRedOff + 3 * 64 * 16;  // float wred[2][4]
constexpr int kExtra = kWredOff + 32;

int lds_bytes(int64_t M, int64_t K) { return (int)(M * (K + 16)) + kExtra; }

// One packed dword (codes of k-offsets 0..15, byte b holding 4b..4b+3) -> the
// 16-byte operand whose byte 4i + b is the code of k-offset 4b + i.
__device__ __forceinline__ v4i unpack_codes_transposed(uint32_t w) {
  v4i a;
  a.x = (int)(w & 0x03030303u);
  a.y = (int)((w >> 2) & 0x03030303u);
  a.z = (int)((w >> 4) & 0x03030303u);
  a.w = (int)((w >> 6) & 0x03030303u);
  return a;
}

__device__ __forceinline__ void store_transposed(uint8_t* smem, int off, const uint32_t xd[4]) {
  uint32_t pd[4];
  transpose4x4_bytes(xd, pd);
  *reinterpret_cast<uint4*>(smem + off) = make_uint4(pd[0], pd[1], pd[2], pd[3]);
}

// Stage activation groups [i0, i0 + kThreads * kStageBatch) of the flattened
// [M][K/16] group index: transpose each 16-byte group into LDS.
__device__ __forceinline__ void stage_groups(uint8_t* smem, const uint4* v, int i0, int tid,
                                             int total, int K16, int stride) {
#pragma unroll
  for (int b = 0; b < kStageBatch; ++b) {
    const int i = i0 + tid + kThreads * b;
    if (i < total) {
      const int t = i / K16, c = i - t * K16;
      const uint32_t xd[4] = {v[b].x, v[b].y, v[b].z, v[b].w};
      store_transposed(smem, t * stride + 16 * c, xd);
    }
  }
}

template <int XMODE, int UNROLL>  // XMODE 0: int8 x_q; 1: fp32 input; 2: bf16 input
__global__ __launch_bounds__(kThreads) void gemv_kernel(
    const uint8_t* __restrict__ wp, const float* __restrict__ w_scale,
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const void* __restrict__ xf, int8_t* __restrict__ xq_out, float* __restrict__ xs_out,
    int M, int N, int K, void* __restrict__ y, int y_bf16, int32_t* __restrict__ acc_out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;  // A operand: weight row of the tile; B operand: token
  const int g = lane >> 4;  // 16-k block of the operand within the instruction
  const int stride = K + 16;
  const int zero_off = M * stride;
  int* sumx = reinterpret_cast<int*>(smem + zero_off + kSumxOff);
  float* scl = reinterpret_cast<float*>(smem + zero_off + kSclOff);
  v4i* red = reinterpret_cast<v4i*>(smem + zero_off + kRedOff);
  float* wred = reinterpret_cast<float*>(smem + zero_off + kWredOff);

  const int n0 = blockIdx.x * kRows;
  const int C = K >> 6;                                 // 16-byte chunks per row
  const int S = (C + 3) >> 2;                           // 256-k super-chunks
  const int J = (S > wave) ? (S - wave + 3) >> 2 : 0;  // super-chunks of this wave
  const uint32_t rowb = (uint32_t)K >> 2;               // packed bytes per row
  const int rows_here = min(kRows, N - n0);
  const auto wr = make_rsrc(wp + (size_t)n0 * rowb, (uint32_t)rows_here * rowb);
  const uint32_t wbase = (uint32_t)r * rowb;            // out of range when r >= rows_here
  // Chunk of iteration j for this lane; iterations j >= J (and chunks past the
  // row) read zeros, so a batch may run past J without changing the result.
  auto woff = [&](int j) -> uint32_t {
    const int c = 4 * (wave + 4 * j) + g;
    return c < C ? wbase + 16u * (uint32_t)c : kOob;
  };
  const int K16 = K >> 4;
  const int total = M * K16;  // 16-byte activation groups, all tokens

  // 1. token scales and the first batch of int8 activation loads, then the first
  //    weight loads, so that waiting for the former does not wait for the latter
  const float xs_t = (XMODE == 0) ? x_scale[min(tid, M - 1)] : 0.0f;
  uint4 xv[kStageBatch];
  const auto xr = make_rsrc(xq, (uint32_t)M * (uint32_t)K);
  if (XMODE == 0) {
#pragma unroll
    for (int b = 0; b < kStageBatch; ++b) {
      const int i = tid + kThreads * b;
      xv[b] = bload16(xr, i < total ? 16u * (uint32_t)i : kOob);
    }
  }
  uint4 buf[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) buf[u] = bload16(wr, woff(u));

  // 2. small LDS state
  if (tid < kMaxM) sumx[tid] = 0;
  if (tid >= 64 && tid < 68)
    reinterpret_cast<uint4*>(smem + zero_off)[tid - 64] = make_uint4(0u, 0u, 0u, 0u);

  // 3. stage the activations, transposed within each 16-byte group
  const float gamma = *w_scale;
  if (XMODE == 0) {
    stage_groups(smem, xv, 0, tid, total, K16, stride);
    for (int i0 = kThreads * kStageBatch; i0 < total; i0 += kThreads * kStageBatch) {
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) {
        const int i = i0 + tid + kThreads * b;
        xv[b] = bload16(xr, i < total ? 16u * (uint32_t)i : kOob);
      }
      stage_groups(smem, xv, i0, tid, total, K16, stride);
    }
    if (tid < M) scl[tid] = gamma * xs_t;
  } else {
    constexpr bool BF = XMODE == 2;
    constexpr uint32_t esz = BF ? 2u : 4u;
    constexpr int L = BF ? 2 : 4;  // 16-byte loads per 16 activations
    const auto fr = make_rsrc(xf, (uint32_t)M * (uint32_t)K * esz);
    for (int t = 0; t < M; ++t) {
      const uint32_t rowoff = (uint32_t)t * (uint32_t)K * esz;
      float a = 0.0f;
      for (int c0 = 0; c0 < K16; c0 += kThreads * 4) {
        uint4 v[4][L];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int c = c0 + tid + kThreads * b;
#pragma unroll
          for (int h = 0; h < L; ++h)
            v[b][h] = bload16(fr, c < K16 ? rowoff + 16u * (uint32_t)(L * c + h) : kOob);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int h = 0; h < L; ++h) {
            const uint32_t d[4] = {v[b][h].x, v[b][h].y, v[b][h].z, v[b][h].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (BF) {
                a = fmaxf(a, fabsf(__uint_as_float(d[e] << 16)));
                a = fmaxf(a, fabsf(__uint_as_float(d[e] & 0xffff0000u)));
              } else {
                a = fmaxf(a, fabsf(__uint_as_float(d[e])));
              }
            }
          }
      }
      a = wave_max(a);
      float* wrd = wred + 4 * (t & 1);
      if (lane == 0) wrd[wave] = a;
      lds_barrier();
      a = fmaxf(fmaxf(wrd[0], wrd[1]), fmaxf(wrd[2], wrd[3]));
      const float astar = fmaxf(a, kEps);
      const float s_t = kQb / astar;
      if (tid == 0) {
        const float d = astar / kQb;
        scl[t] = gamma * d;
        if (blockIdx.x == 0) xs_out[t] = d;
      }
      const void* xrow = BF ? (const void*)(reinterpret_cast<const uint16_t*>(xf) + (size_t)t * K)
                            : (const void*)(reinterpret_cast<const float*>(xf) + (size_t)t * K);
      for (int c = tid; c < K16; c += kThreads) {
        float v[16];
        load16_act<BF>(xrow, c, v);
        uint32_t xd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) xd[i] = quant4(v + 4 * i, s_t);
        if (blockIdx.x == 0)
          reinterpret_cast<uint4*>(xq_out + (size_t)t * K)[c] = make_uint4(xd[0], xd[1], xd[2], xd[3]);
        store_transposed(smem, t * stride + 16 * c, xd);
      }
    }
  }
  lds_barrier();

  // 4. per-token sums of the staged activations (the code-offset correction)
  for (int t = 0; t < M; ++t) {
    int sx = 0;
    for (int c = tid; c < K16; c += kThreads) {
      const v4i v = *reinterpret_cast<const v4i*>(smem + t * stride + 16 * c);
      sx = __builtin_amdgcn_sdot4(v.x, 0x01010101, sx, false);
      sx = __builtin_amdgcn_sdot4(v.y, 0x01010101, sx, false);
      sx = __builtin_amdgcn_sdot4(v.z, 0x01010101, sx, false);
      sx = __builtin_amdgcn_sdot4(v.w, 0x01010101, sx, false);
    }
    sx = wave_sum(sx);
    if (lane == 0) atomicAdd(&sumx[t], sx);
  }

  // 5. stream the weights: batches of UNROLL iterations with a branch-free body
  v4i acc = {0, 0, 0, 0};
  const int bt = (r < M) ? r * stride : -1;
  for (int j0 = 0; j0 < J; j0 += UNROLL) {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int j = j0 + u;
      const int c = 4 * (wave + 4 * j) + g;
      // unpack the whole chunk before refilling its slot, so the refill can land in
      // the same registers (no loop-carried copy that would wait for the load)
      const v4i a0 = unpack_codes_transposed(buf[u].x);
      const v4i a1 = unpack_codes_transposed(buf[u].y);
      const v4i a2 = unpack_codes_transposed(buf[u].z);
      const v4i a3 = unpack_codes_transposed(buf[u].w);
      buf[u] = bload16(wr, woff(j + UNROLL));
      const int bbase = (bt >= 0 && c < C) ? bt + 64 * c : zero_off;
      const v4i* bp = reinterpret_cast<const v4i*>(smem + bbase);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bp[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bp[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, bp[2], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, bp[3], acc, 0, 0, 0);
    }
  }

  // 6. sum the four waves' partial tiles, correct, rescale, store
  if (wave > 0) red[(wave - 1) * 64 + lane] = acc;
  lds_barrier();
  if (wave == 0) {
    acc += red[lane] + red[64 + lane] + red[128 + lane];
    const int t = r;  // D layout: the lane holds rows 4g..4g+3 of the tile for token r
    if (t < M) {
      const int sxt = sumx[t];
      const float sc = scl[t];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = n0 + 4 * g + v;
        if (n < N) {
          const int a = acc[v] - sxt;
          const float yv = (float)a * sc;
          const size_t o = (size_t)t * N + n;
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

}  // namespace

bool gemv_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= kMaxM && K >= 64 && (K % 64) == 0 && lds_bytes(M, K) <= kLdsLimit;
}

bool gemv_fused_fits(int64_t M, int64_t K) { return M <= kMaxFusedM && gemv_fits(M, K); }

template <int XMODE>
void launch_mode(dim3 grid, size_t lds, const Launch& l, int unroll, const uint8_t* wp,
                 const float* w_scale, const int8_t* xq, const float* x_scale, const void* xf,
                 int8_t* xq_out, float* xs_out, int M, int N, int K, void* y, int yb,
                 int32_t* acc_out) {
  if (unroll <= 2)
    launch_kernel(gemv_kernel<XMODE, 2>, grid, dim3(kThreads), lds, l, wp, w_scale, xq,
                       x_scale, xf, xq_out, xs_out, M, N, K, y, yb, acc_out);
  else if (unroll <= 4)
    launch_kernel(gemv_kernel<XMODE, 4>, grid, dim3(kThreads), lds, l, wp, w_scale, xq,
                       x_scale, xf, xq_out, xs_out, M, N, K, y, yb, acc_out);
  else
    launch_kernel(gemv_kernel<XMODE, 8>, grid, dim3(kThreads), lds, l, wp, w_scale, xq,
                       x_scale, xf, xq_out, xs_out, M, N, K, y, yb, acc_out);
}

hipError_t launch_gemv(const uint8_t* wp, const float* w_scale, const int8_t* xq,
                       const float* x_scale, const void* xf, int xf_dtype, int8_t* xq_out,
                       float* xs_out, int M, int N, int K, void* y, bool y_bf16,
                       int32_t* acc_out, const Launch& l) {
  if (!gemv_fits(M, K) || (xf != nullptr && M > kMaxFusedM)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + kRows - 1) / kRows));
  const size_t lds = (size_t)lds_bytes(M, K);
  const int yb = y_bf16 ? 1 : 0;
  // loop depth: the largest per-wave iteration count, rounded up to 2, 4 or 8
  const int jmax = ((K / 64 + 3) / 4 + 3) / 4;
  if (xf == nullptr)
    launch_mode<0>(grid, lds, l, jmax, wp, w_scale, xq, x_scale, xf, xq_out, xs_out, M, N, K, y,
                   yb, acc_out);
  else if (xf_dtype == 1)
    launch_mode<2>(grid, lds, l, jmax, wp, w_scale, xq, x_scale, xf, xq_out, xs_out, M, N, K, y,
                   yb, acc_out);
  else
    launch_mode<1>(grid, lds, l, jmax, wp, w_scale, xq, x_scale, xf, xq_out, xs_out, M, N, K, y,
                   yb, acc_out);
  return hipGetLastError();
}

}  // namespace bitnet
