// Lookup-table decode (M tokens one at a time, 2-bit weights): the contraction
// as table lookups instead of matrix-core products.
//
// Method: juejin.cn, "微软 BitNet：让百亿参数大模型在 CPU 上飞起来", technical
// principles, item 2: bitnet.cpp's kernels follow T-MAC's lookup-table method,
// which turns the matrix product into table lookups (dashen-tech.com, "BitNet.cpp
// 深度解析", section 3.2 names the lookup kernel types TL1 and TL2).  Reading here:
// per token, each pair of int8 activations (x[2g], x[2g+1]) gets a table of 16
// partial sums, entry c0 + 4 c1 = (c0 - 1) x[2g] + (c1 - 1) x[2g+1], so each
// nibble of the 2-bit layout (the codes of two weights) is an index and an
// output is the sum of one lookup per pair of weights.  Integer throughout, so
// the result is the exact accumulator of the matrix-core path.
//
// Design for gfx950 (the pages' lookup kernels are CPU SIMD code that keeps
// 16-entry tables in vector registers):
//  * lut_build: one thread per pair writes its 16 int16 entries (32 bytes) to
//    global memory -- the table of a token is shared by every output row, so it
//    is built once, not per workgroup -- and zeroes the int32 accumulators.
//  * lut_gemv: workgroup = 4 waves x 16 rows = 64 rows, over a split of K of up
//    to 32 chunks of 64 weights.  It copies its split's tables (32 bytes per
//    pair, as many bytes as its 64 rows' packed weights) from L2 into LDS, with
//    a 32-byte pad after each chunk's 32 pairs; the table and weight loads are
//    all issued before the first LDS store.  Lane (row r, lane group s)
//    loads 16 bytes of its row for chunks 4i + s (the 64 lanes of a wave read 16
//    rows x 64 contiguous bytes per load) and makes one LDS lookup (a 16-bit
//    read of an entry stored with a bias of 512, removed from the sum at the
//    end) per nibble.  Lanes of one group read one pair's 32-byte table (at most six
//    distinct dwords for valid codes); the pad puts the four groups' tables in
//    different banks.  The four lane groups of a row are summed with shuffles
//    and the row's partial is added into the accumulator (int32 atomics, exact
//    in any order).
//  * lut_epilogue: y = RN32(float(acc) * RN32(gamma * d)), as every path.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 64;          // rows per workgroup (4 waves x 16)
constexpr int kMaxChunks = 32;     // 64-weight chunks per split (LDS: 33 x 1 KiB)
constexpr int kChunkLds = 33 * 32;  // LDS bytes per chunk: 32 pairs of 32 bytes + a 32-byte pad

// Table entries are stored with a bias of kBias (all entries, including those of
// the unused code 3, lie in [-512, 512)), so that they are read zero-extended
// and the sum's bias is a constant removed at the end.
constexpr int kBias = 512;
typedef __attribute__((address_space(3))) const uint16_t lds_u16;

__global__ __launch_bounds__(kThreads) void lut_build(const int8_t* __restrict__ xq, int K, int N,
                                                      uint4* __restrict__ table,
                                                      int32_t* __restrict__ acc) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < K / 2) {
    const int x0 = xq[2 * i], x1 = xq[2 * i + 1];
    uint32_t e[8];
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int a = 2 * h, b = 2 * h + 1;   // entries c0 + 4 c1
      const int va = ((a & 3) - 1) * x0 + ((a >> 2) - 1) * x1 + kBias;
      const int vb = ((b & 3) - 1) * x0 + ((b >> 2) - 1) * x1 + kBias;
      e[h] = (uint32_t)va | ((uint32_t)vb << 16);
    }
    table[2 * (size_t)i] = make_uint4(e[0], e[1], e[2], e[3]);
    table[2 * (size_t)i + 1] = make_uint4(e[4], e[5], e[6], e[7]);
  }
  if (i < N) acc[i] = 0;
}

__global__ __launch_bounds__(kThreads) void lut_gemv(const uint8_t* __restrict__ wp,
                                                     const uint4* __restrict__ table, int N,
                                                     int K, int split,
                                                     int32_t* __restrict__ acc) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem_[];
  auto* smem = (__attribute__((address_space(3))) uint8_t*)smem_;
  constexpr int kCopy = kMaxChunks * 64 / kThreads;  // 16-byte table pieces per thread
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int C = K >> 6;                            // chunks per row
  const int c0 = (int)blockIdx.y * split;          // first chunk of this split
  const int nc = min(split, C - c0);               // chunks in this split (>= 1)
  const uint32_t rowb = (uint32_t)K >> 2;
  const int row0 = (int)blockIdx.x * kRows;
  const int r = lane & 15, s = lane >> 4;
  const int lrow = 16 * wave + r;                  // row within the workgroup

  // 1. the split's tables (64 pieces of 16 bytes per chunk), then this lane's
  // weights, all in flight together; pieces past the split read zeros and go to
  // a spare slot, chunks past the split read as code 1 (weight 0) through table
  // chunk 0
  const auto ts = make_uniform_rsrc(table + (size_t)c0 * 64, (uint32_t)nc * 1024u);
  uint4 tv[kCopy];
#pragma unroll
  for (int h = 0; h < kCopy; ++h) tv[h] = bload16(ts, 16u * (uint32_t)(tid + kThreads * h));
  const auto rs = make_uniform_rsrc(wp + (size_t)row0 * rowb,
                                    (uint32_t)min(kRows, N - row0) * rowb);
  uint4 w[kMaxChunks / 4];
#pragma unroll
  for (int i = 0; i < kMaxChunks / 4; ++i) {
    const int c = 4 * i + s;
    w[i] = bload16(rs, c < nc ? (uint32_t)lrow * rowb + 16u * (uint32_t)(c0 + c) : kOob);
  }
  // piece u of the split: chunk u / 64 at kChunkLds * (u / 64), byte 16 (u % 64)
#pragma unroll
  for (int h = 0; h < kCopy; ++h) {
    const int u = tid + kThreads * h;
    const int at = u < nc * 64 ? kChunkLds * (u >> 6) + 16 * (u & 63) : kChunkLds * split;
    *reinterpret_cast<__attribute__((address_space(3))) v4i*>(smem + at) =
        (v4i){(int)tv[h].x, (int)tv[h].y, (int)tv[h].z, (int)tv[h].w};
  }
  __syncthreads();

  // 2. one lookup per nibble: pair 8 d + j of chunk c, entry idx, at
  // kChunkLds * c + 32 (8 d + j) + 2 idx (the chunk base is a multiple of 32)
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < kMaxChunks / 4; ++i) {
    const int c = 4 * i + s;
    const bool ok = c < nc;
    const uint32_t wd[4] = {ok ? w[i].x : 0x55555555u, ok ? w[i].y : 0x55555555u,
                            ok ? w[i].z : 0x55555555u, ok ? w[i].w : 0x55555555u};
    const lds_u16* tb = reinterpret_cast<const lds_u16*>(smem + kChunkLds * (ok ? c : 0));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        sum += tb[__builtin_amdgcn_ubfe(wd[d], 4 * j, 4) + 16 * (8 * d + j)];
    }
  }
  int total = (int)sum - kBias * 32 * (kMaxChunks / 4);   // every lane made 256 lookups
  total += __shfl_xor(total, 16, 64);
  total += __shfl_xor(total, 32, 64);
  if (s == 0 && row0 + lrow < N) atomicAdd(acc + row0 + lrow, total);
}

__global__ __launch_bounds__(kThreads) void lut_epilogue(const int32_t* __restrict__ acc,
                                                         const float* __restrict__ w_scale,
                                                         const float* __restrict__ d, int N,
                                                         void* __restrict__ y, bool y_bf16,
                                                         int32_t* __restrict__ acc_out) {
  const int n = blockIdx.x * kThreads + threadIdx.x;
  if (n >= N) return;
  const int a = acc[n];
  const float yv = (float)a * (*w_scale * *d);
  if (acc_out) acc_out[n] = a;
  if (y_bf16)
    reinterpret_cast<uint16_t*>(y)[n] = float_to_bf16_rne(yv);
  else
    reinterpret_cast<float*>(y)[n] = yv;
}

}  // namespace

size_t lut_workspace_bytes(int64_t N, int64_t K) {
  const auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  return (size_t)(up(16 * K) + up(4 * N));
}

hipError_t launch_lut(const uint8_t* wp, const float* w_scale, const int8_t* xq,
                      const float* x_scale, int64_t M, int64_t N, int64_t K, void* y,
                      bool y_bf16, int32_t* acc_out, void* workspace, int cus, hipStream_t s) {
  auto* table = reinterpret_cast<uint4*>(workspace);
  auto* acc = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                         (16 * K + 255) / 256 * 256);
  const int C = (int)(K / 64);
  const int row_blocks = (int)((N + kRows - 1) / kRows);
  // splits of at most kMaxChunks chunks; shorter ones when the row blocks alone
  // give fewer than two workgroups per compute unit
  int split = kMaxChunks;
  while (split > 4 && (int64_t)row_blocks * ((C + split - 1) / split) < 2 * cus) split /= 2;
  const int splits = (C + split - 1) / split;
  const size_t lds = (size_t)kChunkLds * (size_t)split + 16;  // + the spare slot
  const size_t esz = y_bf16 ? 2 : 4;
  for (int64_t m = 0; m < M; ++m) {
    const int64_t items = K / 2 > N ? K / 2 : N;
    hipLaunchKernelGGL(lut_build, dim3((unsigned)((items + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, xq + m * K, (int)K, (int)N, table, acc);
    hipLaunchKernelGGL(lut_gemv, dim3((unsigned)row_blocks, (unsigned)splits), dim3(kThreads),
                       lds, s, wp, table, (int)N, (int)K, split, acc);
    hipLaunchKernelGGL(lut_epilogue, dim3((unsigned)((N + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, s, acc, w_scale, x_scale + m, (int)N,
                       static_cast<char*>(y) + (size_t)m * N * esz, y_bf16,
                       acc_out ? acc_out + m * N : nullptr);
  }
  return hipGetLastError();
}

}  // namespace bitnet
