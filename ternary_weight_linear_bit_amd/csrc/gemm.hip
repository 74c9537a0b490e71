// Prefill kernel (M > 16 tokens): dense int8 contraction on the matrix cores.
//
// Method: dashen-tech.com, "BitNet.cpp 深度解析", section 3.1: ternary weights turn
// the float matmul into an integer one.  At many tokens the contraction is
// compute-bound (hundreds of int8 ops per packed weight byte), so it runs on
// v_mfma_i32_32x32x32_i8 with the ternary weights expanded to int8 in registers.
//
// Workgroup tile: BM tokens x 64 WN output rows of one of up to four matrices that
// share the activations (q, k, v or gate, up), 2 WN waves as 2 (tokens) x WN
// (rows); a wave owns (BM / 2) tokens x 64 rows = (BM / 64) x 2 blocks of 32 x 32
// int32 accumulators.  K advances in steps of 128:
//  * activations: the workgroup stages the BM x 128 int8 tile into LDS (double
//    buffered, one barrier per step), byte-transposed within each 16-byte group;
//    a wave stages step s + 1 in between its matrix instructions of step s, so
//    its vector work overlaps its own matrix-core work;
//  * weights: each wave loads its 64 rows x 128 k of packed codes straight from
//    global memory (16 bytes per lane) and expands them in registers to the codes
//    c = q + 1 with one shift and mask per 2-bit field, whose k order matches the
//    transposed activations, so neither operand needs a per-element shuffle; the
//    matrix cores sum c * x and the epilogue subtracts each token's sum of x
//    (four dot-4 instructions per staged 16-byte group), which saves the byte
//    lookup per field that maps c to q;
//  * loads run D steps ahead of the matrix cores (kDepth = 2; 4 on 64 x 128 tiles).
// Lane (r, h) of a 32 x 32 x 32 operand holds row r and 16 k: with the 16 bytes
// lane h loads per row (k0 + 64h .. k0 + 64h + 63), MFMA j of a step sums over
// k0 + 64h + 16j + (0..15) for h = 0, 1; the A operand reads the matching LDS
// group.  The rescale y = RN32(float(acc) * RN32(gamma * d[m])) is fused into the
// store.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int NBW = 2;          // 32-row weight blocks per wave
constexpr int BK = 128;         // k per step

constexpr int kStride = BK;       // LDS bytes per staged token row (groups XOR-swizzled)

// LDS byte offset of 16-byte group kg of staged token row t (128-byte rows).  The
// group index is XORed with the low bits of t so that consecutive tokens reading
// the same group (the A operand) and the 8 groups of one row (staging writes)
// fall in distinct banks.
__device__ __forceinline__ int lds_group(int t, int kg) {
  return t * kStride + 16 * (kg ^ (t & 7));
}
constexpr int kXcds = 8;          // MI355X: 8 XCDs, each with its own L2
constexpr int kDepth = 2;         // steps of global loads in flight (default)

// Packed dword (16 codes) -> the codes c = q + 1 in {0, 1, 2} as an int8 operand
// in the 4x4-byte-transposed k order (byte 4i + b = code of k-offset 4b + i): one
// shift and one mask per 2-bit field.  The matrix cores then sum c * x, and the
// epilogue subtracts the token's sum of x (q = c - 1).
__device__ __forceinline__ v4i expand_codes(uint32_t w) {
  v4i a;
  a.x = (int)(w & 0x03030303u);
  a.y = (int)((w >> 2) & 0x03030303u);
  a.z = (int)((w >> 4) & 0x03030303u);
  a.w = (int)((w >> 6) & 0x03030303u);
  return a;
}

// Epilogue through LDS: a wave's BM/2 tokens x 64 rows of y, rescaled
// (y = RN32(float(acc - sum x) * RN32(gamma * d))) and rounded to the output type
// (E bytes), pass by pass through the wave's own slice of the activation buffers
// (free once the main loop's last barrier is passed), so that the stores go out
// as 16 bytes per lane, 128 bytes per output row and wave (one store per value
// would write 2 or 4 bytes per lane).  Units of 16 tokens x 64 rows: per unit a
// lane writes its 8 values x NBW rows, then 16-byte reads give each lane 16
// consecutive bytes of one token's row.  Rows of the slice are RB bytes, the two
// halves swapped for tokens with bit 2 set (the two half-waves write tokens 4
// apart, which then land in different banks).
template <int E, int BM, int WN>
__device__ __forceinline__ void store_tile_impl(void* y, const v16i (&acc)[BM / 64][NBW],
                                                const int* xsum, const float* xsc, float gamma,
                                                uint8_t* lds, int m0, int wrow0, int M, int N,
                                                int ldy) {
  constexpr int TB = BM / 64;
  constexpr int RB = 64 * E;                       // bytes per token row of the slice
  constexpr int U = 16 * RB;                       // bytes per unit of 16 tokens
  constexpr int R = 2 * BM * kStride / (2 * WN);   // LDS bytes per wave
  constexpr int UPP = R / U;                       // units per pass
  constexpr int UNITS = 2 * TB;
  static_assert(UPP >= 1 && UNITS % UPP == 0 && (UPP * U) % 1024 == 0, "epilogue passes");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wt = wave / WN;
  const int r = lane & 31, h = lane >> 5;
  uint8_t* base = lds + wave * R;
#pragma unroll
  for (int p = 0; p < UNITS / UPP; ++p) {
#pragma unroll
    for (int uu = 0; uu < UPP; ++uu) {
      const int u = p * UPP + uu, i = u >> 1, hq = u & 1;
#pragma unroll
      for (int vv = 0; vv < 8; ++vv) {
        const int v = 8 * hq + vv;
        const int tl = 8 * (vv >> 2) + 4 * h + (vv & 3);      // token within the unit
        const int ml = wt * (BM / 2) + 32 * i + 16 * hq + tl;
        const float sc = gamma * xsc[ml];
        const int xm = xsum[ml];
        float yv[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b) yv[b] = (float)(acc[i][b][v] - xm) * sc;
        static_assert(NBW == 2, "bf16 values are converted in pairs");
        const uint32_t pk = E == 2 ? bf16x2_rne(yv[0], yv[1]) : 0u;
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
          const int off = uu * U + tl * RB + (((32 * b + r) * E) ^ (((tl >> 2) & 1) * (RB / 2)));
          if constexpr (E == 2)
            *reinterpret_cast<uint16_t*>(base + off) = (uint16_t)(pk >> (16 * b));
          else
            *reinterpret_cast<float*>(base + off) = yv[b];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < UPP * U / 1024; ++q) {
      const int byte = q * 1024 + 16 * lane;
      const int uu = byte / U, rem = byte % U;
      const int tl = rem / RB, c16 = rem % RB;
      const uint4 val = *reinterpret_cast<const uint4*>(
          base + uu * U + tl * RB + (c16 ^ (((tl >> 2) & 1) * (RB / 2))));
      const int u = p * UPP + uu, i = u >> 1, hq = u & 1;
      const int m = m0 + wt * (BM / 2) + 32 * i + 16 * hq + tl;
      const int n = wrow0 + c16 / E;
      if (m < M) {
        char* dst = static_cast<char*>(y) + ((size_t)m * ldy + n) * E;
        if (n + 16 / E <= N) {
          // (non-temporal: the outputs are not read again by this launch, and
          // leaving L2 to the weight and activation tiles measured 1-2% faster)
          typedef unsigned int u4v __attribute__((ext_vector_type(4)));
          __builtin_nontemporal_store(*reinterpret_cast<const u4v*>(&val),
                                      reinterpret_cast<u4v*>(dst));
        } else {
          const uint32_t w[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
          for (int e = 0; e < 16 / E; ++e)
            if (n + e < N) {
              if constexpr (E == 2)
                reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
              else
                reinterpret_cast<uint32_t*>(dst)[e] = w[e];
            }
        }
      }
    }
  }
}

// WN waves along the output rows (2 along the tokens): BN = 32 * NBW * WN rows
// (prefill layout: at least two waves per SIMD, 256 registers at most,
// accumulators included)
template <int BM, int WN, int D, int LAYOUT>
__global__ __launch_bounds__(128 * WN, LAYOUT == 1 ? 2 : 1) void gemm_kernel(
    const GemmArgs args) {
  constexpr int kThreads = 128 * WN;
  constexpr int BN = 32 * NBW * WN;         // output rows per workgroup
  constexpr int TB = BM / 64;               // 32-token blocks per wave
  constexpr int XG = BM * (BK / 16) / kThreads;  // 16-byte activation groups per thread per step
  static_assert(BM <= kThreads, "one token scale per thread");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][BM * kStride];
  __shared__ int xsum[BM];                  // per token: sum of its int8 activations
  __shared__ float xsc[BM];                 // per token: its scale d
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wt = wave / WN, wr = wave % WN;
  const int r = lane & 31, h = lane >> 5;
  const int M = args.M, K = args.K;
  // Tiles are numbered token-tile-major over the row tiles of all the launch's
  // matrices (which share the activations).  XCD-aware order: workgroup b runs
  // on XCD b % 8 (round-robin dispatch); each XCD takes a contiguous run of
  // tiles, so the workgroups that share an activation tile share one XCD's L2.
  const int nbt = args.nb0[args.count];     // row tiles of all matrices
  const int tiles = nbt * ((M + BM - 1) / BM);
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int t = ((int)blockIdx.x % kXcds) * per_xcd + (int)blockIdx.x / kXcds;
  if (t >= tiles) return;
  const int mt = t / nbt, rt = t - mt * nbt;
  // this tile's matrix (entries past count have nb0 = nbt and are never chosen)
  const int jm = (rt >= args.nb0[1]) + (rt >= args.nb0[2]) + (rt >= args.nb0[3]);
  static_assert(kMaxGroup == 4, "matrix selection lists four matrices");
  const uint8_t* wp = args.wp[0];
  const float* w_scale = args.ws[0];
  void* y = args.y[0];
  int32_t* acc_out = args.acc[0];
  int N = args.n[0], nbase = 0, ldy = args.ld[0];
  if (jm >= 1) { wp = args.wp[1]; w_scale = args.ws[1]; y = args.y[1]; acc_out = args.acc[1]; N = args.n[1]; nbase = args.nb0[1]; ldy = args.ld[1]; }
  if (jm >= 2) { wp = args.wp[2]; w_scale = args.ws[2]; y = args.y[2]; acc_out = args.acc[2]; N = args.n[2]; nbase = args.nb0[2]; ldy = args.ld[2]; }
  if (jm >= 3) { wp = args.wp[3]; w_scale = args.ws[3]; y = args.y[3]; acc_out = args.acc[3]; N = args.n[3]; nbase = args.nb0[3]; ldy = args.ld[3]; }
  const int8_t* xq = args.xq;
  const float* x_scale = args.xs;
  const int y_bf16 = args.y_bf16;
  const int m0 = mt * BM;
  const int n0 = (rt - nbase) * BN;
  const uint32_t rowb = (uint32_t)K >> 2;
  const int steps = (K + BK - 1) / BK;   // K % 64 == 0; a last step of 64 k reads zeros past K

  // the epilogue's scalars, loaded first so that their latency hides behind the
  // main loop: gamma, and the tile's token scales (one per thread, zeros past M)
  const float gamma = __uint_as_float(
      __builtin_amdgcn_readfirstlane(bload4(make_uniform_rsrc(w_scale, 4u), 0u)));
  const float xs_t = __uint_as_float(
      bload4(make_uniform_rsrc(x_scale + m0, 4u * (uint32_t)min(BM, M - m0)),
             tid < BM ? 4u * (uint32_t)tid : kOob));

  // activations: group g = tid + 256 i of the BM x 128 tile (token g / 8, k-group g % 8);
  // tokens past M read zeros (range-checked buffer)
  const int mrows = min(BM, M - m0);
  const auto xr = make_uniform_rsrc(xq + (size_t)m0 * K, (uint32_t)mrows * (uint32_t)K);
  auto xoff = [&](int i, int k0) -> uint32_t {
    const int g = tid + kThreads * i;
    const int k = k0 + 16 * (g & 7);
    return k < K ? (uint32_t)(g >> 3) * (uint32_t)K + (uint32_t)k : kOob;
  };
  // weights: this wave's 64 rows; rows past N read zeros.  LAYOUT 0: rows of
  // K/4 bytes, a lane reads 16 bytes of its row (32 rows x 32 bytes per load).
  // LAYOUT 1 (prefill layout): 1024-byte blocks of 32 rows x 128 k, block
  // (row block, step) at (row block * steps + step) * 1024, in the lanes' order,
  // so a load reads 1 KiB contiguous (the padding rows and k read as code 1,
  // which meets zero activations or outputs that are not stored)
  const int wrow0 = n0 + wr * (32 * NBW);
  const int wrows = max(0, min(32 * NBW, N - wrow0));
  const uint32_t wblk = LAYOUT == 1 ? (uint32_t)steps * 1024u : 0u;   // bytes per row block
  const auto wrs = LAYOUT == 1
      ? make_uniform_rsrc(wp + (size_t)(wrow0 >> 5) * wblk, (uint32_t)((wrows + 31) >> 5) * wblk)
      : make_uniform_rsrc(wp + (size_t)wrow0 * rowb, (uint32_t)wrows * rowb);
  auto woff = [&](int b, int k0) -> uint32_t {
    if constexpr (LAYOUT == 1) {
      return (uint32_t)b * wblk + (uint32_t)(k0 >> 7) * 1024u + 16u * (uint32_t)lane;
    } else {
      const int k = k0 + 64 * h;
      return k < K ? (uint32_t)(32 * b + r) * rowb + ((uint32_t)k >> 2) : kOob;
    }
  };

  // (past the last step the offsets leave the buffers and the loads read zeros:
  // no branch around the loads, whose waits would then sit in a skippable block)
  // (the past-the-end bit is ORed in arithmetically: a select on it is turned
  // into a branch, which also drains every load in flight at the loop top)
  auto xload = [&](uint4 (&xv)[XG], int s) {
    const uint32_t past = (uint32_t)(s >= steps) << 31;
#pragma unroll
    for (int i = 0; i < XG; ++i) xv[i] = bload16(xr, xoff(i, s * BK) | past);
  };
  auto wload = [&](uint4 (&wv)[NBW], int s) {
    const uint32_t past = (uint32_t)(s >= steps) << 31;
#pragma unroll
    for (int b = 0; b < NBW; ++b) wv[b] = bload16(wrs, woff(b, s * BK) | past);
  };

  int rsum[XG] = {};   // partial sums of the activations this thread stages (token g / 8)
  // stage activation group i of a step into an LDS buffer (transposed within the
  // 16-byte group) and add it to the token sums
  auto stage = [&](const uint4& v, int i, uint8_t* buf) {
    const int g = tid + kThreads * i;
    const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      rsum[i] = __builtin_amdgcn_sdot4((int)in[e], 0x01010101, rsum[i], false);
    uint32_t o[4];
    if constexpr (LAYOUT == 1) {
      // the prefill layout's expanded weights are in natural k order
      o[0] = in[0];
      o[1] = in[1];
      o[2] = in[2];
      o[3] = in[3];
    } else {
      transpose4x4_bytes(in, o);
    }
    *reinterpret_cast<uint4*>(buf + lds_group(g >> 3, g & 7)) = make_uint4(o[0], o[1], o[2], o[3]);
  };
  auto aread = [&](const uint8_t* buf, int i, int j) -> v4i {
    return *reinterpret_cast<const v4i*>(buf + lds_group(wt * (BM / 2) + 32 * i + r, 4 * h + j));
  };

  v16i acc[TB][NBW];
#pragma unroll
  for (int i = 0; i < TB; ++i)
#pragma unroll
    for (int b = 0; b < NBW; ++b) acc[i][b] = (v16i){};

  // Step s: the matrix cores work on step s (activations staged in xs[s & 1],
  // weights in wv) while the same wave stages the activations of step s + 1
  // (xv) into the other buffer, one 16-byte group per k-slice j, so that its
  // vector work runs under its own matrix instructions.  Register set d holds
  // the weights of step s + d and the activations of step s + 1 + d.
  auto body = [&](uint4 (&xv)[XG], uint4 (&wv)[NBW], int s) {
    const uint8_t* cur = xs[s & 1];
    uint8_t* nxt = xs[(s + 1) & 1];
    uint32_t wd[NBW][4];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      wd[b][0] = wv[b].x;
      wd[b][1] = wv[b].y;
      wd[b][2] = wv[b].z;
      wd[b][3] = wv[b].w;
    }
    v4i a[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) a[i] = aread(cur, i, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v4i bop[NBW];
#pragma unroll
      for (int b = 0; b < NBW; ++b) bop[b] = expand_codes(wd[b][j]);
      v4i an[TB];
      if (j < 3) {
#pragma unroll
        for (int i = 0; i < TB; ++i) an[i] = aread(cur, i, j + 1);
      }
      static_assert(XG == 3 || 4 % XG == 0, "staged groups spread over the k-slices");
      if constexpr (XG == 3) {
        if (j < 3) stage(xv[j], j, nxt);
      } else if (j % (4 / XG) == 0) {
        stage(xv[j / (4 / XG)], j / (4 / XG), nxt);
      }
      if (j == 3) {
        // every use of xv and wv is above this point (the asm takes the last
        // expansion and the token sums), so the refills below reuse their
        // registers without copies, which would wait for the loads in flight
        asm volatile("" : "+v"(bop[0]), "+v"(bop[NBW - 1]), "+v"(rsum[0]), "+v"(rsum[XG - 1])
                     ::"memory");
        xload(xv, s + 1 + D);
        wload(wv, s + D);
      }
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int b = 0; b < NBW; ++b)
          acc[i][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], bop[b], acc[i][b], 0, 0, 0);
      if (j < 3) {
#pragma unroll
        for (int i = 0; i < TB; ++i) a[i] = an[i];
      }
    }
    lds_barrier();  // step s + 1 staged; nobody reads xs[s & 1] any more
  };

  // prologue: the activations of step 0, then the register sets in the order
  // the loop refills them; step 0 is staged before the loop
  uint4 x0[XG];
  xload(x0, 0);
  uint4 xv_[D][XG];
  uint4 wv_[D][NBW];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    asm volatile("" ::: "memory");
    xload(xv_[d], d + 1);
    wload(wv_[d], d);
  }
#pragma unroll
  for (int i = 0; i < XG; ++i) stage(x0[i], i, xs[0]);
  if (tid < BM) xsc[tid] = xs_t;   // loaded before x0, so no extra wait
  lds_barrier();
  // steps past the end (when D does not divide the step count) only add
  // zero products and stage zeros
  for (int s = 0; s < steps; s += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) body(xv_[d], wv_[d], s + d);
  }

  // token sums: the 8 threads of a token are consecutive lanes
#pragma unroll
  for (int i = 0; i < XG; ++i) {
    int v = rsum[i];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    if ((tid & 7) == 0) xsum[(tid >> 3) + (kThreads / 8) * i] = v;
  }
  __syncthreads();

  // D layout (32 x 32): lane l holds output row (n) l % 32 and tokens
  // 8 (v / 4) + 4 (l / 32) + v % 4 for its 16 values v
  if (acc_out) {
#pragma unroll
    for (int i = 0; i < TB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ml = wt * (BM / 2) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        const int m = m0 + ml;
        if (m < M) {
#pragma unroll
          for (int b = 0; b < NBW; ++b) {
            const int n = wrow0 + 32 * b + r;
            if (n < N) acc_out[(size_t)m * ldy + n] = acc[i][b][v] - xsum[ml];   // sum (c - 1) x
          }
        }
      }
  }
  const int es = y_bf16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(y) & 15u) == 0 && ((ldy * es) & 15) == 0) {
    if (y_bf16)
      store_tile_impl<2, BM, WN>(y, acc, xsum, xsc, gamma, &xs[0][0], m0, wrow0, M, N, ldy);
    else
      store_tile_impl<4, BM, WN>(y, acc, xsum, xsc, gamma, &xs[0][0], m0, wrow0, M, N, ldy);
    return;
  }
  // y not 16-byte aligned or rows not a whole number of 16 bytes: one store per value
#pragma unroll
  for (int i = 0; i < TB; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int ml = wt * (BM / 2) + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
      const int m = m0 + ml;
      if (m < M) {
        const float sc = gamma * xsc[ml];
        const int xm = xsum[ml];
        float yv[NBW];
#pragma unroll
        for (int b = 0; b < NBW; ++b) yv[b] = (float)(acc[i][b][v] - xm) * sc;
        const uint32_t pk = bf16x2_rne(yv[0], yv[1]);
#pragma unroll
        for (int b = 0; b < NBW; ++b) {
          const int n = wrow0 + 32 * b + r;
          if (n < N) {
            const size_t o = (size_t)m * ldy + n;
            if (y_bf16)
              reinterpret_cast<uint16_t*>(y)[o] = (uint16_t)(pk >> (16 * b));
            else
              reinterpret_cast<float*>(y)[o] = yv[b];
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

GemmPlan gemm_plan(int64_t M, const int* n, int count, int64_t K, int cus) {
  // Five tile shapes:
  //  * 256 tokens x 256 rows (8 waves of 128 x 64; one workgroup per compute
  //    unit, two waves per SIMD): a wave's weight expansion serves twice the
  //    tokens and the staging of the activations twice the rows, about 5 vector
  //    instructions per matrix instruction instead of 8 (vector and matrix
  //    instructions of one SIMD largely take turns, so this is the main cost
  //    besides the products).  Chosen when its tiles fill at least 80% of the
  //    compute units over the launch's rounds, or, at K >= 4096, at least 60%
  //    of them in a single round (its cheaper steps then outweigh the idle
  //    units: 2B down at 4096 tokens, 6912 -> 2560, 82 -> 76 us; 8B q+k+v at
  //    2048 tokens 54 -> 52 us; at K = 2560 the 2B o projection was slower);
  //  * 192 x 256 (8 waves of 96 x 64, three 32-token blocks each) when they run
  //    in a single round filling at least 80% of the compute units and 256 x 256
  //    tiles fill less than 80% (2B o and down projections at 4096 tokens: 160
  //    tiles of 256 x 256 on 256 compute units, 220 of 192 x 256: 35.9 -> 29.9 us
  //    and 78.9 -> 66 us; the per-step work is 3/4, the weight loads and their
  //    expansion the same);
  //  * 128 x 256 (8 waves of 64 x 64; one per compute unit), when its tiles fill
  //    80-100% of one round (from 90%: 2B gate+up at M = 512 went to these tiles,
  //    the layer 100.7 -> 98.7 us);
  //  * else 128 x 128 (4 waves; three workgroups per compute unit), or 64 x 128
  //    (4 waves of 32 x 64) when 128 x 128 tiles would not cover the compute
  //    units once: twice the tiles, each half as long, at some cost per product
  //    (the weight expansion serves half the tokens).  These short steps leave
  //    the loads' latency exposed, so the 64 x 128 kernel loads four steps ahead
  //    (2B layer at M = 512: 108 -> 100 us; three, five or more steps ahead, or
  //    deeper loads on the other shapes, measured no better).
  // Measured on the prefill shapes; 4 x 32-row blocks per wave measured slower
  // everywhere (registers: one wave per SIMD).
  GemmPlan p{128, 128, 0, 0};
  auto row_tiles = [&](int bn) {
    int64_t t = 0;
    for (int j = 0; j < count; ++j) t += (n[j] + bn - 1) / bn;
    return t;
  };
  const int64_t big_tiles = ((M + 255) / 256) * row_tiles(256);
  const int64_t big_rounds = (big_tiles + cus - 1) / cus;
  const bool big_full = big_tiles > 0 && 5 * big_tiles >= 4 * big_rounds * (int64_t)cus;
  // 192 x 256 tiles in a single round filling at least 80% of the compute units,
  // where 256 x 256 tiles fill less
  const int64_t tall_tiles = ((M + 191) / 192) * row_tiles(256);
  const bool tall = !big_full && tall_tiles <= cus && 5 * tall_tiles >= 4 * (int64_t)cus;
  const bool big = !tall && big_tiles > 0 &&
                   (big_full || (K >= 4096 && big_rounds == 1 && 5 * big_tiles >= 3 * (int64_t)cus));
  // A last round of 256 x 256 tiles that fills under 40% of the compute units
  // idles most of the chip for a whole tile time: the token tiles that fit in the
  // full rounds run as one launch, and the remaining tokens as a second launch
  // with its own tile choice (4096 x 13824 x 2560: 224-227 -> 206-216 us).
  if (big && big_rounds > 1 && 5 * (big_tiles - (big_rounds - 1) * cus) < 2 * (int64_t)cus) {
    const int64_t m1 = (big_rounds - 1) * cus / row_tiles(256) * 256;   // tokens
    if (m1 > 0 && m1 < M) p.first_tokens = m1;
  }
  // A last round left partly empty where the full rounds hold whole token tiles'
  // worth of row tiles (with more row tiles per token tile than divide the
  // compute units, the token split above cannot fill whole rounds): the row tiles
  // of the full rounds, the matrices taken in order, run as one launch, and the
  // remaining rows as a second launch with its own tile, when that tile is
  // smaller (8B gate+up at 2048 tokens: 896 tiles of 256 x 256 in 3.5 rounds ->
  // 768 in 3 rounds, then the last 4096 rows of up in one round of 128 x 256).
  if (big && big_rounds > 1 && p.first_tokens == 0 && big_tiles % cus != 0) {
    const int64_t tt = (M + 255) / 256;                  // token tiles
    const int64_t full = (big_rounds - 1) * (int64_t)cus;
    if (full % tt == 0) {
      const int64_t r1 = full / tt;                      // row tiles in the first launch
      int rest[kMaxGroup];
      int rc = 0;
      int64_t t0 = 0;
      for (int j = 0; j < count; ++j) {
        const int64_t tj = (n[j] + 255) / 256;
        if (t0 + tj > r1) rest[rc++] = (int)(n[j] - (t0 < r1 ? (r1 - t0) * 256 : 0));
        t0 += tj;
      }
      if (rc > 0 && gemm_plan(M, rest, rc, K, cus).bm != 256) p.first_rows = r1 * 256;
    }
  }
  const int64_t mt = (M + 127) / 128;
  const int64_t rows4 = row_tiles(256);
  const bool wide = !big && !tall && rows4 * mt <= cus && 10 * rows4 * mt >= 8 * (int64_t)cus;
  const bool small = !big && !tall && !wide && mt * row_tiles(128) <= cus;
  p.bm = tall ? 192 : big ? 256 : small ? 64 : 128;
  p.bn = big || wide || tall ? 256 : 128;
  return p;
}

hipError_t launch_gemm(GemmArgs a, hipStream_t s) {
  if (a.K % 64 != 0 || a.count < 1 || a.count > kMaxGroup) return hipErrorInvalidValue;
  for (int j = 0; j < a.count; ++j)
    if (a.ld[j] == 0) a.ld[j] = a.n[j];
  const GemmPlan pl = gemm_plan(a.M, a.n, a.count, a.K, device_cus());
  const size_t es = a.y_bf16 ? 2 : 4;
  if (pl.first_tokens > 0 && pl.first_tokens < a.M) {
    const int64_t m1 = pl.first_tokens;
    GemmArgs rest = a;
    rest.M = (int)(a.M - m1);
    rest.xq = a.xq + m1 * a.K;
    rest.xs = a.xs + m1;
    for (int j = 0; j < a.count; ++j) {
      rest.y[j] = static_cast<char*>(a.y[j]) + (size_t)m1 * a.ld[j] * es;
      if (a.acc[j]) rest.acc[j] = a.acc[j] + (size_t)m1 * a.ld[j];
    }
    a.M = (int)m1;
    const hipError_t e = launch_gemm(a, s);
    return e != hipSuccess ? e : launch_gemm(rest, s);
  }
  if (pl.first_rows > 0) {
    // rows [0, h) of each matrix in the first launch, [h, n) in the second: the
    // weights from row h on (prefill layout: 32-row blocks of ceil(K / 128) KiB),
    // the outputs from column h on with the matrix's own row stride
    const int64_t r1 = pl.first_rows / 256;
    GemmArgs head = a, rest = a;
    head.count = rest.count = 0;
    const int64_t blk = (int64_t)((a.K + 127) / 128) * 1024;
    int64_t t0 = 0;
    for (int j = 0; j < a.count; ++j) {
      const int64_t tj = (a.n[j] + 255) / 256;
      const int64_t h = t0 >= r1 ? 0 : t0 + tj <= r1 ? a.n[j] : (r1 - t0) * 256;
      if (h > 0) {
        const int k = head.count++;
        head.wp[k] = a.wp[j];
        head.ws[k] = a.ws[j];
        head.y[k] = a.y[j];
        head.acc[k] = a.acc[j];
        head.n[k] = (int)h;
        head.ld[k] = a.ld[j];
      }
      if (h < a.n[j]) {
        const int k = rest.count++;
        rest.wp[k] = a.wp[j] + (a.layout == 1 ? h / 32 * blk : h * (a.K / 4));
        rest.ws[k] = a.ws[j];
        rest.y[k] = static_cast<char*>(a.y[j]) + (size_t)h * es;
        rest.acc[k] = a.acc[j] ? a.acc[j] + h : nullptr;
        rest.n[k] = (int)(a.n[j] - h);
        rest.ld[k] = a.ld[j];
      }
      t0 += tj;
    }
    const hipError_t e = launch_gemm(head, s);
    return e != hipSuccess ? e : launch_gemm(rest, s);
  }
  const int bm = pl.bm, bn = pl.bn;
  const bool big = bm == 256, small = bm == 64, wide = bm == 128 && bn == 256, tall = bm == 192;
  int64_t nbt = 0;
  for (int j = 0; j < kMaxGroup; ++j) {
    a.nb0[j] = (int)nbt;
    if (j < a.count) nbt += (a.n[j] + bn - 1) / bn;
  }
  a.nb0[kMaxGroup] = (int)nbt;
  for (int j = a.count; j <= kMaxGroup; ++j) a.nb0[j] = (int)nbt;
  const int64_t tiles = nbt * ((a.M + bm - 1) / bm);
  if (tiles == 0) return hipSuccess;
  if (tiles > (int64_t)1 << 30) return hipErrorInvalidValue;  // grid and tile index limits
  const dim3 grid((unsigned)(((tiles + kXcds - 1) / kXcds) * kXcds));
  if (a.layout == 1) {
    if (big)
      hipLaunchKernelGGL((gemm_kernel<256, 4, kDepth, 1>), grid, dim3(512), 0, s, a);
    else if (tall)
      hipLaunchKernelGGL((gemm_kernel<192, 4, kDepth, 1>), grid, dim3(512), 0, s, a);
    else if (small)
      hipLaunchKernelGGL((gemm_kernel<64, 2, 4, 1>), grid, dim3(256), 0, s, a);
    else if (wide)
      hipLaunchKernelGGL((gemm_kernel<128, 4, kDepth, 1>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_kernel<128, 2, kDepth, 1>), grid, dim3(256), 0, s, a);
  } else {
    if (big)
      hipLaunchKernelGGL((gemm_kernel<256, 4, kDepth, 0>), grid, dim3(512), 0, s, a);
    else if (tall)
      hipLaunchKernelGGL((gemm_kernel<192, 4, kDepth, 0>), grid, dim3(512), 0, s, a);
    else if (small)
      hipLaunchKernelGGL((gemm_kernel<64, 2, 4, 0>), grid, dim3(256), 0, s, a);
    else if (wide)
      hipLaunchKernelGGL((gemm_kernel<128, 4, kDepth, 0>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_kernel<128, 2, kDepth, 0>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

// O3 rows (K/4 bytes, K % 64 == 0) -> the prefill layout: one thread per 16-byte
// chunk of the output (row 32 rb + r, k = 128 s + 64 h + 0..63), each dword's bit
// pairs transposed from (byte, pair) to (pair, byte); padding rows and k get
// code 1 (0x55 bytes).
__global__ __launch_bounds__(256) void repack_prefill_kernel(const uint8_t* __restrict__ w,
                                                            int64_t N, int64_t K, int64_t S,
                                                            int64_t chunks,
                                                            uint8_t* __restrict__ out) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  const int64_t blk = c >> 6;
  const int L = (int)(c & 63);
  const int64_t rb = blk / S, st = blk - rb * S;
  const int64_t n = 32 * rb + (L & 31);
  const int64_t k0 = 128 * st + 64 * (L >> 5);
  uint4 v = make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
  if (n < N && k0 < K) {
    const uint4 in = *reinterpret_cast<const uint4*>(w + n * (K >> 2) + (k0 >> 2));
    const uint32_t iw[4] = {in.x, in.y, in.z, in.w};
    uint32_t ow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o = 0;
#pragma unroll
      for (int t = 0; t < 16; ++t)    // weight t: byte t / 4, pair t % 4 -> byte t % 4, pair t / 4
        o |= ((iw[j] >> (8 * (t >> 2) + 2 * (t & 3))) & 3u) << (8 * (t & 3) + 2 * (t >> 2));
      ow[j] = o;
    }
    v = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  }
  reinterpret_cast<uint4*>(out)[c] = v;
}

int64_t prefill_layout_bytes(int64_t N, int64_t K) {
  return ((N + 31) / 32) * ((K + 127) / 128) * 1024;
}

hipError_t launch_repack_prefill(const uint8_t* w, int64_t N, int64_t K, uint8_t* out,
                                 hipStream_t s) {
  const int64_t S = (K + 127) / 128;
  const int64_t chunks = prefill_layout_bytes(N, K) / 16;
  if (chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(repack_prefill_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0,
                     s, w, N, K, S, chunks, out);
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
