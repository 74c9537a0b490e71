// Weight quantisation: exact absolute-mean scale and ternary 2-bit packing.
//
// Method: onedollarvps.pages.dev, "如何在本地運行 BitNet B1.58（1-Bit LLM）",
// section 2 (technical background): weights are divided by their mean absolute
// value, then rounded and clipped to {-1, 0, +1}.  Storage: dashen-tech.com,
// "BitNet.cpp 深度解析", section 2.3 (I2_S): two bits per weight.
//
// gamma is RN32 of the EXACT mean: a 1-ulp change of gamma flips some of the
// ~10^8 weights of a large matrix, so the sum must not depend on summation order.
// Every finite fp32 |w| is an integer count of 2^-149 units: (2^23 + frac) shifted
// left by (biased exponent - 1), or frac for sub-normals.  Pass 1 adds the 24-bit
// significands into 256 uint64 buckets keyed by biased exponent (integer atomics:
// exact and order-free; kWqCopies copies of the buckets, by workgroup, spread the
// global atomics of the hot buckets over more addresses).  Pass 2 (one wave)
// forms the exact sum in a 320-bit integer, divides by N*K and rounds once to
// fp32.  Pass 3 ternarises and packs.
//
// T1 output (five codes per byte, a reading of the same pages' log2(3) ~ 1.58
// bits per weight): the codes c = q + 1 of the weights 80 b + 16 j + i of a row
// form the base-3 value v = sum_j c_j 3^j of byte i of block b, stored as the
// fixed-point fraction ceil(256 v / 243); rows are padded with q = 0 to whole
// 80-weight blocks of 16 bytes.  wq_pack_t1 writes it from the master weights,
// repack_t1 from the 2-bit layout.
//
// Workspace layout (device, caller-owned, >= kWqWorkspaceBytes):
//   [0, kWqThresholdAt)  uint64 buckets[kWqCopies][256]  (bucket 255 counts
//                        Inf/NaN weights)
//   kWqThresholdAt       float threshold  (see wq_finish)
#include "bitnet_internal.h"

#include <mutex>

namespace bitnet {

// Workspace of the allocation-free entry point (bitnet_quantize_weights_noalloc):
// one weight-quantisation workspace per device, created with the code object and
// held until the process ends.  Host code never passes this name to a kernel (on
// the host it is only a stand-in for the symbol): it uses the per-device address
// from hipGetSymbolAddress, taken once per device by wq_scratch.
static __device__ __align__(256) unsigned char scratch[kWqWorkspaceBytes];

namespace {

constexpr int kHistThreads = 256;
constexpr int kPackThreads = 256;

__global__ __launch_bounds__(256) void wq_clear(unsigned long long* __restrict__ buckets) {
  for (int i = threadIdx.x; i < kWqCopies * 256; i += 256) buckets[i] = 0ull;
}

template <bool BF16>
__device__ __forceinline__ uint32_t load_bits(const void* w, int64_t i) {
  if (BF16) return (uint32_t)(reinterpret_cast<const uint16_t*>(w)[i]) << 16;
  return reinterpret_cast<const uint32_t*>(w)[i];
}

__device__ __forceinline__ void hist_add(unsigned long long* sb, uint32_t bits) {
  const uint32_t e = (bits >> 23) & 0xffu;
  const uint32_t f = bits & 0x7fffffu;
  if (e == 0xffu) {
    atomicAdd(&sb[255], 1ull);                      // non-finite flag
  } else {
    const uint32_t m = e ? (f | 0x800000u) : f;     // units of 2^(max(e,1)-1-149)
    if (m) atomicAdd(&sb[e], (unsigned long long)m);
  }
}

// A thread's running sum for a window of kWin consecutive exponents starting at
// base >= 1 (set by its first nonzero normal weight, a few octaves below it): the
// weights of a matrix crowd into a few octaves, so most of them land here and
// only the rest become LDS atomics (which serialise when a wave's lanes hit the
// same bucket, as most of them would).  acc = sum of m * 2^(e - base), i.e. the
// window's part of S in units of 2^(base - 1): added to the buckets as
// (acc mod 2^(kWin-1)) in bucket base and (acc >> (kWin - 1)) in bucket
// base + kWin - 1, it contributes exactly the same S, and the buckets keep their
// bound: less than 2^24 per weight, plus less than 2^7 per thread.
constexpr int kWin = 8;
struct HistWindow {
  unsigned long long acc;
  int base;
};

__device__ __forceinline__ void window_add(HistWindow& h, unsigned long long* sb,
                                           uint32_t bits) {
  const uint32_t e = (bits >> 23) & 0xffu;
  const uint32_t f = bits & 0x7fffffu;
  if (e == 0xffu) {
    atomicAdd(&sb[255], 1ull);                      // non-finite flag
    return;
  }
  if (e == 0u) {                                    // sub-normal: units of 2^-149
    if (f) atomicAdd(&sb[0], (unsigned long long)f);
    return;
  }
  const uint32_t m = f | 0x800000u;                 // units of 2^(e-1-149)
  if (h.base < 0) h.base = min(max((int)e - (kWin - 3), 1), 254 - (kWin - 1));
  const uint32_t d = e - (uint32_t)h.base;
  if (d < (uint32_t)kWin)
    h.acc += (unsigned long long)m << d;
  else
    atomicAdd(&sb[e], (unsigned long long)m);
}

// Pass 1: per-exponent integer sums of the significands of |w|.
template <bool BF16>
__global__ __launch_bounds__(kHistThreads) void wq_hist(const void* __restrict__ w,
                                                        int64_t count, bool vec,
                                                        unsigned long long* __restrict__ gb) {
  __shared__ unsigned long long sb[256];
  sb[threadIdx.x] = 0ull;
  __syncthreads();
  // 16-byte vectors: 4 fp32 or 8 bf16 elements.
  constexpr int kVec = BF16 ? 8 : 4;
  const int64_t nvec = vec ? count / kVec : 0;
  const int64_t stride = (int64_t)gridDim.x * kHistThreads;
  const uint4* wv = reinterpret_cast<const uint4*>(w);
  HistWindow hw;
  hw.acc = 0ull;
  hw.base = -1;
  // four vectors in flight per thread (zeros past the end add nothing)
  constexpr int kIn = 4;
  for (int64_t v = (int64_t)blockIdx.x * kHistThreads + threadIdx.x; v < nvec;
       v += kIn * stride) {
    uint4 p[kIn];
#pragma unroll
    for (int u = 0; u < kIn; ++u)
      p[u] = v + u * stride < nvec ? wv[v + u * stride] : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < kIn; ++u) {
      const uint32_t d[4] = {p[u].x, p[u].y, p[u].z, p[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (BF16) {
          window_add(hw, sb, d[j] << 16);
          window_add(hw, sb, d[j] & 0xffff0000u);
        } else {
          window_add(hw, sb, d[j]);
        }
      }
    }
  }
  if (hw.acc) {
    const unsigned long long lo = hw.acc & ((1ull << (kWin - 1)) - 1ull);
    if (lo) atomicAdd(&sb[hw.base], lo);
    atomicAdd(&sb[hw.base + kWin - 1], hw.acc >> (kWin - 1));
  }
  for (int64_t i = nvec * kVec + (int64_t)blockIdx.x * kHistThreads + threadIdx.x; i < count;
       i += stride)
    hist_add(sb, load_bits<BF16>(w, i));
  __syncthreads();
  const unsigned long long s = sb[threadIdx.x];
  if (s) atomicAdd(&gb[256 * (blockIdx.x % kWqCopies) + threadIdx.x], s);
}

// L += x * 2^sh for a 320-bit L (five 64-bit limbs, least significant first);
// sh <= 253 and the sum stays below 2^320.
__device__ __forceinline__ void add_shifted(uint64_t L[5], uint64_t x, int sh) {
  const int li = sh >> 6, off = sh & 63;
  uint64_t add[5] = {0ull, 0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    if (i == li) add[i] = x << off;
    if (i == li + 1 && off) add[i] = x >> (64 - off);
  }
  uint64_t carry = 0ull;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t s = L[i] + add[i];
    const uint64_t c1 = s < L[i];
    L[i] = s + carry;
    carry = c1 | (L[i] < s);
  }
}

// L += R (320-bit).
__device__ __forceinline__ void add_limbs(uint64_t L[5], const uint64_t R[5]) {
  uint64_t carry = 0ull;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint64_t s = L[i] + R[i];
    const uint64_t c1 = s < L[i];
    L[i] = s + carry;
    carry = c1 | (L[i] < s);
  }
}

// Pass 2 (one wave): gamma* = max(RN32(S * 2^-149 / count), RN32(1e-5)) and the
// ternarisation threshold.  Lane l adds buckets 4l .. 4l + 3, each shifted to its
// place, into a 320-bit partial sum; five rounds of shuffles add the partials
// (integer sums: the same S in any order); lane 0 rounds.
//
// Threshold: q = +1 exactly when RN32(w / gamma*) > 0.5.  The fp32 values next to
// 0.5 are 0.5 - 2^-25 and 0.5 + 2^-24, and a tie at 0.5 + 2^-25 rounds to 0.5
// (even significand), so RN32(v) > 0.5 iff v > 0.5 + 2^-25, i.e. iff
// w > T = gamma* * (0.5 + 2^-25).  T is exact in fp64 (24-bit times 25-bit
// significands), and for fp32 w the test w > T equals w >= thr with thr the
// smallest fp32 above T.  q = -1 is the mirror image.  This gives the quotient's
// correctly rounded decision without a per-weight division.
__global__ __launch_bounds__(64) void wq_finish(const unsigned long long* __restrict__ b,
                                                 unsigned long long count,
                                                 float* __restrict__ w_scale,
                                                 float* __restrict__ thr_out) {
  const int lane = threadIdx.x;
  if (blockIdx.x != 0 || lane >= 64) return;
  // the copies' sums (each below 2^62: N K < 2^38 significands of < 2^24)
  unsigned long long bk[4], nonfinite = 0ull;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    bk[t] = 0ull;
#pragma unroll
    for (int c = 0; c < kWqCopies; ++c) bk[t] += b[256 * c + 4 * lane + t];
  }
#pragma unroll
  for (int c = 0; c < kWqCopies; ++c) nonfinite |= b[256 * c + 255];
  if (nonfinite != 0ull) {
    if (lane == 0) {
      *w_scale = __uint_as_float(0x7fc00000u);
      *thr_out = __uint_as_float(0x7fc00000u);
    }
    return;
  }
  // S = sum_{e>=1} b[e] * 2^(e-1) + b[0]
  uint64_t L[5] = {0ull, 0ull, 0ull, 0ull, 0ull};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int e = 4 * lane + t;
    if (e < 255) add_shifted(L, bk[t], e > 0 ? e - 1 : 0);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t R[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)L[i], o, 64);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(L[i] >> 32), o, 64);
      R[i] = ((uint64_t)hi << 32) | lo;
    }
    add_limbs(L, R);
  }
  if (lane != 0) return;

  float gamma = 0.0f;
  int top = -1;
  for (int i = 4; i >= 0; --i)
    if (L[i] != 0ull) { top = i; break; }
  if (top >= 0) {
    const int bitlen = 64 * top + (64 - __clzll(L[top]));
    const int p = bitlen - 64;  // S = H * 2^p + (lower bits)
    uint64_t H;
    bool sticky = false;
    if (p <= 0) {
      H = L[0] << (-p);
    } else {
      const int li = p >> 6, off = p & 63;
      H = L[li] >> off;
      if (off) H |= L[li + 1] << (64 - off);
      if (off && (L[li] & ((1ull << off) - 1ull))) sticky = true;
      for (int j = 0; j < li; ++j)
        if (L[j]) sticky = true;
    }
    // mean = (H + frac) * 2^(p-149) / count; count < 2^38 so q has >= 26 bits
    const uint64_t q = H / count;
    const uint64_t r = H - q * count;
    const int qb = 64 - __clzll(q);
    int sh = qb - 24;
    uint64_t kept = q >> sh;
    const uint64_t rem = q & ((1ull << sh) - 1ull);
    const uint64_t half = 1ull << (sh - 1);
    const bool inexact = sticky || (r != 0ull);
    if (rem > half || (rem == half && (inexact || (kept & 1ull)))) kept += 1ull;
    if (kept == (1ull << 24)) { kept >>= 1; sh += 1; }
    const int biased = sh + p - 149 + 150;  // value = kept * 2^(sh+p-149)
    if (biased >= 255) {
      gamma = __uint_as_float(0x7f800000u);
    } else if (biased >= 1) {
      gamma = __uint_as_float(((uint32_t)biased << 23) | (uint32_t)(kept & 0x7fffffull));
    } else {
      gamma = 0.0f;  // below 2^-126: the floor below takes over
    }
  }
  const float gstar = gamma > kEps ? gamma : kEps;
  *w_scale = gstar;
  const double T = (double)gstar * (0.5 + 0x1p-25);
  const float f = (float)T;
  *thr_out = ((double)f > T) ? f : __uint_as_float(__float_as_uint(f) + 1u);
}

template <bool BF16>
__device__ __forceinline__ uint32_t code_of(uint32_t bits, float thr) {
  const float a = __uint_as_float(bits & 0x7fffffffu);
  return a >= thr ? ((bits >> 31) ? 0u : 2u) : 1u;
}

// Pass 3: 16 weights -> one packed dword (weights 4j..4j+3 in byte j, first weight
// in the lowest bit pair).  Groups of four consecutive weights never straddle a row
// because K % 4 == 0, so the packed matrix is the flat row-major sequence of groups.
template <bool BF16>
__global__ __launch_bounds__(kPackThreads) void wq_pack(const void* __restrict__ w,
                                                        int64_t count,
                                                        bool vec, const float* __restrict__ thr_p,
                                                        uint8_t* __restrict__ out) {
  const float thr = *thr_p;
  const int64_t n16 = vec ? count / 16 : 0;
  const int64_t stride = (int64_t)gridDim.x * kPackThreads;
  for (int64_t v = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; v < n16; v += stride) {
    uint32_t bits[16];
    if (BF16) {
      const uint4* p = reinterpret_cast<const uint4*>(w) + 2 * v;
      const uint4 a = p[0], b = p[1];
      const uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bits[2 * j] = d[j] << 16;
        bits[2 * j + 1] = d[j] & 0xffff0000u;
      }
    } else {
      const uint4* p = reinterpret_cast<const uint4*>(w) + 4 * v;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 a = p[j];
        bits[4 * j] = a.x;
        bits[4 * j + 1] = a.y;
        bits[4 * j + 2] = a.z;
        bits[4 * j + 3] = a.w;
      }
    }
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < 16; ++j) word |= code_of<BF16>(bits[j], thr) << (2 * j);
    reinterpret_cast<uint32_t*>(out)[v] = word;
  }
  // tail: whole groups of four left after the last full 16
  const int64_t groups = count / 4;
  for (int64_t g = n16 * 4 + (int64_t)blockIdx.x * kPackThreads + threadIdx.x; g < groups;
       g += stride) {
    uint32_t byte = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) byte |= code_of<BF16>(load_bits<BF16>(w, 4 * g + i), thr) << (2 * i);
    out[g] = (uint8_t)byte;
  }
}

// Byte of the T1 layout for the codes c[0..4] of digits 0..4.
__device__ __forceinline__ uint32_t t1_byte(const uint32_t c[5]) {
  const uint32_t v = c[0] + 3u * c[1] + 9u * c[2] + 27u * c[3] + 81u * c[4];
  return (256u * v + 242u) / 243u;  // ceil(256 v / 243)
}

// 16 bytes (one block) from the codes of its five 16-weight digit groups: group j
// holds the codes of weights 16 j .. 16 j + 15 in bit pairs 2i..2i+1.
__device__ __forceinline__ uint4 t1_block(const uint32_t grp[5]) {
  uint32_t o[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t c[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) c[j] = (grp[j] >> (2 * i)) & 3u;
    o[i >> 2] |= t1_byte(c) << (8 * (i & 3));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Pass 3 for the T1 layout: one thread per 16-byte block (row n, block b).
// vec: K % 16 == 0 and a 16-byte aligned base, so each digit group is four (fp32)
// or two (bf16) 16-byte loads, entirely inside or past the row.
template <bool BF16>
__global__ __launch_bounds__(kPackThreads) void wq_pack_t1(const void* __restrict__ w, int64_t N,
                                                           int64_t K, bool vec,
                                                           const float* __restrict__ thr_p,
                                                           uint4* __restrict__ out) {
  const float thr = *thr_p;
  const int64_t nb = (K + 79) / 80;
  const int64_t total = N * nb;
  const int64_t stride = (int64_t)gridDim.x * kPackThreads;
  for (int64_t t = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; t < total; t += stride) {
    const int64_t n = t / nb, b = t - n * nb;
    uint32_t grp[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int64_t k0 = 80 * b + 16 * j;
      uint32_t word = 0u;
      if (vec && k0 < K) {
        uint32_t bits[16];
        if (BF16) {
          const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(w) +
                                                          n * K + k0);
          const uint4 x0 = p[0], x1 = p[1];
          const uint32_t d[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int h = 0; h < 8; ++h) {
            bits[2 * h] = d[h] << 16;
            bits[2 * h + 1] = d[h] & 0xffff0000u;
          }
        } else {
          const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(w) +
                                                          n * K + k0);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const uint4 x = p[h];
            bits[4 * h] = x.x;
            bits[4 * h + 1] = x.y;
            bits[4 * h + 2] = x.z;
            bits[4 * h + 3] = x.w;
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) word |= code_of<BF16>(bits[i], thr) << (2 * i);
      } else {
        for (int i = 0; i < 16; ++i) {
          const int64_t k = k0 + i;
          const uint32_t c = k < K ? code_of<BF16>(load_bits<BF16>(w, n * K + k), thr) : 1u;
          word |= c << (2 * i);
        }
      }
      grp[j] = word;
    }
    out[t] = t1_block(grp);
  }
}

// 2-bit layout -> T1, one thread per 16-byte block.  vec: K % 16 == 0 and a
// 4-byte aligned input, so each digit group is one packed dword.
__global__ __launch_bounds__(kPackThreads) void repack_t1(const uint8_t* __restrict__ in,
                                                          int64_t N, int64_t K, bool vec,
                                                          uint4* __restrict__ out) {
  const int64_t nb = (K + 79) / 80;
  const int64_t total = N * nb;
  const int64_t rowb = K / 4;
  const int64_t stride = (int64_t)gridDim.x * kPackThreads;
  for (int64_t t = (int64_t)blockIdx.x * kPackThreads + threadIdx.x; t < total; t += stride) {
    const int64_t n = t / nb, b = t - n * nb;
    uint32_t grp[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int64_t k0 = 80 * b + 16 * j;
      uint32_t word = 0x55555555u;  // padding: code 1
      if (vec && k0 < K) {
        word = reinterpret_cast<const uint32_t*>(in + n * rowb)[k0 / 16];
      } else if (k0 < K) {
        for (int i = 0; i < 16; i += 4) {
          if (k0 + i < K) {
            const uint32_t byte = in[n * rowb + (k0 + i) / 4];
            word = (word & ~(0xffu << (2 * i))) | (byte << (2 * i));
          }
        }
      }
      grp[j] = word;
    }
    out[t] = t1_block(grp);
  }
}

int grid_for(int64_t work_items, int threads, int max_blocks) {
  int64_t b = (work_items + threads - 1) / threads;
  if (b < 1) b = 1;
  if (b > max_blocks) b = max_blocks;
  return (int)b;
}

// Passes 1 and 2: gamma* into w_scale and the ternarisation threshold into the
// workspace.  Returns the threshold's device address.
float* launch_scale(const void* w, bool w_bf16, int64_t n, float* w_scale, void* workspace,
                    hipStream_t s) {
  auto* buckets = reinterpret_cast<unsigned long long*>(workspace);
  float* thr = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + kWqThresholdAt);
  hipLaunchKernelGGL(wq_clear, dim3(1), dim3(256), 0, s, buckets);
  // 16-byte vector loads need a 16-byte aligned base; otherwise every element
  // takes the scalar loop.
  const bool w_vec = ((uintptr_t)w & 15u) == 0;
  const int64_t per = w_bf16 ? 8 : 4;
  const int hist_blocks = grid_for(n / per + 1, kHistThreads, 2048);
  if (w_bf16)
    hipLaunchKernelGGL(wq_hist<true>, dim3(hist_blocks), dim3(kHistThreads), 0, s, w, n, w_vec,
                       buckets);
  else
    hipLaunchKernelGGL(wq_hist<false>, dim3(hist_blocks), dim3(kHistThreads), 0, s, w, n, w_vec,
                       buckets);
  hipLaunchKernelGGL(wq_finish, dim3(1), dim3(64), 0, s, buckets, (unsigned long long)n, w_scale,
                     thr);
  return thr;
}

}  // namespace

hipError_t launch_wq(const void* w, bool w_bf16, int64_t n, uint8_t* w_packed, float* w_scale,
                     void* workspace, hipStream_t s) {
  const float* thr = launch_scale(w, w_bf16, n, w_scale, workspace, s);
  // Packed dword stores need a 4-byte aligned output.
  const bool pack_vec = (((uintptr_t)w & 15u) == 0) && (((uintptr_t)w_packed & 3u) == 0);
  const int pack_blocks = grid_for(n / 16 + 1, kPackThreads, 8192);
  if (w_bf16)
    hipLaunchKernelGGL(wq_pack<true>, dim3(pack_blocks), dim3(kPackThreads), 0, s, w, n,
                       pack_vec, thr, w_packed);
  else
    hipLaunchKernelGGL(wq_pack<false>, dim3(pack_blocks), dim3(kPackThreads), 0, s, w, n,
                       pack_vec, thr, w_packed);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up once per device
// (with that device current) and kept: each device holds its own copy.
hipError_t wq_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_wq_noalloc(const void* w, bool w_bf16, int64_t n, uint8_t* w_packed,
                             float* w_scale, hipStream_t s) {
  void* ws = nullptr;
  const hipError_t e = wq_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_wq(w, w_bf16, n, w_packed, w_scale, ws, s);
}

hipError_t launch_wq_t1(const void* w, bool w_bf16, int64_t N, int64_t K, uint8_t* w_t1,
                        float* w_scale, void* workspace, hipStream_t s) {
  const float* thr = launch_scale(w, w_bf16, N * K, w_scale, workspace, s);
  const bool vec = (((uintptr_t)w & 15u) == 0) && (K % 16) == 0;
  const int blocks = grid_for(N * ((K + 79) / 80), kPackThreads, 8192);
  auto* out = reinterpret_cast<uint4*>(w_t1);
  if (w_bf16)
    hipLaunchKernelGGL(wq_pack_t1<true>, dim3(blocks), dim3(kPackThreads), 0, s, w, N, K, vec,
                       thr, out);
  else
    hipLaunchKernelGGL(wq_pack_t1<false>, dim3(blocks), dim3(kPackThreads), 0, s, w, N, K, vec,
                       thr, out);
  return hipGetLastError();
}

hipError_t launch_repack_t1(const uint8_t* w_packed, int64_t N, int64_t K, uint8_t* w_t1,
                            hipStream_t s) {
  const bool vec = (((uintptr_t)w_packed & 3u) == 0) && (K % 16) == 0;
  const int blocks = grid_for(N * ((K + 79) / 80), kPackThreads, 8192);
  hipLaunchKernelGGL(repack_t1, dim3(blocks), dim3(kPackThreads), 0, s, w_packed, N, K, vec,
                     reinterpret_cast<uint4*>(w_t1));
  return hipGetLastError();
}

}  // namespace bitnet
