// Decode chain: a stack of fused act-quant + ternary linear stages in one
// cooperative launch per token.
//
// Method: the same integer contraction as the decode kernel (dashen-tech.com,
// "BitNet.cpp 深度解析", section 3.1: with weights in {-1, 0, +1} every output is
// the sum of the inputs under +1 weights minus the sum under -1 weights) on the
// same per-token absmax int8 activations (communeify.com, "微軟 BitNet b1.58
// 震撼登場", section on BitNet b1.58 2B4T, quantisation details: W1.58A8).
// Stage i is bitnet_quant_linear_multi on its input; the launch runs the stages
// in order with a grid-wide barrier between them, so each stage sees every
// earlier stage's outputs and the results are those of the calls made one after
// another.
//
// Why one launch: a dependent launch per stage costs several microseconds of
// fixed time (dispatch, the first loads' latency, staging the input, the tail),
// during which HBM idles; a barrier inside a running kernel costs ~2.5 us, and
// across it the next stage's weights are already being read.
//
// Workgroup = 8 waves.  Waves 0-3 stream weights: a register ring of R loads
// (16 bytes per lane) runs over the whole chain, every stage's tiles one after
// another, so the next stage's first loads are in flight through the epilogue,
// the barrier and the staging of the next input.  Their tile loop, weight
// unpacking and v_mfma_i32_16x16x64_i8 contraction follow the decode kernel
// (K cut into 256-k super-chunks, wave w taking super-chunks w, w + 4, ...;
// partial tiles added into LDS with integer atomics).  Waves 4-7 stage the input:
// per token absmax, quantise, store into LDS in the unpacked weights' k order;
// wave 4 also applies the rescale epilogue and runs the grid barrier.  The
// streaming waves issue no other vector memory operations, so their waits stay
// partial; the barrier's polls come from a wave with no weight loads in flight,
// so it sees the release as soon as it happens.
//
// A stage's 16-row tiles (of all its matrices, one list) are spread evenly over
// the grid, so every workgroup streams about the same bytes.
//
// Cross-workgroup data (stage outputs read as later stage inputs) is written and
// read at agent scope (the sc1 cache policy: past the per-XCD caches, which are
// not coherent with each other), and a workgroup's stores are complete (vmcnt 0)
// before it arrives at the barrier.  The barrier: each workgroup adds 1 to its
// group's counter (workgroup b is in group b % 8); the group's first workgroup
// waits for its group, then adds 1 to the global counter; all wait for the
// global counter.  Counters only
// grow within a launch; the last workgroup to finish resets them.
// Every wait is bounded: past kSpinLimit polls the workgroup sets the plan's
// error word and stops waiting (as do all others once they see it), so a broken
// invariant ends the launch with a nonzero error word, never a hang.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kStreamWaves = 4;
constexpr int kGroups = kChainGroups;
constexpr int kSpinLimit = 1 << 20;
constexpr int kHold = 2;            // staging: groups per thread kept in registers between passes
constexpr int kBatch = 1;           // staging: groups per thread whose loads are issued together
constexpr int kCoherent = 16;       // buffer cache policy sc1: agent-coherent access

// Counter words of the plan header, one 256-byte line each.
__device__ __forceinline__ unsigned* grp_ctr(unsigned* c, int g) { return c + 64 * g; }
__device__ __forceinline__ unsigned* glob_ctr(unsigned* c) { return c + 64 * kGroups; }
__device__ __forceinline__ unsigned* exit_ctr(unsigned* c) { return c + 64 * (kGroups + 1); }
__device__ __forceinline__ unsigned* err_word(unsigned* c) { return c + kChainErrorAt / 4; }

__device__ __forceinline__ unsigned ld_agent(unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void add_agent(unsigned* p) {
  __hip_atomic_fetch_add(p, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until *p >= target.  False when the launch is being abandoned (the error
// word is set, by this wait running out or by another workgroup's).
__device__ bool wait_at_least(unsigned* p, unsigned target, unsigned* err) {
  for (int n = 0;; ++n) {
    if (ld_agent(p) >= target) return true;
    if ((n & 63) == 63 && ld_agent(err) != 0u) return false;
    if (n > kSpinLimit) {
      st_agent(err, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Barrier number i (0-based) over the grid; called by one lane per workgroup
// after its stores are complete.  Workgroup b adds 1 to its group's counter
// (group b % 8); the group's first workgroup waits for the group, then adds 1 to
// the global counter; every workgroup waits for the global counter.
__device__ void grid_barrier(unsigned* ctr, int i, int G) {
  unsigned* err = err_word(ctr);
  if (ld_agent(err) != 0u) return;
  const int b = (int)blockIdx.x;
  const int groups = G < kGroups ? G : kGroups;
  const int g = b % groups;
  add_agent(grp_ctr(ctr, g));
  if (b < groups) {
    const unsigned members = (unsigned)((G - g + groups - 1) / groups);
    if (!wait_at_least(grp_ctr(ctr, g), (unsigned)(i + 1) * members, err)) return;
    add_agent(glob_ctr(ctr));
  }
  wait_at_least(glob_ctr(ctr), (unsigned)(i + 1) * (unsigned)groups, err);
}

// The stage's descriptor fields a streaming wave keeps in scalar registers
// (separate fields, no arrays: an array picked by a computed index would be kept
// in scratch memory).
struct Stage {
  const uint8_t *wp0, *wp1, *wp2, *wp3;
  int n0, n1, n2, n3;
  int tc1, tc2, tc3, total;
  int K, count;
};
__device__ __forceinline__ Stage load_stage(const ChainStage& d) {
  Stage s;
  s.wp0 = d.wp[0];
  s.wp1 = d.wp[1];
  s.wp2 = d.wp[2];
  s.wp3 = d.wp[3];
  s.n0 = d.n[0];
  s.n1 = d.n[1];
  s.n2 = d.n[2];
  s.n3 = d.n[3];
  s.tc1 = d.tc0[1];
  s.tc2 = d.tc0[2];
  s.tc3 = d.tc0[3];
  s.total = d.tc0[kMaxGroup];
  s.K = d.K;
  s.count = d.count;
  return s;
}

// This workgroup's tiles of a stage: [t0, t0 + ntiles) of the stage's tile list.
__device__ __forceinline__ void my_tiles(int total, int G, int b, int& t0, int& ntiles) {
  const int base = total / G, rem = total - base * G;
  t0 = b * base + min(b, rem);
  ntiles = base + (b < rem ? 1 : 0);
}

// Buffer descriptor of global tile t (rows past N read as zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const Stage& s, int t) {
  const uint8_t* wp = s.wp0;
  int n = s.n0, tc = 0;
  if (s.count > 1 && t >= s.tc1) { wp = s.wp1; n = s.n1; tc = s.tc1; }
  if (s.count > 2 && t >= s.tc2) { wp = s.wp2; n = s.n2; tc = s.tc2; }
  if (s.count > 3 && t >= s.tc3) { wp = s.wp3; n = s.n3; tc = s.tc3; }
  const uint32_t rowb = (uint32_t)s.K >> 2;
  const int row0 = (t - tc) * 16;
  const int rows = max(0, min(16, n - row0));
  return make_uniform_rsrc(wp + (size_t)row0 * rowb, (uint32_t)rows * rowb);
}

// Loads per lane of wave `wave` for one tile of K: super-chunks wave, wave + 4, ...
__device__ __forceinline__ int wave_loads(int K, int wave) {
  const int S = ((K >> 6) + 3) >> 2;
  return S > wave ? (S - wave + 3) >> 2 : 0;
}

template <int R>
__global__ __launch_bounds__(kChainThreads) void chain_kernel(const ChainStage* __restrict__ st,
                                                             unsigned* ctr, int n_stages, int M,
                                                             int kstride, int tmax) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = (int)gridDim.x;
  const int b = (int)blockIdx.x;
  uint8_t* xs = smem;                                     // [M][kstride] staged int8 input
  uint8_t* zero = smem + M * kstride;                     // 64 zero bytes
  int* part = reinterpret_cast<int*>(zero + 64);          // [tmax][16 rows][16 tokens]
  unsigned* amax = reinterpret_cast<unsigned*>(part + tmax * 256);  // [4] per-token absmax bits
  float* dsc = reinterpret_cast<float*>(amax + 4);        // [4] token scales

  for (int i = tid; i < tmax * 64; i += kChainThreads)
    reinterpret_cast<uint4*>(part)[i] = make_uint4(0, 0, 0, 0);
  if (tid < 16) reinterpret_cast<uint32_t*>(zero)[tid] = 0u;
  if (tid < 4) amax[tid] = 0u;

  if (wave < kStreamWaves) {
    // ------------------------------------------------------------ streaming
    const int r = lane & 15;  // A operand: row of the tile; B operand: token
    const int g = lane >> 4;  // 16-k block of the operand within a 64-k chunk
    // Producer: its stage, tiles and this wave's super-chunks, one load per call.
    // Every stage takes a multiple of R slots, at least R (slots past the stage's
    // loads read zeros: out of range), so the consumer's last round of a stage
    // refills the ring with exactly the next stage's first R loads.
    int pq = 0, pQ = 0, ptp = 0, pjp = 0, pJ = 1, pC = 0, pt0 = 0;
    uint32_t prowb = 0;
    Stage ps{};
    auto prs = make_rsrc(nullptr, 0u);
    auto pset = [&](int s) {
      pq = 0;
      ptp = 0;
      pjp = 0;
      pQ = 0;
      if (s < n_stages) {
        ps = load_stage(st[s]);
        int nt;
        my_tiles(ps.total, G, b, pt0, nt);
        pC = ps.K >> 6;
        prowb = (uint32_t)ps.K >> 2;
        pJ = wave_loads(ps.K, wave);
        pQ = nt * pJ;
        prs = tile_rsrc(ps, pt0);
      }
    };
    auto next_load = [&]() -> uint4 {
      const bool real = pq < pQ;
      const int c = 4 * (wave + 4 * pjp) + g;
      const uint4 v = bload16(prs, real && c < pC ? (uint32_t)r * prowb + 16u * (uint32_t)c : kOob);
      ++pq;
      if (real && ++pjp == pJ) {
        pjp = 0;
        ++ptp;
        prs = tile_rsrc(ps, pt0 + ptp);
      }
      return v;
    };
    pset(0);
    uint4 ring[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      ring[u] = next_load();
      asm volatile("" ::: "memory");  // keep the ring's loads in slot order
    }
    lds_barrier();  // B0: LDS cleared

    for (int s = 0; s < n_stages; ++s) {
      const ChainStage& d = st[s];
      const int K = d.K;
      int t0, ntiles;
      my_tiles(d.tc0[kMaxGroup], G, b, t0, ntiles);
      const int C = K >> 6;
      const int J = wave_loads(K, wave);
      const int Q = ntiles * J;
      const int Qp = Q > R ? (Q + R - 1) / R * R : R;
      const int bt = r < M ? r * kstride : -1;
      const int zoff = M * kstride;
      lds_barrier();  // B1: staging pass 1 done
      lds_barrier();  // B2: input staged
      int tc = 0, jc = 0;
      v4i acc = {0, 0, 0, 0};
      for (int q0 = 0; q0 < Qp; q0 += R) {
        if (q0 + R >= Qp) pset(s + 1);  // this round's refills start the next stage
#pragma unroll
        for (int u = 0; u < R; ++u) {
          const int c = 4 * (wave + 4 * jc) + g;
          v4i a0 = unpack_weights_transposed(ring[u].x);
          v4i a1 = unpack_weights_transposed(ring[u].y);
          v4i a2 = unpack_weights_transposed(ring[u].z);
          v4i a3 = unpack_weights_transposed(ring[u].w);
          // unpack before the refill, so the refill can land in the same registers
          asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)::"memory");
          ring[u] = next_load();
          const int bb = (bt >= 0 && c < C && tc < ntiles) ? bt + 64 * c : zoff;
          const v4i* bp = reinterpret_cast<const v4i*>(xs + bb);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bp[0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bp[1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, bp[2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, bp[3], acc, 0, 0, 0);
          if (++jc == J) {
            // D layout: the lane holds rows 4g..4g+3 of the tile for token r
            if (tc < ntiles && r < M) {
              int* pt = part + tc * 256 + (4 * g) * 16 + r;
#pragma unroll
              for (int v = 0; v < 4; ++v) atomicAdd(pt + 16 * v, acc[v]);
            }
            acc = (v4i){0, 0, 0, 0};
            jc = 0;
            ++tc;
          }
        }
      }
      lds_barrier();  // B3: partial tiles complete
      if (s + 1 < n_stages) lds_barrier();  // B4: grid barrier passed
    }
    return;
  }

  // -------------------------------------------------------------- staging
  const int sid = tid - 64 * kStreamWaves;        // 0 .. 255
  const int lgG = 8 - (M > 1 ? 32 - __builtin_clz(M - 1) : 0);
  const int Gt = 1 << lgG;                        // threads per token (>= 64)
  const int tk = sid >> lgG;
  const int jg = sid & (Gt - 1);
  const bool control = wave == kStreamWaves;
  lds_barrier();  // B0

  for (int s = 0; s < n_stages; ++s) {
    const ChainStage& d = st[s];
    const int K = d.K;
    const int count = d.count;
    int t0, ntiles;
    my_tiles(d.tc0[kMaxGroup], G, b, t0, ntiles);
    const bool active = ntiles > 0;
    const int K16 = K >> 4;
    const bool xbf = (d.flags & 1) != 0;
    const uint32_t es = xbf ? 2u : 4u;
    float gam[kMaxGroup] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (control && active) {
#pragma unroll
      for (int j = 0; j < kMaxGroup; ++j)
        if (j < count) gam[j] = *as_global(d.ws[j]);
    }
    const auto xr = make_uniform_rsrc(d.x, (uint32_t)M * (uint32_t)K * es);
    // raw words of group c of this thread's token, read at agent scope
    auto load_raw = [&](int c, uint4 raw[4]) {
      const uint32_t base = ((uint32_t)tk * (uint32_t)K + 16u * (uint32_t)c) * es;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        if (h < (xbf ? 2 : 4)) {
          const v4i t = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(base + 16u * h), 0, kCoherent);
          raw[h] = make_uint4((uint32_t)t.x, (uint32_t)t.y, (uint32_t)t.z, (uint32_t)t.w);
        }
      }
    };
    auto to_f32 = [&](const uint4 raw[4], float v[16]) {
      if (xbf) raw_to_f32<true>(raw, v);
      else raw_to_f32<false>(raw, v);
    };
    const int nb = (K16 + Gt - 1) >> lgG;         // groups per thread
    float astar = 0.0f;
    // quantise 16 values of group c with s_t and stage them (workgroup 0 also
    // writes x_q)
    auto put = [&](int c, const float* v, float s_t) {
      const uint4 q = make_uint4(quant4(v, s_t), quant4(v + 4, s_t), quant4(v + 8, s_t),
                                 quant4(v + 12, s_t));
      store_transposed(xs + tk * kstride + 16 * c, q);
      if (b == 0) reinterpret_cast<uint4*>(d.xq_out + (size_t)tk * K)[c] = q;
    };
    // Pass 1: the token's absmax over the whole input (the first kHold groups of
    // each thread stay in registers); pass 2: quantise, reading the other groups
    // again.  Loads are issued kBatch groups at a time.
    float hold[kHold][16];
    if (active && tk < M) {
      float m = 0.0f;
#pragma unroll
      for (int h = 0; h < kHold; ++h) {
        const int c = jg + Gt * h;
        if (h < nb && c < K16) {
          uint4 raw[4];
          load_raw(c, raw);
          to_f32(raw, hold[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < kHold; ++h)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (h < nb && jg + Gt * h < K16) m = fmaxf(m, fabsf(hold[h][e]));
      for (int h0 = kHold; h0 < nb; h0 += kBatch) {
        uint4 raw[kBatch][4];
#pragma unroll
        for (int h = 0; h < kBatch; ++h) {
          const int c = jg + Gt * (h0 + h);
          if (h0 + h < nb && c < K16) load_raw(c, raw[h]);
        }
#pragma unroll
        for (int h = 0; h < kBatch; ++h) {
          const int c = jg + Gt * (h0 + h);
          if (h0 + h < nb && c < K16) {
            float v[16];
            to_f32(raw[h], v);
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
          }
        }
      }
      m = wave_max(m);
      if (lane == 0) atomicMax(&amax[tk], __float_as_uint(m));
    }
    lds_barrier();  // B1
    if (active && tk < M) {
      astar = fmaxf(__uint_as_float(amax[tk]), kEps);
      const float s_t = kQb / astar;
#pragma unroll
      for (int h = 0; h < kHold; ++h) {
        const int c = jg + Gt * h;
        if (h < nb && c < K16) put(c, hold[h], s_t);
      }
      for (int h0 = kHold; h0 < nb; h0 += kBatch) {
        uint4 raw[kBatch][4];
#pragma unroll
        for (int h = 0; h < kBatch; ++h) {
          const int c = jg + Gt * (h0 + h);
          if (h0 + h < nb && c < K16) load_raw(c, raw[h]);
        }
#pragma unroll
        for (int h = 0; h < kBatch; ++h) {
          const int c = jg + Gt * (h0 + h);
          if (h0 + h < nb && c < K16) {
            float v[16];
            to_f32(raw[h], v);
            put(c, v, s_t);
          }
        }
      }
    }
    if (active && tk < M && jg == 0) {
      const float dt = astar / kQb;
      dsc[tk] = dt;
      if (b == 0) d.xs_out[tk] = dt;
    }
    lds_barrier();  // B2
    lds_barrier();  // B3: the streaming waves' partial tiles are complete
    if (control) {
      // rescale y = RN32(float(acc) * RN32(gamma * d[t])), stored at agent scope,
      // index i = (tile * M + token) * 16 + row
      const bool ybf = (d.flags & 2) != 0;
      const int tc1 = d.tc0[1], tc2 = d.tc0[2], tc3 = d.tc0[3];
      const int n0 = d.n[0], n1 = d.n[1], n2 = d.n[2], n3 = d.n[3];
      char* y0 = static_cast<char*>(d.y[0]);
      char* y1 = static_cast<char*>(d.y[1]);
      char* y2 = static_cast<char*>(d.y[2]);
      char* y3 = static_cast<char*>(d.y[3]);
      int32_t *c0 = d.acc[0], *c1 = d.acc[1], *c2 = d.acc[2], *c3 = d.acc[3];
      for (int i = lane; i < ntiles * M * 16; i += 64) {
        const int row = i & 15;
        const int tt = i >> 4;
        const int tl = tt / M;
        const int t = tt - tl * M;
        const int gt = t0 + tl;
        int tcj = 0, nrows = n0;
        char* yp = y0;
        int32_t* accp = c0;
        float g = gam[0];
        if (count > 1 && gt >= tc1) { tcj = tc1; nrows = n1; yp = y1; accp = c1; g = gam[1]; }
        if (count > 2 && gt >= tc2) { tcj = tc2; nrows = n2; yp = y2; accp = c2; g = gam[2]; }
        if (count > 3 && gt >= tc3) { tcj = tc3; nrows = n3; yp = y3; accp = c3; g = gam[3]; }
        const int n = (gt - tcj) * 16 + row;
        int* pp = part + tl * 256 + row * 16 + t;
        const int accv = *pp;
        *pp = 0;
        if (n < nrows) {
          const float yv = (float)accv * (g * dsc[t]);
          const uint32_t o = (uint32_t)t * (uint32_t)nrows + (uint32_t)n;
          if (accp) as_global(accp)[o] = accv;
          // agent-scope stores: later stages on other XCDs read them
          if (ybf) {
            const uint16_t h = float_to_bf16_rne(yv);
            __hip_atomic_store(as_global(reinterpret_cast<uint16_t*>(yp)) + o, h, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          } else {
            __hip_atomic_store(as_global(reinterpret_cast<uint32_t*>(yp)) + o, __float_as_uint(yv),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
      if (lane < 4) amax[lane] = 0u;
      if (s + 1 < n_stages) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this workgroup's outputs are out
        if (lane == 0) grid_barrier(ctr, s, G);
      }
    }
    if (s + 1 < n_stages) lds_barrier();  // B4
  }
  if (control) {
    // the last workgroup out resets the counters for the next launch
    unsigned done = 0;
    if (lane == 0)
      done = __hip_atomic_fetch_add(exit_ctr(ctr), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    done = (unsigned)__shfl((int)done, 0);
    if (done + 1 == (unsigned)G) {
      if (lane < kGroups) st_agent(grp_ctr(ctr, lane), 0u);
      if (lane == 0) {
        st_agent(glob_ctr(ctr), 0u);
        st_agent(exit_ctr(ctr), 0u);
      }
    }
  }
}

template <int R>
const void* chain_kernel_for() {
  return reinterpret_cast<const void*>(chain_kernel<R>);
}

const void* chain_select(int ring) {
  if (ring <= 4) return chain_kernel_for<4>();
  if (ring <= 8) return chain_kernel_for<8>();
  return chain_kernel_for<16>();
}

}  // namespace

size_t chain_lds_bytes(int M, int kmax, int tmax) {
  return (size_t)M * (size_t)(kmax + 16) + 64 + (size_t)tmax * 1024 + 32;
}

size_t chain_plan_bytes(int n_stages) {
  return kChainHeaderBytes + (size_t)n_stages * sizeof(ChainStage);
}

int chain_grid(int M, int kmax, int tmax, int ring) {
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, chain_select(ring), kChainThreads,
                                                   chain_lds_bytes(M, kmax, tmax)) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int per_cu = occ < 2 ? occ : 2;
  return per_cu * device_cus();
}

hipError_t launch_chain(const void* plan, int n_stages, int M, int grid, int kmax, int tmax,
                        int ring, hipStream_t s) {
  char* base = static_cast<char*>(const_cast<void*>(plan));
  const auto* st = reinterpret_cast<const ChainStage*>(base + kChainHeaderBytes);
  unsigned* ctr = reinterpret_cast<unsigned*>(base);
  int kstride = kmax + 16;
  void* args[] = {&st, &ctr, &n_stages, &M, &kstride, &tmax};
  return hipLaunchCooperativeKernel(chain_select(ring), dim3((unsigned)grid),
                                    dim3(kChainThreads), args,
                                    (unsigned)chain_lds_bytes(M, kmax, tmax), s);
}

}  // namespace bitnet
