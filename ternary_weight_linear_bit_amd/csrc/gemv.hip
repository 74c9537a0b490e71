// Decode kernel (M <= 16 tokens): stream packed ternary weights from HBM and
// contract them with int8 activations on the int8 matrix cores.
//
// Method: dashen-tech.com, "BitNet.cpp 深度解析", section 3.1 (integer matmul):
// with weights in {-1, 0, +1} each output is the sum of the inputs under +1
// weights minus the sum under -1 weights, i.e. the dot product of the signed
// weights with the int8 activations.  Every weight is carried as its 2-bit code
// c = q + 1 in {0, 1, 2} (section 2.3: two bits per weight) and turned back into
// the int8 value q in registers, so the matrix cores contract q with x directly.
//
// Design for gfx950 (the pages' kernels are CPU SIMD and lookup-table code):
//  * Workgroup = NW = 4 waves (8 where a launch has at most one tile per compute
//    unit, so that each unit still runs 8 waves); it owns a run of consecutive
//    16-row tiles (of up to kMaxGroup matrices that share the activations).  One
//    tile per workgroup for small launches; large ones spread the tiles over two
//    workgroups per CU, each matrix split on its own or, for some launches, all
//    matrices' tiles as one list in runs that may cross into the next matrix
//    (launch_gemv: balanced runs, or skewed runs where the first-dispatched
//    workgroup of each CU takes more, or equal runs where the second one stages
//    its input at a raised wave priority, PRIO).  K is cut into 256-k
//    super-chunks; wave w takes super-chunks w, w + NW, ..., so one wave load
//    instruction covers 16 rows x 64 contiguous bytes and the waves read 64 NW
//    contiguous bytes of each row per step.
//  * The activations are staged once per workgroup into LDS, byte-transposed
//    within each 16-byte group; this is the order in which a shift, a mask and a
//    byte lookup per field, (w >> 2i) & 0x03030303, unpack the weights, so no
//    per-weight shuffle is needed.  When M * K exceeds the LDS budget, K is
//    processed in phases.
//  * Each wave streams its (tile, super-chunk) sequence with raw buffer loads
//    (16 bytes per lane; rows past N and chunks past K read as zeros) through a
//    ring of R loads in flight that runs on across tiles.  The first loads are
//    issued before the activations are staged, and the LDS-only barriers do not
//    drain them.
//  * v_mfma_i32_16x16x64_i8: A = 16 rows x 64 k of weights (registers), B = 64 k x
//    16 tokens (LDS; tokens >= M read a zero slot), int32 accumulate; the four
//    lane groups take four 16-k blocks, so the matrix core also sums along k.
//  * When a wave finishes a tile it adds its partial tile into LDS with integer
//    atomics (exact in any order); after one barrier the workgroup applies
//    y = RN32(float(acc) * RN32(gamma * d[m])).
//
// XMODE 1-8 fuse the per-token absmax activation quantisation (fp32 / bf16 input,
// M <= kMaxFusedM, one phase): the workgroup quantises the activations with the
// same results as the standalone kernel while staging them (one read of the
// input: each thread's first groups of 16, eight without a prologue and two with
// one, stay in registers between the absmax and the quantise pass; more than
// three groups per thread without a prologue take the eight-group variant), and
// workgroup 0 also writes x_q and x_scale.  With a prologue the weight loads are
// non-temporal, so that the prologue's inputs stay in L2.
// XMODE 3-8 add the layer's input prologue (communeify.com page on BitNet b1.58
// 2B4T, architecture item: squared-ReLU activation, subln norm, no biases): the
// input may be the gate projection, gated as RN32(RN32(relu(x)^2) * up), and / or
// RMS-normalised as u = RN32(RN32(v r) w), r = RN32(1/sqrt(RN32(ms + eps))),
// ms the exactly rounded mean of v^2 (float64 sum of squares over the token's
// threads; near a rounding boundary an exact integer sum in LDS), and u quantised.
//
// FMT 1 reads weights packed five per byte (reading T1: the codes' base-3 value
// v as the fixed-point fraction ceil(256 v / 243); byte i of a 16-byte block
// holds the weights 16 j + i of the block's 80 as digit j).  Digit j of the
// block's 16 bytes covers 16 consecutive weights, so a lane's 16 bytes unpack
// into five natural-order 16-weight operands and the activations are staged
// untransposed.  A digit is the integer part of three times the fraction: one
// packed 16-bit multiply-add per two bytes and digit, whose high byte is the
// signed weight directly (3f - 256 = 256 (c - 1) + next fraction).
#include "bitnet_internal.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;              // 4 waves (eight-wave launches: 512)
constexpr int kMaxTiles = 16;              // row tiles per workgroup
constexpr int kMaxM = 16;
constexpr int kMaxFusedM = 4;
constexpr int kXBudget = 16 * (4096 + 16); // LDS bytes of staged activations per phase:
                                           // K = 4096 in one phase at M = 16 (gfx950's
                                           // 160 KiB of LDS still holds two workgroups
                                           // of up to 14 tiles)
constexpr int kFusedXBudget = 46 * 1024;   // fused quantisation: M * K staged at most
constexpr int kStageBatch = 8;             // 16-byte activation loads per thread per batch
constexpr int kHold = 2;                   // fused with a prologue: groups per thread held in
                                           // registers between the absmax and quantise passes
constexpr int kHoldPlain = 8;              // fused, no prologue: K <= 32768 at M = 1 stays in
                                           // registers (a long input is then read once, with
                                           // all its loads in flight together)
constexpr int64_t kLatencyBytes = 6000000; // launches above this use the bandwidth regime
constexpr int kWgsPerCu = 2;               // bandwidth regime: workgroups per compute unit
constexpr int kFlightLoads = 4096;         // target 1 KiB loads in flight over the chip
constexpr int kPrioSplit = 256;            // MI355X compute units (gemv_kernel PRIO)

// zero slot: one B operand set read for tokens >= M and chunks past the end
constexpr int zero_bytes(int fmt) { return fmt ? 96 : 64; }
// LDS row of one token's staged activations for a phase of kx weights (T1
// stages whole 80-k blocks)
constexpr int stage_stride(int kx, int fmt) {
  return fmt ? 80 * ((kx + 79) / 80) + 16 : kx + 16;
}
// (token, 4096-k block) pieces the int8 staging loads for a phase of klen weights
constexpr int stage_pieces(int M, int klen, int fmt) {
  const int groups = fmt ? 5 * ((klen + 79) / 80) : klen / 16;
  return M * ((groups + 255) / 256);
}

// K range staged per phase: a multiple of 256 (T1: of 1280, one 256-byte run of
// a row) with M * stride <= budget and at most 16 activation pieces, i.e. two
// staging batches.
constexpr int phase_k(int M, int K, int fmt, int budget = kXBudget) {
  const int unit = fmt ? 1280 : 256;
  int kx = ((budget / M - 16) / unit) * unit;
  const int cap = 4096 * (16 / M);
  if (kx > cap) kx = (cap / unit) * unit;
  while (kx > unit && stage_pieces(M, kx, fmt) > 2 * kStageBatch) kx -= unit;
  return kx >= K ? K : kx;
}

// LDS: X [M][stride] | zero | part[T][16][16] int | dsc[16] | wred[16] | wss[8] double
int lds_bytes(int tiles, int M, int K, int fmt) {
  return M * stage_stride(phase_k(M, K, fmt), fmt) + zero_bytes(fmt) + tiles * 1024 + 64 + 64 +
         64;
}

// The launch's scalars.  The ones the first loads depend on (activations, the
// first three matrices' packed weights, row counts and first workgroups, and
// M | T << 5 | count << 10 | K << 13) are the kernel's leading scalar arguments,
// which the hardware preloads into SGPRs at wave launch (this file is built with
// a kernarg preload count of 10): no argument load sits in front of the first
// global loads.  The rest comes from GemvArgs in one round of scalar loads,
// issued once the first weight loads are in flight (the empty asm makes them
// materialise together rather than as dependent rounds after the matrix is
// known); their latency hides behind those loads.  Pairs of ints travel as one
// 64-bit value to stay within the asm operand limit.
// Matrices j >= count have wg0[j] = grid size and are never selected.
struct Prologue {
  const float* ws;
  void* y;
  int32_t* acc;
  const float* xs;
  int y_bf16, mdiv, g3;
};
__device__ __forceinline__ uint64_t arg_pair(const int* p) {
  return *reinterpret_cast<const uint64_t*>(p);
}
__device__ __forceinline__ Prologue load_prologue(const GemvArgs& a, int g1, int g2) {
  static_assert(kMaxGroup == 4, "load_prologue lists four matrices");
  static_assert(offsetof(GemvArgs, wg0) % 8 == 0 && offsetof(GemvArgs, y_bf16) % 8 == 0 &&
                    offsetof(GemvArgs, mdiv) % 8 == 0,
                "64-bit aligned int pairs");
  const float *ws0 = a.ws[0], *ws1 = a.ws[1], *ws2 = a.ws[2], *ws3 = a.ws[3];
  void *y0 = a.y[0], *y1 = a.y[1], *y2 = a.y[2], *y3 = a.y[3];
  int32_t *c0 = a.acc[0], *c1 = a.acc[1], *c2 = a.acc[2], *c3 = a.acc[3];
  uint64_t g23 = arg_pair(&a.wg0[2]), bt = arg_pair(&a.y_bf16), md = arg_pair(&a.mdiv);
  const float* xs = a.xs;
  asm volatile(""
               : "+s"(ws0), "+s"(ws1), "+s"(ws2), "+s"(ws3), "+s"(y0), "+s"(y1), "+s"(y2),
                 "+s"(y3), "+s"(c0), "+s"(c1), "+s"(c2), "+s"(c3), "+s"(g23), "+s"(bt),
                 "+s"(md), "+s"(xs));
  const int b = (int)blockIdx.x;
  const int g3 = (int)(g23 >> 32);
  Prologue v{ws0, y0, c0, xs, (int)bt, (int)md, g3};
  if (b >= g1) { v.ws = ws1; v.y = y1; v.acc = c1; }
  if (b >= g2) { v.ws = ws2; v.y = y2; v.acc = c2; }
  if (b >= g3) { v.ws = ws3; v.y = y3; v.acc = c3; }
  return v;
}

// Balanced runs: the epilogue's scalars for the two matrices of a workgroup's
// run, A = jA and B = jA + 1 (B = A when A is the last slot; launch_gemv fills
// the slots past count with matrix 0's pointers, so B's are always readable).
struct RunPrologue {
  const float *wsA, *wsB;
  void *yA, *yB;
  int32_t *accA, *accB;
  const float* xs;
  int y_bf16, mdiv;
};
__device__ __forceinline__ RunPrologue load_run_prologue(const GemvArgs& a, int jA) {
  const int jB = jA + (jA < kMaxGroup - 1 ? 1 : 0);
  const float *wsA = a.ws[jA], *wsB = a.ws[jB];
  void *yA = a.y[jA], *yB = a.y[jB];
  int32_t *accA = a.acc[jA], *accB = a.acc[jB];
  uint64_t bt = arg_pair(&a.y_bf16), md = arg_pair(&a.mdiv);
  const float* xs = a.xs;
  asm volatile("" : "+s"(wsA), "+s"(wsB), "+s"(yA), "+s"(yB), "+s"(accA), "+s"(accB), "+s"(bt),
                    "+s"(md), "+s"(xs));
  return RunPrologue{wsA, wsB, yA, yB, accA, accB, xs, (int)bt, (int)md};
}

// The matrices of a workgroup's run of tiles (it covers at most two): A, the
// matrix of tile t, and B, the next one; first tiles c1 <= c2 <= c3 of matrices
// 1..3.  Chosen in scalar registers in one block (as compare-and-choose code the
// compiler turned the chain into a table in scratch memory, or repeated a
// compare per choice).
struct RunWindow {
  uint64_t wqA, wqB;   // packed weights
  int nA, nB;          // rows
  int cA, cB;          // first tiles (cB = 2^30: no matrix after A)
  int jA;              // slot of A
};
__device__ __forceinline__ RunWindow run_window(int t, int c1, int c2, int c3, uint64_t w0,
                                                uint64_t w1, uint64_t w2, uint64_t w3, int n0,
                                                int n1, int n2, int n3) {
  RunWindow v{w0, w1, n0, n1, 0, c1, 0};
  asm("s_cmp_ge_i32 %7, %8\n\t"
      "s_cselect_b64 %0, %11, %0\n\t"
      "s_cselect_b64 %1, %12, %1\n\t"
      "s_cselect_b32 %2, %14, %2\n\t"
      "s_cselect_b32 %3, %15, %3\n\t"
      "s_cselect_b32 %4, %8, %4\n\t"
      "s_cselect_b32 %5, %9, %5\n\t"
      "s_cselect_b32 %6, 1, %6\n\t"
      "s_cmp_ge_i32 %7, %9\n\t"
      "s_cselect_b64 %0, %12, %0\n\t"
      "s_cselect_b64 %1, %13, %1\n\t"
      "s_cselect_b32 %2, %15, %2\n\t"
      "s_cselect_b32 %3, %16, %3\n\t"
      "s_cselect_b32 %4, %9, %4\n\t"
      "s_cselect_b32 %5, %10, %5\n\t"
      "s_cselect_b32 %6, 2, %6\n\t"
      "s_cmp_ge_i32 %7, %10\n\t"
      "s_cselect_b64 %0, %13, %0\n\t"
      "s_cselect_b32 %2, %16, %2\n\t"
      "s_cselect_b32 %4, %10, %4\n\t"
      "s_cselect_b32 %5, 0x40000000, %5\n\t"
      "s_cselect_b32 %6, 3, %6"
      : "+s"(v.wqA), "+s"(v.wqB), "+s"(v.nA), "+s"(v.nB), "+s"(v.cA), "+s"(v.cB), "+s"(v.jA)
      : "s"(t), "s"(c1), "s"(c2), "s"(c3), "s"(w1), "s"(w2), "s"(w3), "s"(n1), "s"(n2), "s"(n3)
      : "scc");
  return v;
}
// Weights, rows and first tile of the matrix of tile gt: B's if gt >= cB, else A's.
struct TileMatrix {
  uint64_t wq;
  int n, c;
};
__device__ __forceinline__ TileMatrix tile_matrix(int gt, const RunWindow& w) {
  TileMatrix m{w.wqA, w.nA, w.cA};
  asm("s_cmp_ge_i32 %3, %4\n\t"
      "s_cselect_b64 %0, %5, %0\n\t"
      "s_cselect_b32 %1, %6, %1\n\t"
      "s_cselect_b32 %2, %4, %2"
      : "+s"(m.wq), "+s"(m.n), "+s"(m.c)
      : "s"(gt), "s"(w.cB), "s"(w.wqB), "s"(w.nB)
      : "scc");
  return m;
}

// phase_k(M, K, FMT) == min(K, kx_cap<FMT>(M)): the M-dependent cap, from a
// compile-time table (a run-time division by M would cost a long vector sequence
// in front of the first loads).
template <int FMT>
__device__ __forceinline__ int kx_cap(int M) {
  constexpr int kBig = 1 << 30;
  switch (M) {
#define BITNET_KX_CASE(m) case m: return phase_k(m, kBig, FMT);
    BITNET_KX_CASE(1) BITNET_KX_CASE(2) BITNET_KX_CASE(3) BITNET_KX_CASE(4)
    BITNET_KX_CASE(5) BITNET_KX_CASE(6) BITNET_KX_CASE(7) BITNET_KX_CASE(8)
    BITNET_KX_CASE(9) BITNET_KX_CASE(10) BITNET_KX_CASE(11) BITNET_KX_CASE(12)
    BITNET_KX_CASE(13) BITNET_KX_CASE(14) BITNET_KX_CASE(15)
#undef BITNET_KX_CASE
    default: return phase_k(16, kBig, FMT);
  }
}

__device__ __forceinline__ int ceil_log2(int m) { return m > 1 ? 32 - __builtin_clz(m - 1) : 0; }
int ceil_log2_host(int m) { return m > 1 ? 32 - __builtin_clz((unsigned)(m - 1)) : 0; }

typedef unsigned short us2 __attribute__((ext_vector_type(2)));

// One lane's 16 bytes of a T1 block -> the five A operands: operand j holds the
// signed weights 16 j .. 16 j + 15 of the block in order.  Bytes 0, 2 and 1, 3 of
// each dword go to 16-bit lanes; each step t = 3 f - 256 (mod 2^16) leaves the
// digit minus one in the high byte (as a signed byte) and the remaining fraction
// in the low byte; the high bytes of the two lane pairs are gathered in weight
// order.  The four dwords' chains are interleaved so that no step waits on the
// one just issued.
__device__ __forceinline__ void unpack_t1(const uint4 w, v4i out[5]) {
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
  us2 lo[4], hi[4];
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    lo[x] = __builtin_bit_cast(us2, __builtin_amdgcn_perm(0u, wd[x], 0x0c020c00u));  // bytes 0, 2
    hi[x] = __builtin_bit_cast(us2, __builtin_amdgcn_perm(0u, wd[x], 0x0c030c01u));  // bytes 1, 3
  }
  const us2 three = {3, 3}, minus256 = {0xff00, 0xff00};
#pragma unroll
  for (int j = 4; j >= 0; --j) {  // most significant digit first
    uint32_t tl[4], th[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      tl[x] = __builtin_bit_cast(uint32_t, lo[x] * three + minus256);
      th[x] = __builtin_bit_cast(uint32_t, hi[x] * three + minus256);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      out[j][x] = (int)__builtin_amdgcn_perm(th[x], tl[x], 0x07030501u);
      // the next fractions (low bytes) by byte select: a mask would let the
      // compiler take them from a separate lo * 3, one more multiply per step
      lo[x] = __builtin_bit_cast(us2, __builtin_amdgcn_perm(0u, tl[x], 0x0c020c00u));
      hi[x] = __builtin_bit_cast(us2, __builtin_amdgcn_perm(0u, th[x], 0x0c020c00u));
    }
  }
}

// Stage one 16-byte group of int8 activations in the format's order.
template <int FMT>
__device__ __forceinline__ void store_group(uint8_t* dst, uint4 v) {
  if (FMT == kFmtT1)
    *reinterpret_cast<uint4*>(dst) = v;
  else
    store_transposed(dst, v);
}

// What a workgroup needs before its first loads comes as leading scalar
// arguments, which are preloaded into scalar registers at wave launch (the
// library builds this file with kernarg preload): the activations xin, the
// first three matrices' weights and rows, the split of the tiles over the
// workgroups (s1, s2: per-matrix runs, the first workgroups of matrices 1 and 2;
// list runs, L1 | L2 << 8 and h), and mtck = M | T << 5 | count << 10 | K << 13 (T =
// the most row tiles of a workgroup).  The rest stays in the argument block a,
// read after the first loads are issued.  Arguments are laid out in order, each
// at its natural alignment, so the block starts at kArgsAt.
struct LeadArgs {
  const void* xin;
  const uint8_t *wp0, *wp1, *wp2;
  int n0, n1, n2, s1, s2;
  uint32_t mtck;
};
constexpr int kArgsAt =
    (sizeof(LeadArgs) + alignof(GemvArgs) - 1) / alignof(GemvArgs) * alignof(GemvArgs);

// XMODE 0: int8 x_q.  XMODE 1 + f, f = bf16 (1) | gated by a.xup (2) | RMS norm
// with a.gnorm (4): fp32 / bf16 input quantised in the kernel.  The prologue
// options are compile-time so that no load sits behind a runtime branch.  H:
// groups of 16 inputs per thread held in registers by the fused modes (without a
// prologue, kHoldPlain for inputs longer than kHold groups per thread, so that
// they are read once; else kHold).
// BAL false: per-matrix runs, each workgroup's tiles belong to one matrix (T
// tiles, the last run of a matrix shorter).  BAL true: list runs, the tiles of
// all the launch's matrices form one list, matrix after matrix, and workgroup b
// takes L1 consecutive tiles if b < h, else L2 (a run may cross into the next
// matrix); launch_gemv picks the lengths (this code's extra scalar work measured
// 0.1-0.2 us per launch, so it is not the default).
// With a prologue (PRO) the weights are loaded non-temporal: they are read once,
// and the loads then leave the prologue's inputs (the up projection, the norm
// weight) in L2 for the other workgroups (2B stack with the fused norms and
// gating 0.821 -> 0.778 ms per token; without a prologue the same loads lost 2%
// on the 100B-class stack and nothing was gained on the 2B one).
// PRIO: launches of two workgroups per compute unit (on some or all units) with
// equal tile counts on a chip of kPrioSplit compute units: the second-dispatched
// workgroup of a unit (b >= kPrioSplit) stages its input at wave priority 1.
// Issue arbitration otherwise favours the older waves, so that workgroup waited
// behind the first one's staging and ran 1.6-1.9x longer; raising it for the
// whole launch measured slower, for the staging alone faster (100B-class stack, o and down
// projections of one tile per workgroup: 5.646 -> 5.579 ms per token; q+k+v and
// gate+up in equal list runs instead of skewed ones: 5.64 -> 5.60).
template <int XMODE, int R, int FMT, int H = kHold, bool BAL = false, int NW = 4,
          bool PRIO = false>
__global__ __launch_bounds__(64 * NW) void gemv_kernel(const void* xin, const uint8_t* wp0,
                                                        const uint8_t* wp1, const uint8_t* wp2,
                                                        int n0, int n1, int n2, int s1, int s2,
                                                        uint32_t mtck, const GemvArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int F = XMODE > 0 ? XMODE - 1 : 0;
  constexpr bool BF = (F & 1) != 0;
  constexpr bool GLU = XMODE > 0 && (F & 2) != 0;
  constexpr bool NRM = XMODE > 0 && (F & 4) != 0;
  constexpr bool PRO = GLU || NRM;
  constexpr int NV = BF ? 2 : 4;             // fused: 16-byte words per 16-element group
  constexpr int HOLD = PRO ? kHold : H;       // fused: groups held per thread
  constexpr uint32_t ES = BF ? 2u : 4u;      // fused: input element size
  constexpr int ZB = FMT == kFmtT1 ? 96 : 64;  // zero slot bytes (zero_bytes)
  constexpr int kT = 64 * NW;                // threads
  static_assert(NW == 4 || (NW == 8 && XMODE > 0), "eight waves: fused activations only");
  static_assert(!PRIO || NW == 4, "staging priority: four-wave workgroups");
  if constexpr (PRIO) {
    if (blockIdx.x >= kPrioSplit) __builtin_amdgcn_s_setprio(1);
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform by construction
  const int r = lane & 15;  // A operand: row of the tile; B operand: token
  const int g = lane >> 4;  // 16-k block of the operand within a 64-k chunk
  const int M = (int)(mtck & 31u), T = (int)((mtck >> 5) & 31u), K = (int)(mtck >> 13);
  const int b = (int)blockIdx.x;
  // per-matrix runs: this workgroup's matrix and its first tile in it
  const uint8_t* wmat = wp0;
  int nrows = n0, tl0 = 0;
  // balanced runs: the run's first tile in the list and its two-matrix window
  int t_start = 0;
  RunWindow win{};
  int ntiles;
  if constexpr (!BAL) {
    // only a fourth matrix waits for the argument block
    const int g1 = s1, g2 = s2;
    int wgm = 0;
    if (b >= g1) { wmat = wp1; nrows = n1; wgm = g1; }
    if (b >= g2) { wmat = wp2; nrows = n2; wgm = g2; }
    if (((mtck >> 10) & 7u) == 4u) {
      // (loaded and waited for in one asm block: loads the compiler sees, it
      // hoists to the entry, and every launch would then wait for them before its
      // first weight loads; early-clobber outputs, since the block issues several
      // loads from the one segment pointer)
      int g3, n3;
      uint64_t w3;
      asm volatile(
          "s_load_dword %0, %3, %4\n\t"
          "s_load_dword %1, %3, %5\n\t"
          "s_load_dwordx2 %2, %3, %6\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&s"(g3), "=&s"(n3), "=&s"(w3)
          : "s"(__builtin_amdgcn_kernarg_segment_ptr()),
            "i"(kArgsAt + offsetof(GemvArgs, wg0) + 12),
            "i"(kArgsAt + offsetof(GemvArgs, n) + 12), "i"(kArgsAt + offsetof(GemvArgs, wp) + 24));
      if (b >= g3) {
        wmat = reinterpret_cast<const uint8_t*>(w3);
        nrows = n3;
        wgm = g3;
      }
    }
    tl0 = (b - wgm) * T;
    ntiles = min(T, (nrows + 15) / 16 - tl0);
  } else {
    const int L1 = s1 & 255, L2 = s1 >> 8, h = s2;
    t_start = b < h ? b * L1 : h * L1 + (b - h) * L2;
    ntiles = b < h ? L1 : L2;
    // first tile of matrices 1, 2, 3 (matrices past count have no rows)
    const int c1 = (n0 + 15) >> 4, c2 = c1 + ((n1 + 15) >> 4), c3 = c2 + ((n2 + 15) >> 4);
    const uint8_t* wp3 = wp0;
    int n3 = 0;
    if (t_start + ntiles > c3) {   // only with a fourth matrix (c3 is else the tile count)
      uint64_t w3;
      asm volatile(
          "s_load_dword %0, %2, %3\n\t"
          "s_load_dwordx2 %1, %2, %4\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&s"(n3), "=&s"(w3)
          : "s"(__builtin_amdgcn_kernarg_segment_ptr()),
            "i"(kArgsAt + offsetof(GemvArgs, n) + 12), "i"(kArgsAt + offsetof(GemvArgs, wp) + 24));
      wp3 = reinterpret_cast<const uint8_t*>(w3);
    }
    // the run covers at most two matrices (launch_gemv makes every matrix at
    // least a run long)
    win = run_window(t_start, c1, c2, c3, (uint64_t)wp0, (uint64_t)wp1, (uint64_t)wp2,
                     (uint64_t)wp3, n0, n1, n2, n3);
  }
  const uint32_t rowb = FMT == kFmtT1 ? 16u * (((uint32_t)K + 79u) / 80u)
                                      : (uint32_t)K >> 2;  // packed bytes per row
  // the fused modes stage all of K in one phase (launch_gemv checks it)
  const int kx = XMODE > 0 ? K : min(K, kx_cap<FMT>(M));
  const int phases = XMODE > 0 ? 1 : (K + kx - 1) / kx;
  const int stride = FMT == kFmtT1 ? 80 * ((kx + 79) / 80) + 16 : kx + 16;  // stage_stride

  uint8_t* xs = smem;                                    // [M][stride]
  uint8_t* zero = smem + M * stride;                     // ZB zero bytes
  int* part = reinterpret_cast<int*>(zero + ZB);         // [T][16 rows][16 tokens]
  float* dsc = reinterpret_cast<float*>(part + T * 256);  // [16]
  float* wred = dsc + 16;                                // [16]
  double* wss = reinterpret_cast<double*>(wred + 16);    // [NW]

  // Buffer descriptor of local tile tl (wave-uniform; readfirstlane keeps it in
  // scalar registers so the loads need no per-lane legalisation loop).
  auto tile_rsrc = [&](int tl) {
    int rows;
    uint64_t base;
    if constexpr (BAL) {
      const int gt = __builtin_amdgcn_readfirstlane(t_start + tl);
      const TileMatrix m = tile_matrix(gt, win);
      const int row0 = (gt - m.c) * 16;
      rows = max(0, min(16, m.n - row0));
      base = m.wq + (uint64_t)row0 * rowb;
    } else {
      const int row0 = (tl0 + tl) * 16;
      rows = max(0, min(16, nrows - row0));
      base = (uint64_t)(wmat + (size_t)row0 * rowb);
    }
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    const uint32_t bytes = __builtin_amdgcn_readfirstlane((uint32_t)rows * rowb);
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), bytes);
  };

  // clear the partial tiles and the zero slot
  for (int i = tid; i < T * 64; i += kT) reinterpret_cast<uint4*>(part)[i] = make_uint4(0, 0, 0, 0);
  if (tid < ZB / 4) reinterpret_cast<uint32_t*>(zero)[tid] = 0u;
  // the rest of the arguments and the epilogue's scalars, fetched once the first
  // activation and weight loads are in flight (phase 0 below)
  Prologue pro{};       // per-matrix runs
  RunPrologue rpro{};   // balanced runs
  float xs_t = 0.0f, gamma = 0.0f;
  float gamB = 0.0f;    // balanced runs: gamma* of matrix B (gamma: of A)

  // token groups: G consecutive threads per token (G = 64 NW / 2^ceil(log2 M));
  // threads of tokens >= M idle in the per-token passes
  const int lgG = (NW == 8 ? 9 : 8) - ceil_log2(M);
  const int G = 1 << lgG;
  const int tk = tid >> lgG;
  const int jg = tid & (G - 1);

  // Producer of the weight ring: phase pp, tile tp, step jp of this wave's
  // super-chunks (past the last tile or chunk the offset is out of range and the
  // load reads zeros; a wave without super-chunks never advances past its first
  // tile).  With several phases it runs on into the next one: a phase's last
  // round of refills issues the next phase's first R loads, whose latency then
  // overlaps the barrier and the staging of the next activations.
  int pp = -1, tp = 0, jp = 0, Cp = 0, Jp = 0;
  uint32_t kb0p = 0;
  auto rs = tile_rsrc(0);
  auto producer_phase = [&](int ph) {
    const int k0p = ph * kx, klenp = min(kx, K - k0p);
    Cp = FMT == kFmtT1 ? (klenp + 79) / 80 : klenp >> 6;
    const int Sp = (Cp + 3) >> 2;
    Jp = Sp > wave ? (Sp - wave + NW - 1) / NW : 0;
    kb0p = FMT == kFmtT1 ? (uint32_t)k0p / 5u : (uint32_t)k0p >> 2;
    pp = ph;
    tp = 0;
    jp = 0;
    rs = tile_rsrc(0);
  };
  auto next_load = [&]() -> uint4 {
    const int c = 4 * (wave + NW * jp) + g;
    const uint32_t off = (tp < ntiles && c < Cp) ? (uint32_t)r * rowb + kb0p + 16u * (uint32_t)c
                                                 : kOob;
    const uint4 v = PRO ? bload16_nt(rs, off) : bload16(rs, off);
    if (++jp == Jp) {
      jp = 0;
      ++tp;
      rs = tile_rsrc(tp);
    }
    return v;
  };
  uint4 ring[R];
  bool carried = false;  // the ring already holds this phase's first loads

  for (int p = 0; p < phases; ++p) {
    const int k0 = p * kx;
    const int klen = min(kx, K - k0);
    // chunks (16 packed bytes of a row: 64 k, T1 80 k) in this phase
    const int C = FMT == kFmtT1 ? (klen + 79) / 80 : klen >> 6;
    const int S = (C + 3) >> 2;                    // 256-k super-chunks
    const int J = S > wave ? (S - wave + NW - 1) / NW : 0;
    const int Q = ntiles * J;                      // loads per lane in this phase
    const int K16 = klen >> 4;                     // 16-k groups of activations
    const int K16s = FMT == kFmtT1 ? 5 * C : K16;  // groups staged (T1: zeros past klen)

    // 1. first activation loads of this phase, then the first weight loads.
    // int8 activations come in pieces (token t, 4096-k block j): lane tid loads
    // 16-byte group c = 256 j + tid of the piece (zeros past the phase); the piece
    // counters are uniform, so no per-lane division is needed
    const int J16 = (K16s + 255) >> 8;             // blocks per token
    uint4 xv[kStageBatch];
    const auto xr = make_rsrc(xin, (uint32_t)M * (uint32_t)K);
    int lt = 0, lj = 0;                            // next piece to load
    auto xload = [&]() -> uint4 {
      const int c = 256 * lj + tid;
      const uint4 v = bload16(xr, (lt < M && c < K16) ? (uint32_t)lt * (uint32_t)K +
                                                            (uint32_t)k0 + 16u * (uint32_t)c
                                                      : kOob);
      if (++lj == J16) {
        lj = 0;
        ++lt;
      }
      return v;
    };
    // fused: group c of this thread's token (zeros past the end or for idle threads)
    const auto fr = make_rsrc(xin, (uint32_t)M * (uint32_t)K * ES);
    auto foff = [&](int c, int h) -> uint32_t {
      return (tk < M && c < K16) ? ((uint32_t)tk * (uint32_t)K + 16u * (uint32_t)c) * ES + 16u * h
                                 : kOob;
    };
    // prologue operands: the up projection (same layout as the input) and the
    // norm weight (fp32 [K], 64 bytes per group)
    constexpr bool glu = GLU, nrm = NRM;
    const auto ur = make_rsrc(glu ? a.xup : xin, (uint32_t)M * (uint32_t)K * ES);
    const auto gr = make_rsrc(nrm ? (const void*)a.gnorm : xin, nrm ? 4u * (uint32_t)K : 0u);
    auto goff = [&](int c, int h) -> uint32_t {
      return (tk < M && c < K16) ? 64u * (uint32_t)c + 16u * (uint32_t)h : kOob;
    };
    uint4 hold[HOLD][NV], holdu[HOLD][NV], holdg[HOLD][4];
    if constexpr (XMODE == 0) {
#pragma unroll
      for (int b = 0; b < kStageBatch; ++b) xv[b] = xload();
    } else {
#pragma unroll
      for (int b = 0; b < HOLD; ++b) {
#pragma unroll
        for (int h = 0; h < NV; ++h) hold[b][h] = bload16(fr, foff(jg + G * b, h));
        if (PRO) {
#pragma unroll
          for (int h = 0; h < NV; ++h) holdu[b][h] = glu ? bload16(ur, foff(jg + G * b, h)) : hold[b][h];
#pragma unroll
          for (int h = 0; h < 4; ++h) holdg[b][h] = nrm ? bload16(gr, goff(jg + G * b, h)) : make_uint4(0, 0, 0, 0);
        }
      }
    }
    if (!carried) {
      if (pp != p) producer_phase(p);
#pragma unroll
      for (int u = 0; u < R; ++u) {
        ring[u] = next_load();
        asm volatile("" ::: "memory");  // keep the ring's loads in slot order
      }
    }
    carried = false;
    if (p == 0) {
      // (buffer loads: the pointers come out of the asm in load_prologue as generic
      // pointers, and generic loads would make the compiler's waits conservative)
      const float* xsp;
      if constexpr (BAL) {
        rpro = load_run_prologue(a, win.jA);
        xsp = rpro.xs;
        gamma = __uint_as_float(bload4(make_rsrc(rpro.wsA, 4u), 0u));
        gamB = __uint_as_float(bload4(make_rsrc(rpro.wsB, 4u), 0u));
      } else {
        pro = load_prologue(a, s1, s2);
        xsp = pro.xs;
        gamma = __uint_as_float(bload4(make_rsrc(pro.ws, 4u), 0u));
      }
      if (XMODE == 0)
        xs_t = __uint_as_float(bload4(make_rsrc(xsp, 4u * (uint32_t)M),
                                      4u * (uint32_t)min(tid, M - 1)));
    }

    // 2. stage the activations, transposed within each 16-byte group
    if constexpr (XMODE == 0) {
      // at most two batches (phase_k keeps the pieces <= 2 * kStageBatch);
      // written out rather than as a loop so that the wait for the ring's loads
      // at the top of the stream loop stays a partial one.  Every lane stores
      // (groups past the end read as zeros and go to the zero slot): a store under
      // a lane mask would leave its load's wait inside a skippable block, and the
      // compiler then drains all loads in flight later.
      static_assert(2 * kStageBatch == 16, "phase_k allows 16 pieces");
      int st = 0, sj = 0;                          // next piece to store
      auto store_batch = [&]() {
#pragma unroll
        for (int b = 0; b < kStageBatch; ++b) {
          const int c = 256 * sj + tid;
          store_group<FMT>((st < M && c < K16s) ? xs + st * stride + 16 * c : zero, xv[b]);
          if (++sj == J16) {
            sj = 0;
            ++st;
          }
        }
      };
      store_batch();
      if (M * J16 > kStageBatch) {
#pragma unroll
        for (int b = 0; b < kStageBatch; ++b) xv[b] = xload();
        store_batch();
      }
    } else {
      // v: the values of one group before the norm (the raw input, or the gated
      // one with the up projection)
      auto values = [&](const uint4* xw, const uint4* uw, float q[16]) {
        raw_to_f32<BF>(xw, q);
        if (PRO && glu) {
          float u[16];
          raw_to_f32<BF>(uw, u);
#pragma unroll
          for (int j = 0; j < 16; ++j) q[j] = glu_value(q[j], u[j]);
        }
      };
      // u = RN32(RN32(v r) w) with the norm weight w of the group
      auto normalise = [&](const uint4* gw, float r, float q[16]) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint4 g4 = gw[j >> 2];
          const uint32_t gb = (j & 3) == 0 ? g4.x : (j & 3) == 1 ? g4.y : (j & 3) == 2 ? g4.z : g4.w;
          q[j] = norm_value(q[j], r, __uint_as_float(gb));
        }
      };
      // group c read again: v, or with the norm (norm set) the normalised u
      auto reload = [&](int c, float q[16], bool norm, float r) {
        uint4 xw[NV], uw[NV];
#pragma unroll
        for (int h = 0; h < NV; ++h) xw[h] = bload16(fr, foff(c, h));
        if (PRO && glu) {
#pragma unroll
          for (int h = 0; h < NV; ++h) uw[h] = bload16(ur, foff(c, h));
        }
        values(xw, uw, q);
        if (nrm && norm) {
          uint4 gw[4];
#pragma unroll
          for (int h = 0; h < 4; ++h) gw[h] = bload16(gr, goff(c, h));
          normalise(gw, r, q);
        }
      };
      // the held groups keep their values for the quantise pass; G >= 64 (one
      // token per wave or more)
      const int nb = (K16s + G - 1) >> lgG;      // groups per thread, uniform
      const int nw = G >> 6;                     // waves per token
      float qh[HOLD][16];
      float r = 1.0f;
#pragma unroll
      for (int b = 0; b < HOLD; ++b) values(hold[b], holdu[b], qh[b]);
      if constexpr (nrm) {
        // pass 1: the sum of the squares in float64 over the token's threads
        double ss = 0.0;
#pragma unroll
        for (int b = 0; b < HOLD; ++b)
#pragma unroll
          for (int j = 0; j < 16; ++j) ss += (double)qh[b][j] * (double)qh[b][j];
        for (int b = HOLD; b < nb; ++b) {
          float v[16];
          reload(jg + G * b, v, false, 1.0f);
#pragma unroll
          for (int j = 0; j < 16; ++j) ss += (double)v[j] * (double)v[j];
        }
        ss = wave_sum_f64(ss);
        if (lane == 0) wss[wave] = ss;
        lds_barrier();
        // every thread rounds the mean of every token, so the choice of the
        // exact path is uniform over the workgroup
        float ms = 0.0f;
        bool fast = true;
        for (int t = 0; t < M; ++t) {
          double st = 0.0;
          for (int i = 0; i < nw; ++i) st += wss[(t * nw + i) & (NW - 1)];
          float mt;
          fast = mean_sq_fast(st, K, mt) && fast;
          if (t == tk) ms = mt;
        }
        if (!fast) {
          // a mean near a rounding boundary: the exact sums of the squares of all
          // tokens in carry-save limbs, in the partial tiles' LDS (cleared again
          // afterwards; the stream below starts after two more barriers)
          static_assert(4 * kSqLimbs * 8 + kSqWork * 4 <= 1024, "limbs fit one partial tile");
          unsigned long long* limbs = reinterpret_cast<unsigned long long*>(part);  // [4][kSqLimbs]
          uint32_t* sqwork = reinterpret_cast<uint32_t*>(limbs + 4 * kSqLimbs);
          if (tid < 4 * kSqLimbs) limbs[tid] = 0ull;
          lds_barrier();
          if (tk < M) {
#pragma unroll
            for (int b = 0; b < HOLD; ++b)
#pragma unroll
              for (int j = 0; j < 16; ++j) sq_limbs_add(limbs + tk * kSqLimbs, qh[b][j]);
            for (int b = HOLD; b < nb; ++b) {
              float v[16];
              reload(jg + G * b, v, false, 1.0f);
#pragma unroll
              for (int j = 0; j < 16; ++j) sq_limbs_add(limbs + tk * kSqLimbs, v[j]);
            }
          }
          lds_barrier();
          if (tid == 0)
            for (int t = 0; t < M; ++t) dsc[t] = sq_limbs_mean(limbs + t * kSqLimbs, K, sqwork);
          lds_barrier();
          if (tk < M) ms = dsc[tk];
          for (int i = tid; i < T * 64; i += kT)
            reinterpret_cast<uint4*>(part)[i] = make_uint4(0, 0, 0, 0);
        }
        r = rms_factor_of_mean(ms, a.eps);
#pragma unroll
        for (int b = 0; b < HOLD; ++b) normalise(holdg[b], r, qh[b]);
      }
      // absmax of the token (pass 2 with the norm)
      float amax = 0.0f;
#pragma unroll
      for (int b = 0; b < HOLD; ++b)
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(qh[b][j]));
      for (int b = HOLD; b < nb; ++b) {
        float v[16];
        reload(jg + G * b, v, true, r);
#pragma unroll
        for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
      }
      amax = wave_max(amax);
      if (lane == 0) wred[wave] = amax;
      lds_barrier();
      float tmax = 0.0f;
      for (int i = 0; i < nw; ++i) tmax = fmaxf(tmax, wred[(tk * nw + i) & (NW - 1)]);
      const float astar = fmaxf(tmax, kEps);
      const float s_t = kQb / astar;
      if (jg == 0 && tk < M) {
        const float d = astar / kQb;
        dsc[tk] = d;
        if (blockIdx.x == 0) a.xs_out[tk] = d;
      }
      // quantise; every lane stores (idle lanes and groups past the end hold
      // zeros, which quantise to zeros and go to the zero slot).  The codes are
      // the low bytes of rne_bits (quant4's rounding), gathered by the byte
      // permutes straight into the staged order (the separate transpose and
      // quant4's clamp and conversion took ~6 instructions per value, this 2.75:
      // 100B-class stack 5.82 -> 5.67 ms per token, 2B stack 0.645 -> 0.619)
      auto put = [&](int c, const float* v) {
        uint32_t m[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) m[j] = rne_bits(v[j], s_t);
        if (tk < M && c < K16 && blockIdx.x == 0)
          reinterpret_cast<uint4*>(a.xq_out + (size_t)tk * K)[c] =
              make_uint4(low_bytes(m[0], m[1], m[2], m[3]), low_bytes(m[4], m[5], m[6], m[7]),
                         low_bytes(m[8], m[9], m[10], m[11]),
                         low_bytes(m[12], m[13], m[14], m[15]));
        uint4 q;
        if constexpr (FMT == kFmtT1)   // natural order
          q = make_uint4(low_bytes(m[0], m[1], m[2], m[3]), low_bytes(m[4], m[5], m[6], m[7]),
                         low_bytes(m[8], m[9], m[10], m[11]),
                         low_bytes(m[12], m[13], m[14], m[15]));
        else                           // transposed within the group (store_transposed)
          q = make_uint4(low_bytes(m[0], m[4], m[8], m[12]), low_bytes(m[1], m[5], m[9], m[13]),
                         low_bytes(m[2], m[6], m[10], m[14]),
                         low_bytes(m[3], m[7], m[11], m[15]));
        *reinterpret_cast<uint4*>(tk < M && c < K16s ? xs + tk * stride + 16 * c : zero) = q;
      };
#pragma unroll
      for (int b = 0; b < HOLD; ++b) put(jg + G * b, qh[b]);
      for (int b = HOLD; b < nb; ++b) {
        float v[16];
        reload(jg + G * b, v, true, r);
        put(jg + G * b, v);
      }
    }
    lds_barrier();

    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);   // staged: back to age order
    // 3. stream: consumer position (tc, jc); flush a tile's partial when it ends
    const int bt = r < M ? r * stride : -1;
    int tc = 0, jc = 0;
    v4i acc = {0, 0, 0, 0};
    for (int q0 = 0; q0 < Q; q0 += R) {
      if (XMODE == 0 && q0 + R >= Q && p + 1 < phases) {
        // last round: its refills are the next phase's first loads
        producer_phase(p + 1);
        carried = true;
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int c = 4 * (wave + NW * jc) + g;
        if constexpr (FMT == kFmtT1) {
          v4i t[5];
          unpack_t1(ring[u], t);
          v4i a0 = t[0], a1 = t[1], a2 = t[2], a3 = t[3], a4 = t[4];
          asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(a4)::"memory");
          ring[u] = next_load();
          // (a 24-bit product: a 32-bit one is made a 64-bit multiply-add whose
          // unused high addend can be a register with a load in flight, which the
          // compiler then waits for)
          const int bb = (bt >= 0 && c < C) ? bt + (int)__umul24(80u, (uint32_t)c) : M * stride;
          const v4i* bp = reinterpret_cast<const v4i*>(xs + bb);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bp[0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bp[1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, bp[2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, bp[3], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a4, bp[4], acc, 0, 0, 0);
        } else {
          // unpack the whole chunk before refilling its slot, so the refill can land
          // in the same registers (no loop-carried copy that would wait for the load)
          v4i a0 = unpack_weights_transposed(ring[u].x);
          v4i a1 = unpack_weights_transposed(ring[u].y);
          v4i a2 = unpack_weights_transposed(ring[u].z);
          v4i a3 = unpack_weights_transposed(ring[u].w);
          // the empty asm takes the unpacked operands and orders memory reads after
          // itself, so the scheduler cannot hoist the refill above the unpack
          asm volatile("" : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3)::"memory");
          ring[u] = next_load();
          const int bb = (bt >= 0 && c < C) ? bt + 64 * c : M * stride;
          const v4i* bp = reinterpret_cast<const v4i*>(xs + bb);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, bp[0], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, bp[1], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, bp[2], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, bp[3], acc, 0, 0, 0);
        }
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
    if (p + 1 < phases) lds_barrier();  // the next phase overwrites the staged activations
  }
  // token scales of the int8 input (loaded after the ring, so written only now,
  // when the stream has waited for every load)
  if (XMODE == 0 && tid < M) dsc[tid] = xs_t;
  lds_barrier();

  // 4. rescale, store: index = ((tile * M) + token) * 16 + row
  if constexpr (!BAL) {
    int32_t* accp = pro.acc;
    void* yp = pro.y;
    for (int i = tid; i < ntiles * M * 16; i += kT) {
      const int row = i & 15;
      const int tt = i >> 4;
      const int tl = (int)(((uint32_t)tt * (uint32_t)pro.mdiv) >> 16);  // tt / M
      const int t = tt - tl * M;
      const int n = (tl0 + tl) * 16 + row;
      if (n < nrows) {
        const int accv = part[tl * 256 + row * 16 + t];
        const float yv = (float)accv * (gamma * dsc[t]);
        const size_t o = (size_t)t * nrows + n;
        if (accp) as_global(accp)[o] = accv;
        if (pro.y_bf16)
          as_global(reinterpret_cast<uint16_t*>(yp))[o] = float_to_bf16_rne(yv);
        else
          as_global(reinterpret_cast<float*>(yp))[o] = yv;
      }
    }
  } else {
    // matrix A's part of the run, then B's (tile tl of the run = list tile
    // t_start + tl; within its matrix, tile t_start + tl - c)
    const int t_end = t_start + ntiles;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int c = h2 == 0 ? win.cA : win.cB;
      const int lo = h2 == 0 ? t_start : max(t_start, win.cB);
      const int hi = h2 == 0 ? min(t_end, win.cB) : t_end;
      if (lo >= hi) continue;
      const int nr = h2 == 0 ? win.nA : win.nB;
      void* yp = h2 == 0 ? rpro.yA : rpro.yB;
      int32_t* accp = h2 == 0 ? rpro.accA : rpro.accB;
      const float gm = h2 == 0 ? gamma : gamB;
      for (int i = tid; i < (hi - lo) * M * 16; i += kT) {
        const int row = i & 15;
        const int tt = i >> 4;
        const int tq = (int)(((uint32_t)tt * (uint32_t)rpro.mdiv) >> 16);  // tt / M
        const int t = tt - tq * M;
        const int tl = lo - t_start + tq;
        const int n = (lo - c + tq) * 16 + row;
        if (n < nr) {
          const int accv = part[tl * 256 + row * 16 + t];
          const float yv = (float)accv * (gm * dsc[t]);
          const size_t o = (size_t)t * nr + n;
          if (accp) as_global(accp)[o] = accv;
          if (rpro.y_bf16)
            as_global(reinterpret_cast<uint16_t*>(yp))[o] = float_to_bf16_rne(yv);
          else
            as_global(reinterpret_cast<float*>(yp))[o] = yv;
        }
      }
    }
  }
}

// Kernel for activation mode XMODE, weight format FMT and ring depth 2, 4, 8 or
// 16 (smallest >= R).
// (balanced runs come only with more than 256 workgroups, where the ring is at
// most 4 deep: built for depths 2 and 4)
template <int XMODE, int FMT, int H>
const void* ring_kernel(int R, bool bal, bool wide, bool prio) {
  if constexpr ((XMODE == 1 || XMODE == 2) && FMT == kFmt2) {
    // eight-wave workgroups of one tile (per-matrix runs, ring depth 2 or 4)
    if (wide && !bal)
      return R <= 2 ? reinterpret_cast<const void*>(gemv_kernel<XMODE, 2, FMT, H, false, 8>)
                    : reinterpret_cast<const void*>(gemv_kernel<XMODE, 4, FMT, H, false, 8>);
  }
  if constexpr ((XMODE == 1 || XMODE == 2) && FMT == kFmt2) {
    // staging priority for the second workgroup of each compute unit (ring depth 4)
    if (prio && R > 2 && R <= 4)
      return bal ? reinterpret_cast<const void*>(gemv_kernel<XMODE, 4, FMT, H, true, 4, true>)
                 : reinterpret_cast<const void*>(gemv_kernel<XMODE, 4, FMT, H, false, 4, true>);
  }
  if (bal)
    return R <= 2 ? reinterpret_cast<const void*>(gemv_kernel<XMODE, 2, FMT, H, true>)
                  : reinterpret_cast<const void*>(gemv_kernel<XMODE, 4, FMT, H, true>);
  if (R <= 2) return reinterpret_cast<const void*>(gemv_kernel<XMODE, 2, FMT, H>);
  if (R <= 4) return reinterpret_cast<const void*>(gemv_kernel<XMODE, 4, FMT, H>);
  if (R <= 8) return reinterpret_cast<const void*>(gemv_kernel<XMODE, 8, FMT, H>);
  return reinterpret_cast<const void*>(gemv_kernel<XMODE, 16, FMT, H>);
}

template <int FMT>
const void* select_kernel(int xmode, int R, bool long_input, bool bal, bool wide, bool prio) {
  switch (xmode) {
    case 0: return ring_kernel<0, FMT, kHold>(R, bal, wide, prio);
    case 1:
      return long_input ? ring_kernel<1, FMT, kHoldPlain>(R, bal, wide, prio)
                        : ring_kernel<1, FMT, kHold>(R, bal, wide, prio);
    case 2:
      return long_input ? ring_kernel<2, FMT, kHoldPlain>(R, bal, wide, prio)
                        : ring_kernel<2, FMT, kHold>(R, bal, wide, prio);
    case 3: return ring_kernel<3, FMT, kHold>(R, bal, wide, prio);
    case 4: return ring_kernel<4, FMT, kHold>(R, bal, wide, prio);
    case 5: return ring_kernel<5, FMT, kHold>(R, bal, wide, prio);
    case 6: return ring_kernel<6, FMT, kHold>(R, bal, wide, prio);
    case 7: return ring_kernel<7, FMT, kHold>(R, bal, wide, prio);
    default: return ring_kernel<8, FMT, kHold>(R, bal, wide, prio);
  }
}


}  // namespace

// Compute units of the current device (1 if the runtime cannot say).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();
    cus = 1;
  }
  return cus;
}

bool gemv_fits(int64_t M, int64_t K, int fmt) {
  return M >= 1 && M <= kMaxM && K <= kGemvMaxK &&
         (fmt == kFmtT1 ? K >= 16 && (K % 16) == 0 : K >= 64 && (K % 64) == 0);
}

bool gemv_fused_fits(int64_t M, int64_t K, int fmt) {
  return gemv_fits(M, K, fmt) && M <= kMaxFusedM &&
         phase_k((int)M, (int)K, fmt, kFusedXBudget) == K;
}

hipError_t launch_gemv(GemvArgs a, int xf_dtype, int fmt, hipStream_t s) {
  const bool fused = a.xf != nullptr;
  if (a.count < 1 || a.count > kMaxGroup || (fmt != kFmt2 && fmt != kFmtT1) ||
      !gemv_fits(a.M, a.K, fmt) || (fused && !gemv_fused_fits(a.M, a.K, fmt)))
    return hipErrorInvalidValue;
  if ((a.xup != nullptr || a.gnorm != nullptr) && !fused) return hipErrorInvalidValue;
  const int xmode = !fused ? 0
                           : 1 + (xf_dtype == 1 ? 1 : 0) + (a.xup ? 2 : 0) + (a.gnorm ? 4 : 0);
  int tiles[kMaxGroup] = {0, 0, 0, 0};
  int total_tiles = 0;
  for (int j = 0; j < a.count; ++j) total_tiles += tiles[j] = (a.n[j] + 15) / 16;
  if (total_tiles == 0) return hipSuccess;
  // loads per lane of one tile in the first phase (the busiest wave)
  const int kx = phase_k(a.M, a.K, fmt);
  const int chunks = fmt == kFmtT1 ? (kx + 79) / 80 : kx / 64;
  const int per_tile = ((chunks + 3) / 4 + 3) / 4;
  const int64_t row_bytes = fmt == kFmtT1 ? 16 * ((a.K + 79) / 80) : a.K / 4;
  // Two regimes (measured on the decode shapes): a launch of at most
  // kLatencyBytes of packed weights gives every tile its own workgroup, so all
  // loads issue at once; a larger one is spread as kWgsPerCu workgroups per
  // compute unit with equal tile counts.  The ring depth targets kFlightLoads
  // 1 KiB loads in flight over the whole chip (in effect: R = 4 from 129
  // workgroups up): deeper rings measured slower (more requests queue without
  // more throughput).
  const int cus = device_cus();
  auto count_wgs = [&](int t) {
    int w = 0;
    for (int j = 0; j < a.count; ++j) w += (tiles[j] + t - 1) / t;
    return w;
  };
  // fused input groups of 16 per thread: held in registers when they are more
  // than kHold + 1 (and at most kHoldPlain); with kHold + 1, two are held and
  // the third read twice, cheaper than issuing kHoldPlain hold loads (T1 input
  // of 8192: 515 groups; 100B-class T1 stack 8.28 -> 7.87 ms per token)
  const int staged = fmt == kFmtT1 ? 5 * ((a.K + 79) / 80) : a.K / 16;
  auto long_input = [&](int threads) {
    const int g = threads >> ceil_log2_host(a.M);   // threads per token
    return fused && (staged + g - 1) / g > kHold + 1;
  };
  struct Plan {
    int tpw, wgs;
    bool bal;
    const void* kernel;
    size_t lds;
    int l1, l2, h;   // list runs: L1 tiles for workgroups b < h, else L2
    bool wide;       // eight-wave workgroups
    bool prio;       // staging priority for the second workgroup of each CU
  };
  // latency regime: at most kLatencyBytes of packed weights
  const bool latency = (int64_t)total_tiles * 16 * row_bytes <= kLatencyBytes;
  auto plan = [&](int t, bool bal, int wgs = 0, bool wide = false, bool prio = false) {
    Plan p{t, wgs ? wgs : bal ? (total_tiles + t - 1) / t : count_wgs(t), bal, nullptr, 0, 0, 0, 0,
           wide, prio};
    const int nw = wide ? 8 : 4;
    const int per_tile_w = ((chunks + 3) / 4 + nw - 1) / nw;   // loads per lane of a tile
    int ring = 4;
    while (!wide && ring < 16 && 2 * ring * nw * p.wgs <= kFlightLoads) ring *= 2;
    // several tiles per workgroup but short rows (at most 6 loads per wave in
    // all, over more than 256 workgroups): two loads ahead measured faster than
    // four (2B gate+up, 2560 -> 13824: the chain 5.49 -> 5.34 us per launch);
    // longer streams lose with it (100B-class stack 16.3 -> 18.0 us)
    if (p.wgs > 256 && t >= 2 && t * per_tile <= 6) ring = 2;
    // T1 weights: two loads ahead on every launch (its decode keeps each load's
    // registers longer; 2B T1 stack 0.668 -> 0.647 ms per token, 100B-class
    // 7.86 -> 7.78 ms; 8 and 16 slower)
    if (fmt == kFmtT1) ring = 2;
    if (ring > t * per_tile_w) ring = t * per_tile_w;
    const bool li = long_input(64 * nw);
    p.kernel = fmt == kFmtT1 ? select_kernel<kFmtT1>(xmode, ring, li, bal, wide, prio)
                             : select_kernel<kFmt2>(xmode, ring, li, bal, wide, prio);
    p.lds = (size_t)lds_bytes(t, a.M, a.K, fmt);
    return p;
  };
  Plan pl = plan(1, false);
  if (!latency) {
    int k = kWgsPerCu;
    for (;; ++k)
      if ((total_tiles + cus * k - 1) / (cus * k) <= kMaxTiles) break;
    const int t = (total_tiles + cus * k - 1) / (cus * k);
    pl = plan(t, false);
    // List runs (the tiles of all the matrices as one list, a run may cross into
    // the next matrix; every matrix at least a run long, so that a run covers at
    // most two) in two cases, measured on the 100B-class stack:
    //  * with the two workgroups per compute unit, the one dispatched first (b <
    //    cus) streams faster (its waves are the older ones), and the other then
    //    runs alone: when the tiles come to S = total / cus per compute unit,
    //    S >= 5, the first takes L1 = S / 2 + 1 (rounded down) and the second the
    //    rest (q+k+v, three 8192-row matrices: 4 + 2 tiles, 12.5 -> 12.2 us;
    //    gate+up, two 28672-row matrices: 8 + 6, 24.0 -> 23.3 us, where 9 + 5
    //    and the equal split were slower; the 8B-class gate+up, two 14336-row
    //    matrices, 4 + 3 in 512 workgroups instead of 448 runs of 4: 8B-class
    //    stack 0.921 -> 0.897 ms per token), or, where the second one stages at
    //    a raised priority (below), S / 2 each;
    //  * else, where each matrix's split rounded up needs more workgroups than
    //    the compute units hold two at a time (three 8192-row matrices in runs of
    //    3: 513), runs of qt + 1 for the first rt workgroups and qt for the rest
    //    (6.01 -> 5.91 ms per 100B-class token).
    auto runs_fit = [&](int len) {
      for (int j = 0; j < a.count; ++j)
        if (tiles[j] < len) return false;
      return true;
    };
    const int S = total_tiles % cus == 0 ? total_tiles / cus : 0;
    // With the staging priority (even S on a chip of kPrioSplit compute units,
    // fused 2-bit launches) the two workgroups take S / 2 tiles each: 100B-class
    // q+k+v 3 + 3, gate+up 7 + 7, stack 5.64 -> 5.60 ms per token (for odd S, the
    // 8B-class gate+up 3 + 4 with it was 2% slower than 4 + 3 without).
    const bool even_prio = (xmode == 1 || xmode == 2) && fmt == kFmt2 && cus == kPrioSplit &&
                           S % 2 == 0;
    const int L1 = even_prio ? S / 2 : S / 2 + 1;
    if (k == kWgsPerCu && S >= 5 && L1 <= kMaxTiles && runs_fit(L1)) {
      pl = plan(L1, true, 2 * cus, false, even_prio);
      pl.l1 = L1;
      pl.l2 = S - pl.l1;
      pl.h = cus;
    } else if (pl.wgs > cus * k && a.count > 1 && (total_tiles + t - 1) / t <= cus * k &&
               runs_fit(t)) {
      pl = plan(t, true);
      pl.l2 = total_tiles / pl.wgs;
      pl.l1 = pl.l2 + 1;
      pl.h = total_tiles % pl.wgs;
    }
    // At most one tile per compute unit (the 8B-class down projection, 14336 ->
    // 4096: 256 tiles): four-wave workgroups would leave each compute unit one
    // workgroup, half its wave slots; eight-wave workgroups split each tile's K
    // over twice the waves (fused 2-bit launches; 9.0 -> 7.1 us).  With more
    // tiles than compute units, two four-wave workgroups per compute unit
    // measured faster (eight-wave workgroups of 2-14 tiles: 8B-class q+k+v 5.66
    // -> 5.77 us, gate+up 8.85 -> 10.2; 100B-class launches +0.3-4%)
    if ((xmode == 1 || xmode == 2) && fmt == kFmt2 && total_tiles <= cus)
      pl = plan(1, false, 0, true);
    // one tile per workgroup, two workgroups on some or every compute unit: the
    // second one stages at a raised wave priority (gemv_kernel PRIO; ring depth 4
    // only; the 8B-class q+k+v, 384 workgroups: stack 0.795 -> 0.790 ms per token)
    else if ((xmode == 1 || xmode == 2) && fmt == kFmt2 && cus == kPrioSplit && !pl.bal &&
             pl.tpw == 1 && pl.wgs > cus && pl.wgs <= kWgsPerCu * cus)
      pl = plan(1, false, 0, false, true);
  }
  const int tpw = pl.tpw, wgs = pl.wgs;
  const void* kernel = pl.kernel;
  const size_t lds = pl.lds;
  a.tiles_per_wg = tpw;
  a.mdiv = (65536 + a.M - 1) / a.M;  // tt / M == (tt * mdiv) >> 16 for tt < 256, M <= 16
  int w0 = 0;
  for (int j = 0; j < kMaxGroup; ++j) {
    a.wg0[j] = w0;
    if (j < a.count) w0 += (tiles[j] + tpw - 1) / tpw;
  }
  // the preloaded leading arguments (LeadArgs)
  const void* xin = fused ? a.xf : static_cast<const void*>(a.xq);
  const uint8_t* wp0 = a.wp[0];
  const uint8_t* wp1 = a.count > 1 ? a.wp[1] : a.wp[0];
  const uint8_t* wp2 = a.count > 2 ? a.wp[2] : a.wp[0];
  int n0 = a.n[0], n1 = a.count > 1 ? a.n[1] : 0, n2 = a.count > 2 ? a.n[2] : 0;
  for (int j = a.count; j < kMaxGroup; ++j) {   // balanced runs load slot count, never use it
    a.ws[j] = a.ws[0];
    a.y[j] = a.y[0];
    a.acc[j] = a.acc[0];
  }
  // per-matrix runs: the first workgroups of matrices 1 and 2; list runs:
  // L1 | L2 << 8 and h
  int s1 = pl.bal ? pl.l1 | (pl.l2 << 8) : a.wg0[1];
  int s2 = pl.bal ? pl.h : a.wg0[2];
  uint32_t mtck = (uint32_t)a.M | ((uint32_t)tpw << 5) | ((uint32_t)a.count << 10) |
                  ((uint32_t)a.K << 13);
  void* args[] = {&xin, &wp0, &wp1, &wp2, &n0, &n1, &n2, &s1, &s2, &mtck, &a};
  return hipLaunchKernel(kernel, dim3((unsigned)wgs), dim3(pl.wide ? 512 : kThreads), args, lds,
                         s);
}

}  // namespace bitnet
