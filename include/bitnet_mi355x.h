/*
 * bitnet_mi355x.h - C ABI of the BitNet b1.58 W1.58A8 ternary linear layer for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (web pages, cited by title and section):
 *  - onedollarvps.pages.dev, "如何在本地運行 BitNet B1.58（1-Bit LLM）", section 2
 *    (technical background, 1-bit vs 1.58-bit quantisation): weights are divided by
 *    their mean absolute value, then rounded and clipped to {-1, 0, +1}.
 *  - dashen-tech.com, "BitNet.cpp 深度解析", section 2.3 (I2_S format): two bits per
 *    stored weight; section 3.1 (integer matmul): with ternary weights the product
 *    is the sum of inputs under +1 weights minus the sum under -1 weights.
 *  - communeify.com, "微軟 BitNet b1.58 震撼登場", 2B4T section, quantisation
 *    details: W1.58A8, i.e. ternary weights and 8-bit integer activations.
 *
 * Readings where the pages are silent (the CPU oracle uses the same ones):
 *  gamma  = RN32(exact sum|W| / (N*K)), gamma* = max(gamma, RN32(1e-5));
 *  q      = clip(round_half_even(RN32(W / gamma*)), -1, 1);
 *  packed = code q+1 in {0,1,2}, four codes per byte, least significant pair
 *           first, row n at bytes [n*K/4, (n+1)*K/4);
 *  per token m: astar = max(max_k |x[m,k]|, RN32(1e-5)), s = RN32(127 / astar),
 *           xq = clip(round_half_even(RN32(x*s)), -128, 127), d[m] = RN32(astar / 127);
 *  acc[m,n] = sum_k q[n,k] * xq[m,k] (exact int32);
 *  y[m,n]   = RN32(float(acc) * RN32(gamma* * d[m])); bf16 y = round-to-nearest-even
 *             (a NaN y, possible only from non-finite inputs, has an unspecified payload).
 * Every integer result (packed bytes, gamma*, xq, d, acc) is bit-identical to the
 * CPU oracle, and so is y under the rescale order above.
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers owned by the caller.  Row-major,
 *    contiguous, no strides.  No call allocates, frees, synchronises or keeps a
 *    pointer after it returns.
 *  - All work is enqueued on `stream` (0 = the legacy default stream); results are
 *    ready when the caller's own synchronisation on that stream completes.
 *  - Arguments are validated before any HIP call; a bad argument returns its
 *    status and enqueues nothing.  A failed launch returns BITNET_ERR_HIP.  A fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - 16-byte aligned packed weights / int8 activations with K % 64 == 0 take the
 *    fast kernels; any other K % 4 == 0 layout takes a slower generic kernel with
 *    identical results.
 *  - The library keeps no mutable global state: calls are thread-safe.  Calls that
 *    share an output buffer on different streams race, as with any kernel.
 */
#ifndef BITNET_MI355X_H
#define BITNET_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bitnet_status {
  BITNET_OK = 0,
  BITNET_ERR_NULL = 1,      /* a required pointer is NULL */
  BITNET_ERR_SHAPE = 2,     /* a size is negative, K % 4 != 0, or a size limit is exceeded */
  BITNET_ERR_DTYPE = 3,     /* unknown bitnet_dtype value */
  BITNET_ERR_ALIGN = 4,     /* an fp32/bf16 pointer is not aligned to its element size */
  BITNET_ERR_WORKSPACE = 5, /* workspace NULL or smaller than the queried size */
  BITNET_ERR_HIP = 6        /* a HIP launch failed (hipGetLastError) */
} bitnet_status;

typedef enum bitnet_dtype { BITNET_F32 = 0, BITNET_BF16 = 1 } bitnet_dtype;

/* One weight matrix of a grouped call (all pointers device memory; they may be
 * NULL when the call has no tokens or the matrix no rows). */
typedef struct bitnet_matrix {
  const uint8_t *w_packed; /* [N][K/4] packed codes from bitnet_quantize_weights */
  const float *w_scale;    /* [1] gamma* */
  int64_t N;               /* output features, >= 0 */
  void *y;                 /* [M][N] fp32 or bf16 out */
  int32_t *acc_out;        /* optional [M][N] int32 accumulators, or NULL */
} bitnet_matrix;

/* Largest N*K accepted by bitnet_quantize_weights (exact-sum limit): 2^38 - 1. */
#define BITNET_MAX_WEIGHTS ((int64_t)1 << 38)
/* Largest K accepted by the linear calls: |acc| <= 127*K stays below 2^24, so
 * float(acc) is exact. */
#define BITNET_MAX_K ((int64_t)131072)

/* Human-readable name of a status value (static string, never NULL). */
const char *bitnet_status_string(int status);

/* Bytes of the packed weight matrix: N * (K / 4).  0 for invalid sizes. */
size_t bitnet_packed_bytes(int64_t N, int64_t K);

/* Bytes of device workspace bitnet_quantize_weights needs (a constant 16640). */
size_t bitnet_quantize_weights_workspace_bytes(int64_t N, int64_t K);

/*
 * Weight quantisation: the absolute-mean scale and the ternary 2-bit packing
 * (onedollarvps, section 2; dashen-tech, section 2.3).
 *   w        [N][K] fp32 or bf16 master weights (w_dtype), element-aligned.
 *   N, K     N >= 1, K >= 4, K % 4 == 0, N*K < BITNET_MAX_WEIGHTS.
 *   w_packed [N][K/4] uint8 out (layout above).
 *   w_scale  [1] fp32 out: gamma*.  If W holds Inf or NaN, *w_scale = NaN and
 *            w_packed is unspecified (detected by the caller after its sync).
 *   workspace >= bitnet_quantize_weights_workspace_bytes() bytes of device memory,
 *            8-byte aligned; clobbered; may be reused once the call's work is done.
 * The sum of |W| is exact (integer per-exponent buckets), so gamma* does not
 * depend on the launch configuration.
 */
bitnet_status bitnet_quantize_weights(const void *w, int w_dtype, int64_t N, int64_t K,
                                      uint8_t *w_packed, float *w_scale, void *workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * bitnet_quantize_weights for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the library's own workspace in
 * place of the caller's.  That workspace is a device array of 16640 bytes
 * (bitnet_quantize_weights_workspace_bytes()) in the library's code object: each
 * device holds one copy from the first call on it until the process ends.  The
 * call allocates and frees nothing.  Arguments and limits as for
 * bitnet_quantize_weights (N*K < BITNET_MAX_WEIGHTS; the workspace size does not
 * depend on N or K).  Every call on one device shares its array and clears it
 * first (with a kernel): calls that overlap on one device (two streams, or two
 * host threads) race and must be serialised by the caller.  First call on a
 * device: BITNET_ERR_HIP if the array's address cannot be looked up.
 */
bitnet_status bitnet_quantize_weights_noalloc(const void *w, int w_dtype, int64_t N, int64_t K,
                                              uint8_t *w_packed, float *w_scale,
                                              hipStream_t stream);

/*
 * Per-token absmax int8 activation quantisation (communeify, quantisation
 * details: 8-bit activations; the scheme is the per-token reading above).
 *   x        [M][K] fp32 or bf16 (x_dtype), finite values, element-aligned.
 *   M, K     M >= 0 (M == 0 is a no-op), K >= 0 (K == 0: d = RN32(RN32(1e-5)/127)).
 *   x_q      [M][K] int8 out, values in [-127, 127].
 *   x_scale  [M] fp32 out: d[m].
 */
bitnet_status bitnet_quantize_acts(const void *x, int x_dtype, int64_t M, int64_t K,
                                   int8_t *x_q, float *x_scale, hipStream_t stream);

/*
 * Ternary linear layer on quantised inputs: integer contraction and rescale
 * (dashen-tech, section 3.1).
 *   w_packed [N][K/4] uint8 from bitnet_quantize_weights.
 *   w_scale  [1] fp32 gamma* (device).
 *   x_q      [M][K] int8; x_scale [M] fp32 d[m].
 *   M, N, K  M >= 0, N >= 0 (0 = no-op), K % 4 == 0, 0 <= K <= BITNET_MAX_K.
 *   y        [M][N] out, fp32 or bf16 (y_dtype), element-aligned.
 *   acc_out  optional [M][N] int32 out (NULL to skip): the exact accumulator.
 * M <= 16 (K % 64 == 0) runs the HBM-streaming decode kernel, larger M the
 * int8-MFMA prefill kernel; both produce identical integers.
 */
bitnet_status bitnet_ternary_linear(const uint8_t *w_packed, const float *w_scale,
                                    const int8_t *x_q, const float *x_scale, int64_t M,
                                    int64_t N, int64_t K, void *y, int y_dtype,
                                    int32_t *acc_out, hipStream_t stream);

/*
 * Several weight matrices that share one input (for example the q, k and v
 * projections, or gate and up): the same results as `count` calls of
 * bitnet_ternary_linear with the same x_q / x_scale, in as few kernel launches as
 * the decode kernel allows (up to 4 matrices per launch when M <= 16).
 *   mats     HOST array of `count` >= 1 descriptors (read during the call only).
 *   x_q, x_scale, M, K, y_dtype  as bitnet_ternary_linear; every y has y_dtype.
 */
bitnet_status bitnet_ternary_linear_multi(const bitnet_matrix *mats, int count,
                                          const int8_t *x_q, const float *x_scale, int64_t M,
                                          int64_t K, int y_dtype, hipStream_t stream);

/*
 * Activation quantisation fused into the layer, for chaining layers without a
 * separate quantisation launch (one chained step: y = linear(quant(x))).
 *   x        [M][K] fp32 or bf16 (x_dtype), finite values.
 *   x_q, x_scale  [M][K] int8 and [M] fp32 out: the same values
 *            bitnet_quantize_acts(x) writes (so further layers that share this
 *            input can call bitnet_ternary_linear on them).
 *   other arguments as bitnet_ternary_linear.
 * For M <= 4 with M*(K+16) <= 46 KiB (and K % 64 == 0) each workgroup of the
 * decode kernel quantises the activations itself; otherwise this is
 * bitnet_quantize_acts followed by bitnet_ternary_linear on the same stream.
 */
bitnet_status bitnet_quant_linear(const uint8_t *w_packed, const float *w_scale,
                                  const void *x, int x_dtype, int64_t M, int64_t N, int64_t K,
                                  int8_t *x_q, float *x_scale, void *y, int y_dtype,
                                  int32_t *acc_out, hipStream_t stream);

/*
 * bitnet_quant_linear for several matrices sharing the input x: quantises x once
 * (into x_q / x_scale) and applies every matrix, fused into one launch for up to
 * 4 matrices when M <= 4 and M*(K+16) <= 46 KiB.
 */
bitnet_status bitnet_quant_linear_multi(const bitnet_matrix *mats, int count, const void *x,
                                        int x_dtype, int64_t M, int64_t K, int8_t *x_q,
                                        float *x_scale, int y_dtype, hipStream_t stream);

/*
 * Input prologue of a layer: its neighbours on the path, applied before the
 * int8 quantisation (communeify.com, section on BitNet b1.58 2B4T, architecture
 * item: squared-ReLU activation, subln normalisation, no bias terms).
 *   up           NULL, or the up projection [M][K] (same dtype and alignment as
 *                x): x is then the gate projection and the layer input is
 *                v = RN32(RN32(max(x, 0)^2) * up), elementwise.
 *   norm_weight  NULL, or the RMS norm weight w [K] fp32 (device, 4-byte
 *                aligned): the layer input v is RMS-normalised and scaled,
 *                u = RN32(RN32(v * r) * w) elementwise, with
 *                r = RN32(1 / sqrt(RN32(ms + eps))) (square root and division in
 *                float64) and ms = the exactly rounded mean of v^2 over the token
 *                (one rounding of the exact sum / K, whatever the order of the
 *                launch's sums); u is then quantised per token as above, so
 *                x_scale is max|u| / 127.  Bit-exact against that definition.
 *                Needs K >= 1.
 *   norm_eps     eps >= 0, finite.  With eps = 0 a token whose ms rounds to 0
 *                (all zeros, or a mean below 2^-150) has r = +inf and its codes
 *                and scale are undefined.
 */
typedef struct bitnet_act_prologue {
  const void *up;
  const float *norm_weight;
  float norm_eps;
} bitnet_act_prologue;

/*
 * bitnet_quantize_acts with the input prologue `pro` (NULL: none): the codes
 * and scales of the prologue's output u.
 */
bitnet_status bitnet_quantize_acts_ex(const void *x, int x_dtype, const bitnet_act_prologue *pro,
                                      int64_t M, int64_t K, int8_t *x_q, float *x_scale,
                                      hipStream_t stream);

/*
 * bitnet_quant_linear_multi with the input prologue `pro` (NULL: none): the
 * layers see the gated and / or normalised input, quantised as
 * bitnet_quantize_acts_ex writes it (also into x_q / x_scale).  Fused into the
 * decode kernel under the same conditions as bitnet_quant_linear_multi when x,
 * up and norm_weight are 16-byte aligned.
 */
bitnet_status bitnet_quant_linear_ex(const bitnet_matrix *mats, int count, const void *x,
                                     int x_dtype, const bitnet_act_prologue *pro, int64_t M,
                                     int64_t K, int8_t *x_q, float *x_scale, int y_dtype,
                                     hipStream_t stream);

/*
 * Five ternary weights per byte ("T1"): a denser layout for the HBM-bound decode
 * path.  A ternary weight carries log2(3) ~ 1.58 bits (onedollarvps, section 1
 * and section 2); the 0.4 GB of non-embedding memory the communeify comparison
 * table gives for the 2B model is about 1.6 bits per weight, which 3^5 = 243 <=
 * 256 reaches.  The pages define no layout; this one is:
 *   the codes c_j = q_j + 1 of five weights form v = sum_j c_j * 3^j, stored as
 *   the byte ceil(256 * v / 243) (the base-3 fraction v/243 in 8-bit fixed
 *   point, rounded up; 13 byte values are never written);
 *   a row is padded with q = 0 to a multiple of 80 weights and cut into blocks
 *   of 80 weights in 16 bytes: byte i of block b holds the weights
 *   k = 80*b + 16*j + i as digit j (j = 0..4);
 *   row n occupies bytes [n*R, (n+1)*R), R = 16 * ceil(K / 80).
 * Results of the T1 calls are bit-identical to the 2-bit calls on the same
 * ternary weights.
 */

/* Bytes of a T1 matrix: N * 16 * ceil(K / 80).  0 for negative sizes. */
size_t bitnet_t1_packed_bytes(int64_t N, int64_t K);

/*
 * bitnet_quantize_weights with the T1 output layout.
 *   N >= 1, K >= 1 (any K: rows are padded), N*K < BITNET_MAX_WEIGHTS.
 *   w_t1     [N][16*ceil(K/80)] uint8 out, 16-byte aligned.
 *   other arguments, gamma* and the non-finite behaviour as bitnet_quantize_weights.
 */
bitnet_status bitnet_quantize_weights_t1(const void *w, int w_dtype, int64_t N, int64_t K,
                                         uint8_t *w_t1, float *w_scale, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * Exact conversion of a 2-bit packed matrix (bitnet_quantize_weights layout,
 * K >= 4, K % 4 == 0, N >= 0) to T1.  w_t1 [N][16*ceil(K/80)], 16-byte aligned.
 * Bytes holding the unused 2-bit code 3 give unspecified output bytes.
 */
bitnet_status bitnet_repack_t1(const uint8_t *w_packed, int64_t N, int64_t K, uint8_t *w_t1,
                               hipStream_t stream);

/*
 * bitnet_ternary_linear_multi on T1 weights: every mats[i].w_packed is a T1
 * matrix (16-byte aligned).  Needs K >= 16, K % 16 == 0 and a 16-byte aligned
 * x_q; otherwise BITNET_ERR_SHAPE / BITNET_ERR_ALIGN (there is no generic
 * kernel for this layout).  Runs the decode kernel; M > 16 runs in groups of
 * 16 tokens, each streaming the weights again.
 */
bitnet_status bitnet_ternary_linear_t1(const bitnet_matrix *mats, int count, const int8_t *x_q,
                                       const float *x_scale, int64_t M, int64_t K, int y_dtype,
                                       hipStream_t stream);

/*
 * Prefill weight layout: the same 2-bit codes, rearranged once for the prefill
 * kernel (matrix cores) so that each of its 16-byte loads reads 1 KiB of
 * contiguous memory per wave and the codes expand to int8 in natural k order
 * without byte shuffles (dashen-tech.com, "BitNet.cpp 深度解析", section 2.3,
 * describes the 2-bit storage; this arrangement is the library's own).  Rows
 * are padded with q = 0 to a multiple of 32 and K to a multiple of 128; blocks
 * of 32 rows x 128 k (1024 bytes) are stored block-row-major, block (rb, s) at
 * byte (rb * ceil(K/128) + s) * 1024; 16-byte chunk L = r + 32 h of a block
 * holds row 32 rb + r at k = 128 s + 64 h + 0..63, and its dword j the weights
 * k = 128 s + 64 h + 16 j + t (t = 0..15), the code q + 1 of weight t at bits
 * 8 (t mod 4) + 2 (t div 4).
 * bitnet_prefill_layout_bytes: ceil(N/32) * ceil(K/128) * 1024 (0 for N < 0 or
 * K < 0).
 */
size_t bitnet_prefill_layout_bytes(int64_t N, int64_t K);

/*
 * Exact conversion of a 2-bit packed matrix (bitnet_quantize_weights layout) to
 * the prefill layout.  K >= 64, K % 64 == 0, N >= 0, N*K < BITNET_MAX_WEIGHTS;
 * w_packed and w_prefill (bitnet_prefill_layout_bytes(N, K) bytes, caller-owned)
 * 16-byte aligned.  Bytes holding the unused code 3 give unspecified output.
 */
bitnet_status bitnet_repack_prefill(const uint8_t *w_packed, int64_t N, int64_t K,
                                    uint8_t *w_prefill, hipStream_t stream);

/*
 * bitnet_ternary_linear_multi on weights in the prefill layout (every
 * mats[i].w_packed, 16-byte aligned): the prefill kernel for any M >= 1, up to
 * four matrices per launch, the same results bit for bit.  Needs K >= 64,
 * K % 64 == 0 and a 16-byte aligned x_q; otherwise BITNET_ERR_SHAPE /
 * BITNET_ERR_ALIGN (there is no generic kernel for this layout).
 */
bitnet_status bitnet_ternary_linear_prefill(const bitnet_matrix *mats, int count,
                                            const int8_t *x_q, const float *x_scale, int64_t M,
                                            int64_t K, int y_dtype, hipStream_t stream);

/*
 * bitnet_quant_linear_ex on T1 weights (same layout requirements as
 * bitnet_ternary_linear_t1).  The quantisation and prologue are fused into the
 * decode launch when M <= 4 and the activations of all tokens fit one LDS phase
 * (M * (80 * ceil(K/80) + 16) <= 46 KiB) and x, up and norm_weight are 16-byte
 * aligned.
 */
bitnet_status bitnet_quant_linear_t1(const bitnet_matrix *mats, int count, const void *x,
                                     int x_dtype, const bitnet_act_prologue *pro, int64_t M,
                                     int64_t K, int8_t *x_q, float *x_scale, int y_dtype,
                                     hipStream_t stream);

/*
 * The contraction by table lookup (juejin.cn, "Microsoft BitNet", technical
 * principles, item 2: bitnet.cpp's kernels use T-MAC's lookup-table method;
 * dashen-tech, section 3.2: the TL1/TL2 kernel types).  Per token, each pair of
 * int8 activations gets a table of 16 partial sums, entry c0 + 4*c1 =
 * (c0 - 1)*x[2g] + (c1 - 1)*x[2g+1], and each nibble of the 2-bit layout (two
 * weights' codes) indexes it.  Same integers and outputs as
 * bitnet_ternary_linear; a second kernel family for comparison with the
 * matrix-core decode kernel.
 */

/* Bytes of workspace bitnet_ternary_linear_lut needs: 16*K (one token's tables)
 * plus 4*N (accumulators), each rounded up to 256.  0 for negative sizes. */
size_t bitnet_lut_workspace_bytes(int64_t N, int64_t K);

/*
 * bitnet_ternary_linear by table lookup.
 *   w_packed [N][K/4] (2-bit layout), 16-byte aligned; K >= 64, K % 64 == 0.
 *   workspace >= bitnet_lut_workspace_bytes(N, K) bytes of device memory,
 *            16-byte aligned; clobbered.
 *   other arguments as bitnet_ternary_linear.
 * Tokens run one after another, three launches each (tables, lookups,
 * rescale), so the weights stream once per token.
 */
bitnet_status bitnet_ternary_linear_lut(const uint8_t *w_packed, const float *w_scale,
                                        const int8_t *x_q, const float *x_scale, int64_t M,
                                        int64_t N, int64_t K, void *y, int y_dtype,
                                        int32_t *acc_out, void *workspace,
                                        size_t workspace_bytes, hipStream_t stream);

/*
 * Query of this library's launch (no page passage: it describes the
 * implementation, for callers and tests that need to know which kernel variant a
 * call uses): the tile of the prefill kernel (M > 16 tokens, K % 64 == 0) that
 * bitnet_ternary_linear_multi uses for M tokens over `count` matrices of N[j]
 * rows and inputs of K on the current device: *tokens_per_tile x *rows_per_tile
 * per workgroup (256 x 256, 192 x 256, 128 x 256, 128 x 128 or 64 x 128).  If
 * *first_launch_tokens > 0, the first *first_launch_tokens tokens run as one
 * launch with that tile and the remaining tokens as a second launch with the
 * tile this query returns for them.  If *first_launch_rows > 0 (a multiple of
 * 256), the matrices' rows are taken in order, each matrix's row count rounded
 * up to a multiple of 256, and the first *first_launch_rows of them run as one
 * launch with that tile, the remaining rows (the rest of the matrix the cut
 * falls in, then the following matrices) as a second launch with the tile this
 * query returns for those row counts.  M in 1..2^31-1, count in 1..4, N[j] >= 1,
 * K >= 1 (BITNET_ERR_SHAPE otherwise); asks the HIP runtime for the compute unit
 * count (1 if it cannot say).
 */
bitnet_status bitnet_prefill_tile(int64_t M, const int64_t *N, int count, int64_t K,
                                  int *tokens_per_tile, int *rows_per_tile,
                                  int64_t *first_launch_tokens, int64_t *first_launch_rows);

/*
 * Decode chain: a sequence of fused act-quant + ternary linear stages (each one
 * bitnet_quant_linear_multi: quantise the stage input per token, then apply up
 * to four matrices that share it) run in ONE launch per token, with a grid-wide
 * barrier between stages, so a stage may read any earlier stage's outputs (the
 * layer stack of a decoder: q, k, v from the layer input, o from q, gate and up
 * from o, down from up, the next layer from down).  Results are those of the
 * bitnet_quant_linear_multi calls made one after another, bit for bit (same
 * arithmetic: onedollarvps section 2, dashen-tech sections 2.3 and 3.1,
 * communeify quantisation details).
 *
 * Plan once, run per token:
 *   bitnet_chain_plan checks every stage, assigns row tiles to workgroups and
 *   copies the stage table into `plan` (device memory of
 *   bitnet_chain_plan_bytes(n_stages) bytes, 256-byte aligned, caller-owned,
 *   untouched by anything else while the chain is in use).  It synchronises
 *   (blocking copy), so it is a set-up call: not under graph capture.
 *   bitnet_chain_run enqueues one cooperative launch on `stream`; the pointers
 *   in the stages must stay valid.  Runs on one device must not overlap (they
 *   share the plan's barrier counters).
 * Stage requirements: M in 1..4 (decode), K % 64 == 0, 64 <= K, M * (K + 16) <=
 * 65536; x, x_q, every w_packed 16-byte aligned; y and acc_out as for
 * bitnet_quant_linear_multi; N >= 1 per matrix; 1..4 matrices per stage.
 * Otherwise BITNET_ERR_SHAPE / BITNET_ERR_NULL / BITNET_ERR_ALIGN /
 * BITNET_ERR_DTYPE, and nothing is copied.
 * Every wait inside the launch is bounded: if a barrier does not complete (it
 * cannot while the chain's workgroups are all resident, which the cooperative
 * launch guarantees), the launch stops waiting and sets a sticky error word,
 * readable with bitnet_chain_error (1 = abandoned, outputs unspecified; reset
 * by planning again).
 */
typedef struct bitnet_chain_stage {
  const void *x;               /* stage input [M][K] */
  int x_dtype;                 /* BITNET_F32 or BITNET_BF16 */
  int y_dtype;                 /* dtype of every output y of the stage */
  int64_t K;
  const bitnet_matrix *mats;   /* 1..4 matrices sharing x (read at plan time) */
  int count;
  int8_t *x_q;                 /* out [M][K]: the quantised input */
  float *x_scale;              /* out [M]: its token scales */
} bitnet_chain_stage;

typedef struct bitnet_chain {
  void *plan;                  /* the device memory given to bitnet_chain_plan */
  int n_stages, M;
  int grid;                    /* workgroups of the launch (all co-resident) */
  int kmax, tmax;              /* largest K and row tiles per workgroup of any stage */
  int ring;                    /* weight loads in flight per lane: 4 (default), 8 or 16 */
} bitnet_chain;

size_t bitnet_chain_plan_bytes(int n_stages);
bitnet_status bitnet_chain_plan(const bitnet_chain_stage *stages, int n_stages, int64_t M,
                                void *plan, size_t plan_bytes, bitnet_chain *chain);
bitnet_status bitnet_chain_run(const bitnet_chain *chain, hipStream_t stream);
/* Reads the plan's error word into *error (0 = every run so far completed its
 * barriers).  Synchronises with the device. */
bitnet_status bitnet_chain_error(const bitnet_chain *chain, int *error);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_MI355X_H */
