// C ABI of libbitnet_mi355x: argument validation and kernel dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues nothing.
#include "bitnet_mi355x.h"
#include "bitnet_internal.h"

#include <string.h>

#include <vector>

namespace {

constexpr int64_t kInt32Max = 2147483647;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool valid_dtype(int d) { return d == BITNET_F32 || d == BITNET_BF16; }
uintptr_t esize(int d) { return d == BITNET_BF16 ? 2 : 4; }

bitnet_status from_hip(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_ERR_HIP; }

// Fast kernels read 16-byte vectors of packed weights and int8 activations.
bool fast_layout(const void* w_packed, const void* x_q, int64_t K) {
  return K >= 64 && (K % 64) == 0 && aligned(w_packed, 16) && aligned(x_q, 16);
}

bitnet_status check_sizes(int64_t M, int64_t K) {
  if (M < 0 || K < 0 || (K % 4) != 0 || K > BITNET_MAX_K || M > kInt32Max) return BITNET_ERR_SHAPE;
  return BITNET_OK;
}

// Per-matrix checks shared by the single and grouped calls.  A matrix with no
// outputs (M == 0 or N == 0) is never read or written, so its pointers may be NULL.
bitnet_status check_matrix(const bitnet_matrix& m, int64_t M, int64_t K, int y_dtype) {
  if (m.N < 0 || m.N > kInt32Max || M * m.N > ((int64_t)1 << 46)) return BITNET_ERR_SHAPE;
  if (M == 0 || m.N == 0) return BITNET_OK;
  if (!m.w_scale || !m.y || (K > 0 && !m.w_packed)) return BITNET_ERR_NULL;
  if (!aligned(m.y, esize(y_dtype)) || !aligned(m.w_scale, 4) ||
      (m.acc_out && !aligned(m.acc_out, 4)))
    return BITNET_ERR_ALIGN;
  return BITNET_OK;
}

bitnet_status check_group(const bitnet_matrix* mats, int count, int64_t M, int64_t K,
                          int y_dtype) {
  if (!mats) return BITNET_ERR_NULL;
  if (count < 1) return BITNET_ERR_SHAPE;
  if (!valid_dtype(y_dtype)) return BITNET_ERR_DTYPE;
  const bitnet_status s = check_sizes(M, K);
  if (s != BITNET_OK) return s;
  for (int i = 0; i < count; ++i) {
    const bitnet_status st = check_matrix(mats[i], M, K, y_dtype);
    if (st != BITNET_OK) return st;
  }
  return BITNET_OK;
}

bitnet::GemvArgs gemv_args(const bitnet_matrix* mats, int count, int64_t M, int64_t K,
                           int y_dtype) {
  bitnet::GemvArgs a{};
  for (int j = 0; j < count; ++j) {
    a.wp[j] = mats[j].w_packed;
    a.ws[j] = mats[j].w_scale;
    a.y[j] = mats[j].y;
    a.acc[j] = mats[j].acc_out;
    a.n[j] = (int)mats[j].N;
  }
  a.count = count;
  a.M = (int)M;
  a.K = (int)K;
  a.y_bf16 = y_dtype == BITNET_BF16 ? 1 : 0;
  return a;
}

bool all_fast(const bitnet_matrix* mats, int count, const void* x_q, int64_t K) {
  for (int j = 0; j < count; ++j)
    if (!fast_layout(mats[j].w_packed, x_q, K)) return false;
  return true;
}

// Quantised activations already in x_q / x_scale; M, K and every matrix valid.
bitnet_status run_linear(const bitnet_matrix* mats, int count, const int8_t* x_q,
                         const float* x_scale, int64_t M, int64_t K, int y_dtype,
                         hipStream_t stream) {
  if (M == 0) return BITNET_OK;
  const bool yb = y_dtype == BITNET_BF16;
  if (all_fast(mats, count, x_q, K) && bitnet::gemv_fits(M, K, bitnet::kFmt2)) {
    for (int j0 = 0; j0 < count; j0 += bitnet::kMaxGroup) {
      const int c = count - j0 < bitnet::kMaxGroup ? count - j0 : bitnet::kMaxGroup;
      bitnet::GemvArgs a = gemv_args(mats + j0, c, M, K, y_dtype);
      a.xq = x_q;
      a.xs = x_scale;
      const bitnet_status st = from_hip(bitnet::launch_gemv(a, 0, bitnet::kFmt2, stream));
      if (st != BITNET_OK) return st;
    }
    return BITNET_OK;
  }
  // prefill: matrices in the fast layout go to the matrix-core kernel in groups
  // of up to four per launch; the others to the generic kernel
  bitnet::GemmArgs g{};
  auto flush = [&]() -> bool {
    if (g.count == 0) return true;
    g.xq = x_q;
    g.xs = x_scale;
    g.M = (int)M;
    g.K = (int)K;
    g.y_bf16 = yb ? 1 : 0;
    const bool ok = bitnet::launch_gemm(g, stream) == hipSuccess;
    g = bitnet::GemmArgs{};
    return ok;
  };
  for (int j = 0; j < count; ++j) {
    const bitnet_matrix& m = mats[j];
    if (m.N == 0) continue;
    if (fast_layout(m.w_packed, x_q, K)) {
      g.wp[g.count] = m.w_packed;
      g.ws[g.count] = m.w_scale;
      g.y[g.count] = m.y;
      g.acc[g.count] = m.acc_out;
      g.n[g.count] = (int)m.N;
      if (++g.count == bitnet::kMaxGroup && !flush()) return BITNET_ERR_HIP;
    } else if (bitnet::launch_generic_linear(m.w_packed, m.w_scale, x_q, x_scale, M, m.N, K, m.y,
                                             yb, m.acc_out, stream) != hipSuccess) {
      return BITNET_ERR_HIP;
    }
  }
  return flush() ? BITNET_OK : BITNET_ERR_HIP;
}

bitnet::ActPrologue act_prologue(const bitnet_act_prologue* pro) {
  bitnet::ActPrologue p{nullptr, nullptr, 0.0f};
  if (pro) {
    p.up = pro->up;
    p.w = pro->norm_weight;
    p.eps = pro->norm_eps;
  }
  return p;
}

// The prologue's own operands (x, M, K already checked).
bitnet_status check_prologue(const bitnet_act_prologue* pro, int x_dtype, int64_t M, int64_t K) {
  if (!pro || M == 0) return BITNET_OK;
  if (pro->norm_weight) {
    if (K < 1) return BITNET_ERR_SHAPE;
    if (!aligned(pro->norm_weight, 4)) return BITNET_ERR_ALIGN;
    if (!(pro->norm_eps >= 0.0f) || pro->norm_eps > 3.4e38f) return BITNET_ERR_SHAPE;
  }
  if (pro->up && !aligned(pro->up, esize(x_dtype))) return BITNET_ERR_ALIGN;
  return BITNET_OK;
}

bitnet_status quant_linear(const bitnet_matrix* mats, int count, const void* x, int x_dtype,
                           const bitnet::ActPrologue& pro, int64_t M, int64_t K, int8_t* x_q,
                           float* x_scale, int y_dtype, hipStream_t stream) {
  if (M == 0) return BITNET_OK;
  if (all_fast(mats, count, x_q, K) && aligned(x, 16) && bitnet::gemv_fused_fits(M, K, bitnet::kFmt2) &&
      (!pro.up || aligned(pro.up, 16)) && (!pro.w || aligned(pro.w, 16))) {
    const int c = count < bitnet::kMaxGroup ? count : bitnet::kMaxGroup;
    bitnet::GemvArgs a = gemv_args(mats, c, M, K, y_dtype);
    a.xf = x;
    a.xq = x_q;
    a.xq_out = x_q;
    a.xs_out = x_scale;
    a.xup = pro.up;
    a.gnorm = pro.w;
    a.eps = pro.eps;
    if (bitnet::launch_gemv(a, x_dtype, bitnet::kFmt2, stream) != hipSuccess) return BITNET_ERR_HIP;
    if (count == c) return BITNET_OK;
    return run_linear(mats + c, count - c, x_q, x_scale, M, K, y_dtype, stream);
  }
  if (bitnet::launch_aq(x, x_dtype == BITNET_BF16, M, K, x_q, x_scale, pro, stream) != hipSuccess)
    return BITNET_ERR_HIP;
  return run_linear(mats, count, x_q, x_scale, M, K, y_dtype, stream);
}

// T1 weights (five codes per byte): only the decode kernel reads them, so M > 16
// runs as groups of 16 tokens.  Every matrix, x_q and K checked by check_t1.
bitnet_status run_linear_t1(const bitnet_matrix* mats, int count, const int8_t* x_q,
                            const float* x_scale, int64_t M, int64_t K, int y_dtype,
                            hipStream_t stream) {
  const int64_t ye = (int64_t)esize(y_dtype);
  for (int64_t t0 = 0; t0 < M; t0 += bitnet::kGemvMaxM) {
    const int64_t mt = M - t0 < bitnet::kGemvMaxM ? M - t0 : bitnet::kGemvMaxM;
    for (int j0 = 0; j0 < count; j0 += bitnet::kMaxGroup) {
      const int c = count - j0 < bitnet::kMaxGroup ? count - j0 : bitnet::kMaxGroup;
      bitnet_matrix sub[bitnet::kMaxGroup];
      for (int j = 0; j < c; ++j) {
        sub[j] = mats[j0 + j];
        sub[j].y = static_cast<char*>(sub[j].y) + t0 * sub[j].N * ye;
        if (sub[j].acc_out) sub[j].acc_out += t0 * sub[j].N;
      }
      bitnet::GemvArgs a = gemv_args(sub, c, mt, K, y_dtype);
      a.xq = x_q + t0 * K;
      a.xs = x_scale + t0;
      if (bitnet::launch_gemv(a, 0, bitnet::kFmtT1, stream) != hipSuccess) return BITNET_ERR_HIP;
    }
  }
  return BITNET_OK;
}

// T1 layout requirements on top of check_group: K % 16 == 0, K >= 16, 16-byte
// aligned weights and int8 activations.
bitnet_status check_t1(const bitnet_matrix* mats, int count, const void* x_q, int64_t M,
                       int64_t K) {
  if (K < 16 || K > bitnet::kGemvMaxK || (K % 16) != 0) return BITNET_ERR_SHAPE;
  if (M > 0 && !aligned(x_q, 16)) return BITNET_ERR_ALIGN;
  for (int j = 0; j < count; ++j)
    if (!aligned(mats[j].w_packed, 16)) return BITNET_ERR_ALIGN;
  return BITNET_OK;
}

bitnet_status quant_linear_t1(const bitnet_matrix* mats, int count, const void* x, int x_dtype,
                              const bitnet::ActPrologue& pro, int64_t M, int64_t K, int8_t* x_q,
                              float* x_scale, int y_dtype, hipStream_t stream) {
  if (M == 0) return BITNET_OK;
  if (aligned(x, 16) && bitnet::gemv_fused_fits(M, K, bitnet::kFmtT1) &&
      (!pro.up || aligned(pro.up, 16)) && (!pro.w || aligned(pro.w, 16))) {
    const int c = count < bitnet::kMaxGroup ? count : bitnet::kMaxGroup;
    bitnet::GemvArgs a = gemv_args(mats, c, M, K, y_dtype);
    a.xf = x;
    a.xq = x_q;
    a.xq_out = x_q;
    a.xs_out = x_scale;
    a.xup = pro.up;
    a.gnorm = pro.w;
    a.eps = pro.eps;
    if (bitnet::launch_gemv(a, x_dtype, bitnet::kFmtT1, stream) != hipSuccess) return BITNET_ERR_HIP;
    if (count == c) return BITNET_OK;
    return run_linear_t1(mats + c, count - c, x_q, x_scale, M, K, y_dtype, stream);
  }
  if (bitnet::launch_aq(x, x_dtype == BITNET_BF16, M, K, x_q, x_scale, pro, stream) != hipSuccess)
    return BITNET_ERR_HIP;
  return run_linear_t1(mats, count, x_q, x_scale, M, K, y_dtype, stream);
}

}  // namespace

extern "C" {

const char* bitnet_status_string(int status) {
  switch (status) {
    case BITNET_OK: return "ok";
    case BITNET_ERR_NULL: return "required pointer is NULL";
    case BITNET_ERR_SHAPE: return "invalid or unsupported shape";
    case BITNET_ERR_DTYPE: return "unknown dtype";
    case BITNET_ERR_ALIGN: return "pointer not aligned to its element size";
    case BITNET_ERR_WORKSPACE: return "workspace NULL or too small";
    case BITNET_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t bitnet_packed_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || (K % 4) != 0) return 0;
  return (size_t)N * (size_t)(K / 4);
}

size_t bitnet_quantize_weights_workspace_bytes(int64_t N, int64_t K) {
  (void)N;
  (void)K;
  return bitnet::kWqWorkspaceBytes;
}

bitnet_status bitnet_quantize_weights(const void* w, int w_dtype, int64_t N, int64_t K,
                                      uint8_t* w_packed, float* w_scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!w || !w_packed || !w_scale) return BITNET_ERR_NULL;
  if (!valid_dtype(w_dtype)) return BITNET_ERR_DTYPE;
  if (N < 1 || K < 4 || (K % 4) != 0 || N >= BITNET_MAX_WEIGHTS / K) return BITNET_ERR_SHAPE;
  if (!workspace || workspace_bytes < bitnet::kWqWorkspaceBytes) return BITNET_ERR_WORKSPACE;
  if (!aligned(w, esize(w_dtype)) || !aligned(w_scale, 4) || !aligned(workspace, 8))
    return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_wq(w, w_dtype == BITNET_BF16, N * K, w_packed, w_scale, workspace,
                                    stream));
}

bitnet_status bitnet_quantize_weights_noalloc(const void* w, int w_dtype, int64_t N, int64_t K,
                                              uint8_t* w_packed, float* w_scale,
                                              hipStream_t stream) {
  if (!w || !w_packed || !w_scale) return BITNET_ERR_NULL;
  if (!valid_dtype(w_dtype)) return BITNET_ERR_DTYPE;
  if (N < 1 || K < 4 || (K % 4) != 0 || N >= BITNET_MAX_WEIGHTS / K) return BITNET_ERR_SHAPE;
  if (!aligned(w, esize(w_dtype)) || !aligned(w_scale, 4)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_wq_noalloc(w, w_dtype == BITNET_BF16, N * K, w_packed, w_scale,
                                            stream));
}

size_t bitnet_t1_packed_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return (size_t)N * (size_t)(16 * ((K + 79) / 80));
}

bitnet_status bitnet_quantize_weights_t1(const void* w, int w_dtype, int64_t N, int64_t K,
                                         uint8_t* w_t1, float* w_scale, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  if (!w || !w_t1 || !w_scale) return BITNET_ERR_NULL;
  if (!valid_dtype(w_dtype)) return BITNET_ERR_DTYPE;
  if (N < 1 || K < 1 || N >= BITNET_MAX_WEIGHTS / K) return BITNET_ERR_SHAPE;
  if (!workspace || workspace_bytes < bitnet::kWqWorkspaceBytes) return BITNET_ERR_WORKSPACE;
  if (!aligned(w, esize(w_dtype)) || !aligned(w_scale, 4) || !aligned(workspace, 8) ||
      !aligned(w_t1, 16))
    return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_wq_t1(w, w_dtype == BITNET_BF16, N, K, w_t1, w_scale, workspace,
                                       stream));
}

bitnet_status bitnet_repack_t1(const uint8_t* w_packed, int64_t N, int64_t K, uint8_t* w_t1,
                               hipStream_t stream) {
  if (!w_packed || !w_t1) return BITNET_ERR_NULL;
  if (N < 0 || K < 4 || (K % 4) != 0 || (N > 0 && N >= BITNET_MAX_WEIGHTS / K))
    return BITNET_ERR_SHAPE;
  if (!aligned(w_t1, 16)) return BITNET_ERR_ALIGN;
  if (N == 0) return BITNET_OK;
  return from_hip(bitnet::launch_repack_t1(w_packed, N, K, w_t1, stream));
}

bitnet_status bitnet_ternary_linear_t1(const bitnet_matrix* mats, int count, const int8_t* x_q,
                                       const float* x_scale, int64_t M, int64_t K, int y_dtype,
                                       hipStream_t stream) {
  if (M > 0 && (!x_scale || !x_q)) return BITNET_ERR_NULL;
  bitnet_status st = check_group(mats, count, M, K, y_dtype);
  if (st != BITNET_OK) return st;
  st = check_t1(mats, count, x_q, M, K);
  if (st != BITNET_OK) return st;
  if (x_scale && !aligned(x_scale, 4)) return BITNET_ERR_ALIGN;
  if (M == 0) return BITNET_OK;
  return run_linear_t1(mats, count, x_q, x_scale, M, K, y_dtype, stream);
}

bitnet_status bitnet_quant_linear_t1(const bitnet_matrix* mats, int count, const void* x,
                                     int x_dtype, const bitnet_act_prologue* pro, int64_t M,
                                     int64_t K, int8_t* x_q, float* x_scale, int y_dtype,
                                     hipStream_t stream) {
  if (M > 0 && (!x_scale || !x || !x_q)) return BITNET_ERR_NULL;
  if (!valid_dtype(x_dtype)) return BITNET_ERR_DTYPE;
  bitnet_status st = check_group(mats, count, M, K, y_dtype);
  if (st != BITNET_OK) return st;
  st = check_t1(mats, count, x_q, M, K);
  if (st != BITNET_OK) return st;
  if (!aligned(x, esize(x_dtype)) || (x_scale && !aligned(x_scale, 4))) return BITNET_ERR_ALIGN;
  st = check_prologue(pro, x_dtype, M, K);
  if (st != BITNET_OK) return st;
  return quant_linear_t1(mats, count, x, x_dtype, act_prologue(pro), M, K, x_q, x_scale, y_dtype,
                         stream);
}

size_t bitnet_lut_workspace_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return bitnet::lut_workspace_bytes(N, K);
}

bitnet_status bitnet_ternary_linear_lut(const uint8_t* w_packed, const float* w_scale,
                                        const int8_t* x_q, const float* x_scale, int64_t M,
                                        int64_t N, int64_t K, void* y, int y_dtype,
                                        int32_t* acc_out, void* workspace,
                                        size_t workspace_bytes, hipStream_t stream) {
  if (!valid_dtype(y_dtype)) return BITNET_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 64 || (K % 64) != 0 || K > BITNET_MAX_K || M > kInt32Max ||
      N > kInt32Max || M * N > ((int64_t)1 << 46))
    return BITNET_ERR_SHAPE;
  if (M == 0 || N == 0) return BITNET_OK;
  if (!w_packed || !w_scale || !x_q || !x_scale || !y) return BITNET_ERR_NULL;
  if (!workspace || workspace_bytes < bitnet::lut_workspace_bytes(N, K))
    return BITNET_ERR_WORKSPACE;
  if (!aligned(w_packed, 16) || !aligned(workspace, 16) || !aligned(w_scale, 4) ||
      !aligned(x_scale, 4) || !aligned(y, esize(y_dtype)) || (acc_out && !aligned(acc_out, 4)))
    return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_lut(w_packed, w_scale, x_q, x_scale, M, N, K, y,
                                     y_dtype == BITNET_BF16, acc_out, workspace,
                                     bitnet::device_cus(), stream));
}

bitnet_status bitnet_quantize_acts_ex(const void* x, int x_dtype, const bitnet_act_prologue* pro,
                                      int64_t M, int64_t K, int8_t* x_q, float* x_scale,
                                      hipStream_t stream) {
  if (!valid_dtype(x_dtype)) return BITNET_ERR_DTYPE;
  if (M < 0 || K < 0 || M > kInt32Max) return BITNET_ERR_SHAPE;
  if (M == 0) return BITNET_OK;
  if (!x_scale || (K > 0 && (!x || !x_q))) return BITNET_ERR_NULL;
  if (!aligned(x, esize(x_dtype)) || !aligned(x_scale, 4)) return BITNET_ERR_ALIGN;
  const bitnet_status st = check_prologue(pro, x_dtype, M, K);
  if (st != BITNET_OK) return st;
  return from_hip(bitnet::launch_aq(x, x_dtype == BITNET_BF16, M, K, x_q, x_scale,
                                    act_prologue(pro), stream));
}

bitnet_status bitnet_quantize_acts(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* x_q,
                                   float* x_scale, hipStream_t stream) {
  return bitnet_quantize_acts_ex(x, x_dtype, nullptr, M, K, x_q, x_scale, stream);
}

bitnet_status bitnet_ternary_linear_multi(const bitnet_matrix* mats, int count,
                                          const int8_t* x_q, const float* x_scale, int64_t M,
                                          int64_t K, int y_dtype, hipStream_t stream) {
  if (M > 0 && (!x_scale || (K > 0 && !x_q))) return BITNET_ERR_NULL;
  const bitnet_status st = check_group(mats, count, M, K, y_dtype);
  if (st != BITNET_OK) return st;
  if (x_scale && !aligned(x_scale, 4)) return BITNET_ERR_ALIGN;
  return run_linear(mats, count, x_q, x_scale, M, K, y_dtype, stream);
}

size_t bitnet_prefill_layout_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return (size_t)bitnet::prefill_layout_bytes(N, K);
}

bitnet_status bitnet_repack_prefill(const uint8_t* w_packed, int64_t N, int64_t K,
                                    uint8_t* w_prefill, hipStream_t stream) {
  if (!w_packed || !w_prefill) return BITNET_ERR_NULL;
  if (N < 0 || K < 64 || (K % 64) != 0 || K > BITNET_MAX_K ||
      (N > 0 && N >= BITNET_MAX_WEIGHTS / K))
    return BITNET_ERR_SHAPE;
  if (!aligned(w_packed, 16) || !aligned(w_prefill, 16)) return BITNET_ERR_ALIGN;
  if (N == 0) return BITNET_OK;
  return from_hip(bitnet::launch_repack_prefill(w_packed, N, K, w_prefill, stream));
}

bitnet_status bitnet_ternary_linear_prefill(const bitnet_matrix* mats, int count,
                                            const int8_t* x_q, const float* x_scale, int64_t M,
                                            int64_t K, int y_dtype, hipStream_t stream) {
  if (M > 0 && (!x_scale || !x_q)) return BITNET_ERR_NULL;
  const bitnet_status st = check_group(mats, count, M, K, y_dtype);
  if (st != BITNET_OK) return st;
  if (K < 64 || (K % 64) != 0) return BITNET_ERR_SHAPE;
  if (x_scale && !aligned(x_scale, 4)) return BITNET_ERR_ALIGN;
  if (M > 0 && !aligned(x_q, 16)) return BITNET_ERR_ALIGN;
  for (int j = 0; j < count; ++j)
    if (M > 0 && mats[j].N > 0 && !aligned(mats[j].w_packed, 16)) return BITNET_ERR_ALIGN;
  if (M == 0) return BITNET_OK;
  bitnet::GemmArgs g{};
  for (int j = 0; j < count; ++j) {
    const bitnet_matrix& m = mats[j];
    if (m.N == 0) continue;
    g.wp[g.count] = m.w_packed;
    g.ws[g.count] = m.w_scale;
    g.y[g.count] = m.y;
    g.acc[g.count] = m.acc_out;
    g.n[g.count] = (int)m.N;
    if (++g.count == bitnet::kMaxGroup || j == count - 1) {
      g.xq = x_q;
      g.xs = x_scale;
      g.M = (int)M;
      g.K = (int)K;
      g.y_bf16 = y_dtype == BITNET_BF16 ? 1 : 0;
      g.layout = 1;
      if (bitnet::launch_gemm(g, stream) != hipSuccess) return BITNET_ERR_HIP;
      g = bitnet::GemmArgs{};
    }
  }
  if (g.count > 0) {      // the last matrices had N == 0 after a partial group
    g.xq = x_q;
    g.xs = x_scale;
    g.M = (int)M;
    g.K = (int)K;
    g.y_bf16 = y_dtype == BITNET_BF16 ? 1 : 0;
    g.layout = 1;
    if (bitnet::launch_gemm(g, stream) != hipSuccess) return BITNET_ERR_HIP;
  }
  return BITNET_OK;
}

bitnet_status bitnet_ternary_linear(const uint8_t* w_packed, const float* w_scale,
                                    const int8_t* x_q, const float* x_scale, int64_t M,
                                    int64_t N, int64_t K, void* y, int y_dtype, int32_t* acc_out,
                                    hipStream_t stream) {
  const bitnet_matrix m{w_packed, w_scale, N, y, acc_out};
  return bitnet_ternary_linear_multi(&m, 1, x_q, x_scale, M, K, y_dtype, stream);
}

bitnet_status bitnet_quant_linear_ex(const bitnet_matrix* mats, int count, const void* x,
                                     int x_dtype, const bitnet_act_prologue* pro, int64_t M,
                                     int64_t K, int8_t* x_q, float* x_scale, int y_dtype,
                                     hipStream_t stream) {
  if (M > 0 && (!x_scale || (K > 0 && (!x || !x_q)))) return BITNET_ERR_NULL;
  if (!valid_dtype(x_dtype)) return BITNET_ERR_DTYPE;
  bitnet_status st = check_group(mats, count, M, K, y_dtype);
  if (st != BITNET_OK) return st;
  if (!aligned(x, esize(x_dtype)) || (x_scale && !aligned(x_scale, 4))) return BITNET_ERR_ALIGN;
  st = check_prologue(pro, x_dtype, M, K);
  if (st != BITNET_OK) return st;
  return quant_linear(mats, count, x, x_dtype, act_prologue(pro), M, K, x_q, x_scale, y_dtype,
                      stream);
}

bitnet_status bitnet_quant_linear_multi(const bitnet_matrix* mats, int count, const void* x,
                                        int x_dtype, int64_t M, int64_t K, int8_t* x_q,
                                        float* x_scale, int y_dtype, hipStream_t stream) {
  return bitnet_quant_linear_ex(mats, count, x, x_dtype, nullptr, M, K, x_q, x_scale, y_dtype,
                                stream);
}

bitnet_status bitnet_quant_linear(const uint8_t* w_packed, const float* w_scale, const void* x,
                                  int x_dtype, int64_t M, int64_t N, int64_t K, int8_t* x_q,
                                  float* x_scale, void* y, int y_dtype, int32_t* acc_out,
                                  hipStream_t stream) {
  const bitnet_matrix m{w_packed, w_scale, N, y, acc_out};
  return bitnet_quant_linear_multi(&m, 1, x, x_dtype, M, K, x_q, x_scale, y_dtype, stream);
}

bitnet_status bitnet_prefill_tile(int64_t M, const int64_t* N, int count, int64_t K,
                                 int* tokens_per_tile, int* rows_per_tile,
                                 int64_t* first_launch_tokens, int64_t* first_launch_rows) {
  if (!N || !tokens_per_tile || !rows_per_tile || !first_launch_tokens || !first_launch_rows)
    return BITNET_ERR_NULL;
  if (M < 1 || M > kInt32Max || count < 1 || count > bitnet::kMaxGroup || K < 1)
    return BITNET_ERR_SHAPE;
  int n[bitnet::kMaxGroup] = {0, 0, 0, 0};
  for (int j = 0; j < count; ++j) {
    if (N[j] < 1 || N[j] > kInt32Max) return BITNET_ERR_SHAPE;
    n[j] = (int)N[j];
  }
  const bitnet::GemmPlan p = bitnet::gemm_plan(M, n, count, K, bitnet::device_cus());
  *tokens_per_tile = p.bm;
  *rows_per_tile = p.bn;
  *first_launch_tokens = p.first_tokens;
  *first_launch_rows = p.first_rows;
  return BITNET_OK;
}

size_t bitnet_chain_plan_bytes(int n_stages) {
  if (n_stages < 1) return 0;
  return bitnet::chain_plan_bytes(n_stages);
}

bitnet_status bitnet_chain_plan(const bitnet_chain_stage* stages, int n_stages, int64_t M,
                                void* plan, size_t plan_bytes, bitnet_chain* chain) {
  if (!stages || !plan || !chain) return BITNET_ERR_NULL;
  if (n_stages < 1 || M < 1 || M > bitnet::kChainMaxM) return BITNET_ERR_SHAPE;
  if (plan_bytes < bitnet_chain_plan_bytes(n_stages)) return BITNET_ERR_WORKSPACE;
  if (!aligned(plan, 256)) return BITNET_ERR_ALIGN;
  int kmax = 64;
  for (int s = 0; s < n_stages; ++s) {
    const bitnet_chain_stage& st = stages[s];
    if (!st.x || !st.x_q || !st.x_scale || !st.mats) return BITNET_ERR_NULL;
    if (!valid_dtype(st.x_dtype) || !valid_dtype(st.y_dtype)) return BITNET_ERR_DTYPE;
    if (st.count < 1 || st.count > bitnet::kMaxGroup || st.K < 64 || (st.K % 64) != 0 ||
        M * (st.K + 16) > 65536)
      return BITNET_ERR_SHAPE;
    if (!aligned(st.x, 16) || !aligned(st.x_q, 16) || !aligned(st.x_scale, 4))
      return BITNET_ERR_ALIGN;
    for (int j = 0; j < st.count; ++j) {
      const bitnet_matrix& m = st.mats[j];
      if (m.N < 1 || M * m.N >= ((int64_t)1 << 30)) return BITNET_ERR_SHAPE;
      if (!m.w_packed || !m.w_scale || !m.y) return BITNET_ERR_NULL;
      if (!aligned(m.w_packed, 16) || !aligned(m.w_scale, 4) || !aligned(m.y, esize(st.y_dtype)) ||
          (m.acc_out && !aligned(m.acc_out, 4)))
        return BITNET_ERR_ALIGN;
    }
    if (st.K > kmax) kmax = (int)st.K;
  }
  const int ring = 4;
  const int grid = bitnet::chain_grid((int)M, kmax, bitnet::kChainMaxTiles, ring);
  if (grid < 1) return BITNET_ERR_HIP;
  // host image of the plan: zeroed counters, then the stage table
  std::vector<char> host(bitnet_chain_plan_bytes(n_stages), 0);
  auto* table = reinterpret_cast<bitnet::ChainStage*>(host.data() + bitnet::kChainHeaderBytes);
  int tmax = 1;
  for (int s = 0; s < n_stages; ++s) {
    const bitnet_chain_stage& st = stages[s];
    bitnet::ChainStage d;
    memset(&d, 0, sizeof(d));
    d.x = st.x;
    d.xq_out = st.x_q;
    d.xs_out = st.x_scale;
    int total = 0;
    for (int j = 0; j < bitnet::kMaxGroup; ++j) {
      d.tc0[j] = total;
      if (j < st.count) {
        d.wp[j] = st.mats[j].w_packed;
        d.ws[j] = st.mats[j].w_scale;
        d.y[j] = st.mats[j].y;
        d.acc[j] = st.mats[j].acc_out;
        d.n[j] = (int)st.mats[j].N;
        total += (int)((st.mats[j].N + 15) / 16);
      }
    }
    d.tc0[bitnet::kMaxGroup] = total;
    // the tile list is spread evenly: at most ceil(total / grid) tiles per workgroup
    const int T = (total + grid - 1) / grid;
    if (T > bitnet::kChainMaxTiles) return BITNET_ERR_SHAPE;
    if (T > tmax) tmax = T;
    d.K = (int)st.K;
    d.count = st.count;
    d.flags = (st.x_dtype == BITNET_BF16 ? 1 : 0) | (st.y_dtype == BITNET_BF16 ? 2 : 0);
    table[s] = d;
  }
  if (hipMemcpy(plan, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess)
    return BITNET_ERR_HIP;
  chain->plan = plan;
  chain->n_stages = n_stages;
  chain->M = (int)M;
  chain->grid = grid;
  chain->kmax = kmax;
  chain->tmax = tmax;
  chain->ring = ring;
  return BITNET_OK;
}

bitnet_status bitnet_chain_run(const bitnet_chain* chain, hipStream_t stream) {
  if (!chain || !chain->plan) return BITNET_ERR_NULL;
  if (chain->n_stages < 1 || chain->M < 1 || chain->M > bitnet::kChainMaxM || chain->grid < 1 ||
      chain->kmax < 64 || chain->tmax < 1 || chain->tmax > bitnet::kChainMaxTiles ||
      (chain->ring != 4 && chain->ring != 8 && chain->ring != 16))
    return BITNET_ERR_SHAPE;
  return from_hip(bitnet::launch_chain(chain->plan, chain->n_stages, chain->M, chain->grid,
                                       chain->kmax, chain->tmax, chain->ring, stream));
}

bitnet_status bitnet_chain_error(const bitnet_chain* chain, int* error) {
  if (!chain || !chain->plan || !error) return BITNET_ERR_NULL;
  unsigned word = 0;
  const char* at = static_cast<const char*>(chain->plan) + bitnet::kChainErrorAt;
  if (hipMemcpy(&word, at, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return BITNET_ERR_HIP;
  *error = (int)word;
  return BITNET_OK;
}

}  // extern "C"
