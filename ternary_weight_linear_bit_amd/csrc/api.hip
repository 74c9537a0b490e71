// C ABI of libbitnet_mi355x: argument validation and kernel dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues nothing.
#include "bitnet_mi355x.h"
#include "bitnet_internal.h"

namespace {

constexpr size_t kWqWorkspaceBytes = 4096;
constexpr int64_t kInt32Max = 2147483647;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
bool valid_dtype(int d) { return d == BITNET_F32 || d == BITNET_BF16; }
uintptr_t esize(int d) { return d == BITNET_BF16 ? 2 : 4; }

bitnet_status from_hip(hipError_t e) { return e == hipSuccess ? BITNET_OK : BITNET_ERR_HIP; }

// Fast kernels read 16-byte vectors of packed weights and int8 activations.
bool fast_layout(const void* w_packed, const void* x_q, int64_t K) {
  return K >= 64 && (K % 64) == 0 && aligned(w_packed, 16) && aligned(x_q, 16);
}

bitnet_status check_linear_args(const uint8_t* w_packed, const float* w_scale, const float* x_scale,
                                int64_t M, int64_t N, int64_t K, void* y, int y_dtype,
                                int32_t* acc_out) {
  if (!w_scale || !x_scale || !y || (K > 0 && !w_packed)) return BITNET_ERR_NULL;
  if (!valid_dtype(y_dtype)) return BITNET_ERR_DTYPE;
  if (M < 0 || N < 0 || K < 0 || (K % 4) != 0 || K > BITNET_MAX_K || M > kInt32Max ||
      N > kInt32Max)
    return BITNET_ERR_SHAPE;
  if (!aligned(y, esize(y_dtype)) || !aligned(w_scale, 4) || !aligned(x_scale, 4) ||
      (acc_out && !aligned(acc_out, 4)))
    return BITNET_ERR_ALIGN;
  return BITNET_OK;
}

bitnet_status run_linear(const uint8_t* w_packed, const float* w_scale, const int8_t* x_q,
                         const float* x_scale, int64_t M, int64_t N, int64_t K, void* y,
                         int y_dtype, int32_t* acc_out, const bitnet::Launch& l) {
  const bool yb = y_dtype == BITNET_BF16;
  if (fast_layout(w_packed, x_q, K)) {
    if (bitnet::gemv_fits(M, K))
      return from_hip(bitnet::launch_gemv(w_packed, w_scale, x_q, x_scale, nullptr, 0, nullptr,
                                          nullptr, (int)M, (int)N, (int)K, y, yb, acc_out, l));
    return from_hip(bitnet::launch_gemm(w_packed, w_scale, x_q, x_scale, (int)M, (int)N, (int)K, y,
                                        yb, acc_out, l));
  }
  return from_hip(bitnet::launch_generic_linear(w_packed, w_scale, x_q, x_scale, M, N, K, y, yb,
                                                acc_out, l));
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
  return kWqWorkspaceBytes;
}

bitnet_status bitnet_quantize_weights(const void* w, int w_dtype, int64_t N, int64_t K,
                                      uint8_t* w_packed, float* w_scale, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  if (!w || !w_packed || !w_scale) return BITNET_ERR_NULL;
  if (!valid_dtype(w_dtype)) return BITNET_ERR_DTYPE;
  if (N < 1 || K < 4 || (K % 4) != 0 || N >= BITNET_MAX_WEIGHTS / K) return BITNET_ERR_SHAPE;
  if (!workspace || workspace_bytes < kWqWorkspaceBytes) return BITNET_ERR_WORKSPACE;
  if (!aligned(w, esize(w_dtype)) || !aligned(w_scale, 4) || !aligned(workspace, 8))
    return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_wq(w, w_dtype == BITNET_BF16, N * K, w_packed, w_scale, workspace,
                                    stream));
}

bitnet_status bitnet_quantize_acts(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* x_q,
                                   float* x_scale, hipStream_t stream) {
  if (!valid_dtype(x_dtype)) return BITNET_ERR_DTYPE;
  if (M < 0 || K < 0 || M > kInt32Max) return BITNET_ERR_SHAPE;
  if (M == 0) return BITNET_OK;
  if (!x_scale || (K > 0 && (!x || !x_q))) return BITNET_ERR_NULL;
  if (!aligned(x, esize(x_dtype)) || !aligned(x_scale, 4)) return BITNET_ERR_ALIGN;
  return from_hip(bitnet::launch_aq(x, x_dtype == BITNET_BF16, M, K, x_q, x_scale, stream));
}

bitnet_status bitnet_ternary_linear(const uint8_t* w_packed, const float* w_scale,
                                    const int8_t* x_q, const float* x_scale, int64_t M,
                                    int64_t N, int64_t K, void* y, int y_dtype, int32_t* acc_out,
                                    hipStream_t stream) {
  if (K > 0 && M > 0 && !x_q) return BITNET_ERR_NULL;
  const bitnet_status st =
      check_linear_args(w_packed, w_scale, x_scale, M, N, K, y, y_dtype, acc_out);
  if (st != BITNET_OK) return st;
  if (M == 0 || N == 0) return BITNET_OK;
  return run_linear(w_packed, w_scale, x_q, x_scale, M, N, K, y, y_dtype, acc_out,
                    bitnet::Launch{stream, nullptr, nullptr});
}

bitnet_status bitnet_ternary_linear_timed(const uint8_t* w_packed, const float* w_scale,
                                          const int8_t* x_q, const float* x_scale, int64_t M,
                                          int64_t N, int64_t K, void* y, int y_dtype,
                                          int32_t* acc_out, hipEvent_t start, hipEvent_t stop,
                                          hipStream_t stream) {
  if (K > 0 && M > 0 && !x_q) return BITNET_ERR_NULL;
  const bitnet_status st =
      check_linear_args(w_packed, w_scale, x_scale, M, N, K, y, y_dtype, acc_out);
  if (st != BITNET_OK) return st;
  if (M == 0 || N == 0) return BITNET_OK;
  return run_linear(w_packed, w_scale, x_q, x_scale, M, N, K, y, y_dtype, acc_out,
                    bitnet::Launch{stream, start, stop});
}

bitnet_status bitnet_quant_linear(const uint8_t* w_packed, const float* w_scale, const void* x,
                                  int x_dtype, int64_t M, int64_t N, int64_t K, int8_t* x_q,
                                  float* x_scale, void* y, int y_dtype, int32_t* acc_out,
                                  hipStream_t stream) {
  if (K > 0 && M > 0 && (!x || !x_q)) return BITNET_ERR_NULL;
  if (!valid_dtype(x_dtype)) return BITNET_ERR_DTYPE;
  const bitnet_status st =
      check_linear_args(w_packed, w_scale, x_scale, M, N, K, y, y_dtype, acc_out);
  if (st != BITNET_OK) return st;
  if (!aligned(x, esize(x_dtype))) return BITNET_ERR_ALIGN;
  if (M == 0) return BITNET_OK;
  const bitnet::Launch l{stream, nullptr, nullptr};
  if (N > 0 && fast_layout(w_packed, x_q, K) && aligned(x, 16) && bitnet::gemv_fused_fits(M, K))
    return from_hip(bitnet::launch_gemv(w_packed, w_scale, nullptr, nullptr, x,
                                        x_dtype == BITNET_BF16 ? 1 : 0, x_q, x_scale, (int)M,
                                        (int)N, (int)K, y, y_dtype == BITNET_BF16, acc_out, l));
  const hipError_t e = bitnet::launch_aq(x, x_dtype == BITNET_BF16, M, K, x_q, x_scale, stream);
  if (e != hipSuccess) return BITNET_ERR_HIP;
  if (N == 0) return BITNET_OK;
  return run_linear(w_packed, w_scale, x_q, x_scale, M, N, K, y, y_dtype, acc_out, l);
}

}  // extern "C"
