// Diagnostic: the int8 matrix-core rate of this chip, as the ceiling against
// which the prefill kernel is read (not part of the method).
//
// Each wave runs v_mfma_i32_32x32x32_i8 on four accumulator chains with its
// operands cycling through eight register sets.  The operands come from memory
// once: all-zero ones show the issue rate; random int8 activations against random
// ternary codes {0, 1, 2} (the prefill kernel's operands) show the rate the chip
// sustains while switching real data (its power management lowers the clock).
// No memory traffic inside the loop.
#include "bitnet_internal.h"

namespace bitnet {
namespace {

typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe(const v4i* __restrict__ ops, int iters,
                                                 v16i* __restrict__ out) {
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  v4i a[8], b[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a[s] = ops[t * 16 + s];
    b[s] = ops[t * 16 + 8 + s];
  }
  v16i acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (v16i){};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s], b[(s + c) & 7], acc[c], 0, 0, 0);
    }
  }
  out[t] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

hipError_t launch_mfma_probe(const void* ops, int workgroups, int iters, void* out,
                             hipStream_t s) {
  hipLaunchKernelGGL(mfma_probe, dim3((unsigned)workgroups), dim3(256), 0, s,
                     static_cast<const v4i*>(ops), iters, static_cast<v16i*>(out));
  return hipGetLastError();
}

}  // namespace bitnet
