// Bench-only diagnostic, built into its own library (libbitnet_bench_probe.so)
// and loaded only by bench.py: the int8 matrix-core rate of this chip, the
// ceiling against which the prefill kernel is read.  Not part of the method and
// not part of the public ABI.
//
// Each wave runs v_mfma_i32_32x32x32_i8 on four accumulator chains with its
// operands cycling through eight register sets.  The operands come from memory
// once: all-zero ones show the issue rate; random int8 activations against random
// ternary codes {0, 1, 2} (the prefill kernel's operands) show the rate the chip
// sustains while switching real data (its power management lowers the clock).
// No memory traffic inside the loop.  Built with the accumulators in arch VGPRs
// (-amdgpu-mfma-vgpr-form): in AGPRs, two waves per SIMD of this loop ran at
// 1207 instead of 2046 int8 ops per clock and SIMD on gfx950.  The kernel also
// reads the shader clock (s_memtime) against the 100 MHz constant clock
// (s_memrealtime) per wave, so the rate can be read per clock as well.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe(const v4i* __restrict__ ops, int iters,
                                                 v16i* __restrict__ out,
                                                 unsigned long long* __restrict__ clk) {
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
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s], b[(s + c) & 7], acc[c], 0, 0, 0);
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  out[t] = acc[0] + acc[1] + acc[2] + acc[3];
  if (clk != nullptr && (threadIdx.x & 63) == 0) {
    clk[2 * (t >> 6)] = c1 - c0;        // shader clocks of the loop
    clk[2 * (t >> 6) + 1] = r1 - r0;    // 100 MHz ticks of the loop
  }
}

}  // namespace

// Launches `workgroups` x 256 threads; each wave runs `iters` x 32
// v_mfma_i32_32x32x32_i8 (65536 int8 ops each) on operands read once from `ops`
// (workgroups * 65536 bytes, 16-byte aligned: per thread 8 A then 8 B operand
// vectors of 16 bytes) and writes 64 bytes per thread to `out`; with `clk`
// (workgroups * 64 bytes, or NULL) each wave also writes the shader clocks and
// the 100 MHz ticks its loop took (two uint64).  Returns 0, 2 for bad sizes, 4
// for misalignment, 6 for a failed launch.  The caller times it:
// rate = workgroups * 4 * iters * 32 * 65536 / time.
extern "C" int bitnet_bench_probe_mfma_i8(const void* ops, int workgroups, int iters, void* out,
                                          void* clk, hipStream_t s) {
  if (!ops || !out) return 1;
  if (workgroups < 1 || iters < 1) return 2;
  if (((uintptr_t)ops & 15) || ((uintptr_t)out & 15) || ((uintptr_t)clk & 7)) return 4;
  hipLaunchKernelGGL(mfma_probe, dim3((unsigned)workgroups), dim3(256), 0, s,
                     static_cast<const v4i*>(ops), iters, static_cast<v16i*>(out),
                     static_cast<unsigned long long*>(clk));
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
