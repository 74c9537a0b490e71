// Bench-only diagnostics, built into the probe library (libbitnet_bench_probe.so)
// and loaded only by bench.py: the HBM read rate of this chip for two access
// patterns, and the cost of a dependent launch.  The rates against which the
// decode kernel is read; not part of the method and not part of the public ABI.
//
// Pattern 0 streams a buffer with 16-byte loads, consecutive lanes on
// consecutive 16-byte units (a wave reads 1 KiB contiguous), four loads in flight
// per lane.  Pattern 1 reads it as a row-major matrix of 16-row tiles the way the
// decode kernel does: one wave load covers 16 rows x 64 bytes (lane r + 16 g
// reads bytes 16 g .. 16 g + 15 of a 64-byte super-chunk of row r), wave w of a
// workgroup takes super-chunks w, w + 4, ... of each tile, four loads in flight.
// Every lane folds what it read into one 16-byte value that it stores, so no load
// is dead code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint4 fold(uint4 a, uint4 b) {
  return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w);
}

__global__ __launch_bounds__(256) void read_stream(const uint4* __restrict__ buf, uint64_t units,
                                                   uint4* __restrict__ out) {
  const uint64_t threads = (uint64_t)gridDim.x * 256u;
  uint64_t u = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, a2 = a0, a3 = a0;
  for (; u + 3 * threads < units; u += 4 * threads) {
    a0 = fold(a0, buf[u]);
    a1 = fold(a1, buf[u + threads]);
    a2 = fold(a2, buf[u + 2 * threads]);
    a3 = fold(a3, buf[u + 3 * threads]);
  }
  for (; u < units; u += threads) a0 = fold(a0, buf[u]);
  out[(uint64_t)blockIdx.x * 256u + threadIdx.x] = fold(fold(a0, a1), fold(a2, a3));
}

// rowb = bytes per row (a multiple of 256); tiles = rows / 16
__global__ __launch_bounds__(256) void read_tiles(const uint8_t* __restrict__ buf, uint32_t rowb,
                                                  uint32_t tiles, uint4* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const uint32_t chunks = rowb >> 6;       // 64-byte super-chunks per row, a multiple of 4
  uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, a2 = a0, a3 = a0;
  for (uint32_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const uint8_t* row = buf + ((uint64_t)t * 16u + (uint64_t)r) * rowb + 16u * (uint32_t)g;
    uint32_t c = (uint32_t)wave;
    for (; c + 12 < chunks; c += 16) {
      a0 = fold(a0, *reinterpret_cast<const uint4*>(row + 64u * c));
      a1 = fold(a1, *reinterpret_cast<const uint4*>(row + 64u * (c + 4)));
      a2 = fold(a2, *reinterpret_cast<const uint4*>(row + 64u * (c + 8)));
      a3 = fold(a3, *reinterpret_cast<const uint4*>(row + 64u * (c + 12)));
    }
    for (; c < chunks; c += 4) a0 = fold(a0, *reinterpret_cast<const uint4*>(row + 64u * c));
  }
  out[(uint64_t)blockIdx.x * 256u + threadIdx.x] = fold(fold(a0, a1), fold(a2, a3));
}

__global__ void empty_kernel() {}

}  // namespace

// Reads `bytes` of `buf` (16-byte aligned) once with `workgroups` x 256 threads
// in pattern 0 (stream) or 1 (16-row tiles of `rowb` bytes per row: rowb a
// multiple of 256, bytes a multiple of 16 * rowb) and writes 16 bytes per thread
// to `out` (workgroups * 4096 bytes).  Returns 0, 1 for null pointers, 2 for bad
// sizes, 4 for misalignment, 6 for a failed launch.
extern "C" int bitnet_bench_probe_read(const void* buf, uint64_t bytes, int pattern, int rowb,
                                       int workgroups, void* out, hipStream_t s) {
  if (!buf || !out) return 1;
  if (workgroups < 1 || bytes == 0 || (bytes & 15u)) return 2;
  if (((uintptr_t)buf & 15) || ((uintptr_t)out & 15)) return 4;
  if (pattern == 0) {
    hipLaunchKernelGGL(read_stream, dim3((unsigned)workgroups), dim3(256), 0, s,
                       static_cast<const uint4*>(buf), bytes >> 4, static_cast<uint4*>(out));
  } else if (pattern == 1) {
    if (rowb < 256 || (rowb & 255) || bytes % (16ull * (uint64_t)rowb) != 0 ||
        bytes / (16ull * (uint64_t)rowb) >= (1ull << 32))
      return 2;
    hipLaunchKernelGGL(read_tiles, dim3((unsigned)workgroups), dim3(256), 0, s,
                       static_cast<const uint8_t*>(buf), (uint32_t)rowb,
                       (uint32_t)(bytes / (16ull * (uint64_t)rowb)), static_cast<uint4*>(out));
  } else {
    return 2;
  }
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

// An empty kernel of `workgroups` x 256 threads (the cost of a launch).
extern "C" int bitnet_bench_probe_empty(int workgroups, hipStream_t s) {
  if (workgroups < 1) return 2;
  hipLaunchKernelGGL(empty_kernel, dim3((unsigned)workgroups), dim3(256), 0, s);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}
