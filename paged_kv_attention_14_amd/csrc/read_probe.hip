// Streaming-read probe for gfx950: the achievable read bandwidth that the
// decode kernel's HBM bound is compared against on the same box.
//
// A measurement aid, built into its own library (libpd_probe.so), not part
// of the decode ABI. Every lane reads 16 contiguous bytes per load, a wave
// 1 KiB, in a grid-stride loop over the buffer with a chosen number of loads
// in flight per lane; the loaded words are folded into one value that is stored only
// if it equals a constant the data never produces in practice, so the loads
// cannot be removed while the probe writes (almost) nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Each round a workgroup reads one contiguous chunk of U * 256 16-byte
// elements (U loads per lane, issued before any is used); the chunks of one
// round are adjacent across the grid, so the reads in flight cover one
// contiguous window of the buffer.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                          int64_t n16, uint32_t* sink) {
  const int64_t chunk = (int64_t)U * blockDim.x;
  const int64_t step = chunk * gridDim.x;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * chunk; base < n16; base += step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = base + u * (int64_t)blockDim.x + threadIdx.x;
      v[u] = (j < n16) ? buf[j] : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16, buffer 16-byte aligned) from device memory
// `buf` on `stream` with `grid` workgroups of 256 threads (<= 0: 4096) and
// `unroll` loads per lane per round (1, 2, 4 or 8). `sink` must hold `grid`
// uint32 words (device memory). Returns a hipError_t code.
int pd_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int grid, int unroll,
                         hipStream_t stream) {
  if (!buf || !sink || bytes < 0 || (bytes & 15) || (reinterpret_cast<uintptr_t>(buf) & 15))
    return (int)hipErrorInvalidValue;
  if (grid <= 0) grid = 4096;
  const u32x4* b = static_cast<const u32x4*>(buf);
  const int64_t n16 = bytes / 16;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_read_kernel<1>, dim3(grid), dim3(256), 0, stream, b, n16, sink); break;
    case 2: hipLaunchKernelGGL(stream_read_kernel<2>, dim3(grid), dim3(256), 0, stream, b, n16, sink); break;
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, dim3(grid), dim3(256), 0, stream, b, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, dim3(grid), dim3(256), 0, stream, b, n16, sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // extern "C"
