// Streaming-read probe: the achievable HBM read rate of the device, measured
// beside the nominal peak.  Not part of the decode path.
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "ffd_device.h"
#include "ffd_launch.h"

namespace ffd {

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;  // 16-byte loads in flight per thread per iteration

// Work-group g reads the 16-byte words g*1024 + k*256 + t (k < 4) of every
// grid-stride step, so each load instruction of a wave covers 1 KB contiguous
// (whole lines, non-temporal hint); every work-group writes the XOR of the
// 32-bit words it read to sink[g] (the XOR over all of sink equals that of the
// whole buffer).
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                                    uint32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  const size_t step = (size_t)gridDim.x * kProbeThreads * kProbeUnroll;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * kProbeThreads * kProbeUnroll; base < n16; base += step) {
    uint4 v[kProbeUnroll];
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) {
      const size_t i = base + (size_t)k * kProbeThreads + tid;
      v[k] = i < n16 ? load_b128_nt(src + i) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kProbeUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((tid & 63) == 0) part[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, void* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadGroups), dim3(kProbeThreads), 0, s,
                     static_cast<const uint4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace ffd
