// Streaming read of a device buffer: the box's own HBM read ceiling, measured
// with a kernel of known traffic so that a kernel's achieved bandwidth can be
// reported as a fraction of what this GPU streams as well as of the vendor
// peak.  Not part of the layer.
//
// Every byte is read exactly once with 16-byte non-temporal vector loads,
// eight per lane in flight per step of a grid-stride walk over 32 workgroups
// per CU (the fastest of the plain / non-temporal, 4 / 8 loads, 4-32
// workgroups per CU forms measured here); nothing is written unless the XOR
// of a lane's words equals a fixed pattern (so the loads cannot be dropped
// and the traffic is reads only).
#include "device.h"
#include "launch.h"

namespace qmoe {

constexpr int kStreamThreads = 256;
constexpr int kStreamBlocks = 8192;  // 32 workgroups of 4 wavefronts per CU
constexpr int kStreamUnroll = 8;

__global__ __launch_bounds__(kStreamThreads) void k_stream_read(const u32x4* __restrict__ src, int64_t n16,
                                                                uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; u++) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; u++) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (v == 0x9e3779b9u) sink[0] = v;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_stream_read, dim3(kStreamBlocks), dim3(kStreamThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace qmoe
