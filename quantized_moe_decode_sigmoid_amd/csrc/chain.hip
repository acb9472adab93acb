// Chaining of consecutive layers in the stack workload (not part of the MoE
// layer): the next layer's input is bf16(rmsnorm(x + out)) without a weight,
// eps 1e-6 -- the residual add and normalisation that stand in for the rest of
// a decoder block between two MoE layers.  One kernel instead of the four
// elementwise / reduction kernels a framework would launch for it.
//
// One workgroup per token row: h = fp32(x) + out (one rounding, as the
// framework's widening + add), the mean of h^2 over the row in fp32 (wavefront
// shuffles, then the 4 wavefront sums in order), y = bf16(h * rsqrt(mean + eps))
// rounded to nearest even.
#include "device.h"
#include "launch.h"

namespace qmoe {

constexpr int kChainThreads = 256;

// y may alias x: every element is read and then written by the same thread.
__global__ __launch_bounds__(kChainThreads) void k_residual_rmsnorm(const float* __restrict__ out, const uint16_t* x,
                                                                    int H, float eps, uint16_t* y) {
  __shared__ float s_part[kChainThreads / 64];
  const int t = blockIdx.x;
  const float* o = out + (size_t)t * H;
  const uint16_t* xr = x + (size_t)t * H;
  uint16_t* yr = y + (size_t)t * H;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < H; i += kChainThreads) {
    const float h = bf16_bits_to_f32(xr[i]) + o[i];
    ss = __builtin_fmaf(h, h, ss);
  }
  ss = wave_xor_sum(ss);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kChainThreads / 64; w++) tot += s_part[w];
  const float r = 1.0f / __builtin_sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += kChainThreads) {
    const float h = bf16_bits_to_f32(xr[i]) + o[i];
    yr[i] = f32_to_bf16_rne(h * r);
  }
}

hipError_t launch_residual_rmsnorm(const float* out, const uint16_t* x, int T, int H, float eps, uint16_t* y,
                                   hipStream_t stream) {
  if (T == 0) return hipSuccess;
  clear_last_error();
  hipLaunchKernelGGL(k_residual_rmsnorm, dim3(T), dim3(kChainThreads), 0, stream, out, x, H, eps, y);
  return hipGetLastError();
}

}  // namespace qmoe
