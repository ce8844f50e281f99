// Small elementwise kernels of the adapter path: the fixed-order sum of
// split planes and zero fill.
#include "kernels.h"

namespace qlora {

// Sum of split-K planes over a contiguous [rows][cols] region:
// out_f32 = Σ_z part[z]; out_bf16 = bf16(scale·Σ_z part[z]).  Four
// elements per thread, fixed summation order.
__global__ __launch_bounds__(256) void k_reduce_planes(const float* __restrict__ part, int splits,
                                                       int64_t plane, int64_t count,
                                                       float* __restrict__ out_f32,
                                                       uint16_t* __restrict__ out_bf16, float scale) {
  const int64_t n4 = count / 4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * blockDim.x) {
    // planes summed in order, four loads in flight at a time
    float4 s = reinterpret_cast<const float4*>(part)[i];
    int z = 1;
    for (; z + 4 <= splits; z += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = reinterpret_cast<const float4*>(part + (int64_t)(z + u) * plane)[i];
#pragma unroll
      for (int u = 0; u < 4; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
    }
    for (; z < splits; ++z) {
      const float4 v = reinterpret_cast<const float4*>(part + (int64_t)z * plane)[i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (out_f32) reinterpret_cast<float4*>(out_f32)[i] = s;
    if (out_bf16) {
      uint2 o;
      o.x = pack_bf16x2(scale * s.x, scale * s.y);
      o.y = pack_bf16x2(scale * s.z, scale * s.w);
      reinterpret_cast<uint2*>(out_bf16)[i] = o;
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_zero_bf16(uint16_t* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

// fp32 -> bf16(scale·x), elementwise.
// ------------------------------------------------------------------ launchers
hipError_t launch_reduce_planes(const float* part, int splits, int64_t plane, int64_t count,
                                float* out_f32, uint16_t* out_bf16, float scale, hipStream_t st) {
  if (count == 0) return hipSuccess;
  int64_t blocks = (count / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_reduce_planes, dim3((unsigned)blocks), dim3(256), 0, st, part, splits,
                     plane, count, out_f32, out_bf16, scale);
  return hipGetLastError();
}

hipError_t launch_fill_zero_bf16(uint16_t* y, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_fill_zero_bf16, dim3((unsigned)blocks), dim3(256), 0, st, y, n);
  return hipGetLastError();
}

}  // namespace qlora
