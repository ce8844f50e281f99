// Small elementwise kernels of the adapter path: the fixed-order sum of
// split planes and zero fill.
#include "kernels.h"

namespace qlora {

// Sum of split planes over a contiguous region: out_f32 = Σ_z part[z];
// out_bf16 = bf16(scale·Σ_z part[z]).  Four elements per thread, fixed
// summation order.  Workgroups [0, blocks_a) serve job a, the rest job b.
__global__ __launch_bounds__(256) void k_reduce_planes(ReduceJob a, ReduceJob b, int blocks_a) {
  const bool first = (int)blockIdx.x < blocks_a;
  const ReduceJob& jo = first ? a : b;
  const int64_t blk = first ? blockIdx.x : blockIdx.x - blocks_a;
  const int64_t nblk = first ? blocks_a : gridDim.x - blocks_a;
  const int64_t n4 = jo.count / 4;
  for (int64_t i = blk * blockDim.x + threadIdx.x; i < n4; i += nblk * blockDim.x)
    reduce_planes_quad(jo, i);
}

__global__ __launch_bounds__(256) void k_fill_zero_bf16(uint16_t* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_reduce_planes(const ReduceJob& a, const ReduceJob& b, hipStream_t st) {
  auto blocks = [](int64_t count) -> int {
    const int64_t n = (count / 4 + 255) / 256;
    return (int)(n > 4096 ? 4096 : n);
  };
  const int ba = blocks(a.count), bb = blocks(b.count);
  if (ba + bb == 0) return hipSuccess;
  launch(k_reduce_planes, dim3((unsigned)(ba + bb)), dim3(256), 0, st, a, b, ba);
  return hipGetLastError();
}

hipError_t launch_fill_zero_bf16(uint16_t* y, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  launch(k_fill_zero_bf16, dim3((unsigned)blocks), dim3(256), 0, st, y, n);
  return hipGetLastError();
}

}  // namespace qlora
