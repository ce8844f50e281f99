// Adapter merge for re-quantization ("074｜QLoRA：把大模型放进显存，再用小适配器
// 改变它" §五, §六: merging an adapter into the weights and quantizing again can
// change the outputs; the weimeta QLoRA glossary FAQ: merge at 16-bit or
// better, never on the 4-bit codes):
//
//     W_out[n][k] = fl32( ŵ[n][k] + fl32(s · Δ[k][n]) ),   Δ = A·B,
//
// with Δ accumulated by fp32 fused multiply-adds in increasing j (each
// bf16 × bf16 product is exact in fp32, so every step rounds once) and ŵ the
// fp32 dequantized weight fl32(V[k]·fl32(q8·step)).  The caller quantizes
// W_out with the ordinary quantizer to obtain the merged 4-bit layer.
//
// A workgroup computes a 128 (n) × 128 (k) tile; each thread an 8 × 8 block
// of it, so one pass of four rank steps reads 16 float4 from LDS for 256
// FMAs.  Rank chunks of 64 of A [k][j] and B (transposed to [n][j]) are
// staged in LDS as fp32, with float4 column index XOR-swizzled by the
// 8-row group so that the 16 distinct rows a wave reads fall in distinct
// banks.  The epilogue dequantizes the thread's 8 consecutive weights of
// each of its rows from one code word and one scale, adds, and stores.
#include "kernels.h"

namespace qlora {

namespace {
constexpr int kMgN = 128, kMgK = 128, kMgJ = 64;

__device__ __forceinline__ int mg_swz(int row, int q) { return q ^ ((row >> 3) & 15); }
}  // namespace

__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ codes,
                                               const uint8_t* __restrict__ scale8,
                                               const float* __restrict__ scale2, int64_t o,
                                               int64_t d, const uint16_t* __restrict__ A,
                                               const uint16_t* __restrict__ B, int r, float s,
                                               float* __restrict__ W_out, Codebook cb) {
#pragma clang fp contract(off)
  __shared__ __attribute__((aligned(16))) float4 sA[kMgK * kMgJ / 4];   // [k][j], swizzled
  __shared__ __attribute__((aligned(16))) float4 sB[kMgN * kMgJ / 4];   // [n][j], swizzled
  __shared__ float s_v[16];
  const int t = threadIdx.x, tn = t >> 4, tk = t & 15;
  const int64_t n0 = (int64_t)blockIdx.y * kMgN, k0 = (int64_t)blockIdx.x * kMgK;
  if (t < 16) s_v[t] = cb.v[t];

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.0f;

  for (int j0 = 0; j0 < r; j0 += kMgJ) {
    const int jn = r - j0 < kMgJ ? r - j0 : kMgJ;          // a multiple of 8
    __syncthreads();                                        // the previous chunk is consumed
    // A[k0 + row][j0 + 8c8 .. +8] -> sA (1024 pieces of 8, 4 per thread)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = u * 256 + t, row = pc >> 3, c8 = pc & 7;
      const int64_t k = k0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k < d && 8 * c8 < jn) v = *reinterpret_cast<const uint4*>(A + k * r + j0 + 8 * c8);
      const float4 lo = make_float4(bf16_to_f32((uint16_t)(v.x & 0xFFFF)), bf16_to_f32((uint16_t)(v.x >> 16)),
                                    bf16_to_f32((uint16_t)(v.y & 0xFFFF)), bf16_to_f32((uint16_t)(v.y >> 16)));
      const float4 hi = make_float4(bf16_to_f32((uint16_t)(v.z & 0xFFFF)), bf16_to_f32((uint16_t)(v.z >> 16)),
                                    bf16_to_f32((uint16_t)(v.w & 0xFFFF)), bf16_to_f32((uint16_t)(v.w >> 16)));
      sA[row * 16 + mg_swz(row, 2 * c8)] = lo;
      sA[row * 16 + mg_swz(row, 2 * c8 + 1)] = hi;
    }
    // B[j0 + jj][n0 + 8c16 .. +8] -> sB[n][jj] (1024 pieces of 8, 4 per thread)
    float* sBf = reinterpret_cast<float*>(sB);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pc = u * 256 + t, jj = pc >> 4, c16 = pc & 15;
      const int64_t n = n0 + 8 * c16;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (jj < jn && n < o) v = *reinterpret_cast<const uint4*>(B + (int64_t)(j0 + jj) * o + n);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = 8 * c16 + e;
        const uint16_t h = (uint16_t)(e & 1 ? w[e >> 1] >> 16 : w[e >> 1] & 0xFFFF);
        sBf[(row * 16 + mg_swz(row, jj >> 2)) * 4 + (jj & 3)] = bf16_to_f32(h);
      }
    }
    __syncthreads();
    for (int jj = 0; jj < jn; jj += 4) {
      float4 a[8], b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ka = tk * 8 + i, nb = tn * 8 + i;
        a[i] = sA[ka * 16 + mg_swz(ka, jj >> 2)];
        b[i] = sB[nb * 16 + mg_swz(nb, jj >> 2)];
      }
      // increasing j: component x, y, z, w of the four-step group
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(a[c].x, b[i].x, acc[i][c]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(a[c].y, b[i].y, acc[i][c]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(a[c].z, b[i].z, acc[i][c]);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = __builtin_fmaf(a[c].w, b[i].w, acc[i][c]);
    }
  }
  __syncthreads();                                          // s_v written by the first threads

  // ---- ŵ + fl32(s·Δ) for the thread's 8 rows × 8 consecutive columns
  const int64_t k = k0 + tk * 8;
  if (k >= d) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = n0 + tn * 8 + i;
    if (n >= o) continue;
    const int64_t e = n * d + k;                            // 8 weights in one code word, one block
    const uint32_t word = reinterpret_cast<const uint32_t*>(codes)[e >> 3];
    const int64_t blk = e >> 6;
    const float chat = (float)scale8[blk] * scale2[blk >> 8];
    float out[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t code = (word >> (8 * (c & 3) + 4 * (c >> 2))) & 15u;
      const float w = s_v[code] * chat;
      out[c] = w + s * acc[i][c];
    }
    float4* dst = reinterpret_cast<float4*>(W_out + e);
    dst[0] = make_float4(out[0], out[1], out[2], out[3]);
    dst[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

hipError_t launch_merge(const uint8_t* codes, const uint8_t* scale8, const float* scale2,
                        int64_t o, int64_t d, const uint16_t* A, const uint16_t* B, int r, float s,
                        float* W_out, const Codebook& cb, hipStream_t st) {
  if (o == 0 || d == 0) return hipSuccess;
  const dim3 grid((unsigned)((d + kMgK - 1) / kMgK), (unsigned)((o + kMgN - 1) / kMgN));
  launch(k_merge, grid, dim3(256), 0, st, codes, scale8, scale2, o, d, A, B, r, s,
                     W_out, cb);
  return hipGetLastError();
}

}  // namespace qlora
