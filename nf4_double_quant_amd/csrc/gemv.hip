// Few-token forward (M <= 16): fused NF4 dequant-GEMV with the adapter term
// in the epilogue,  Y = X·Ŵ + s·(X·A)·B  ("074｜QLoRA：把大模型放进显存，再用
// 小适配器改变它" §一 for the layer, §三 for dequantizing the needed weights
// to BF16 on demand).
//
// The weight stream is the whole cost (0.516 byte per weight at 4.127 bits),
// so the kernel reads every code byte once, coalesced, and never writes a
// dequantized weight anywhere:
//  * a workgroup owns 16 output rows n; its waves split the reduction d;
//  * lane l works on row n0 + l%16 and, per step, one whole 64-weight block
//    (4 consecutive blocks per row per wave step = one 128-byte line);
//  * the lane builds that block's 16-entry table bf16(V[k]·ĉ) once (exact
//    fp32 products, nearest-even bf16, identical to the standalone dequant)
//    and expands its 64 codes with byte permutes into bf16 operands of
//    v_mfma_f32_16x16x32_bf16 — the activations are the 16×32 A operand
//    (rows m >= M are zero), the dequantized weights the 32×16 B operand;
//  * codes are stored 8 per word with byte j = code j | code j+4 << 4, so
//    masking the word with 0x0F0F0F0F and its 4-bit shift yields selector
//    bytes for codes 0..3 and 4..7 directly, in natural order;
//  * waves reduce through LDS in a fixed order, then the epilogue adds
//    s·T·B with T summed from a few split-K planes, and rounds once to bf16.
//
// T = X·A for few tokens comes from k_lora_down_small: MFMA 16x16x32 with
// the activations as the A operand straight from memory and A's columns as
// the B operand, read from a row-major LDS tile with ds_read_b64_tr_b16
// (each 16-lane group gathers 4 consecutive k of 16 columns).
#include "kernels.h"

namespace qlora {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
}

// Split-K planes of T = X·A for M <= 16: workgroup (z, c) sums k in
// [512 z, 512 z + 512) for the adapter columns [64 c, 64 c + 64).
constexpr int kPrepK = 512;
constexpr int kPrepStride = 80;  // bf16 per LDS row: 64 + 16 pad, conflict-free transposed reads

__global__ __launch_bounds__(256) void k_lora_down_small(const uint16_t* __restrict__ X, int M,
                                                         int64_t d, const uint16_t* __restrict__ A,
                                                         int r, float* __restrict__ Tpart) {
  __shared__ __attribute__((aligned(16))) uint16_t s_a[kPrepK * kPrepStride];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t k0 = (int64_t)blockIdx.x * kPrepK;
  const int c0 = blockIdx.y * 64;
  // stage A[k0:k0+512][c0:c0+64] (zeros outside); all 16 loads of a thread
  // are in flight before the first store
  {
    uint4 v[kPrepK * 8 / 256];
#pragma unroll
    for (int u = 0; u < kPrepK * 8 / 256; ++u) {
      const int i = u * 256 + t, row = i >> 3, ch = i & 7;
      const int64_t k = k0 + row;
      const int col = c0 + ch * 8;
      v[u] = make_uint4(0, 0, 0, 0);
      if (k < d && col < r) v[u] = *reinterpret_cast<const uint4*>(A + k * r + col);
    }
#pragma unroll
    for (int u = 0; u < kPrepK * 8 / 256; ++u) {
      const int i = u * 256 + t, row = i >> 3, ch = i & 7;
      *reinterpret_cast<uint4*>(s_a + row * kPrepStride + ch * 8) = v[u];
    }
  }
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const int m = lane & 15, g = lane >> 4, s = lane & 15;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int kq = w * 4 + q;                    // 32-wide k step inside the slice
    const int64_t kx = k0 + kq * 32 + 8 * g;
    uint4 xv = make_uint4(0, 0, 0, 0);
    if (m < M && kx < d) xv = *reinterpret_cast<const uint4*>(X + (int64_t)m * d + kx);
    const bf16x8 a = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = kq * 32 + 8 * g + (s >> 2);
      const int col = j * 16 + 4 * (s & 3);
      const s16x4 lo = lds_read_tr(s_a + row * kPrepStride + col);
      const s16x4 hi = lds_read_tr(s_a + (row + 4) * kPrepStride + col);
      const short __attribute__((ext_vector_type(8))) bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
    }
  }
  __syncthreads();
  float* red = reinterpret_cast<float*>(s_a);      // [4 waves][16 m][64 cols]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(w * 16 + 4 * g + v) * 64 + j * 16 + (lane & 15)] = acc[j][v];
  __syncthreads();
  for (int i = t; i < 16 * 64; i += 256) {
    const int mm = i >> 6, cc = i & 63;
    if (mm < M && c0 + cc < r) {
      const float v = red[(0 * 16 + mm) * 64 + cc] + red[(1 * 16 + mm) * 64 + cc] +
                      red[(2 * 16 + mm) * 64 + cc] + red[(3 * 16 + mm) * 64 + cc];
      Tpart[((int64_t)blockIdx.x * M + mm) * r + c0 + cc] = v;
    }
  }
}

struct GemvArgs {
  const uint16_t* X;    // [M][d]
  const uint8_t* codes; const uint8_t* scale8; const float* scale2;
  const float* Tpart;   // [tsplits][M][r]
  const uint16_t* B;    // [r][o]
  uint16_t* Y;          // [M][o]
  float* T_out;         // [M][r] or null
  int64_t d, o;
  int M, r, tsplits;
  float s;
  Codebook cb;
};

// Byte planes of a 16-entry bf16 table given as 8 dwords (entries 2i, 2i+1).
struct Lut {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ void build_lut(const Codebook& cb, float chat, Lut& t) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = pack_bf16x2(cb.v[2 * i] * chat, cb.v[2 * i + 1] * chat);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], 0x06040200u);
    t.hi[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], 0x07050301u);
  }
}

// Look up 4 codes (one per byte of sel, values 0..15) in a byte plane.
// mask has 0xFF in the bytes whose code is >= 8.
__device__ __forceinline__ uint32_t plane4(const uint32_t (&pl)[4], uint32_t sel7, uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(pl[1], pl[0], sel7);
  const uint32_t b = __builtin_amdgcn_perm(pl[3], pl[2], sel7);
  return (b & mask) | (a & ~mask);
}

// 8 codes (one word: byte j = code j | code j+4 << 4) -> 8 bf16, natural order.
__device__ __forceinline__ bf16x8 expand8(const Lut& t, uint32_t w) {
  const uint32_t s0 = w & 0x07070707u, s1 = (w >> 4) & 0x07070707u;
  // bit 3 of each nibble -> 0xFF per byte, via the byte-sign selectors of v_perm
  const uint32_t w4 = w << 4;
  const uint32_t m0 = __builtin_amdgcn_perm(w4 << 8, w4, 0x090B080Au);
  const uint32_t m1 = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const uint32_t l0 = plane4(t.lo, s0, m0), h0 = plane4(t.hi, s0, m0);
  const uint32_t l1 = plane4(t.lo, s1, m1), h1 = plane4(t.hi, s1, m1);
  u32x4 r;
  r.x = __builtin_amdgcn_perm(h0, l0, 0x05010400u);  // codes 0, 1
  r.y = __builtin_amdgcn_perm(h0, l0, 0x07030602u);  // codes 2, 3
  r.z = __builtin_amdgcn_perm(h1, l1, 0x05010400u);  // codes 4, 5
  r.w = __builtin_amdgcn_perm(h1, l1, 0x07030602u);  // codes 6, 7
  return __builtin_bit_cast(bf16x8, r);
}

typedef __amdgpu_buffer_rsrc_t GRsrc;
constexpr uint32_t kGOob = 0x7FFFFF00u;   // an offset every descriptor rejects

// Range-checked buffer descriptor: loads past `bytes` read 0.
__device__ __forceinline__ GRsrc grsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)),
                                           0x00020000);
}
__device__ __forceinline__ uint4 gload16(GRsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// One 4-block group of a wave: lane (n = lane%16, q = lane/16) holds block
// 4·g + q of row n — 64 codes, its 8-bit scale and its group step.
struct GemvCodes {
  uint4 c0, c1;
  uint32_t q8;
  float step;
};

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(GemvArgs p) {
  __shared__ float s_part[WAVES][16][17];
  __shared__ float s_T[16 * kMaxGemvRank];
  __shared__ float s_B[kMaxGemvRank * 16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const uint32_t nblk = (uint32_t)(p.d / kBlock);
  const uint32_t ngrp = (nblk + 3) / 4;
  const int nl = lane & 15, q = lane >> 4, m = lane & 15;
  const int64_t n = n0 + nl;
  const bool lora = p.r > 0 && p.s != 0.0f;

  // ---- weight stream.  Every offset is 32-bit (the host bounds the weight
  // count); rows past o and blocks past the row end read 0 (a zero table
  // and zero activations contribute nothing).
  const uint32_t nbt = (uint32_t)(p.o * nblk);            // blocks in Wq
  const GRsrc rc = grsrc(p.codes, (int64_t)nbt * 32);
  const GRsrc rs8 = grsrc(p.scale8, nbt);
  const GRsrc rs2 = grsrc(p.scale2, (int64_t)((nbt + kGroup - 1) / kGroup) * 4);
  const GRsrc rx = grsrc(p.X, (int64_t)p.M * p.d * 2);
  const bool row_ok = n < p.o;
  const uint32_t brow = row_ok ? (uint32_t)n * nblk : 0u;
  // groups of this wave: g = w, w + WAVES, ...; iterations past the end read 0
  const int niter = (int)ngrp > w ? ((int)ngrp - w + WAVES - 1) / WAVES : 0;
  auto load_codes = [&](int it, GemvCodes& c) {
    const uint32_t kb = (uint32_t)(w + it * WAVES) * 4 + q;
    const bool ok = row_ok && kb < nblk;
    const uint32_t b = brow + kb;
    c.c0 = gload16(rc, ok ? b * 32 : kGOob);
    c.c1 = gload16(rc, ok ? b * 32 + 16 : kGOob);
    c.q8 = __builtin_amdgcn_raw_buffer_load_b8(rs8, (int)(ok ? b : kGOob), 0, 0);
    c.step = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs2, (int)(ok ? (b / kGroup) * 4 : kGOob), 0, 0));
  };
  auto load_x = [&](int it, uint4 (&x)[8]) {
    const uint32_t kb = (uint32_t)(w + it * WAVES) * 4 + q;
    const bool ok = m < p.M && kb < nblk;
    const uint32_t o0 = ok ? ((uint32_t)m * (uint32_t)p.d + kb * kBlock) * 2 : kGOob;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = gload16(rx, o0 + 16 * j);
  };
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const GemvCodes& c, const uint4 (&x)[8]) {
    Lut lut;
    build_lut(p.cb, (float)c.q8 * c.step, lut);   // ĉ = fl32(q8·step)
    const uint32_t cw[8] = {c.c0.x, c.c0.y, c.c0.z, c.c0.w, c.c1.x, c.c1.y, c.c1.z, c.c1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x[j]), expand8(lut, cw[j]),
                                                    acc, 0, 0, 0);
  };
  // codes of four groups in flight, activations of two (branch-free: the
  // steps past niter load and multiply zeros)
  GemvCodes c0, c1, c2, c3;
  uint4 xa[8], xb[8];
  load_codes(0, c0); load_codes(1, c1); load_codes(2, c2); load_codes(3, c3);
  load_x(0, xa);
  // ---- the adapter pieces the epilogue needs, fetched after the first
  // weight loads are in flight so their latency overlaps: T (summed over
  // its split-K planes, fixed order) and B[:, n0:n0+16]
  if (lora || (p.T_out != nullptr && blockIdx.x == 0)) {
    const int64_t plane = (int64_t)p.M * p.r;
    for (int i = t; i < p.M * p.r; i += WAVES * 64) {
      // planes summed in order, eight loads in flight at a time
      float sum = 0.0f;
      int z = 0;
      for (; z + 8 <= p.tsplits; z += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = p.Tpart[(int64_t)(z + u) * plane + i];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += v[u];
      }
      for (; z < p.tsplits; ++z) sum += p.Tpart[(int64_t)z * plane + i];
      s_T[i] = sum;
      if (p.T_out != nullptr && blockIdx.x == 0) p.T_out[i] = sum;
    }
  }
  if (lora) {
    for (int i = t; i < p.r * 16; i += WAVES * 64) {
      const int j = i >> 4, c = i & 15;
      s_B[i] = n0 + c < p.o ? bf16_to_f32(p.B[(int64_t)j * p.o + n0 + c]) : 0.0f;
    }
  }

  for (int it = 0; it < niter; it += 4) {
    load_x(it + 1, xb);
    compute(c0, xa);
    load_codes(it + 4, c0);
    load_x(it + 2, xa);
    compute(c1, xb);
    load_codes(it + 5, c1);
    if (it + 2 < niter) {
      load_x(it + 3, xb);
      compute(c2, xa);
      load_codes(it + 6, c2);
      load_x(it + 4, xa);
      compute(c3, xb);
      load_codes(it + 7, c3);
    }
  }
  // lane holds rows m = 4*(lane/16) + v of column n = lane%16
#pragma unroll
  for (int v = 0; v < 4; ++v) s_part[w][4 * (lane >> 4) + v][lane & 15] = acc[v];
  __syncthreads();
  if (t < 256) {
    const int mm = t >> 4, nc = t & 15;
    const int64_t nn = n0 + nc;
    if (mm < p.M && nn < p.o) {
      float y = 0.0f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) y += s_part[ww][mm][nc];
      if (lora) {
        float l = 0.0f;
        for (int j = 0; j < p.r; ++j) l += s_T[mm * p.r + j] * s_B[j * 16 + nc];
        y += p.s * l;
      }
      p.Y[(int64_t)mm * p.o + nn] = bf16_bits(y);
    }
  }
}

int gemv_tsplits(int64_t d) { return (int)((d + kPrepK - 1) / kPrepK); }

hipError_t launch_gemv_fwd(const uint16_t* X, int M, int64_t d, const uint8_t* codes,
                           const uint8_t* scale8, const float* scale2, int64_t o,
                           const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                           float* T_out, float* Tpart, const Codebook& cb, hipStream_t st) {
  const int ts = gemv_tsplits(d);
  const int rr = (r > 0 && (s != 0.0f || T_out != nullptr)) ? r : 0;
  if (rr > 0) {
    hipLaunchKernelGGL(k_lora_down_small, dim3(ts, (rr + 63) / 64), dim3(256), 0, st, X, M, d, A,
                       rr, Tpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  GemvArgs p{X, codes, scale8, scale2, Tpart, B, Y, T_out, d, o, M, rr, ts, s, cb};
  const unsigned grid = (unsigned)((o + 15) / 16);
  // enough waves to keep every CU streaming: split the reduction 4 ways
  // when there are many row groups, 8 ways otherwise
  if (o >= 16 * 512)
    hipLaunchKernelGGL(k_gemv<4>, dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(k_gemv<8>, dim3(grid), dim3(512), 0, st, p);
  return hipGetLastError();
}

}  // namespace qlora
