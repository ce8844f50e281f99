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
//  * the permute expansion yields the 8 weights of a code dword in the order
//    0,2,4,6,1,3,5,7; the dot product does not care about the order of k as
//    long as both operands share it, so X is staged once per call in that
//    order (k_prep_small) instead of permuting per weight;
//  * waves reduce through LDS in a fixed order, then the epilogue adds
//    s·T·B with T summed from a few split-K planes, and rounds once to bf16.
#include "kernels.h"

namespace qlora {

// Reorder each group of 8 activations to 0,2,4,6,1,3,5,7 (bf16 lanes).
__device__ __forceinline__ uint4 even_odd8(uint4 x) {
  uint4 y;
  y.x = __builtin_amdgcn_perm(x.y, x.x, 0x05040100u);  // x0, x2
  y.y = __builtin_amdgcn_perm(x.w, x.z, 0x05040100u);  // x4, x6
  y.z = __builtin_amdgcn_perm(x.y, x.x, 0x07060302u);  // x1, x3
  y.w = __builtin_amdgcn_perm(x.w, x.z, 0x07060302u);  // x5, x7
  return y;
}

// X -> Xp (even/odd order per 8) and split-K planes of T = X·A.
// Grid: (tsplits); every block also reorders its k-slice of X.
__global__ __launch_bounds__(256) void k_prep_small(const uint16_t* __restrict__ X, int M, int64_t d,
                                                    const uint16_t* __restrict__ A, int r,
                                                    int64_t kslice, uint16_t* __restrict__ Xp,
                                                    float* __restrict__ Tpart) {
  const int z = blockIdx.x;
  const int64_t k0 = (int64_t)z * kslice;
  const int64_t k1 = min(d, k0 + kslice);
  // reorder X[m][k0:k1] in 8-element groups
  const int64_t groups = (k1 - k0) / 8;
  for (int64_t i = threadIdx.x; i < (int64_t)M * groups; i += blockDim.x) {
    const int64_t m = i / groups, g = i % groups;
    const int64_t off = m * d + k0 + g * 8;
    *reinterpret_cast<uint4*>(Xp + off) = even_odd8(*reinterpret_cast<const uint4*>(X + off));
  }
  // T partial over this k-slice: one (m, j) output per thread per pass
  for (int i = threadIdx.x; i < M * r; i += blockDim.x) {
    const int m = i / r, j = i % r;
    float acc = 0.0f;
    const uint16_t* xr = X + (int64_t)m * d;
    for (int64_t k = k0; k < k1; ++k) acc += bf16_to_f32(xr[k]) * bf16_to_f32(A[k * r + j]);
    Tpart[((int64_t)z * M + m) * r + j] = acc;
  }
}

struct GemvArgs {
  const uint16_t* Xp;   // [M][d], even/odd order per 8
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

// 8 codes (one dword) -> 8 bf16 in the order 0,2,4,6,1,3,5,7.
__device__ __forceinline__ bf16x8 expand8(const Lut& t, uint32_t w) {
  const uint32_t se = w & 0x07070707u, so = (w >> 4) & 0x07070707u;
  // bit 3 of each nibble -> 0xFF per byte, via the byte-sign selectors of v_perm
  const uint32_t w4 = w << 4;
  const uint32_t me = __builtin_amdgcn_perm(w4 << 8, w4, 0x090B080Au);
  const uint32_t mo = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);
  const uint32_t le = plane4(t.lo, se, me), he = plane4(t.hi, se, me);
  const uint32_t lo = plane4(t.lo, so, mo), ho = plane4(t.hi, so, mo);
  u32x4 r;
  r.x = __builtin_amdgcn_perm(he, le, 0x05010400u);
  r.y = __builtin_amdgcn_perm(he, le, 0x07030602u);
  r.z = __builtin_amdgcn_perm(ho, lo, 0x05010400u);
  r.w = __builtin_amdgcn_perm(ho, lo, 0x07030602u);
  return __builtin_bit_cast(bf16x8, r);
}

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_gemv(GemvArgs p) {
  __shared__ float s_part[WAVES][16][17];
  __shared__ float s_T[16 * kMaxGemvRank];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t nblk = p.d / kBlock;
  const int64_t ngrp = (nblk + 3) / 4;
  const int64_t n = n0 + (lane & 15);
  const int m = lane & 15;
  const bool row_ok = n < p.o;
  const bool m_ok = m < p.M;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int64_t gi = w; gi < ngrp; gi += WAVES) {
    const int64_t kb = gi * 4 + (lane >> 4);
    const bool ok = row_ok && kb < nblk;
    uint4 c0 = make_uint4(0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u), c1 = c0;
    float chat = 0.0f;
    if (ok) {
      const int64_t b = n * nblk + kb;
      const uint4* cp = reinterpret_cast<const uint4*>(p.codes + b * (kBlock / 2));
      c0 = cp[0];
      c1 = cp[1];
      chat = (float)p.scale8[b] * p.scale2[b / kGroup];
    }
    Lut lut;
    build_lut(p.cb, chat, lut);
    const uint4* xp = reinterpret_cast<const uint4*>(p.Xp + (int64_t)m * p.d + kb * kBlock);
    const bool xok = m_ok && kb < nblk;
    const uint32_t cw[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 xv = xok ? xp[j] : make_uint4(0, 0, 0, 0);
      const bf16x8 a = __builtin_bit_cast(bf16x8, xv);
      const bf16x8 bw = expand8(lut, cw[j]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bw, acc, 0, 0, 0);
    }
  }
  // lane holds rows m = 4*(lane/16) + v of column n = lane%16
#pragma unroll
  for (int v = 0; v < 4; ++v) s_part[w][4 * (lane >> 4) + v][lane & 15] = acc[v];

  const bool lora = p.r > 0 && p.s != 0.0f;
  if (lora || (p.T_out != nullptr && blockIdx.x == 0)) {
    for (int i = t; i < p.M * p.r; i += WAVES * 64) {
      float sum = 0.0f;
      for (int z = 0; z < p.tsplits; ++z) sum += p.Tpart[(int64_t)z * p.M * p.r + i];
      s_T[i] = sum;
      if (p.T_out != nullptr && blockIdx.x == 0) p.T_out[i] = sum;
    }
  }
  __syncthreads();
  if (t < 256) {
    const int mm = t >> 4, nl = t & 15;
    const int64_t nn = n0 + nl;
    if (mm < p.M && nn < p.o) {
      float y = 0.0f;
#pragma unroll
      for (int ww = 0; ww < WAVES; ++ww) y += s_part[ww][mm][nl];
      if (lora) {
        float l = 0.0f;
        for (int j = 0; j < p.r; ++j) l += s_T[mm * p.r + j] * bf16_to_f32(p.B[(int64_t)j * p.o + nn]);
        y += p.s * l;
      }
      p.Y[(int64_t)mm * p.o + nn] = bf16_bits(y);
    }
  }
}

int gemv_tsplits(int64_t d) {
  const int64_t s = d / 512;
  return (int)(s < 1 ? 1 : (s > 16 ? 16 : s));
}

hipError_t launch_gemv_fwd(const uint16_t* X, int M, int64_t d, const uint8_t* codes,
                           const uint8_t* scale8, const float* scale2, int64_t o,
                           const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                           float* T_out, uint16_t* Xp, float* Tpart, hipStream_t st) {
  const int ts = gemv_tsplits(d);
  const int64_t kslice = ((d / 8 + ts - 1) / ts) * 8;
  const int rr = (r > 0 && (s != 0.0f || T_out != nullptr)) ? r : 0;
  hipLaunchKernelGGL(k_prep_small, dim3(ts), dim3(256), 0, st, X, M, d, A, rr, kslice, Xp, Tpart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemvArgs p{Xp, codes, scale8, scale2, Tpart, B, Y, T_out, d, o, M, rr, ts, s, host_codebook()};
  const unsigned grid = (unsigned)((o + 15) / 16);
  if (o >= 16 * 512)
    hipLaunchKernelGGL(k_gemv<4>, dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL(k_gemv<16>, dim3(grid), dim3(1024), 0, st, p);
  return hipGetLastError();
}

}  // namespace qlora
