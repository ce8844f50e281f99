// Fused NF4 dequant-GEMM for many tokens (gfx950):
//   forward   Y  = X·Ŵ  + (s·T)·B      with Ŵ = Wqᵀ, blocks of Wq run along k
//   backward  dX = dY·Ŵᵀ + (s·U)·Aᵀ    blocks of Wq run along n
// ("074｜QLoRA：把大模型放进显存，再用小适配器改变它" §一 for the layer and the
// input gradient through Ŵᵀ; §三: dequantize the needed weights to BF16 on
// demand, then compute base plus adapter output).
//
// Tile 256×256×64, 4 waves in a 2×2 grid, each wave 128×128 of fp32
// accumulators fed by v_mfma_f32_32x32x16_bf16.  Per k-step each of the 256
// threads owns exactly one 64-weight block of the 256×64 weight tile: it
// loads 32 code bytes, one 8-bit scale and the group step, builds the block's
// 16-entry table bf16(V[k]·fl32(q8·step)) (exact fp32 products, the same bits
// as the standalone dequant), expands the 64 codes with byte permutes and
// writes 128 bytes of bf16 into LDS.  Codes are loaded two k-steps ahead, so
// the permute work of step s+1 overlaps the MFMAs of step s.
//
//  * forward: the weight tile is [n][k] like the activation tile (k-major
//    rows, XOR-swizzled 16-byte chunks), read with ds_read_b128;
//  * backward: a block is 64 consecutive n of one k, so the tile is stored
//    [k][n] (rows padded to 544 bytes) and the MFMA B operand is gathered
//    with ds_read_b64_tr_b16, four k of one n per lane per read.
// The adapter term is one (or a few) extra k-steps over [s·T ‖ B] or
// [s·U ‖ A], accumulated into the same registers, so Y and dX are rounded
// to bf16 once.  B [r][o] is n-major like the backward weight tile and A
// [d][r] k-major like the forward one, so neither needs a transposed copy.  Workgroups are numbered so that each XCD (round-robin
// dispatch over 8) works on a contiguous band of output tiles.
#include <type_traits>

#include "kernels.h"

namespace qlora {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 256;

__device__ __forceinline__ int swz8(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ s16x4 lds_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
}

struct Lut {
  uint32_t lo[4], hi[4];
};

__device__ __forceinline__ void make_lut(const Codebook& cb, float chat, Lut& t) {
  uint32_t p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = pack_bf16x2(cb.v[2 * i] * chat, cb.v[2 * i + 1] * chat);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], 0x06040200u);
    t.hi[i] = __builtin_amdgcn_perm(p[2 * i + 1], p[2 * i], 0x07050301u);
  }
}

__device__ __forceinline__ uint32_t plane(const uint32_t (&pl)[4], uint32_t sel7, uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(pl[1], pl[0], sel7);
  const uint32_t b = __builtin_amdgcn_perm(pl[3], pl[2], sel7);
  return (b & mask) | (a & ~mask);
}

// One packed code word (byte j = code j | code j+4 << 4) -> 8 bf16, natural order.
__device__ __forceinline__ uint4 expand(const Lut& t, uint32_t w) {
  const uint32_t s0 = w & 0x07070707u, s1 = (w >> 4) & 0x07070707u;
  const uint32_t w4 = w << 4;
  const uint32_t m0 = __builtin_amdgcn_perm(w4 << 8, w4, 0x090B080Au);  // bit 3 of low nibbles
  const uint32_t m1 = __builtin_amdgcn_perm(w << 8, w, 0x090B080Au);    // bit 3 of high nibbles
  const uint32_t l0 = plane(t.lo, s0, m0), h0 = plane(t.hi, s0, m0);
  const uint32_t l1 = plane(t.lo, s1, m1), h1 = plane(t.hi, s1, m1);
  return make_uint4(__builtin_amdgcn_perm(h0, l0, 0x05010400u), __builtin_amdgcn_perm(h0, l0, 0x07030602u),
                    __builtin_amdgcn_perm(h1, l1, 0x05010400u), __builtin_amdgcn_perm(h1, l1, 0x07030602u));
}

struct CodeReg {
  uint4 c0, c1;
  float chat;
};

}  // namespace

struct QGemmArgs {
  const uint16_t* A; int64_t lda;    // activations [M][K]
  const uint8_t* codes; const uint8_t* scale8; const float* scale2;   // Wq[o][d]
  int64_t d;                         // row length of Wq
  const uint16_t* A2; int64_t lda2;  // adapter activations [M][K2]
  const uint16_t* B2; int64_t ldb2;  // forward: B [K2][N]; backward: A [N][K2]
  int64_t M, N, K, K2;
  uint16_t* C; int64_t ldc;
  Codebook cb;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOobOff = 0x7FFFFFF0u;   // an offset every descriptor rejects

// Range-checked buffer descriptor (gfx9 family): loads past `bytes` read 0,
// stores past it are dropped.
__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;  // offsets are 32-bit
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)),
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

template <bool kTransW>
__global__ __launch_bounds__(kThreads) void k_qgemm(QGemmArgs p) {
  constexpr int BSTR = kTransW ? kBN + 16 : kBK;  // bf16 per weight-tile row in LDS
  constexpr int BROWS = kTransW ? kBK : kBN;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BROWS * BSTR];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w & 1, wn = w >> 1;

  // XCD-aware tile order: dispatch sends workgroup i to XCD i % 8; give each
  // XCD a contiguous run of tiles (row-major over the n-tiles).
  const int ntn = (int)((p.N + kBN - 1) / kBN), ntm = (int)((p.M + kBM - 1) / kBM);
  const int T = ntn * ntm;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = T >> 3, rem = T & 7;
  const int v = xcd * per + min(xcd, rem) + slot;
  const int64_t m0 = (int64_t)(v / ntn) * kBM, n0 = (int64_t)(v % ntn) * kBN;
  const int64_t mrows = min((int64_t)kBM, p.M - m0);

  // activations: descriptor rebased at the tile's first row; rows past M read 0
  const Rsrc ra_src = rsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  const int nk = (int)((p.K + kBK - 1) / kBK);
  const int nk2 = (int)((p.K2 + kBK - 1) / kBK);
  // chunk c = i*256 + t of the [256][64] tile: row c/8 = 32 i + t/8, chunk t%8
  const uint32_t a_off0 = (uint32_t)(((t >> 3) * p.lda + (t & 7) * 8) * 2);
  const uint32_t a_rowstep = (uint32_t)(32 * p.lda * 2);

  // quantized weight: codes, 8-bit scales, steps (reads past the end give 0,
  // which makes the block's table all zeros)
  const int64_t nW = kTransW ? p.K * p.d : p.N * p.d;   // weights in Wq
  const Rsrc rc = rsrc(p.codes, (nW + 7) / 8 * 4);
  const Rsrc rs8 = rsrc(p.scale8, (nW + kBlock - 1) / kBlock);
  const Rsrc rs2 = rsrc(p.scale2, ((nW + kBlock - 1) / kBlock + kGroup - 1) / kGroup * 4);
  // element index of this thread's block at k-step 0, and its advance per k-step
  const int64_t e0 = kTransW ? (int64_t)(t & 63) * p.d + n0 + 64 * (t >> 6) : (n0 + t) * p.d;
  const int64_t e_step = kTransW ? (int64_t)kBK * p.d : kBK;
  const bool w_row_ok = kTransW ? true : (n0 + t < p.N);

  uint4 ra[8];
  auto load_a = [&](int s) {
    const uint32_t base = a_off0 + (uint32_t)(s * kBK * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i) ra[i] = bload16(ra_src, base + i * a_rowstep);
  };
  auto store_a = [&](uint16_t* sa) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = i * 32 + (t >> 3), ch = t & 7;
      *reinterpret_cast<uint4*>(sa + row * kBK + ((ch ^ swz8(row)) << 3)) = ra[i];
    }
  };
  auto load_codes = [&](int s, CodeReg& c) {
    const int64_t e = e0 + (int64_t)s * e_step;
    const bool ok = w_row_ok && e < nW;
    const uint32_t ce = ok ? (uint32_t)(e / 2) : 0x7FFFFFF0u;
    c.c0 = bload16(rc, ce);
    c.c1 = bload16(rc, ce + 16);
    const uint32_t b = ok ? (uint32_t)(e / kBlock) : 0x7FFFFFF0u;
    const uint32_t q = __builtin_amdgcn_raw_buffer_load_b8(rs8, (int)b, 0, 0);
    const float st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs2, (int)((b / kGroup) * 4), 0, 0));
    c.chat = (float)q * st;
  };
  auto dequant = [&](const CodeReg& c, uint4 (&o)[8]) {
    Lut lut;
    make_lut(p.cb, c.chat, lut);
    const uint32_t ws[8] = {c.c0.x, c.c0.y, c.c0.z, c.c0.w, c.c1.x, c.c1.y, c.c1.z, c.c1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = expand(lut, ws[j]);
  };
  auto store_w = [&](const uint4 (&o)[8], uint16_t* sb) {
    if (!kTransW) {
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(sb + t * kBK + ((j ^ swz8(t)) << 3)) = o[j];
    } else {
      uint16_t* row = sb + (t & 63) * BSTR + 64 * (t >> 6);
#pragma unroll
      for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4*>(row + 8 * j) = o[j];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // The weight fragment is the MFMA's first operand and the activation
  // fragment its second, so each lane accumulates 4 consecutive output
  // columns of one output row (the epilogue stores 8 bytes at a time).
  // kBTr: the weight-side tile is [k][n] (read transposed) instead of [n][k].
  auto compute = [&](auto btr_tag, const uint16_t* sa, const uint16_t* sb) {
    constexpr bool kBTr = decltype(btr_tag)::value;
    constexpr int TSTR = kBN + 16;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 a[4], b[4];
      const int ch = kk * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8*>(sa + row * kBK + ((ch ^ swz8(row)) << 3));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!kBTr) {
          const int row = wn * 128 + j * 32 + (lane & 31);
          b[j] = *reinterpret_cast<const bf16x8*>(sb + row * kBK + ((ch ^ swz8(row)) << 3));
        } else {
          const int g = lane >> 4, s = lane & 15;
          const int col = wn * 128 + j * 32 + 16 * (g & 1) + 4 * (s & 3);
          const int kr = kk * 16 + 8 * (g >> 1) + (s >> 2);
          const s16x4 lo = lds_tr(sb + kr * TSTR + col);
          const s16x4 hi = lds_tr(sb + (kr + 4) * TSTR + col);
          const s16x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          b[j] = __builtin_bit_cast(bf16x8, bv);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    }
  };
  using WTag = std::integral_constant<bool, kTransW>;
  using ATag = std::integral_constant<bool, !kTransW>;

  // ---- main loop over the quantized weight: one branch-free block per k-step
  if (nk > 0) {
    CodeReg r0, r1;
    load_codes(0, r0);
    load_codes(1, r1);
    load_a(0);
    {
      uint4 dq[8];
      dequant(r0, dq);
      store_a(sA[0]);
      store_w(dq, sB[0]);
    }
    __syncthreads();
    // step s: prefetch activations of s+1 and codes of s+2, expand the codes
    // of s+1, multiply step s, then publish s+1 (past the end the extra
    // loads read zeros or in-range data and land in the idle buffer)
    auto iteration = [&](int s, CodeReg& refill, const CodeReg& next) {
      const int cur = s & 1;
      load_a(s + 1);
      load_codes(s + 2, refill);
      uint4 dq[8];
      dequant(next, dq);
      compute(WTag{}, sA[cur], sB[cur]);
      store_a(sA[cur ^ 1]);
      store_w(dq, sB[cur ^ 1]);
      __syncthreads();
    };
    int s = 0;
    for (; s + 1 < nk; s += 2) {
      iteration(s, r0, r1);
      iteration(s + 1, r1, r0);
    }
    if (s < nk) iteration(s, r0, r1);
  }

  // ---- adapter k-steps: [s·T ‖ B] (forward, B is [r][N]: an n-major tile
  // read transposed) or [s·U ‖ A] (backward, A is [N][r]: a k-major tile)
  if (nk2 > 0) {
    constexpr int TSTR = kBN + 16;
    uint16_t* sb = &sB[0][0];          // spans both stages (up to 34 KB used)
    const Rsrc r2 = rsrc(p.A2 + m0 * p.lda2, mrows * p.lda2 * 2);
    const Rsrc rb2 = !kTransW ? rsrc(p.B2, p.K2 * p.ldb2 * 2)
                              : rsrc(p.B2 + n0 * p.ldb2, min((int64_t)kBN, p.N - n0) * p.ldb2 * 2);
    for (int ls = 0; ls < nk2; ++ls) {
      const int64_t k0 = (int64_t)ls * kBK;
      uint4 rb[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = i * kThreads + t;
        const int row = c >> 3;
        const int64_t gk = k0 + (c & 7) * 8;
        ra[i] = bload16(r2, gk < p.K2 ? (uint32_t)((row * p.lda2 + gk) * 2) : kOobOff);
        if (kTransW) {   // A rows n, k-major
          rb[i] = bload16(rb2, gk < p.K2 ? (uint32_t)((row * p.ldb2 + gk) * 2) : kOobOff);
        } else {         // B rows k, n-major
          const int kr = c >> 5;
          const int64_t gk2 = k0 + kr, gn = n0 + (c & 31) * 8;
          rb[i] = bload16(rb2, (gk2 < p.K2 && gn < p.N) ? (uint32_t)((gk2 * p.ldb2 + gn) * 2) : kOobOff);
        }
      }
      store_a(sA[0]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int c = i * kThreads + t;
        if (kTransW) {
          const int row = c >> 3, ch = c & 7;
          *reinterpret_cast<uint4*>(sb + row * kBK + ((ch ^ swz8(row)) << 3)) = rb[i];
        } else {
          *reinterpret_cast<uint4*>(sb + (c >> 5) * TSTR + (c & 31) * 8) = rb[i];
        }
      }
      __syncthreads();
      compute(ATag{}, sA[0], sb);
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds output row m = lane%32 of each 32×32 block and
  // columns 8(e/4) + 4(lane/32) + e%4: four consecutive columns per 8-byte store
  const Rsrc rcout = rsrc(p.C + m0 * p.ldc, mrows * p.ldc * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = wm * 128 + i * 32 + (lane & 31);
        const int64_t col = n0 + wn * 128 + j * 32 + q * 8 + (lane >> 5) * 4;
        const uint32_t off = col < p.N ? (uint32_t)((row * p.ldc + col) * 2) : 0x7FFFFFF0u;
        const uint32_t lo = pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]);
        const uint32_t hi = pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        const i32x2 val = {(int)lo, (int)hi};
        __builtin_amdgcn_raw_buffer_store_b64(val, rcout, (int)off, 0, 0);
      }
}

hipError_t launch_qgemm(bool trans_w, const uint16_t* A, int64_t lda, const uint8_t* codes,
                        const uint8_t* scale8, const float* scale2, int64_t d,
                        const uint16_t* A2, int64_t lda2, const uint16_t* B2, int64_t ldb2,
                        int64_t M, int64_t N, int64_t K, int64_t K2, uint16_t* C, int64_t ldc,
                        hipStream_t st) {
  if (M == 0 || N == 0) return hipSuccess;
  QGemmArgs p{A, lda, codes, scale8, scale2, d, A2, lda2, B2, ldb2, M, N, K, K2, C, ldc,
              host_codebook()};
  const unsigned tiles = (unsigned)(((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN));
  if (trans_w)
    hipLaunchKernelGGL(k_qgemm<true>, dim3(tiles), dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(k_qgemm<false>, dim3(tiles), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace qlora
