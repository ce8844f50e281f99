// Rank-r products of the adapter path ("074｜QLoRA：把大模型放进显存，再用
// 小适配器改变它" §一: Y = X·Ŵ + s·X·A·B; the backward needs U = dY·Bᵀ and the
// adapter gradients dA = s·Xᵀ·U, dB = s·(X·A)ᵀ·dY).
//
// Both kernels are bandwidth-bound on the big operand (X or dY, M×d or M×o
// bf16) and use v_mfma_f32_16x16x32_bf16 on fragments that never need a
// transposed copy in memory:
//  * k_rank_down: planes of P·Q over K-slices, P = X or dY ([M][K], K-major,
//    streamed into LDS by buffer_load ... lds and read as A fragments), Q = A
//    ([K][r]: staged in LDS and gathered with ds_read_b64_tr_b16) or Bᵀ (B is
//    [r][K], K-major: staged in LDS, read with ds_read_b128).
//  * k_rank_grad: planes of Σ_m BIG[m][p]·SMALL[m][j] over token slices, for
//    dA and dB in one launch; both operands are token-major, streamed into
//    LDS as [m][·] rows and gathered with ds_read_b64_tr_b16 (4 consecutive
//    tokens of one column per read).
// Split planes are summed in a fixed order (k_reduce_planes, or the tail of
// the backward dX launch for the dA and dB planes), so results are bitwise
// reproducible.  (Summing them inside these kernels, with the last
// workgroup of a row block reducing, costs more on this chip.  With
// device-scope release fences every workgroup writes back its XCD's whole
// L2; with planes written through to the device-coherent level and a relaxed
// count instead, the sums stay bitwise the same, but the last workgroups of
// the 32 row blocks of a 4096-token product do all of the summing on 32 of
// the 256 CUs: 20 µs per product against 9 + 4 for the product and
// k_reduce_planes.)
#include <type_traits>

#include "kernels.h"

namespace qlora {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ s16x4 lds_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
}

// B/A fragment of 16x16x32 from a row-major LDS tile [k][x] (row stride `ld`
// elements): column x0 + lane%16, rows k0 + 8*(lane/16) .. +7.
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* tile, int ld, int k0, int x0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const uint16_t* p = tile + (k0 + 8 * g + (s >> 2)) * ld + x0 + 4 * (s & 3);
  const s16x4 lo = lds_tr(p);
  const s16x4 hi = lds_tr(p + 4 * ld);
  const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)),
                                           0x00020000);
}
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
constexpr uint32_t kOob = 0x7FFFFFF0u;   // an offset every descriptor rejects

constexpr int kDownRows = 128;    // rows of P per workgroup (8 waves × 16)
constexpr int kDownK = 512;       // k-slice per workgroup
constexpr int kDownLd = 80;       // LDS row stride (bf16) of the [k][j] Q tile: 64 + 16 pad
constexpr int kDownKLd = kDownK + 8;   // LDS row stride (bf16) of the [j][k] Q tile
constexpr int kWaveStage = 16 * 64;    // one wave's 16 rows × 64 k of P (2 KB)

// s_waitcnt vmcnt(N) (N < 64: low 4 bits in [3:0], high 2 in [15:14]),
// other counters not waited on
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (N & 0xF));
}

// 16-byte chunk swizzle of a 128-byte P row
__device__ __forceinline__ int pswz(int row) { return (row >> 1) & 7; }


}  // namespace

// part[z][m][j] = Σ_{k in slice z} P[m][k]·Q(k, j),  j in [64 c, 64 c + 64).
// kQRowMajorK: Q(k, j) = Bsrc[j][k] (K-major rows of length K); otherwise
// Q(k, j) = Asrc[k][j] (row length r).
//
// P streams memory -> LDS by buffer_load ... lds: each of the 8 waves owns
// 16 rows (two waves per SIMD, since the adapter tile leaves room for one
// workgroup per CU) and moves them in 64-k stages (8 rows × 128 B per
// instruction, whole cache lines) through a 4-slot ring of its own, so the
// only waits are the wave's own vmcnt; 16-byte chunks are XOR-swizzled by
// (row / 2) % 8 so the A fragments (16 rows × 16 B per read) hit every bank
// once.
template <bool kQRowMajorK>
__global__ __launch_bounds__(512) void k_rank_down(const uint16_t* __restrict__ P, int64_t M,
                                                   int64_t K, const uint16_t* __restrict__ Q,
                                                   int r, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kQRowMajorK ? 64 * kDownKLd : kDownK * kDownLd];
  // ring slots in separate arrays: the compiler can tell a slot being read
  // from the slots the DMA is filling
  __shared__ __attribute__((aligned(16))) uint16_t s_p0[8 * kWaveStage], s_p1[8 * kWaveStage],
      s_p2[8 * kWaveStage], s_p3[8 * kWaveStage];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * kDownRows;
  const int64_t k0 = (int64_t)blockIdx.y * kDownK;
  const int c0 = blockIdx.z * 64;
  const int64_t kn = min((int64_t)kDownK, K - k0);       // valid k in this slice (multiple of 8)
  const int64_t mrows = min((int64_t)kDownRows, M - m0);

  // ---- Q tile loads (registers), issued first
  constexpr int kQLoads = kQRowMajorK ? 64 * kDownK / 8 / 512 : kDownK * 8 / 512;
  uint4 vq[kQLoads];
  if (!kQRowMajorK) {
    // Q[k0:k0+512][c0:c0+64]; rows past K and columns past r read 0
    const Rsrc rq = rsrc(Q + k0 * r, kn * r * 2);
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int i = u * 512 + t, row = i >> 3, col = c0 + (i & 7) * 8;
      vq[u] = bload16(rq, col < r ? (uint32_t)((row * r + col) * 2) : kOob);
    }
  } else {
    // Q[c0:c0+64][k0:k0+512] (rows j of B, K-major); rows past r and columns past K read 0
    const Rsrc rq = rsrc(Q + k0, ((int64_t)(r - 1) * K + kn) * 2);
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int i = u * 512 + t, row = i >> 6, ch = i & 63;     // 64 rows × 64 chunks
      const int j = c0 + row, kk = ch * 8;
      vq[u] = bload16(rq, (j < r && kk < kn) ? (uint32_t)(((int64_t)j * K + kk) * 2) : kOob);
    }
  }

  // ---- P stages: stage st covers k0 + 64 st .. +63; chunks past kn or rows
  // past M read 0 (a slice shorter than 512 streams zero stages)
  const Rsrc rp = rsrc(P + m0 * K + k0, mrows > 0 ? ((mrows - 1) * K + kn) * 2 : 0);
  auto slot = [&](int st) -> uint16_t* {
    uint16_t* s = (st & 3) == 0 ? s_p0 : (st & 3) == 1 ? s_p1 : (st & 3) == 2 ? s_p2 : s_p3;
    return s + w * kWaveStage;
  };
  auto dma = [&](int st) {
    uint16_t* dst = slot(st);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = w * 16 + q * 8 + (lane >> 3);
      const int kk = st * 64 + (((lane & 7) ^ pswz(row)) << 3);
      const uint32_t off = (row < mrows && kk < kn) ? (uint32_t)((row * K + kk) * 2) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rp, (__attribute__((address_space(3))) void*)(dst + q * 8 * 64), 16, off, 0, 0, 0);
    }
  };
#pragma unroll
  for (int st = 0; st < 4; ++st) dma(st);

  // ---- Q tile to LDS once its loads are in (the P stages stay in flight)
#pragma unroll
  for (int u = 0; u < kQLoads; ++u) {
    const int i = u * 512 + t;
    if (!kQRowMajorK)
      *reinterpret_cast<uint4*>(s_q + (i >> 3) * kDownLd + (i & 7) * 8) = vq[u];
    else   // row stride 1040 bytes: the 16 rows one ds_read_b128 touches fall in different banks
      *reinterpret_cast<uint4*>(s_q + (i >> 6) * kDownKLd + (i & 63) * 8) = vq[u];
  }
  // LDS-only barrier: the P stages stay in flight (a fence here would wait
  // for them, since they write LDS)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  f32x4 acc[4];                          // the wave's 16 rows × 4 blocks of 16 columns
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int g = lane >> 4, l16 = lane & 15;
  const int sw = pswz(l16);              // = pswz of rows w*16 + l16
#pragma unroll
  for (int st = 0; st < kDownK / 64; ++st) {
    // this wave's DMA for stage st is in once at most the later stages' are outstanding
    const int later = min(3, kDownK / 64 - 1 - st);
    if (later == 3) wait_vm<6>(); else if (later == 2) wait_vm<4>(); else if (later == 1) wait_vm<2>(); else wait_vm<0>();
    const uint16_t* sp = slot(st);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kq = st * 2 + h;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(sp + l16 * 64 + (((4 * h + g) ^ sw) << 3));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b =
            kQRowMajorK ? *reinterpret_cast<const bf16x8*>(s_q + (j * 16 + l16) * kDownKLd + kq * 32 + 8 * g)
                        : frag_tr(s_q, kDownLd, kq * 32, j * 16, lane);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
    // the slot is free again once this stage's fragments are in registers
    if (st + 4 < kDownK / 64) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      dma(st + 4);
    }
  }
  // lane holds rows 4*(lane/16)+v of column lane%16 in each 16×16 block
  float* out = part + (int64_t)blockIdx.y * M * r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = m0 + w * 16 + 4 * g + v;
      const int col = c0 + j * 16 + l16;
      if (row < M && col < r) out[row * r + col] = acc[j][v];
    }
}

namespace {
constexpr int kGradP = 128;       // big-dimension columns per workgroup (8 waves × 16)
constexpr int kGradM = 1024;      // tokens per workgroup (split of the reduction)
constexpr int kGradChunk = 64;    // tokens per LDS stage
constexpr int kBigStage = kGradChunk * kGradP;   // bf16 elements of a BIG stage (16 KB)
constexpr int kSmallStage = kGradChunk * 64;     // bf16 elements of a SMALL stage (8 KB)

// 16-byte chunk swizzles of the token-major stages.  Even XOR values keep
// each 32-byte pair together; a half-wave of a transposed fragment read
// touches rows R..R+3 and R+8..R+11 (R % 4 == 0), 32 bytes each, and these
// put the eight pieces in eight different 32-byte bank groups.
__device__ __forceinline__ int big_swz(int row) {     // 256-byte rows
  return 2 * ((row & 3) | (((row >> 3) & 1) << 2));
}
__device__ __forceinline__ int small_swz(int row) {   // 128-byte rows
  return 2 * (((row >> 1) & 1) | (((row >> 3) & 1) << 1));
}

// LDS byte address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Byte offset, within a swizzled token-major stage, of the first of the two
// ds_read_b64_tr_b16 of a 16x16x32 fragment: column x0 + lane%16, tokens
// 8*(lane/16) .. +7 (the second read is 4 rows further; rows r, r+4 and
// r+32 share a swizzle).
template <bool kBig>
__device__ __forceinline__ uint32_t frag_off(int x0, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int row = 8 * g + (s >> 2), col = x0 + 4 * (s & 3);
  const int sw = kBig ? big_swz(row) : small_swz(row);
  return (uint32_t)(row * (kBig ? 2 * kGradP : 128) + ((((col >> 3) ^ sw)) << 4) + (col & 7) * 2);
}

// The ten transposed reads of one 32-token step: the BIG fragment at b0
// (second read +1024 bytes), SMALL fragments at s0..s3 (+512 bytes).  The
// reads target LDS filled by buffer_load ... lds, so they are issued here
// with an explicit wait: the block returns with every result in place.
struct GradFrags {
  s16x4 b[2], s[4][2];
};
__device__ __forceinline__ void grad_reads(GradFrags& f, uint32_t b0, uint32_t s0, uint32_t s1,
                                           uint32_t s2, uint32_t s3) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %10\n\t"
      "ds_read_b64_tr_b16 %1, %10 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %11\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:512\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %12 offset:512\n\t"
      "ds_read_b64_tr_b16 %6, %13\n\t"
      "ds_read_b64_tr_b16 %7, %13 offset:512\n\t"
      "ds_read_b64_tr_b16 %8, %14\n\t"
      "ds_read_b64_tr_b16 %9, %14 offset:512\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f.b[0]), "=&v"(f.b[1]), "=&v"(f.s[0][0]), "=&v"(f.s[0][1]), "=&v"(f.s[1][0]),
        "=&v"(f.s[1][1]), "=&v"(f.s[2][0]), "=&v"(f.s[2][1]), "=&v"(f.s[3][0]), "=&v"(f.s[3][1])
      : "v"(b0), "v"(s0), "v"(s1), "v"(s2), "v"(s3)
      : "memory");
}
__device__ __forceinline__ bf16x8 join(const s16x4 (&x)[2]) {
  const s16x8 v = {x[0][0], x[0][1], x[0][2], x[0][3], x[1][0], x[1][1], x[1][2], x[1][3]};
  return __builtin_bit_cast(bf16x8, v);
}
}  // namespace

// part[z][...] = Σ_{m in slice z} BIG[m][p]·SMALL[m][j] for p in a 128-wide
// tile and j in [64 c, 64 c + 64), for two independent products in one
// launch (workgroups [0, a.tiles) take a, the rest b).  out_pj: stored as
// [p][j] (row length r), else as [j][p] (row length P).
//
// BIG [64 tokens][128 p] and SMALL [64 tokens][64 j] stages stream memory ->
// LDS by buffer_load ... lds (whole cache lines, 1 KB per instruction)
// through a 3-slot ring, two stages ahead; one LDS barrier per stage.  8
// waves of 16 columns p (90 VGPRs): two workgroups per CU, four waves per
// SIMD.
__global__ __launch_bounds__(512) void k_rank_grad(RankGradJob ja, RankGradJob jb, int r, int64_t M) {
  __shared__ __attribute__((aligned(16))) uint16_t sb0[kBigStage], sb1[kBigStage], sb2[kBigStage];
  __shared__ __attribute__((aligned(16))) uint16_t ss0[kSmallStage], ss1[kSmallStage], ss2[kSmallStage];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool first = (int)blockIdx.x < ja.tiles;
  const uint16_t* big = first ? ja.big : jb.big;
  const uint16_t* small = first ? ja.small : jb.small;
  float* part = first ? ja.part : jb.part;
  const int64_t P = first ? ja.P : jb.P;
  const bool out_pj = first ? ja.out_pj : jb.out_pj;
  const int64_t p0 = (int64_t)(first ? blockIdx.x : blockIdx.x - ja.tiles) * kGradP;
  const int64_t mz = (int64_t)blockIdx.y * kGradM;
  const int c0 = blockIdx.z * 64;
  const int64_t mlen = min((int64_t)kGradM, M - mz);
  const Rsrc rb = rsrc(big + mz * P, mlen * P * 2);
  const Rsrc rs = rsrc(small + mz * r, mlen * r * 2);

  auto big_slot = [&](int c) -> uint16_t* { return c % 3 == 0 ? sb0 : c % 3 == 1 ? sb1 : sb2; };
  auto small_slot = [&](int c) -> uint16_t* { return c % 3 == 0 ? ss0 : c % 3 == 1 ? ss1 : ss2; };
  // stage c of the slice (tokens mz + 64 c ..); tokens past M, columns past
  // P or r read 0.  Wave w moves BIG rows 8w .. 8w+7 and SMALL rows
  // 8w .. 8w+7.
  auto dma = [&](int c) {
    uint16_t* sb = big_slot(c);
    uint16_t* ss = small_slot(c);
#pragma unroll
    for (int u = 0; u < 2; ++u) {              // 4 rows × 256 bytes per instruction
      const int q = 2 * w + u, row = 4 * q + (lane >> 4);
      const int tok = c * kGradChunk + row;
      const int64_t col = p0 + 8 * ((lane & 15) ^ big_swz(row));
      const uint32_t off = (tok < mlen && col < P) ? (uint32_t)((tok * P + col) * 2) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, (__attribute__((address_space(3))) void*)(sb + q * 512), 16, off, 0, 0, 0);
    }
    {                                          // 8 rows × 128 bytes per instruction
      const int q = w, row = 8 * q + (lane >> 3);
      const int tok = c * kGradChunk + row;
      const int col = c0 + 8 * ((lane & 7) ^ small_swz(row));
      const uint32_t off = (tok < mlen && col < r) ? (uint32_t)((tok * r + col) * 2) : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(ss + q * 512), 16, off, 0, 0, 0);
    }
  };

  // the main loop and the epilogue, for one output layout (uniform per workgroup)
  auto body = [&](auto pj_tag) {
  constexpr bool kOutPJ = decltype(pj_tag)::value;
  f32x4 acc[4];                          // the wave's 16 columns p × 4 blocks of 16 j
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int kChunks = kGradM / kGradChunk;   // a slice shorter than kGradM streams zero stages
  const uint32_t ob0 = frag_off<true>(w * 16, lane);
  const uint32_t os0 = frag_off<false>(0, lane), os1 = frag_off<false>(16, lane);
  const uint32_t os2 = frag_off<false>(32, lane), os3 = frag_off<false>(48, lane);
  dma(0);
  dma(1);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    // this wave's part of stage c is in once at most stage c+1 is outstanding
    if (c + 1 < kChunks) wait_vm<3>(); else wait_vm<0>();
    // every wave's part has landed and every wave is done with stage c-1
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (c + 2 < kChunks) dma(c + 2);           // into the slot of stage c-1
    const uint32_t ab = lds_addr(big_slot(c)), as = lds_addr(small_slot(c));
#pragma unroll
    for (int kq = 0; kq < kGradChunk / 32; ++kq) {
      // 32 tokens further: 32 rows of 256 (BIG) or 128 (SMALL) bytes
      GradFrags f;
      grad_reads(f, ab + ob0 + kq * 8192, as + os0 + kq * 4096,
                 as + os1 + kq * 4096, as + os2 + kq * 4096, as + os3 + kq * 4096);
      const bf16x8 fb = join(f.b);
      bf16x8 fs[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) fs[j] = join(f.s[j]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = kOutPJ ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fs[j], acc[j], 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fs[j], fb, acc[j], 0, 0, 0);
    }
  }
  // out_pj: block j is D[p][j]: lane holds j = lane%16, p rows 4*(lane/16)+v.
  // else:   block j is D[j][p]: lane holds p = lane%16, j rows 4*(lane/16)+v.
  const int g = lane >> 4, l16 = lane & 15;
  float* out = part + (int64_t)blockIdx.y * P * r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (kOutPJ) {
        const int64_t p = p0 + w * 16 + 4 * g + v;
        const int jj = c0 + j * 16 + l16;
        if (p < P && jj < r) out[p * r + jj] = acc[j][v];
      } else {
        const int64_t p = p0 + w * 16 + l16;
        const int jj = c0 + j * 16 + 4 * g + v;
        if (p < P && jj < r) out[(int64_t)jj * P + p] = acc[j][v];
      }
    }
  };
  if (out_pj) body(std::true_type{}); else body(std::false_type{});
}

int rank_down_splits(int64_t K) { return (int)((K + kDownK - 1) / kDownK); }
int rank_grad_splits(int64_t M) { return (int)((M + kGradM - 1) / kGradM); }

hipError_t launch_rank_down(bool q_rowmajor_k, const uint16_t* P, int64_t M, int64_t K,
                            const uint16_t* Q, int r, float* part, hipStream_t st) {
  if (M == 0 || r == 0) return hipSuccess;
  dim3 grid((unsigned)((M + kDownRows - 1) / kDownRows), (unsigned)rank_down_splits(K),
            (unsigned)((r + 63) / 64));
  if (q_rowmajor_k)
    launch(k_rank_down<true>, grid, dim3(512), 0, st, P, M, K, Q, r, part);
  else
    launch(k_rank_down<false>, grid, dim3(512), 0, st, P, M, K, Q, r, part);
  return hipGetLastError();
}

hipError_t launch_rank_grads(RankGradJob a, RankGradJob b, int r, int64_t M, hipStream_t st) {
  a.tiles = a.P > 0 ? (int)((a.P + kGradP - 1) / kGradP) : 0;
  b.tiles = b.P > 0 ? (int)((b.P + kGradP - 1) / kGradP) : 0;
  if (a.tiles + b.tiles == 0 || r == 0 || M == 0) return hipSuccess;
  dim3 grid((unsigned)(a.tiles + b.tiles), (unsigned)rank_grad_splits(M), (unsigned)((r + 63) / 64));
  launch(k_rank_grad, grid, dim3(512), 0, st, a, b, r, M);
  return hipGetLastError();
}

}  // namespace qlora
