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
//  * k_rank_grad: planes of Σ_m BIG[m][p]·SMALL[m][j] over token slices; both
//    operands are token-major, staged in LDS as [m][·] rows and gathered
//    with ds_read_b64_tr_b16 (4 consecutive tokens of one column per read).
// Split planes are summed in a fixed order by k_reduce_planes, so results
// are bitwise reproducible.  (Summing them inside these kernels, with the
// last workgroup of a tile reducing, costs more on this chip: every
// device-scope release fence writes back the XCD's whole L2.)
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

constexpr int kDownRows = 128;    // rows of P per workgroup (4 waves × 32)
constexpr int kDownK = 512;       // k-slice per workgroup
constexpr int kDownLd = 80;       // LDS row stride (bf16) of the [k][j] Q tile: 64 + 16 pad
constexpr int kDownKLd = kDownK + 8;   // LDS row stride (bf16) of the [j][k] Q tile
constexpr int kWaveStage = 32 * 64;    // one wave's 32 rows × 64 k of P (4 KB)

// s_waitcnt vmcnt(N) (N < 16), other counters not waited on
template <int N>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt((0xF << 8) | (0x7 << 4) | N); }

// 16-byte chunk swizzle of a 128-byte P row
__device__ __forceinline__ int pswz(int row) { return (row >> 1) & 7; }


}  // namespace

// part[z][m][j] = Σ_{k in slice z} P[m][k]·Q(k, j),  j in [64 c, 64 c + 64).
// kQRowMajorK: Q(k, j) = Bsrc[j][k] (K-major rows of length K); otherwise
// Q(k, j) = Asrc[k][j] (row length r).
//
// P streams memory -> LDS by buffer_load ... lds: each wave owns 32 rows and
// moves them in 64-k stages (8 rows × 128 B per instruction, whole cache
// lines) through a 4-slot ring of its own, so the only waits are the wave's
// own vmcnt; 16-byte chunks are XOR-swizzled by (row / 2) % 8 so the A
// fragments (16 rows × 16 B per read) hit every bank once.
template <bool kQRowMajorK>
__global__ __launch_bounds__(256) void k_rank_down(const uint16_t* __restrict__ P, int64_t M,
                                                   int64_t K, const uint16_t* __restrict__ Q,
                                                   int r, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kQRowMajorK ? 64 * kDownKLd : kDownK * kDownLd];
  // ring slots in separate arrays: the compiler can tell a slot being read
  // from the slots the DMA is filling
  __shared__ __attribute__((aligned(16))) uint16_t s_p0[4 * kWaveStage], s_p1[4 * kWaveStage],
      s_p2[4 * kWaveStage], s_p3[4 * kWaveStage];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t m0 = (int64_t)blockIdx.x * kDownRows;
  const int64_t k0 = (int64_t)blockIdx.y * kDownK;
  const int c0 = blockIdx.z * 64;
  const int64_t kn = min((int64_t)kDownK, K - k0);       // valid k in this slice (multiple of 8)
  const int64_t mrows = min((int64_t)kDownRows, M - m0);

  // ---- Q tile loads (registers), issued first
  constexpr int kQLoads = kQRowMajorK ? 64 * kDownK / 8 / 256 : kDownK * 8 / 256;
  uint4 vq[kQLoads];
  if (!kQRowMajorK) {
    // Q[k0:k0+512][c0:c0+64]; rows past K and columns past r read 0
    const Rsrc rq = rsrc(Q + k0 * r, kn * r * 2);
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int i = u * 256 + t, row = i >> 3, col = c0 + (i & 7) * 8;
      vq[u] = bload16(rq, col < r ? (uint32_t)((row * r + col) * 2) : kOob);
    }
  } else {
    // Q[c0:c0+64][k0:k0+512] (rows j of B, K-major); rows past r and columns past K read 0
    const Rsrc rq = rsrc(Q + k0, ((int64_t)(r - 1) * K + kn) * 2);
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int i = u * 256 + t, row = i >> 6, ch = i & 63;     // 64 rows × 64 chunks
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
    for (int q = 0; q < 4; ++q) {
      const int row = w * 32 + q * 8 + (lane >> 3);
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
    const int i = u * 256 + t;
    if (!kQRowMajorK)
      *reinterpret_cast<uint4*>(s_q + (i >> 3) * kDownLd + (i & 7) * 8) = vq[u];
    else   // row stride 1040 bytes: the 16 rows one ds_read_b128 touches fall in different banks
      *reinterpret_cast<uint4*>(s_q + (i >> 6) * kDownKLd + (i & 63) * 8) = vq[u];
  }
  // LDS-only barrier: the P stages stay in flight (a fence here would wait
  // for them, since they write LDS)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int g = lane >> 4, l16 = lane & 15;
  const int sw = pswz(l16);              // = pswz of rows w*32 + 16 i + l16
#pragma unroll
  for (int st = 0; st < kDownK / 64; ++st) {
    // this wave's DMA for stage st is in once at most the later stages' are outstanding
    const int later = min(3, kDownK / 64 - 1 - st);
    if (later == 3) wait_vm<12>(); else if (later == 2) wait_vm<8>(); else if (later == 1) wait_vm<4>(); else wait_vm<0>();
    const uint16_t* sp = slot(st);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kq = st * 2 + h;
      bf16x8 a[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sp + (i * 16 + l16) * 64 + (((4 * h + g) ^ sw) << 3));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bf16x8 b =
            kQRowMajorK ? *reinterpret_cast<const bf16x8*>(s_q + (j * 16 + l16) * kDownKLd + kq * 32 + 8 * g)
                        : frag_tr(s_q, kDownLd, kq * 32, j * 16, lane);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
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
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t row = m0 + w * 32 + i * 16 + 4 * g + v;
        const int col = c0 + j * 16 + l16;
        if (row < M && col < r) out[row * r + col] = acc[i][j][v];
      }
}

namespace {
constexpr int kGradP = 128;       // big-dimension columns per workgroup (4 waves × 32)
constexpr int kGradM = 512;       // tokens per workgroup (split of the reduction)
constexpr int kGradChunk = 64;    // tokens staged per LDS round
constexpr int kBigLd = kGradP + 16;
constexpr int kSmallLd = 64 + 16;
}  // namespace

// part[z][...] = Σ_{m in slice z} BIG[m][p]·SMALL[m][j] for p in a 128-wide
// tile and j in [64 c, 64 c + 64).  kOutPJ: stored as [p][j] (row length r),
// else as [j][p] (row length P).
// kSmallF32: SMALL is fp32 and enters as bf16(small_scale · SMALL).
template <bool kOutPJ, bool kSmallF32>
__global__ __launch_bounds__(256) void k_rank_grad(const uint16_t* __restrict__ big, int64_t P,
                                                   const void* __restrict__ small, float small_scale,
                                                   int r, int64_t M, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_big[kGradChunk * kBigLd];
  __shared__ __attribute__((aligned(16))) uint16_t s_small[kGradChunk * kSmallLd];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t p0 = (int64_t)blockIdx.x * kGradP;
  const int64_t mz = (int64_t)blockIdx.y * kGradM;
  const int c0 = blockIdx.z * 64;
  const int64_t mlen = min((int64_t)kGradM, M - mz);
  const Rsrc rb = rsrc(big + mz * P, mlen * P * 2);
  const Rsrc rs = rsrc(static_cast<const char*>(small) + mz * r * (kSmallF32 ? 4 : 2),
                      mlen * r * (kSmallF32 ? 4 : 2));

  f32x4 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // BIG[mc:mc+64][p0:p0+128] and SMALL[mc:mc+64][c0:c0+64] of chunk c go
  // through registers into LDS; the loads of chunk c+1 are issued before the
  // MFMAs of chunk c, so memory latency overlaps them.
  constexpr int kChunks = kGradM / kGradChunk;
  constexpr int kSmallLoads = kSmallF32 ? 4 : 2;   // 16-byte loads per thread per chunk
  uint4 vb[kChunks][4], vs[kChunks][kSmallLoads];
  auto load = [&](int c) {
    const int mc = c * kGradChunk;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = q * 256 + t;                 // 64 rows × 16 chunks
      const int row = i >> 4, ch = i & 15;
      const int64_t col = p0 + ch * 8;
      vb[c][q] = bload16(rb, col < P ? (uint32_t)(((mc + row) * P + col) * 2) : kOob);
    }
#pragma unroll
    for (int q = 0; q < kSmallLoads; ++q) {
      const int i = q * 256 + t;
      if (kSmallF32) {                           // 64 rows × 16 chunks of 4 fp32
        const int row = i >> 4, col = c0 + (i & 15) * 4;
        vs[c][q] = bload16(rs, col < r ? (uint32_t)(((mc + row) * r + col) * 4) : kOob);
      } else {                                   // 64 rows × 8 chunks of 8 bf16
        const int row = i >> 3, col = c0 + (i & 7) * 8;
        vs[c][q] = bload16(rs, col < r ? (uint32_t)(((mc + row) * r + col) * 2) : kOob);
      }
    }
  };
  load(0);
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    if (c + 1 < kChunks) load(c + 1);
    __syncthreads();   // previous round's fragments are consumed
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = q * 256 + t;
      *reinterpret_cast<uint4*>(s_big + (i >> 4) * kBigLd + (i & 15) * 8) = vb[c][q];
    }
#pragma unroll
    for (int q = 0; q < kSmallLoads; ++q) {
      const int i = q * 256 + t;
      if (kSmallF32) {
        const float4 x = __builtin_bit_cast(float4, vs[c][q]);
        const uint2 b = make_uint2(pack_bf16x2(small_scale * x.x, small_scale * x.y),
                                   pack_bf16x2(small_scale * x.z, small_scale * x.w));
        *reinterpret_cast<uint2*>(s_small + (i >> 4) * kSmallLd + (i & 15) * 4) = b;
      } else {
        *reinterpret_cast<uint4*>(s_small + (i >> 3) * kSmallLd + (i & 7) * 8) = vs[c][q];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kq = 0; kq < kGradChunk / 32; ++kq) {
      bf16x8 fb[2], fs[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) fb[i] = frag_tr(s_big, kBigLd, kq * 32, w * 32 + i * 16, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fs[j] = frag_tr(s_small, kSmallLd, kq * 32, j * 16, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = kOutPJ ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[i], fs[j], acc[i][j], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fs[j], fb[i], acc[i][j], 0, 0, 0);
    }
  }
  // kOutPJ: block (i, j) is D[p][j]: lane holds j = lane%16, p rows 4*(lane/16)+v.
  // else:   block (i, j) is D[j][p]: lane holds p = lane%16, j rows 4*(lane/16)+v.
  const int g = lane >> 4, l16 = lane & 15;
  float* out = part + (int64_t)blockIdx.y * P * r;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        if (kOutPJ) {
          const int64_t p = p0 + w * 32 + i * 16 + 4 * g + v;
          const int jj = c0 + j * 16 + l16;
          if (p < P && jj < r) out[p * r + jj] = acc[i][j][v];
        } else {
          const int64_t p = p0 + w * 32 + i * 16 + l16;
          const int jj = c0 + j * 16 + 4 * g + v;
          if (p < P && jj < r) out[(int64_t)jj * P + p] = acc[i][j][v];
        }
      }
}

int rank_down_splits(int64_t K) { return (int)((K + kDownK - 1) / kDownK); }
int rank_grad_splits(int64_t M) { return (int)((M + kGradM - 1) / kGradM); }

hipError_t launch_rank_down(bool q_rowmajor_k, const uint16_t* P, int64_t M, int64_t K,
                            const uint16_t* Q, int r, float* part, hipStream_t st) {
  if (M == 0 || r == 0) return hipSuccess;
  dim3 grid((unsigned)((M + kDownRows - 1) / kDownRows), (unsigned)rank_down_splits(K),
            (unsigned)((r + 63) / 64));
  if (q_rowmajor_k)
    hipLaunchKernelGGL(k_rank_down<true>, grid, dim3(256), 0, st, P, M, K, Q, r, part);
  else
    hipLaunchKernelGGL(k_rank_down<false>, grid, dim3(256), 0, st, P, M, K, Q, r, part);
  return hipGetLastError();
}

hipError_t launch_rank_grad(bool out_pj, const uint16_t* big, int64_t P, const void* small,
                            bool small_f32, float small_scale, int r, int64_t M, float* part,
                            hipStream_t st) {
  if (P == 0 || r == 0) return hipSuccess;
  dim3 grid((unsigned)((P + kGradP - 1) / kGradP), (unsigned)rank_grad_splits(M),
            (unsigned)((r + 63) / 64));
#define QL_GRAD(PJ, F32) \
  hipLaunchKernelGGL((k_rank_grad<PJ, F32>), grid, dim3(256), 0, st, big, P, small, small_scale, r, M, part)
  if (out_pj) {
    if (small_f32) QL_GRAD(true, true); else QL_GRAD(true, false);
  } else {
    if (small_f32) QL_GRAD(false, true); else QL_GRAD(false, false);
  }
#undef QL_GRAD
  return hipGetLastError();
}

}  // namespace qlora
