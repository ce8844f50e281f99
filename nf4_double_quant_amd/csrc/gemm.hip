// bf16 MFMA GEMM tiles for the QLoRA linear layer (gfx950).
//
//   C[M][N] = Σ_k Aop[m][k]·Bop[n][k]  (+ a second "LoRA" K-segment)
//
// Operands are bf16 with fp32 accumulation in v_mfma_f32_32x32x16_bf16.
// Each operand is either K-major (row-major [rows][K], as X, dY, Wq, A, Bᵀ
// are for the products over d or o) or M-major ([K][rows], as X, T, U, dY
// are for the adapter gradients, whose reduction runs over the tokens).
// M-major tiles are transposed in registers (8×8 bf16 blocks with v_perm)
// so LDS always holds [rows][64 k] tiles.
//
// LDS tiles are [rows][64] bf16 (128 B per row) with the 16-byte chunk
// index XOR-swizzled by (row ^ row>>3) & 7: the MFMA operand reads (32
// consecutive rows, one chunk) and the transposed writes (rows 8 apart) are
// both free of bank conflicts without padding.  Two LDS stages; the next
// stage's global loads are in flight while the current one is multiplied.
//
// The second K-segment carries the adapter term as extra reduction columns,
// [X ‖ s·T]·[Ŵ ‖ Bᵀ]ᵀ = X·Ŵ + s·T·B, so the product and the adapter share one
// accumulator and one rounding to bf16.
#include "kernels.h"

namespace qlora {


__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// 8×8 bf16 transpose: in[k] holds rows 0..7 at reduction index k; out[r]
// holds reduction indices 0..7 of row r.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const uint32_t sel = (r & 1) ? 0x07060302u : 0x05040100u;
    uint32_t d[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 lo = in[2 * c], hi = in[2 * c + 1];
      const uint32_t a = (r >> 1) == 0 ? lo.x : (r >> 1) == 1 ? lo.y : (r >> 1) == 2 ? lo.z : lo.w;
      const uint32_t b = (r >> 1) == 0 ? hi.x : (r >> 1) == 1 ? hi.y : (r >> 1) == 2 ? hi.z : hi.w;
      d[c] = __builtin_amdgcn_perm(b, a, sel);
    }
    out[r] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

template <int ROWS, int NT, bool kTrans>
struct TileLoader {
  // K-major: ROWS*8 16-byte chunks; M-major: ROWS sub-blocks of 8×8.
  static constexpr int kChunks = kTrans ? 0 : (ROWS * 8 + NT - 1) / NT;
  static constexpr int kSub = kTrans ? (ROWS + NT - 1) / NT : 0;
  uint4 r[kTrans ? kSub * 8 : kChunks];

  __device__ __forceinline__ void load(const uint16_t* base, int64_t ld, int64_t row0,
                                       int64_t nrows, int64_t k0, int64_t klim, int t) {
    if (!kTrans) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = i * NT + t;
        const int row = c >> 3, kc = (c & 7) * 8;
        const int64_t gr = row0 + row, gk = k0 + kc;
        r[i] = (c < ROWS * 8 && gr < nrows && gk < klim) ? ld16(base + gr * ld + gk)
                                                         : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        const int sb = i * NT + t;
        const int rg = sb % (ROWS / 8), kg = sb / (ROWS / 8);
        const int64_t gr = row0 + rg * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int64_t gk = k0 + kg * 8 + kk;
          r[i * 8 + kk] = (sb < ROWS && gr < nrows && gk < klim) ? ld16(base + gk * ld + gr)
                                                                 : make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* s, int t) {
    if (!kTrans) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = i * NT + t;
        if (c < ROWS * 8) {
          const int row = c >> 3, ch = c & 7;
          *reinterpret_cast<uint4*>(s + row * 64 + ((ch ^ swz(row)) << 3)) = r[i];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kSub; ++i) {
        const int sb = i * NT + t;
        if (sb < ROWS) {
          const int rg = sb % (ROWS / 8), kg = sb / (ROWS / 8);
          uint4 in[8], out[8];
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) in[kk] = r[i * 8 + kk];
          transpose8x8(in, out);
#pragma unroll
          for (int rr = 0; rr < 8; ++rr) {
            const int row = rg * 8 + rr;
            *reinterpret_cast<uint4*>(s + row * 64 + ((kg ^ swz(row)) << 3)) = out[rr];
          }
        }
      }
    }
  }
};

template <int BM, int BN, int WM, int WN, bool kTransA, bool kTransB, bool kF32Out>
__global__ __launch_bounds__(WM * WN * 64) void k_gemm(GemmArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM / 32, TN = BN / WN / 32;
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 block");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BN * 64];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w % WM, wn = w / WM;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t kbeg = (int64_t)blockIdx.z * p.k_split;
  const int64_t kend = min(p.K, kbeg + p.k_split);
  const int nk1 = kend > kbeg ? (int)((kend - kbeg + 63) / 64) : 0;
  const int nk2 = blockIdx.z == 0 ? (int)((p.K2 + 63) / 64) : 0;
  const int nks = nk1 + nk2;

  TileLoader<BM, NT, kTransA> la;
  TileLoader<BN, NT, kTransB> lb;

  auto load = [&](int s) {
    if (s < nk1) {
      const int64_t k0 = kbeg + (int64_t)s * 64;
      la.load(p.A, p.lda, m0, p.M, k0, kend, t);
      lb.load(p.B, p.ldb, n0, p.N, k0, kend, t);
    } else if constexpr (!kTransA && !kTransB) {
      // the adapter segment (only used with K-major operands)
      const int64_t k0 = (int64_t)(s - nk1) * 64;
      la.load(p.A2, p.lda2, m0, p.M, k0, p.K2, t);
      lb.load(p.B2, p.ldb2, n0, p.N, k0, p.K2, t);
    }
  };
  auto store = [&](int buf) {
    la.store(sA[buf], t);
    lb.store(sB[buf], t);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int ar0 = wm * (BM / WM), bc0 = wn * (BN / WN);
  auto compute = [&](int buf) {
    const uint16_t* a_s = sA[buf];
    const uint16_t* b_s = sB[buf];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      bf16x8 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = ar0 + i * 32 + (lane & 31);
        a[i] = *reinterpret_cast<const bf16x8*>(a_s + row * 64 + ((ch ^ swz(row)) << 3));
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = bc0 + j * 32 + (lane & 31);
        b[j] = *reinterpret_cast<const bf16x8*>(b_s + row * 64 + ((ch ^ swz(row)) << 3));
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };

  if (nks > 0) {
    load(0);
    store(0);
    __syncthreads();
    for (int s = 0; s < nks; ++s) {
      if (s + 1 < nks) load(s + 1);
      compute(s & 1);
      if (s + 1 < nks) store((s + 1) & 1);
      __syncthreads();
    }
  }

  // epilogue: lane holds column (lane & 31); register v holds row
  // 8*(v/4) + 4*(lane/32) + v%4 of each 32×32 block.
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + ar0 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int64_t col = n0 + bc0 + j * 32 + (lane & 31);
        if (row < p.M && col < p.N) {
          if (kF32Out)
            reinterpret_cast<float*>(p.C)[(int64_t)blockIdx.z * p.plane + row * p.ldc + col] =
                acc[i][j][v];
          else
            reinterpret_cast<uint16_t*>(p.C)[row * p.ldc + col] = bf16_bits(acc[i][j][v]);
        }
      }
}

// Sum of split-K planes: out_f32 = Σ_z part[z]; out_bf16 = bf16(scale·Σ_z part[z]).
__global__ __launch_bounds__(256) void k_reduce_planes(const float* __restrict__ part, int splits,
                                                       int64_t plane, int64_t rows, int64_t cols,
                                                       int64_t ldp, float* __restrict__ out_f32,
                                                       int64_t ldf, uint16_t* __restrict__ out_bf16,
                                                       int64_t ldb, float scale) {
  const int64_t total = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / cols, c = i % cols;
    float s = 0.0f;
    for (int z = 0; z < splits; ++z) s += part[(int64_t)z * plane + r * ldp + c];
    if (out_f32) out_f32[r * ldf + c] = s;
    if (out_bf16) out_bf16[r * ldb + c] = bf16_bits(scale * s);
  }
}

// bf16 transpose dst[C][R] = src[R][C]ᵀ (small adapter matrices).
__global__ __launch_bounds__(256) void k_transpose_bf16(const uint16_t* __restrict__ src,
                                                        int64_t R, int64_t C,
                                                        uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[32][33];
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 × 8
  const int64_t r0 = (int64_t)blockIdx.y * 32, c0 = (int64_t)blockIdx.x * 32;
  for (int k = ty; k < 32; k += 8) {
    const int64_t r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < R && c < C) ? src[r * C + c] : 0;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int64_t c = c0 + k, r = r0 + tx;
    if (c < C && r < R) dst[c * R + r] = tile[tx][k];
  }
}

__global__ __launch_bounds__(256) void k_fill_zero_bf16(uint16_t* __restrict__ y, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

// fp32 -> bf16(scale·x), elementwise.
__global__ __launch_bounds__(256) void k_scale_to_bf16(const float* __restrict__ x, int64_t n,
                                                       float scale, uint16_t* __restrict__ y) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    y[i] = bf16_bits(scale * x[i]);
}

// ------------------------------------------------------------------ launchers
static inline unsigned cdiv(int64_t a, int64_t b) { return (unsigned)((a + b - 1) / b); }

// Main products: C = A·Bᵀ (+ A2·B2ᵀ), K-major operands, bf16 output.
hipError_t launch_gemm_nt_bf16(const GemmArgs& a, hipStream_t st) {
  GemmArgs p = a;
  p.k_split = p.K;
  p.plane = 0;
  dim3 grid(cdiv(p.N, 256), cdiv(p.M, 256), 1);
  hipLaunchKernelGGL((k_gemm<256, 256, 2, 2, false, false, false>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// Skinny product with split-K into fp32 planes: part[z] = A·Bᵀ over K-slice z.
hipError_t launch_gemm_nt_splitk(const GemmArgs& a, int splits, hipStream_t st) {
  GemmArgs p = a;
  p.K2 = 0;
  p.k_split = ((p.K + (int64_t)splits * 64 - 1) / ((int64_t)splits * 64)) * 64;
  p.plane = p.M * p.ldc;
  dim3 grid(cdiv(p.N, 64), cdiv(p.M, 64), (unsigned)splits);
  hipLaunchKernelGGL((k_gemm<64, 64, 2, 2, false, false, true>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// Adapter-gradient product, both operands M-major: part[z] = Σ_{m in slice z} L[m]ᵀR[m].
hipError_t launch_gemm_tn_splitk(const GemmArgs& a, int splits, hipStream_t st) {
  GemmArgs p = a;
  p.K2 = 0;
  p.k_split = ((p.K + (int64_t)splits * 64 - 1) / ((int64_t)splits * 64)) * 64;
  p.plane = p.M * p.ldc;
  if (p.M <= 64) {
    dim3 grid(cdiv(p.N, 128), cdiv(p.M, 64), (unsigned)splits);
    hipLaunchKernelGGL((k_gemm<64, 128, 2, 2, true, true, true>), grid, dim3(256), 0, st, p);
  } else {
    dim3 grid(cdiv(p.N, 64), cdiv(p.M, 128), (unsigned)splits);
    hipLaunchKernelGGL((k_gemm<128, 64, 2, 2, true, true, true>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_planes(const float* part, int splits, int64_t plane, int64_t rows,
                                int64_t cols, int64_t ldp, float* out_f32, int64_t ldf,
                                uint16_t* out_bf16, int64_t ldb, float scale, hipStream_t st) {
  const int64_t total = rows * cols;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_reduce_planes, dim3((unsigned)blocks), dim3(256), 0, st, part, splits,
                     plane, rows, cols, ldp, out_f32, ldf, out_bf16, ldb, scale);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t st) {
  if (R == 0 || C == 0) return hipSuccess;
  dim3 grid(cdiv(C, 32), cdiv(R, 32));
  hipLaunchKernelGGL(k_transpose_bf16, grid, dim3(256), 0, st, src, R, C, dst);
  return hipGetLastError();
}

hipError_t launch_scale_to_bf16(const float* x, int64_t n, float scale, uint16_t* y,
                                hipStream_t st) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_scale_to_bf16, dim3((unsigned)blocks), dim3(256), 0, st, x, n, scale, y);
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
