// Internal launchers of the HIP kernels (host side).  Each enqueues on the
// given stream and returns the launch status; shapes are checked by callers.
#pragma once

#include "common.h"

namespace qlora {

struct GemmArgs {
  const uint16_t* A;  int64_t lda;   // K-major: [M][lda]; M-major: [K][lda]
  const uint16_t* B;  int64_t ldb;   // K-major: [N][ldb]; M-major: [K][ldb]
  const uint16_t* A2; int64_t lda2;  // adapter segment, K-major [M][K2]
  const uint16_t* B2; int64_t ldb2;  // adapter segment, K-major [N][K2]
  int64_t M, N, K, K2;
  void* C; int64_t ldc;              // bf16 [M][ldc], or fp32 planes [z][M][ldc]
  int64_t k_split;                   // main-segment K handled per blockIdx.z
  int64_t plane;                     // fp32 elements between partial planes
};

hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale8,
                           float* scale2, int32_t* flags, hipStream_t st);
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scale8, const float* scale2,
                          int64_t n, bool bf16, void* out, hipStream_t st);
hipError_t launch_dequant_t(const uint8_t* codes, const uint8_t* scale8, const float* scale2,
                            int64_t o, int64_t d, uint16_t* WT, hipStream_t st);

hipError_t launch_gemm_nt_bf16(const GemmArgs& a, hipStream_t st);

// Fused NF4 dequant-GEMM: C = A·Ŵ (+ A2·B2) with Ŵ from the quantized Wq[o][d].
// trans_w = false: forward, C[M][N=o] = A[M][K=d]·Wqᵀ, B2 = Bᵀ [N][K2].
// trans_w = true:  backward, C[M][N=d] = A[M][K=o]·Wq, B2 = Aᵀ [K2][N].
hipError_t launch_qgemm(bool trans_w, const uint16_t* A, int64_t lda, const uint8_t* codes,
                        const uint8_t* scale8, const float* scale2, int64_t d,
                        const uint16_t* A2, int64_t lda2, const uint16_t* B2, int64_t ldb2,
                        int64_t M, int64_t N, int64_t K, int64_t K2, uint16_t* C, int64_t ldc,
                        hipStream_t st);
hipError_t launch_gemm_nt_splitk(const GemmArgs& a, int splits, hipStream_t st);
hipError_t launch_gemm_tn_splitk(const GemmArgs& a, int splits, hipStream_t st);
hipError_t launch_reduce_planes(const float* part, int splits, int64_t plane, int64_t rows,
                                int64_t cols, int64_t ldp, float* out_f32, int64_t ldf,
                                uint16_t* out_bf16, int64_t ldb, float scale, hipStream_t st);
hipError_t launch_transpose_bf16(const uint16_t* src, int64_t R, int64_t C, uint16_t* dst,
                                 hipStream_t st);
hipError_t launch_scale_to_bf16(const float* x, int64_t n, float scale, uint16_t* y,
                                hipStream_t st);
hipError_t launch_fill_zero_bf16(uint16_t* y, int64_t n, hipStream_t st);

// Few-token forward (M <= kGemvMaxTokens): Tpart [gemv_tsplits(d)][M][r]
// fp32 is workspace.
constexpr int kGemvMaxTokens = 16;
constexpr int kMaxGemvRank = 256;
int gemv_tsplits(int64_t d);
hipError_t launch_gemv_fwd(const uint16_t* X, int M, int64_t d, const uint8_t* codes,
                           const uint8_t* scale8, const float* scale2, int64_t o,
                           const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                           float* T_out, float* Tpart, hipStream_t st);

}  // namespace qlora
