// Internal launchers of the HIP kernels (host side).  Each enqueues on the
// given stream and returns the launch status; shapes are checked by callers.
#pragma once

#include <hip/hip_ext.h>

#include "common.h"

namespace qlora {

// Every kernel of the library is launched through launch().  While the
// timing diagnostics have armed this thread's event pair (the launches of
// one timed call), the first kernel records the start event and every kernel
// the stop event, at the dispatch's own begin and end; otherwise it is a
// plain launch.
struct LaunchEvents {
  hipEvent_t start, stop;
  bool fired;
};
LaunchEvents*& armed_launch_events();

template <typename K, typename... Args>
inline void launch(K kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t st, Args... args) {
  LaunchEvents* ev = armed_launch_events();
  if (ev == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
    return;
  }
  hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)shmem, st, ev->start, ev->stop, 0u, args...);
  ev->start = nullptr;
  ev->fired = true;
}


// fmt: the 16-entry table of the codes (host_codebook(fmt), with its
// host_encode_guide(fmt)); hipErrorInvalidValue when the guide is unusable.
hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale8,
                           float* scale2, int32_t* flags, int fmt, hipStream_t st);
// Several tensors of one table in one launch: job k covers workgroups
// [g0, g0 + ceil(n/16384)), the jobs in order with g0 the running sum.
constexpr int kMaxQuantJobs = 16;
struct QuantJob {
  const float* W;
  uint8_t* codes;
  uint8_t* scale8;
  float* scale2;
  int64_t n, g0;
};
struct QuantJobs {
  QuantJob j[kMaxQuantJobs];
  int count;
};
hipError_t launch_quantize_grouped(const QuantJobs& jobs, int32_t* flags, int fmt, hipStream_t st);
// dq: second-level variant (0 default; 1 int8 around the tensor mean; 2 E4M3
// around it, the mean stored after the steps in scale2).
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scale8, const float* scale2,
                          int64_t n, bool bf16, void* out, const Codebook& cb, hipStream_t st,
                          int dq = 0);
// Rewrites scale8 and scale2 (+ the mean) for variant dq after launch_quantize.
// psum: device workspace of ceil(n/16384) doubles.
hipError_t launch_dq_variant(const float* W, int64_t n, uint8_t* scale8, float* scale2, int dq,
                             double* psum, hipStream_t st);


// Contiguous split planes [splits][count] (count % 4 == 0) -> their sum, in
// plane order: out_f32 = Σ, out_bf16 = bf16(scale·Σ).  With one plane it is
// the conversion to bf16(scale·x).  Two independent jobs per launch (the
// second may have count 0).
struct ReduceJob {
  const float* part;
  int splits;
  int64_t plane, count;
  float* out_f32;
  uint16_t* out_bf16;
  float scale;
};
hipError_t launch_reduce_planes(const ReduceJob& a, const ReduceJob& b, hipStream_t st);

// Element quad i (of count/4) of a plane sum: the planes are added in order,
// up to eight loads in flight.
__device__ __forceinline__ void reduce_planes_quad(const ReduceJob& jo, int64_t i) {
  const float4* part = reinterpret_cast<const float4*>(jo.part);
  const int64_t pl = jo.plane / 4;
  const int nb = jo.splits < 8 ? jo.splits : 8;      // the first batch, plane 0 included
  float4 v0[8];
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (u < nb) v0[u] = part[(int64_t)u * pl + i];
  float4 s = v0[0];
#pragma unroll
  for (int u = 1; u < 8; ++u)
    if (u < nb) { s.x += v0[u].x; s.y += v0[u].y; s.z += v0[u].z; s.w += v0[u].w; }
  int z = nb;
  for (; z + 8 <= jo.splits; z += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(z + u) * pl + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
  }
  for (; z < jo.splits; ++z) {
    const float4 v = part[(int64_t)z * pl + i];
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (jo.out_f32) reinterpret_cast<float4*>(jo.out_f32)[i] = s;
  if (jo.out_bf16) {
    uint2 o;
    o.x = pack_bf16x2(jo.scale * s.x, jo.scale * s.y);
    o.y = pack_bf16x2(jo.scale * s.z, jo.scale * s.w);
    reinterpret_cast<uint2*>(jo.out_bf16)[i] = o;
  }
}

// Fused NF4 dequant-GEMM: C = A·Ŵ (+ A2·B2) with Ŵ from the quantized Wq[o][d].
// trans_w = false: forward, C[M][N=o] = A[M][K=d]·Wqᵀ + A2·B2, B2 = B [K2][N].
// trans_w = true:  backward, C[M][N=d] = A[M][K=o]·Wq + A2·B2ᵀ, B2 = A [N][K2].
// tail_a/tail_b: plane sums (as launch_reduce_planes) that the same launch
// performs after its tiles, their planes complete before it starts; jobs
// with count 0 are skipped.
hipError_t launch_qgemm(bool trans_w, const uint16_t* A, int64_t lda, const uint8_t* codes,
                        const uint8_t* scale8, const float* scale2, int64_t d,
                        const uint16_t* A2, int64_t lda2, const uint16_t* B2, int64_t ldb2,
                        int64_t M, int64_t N, int64_t K, int64_t K2, uint16_t* C, int64_t ldc,
                        const Codebook& cb, hipStream_t st, const ReduceJob& tail_a = ReduceJob{},
                        const ReduceJob& tail_b = ReduceJob{});

// Rank-r products (split planes, summed by launch_reduce_planes):
// part[z][M][r] = P[M][K-slice z]·Q with Q = Qsrc[K][r], or Q = Qsrc[r][K]ᵀ
// when q_rowmajor_k; rank_down_splits(K) planes.
int rank_down_splits(int64_t K);
hipError_t launch_rank_down(bool q_rowmajor_k, const uint16_t* P, int64_t M, int64_t K,
                            const uint16_t* Q, int r, float* part, hipStream_t st);
// One product of launch_rank_grads: part[z] = Σ_{m in token slice z}
// big[m][p]·small[m][j] (big [M][P], small [M][r], both bf16), stored
// [P][r] when out_pj, else [r][P]; rank_grad_splits(M) planes.  A job with
// P == 0 is skipped.
struct RankGradJob {
  const uint16_t* big;
  int64_t P;
  const uint16_t* small;
  float* part;
  bool out_pj;
  int tiles;   // set by the launcher
};
int rank_grad_splits(int64_t M);
hipError_t launch_rank_grads(RankGradJob a, RankGradJob b, int r, int64_t M, hipStream_t st);

hipError_t launch_fill_zero_bf16(uint16_t* y, int64_t n, hipStream_t st);

// Few-token forward (M <= kGemvMaxTokens): Tpart [gemv_tsplits(d)][M][r]
// fp32 is workspace.
constexpr int kGemvMaxTokens = 16;
constexpr int kMaxGemvRank = 256;
int gemv_tsplits(int64_t d);
// Whether the few-token kernel serves these sizes (its shared memory and
// staged scales fit); otherwise the forward takes the GEMM path.
bool gemv_fits(int64_t M, int64_t d, int64_t r);
// adapter != null: one adapter per token, A [n_ad][d][r], B [n_ad][r][o],
// scales s_ad[n_ad] (host); an index outside [0, n_ad) selects no adapter.
constexpr int kMaxAdapters = 64;
// The T planes of the few-token kernel (k_lora_down_small): Tpart
// [gemv_tsplits(d)][M][r]; launch_gemv_fwd with tdown = false then skips them.
hipError_t launch_gemv_tdown(const uint16_t* X, int M, int64_t d, const uint16_t* A, int r,
                             float* Tpart, hipStream_t st, const int32_t* adapter = nullptr,
                             int n_ad = 0);
hipError_t launch_gemv_fwd(const uint16_t* X, int M, int64_t d, const uint8_t* codes,
                           const uint8_t* scale8, const float* scale2, int64_t o,
                           const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                           float* T_out, float* Tpart, const Codebook& cb, hipStream_t st,
                           const int32_t* adapter = nullptr, int n_ad = 0,
                           const float* s_ad = nullptr, bool tdown = true);

// Adapter merge: W_out[n][k] = fl32(ŵ[n][k] + fl32(s·Σ_j A[k][j]·B[j][n])),
// the rank sum by fp32 FMAs in increasing j.  d % 64 == 0, o % 8 == 0.
hipError_t launch_merge(const uint8_t* codes, const uint8_t* scale8, const float* scale2,
                        int64_t o, int64_t d, const uint16_t* A, const uint16_t* B, int r, float s,
                        float* W_out, const Codebook& cb, hipStream_t st);

// AdamW of the adapter parameters (optim.hip).
struct AdamwConsts {
  float b1, b2, c1, c2, rs, keep, lr1, eps;
};
AdamwConsts adamw_consts(float lr, float b1, float b2, float eps, float wd, int64_t t);
hipError_t launch_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m, float* v, int64_t n,
                        const AdamwConsts& k, hipStream_t st);
int64_t paged_adamw_page_elems(size_t pool_bytes);
hipError_t launch_paged_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m_host,
                              float* v_host, int64_t n, const AdamwConsts& k, void* pool,
                              size_t pool_bytes, hipStream_t st);

}  // namespace qlora
