// Blockwise NF4 quantization with double quantization, and dequantization.
//
// Method: "074｜QLoRA：把大模型放进显存，再用小适配器改变它" §二 (NF4 codes,
// absmax per 64 weights, 8-bit first-level constants with one fp32
// second-level constant per 256 of them) and §三 (quantize the weights with
// the first-level constants, then quantize those constants).
//
// gfx950 design
//  * One workgroup of 8 waves per double-quant group (16384 weights = 64 KB
//    of fp32): the group's second-level constant needs every block's
//    absmax, so the whole group is loaded at once into VGPRs (8 float4 per
//    lane) and HBM is read exactly once.  Eight waves per group (rather than
//    four with twice the weights per lane) halve each group's encode time
//    and leave two groups per CU in flight, which streams large tensors
//    from HBM faster than more, slower groups per CU.
//  * 8 lanes per 64-weight block, 8 consecutive weights per lane, 4 blocks
//    per lane.  A block's codes need only its own absmax, so only the small
//    second level waits for the whole group: pass 1 takes each block's
//    absmax, thresholds and cell reciprocal as its two loads land; pass 2
//    encodes the four blocks of a lane two at a time (their LDS reads in
//    flight together) and stores them.
//  * The block absmax is an 8-lane DPP max on the integer bits of |w|
//    (integer order equals float order for non-negative floats, and NaN/Inf
//    land above every finite value, which is how non-finite input is
//    detected).
//  * Exact nearest-value encode without fp64 per weight: the 15 decision
//    points c1·mid_t are exact fp64 products; rounding each one DOWN to fp32
//    gives a threshold th_t with  w > c1·mid_t  <=>  w > th_t  for every
//    fp32 w.  The 8 lanes of a block compute its 16 entries (the last one
//    +inf) into shared memory.  A weight's code is then a guess and one
//    compare: the cell of w·S/c1 on a 1/S grid (S = 128) indexes a table of
//    the code at each cell's lower edge, which the host built so that the
//    true code is that code or the next one, and  w > th_guess  adds the 1.
//    All-zero and non-finite blocks take the cell of a code-7 guess;
//    blocks with absmax below 2^-100 (and a group that ends inside a code
//    word) take a rare, wave-uniform generic copy of pass 2.
//  * Each lane packs its 8 codes into one 32-bit word (byte j = code j |
//    code j+4 << 4) and a wave's store covers 8 consecutive blocks (256 B).
#include <type_traits>

#include "kernels.h"

namespace qlora {

// The largest fp32 values <= two fp64 values: the conversions run with the
// wave's fp32 rounding mode (MODE bits 1:0) set to toward −inf, restored to
// nearest-even inside the same block so no other arithmetic sees it (the
// block is then a pure function of its inputs and may be scheduled freely).
__device__ __forceinline__ float2 round_down_pair(double a, double b) {
  float x, y;
  asm(
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 2\n\t"
      "s_nop 1\n\t"
      "v_cvt_f32_f64 %0, %2\n\t"
      "v_cvt_f32_f64 %1, %3\n\t"
      "s_setreg_imm32_b32 hwreg(HW_REG_MODE, 0, 2), 0\n\t"
      "s_nop 1"
      : "=&v"(x), "=&v"(y)
      : "v"(a), "v"(b));
  return make_float2(x, y);
}

// max over the 8 lanes of each half of a DPP row (rotations by 4, 2, 1
// within the half: row_half_mirror then quad permutes)
__device__ __forceinline__ uint32_t row_max8(uint32_t a) {
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x141, 0xF, 0xF, false));  // half-row mirror
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  return a;
}

__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc rsrc(const void* base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes)),
                                           0x00020000);
}

constexpr int kQuantWaves = 8;                                   // waves per group
constexpr int kLaneBlocks = kGroup / (kQuantWaves * 8);        // blocks per lane: 4

// Group g of one tensor (a workgroup of 64·kQuantWaves threads).
// kStream: the launch streams from HBM; its code words are stored with the
// non-temporal hint (the next reader is another launch, long after).
template <bool kStream>
__device__ __forceinline__ void quantize_group(const float* __restrict__ W, int64_t n,
                                               uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scale8,
                                               float* __restrict__ scale2,
                                               int32_t* __restrict__ flags, const Codebook& cb,
                                               const EncodeGuide& eg, int64_t g) {
  __shared__ __attribute__((aligned(16))) float s_thr[kGroup][16];   // per-block thresholds
  __shared__ uint32_t s_guide[(kGuideCells + 3) / 4];
  __shared__ double s_mid[16];
  __shared__ uint32_t s_c1[kGroup];
  __shared__ uint32_t s_red[kQuantWaves];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int sub = lane & 7, row = lane >> 3;      // 8 lanes per block, 8 weights per lane
  const int64_t base = g * kGroupElems;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t nvalid = n - base;

  // ---- issue every load of the group (reads past n return 0)
  const Rsrc rw = rsrc(W + base, (min((int64_t)kGroupElems, nvalid)) * 4);
  float4 v[2 * kLaneBlocks];
#pragma unroll
  for (int j = 0; j < kLaneBlocks; ++j) {
    const int bl = (wave * kLaneBlocks + j) * 8 + row;
    const int off = (bl * kBlock + sub * 8) * 4;
    v[2 * j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
    v[2 * j + 1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rw, off + 16, 0, 0));
  }
  if (t < (kGuideCells + 3) / 4) s_guide[t] = eg.packed[t];
  if (t < 16) s_mid[t] = t < 15 ? cb.mid[t] : __builtin_inf();
  __syncthreads();
  // this lane's two thresholds of each block: indices sub and sub + 8
  // (index 15 is +inf: a code never exceeds 15)
  const double mid_lo = s_mid[sub], mid_hi = s_mid[sub + 8];
  const uint8_t* guide = reinterpret_cast<const uint8_t*>(s_guide);
  const float zero_base = (float)eg.zero_cell + 0.5f;
  const float cell_base = (float)kGuideScale + 0.5f;

  const int nv_group = (int)min(nvalid, (int64_t)kGroupElems);    // 32-bit: a scalar test
  const bool ragged = nv_group < kGroupElems && (nv_group & 7) != 0;
  const int64_t code_bytes = (n + 7) / 8 * 4;
  const int64_t cbase = g * (kGroupElems / 2);
  const Rsrc rcod = rsrc(codes + cbase, code_bytes - cbase);

  // ---- pass 1, per block as its loads land: absmax, thresholds and the
  // factors of the cell computation
  uint32_t bad = 0, tiny_any = 0;
  float inv[kLaneBlocks];
#pragma unroll
  for (int j = 0; j < kLaneBlocks; ++j) {
    const int bl = (wave * kLaneBlocks + j) * 8 + row;
    const float4 p = v[2 * j], q = v[2 * j + 1];
    uint32_t a = max(max(max(abs_bits(p.x), abs_bits(p.y)), max(abs_bits(p.z), abs_bits(p.w))),
                     max(max(abs_bits(q.x), abs_bits(q.y)), max(abs_bits(q.z), abs_bits(q.w))));
    a = row_max8(a);
    bad |= (a >= 0x7F800000u);
    s_c1[bl] = a;                                  // the 8 lanes agree
    const float c1 = __uint_as_float(a);
    const double c1d = (double)c1;
    // th_t = c1·mid_t rounded down to fp32: w > th_t exactly when w > c1·mid_t
    const float2 th = round_down_pair(c1d * mid_lo, c1d * mid_hi);
    s_thr[bl][sub] = th.x;
    s_thr[bl][sub + 8] = th.y;
    // S/c1 = 1/(c1·2^-7) with S = 128: for c1 in [2^-100, FLT_MAX] both the
    // argument and the result of the reciprocal are normal floats.  Blocks
    // with 0 < c1 < 2^-100 scale w and c1 by 2^64 (pass 2's generic copy);
    // all-zero and non-finite blocks take zero_cell.
    const bool tiny = a - 1u < 0x0D800000u - 1u;
    tiny_any |= tiny;
    const float rc = __builtin_amdgcn_rcpf(c1 * (a < 0x0D800000u ? 0x1p57f : 0x1p-7f));
    inv[j] = a - 1u < 0x7F7FFFFFu ? rc : 0.0f;       // finite, nonzero c1 (a finite reciprocal is never 0)
  }

  // ---- pass 2: encode and store.  The cell of x = w/c1 gives a guide code
  // that is the code of w or one below it, and one threshold compare decides.
  // Straight-line over the lane's blocks unless a block is tiny or the group
  // ends inside a code word.
  auto encode_store = [&](auto generic) {
    constexpr bool kGeneric = decltype(generic)::value;
#pragma unroll
    for (int jp = 0; jp < kLaneBlocks; jp += 2) {                // two blocks at a time
      uint32_t cell[16], g0[16], k[16];
      float th[16];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = jp + h;
        const float4 p = v[2 * j], q = v[2 * j + 1];
        const float w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
        float sc = 1.0f;
        if constexpr (kGeneric) sc = s_c1[(wave * kLaneBlocks + j) * 8 + row] - 1u < 0x0D800000u - 1u ? 0x1p64f : 1.0f;
        // inv = 0 marks an all-zero or non-finite block
        const float c0 = inv[j] != 0.0f ? cell_base : zero_base;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = kGeneric ? w[e] * sc : w[e];
          // v_cvt_u32_f32: NaN (a non-finite block) gives 0, still a valid cell
          asm("v_cvt_u32_f32 %0, %1" : "=v"(cell[8 * h + e]) : "v"(__builtin_fmaf(x, inv[j], c0)));
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) g0[e] = guide[cell[e]];
#pragma unroll
      for (int e = 0; e < 16; ++e) th[e] = s_thr[(wave * kLaneBlocks + jp + (e >> 3)) * 8 + row][g0[e]];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = jp + h;
        const float4 p = v[2 * j], q = v[2 * j + 1];
        const float w[8] = {p.x, p.y, p.z, p.w, q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) k[8 * h + e] = g0[8 * h + e] + (w[e] > th[8 * h + e] ? 1u : 0u);
        const uint32_t* kk = k + 8 * h;
        // word `sub` of the block: byte e = code e | code e+4 << 4
        uint32_t word = (kk[0] | (kk[4] << 4)) | ((kk[1] | (kk[5] << 4)) << 8) |
                        ((kk[2] | (kk[6] << 4)) << 16) | ((kk[3] | (kk[7] << 4)) << 24);
        const int wi = ((wave * kLaneBlocks + j) * 8 + row) * 8 + sub;     // word within the group
        if constexpr (kGeneric) {
          // The word holding code n-1 may end in codes past n; they are
          // stored as 7, the layout's padding, whatever a zero weight
          // encodes to.
          const int nv = nv_group - wi * 8;                     // valid codes of this word
          if (nv > 0 && nv < 8) {
            uint32_t keep = 0;
            for (int c = 0; c < nv; ++c) keep |= 0xFu << (8 * (c & 3) + 4 * (c >> 2));
            word = (word & keep) | (0x77777777u & ~keep);
          }
        }
        // (stores past the code buffer are dropped; cache policy 2 = nt)
        __builtin_amdgcn_raw_buffer_store_b32(word, rcod, wi * 4, 0, kStream ? 2 : 0);
      }
    }
  };
  if (ragged || __builtin_amdgcn_ballot_w64(tiny_any != 0))
    encode_store(std::true_type{});
  else
    encode_store(std::false_type{});
  __syncthreads();

  // ---- second level: one thread per block (threads 0..255)
  const uint32_t c1_bits = t < kGroup ? s_c1[t] : 0u;
  uint32_t m = c1_bits;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = s_red[0];
#pragma unroll
  for (int i = 1; i < kQuantWaves; ++i) m = max(m, s_red[i]);
  const float c1 = __uint_as_float(c1_bits);
  const float c2 = __uint_as_float(m);
  // fp64 quotient of fp32 operands rounded to fp32 is the correctly rounded quotient.
  const float step = (float)((double)c2 / 255.0);

  uint32_t q = 0;
  if (step > 0.0f) {
    const double cd = (double)c1, sd = (double)step;
    double qf = floor(cd / sd);
    if (!(qf < 255.0)) qf = 255.0;
    const int q0 = (int)qf;
    // Exact: (2q0+1)·step has at most 33 significant bits.
    q = (uint32_t)q0 + (cd > (2.0 * (double)q0 + 1.0) * sd * 0.5 ? 1u : 0u);
    q = min(q, 255u);
  }
  const int64_t b_glob = g * kGroup + t;
  if (t < kGroup && b_glob < nb) scale8[b_glob] = (uint8_t)q;
  if (t == 0) scale2[g] = step;
  if (bad && flags != nullptr) flags[0] = flags[0] | 1;
}

// kWavesPerSimd: the occupancy the registers are fitted to; kStream: the
// launch streams its input from HBM (see the launchers)
template <int kWavesPerSimd, bool kStream>
__global__ __launch_bounds__(64 * kQuantWaves) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd))) void k_quantize(const float* __restrict__ W, int64_t n,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scale8,
                                                  float* __restrict__ scale2,
                                                  int32_t* __restrict__ flags, Codebook cb,
                                                  EncodeGuide eg) {
  quantize_group<kStream>(W, n, codes, scale8, scale2, flags, cb, eg, blockIdx.x);
}

// Several tensors in one launch: workgroup i quantizes group i - g0 of the
// last job whose first workgroup g0 is <= i.  The job is picked by a uniform
// scan with constant indices, so the table stays in kernel-argument memory.
template <int kWavesPerSimd, bool kStream>
__global__ __launch_bounds__(64 * kQuantWaves) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd))) void k_quantize_grouped(QuantJobs jobs, int32_t* __restrict__ flags,
                                                          Codebook cb, EncodeGuide eg) {
  const int64_t i = blockIdx.x;
  QuantJob j = jobs.j[0];
#pragma unroll
  for (int k = 1; k < kMaxQuantJobs; ++k)
    if (k < jobs.count && i >= jobs.j[k].g0) j = jobs.j[k];
  quantize_group<kStream>(j.W, j.n, j.codes, j.scale8, j.scale2, flags, cb, eg, i - j.g0);
}

// ------------------------------------------------------------------ dequant
// Code j (0..7) of a packed word.
__device__ __forceinline__ uint32_t code_of(uint32_t w, int j) {
  return (w >> (8 * (j & 3) + 4 * (j >> 2))) & 15u;
}

// E4M3 value of an 8-bit pattern (bias 7, subnormals; 0x7F/0xFF never
// produced by the encoder).
__device__ __forceinline__ float e4m3_value(uint32_t q) {
  const int e = (int)((q >> 3) & 15), m = (int)(q & 7);
  const float mag = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
  return (q & 0x80) ? -mag : mag;
}

// ĉ of block b for the second-level variant dq (0: q8·step; 1: int8 around
// the tensor mean μ; 2: E4M3 around μ), each operation rounded to fp32.
__device__ __forceinline__ float block_chat(const uint8_t* scale8, const float* scale2, int64_t b,
                                            int dq, float mu) {
#pragma clang fp contract(off)
  const uint32_t q = scale8[b];
  const float step = scale2[b / kGroup];
  if (dq == 0) return (float)q * step;
  const float qv = dq == 1 ? (float)(int8_t)q : e4m3_value(q);
  return qv * step + mu;
}

// Eight weights per thread (one code word); ŵ = fl32(V[k]·ĉ) with ĉ of the
// block's second-level variant (fl32(q8·step) by default).
template <bool kBf16>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scale8,
                                                 const float* __restrict__ scale2, int64_t n,
                                                 void* __restrict__ out, Codebook cb, int dq) {
#pragma clang fp contract(off)
  __shared__ float s_v[16];
  const int64_t ngr = ((n + kBlock - 1) / kBlock + kGroup - 1) / kGroup;
  const float mu = dq != 0 ? scale2[ngr] : 0.0f;
  if (threadIdx.x < 16) s_v[threadIdx.x] = cb.v[threadIdx.x];
  __syncthreads();
  const int64_t n8 = (n + 7) / 8;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e0 = i * 8;
    const int64_t b = e0 / kBlock;
    const float chat = block_chat(scale8, scale2, b, dq, mu);
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[i];
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = s_v[code_of(w, k)] * chat;
    if (kBf16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      if (e0 + 8 <= n && ((reinterpret_cast<uintptr_t>(o + e0) & 15) == 0)) {
        uint4 pk;
        pk.x = pack_bf16x2(r[0], r[1]);
        pk.y = pack_bf16x2(r[2], r[3]);
        pk.z = pack_bf16x2(r[4], r[5]);
        pk.w = pack_bf16x2(r[6], r[7]);
        *reinterpret_cast<uint4*>(o + e0) = pk;
      } else {
        for (int k = 0; k < 8; ++k)
          if (e0 + k < n) o[e0 + k] = bf16_bits(r[k]);
      }
    } else {
      float* o = reinterpret_cast<float*>(out);
      if (e0 + 8 <= n) {
        reinterpret_cast<float4*>(o + e0)[0] = make_float4(r[0], r[1], r[2], r[3]);
        reinterpret_cast<float4*>(o + e0)[1] = make_float4(r[4], r[5], r[6], r[7]);
      } else {
        for (int k = 0; k < 8; ++k)
          if (e0 + k < n) o[e0 + k] = r[k];
      }
    }
  }
}

// ------------------------------------------------------------------ second-level variants
// The constants centred on the tensor mean μ before their 8-bit code (the
// offset the QLoRA page mentions beside the 8-bit constants; int8 or E4M3
// codes).  Three launches after k_quantize has written the codes: per-group
// sums of c1, the mean, then each group's new step and codes.  The sums and
// the mean use fixed orders, so the results are reproducible bit for bit.

// c1 of block b (valid weights only), as k_quantize computes it.
__device__ __forceinline__ float dq_block_c1(const float* W, int64_t n, int64_t b) {
  const int64_t e0 = b * kBlock;
  uint32_t m = 0;
  for (int k = 0; k < kBlock; ++k)
    if (e0 + k < n) m = max(m, abs_bits(W[e0 + k]));
  return __uint_as_float(m);
}

__global__ __launch_bounds__(256) void k_dq_psum(const float* __restrict__ W, int64_t n,
                                                 double* __restrict__ psum) {
  __shared__ float s_c1[kGroup];
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t b = (int64_t)blockIdx.x * kGroup + threadIdx.x;
  s_c1[threadIdx.x] = b < nb ? dq_block_c1(W, n, b) : 0.0f;
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int i = 0; i < kGroup; ++i) sum += (double)s_c1[i];   // increasing block order
    psum[blockIdx.x] = sum;
  }
}

__global__ void k_dq_mean(const double* __restrict__ psum, int64_t ng, int64_t nb,
                          float* __restrict__ scale2) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  double tot = 0.0;
  for (int64_t g = 0; g < ng; ++g) tot += psum[g];              // increasing group order
  scale2[ng] = (float)(tot / (double)nb);
}

// Largest E4M3 value of a 7-bit magnitude code, as fp64.
__device__ __forceinline__ double e4m3_mag(int code) {
  const int e = code >> 3, m = code & 7;
  return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

__global__ __launch_bounds__(256) void k_dq_second(const float* __restrict__ W, int64_t n,
                                                   uint8_t* __restrict__ scale8,
                                                   float* __restrict__ scale2, int dq) {
#pragma clang fp contract(off)
  __shared__ uint32_t s_red[4];
  const int t = threadIdx.x;
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  const int64_t b = (int64_t)blockIdx.x * kGroup + t;
  const float mu = scale2[ng];
  const float c1 = b < nb ? dq_block_c1(W, n, b) : 0.0f;
  const float cp = b < nb ? c1 - mu : 0.0f;                     // one fp32 rounding
  // group max |c'| (bit order of non-negative floats)
  uint32_t m = abs_bits(cp);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if ((t & 63) == 0) s_red[t >> 6] = m;
  __syncthreads();
  m = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
  const double top = dq == 1 ? 127.0 : 448.0;
  // correctly rounded fp32 quotient (fp64 quotient of fp32 values, rounded once more)
  const float step = (float)((double)__uint_as_float(m) / top);
  const double sd = (double)step, x = fabs((double)cp);
  uint32_t code = 0;
  if (step > 0.0f) {
    if (dq == 1) {
      // q = number of half-steps strictly below |c'|, at most 127 (exact in fp64)
      int q = (int)floor(x / sd + 0.5);
      q = q < 0 ? 0 : (q > 127 ? 127 : q);
      while (q > 0 && !(x > (2.0 * q - 1.0) * sd * 0.5)) --q;
      while (q < 127 && x > (2.0 * q + 1.0) * sd * 0.5) ++q;
      code = (uint32_t)(uint8_t)(int8_t)(cp < 0.0f ? -q : q);
    } else {
      // k = number of E4M3 midpoints strictly below |c'|/step (binary search on
      // exact thresholds), a tie going to the even code
      int lo = 0, hi = 126;                                       // answer in [0, 126]
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        const double thr = 0.5 * (e4m3_mag(mid) + e4m3_mag(mid + 1)) * sd;
        if (x > thr) lo = mid + 1; else hi = mid;
      }
      int k = lo;
      if (k < 126 && x == 0.5 * (e4m3_mag(k) + e4m3_mag(k + 1)) * sd && ((k + 1) & 1) == 0) ++k;
      code = (uint32_t)k | ((cp < 0.0f && k != 0) ? 0x80u : 0u);
    }
  }
  if (b < nb) scale8[b] = (uint8_t)code;
  if (t == 0) scale2[blockIdx.x] = step;
}

hipError_t launch_dq_variant(const float* W, int64_t n, uint8_t* scale8, float* scale2, int dq,
                             double* psum, hipStream_t st) {
  const int64_t nb = (n + kBlock - 1) / kBlock;
  const int64_t ng = (nb + kGroup - 1) / kGroup;
  if (ng == 0 || dq == 0) return hipSuccess;
  launch(k_dq_psum, dim3((unsigned)ng), dim3(256), 0, st, W, n, psum);
  launch(k_dq_mean, dim3(1), dim3(64), 0, st, psum, ng, nb, scale2);
  launch(k_dq_second, dim3((unsigned)ng), dim3(256), 0, st, W, n, scale8, scale2, dq);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
// Workgroups per CU.  While the fp32 input stays in the 256 MB MALL the
// quantizer runs three groups per CU (registers fitted to six waves per
// SIMD: 80 VGPRs); a launch that streams more than kQuantStreamBytes from
// HBM runs two (five waves per SIMD: 85 VGPRs), whose fewer, longer bursts
// stream better.  Measured on one box against two per CU: 4096² 1–9 %
// faster, 11008×4096 4–5 %, 8192² (268 MB) 1 %; with three per CU
// 12288×8192 was 7 % and 22016×8192 9 % slower.  The streaming launch also
// stores its code words non-temporally: 22016×8192 4–6 % and 12288×8192 4 %
// faster, the seven 65B-style tensors 3–5 % (non-temporal loads of W were
// 12 % slower, non-temporal 8-bit scales no faster, and the hint changed
// nothing on the shapes that stay in the MALL).
constexpr int64_t kQuantStreamBytes = 320ll << 20;
static bool quant_streams(int64_t groups) { return groups * (int64_t)kGroupElems * 4 > kQuantStreamBytes; }

hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale8,
                           float* scale2, int32_t* flags, int fmt, hipStream_t st) {
  const int64_t ng = (n + kGroupElems - 1) / kGroupElems;
  if (ng == 0) return hipSuccess;
  const EncodeGuide& eg = host_encode_guide(fmt);
  if (eg.zero_cell < 0) return hipErrorInvalidValue;
  if (quant_streams(ng))
    launch(k_quantize<5, true>, dim3((unsigned)ng), dim3(64 * kQuantWaves), 0, st, W, n, codes, scale8, scale2,
           flags, host_codebook(fmt), eg);
  else
    launch(k_quantize<6, false>, dim3((unsigned)ng), dim3(64 * kQuantWaves), 0, st, W, n, codes, scale8, scale2,
           flags, host_codebook(fmt), eg);
  return hipGetLastError();
}

hipError_t launch_quantize_grouped(const QuantJobs& jobs, int32_t* flags, int fmt, hipStream_t st) {
  if (jobs.count < 1 || jobs.count > kMaxQuantJobs) return hipErrorInvalidValue;
  const QuantJob& last = jobs.j[jobs.count - 1];
  const int64_t groups = last.g0 + (last.n + kGroupElems - 1) / kGroupElems;
  if (groups == 0) return hipSuccess;
  if (groups > 0x7FFFFFFF) return hipErrorInvalidValue;
  const EncodeGuide& eg = host_encode_guide(fmt);
  if (eg.zero_cell < 0) return hipErrorInvalidValue;
  if (quant_streams(groups))
    launch(k_quantize_grouped<5, true>, dim3((unsigned)groups), dim3(64 * kQuantWaves), 0, st, jobs, flags,
           host_codebook(fmt), eg);
  else
    launch(k_quantize_grouped<6, false>, dim3((unsigned)groups), dim3(64 * kQuantWaves), 0, st, jobs, flags,
           host_codebook(fmt), eg);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scale8, const float* scale2,
                          int64_t n, bool bf16, void* out, const Codebook& cb, hipStream_t st,
                          int dq) {
  const int64_t n8 = (n + 7) / 8;
  if (n8 == 0) return hipSuccess;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (bf16)
    launch(k_dequant<true>, dim3((unsigned)blocks), dim3(256), 0, st, codes, scale8,
                       scale2, n, out, cb, dq);
  else
    launch(k_dequant<false>, dim3((unsigned)blocks), dim3(256), 0, st, codes, scale8,
                       scale2, n, out, cb, dq);
  return hipGetLastError();
}

}  // namespace qlora
