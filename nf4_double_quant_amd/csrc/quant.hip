// Blockwise NF4 quantization with double quantization, and dequantization.
//
// Method: "074｜QLoRA：把大模型放进显存，再用小适配器改变它" §二 (NF4 codes,
// absmax per 64 weights, 8-bit first-level constants with one fp32
// second-level constant per 256 of them) and §三 (quantize the weights with
// the first-level constants, then quantize those constants).
//
// gfx950 design
//  * One workgroup per double-quant group (16384 weights = 64 KB of fp32):
//    the group's second-level constant needs every block's absmax, so the
//    whole group stays in VGPRs (16 float4 per lane) between the reduction
//    and the encode, and HBM is read exactly once.
//  * 16 lanes per 64-weight block, one float4 each: every load instruction
//    covers 1 KB contiguous.  The block absmax is a 16-lane xor-shuffle max
//    on the integer bits of |w| (integer order equals float order for
//    non-negative floats, and NaN/Inf land above every finite value, which
//    is how non-finite input is detected).
//  * Exact nearest-value encode without fp64 per weight: for each block the
//    15 decision points c1·mid_t are exact fp64 products; rounding each one
//    DOWN to fp32 gives a threshold th_t with  w > c1·mid_t  <=>  w > th_t
//    for every fp32 w.  A thread per block builds them once, as unsigned
//    keys with the order of the fp32 values, into shared memory; each weight
//    then takes a 4-level binary search that reads one threshold per level
//    and shifts the comparison's borrow into the code (two VALU operations).
//  * Codes are packed 8 per 32-bit word (byte j = code j | code j+4 << 4):
//    the two lanes holding a word's halves merge them with one shuffle, the
//    words are gathered in LDS and written out as 16-byte stores.
#include "kernels.h"

namespace qlora {

// Largest fp32 <= the exact (nonzero) fp64 value p.
__device__ __forceinline__ float round_down_f32(double p) {
  float f = (float)p;
  if ((double)f > p) {
    int32_t bits = __float_as_int(f);
    f = __int_as_float(bits > 0 ? bits - 1 : bits + 1);  // toward −inf
  }
  return f;
}

// Unsigned key with the order of the fp32 values (-0 just below +0): for the
// thresholds used here, none of them -0, k(w) > k(t) exactly when w > t.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t b = __float_as_uint(x);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// 2k + (t < u): the borrow of t - u carried into k + k (two VALU operations)
__device__ __forceinline__ uint32_t bit_in(uint32_t k, uint32_t t, uint32_t u) {
  uint32_t d, r;
  asm("v_sub_co_u32 %0, vcc, %2, %3\n\tv_addc_co_u32 %1, vcc, %4, %4, vcc"
      : "=&v"(d), "=v"(r) : "v"(t), "v"(u), "v"(k) : "vcc");
  return r;
}

// max over the 16 lanes of a DPP row (rotations by 8, 4, 2, 1)
__device__ __forceinline__ uint32_t row_max16(uint32_t a) {
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x128, 0xF, 0xF, false));
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x124, 0xF, 0xF, false));
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x122, 0xF, 0xF, false));
  a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x121, 0xF, 0xF, false));
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

__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ W, int64_t n,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scale8,
                                                  float* __restrict__ scale2,
                                                  int32_t* __restrict__ flags, Codebook cb) {
  __shared__ __attribute__((aligned(16))) uint32_t s_thr[kGroup][16];   // threshold order keys
  __shared__ __attribute__((aligned(16))) uint32_t s_codes[kGroupElems / 8];
  __shared__ uint32_t s_c1[kGroup];
  __shared__ uint32_t s_red[4];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int sub = lane & 15, quad = lane >> 4;
  const int64_t g = blockIdx.x;
  const int64_t base = g * kGroupElems;
  const int64_t nb = (n + kBlock - 1) / kBlock;

  // ---- load the group (reads past n return 0) and take per-block absmax
  const Rsrc rw = rsrc(W + base, (min((int64_t)kGroupElems, n - base)) * 4);
  float4 v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bl = wave * 64 + j * 4 + quad;
    const int off = (bl * kBlock + sub * 4) * 4;
    v[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0));
  }
  uint32_t bad = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t a = max(max(abs_bits(v[j].x), abs_bits(v[j].y)), max(abs_bits(v[j].z), abs_bits(v[j].w)));
    a = row_max16(a);
    bad |= (a >= 0x7F800000u);
    if (sub == 0) s_c1[wave * 64 + j * 4 + quad] = a;
  }
  __syncthreads();

  // ---- second level: one thread per block
  const uint32_t c1_bits = s_c1[t];
  uint32_t m = c1_bits;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, 64));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  m = max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3]));
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
  if (b_glob < nb) scale8[b_glob] = (uint8_t)q;
  if (t == 0) scale2[g] = step;

  // decision thresholds of this block
  {
    float th[16];
    if (c1_bits == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) th[i] = i < 7 ? -1.0f : 0.0f;  // everything -> code 7
    } else {
#pragma unroll
      for (int i = 0; i < 15; ++i) th[i] = round_down_f32((double)c1 * cb.mid[i]);
      th[15] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s_thr[t][i] = order_key(th[i]);
  }
  __syncthreads();

  // ---- encode
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int bl = wave * 64 + j * 4 + quad;
    // binary search on order keys, level by level for the four weights:
    // k collects the code bits from the top, and each level reads the one
    // threshold it compares against (index 8k+3, 4k+1, 2k)
    const uint32_t* T = s_thr[bl];
    const uint32_t t7 = T[7];
    const uint32_t u[4] = {order_key(v[j].x), order_key(v[j].y), order_key(v[j].z), order_key(v[j].w)};
    uint32_t kk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) kk[e] = bit_in(0u, t7, u[e]);
#pragma unroll
    for (int lev = 0; lev < 3; ++lev) {
      uint32_t th[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) th[e] = T[lev == 0 ? 8 * kk[e] + 3 : lev == 1 ? 4 * kk[e] + 1 : 2 * kk[e]];
#pragma unroll
      for (int e = 0; e < 4; ++e) kk[e] = bit_in(kk[e], th[e], u[e]);
    }
    const uint32_t k0 = kk[0], k1 = kk[1], k2 = kk[2], k3 = kk[3];
    // lane `sub` holds codes 4·sub..4·sub+3 of the block: low nibbles of a
    // word for even sub, high nibbles for odd sub; neighbours merge by DPP
    const uint32_t half = (k0 | (k1 << 8) | (k2 << 16) | (k3 << 24)) << ((sub & 1) * 4);
    const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)half, 0xB1, 0xF, 0xF, false);
    if ((sub & 1) == 0) s_codes[bl * 8 + (sub >> 1)] = half | other;
  }
  __syncthreads();

  // ---- write the group's 8192 code bytes (stores past the buffer are dropped)
  const int64_t code_bytes = (n + 7) / 8 * 4;
  const int64_t cbase = g * (kGroupElems / 2);
  const Rsrc rcod = rsrc(codes + cbase, code_bytes - cbase);
  uint4 a = reinterpret_cast<const uint4*>(s_codes)[t * 2];
  uint4 b = reinterpret_cast<const uint4*>(s_codes)[t * 2 + 1];
  // The word holding code n-1 may end in codes past n; they are stored as 7,
  // the layout's padding, whatever a zero weight encodes to in this table.
  const int64_t nvalid = n - base;
  if (nvalid < kGroupElems && (nvalid & 7) != 0 && (nvalid >> 6) == t) {
    uint32_t keep = 0;
    for (int j = 0; j < (int)(nvalid & 7); ++j) keep |= 0xFu << (8 * (j & 3) + 4 * (j >> 2));
    const int wi = (int)((nvalid >> 3) & 7);
    uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k == wi) w[k] = (w[k] & keep) | (0x77777777u & ~keep);
    a = make_uint4(w[0], w[1], w[2], w[3]);
    b = make_uint4(w[4], w[5], w[6], w[7]);
  }
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, a), rcod, t * 32, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, b), rcod, t * 32 + 16, 0, 0);
  if (bad && flags != nullptr) flags[0] = flags[0] | 1;
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
  hipLaunchKernelGGL(k_dq_psum, dim3((unsigned)ng), dim3(256), 0, st, W, n, psum);
  hipLaunchKernelGGL(k_dq_mean, dim3(1), dim3(64), 0, st, psum, ng, nb, scale2);
  hipLaunchKernelGGL(k_dq_second, dim3((unsigned)ng), dim3(256), 0, st, W, n, scale8, scale2, dq);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
hipError_t launch_quantize(const float* W, int64_t n, uint8_t* codes, uint8_t* scale8,
                           float* scale2, int32_t* flags, const Codebook& cb, hipStream_t st) {
  const int64_t ng = (n + kGroupElems - 1) / kGroupElems;
  if (ng == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)ng), dim3(256), 0, st, W, n, codes, scale8,
                     scale2, flags, cb);
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
    hipLaunchKernelGGL(k_dequant<true>, dim3((unsigned)blocks), dim3(256), 0, st, codes, scale8,
                       scale2, n, out, cb, dq);
  else
    hipLaunchKernelGGL(k_dequant<false>, dim3((unsigned)blocks), dim3(256), 0, st, codes, scale8,
                       scale2, n, out, cb, dq);
  return hipGetLastError();
}

}  // namespace qlora
