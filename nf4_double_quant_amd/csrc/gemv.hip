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
#include <algorithm>

#include "kernels.h"

namespace qlora {

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (s16x4 __attribute__((address_space(3)))*)(p));
}

// Split-K planes of T = X·A for M <= 16: workgroup (z, c) sums k in
// [512 z, 512 z + 512) for the adapter columns [64 c, 64 c + 64).  With one
// adapter per token (adapter != null) workgroup layer blockIdx.z serves the
// single row blockIdx.z with that row's adapter.
constexpr int kPrepK = 512;
constexpr int kPrepStride = 80;  // bf16 per LDS row: 64 + 16 pad, conflict-free transposed reads

__global__ __launch_bounds__(256) void k_lora_down_small(const uint16_t* __restrict__ X, int M,
                                                         int64_t d, const uint16_t* __restrict__ A,
                                                         int r, float* __restrict__ Tpart,
                                                         const int32_t* __restrict__ adapter,
                                                         int n_ad) {
  __shared__ __attribute__((aligned(16))) uint16_t s_a[kPrepK * kPrepStride];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t k0 = (int64_t)blockIdx.x * kPrepK;
  const int c0 = blockIdx.y * 64;
  const int m = lane & 15, g = lane >> 4, s = lane & 15;
  int only = -1;                                   // the one row served, or -1 for all
  if (adapter != nullptr) {
    only = (int)blockIdx.z;
    const int a = adapter[only];
    if (a < 0 || a >= n_ad) {                      // no adapter: T[only] = 0 (whole workgroup)
      if (t < 64 && c0 + t < r) Tpart[((int64_t)blockIdx.x * M + only) * r + c0 + t] = 0.0f;
      return;
    }
    A += (int64_t)a * d * r;
  }
  // this lane's activations for its four 32-wide k steps, requested before
  // the adapter tile so that both arrive in one round trip.  Every load is
  // unconditional (offsets outside a buffer read 0): a branch around a load
  // would make the compiler wait for all earlier loads before the next one.
  // (32-bit offsets from descriptors based at this slice: M·d and 512·r
  // elements are far below 2^31)
  const int kn = (int)min<int64_t>(kPrepK, d - k0);    // valid k of the slice
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + k0), (short)0, (int)(((int64_t)(M - 1) * d + kn) * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(A + k0 * r), (short)0, kn * r * 2, 0x00020000);
  constexpr uint32_t kOff = 0x7FFFFFF0u;           // an offset every descriptor rejects
  const uint32_t d32 = (uint32_t)d;
  uint4 xv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int kx = (w * 4 + q) * 32 + 8 * g;        // within the slice
    const bool ok = m < M && kx < kn && (only < 0 || m == only);
    xv[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                          rx, (int)(ok ? ((uint32_t)m * d32 + (uint32_t)kx) * 2u : kOff), 0, 0));
  }
  // stage A[k0:k0+512][c0:c0+64] (zeros outside); all 16 loads of a thread
  // are in flight before the first store
  {
    uint4 v[kPrepK * 8 / 256];
#pragma unroll
    for (int u = 0; u < kPrepK * 8 / 256; ++u) {
      const int i = u * 256 + t, row = i >> 3, ch = i & 7;
      const int col = c0 + ch * 8;
      const bool ok = row < kn && col < r;
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                           ra, (int)(ok ? (uint32_t)(row * r + col) * 2u : kOff), 0, 0));
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
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int kq = w * 4 + q;                    // 32-wide k step inside the slice
    const bf16x8 a = __builtin_bit_cast(bf16x8, xv[q]);
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
    if (mm < M && c0 + cc < r && (only < 0 || mm == only)) {
      const float v = red[(0 * 16 + mm) * 64 + cc] + red[(1 * 16 + mm) * 64 + cc] +
                      red[(2 * 16 + mm) * 64 + cc] + red[(3 * 16 + mm) * 64 + cc];
      Tpart[((int64_t)blockIdx.x * M + mm) * r + c0 + cc] = v;
    }
  }
}

constexpr int kGemvMaxWaves = 12;
constexpr int kGemvMaxLds = 65536;

struct GemvArgs {
  const uint16_t* X;    // [M][d]
  const uint8_t* codes; const uint8_t* scale8; const float* scale2;
  const float* Tpart;   // [tsplits][M][r]
  const uint16_t* B;    // [r][o]
  uint16_t* Y;          // [M][o]
  float* T_out;         // [M][r] or null
  int64_t d, o;
  int M, r, tsplits;
  int t_regs;           // 1: T planes take the register path (16 tokens, host-checked LDS size)
  float s;
  Codebook cb;
  const int32_t* adapter;  // one adapter per token ([M]), or null
  int n_ad;
  float s_ad[kMaxAdapters];
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

// One 4-block group of a wave: lane (n = lane%16, q = lane/16) holds the 64
// codes of one block of row n.
struct GemvCodes {
  uint4 c0, c1;
  uint32_t q8;          // the dword of scale8 holding the block's byte
  float step;
};

// Shared-memory layout of k_gemv, computed identically on host and device.
struct GemvSmem {
  int x, part, tp, t, b, bytes;   // byte offsets of each region, total size
};
__host__ __device__ inline GemvSmem gemv_smem(int nw, int mx, int M, int r, int tplanes,
                                              bool t_regs) {
  GemvSmem s;
  int off = 0;
  s.x = off;    off += nw * (mx + 1) * 36 * 16;              // staged activations + a zero row
  s.part = off; off += nw * 16 * 17 * 4;                      // per-wave partial sums
  s.tp = off;   off += t_regs ? tplanes * M * r * 4 : 0;      // T planes (register path)
  s.t = off;    off += M * r * 4;                             // T = X·A
  s.b = off;    off += r * 16 * 4;                            // B[:, n0:n0+16]
  s.bytes = off;
  return s;
}

// The waves of a workgroup share its 16 rows and split the reduction in
// 256-weight groups (4 blocks): wave w takes groups w, w + nw, ....  The
// host picks nw = ceil(groups / 4) up to kGemvMaxWaves, so for d <= 12288
// every wave owns at most four groups and issues all its loads at once.
//
// The activations reach the MFMA A operand through a wave-private LDS
// tile: the operand lane (m, q) needs the 128 bytes of row m under its
// block, while the wave loads the group's M×512 bytes as whole 1 KB runs
// (ceil(M/2) 16-byte loads per lane; MX, the largest M the instance serves,
// sizes the tile) and redistributes them.  For MX <= 4 four groups of codes
// and activations are in flight; the 16-token instance keeps activations
// one group ahead and, holding 8 staged chunks per lane, runs at most 8
// waves with more registers each.
__host__ __device__ constexpr int gemv_max_waves(int mx) { return mx == 16 ? 8 : kGemvMaxWaves; }

template <int MX>
__global__ __launch_bounds__(gemv_max_waves(MX) * 64) void k_gemv(GemvArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  constexpr int kNX = (MX * 32 + 63) / 64;                  // activation loads per lane per group
  constexpr int kXRow = 36;                                 // staged row: 4 blocks × (8 + 1 pad) uint4
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int nw = (int)(blockDim.x >> 6), nthr = (int)blockDim.x;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const uint32_t nblk = (uint32_t)(p.d / kBlock);
  const uint32_t ngrp = (nblk + 3) / 4;
  const int nl = lane & 15, q = lane >> 4, m = lane & 15;
  const int64_t n = n0 + nl;
  const bool multi = p.adapter != nullptr;
  const bool lora = p.r > 0 && (multi || p.s != 0.0f);
  const bool want_t = lora || (p.T_out != nullptr && blockIdx.x == 0);
  const int tpl = p.tsplits * p.M * p.r;                    // T-plane elements
  const bool t_regs = want_t && p.t_regs != 0;
  const bool b_regs = MX == 16 && lora && !multi && p.r * 8 <= 2 * nthr;
  const GemvSmem L = gemv_smem(nw, MX, p.M, p.r, p.tsplits, p.t_regs != 0);
  float* s_part = reinterpret_cast<float*>(smem + L.part);  // [nw][16][17]
  float* s_tp = reinterpret_cast<float*>(smem + L.tp);      // [tsplits][M][r]
  float* s_T = reinterpret_cast<float*>(smem + L.t);        // [M][r]
  float* s_B = reinterpret_cast<float*>(smem + L.b);        // [r][16]
  uint4* s_x = reinterpret_cast<uint4*>(smem + L.x) + w * ((MX + 1) * kXRow);

  // ---- every global load is unconditional (offsets past a buffer read 0),
  // so the wait before each use counts exactly the loads issued after it.
  // Offsets are 32-bit (the host bounds the sizes); rows past o and blocks
  // past the row end read 0 (a zero table and zero activations contribute
  // nothing).
  const uint32_t nbt = (uint32_t)(p.o * nblk);            // blocks in Wq (a multiple of 8)
  const GRsrc rc = grsrc(p.codes, (int64_t)nbt * 32);
  const GRsrc rs8 = grsrc(p.scale8, nbt);
  const GRsrc rs2 = grsrc(p.scale2, (int64_t)((nbt + kGroup - 1) / kGroup) * 4);
  const GRsrc rx = grsrc(p.X, (int64_t)p.M * p.d * 2);
  const GRsrc rt = grsrc(p.Tpart, t_regs ? (int64_t)tpl * 4 : 0);
  const GRsrc rb = grsrc(p.B, lora ? (int64_t)p.r * p.o * 2 : 0);

  // 16 tokens: T split-K planes and B[:, n0:n0+16] for the epilogue,
  // requested before the weight stream so that no later wait holds it up.
  // The instances for up to 4 tokens read both in the epilogue instead
  // (about 1 µs less per 7B MLP at 1 and 2 tokens, the same at 4).
  float tp[4];
  uint32_t bb[2];
  if (t_regs) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = t + u * nthr;
      tp[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                            rt, (int)(e < tpl ? (uint32_t)e * 4 : kGOob), 0, 0));
    }
  }
  if (b_regs) {
    // dword i: row j = i/8 of B, columns n0 + 2(i%8), +1 (o is a multiple of 8)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = t + u * nthr, j = i >> 3, c2 = i & 7;
      const bool ok = i < p.r * 8 && n0 + 2 * c2 < p.o;
      bb[u] = __builtin_amdgcn_raw_buffer_load_b32(
          rb, (int)(ok ? ((uint32_t)j * (uint32_t)p.o + (uint32_t)n0 + 2 * c2) * 2 : kGOob), 0, 0);
    }
  }

  if (lane < kXRow) s_x[MX * kXRow + lane] = make_uint4(0, 0, 0, 0);
  const bool row_ok = n < p.o;
  const uint32_t brow = row_ok ? (uint32_t)n * nblk : 0u;
  // the 8-bit scale of block b is byte b%4 of dword b/4; b%4 = (brow + q)%4
  // for every block this lane touches
  const uint32_t sh8 = ((brow + (uint32_t)q) & 3u) * 8u;
  const int niter = (int)ngrp > w ? ((int)ngrp - w + nw - 1) / nw : 0;
  // group of the wave's slot `it`
  auto group_of = [&](int it) -> uint32_t {
    return (uint32_t)(w + it * nw);
  };
  auto load_codes = [&](int it, GemvCodes& c) {
    const uint32_t kb = group_of(it) * 4 + q;
    const bool ok = row_ok && kb < nblk;
    const uint32_t b = brow + kb;
    c.c0 = gload16(rc, ok ? b * 32 : kGOob);
    c.c1 = gload16(rc, ok ? b * 32 + 16 : kGOob);
    c.q8 = __builtin_amdgcn_raw_buffer_load_b32(rs8, (int)(ok ? b & ~3u : kGOob), 0, 0);
    c.step = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs2, (int)(ok ? (b / kGroup) * 4 : kGOob), 0, 0));
  };
  // activations of slot `it` in the staged layout: chunk c = u·64 + lane
  // holds row c/32, 8 values at k = 8·(c%32) of the group (1 KB per load)
  auto load_x = [&](int it, uint4 (&x)[kNX]) {
    const uint32_t g = group_of(it);
#pragma unroll
    for (int u = 0; u < kNX; ++u) {
      const int c = u * 64 + lane, mm = c >> 5, kc = c & 31;
      const bool ok = mm < p.M && g * 4 + (kc >> 3) < nblk;
      const uint32_t off = ((uint32_t)mm * (uint32_t)p.d + g * 256 + kc * 8) * 2;
      x[u] = gload16(rx, ok ? off : kGOob);
    }
  };
  // staged activations -> operand layout, through this wave's LDS tile
  // (row stride and a pad after every block make the reads conflict-free)
  auto operands = [&](const uint4 (&x)[kNX], uint4 (&xa)[8]) {
#pragma unroll
    for (int u = 0; u < kNX; ++u) {
      const int c = u * 64 + lane, mm = c >> 5, kc = c & 31;
      if (mm < MX) s_x[mm * kXRow + kc + (kc >> 3)] = x[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // operand rows m >= M read zeros: rows M..MX-1 were staged from
    // out-of-range loads, and row MX is the zero row
    const int mr = m < MX ? m : MX;
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = s_x[mr * kXRow + q * 9 + j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // one group: the block's table, its 64 codes expanded, 8 MFMAs
  auto compute_ops = [&](const GemvCodes& c, const uint4 (&xa)[8]) {
    Lut lut;
    const float q8 = (float)__builtin_amdgcn_ubfe(c.q8, sh8, 8);
    build_lut(p.cb, q8 * c.step, lut);            // ĉ = fl32(q8·step)
    const uint32_t cw[8] = {c.c0.x, c.c0.y, c.c0.z, c.c0.w, c.c1.x, c.c1.y, c.c1.z, c.c1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[j]), expand8(lut, cw[j]),
                                                    acc, 0, 0, 0);
  };
  auto compute = [&](const GemvCodes& c, const uint4 (&x)[kNX]) {
    uint4 xa[8];
    operands(x, xa);
    compute_ops(c, xa);
  };

  // Four groups of codes in flight; the loop runs while more chunks follow
  // the one held, and the last four slots are computed after it with no
  // further loads (slots past niter hold zeros; branching around them costs
  // more than the few wasted ones).
  GemvCodes c0, c1, c2, c3;
  if constexpr (MX <= 4) {
    uint4 x0[kNX], x1[kNX], x2[kNX], x3[kNX];
    // (the scheduling barriers keep each group's loads together, in order,
    // so that the wait for a group never covers a later one)
    load_codes(0, c0); load_x(0, x0); __builtin_amdgcn_sched_barrier(0);
    load_codes(1, c1); load_x(1, x1); __builtin_amdgcn_sched_barrier(0);
    load_codes(2, c2); load_x(2, x2); __builtin_amdgcn_sched_barrier(0);
    load_codes(3, c3); load_x(3, x3); __builtin_amdgcn_sched_barrier(0);
    int it = 0;
    for (; it + 4 < niter; it += 4) {
      compute(c0, x0); load_codes(it + 4, c0); load_x(it + 4, x0); __builtin_amdgcn_sched_barrier(0);
      compute(c1, x1); load_codes(it + 5, c1); load_x(it + 5, x1); __builtin_amdgcn_sched_barrier(0);
      compute(c2, x2); load_codes(it + 6, c2); load_x(it + 6, x2); __builtin_amdgcn_sched_barrier(0);
      compute(c3, x3); load_codes(it + 7, c3); load_x(it + 7, x3); __builtin_amdgcn_sched_barrier(0);
    }
    compute(c0, x0);
    compute(c1, x1);
    compute(c2, x2);
    compute(c3, x3);
  } else {
    // 16 tokens: the tile takes a group's activations as soon as they
    // arrive, so registers hold only the next group's chunks (one group
    // ahead) besides the operands in use, and codes run two groups ahead;
    // that keeps three waves per SIMD.  Rows of the tile are rewritten only
    // after this wave's reads of the previous group (its LDS operations run
    // in order).
    uint4 xn[kNX];
    auto stage_write = [&]() {
#pragma unroll
      for (int u = 0; u < kNX; ++u) {
        const int c = u * 64 + lane, mm = c >> 5, kc = c & 31;
        s_x[mm * kXRow + kc + (kc >> 3)] = xn[u];
      }
    };
    auto stage_read = [&](uint4 (&xa)[8]) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[j] = s_x[m * kXRow + q * 9 + j];
    };
    auto step = [&](int it, GemvCodes& c) {
      uint4 xa[8];
      stage_read(xa);                  // group it
      stage_write();                   // group it + 1
      load_x(it + 2, xn);
      compute_ops(c, xa);
      load_codes(it + 2, c);
    };
    load_codes(0, c0); load_x(0, xn); __builtin_amdgcn_sched_barrier(0);
    load_codes(1, c1); __builtin_amdgcn_sched_barrier(0);
    stage_write();
    load_x(1, xn);
    for (int it = 0; it < niter; it += 2) {
      step(it, c0);
      if (it + 1 >= niter) break;
      step(it + 1, c1);
    }
  }

  // ---- epilogue: Y = Σ partials + s·T·B
  // lane holds rows m = 4*(lane/16) + v of column n = lane%16
#pragma unroll
  for (int v = 0; v < 4; ++v) s_part[(w * 16 + 4 * (lane >> 4) + v) * 17 + (lane & 15)] = acc[v];
  if (t_regs) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = t + u * nthr;
      if (e < tpl) s_tp[e] = tp[u];
    }
  }
  if (b_regs) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = t + u * nthr;
      if (i < p.r * 8) {
        s_B[2 * i] = bf16_to_f32((uint16_t)(bb[u] & 0xFFFFu));
        s_B[2 * i + 1] = bf16_to_f32((uint16_t)(bb[u] >> 16));
      }
    }
  } else if (lora && !multi) {
    for (int i = t; i < p.r * 16; i += nthr) {
      const int j = i >> 4, c = i & 15;
      s_B[i] = n0 + c < p.o ? bf16_to_f32(p.B[(int64_t)j * p.o + n0 + c]) : 0.0f;
    }
  }
  if (want_t && !t_regs) {
    const int64_t plane = (int64_t)p.M * p.r;
    for (int i = t; i < p.M * p.r; i += nthr) {
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
  __syncthreads();
  if (t_regs) {
    // T planes summed in a fixed order
    const int plane = p.M * p.r;
    for (int i = t; i < plane; i += nthr) {
      float sum = 0.0f;
      for (int z = 0; z < p.tsplits; ++z) sum += s_tp[z * plane + i];
      s_T[i] = sum;
      if (p.T_out != nullptr && blockIdx.x == 0) p.T_out[i] = sum;
    }
    __syncthreads();
  }
  for (int i = t; i < p.M * 16; i += nthr) {
    const int mm = i >> 4, nc = i & 15;
    const int64_t nn = n0 + nc;
    if (nn < p.o) {
      float y = 0.0f;
      for (int ww = 0; ww < nw; ++ww) y += s_part[(ww * 16 + mm) * 17 + nc];
      if (lora && !multi) {
        float l = 0.0f;
        for (int j = 0; j < p.r; ++j) l += s_T[mm * p.r + j] * s_B[j * 16 + nc];
        y += p.s * l;
      } else if (lora) {
        // this row's adapter (same products, same order as the single case)
        const int a = p.adapter[mm];
        if (a >= 0 && a < p.n_ad) {
          const uint16_t* Ba = p.B + ((int64_t)a * p.r) * p.o + nn;
          float l = 0.0f;
          for (int j = 0; j < p.r; ++j) l += s_T[mm * p.r + j] * bf16_to_f32(Ba[(int64_t)j * p.o]);
          y += p.s_ad[a] * l;
        }
      }
      p.Y[(int64_t)mm * p.o + nn] = bf16_bits(y);
    }
  }
}

int gemv_tsplits(int64_t d) { return (int)((d + kPrepK - 1) / kPrepK); }

namespace {
struct GemvPlan {
  int nw, mx, rr;
  bool t_regs;
  int lds;
};
GemvPlan gemv_plan(int M, int64_t d, int r, bool lora, bool want_t) {
  GemvPlan g{};
  const int64_t nblk = d / kBlock;
  const int64_t chunks = (nblk + 15) / 16;
  g.mx = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 16;
  g.rr = r;
  const int ts = gemv_tsplits(d);
  // as many waves as four-group chunks, up to kGemvMaxWaves, fewer when the
  // staged activations of that many waves would not fit the shared memory
  for (g.nw = (int)std::min<int64_t>(gemv_max_waves(g.mx), std::max<int64_t>(1, chunks)); ; --g.nw) {
    g.t_regs = want_t && g.mx == 16 && (int64_t)ts * M * r <= 4 * g.nw * 64;
    if (g.t_regs && gemv_smem(g.nw, g.mx, M, r, ts, true).bytes > kGemvMaxLds) g.t_regs = false;
    g.lds = gemv_smem(g.nw, g.mx, M, r, ts, g.t_regs).bytes;
    if (g.lds <= kGemvMaxLds || g.nw == 1) break;
  }
  (void)lora;
  return g;
}
}  // namespace

bool gemv_fits(int64_t M, int64_t d, int64_t r) {
  if (M < 1 || M > kGemvMaxTokens || r > kMaxGemvRank || d % kBlock != 0) return false;
  return gemv_plan((int)M, d, (int)r, r > 0, r > 0).lds <= kGemvMaxLds;
}

hipError_t launch_gemv_tdown(const uint16_t* X, int M, int64_t d, const uint16_t* A, int r,
                             float* Tpart, hipStream_t st, const int32_t* adapter, int n_ad) {
  if (r <= 0) return hipSuccess;
  launch(k_lora_down_small, dim3(gemv_tsplits(d), (r + 63) / 64, adapter != nullptr ? M : 1),
         dim3(256), 0, st, X, M, d, A, r, Tpart, adapter, n_ad);
  return hipGetLastError();
}

hipError_t launch_gemv_fwd(const uint16_t* X, int M, int64_t d, const uint8_t* codes,
                           const uint8_t* scale8, const float* scale2, int64_t o,
                           const uint16_t* A, const uint16_t* B, int r, float s, uint16_t* Y,
                           float* T_out, float* Tpart, const Codebook& cb, hipStream_t st,
                           const int32_t* adapter, int n_ad, const float* s_ad, bool tdown) {
  const int ts = gemv_tsplits(d);
  const bool multi = adapter != nullptr;
  if (multi && (n_ad < 1 || n_ad > kMaxAdapters || s_ad == nullptr)) return hipErrorInvalidValue;
  const int rr = (r > 0 && (multi || s != 0.0f || T_out != nullptr)) ? r : 0;
  if (rr > 0 && tdown) {
    hipError_t e = launch_gemv_tdown(X, M, d, A, rr, Tpart, st, adapter, n_ad);
    if (e != hipSuccess) return e;
  }
  const unsigned grid = (unsigned)((o + 15) / 16);
  const bool lora = rr > 0 && (multi || s != 0.0f);
  const GemvPlan g = gemv_plan(M, d, rr, lora, lora || T_out != nullptr);
  if (g.lds > kGemvMaxLds) return hipErrorInvalidConfiguration;
  GemvArgs p{X, codes, scale8, scale2, Tpart, B, Y, T_out, d, o, M, rr, ts, g.t_regs ? 1 : 0, s, cb,
             adapter, multi ? n_ad : 0, {}};
  for (int i = 0; multi && i < n_ad; ++i) p.s_ad[i] = s_ad[i];
  const size_t lds = (size_t)g.lds;
  switch (g.mx) {
    case 1: launch(k_gemv<1>, dim3(grid), dim3(64 * g.nw), lds, st, p); break;
    case 2: launch(k_gemv<2>, dim3(grid), dim3(64 * g.nw), lds, st, p); break;
    case 4: launch(k_gemv<4>, dim3(grid), dim3(64 * g.nw), lds, st, p); break;
    default: launch(k_gemv<16>, dim3(grid), dim3(64 * g.nw), lds, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace qlora
