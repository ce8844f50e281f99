// Fused NF4 dequant-GEMM for many tokens (gfx950):
//   forward   Y  = X·Ŵ  + (s·T)·B      with Ŵ = Wqᵀ, blocks of Wq run along k
//   backward  dX = dY·Ŵᵀ + (s·U)·Aᵀ    blocks of Wq run along n
// ("074｜QLoRA：把大模型放进显存，再用小适配器改变它" §一 for the layer and the
// input gradient through Ŵᵀ; §三: dequantize the needed weights to BF16 on
// demand, then compute base plus adapter output).
//
// Tile 512×128×64: 4 waves stacked along M, each 128×128 of fp32
// accumulators fed by v_mfma_f32_32x32x16_bf16.  Every weight is expanded
// once per workgroup, so the tall tile halves the expansion work per MFMA
// compared with 256×256.  Per k-step each of the 256 threads expands half of
// one 64-weight block: 16 code bytes, the block's 8-bit scale and group
// step, a 16-entry table bf16(V[k]·fl32(q8·step)) (exact fp32 products, the
// same bits as the standalone dequant), byte permutes, and 64 bytes of bf16
// written to LDS.  The activation tile goes memory -> LDS directly
// (buffer_load ... lds) one k-step ahead, its instructions spread between
// the MFMAs; each wave loads exactly the 128 rows it multiplies, so the one
// barrier per k-step publishes only the expanded weights and each wave
// waits for its own DMA.  Codes are loaded one k-step ahead of their
// expansion.  The finished block leaves through the idle activation stages
// as whole 256-byte rows.
//
//  * forward: the weight tile is [n][k] like the activation tile (k-major
//    rows, XOR-swizzled 16-byte chunks), read with ds_read_b128;
//  * backward: a block is 64 consecutive n of one k, so the tile is stored
//    [k][n] (16-byte chunks placed by chunk_tr) and
//    the MFMA B operand is gathered with ds_read_b64_tr_b16, four k of one n
//    per lane per read.
// The adapter term is one (or a few) extra k-steps over [s·T ‖ B] or
// [s·U ‖ A], accumulated into the same registers, so Y and dX are rounded
// to bf16 once.  B [r][o] is n-major like the backward weight tile and A
// [d][r] k-major like the forward one, so neither needs a transposed copy.
// Workgroups are numbered so that each XCD (round-robin dispatch over 8)
// works on a contiguous band of output tiles.
#include <type_traits>

#include <stddef.h>

#include "kernels.h"

namespace qlora {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 512, kBN = 128, kBK = 64;
// Waves per workgroup: 4 (one per SIMD, 128 rows each, accumulators in
// AGPRs) or 8 (two per SIMD, 64 rows each).  Both measure the same on the
// 4096-square layer; 4 keeps the register budget simple.
constexpr int kWaves = 4;

// XOR swizzle of the 16-byte chunks of a 128-byte LDS row: eight consecutive
// rows, and rows 8 apart, land in different chunks.  It depends on row % 32
// only.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 3); }

// Position of 16-byte chunk c (0..15) in row k of a [k][n] tile (256-byte
// rows): c ^ h(k mod 4) with h = 0, 3, 6, 5, then bit 3 flipped by bit 1 of
// c and by bit 2 of k (a bijection of the chunks of each row).  A transposed
// fragment read covers 4 consecutive rows × 2 adjacent chunks per 16 lanes,
// and the two 16-lane groups of a half-wave chunks 2 apart; an expansion
// write covers rows k..k+3 (8 lanes) or k..k+7 (16 lanes) with 2 chunks 4
// apart.  The positions differ mod 8 within 16 lanes of a read and 8 lanes
// of a write, and mod 16 within 32 and 16 lanes, so neither conflicts with
// 32 banks nor with 64.
__device__ __forceinline__ int chunk_tr(int k, int c) {
  return c ^ (((k & 3) << 1) ^ (k & 3)) ^ (((k >> 2) & 1) << 3) ^ ((c & 2) << 2);
}

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
  ReduceJob tail_a, tail_b;          // plane sums done after the tiles (count 0: none)
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

// Publish LDS written by this workgroup (ds_write and, after an explicit
// vmcnt wait, buffer_load ... lds) without waiting for other vector-memory
// loads still in flight: the fences cover the LDS address space only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <bool kTransW, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void k_qgemm(QGemmArgs p) {
  constexpr int kT = 64 * kWaves;        // threads
  constexpr int kWR = kBM / kWaves;      // activation rows per wave
  constexpr int kI = kWR / 32;           // 32-row MFMA blocks per wave
  constexpr int kQ = kWR / 8;            // DMA instructions per wave per k-step
  constexpr int kWT = kBN * kBK / kT;    // weights one thread expands per k-step
  constexpr int kCW = kWT / 8;           // code words (8 codes each) per thread
  constexpr int kParts = kBlock / kWT;   // threads sharing one 64-weight block
  static_assert(kCW == 2 || kCW == 4, "a thread expands 16 or 32 weights");

  // stages in separate arrays (the compiler can tell writes to the idle
  // stage from reads of the busy one); 2 × 64 KB + 2 × 16 KB = 160 KB
  __shared__ __attribute__((aligned(16))) uint16_t sA0[kBM * kBK], sA1[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t sB0[kBN * kBK], sB1[kBN * kBK];

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wq = __builtin_amdgcn_readfirstlane(w);

  // XCD-aware tile order: dispatch sends workgroup i to XCD i % 8; give each
  // XCD a contiguous run of tiles (row-major over the n-tiles).
  const int ntn = (int)((p.N + kBN - 1) / kBN), ntm = (int)((p.M + kBM - 1) / kBM);
  const int T = ntn * ntm;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = T >> 3, rem = T & 7;
  const int v = xcd * per + min(xcd, rem) + slot;
  const int64_t m0 = (int64_t)(v / ntn) * kBM, n0 = (int64_t)(v % ntn) * kBN;
  const int mrows = (int)min((int64_t)kBM, p.M - m0);
  const int nk2 = (int)((p.K2 + kBK - 1) / kBK);

  // ---- activation tile [512][64]: memory -> LDS (buffer_load ... lds).  Each
  // wave instruction q fills 1 KB = 8 rows; lane l lands at byte 16·l, i.e.
  // row 8q + l/8 of the wave's rows and physical chunk l%8, so it fetches
  // logical chunk (l%8) ^ swz(row).  The descriptor's base moves with k0, so
  // a lane's offset is fixed: row·lda + 8·chunk elements, or an offset every
  // descriptor rejects for rows past M (those read 0).  Columns are checked
  // against klim only with kCheck (a k-step that reaches past K); without it
  // columns past K read the next row, which is in range but must not be used.
  const uint32_t lda2b = (uint32_t)p.lda * 2u;
  auto dma_a = [&](auto check_tag, const uint16_t* base, uint32_t ld2b, int64_t k0, int64_t klim,
                   uint16_t* sa, int qlo = 0, int qhi = kBM / 8) {
    constexpr bool kCheck = decltype(check_tag)::value;
    const int64_t left = (int64_t)mrows * (ld2b / 2) - k0;
    const Rsrc src = rsrc(base + k0, left * 2);
    const int krem = (int)min<int64_t>(klim - k0, kBK);   // columns of this step in range
    // The wave's LDS rows start at sa + wrow; hiding wrow from the optimiser
    // keeps it from holding every destination address of both stages in
    // SGPRs across the loop (each instruction then adds its constant to M0).
    int wrow = wq * kWR * kBK;
    asm volatile("" : "+s"(wrow));
    uint16_t* sw = sa + wrow;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      if (q < qlo || q >= qhi) continue;
      const int row = wq * kWR + q * 8 + (lane >> 3);
      const int ch = (lane & 7) ^ swz(row);
      uint32_t off = row < mrows ? (uint32_t)row * ld2b + (uint32_t)ch * 16u : kOobOff;
      if (kCheck) off = ch * 8 < krem ? off : kOobOff;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          src, (__attribute__((address_space(3))) void*)(sw + q * 8 * kBK), 16, off, 0, 0, 0);
    }
  };
  using Unchecked = std::false_type;
  using Checked = std::true_type;

  // ---- quantized weight: codes, 8-bit scales, steps.  Reads past the end
  // give 0, which makes a block's table all zeros.  kParts consecutive
  // threads share a block; thread part pp expands weights kWT·pp .. +kWT-1
  // of it.  At k-step 0, in weights (advance per k-step):
  //   forward  row n = t / kParts:              e0 = (n0 + n)·d + kWT·pp        (+64)
  //   backward row k = (t / kParts) % 64, block hb = t / (64·kParts) of the
  //            tile's two: e0 = k·d + n0 + 64·hb + kWT·pp                    (+64·d)
  // Every offset fits in 32 bits (the host checks the weight count).
  const int pp = t % kParts;
  const int wrow_n = t / kParts;                     // forward: tile row n
  const int wrow_k = (t / kParts) & 63, hb = t / (64 * kParts);   // backward
  const uint32_t nW = (uint32_t)((kTransW ? p.K : p.N) * p.d);   // weights in Wq
  const uint32_t nb = (nW + kBlock - 1) / kBlock;
  const Rsrc rc = rsrc(p.codes, ((int64_t)nW + 7) / 8 * 4);
  const Rsrc rs8 = rsrc(p.scale8, nb);
  const Rsrc rs2 = rsrc(p.scale2, (int64_t)((nb + kGroup - 1) / kGroup) * 4);
  const uint32_t e0 = kTransW ? (uint32_t)(wrow_k * p.d + n0 + 64 * hb + kWT * pp)
                              : (uint32_t)((n0 + wrow_n) * p.d + kWT * pp);
  const uint32_t e_step = kTransW ? (uint32_t)(kBK * p.d) : (uint32_t)kBK;
  // rows past N (forward) or past K (backward) start at or beyond nW
  const uint32_t c_off0 = e0 < nW ? e0 / 2 : kOobOff, b0 = e0 / kBlock;
  struct Codes {
    uint32_t c[kCW];
    uint32_t q8;
    float step;
  };
  auto load_codes = [&](int s, Codes& c) {
    const uint32_t b = b0 + (uint32_t)s * (e_step / kBlock);
    const uint32_t o = c_off0 == kOobOff ? kOobOff : c_off0 + (uint32_t)s * (e_step / 2);
    if constexpr (kCW == 4) {
      const uint4 x = bload16(rc, o);
      c.c[0] = x.x; c.c[1] = x.y; c.c[2] = x.z; c.c[3] = x.w;
    } else {
      typedef int i32x2 __attribute__((ext_vector_type(2)));
      const i32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rc, (int)o, 0, 0);
      c.c[0] = (uint32_t)x[0]; c.c[1] = (uint32_t)x[1];
    }
    c.q8 = __builtin_amdgcn_raw_buffer_load_b8(rs8, (int)b, 0, 0);
    c.step = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs2, (int)(b < nb ? (b / kGroup) * 4 : kOobOff), 0, 0));
  };
  // LDS position of code word c's 8 weights (one 16-byte chunk)
  auto w_slot = [&](uint16_t* sb, int c) -> uint16_t* {
    if (!kTransW) {
      return sb + wrow_n * kBK + (((kCW * pp + c) ^ swz(wrow_n)) << 3);
    } else {
      return sb + wrow_k * kBN + (chunk_tr(wrow_k, 8 * hb + kCW * pp + c) << 3);
    }
  };

  f32x16 acc[kI][4];
  // zeroed while the first k-step's loads are in flight (256 AGPR writes)
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  };

  // Fragments of one 16-wide k sub-step: kI activation row blocks × 4 weight
  // column blocks.  kBTr: the weight-side tile is [k][n] (read transposed).
  // swz(row) depends on row % 32 only, so the row blocks of a fragment set
  // differ by constant offsets.
  struct Frags {
    bf16x8 a[kI], b[4];
  };
  auto read_frags = [&](auto btr_tag, Frags& f, const uint16_t* sa, const uint16_t* sb, int kk) {
    constexpr bool kBTr = decltype(btr_tag)::value;
    const int ch = kk * 2 + (lane >> 5);
    const int r32 = lane & 31;
    const uint16_t* pa = sa + (wq * kWR + r32) * kBK + ((ch ^ swz(r32)) << 3);
#pragma unroll
    for (int i = 0; i < kI; ++i) f.a[i] = *reinterpret_cast<const bf16x8*>(pa + i * 32 * kBK);
    if (!kBTr) {
      const uint16_t* pb = sb + r32 * kBK + ((ch ^ swz(r32)) << 3);
#pragma unroll
      for (int j = 0; j < 4; ++j) f.b[j] = *reinterpret_cast<const bf16x8*>(pb + j * 32 * kBK);
    } else {
      const int g = lane >> 4, s = lane & 15;
      const int kr = kk * 16 + 8 * (g >> 1) + (s >> 2);
      const uint16_t* qlo = sb + kr * kBN + 4 * (s & 1);
      const uint16_t* qhi = qlo + 4 * kBN;                            // rows kr + 4
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // logical 16-byte chunk 4j + 2(g%2) + (s%4)/2 of rows kr and kr + 4
        const int c = 4 * j + 2 * (g & 1) + ((s & 3) >> 1);
        const s16x4 lo = lds_tr(qlo + (chunk_tr(kr, c) << 3));
        const s16x4 hi = lds_tr(qhi + (chunk_tr(kr + 4, c) << 3));
        const s16x8 bv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        f.b[j] = __builtin_bit_cast(bf16x8, bv);
      }
    }
  };
  // The weight fragment is the MFMA's first operand and the activation
  // fragment its second, so each lane accumulates 4 consecutive output
  // columns of one output row (the epilogue stores 8 bytes at a time).
  auto mfmas = [&](const Frags& f) {
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
  };
  using WTag = std::integral_constant<bool, kTransW>;
  using ATag = std::integral_constant<bool, !kTransW>;
  const uint16_t* a_base = p.A + m0 * p.lda;

  // One k-step without pipelining (the partial last weight step and the
  // adapter steps): publish the staged tiles, MFMAs per sub-step, and
  // release the buffers.
  auto plain_step = [&](auto btr_tag) {
    __builtin_amdgcn_s_waitcnt((0 & 0xF) | (0x7 << 4) | (0xF << 8));
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      Frags f;
      read_frags(btr_tag, f, sA0, sB0, kk);
      mfmas(f);
    }
    __syncthreads();
  };
  auto expand_block = [&](const Codes& c, uint16_t* sb) {
    Lut lut;
    make_lut(p.cb, (float)c.q8 * c.step, lut);   // ĉ = fl32(q8·step)
#pragma unroll
    for (int k = 0; k < kCW; ++k) *reinterpret_cast<uint4*>(w_slot(sb, k)) = expand(lut, c.c[k]);
  };

  // ---- main loop over the full k-steps of the quantized weight
  const int nkf = (int)(p.K / kBK);
  constexpr int kWaitAll = (0 & 0xF) | (0x7 << 4) | (0xF << 8);   // vmcnt(0)
  if (nkf > 0) {
    Codes r0, r1;
    dma_a(Unchecked{}, a_base, lda2b, 0, p.K, sA0);
    load_codes(0, r0);
    load_codes(1, r1);
    zero_acc();
    // pin the zeroing here: otherwise it sinks past the first barrier
#pragma unroll
    for (int i = 0; i < kI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
    expand_block(r0, sB0);
    __builtin_amdgcn_s_waitcnt(kWaitAll);
    __syncthreads();
    // step s: per 16-wide k sub-step read the fragments of the next
    // sub-step, issue a share of the activation DMA of s+1 (the code loads of
    // s+2 go out with the second share and get most of a step), expand code words
    // of s+1 into the idle weight buffer and issue the MFMAs, DMA instructions
    // interleaved with MFMAs so the address FIFO never backs up and stalls the
    // wave; then publish the weight tile.  Loads for steps at or past nkf
    // land in the idle buffers and are never used (the barriers after the
    // loop wait for them).
    auto iteration = [&](auto stage, int s, Codes& refill, const Codes& next) {
      constexpr bool kOdd = decltype(stage)::value;
      uint16_t* a_cur = kOdd ? sA1 : sA0;
      uint16_t* a_nxt = kOdd ? sA0 : sA1;
      uint16_t* b_cur = kOdd ? sB1 : sB0;
      uint16_t* b_nxt = kOdd ? sB0 : sB1;
      Frags f[2];
      // this wave's own activation rows of step s (its DMA) are in
      __builtin_amdgcn_s_waitcnt(kWaitAll);
      read_frags(WTag{}, f[0], a_cur, b_cur, 0);
      __builtin_amdgcn_sched_barrier(0);
      Lut lut;
      make_lut(p.cb, (float)next.q8 * next.step, lut);   // ĉ = fl32(q8·step)
      constexpr int kPer = kQ / 4;          // DMA instructions per sub-step
      constexpr int kMfma = 4 * kI;         // MFMAs per sub-step
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) read_frags(WTag{}, f[(kk + 1) & 1], a_cur, b_cur, kk + 1);
        if (kk == 1) load_codes(s + 2, refill);
        dma_a(Unchecked{}, a_base, lda2b, (int64_t)(s + 1) * kBK, p.K, a_nxt, kk * kPer, kk * kPer + kPer);
        if (kk % (4 / kCW) == 0)
          *reinterpret_cast<uint4*>(w_slot(b_nxt, kk / (4 / kCW))) = expand(lut, next.c[kk / (4 / kCW)]);
        mfmas(f[kk & 1]);
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
          __builtin_amdgcn_sched_group_barrier(0x008, kMfma / kPer / 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // publish the expanded weight tile of step s+1 (LDS writes only: each
      // wave's activation rows are its own, and it waits for their DMA at the
      // top of the next step; a fence here would wait for the DMA as well)
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    int s = 0;
    for (; s + 1 < nkf; s += 2) {
      iteration(std::false_type{}, s, r0, r1);
      iteration(std::true_type{}, s + 1, r1, r0);
    }
    if (s < nkf) iteration(std::false_type{}, s, r0, r1);
  } else {
    zero_acc();
  }
  // ---- the partial last k-step (K % 64 != 0): weight rows past K read 0
  if (nkf * kBK < p.K) {
    Codes c;
    dma_a(Checked{}, a_base, lda2b, (int64_t)nkf * kBK, p.K, sA0);
    load_codes(nkf, c);
    expand_block(c, sB0);
    plain_step(WTag{});
  }

  // ---- adapter k-steps: [s·T ‖ B] (forward: B [r][N] is an n-major tile,
  // read transposed) or [s·U ‖ A] (backward: A [N][r] is a k-major tile)
  if (nk2 > 0) {
    const uint16_t* a2_base = p.A2 + m0 * p.lda2;
    const Rsrc rb2 = !kTransW ? rsrc(p.B2, p.K2 * p.ldb2 * 2)
                              : rsrc(p.B2 + n0 * p.ldb2, min((int64_t)kBN, p.N - n0) * p.ldb2 * 2);
    constexpr int kChunks = kBN * kBK * 2 / 16 / kT;   // 16-byte chunks per thread
    for (int ls = 0; ls < nk2; ++ls) {
      const int64_t k0 = (int64_t)ls * kBK;
      dma_a(Checked{}, a2_base, (uint32_t)p.lda2 * 2u, k0, p.K2, sA0);
      uint4 rb[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = i * kT + t;
        if (kTransW) {   // A rows n (128) × 8 chunks of k
          const int row = c >> 3, ch = c & 7;
          const int64_t gk = k0 + ch * 8;
          rb[i] = bload16(rb2, gk < p.K2 ? (uint32_t)((row * p.ldb2 + gk) * 2) : kOobOff);
        } else {         // B rows k (64) × 16 chunks of n
          const int kr = c >> 4, ch = c & 15;
          const int64_t gk = k0 + kr, gn = n0 + ch * 8;
          rb[i] = bload16(rb2, (gk < p.K2 && gn < p.N) ? (uint32_t)((gk * p.ldb2 + gn) * 2) : kOobOff);
        }
      }
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int c = i * kT + t;
        if (kTransW) {
          const int row = c >> 3, ch = c & 7;
          *reinterpret_cast<uint4*>(sB0 + row * kBK + ((ch ^ swz(row)) << 3)) = rb[i];
        } else {
          const int kr = c >> 4, ch = c & 15;
          *reinterpret_cast<uint4*>(sB0 + kr * kBN + (chunk_tr(kr, ch) << 3)) = rb[i];
        }
      }
      plain_step(ATag{});
    }
  }

  // ---- epilogue.  Lane holds output row m = lane%32 of each 32×32 block and
  // columns 8(e/4) + 4(lane/32) + e%4 (four consecutive columns per register
  // quad).  Stored directly that would be 16-byte pieces of 32 rows per
  // instruction; instead each wave puts its kWR×128 block, rounded to bf16,
  // into its own part of the idle activation stages (256-byte rows, 16-byte
  // chunks XOR-swizzled by row % 16 so the row-wise reads are conflict-free)
  // and writes it back as whole rows: 4 rows × 256 bytes per instruction.
  __syncthreads();   // every wave is done with the stages
  static_assert(kWaves * kWR * kBN <= 2 * kBM * kBK, "the output block fits the two stages");
  const int stage_off = wq * kWR * kBN;          // bf16 elements
  uint16_t* st_out = stage_off < kBM * kBK ? sA0 + stage_off : sA1 + (stage_off - kBM * kBK);
#pragma unroll
  for (int i = 0; i < kI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = i * 32 + (lane & 31), c = 4 * j + q;
        const uint2 v = make_uint2(pack_bf16x2(acc[i][j][4 * q + 0], acc[i][j][4 * q + 1]),
                                   pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
        *reinterpret_cast<uint2*>(st_out + r * kBN + ((c ^ (r & 15)) << 3) + (lane >> 5) * 4) = v;
      }
  // the wave reads back only what its own lanes wrote
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const Rsrc rcout = rsrc(p.C + m0 * p.ldc, (int64_t)mrows * p.ldc * 2);   // rows past M: dropped
#pragma unroll 8
  for (int t = 0; t < kWR / 4; ++t) {
    const int r = 4 * t + (lane >> 4), c = lane & 15;
    const uint4 v = *reinterpret_cast<const uint4*>(st_out + r * kBN + ((c ^ (r & 15)) << 3));
    const int row = wq * kWR + r;
    const int64_t col = n0 + 8 * c;              // N % 8 == 0: a chunk is all in or all out
    const uint32_t off = col < p.N ? (uint32_t)((row * p.ldc + col) * 2) : kOobOff;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), rcout, (int)off, 0, 0);
  }

  // ---- plane sums handed to this launch (their planes were written by an
  // earlier launch): every workgroup takes a strided share of the quads.
  // The jobs are read from the kernel arguments only here, through a pointer
  // the compiler cannot see through, so they are not loaded at entry and
  // held in (spilled) scalar registers across the main loop.
  typedef const __attribute__((address_space(4))) char KChar;
  KChar* ka = (KChar*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ka));
  typedef const __attribute__((address_space(4))) ReduceJob KJob;
  const KJob* tails = reinterpret_cast<const KJob*>(ka + offsetof(QGemmArgs, tail_a));
  static_assert(offsetof(QGemmArgs, tail_b) == offsetof(QGemmArgs, tail_a) + sizeof(ReduceJob),
                "the two jobs are adjacent");
  const int64_t tstride = (int64_t)gridDim.x * kT;
#pragma unroll 1
  for (int u = 0; u < 2; ++u) {
    ReduceJob job;
    job.part = tails[u].part;
    job.splits = tails[u].splits;
    job.plane = tails[u].plane;
    job.count = tails[u].count;
    job.out_f32 = tails[u].out_f32;
    job.out_bf16 = tails[u].out_bf16;
    job.scale = tails[u].scale;
    for (int64_t i = (int64_t)blockIdx.x * kT + t; i < job.count / 4; i += tstride)
      reduce_planes_quad(job, i);
  }
}

hipError_t launch_qgemm(bool trans_w, const uint16_t* A, int64_t lda, const uint8_t* codes,
                        const uint8_t* scale8, const float* scale2, int64_t d,
                        const uint16_t* A2, int64_t lda2, const uint16_t* B2, int64_t ldb2,
                        int64_t M, int64_t N, int64_t K, int64_t K2, uint16_t* C, int64_t ldc,
                        const Codebook& cb, hipStream_t st, const ReduceJob& tail_a,
                        const ReduceJob& tail_b) {
  if (M == 0 || N == 0)   // no tiles: the plane sums run on their own
    return tail_a.count + tail_b.count > 0 ? launch_reduce_planes(tail_a, tail_b, st) : hipSuccess;
  QGemmArgs p{A, lda, codes, scale8, scale2, d, A2, lda2, B2, ldb2, M, N, K, K2, C, ldc,
              cb, tail_a, tail_b};
  const unsigned tiles = (unsigned)(((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN));
  if (trans_w)
    launch(k_qgemm<true, kWaves>, dim3(tiles), dim3(64 * kWaves), 0, st, p);
  else
    launch(k_qgemm<false, kWaves>, dim3(tiles), dim3(64 * kWaves), 0, st, p);
  return hipGetLastError();
}

}  // namespace qlora
