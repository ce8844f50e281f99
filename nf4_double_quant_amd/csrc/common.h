// Shared device types and helpers of the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;     // weights per absmax block
constexpr int kGroup = 256;    // blocks per double-quant group
constexpr int kGroupElems = kBlock * kGroup;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Codebook handed to kernels by value (kernel arguments live in SGPR-loaded
// constant memory): the 16 fp32 values and the 15 fp64 midpoints between
// neighbours, (V[t] + V[t+1]) / 2, which are exact in fp64.
struct Codebook {
  float v[16];
  double mid[15];
};

// Host-side 16-entry tables, built once when the library loads: 0 = NF4,
// 1 = int4, 2 = FP4 E2M1, 3 = FP4 E3M0 (the qlora_fmt values).
const Codebook& host_codebook(int fmt = 0);

// First guess of the encode.  Cell c = floor(x·S + S + 1/2) of x = w/c1 in
// [-1, 1] covers [(c − S − 1/2)/S, (c − S + 1/2)/S); code[c] is the number
// of midpoints below the cell's lower edge.  The builder checks that every
// cell holds at most one midpoint and that no midpoint lies within 1/1000 of
// a cell of an edge; then for any cell computed from x with an error below
// that margin, the code of w is code[c] or code[c] + 1, and one threshold
// compare decides.  zero_cell is a cell whose code is 7 (all-zero blocks),
// or −1 when the table fails the checks.
constexpr int kGuideScale = 128;
constexpr int kGuideCells = 2 * kGuideScale + 1;
struct EncodeGuide {
  uint32_t packed[(kGuideCells + 3) / 4];   // byte c = code[c]
  int32_t zero_cell;
};
const EncodeGuide& host_encode_guide(int fmt = 0);

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  // gfx950 converts with round-to-nearest-even (v_cvt_pk_bf16_f32).
  __bf16 h = (__bf16)x;
  return __builtin_bit_cast(uint16_t, h);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two RNE conversions in one v_cvt_pk_bf16_f32; `lo` lands in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

}  // namespace qlora
