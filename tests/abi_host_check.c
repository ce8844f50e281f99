/* Host-side checks of the C ABI, written against include/qlora.h as a plain
 * C caller would use it.  The test suite builds this file together with the
 * library's sources under AddressSanitizer and UndefinedBehaviorSanitizer
 * (host code only) and runs it without a device: every call below returns
 * its status from argument validation, from the size helpers, or (for valid
 * arguments, only when no device is visible) QLORA_E_NO_DEVICE.  No pointer
 * passed here is ever dereferenced: the fake device addresses are never
 * touched, so a sanitizer report means the library read or computed
 * something it should not have.
 *
 * Exit status 0 when every check holds; each failure prints its line. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "qlora.h"

static int g_fail = 0, g_checks = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    ++g_checks;                                                       \
    if (!(cond)) {                                                    \
      ++g_fail;                                                       \
      fprintf(stderr, "abi_host_check: line %d: %s\n", __LINE__, #cond); \
    }                                                                 \
  } while (0)

/* Fake 16-byte-aligned device addresses, never dereferenced. */
#define A16 ((void*)(uintptr_t)0x10000)
#define MIS(k) ((void*)(uintptr_t)(0x10000 + (k)))

static qlora_nf4dq view(int64_t n, int fmt, int dq) {
  qlora_nf4dq v;
  memset(&v, 0, sizeof v);
  v.codes = (uint8_t*)A16;
  v.scale8 = (uint8_t*)A16;
  v.scale2 = (float*)A16;
  v.n = n;
  v.fmt = fmt;
  v.dq = dq;
  return v;
}

static int fwd(const qlora_nf4dq* v, const void* X, int64_t M, int64_t d, int64_t o,
               const void* A, int64_t r, size_t ws_bytes) {
  return qlora_linear_fwd((const qlora_bf16*)X, M, d, v, o, (const qlora_bf16*)A,
                          (const qlora_bf16*)A16, r, 2.0f, (qlora_bf16*)A16, NULL, A16, ws_bytes,
                          NULL);
}

static void sizes(void) {
  int64_t c = -1, s8 = -1, s2 = -1, w = -1;
  CHECK(qlora_quant_sizes(16384, &c, &s8, &s2) == QLORA_OK);
  CHECK(c == 8192 && s8 == 256 && s2 == 4);           /* 8192 + 256 + 4 bytes */
  CHECK(qlora_quant_sizes(0, &c, &s8, &s2) == QLORA_OK && c == 0 && s8 == 0 && s2 == 0);
  CHECK(qlora_quant_sizes(65, &c, &s8, &s2) == QLORA_OK && c == 36 && s8 == 2 && s2 == 4);
  CHECK(qlora_quant_sizes(-1, &c, &s8, &s2) == QLORA_E_INVALID);
  CHECK(qlora_quant_sizes(16384, NULL, NULL, NULL) == QLORA_OK);
  /* the largest n: the ceilings must not overflow */
  CHECK(qlora_quant_sizes(INT64_MAX, &c, &s8, &s2) == QLORA_OK);
  CHECK(c > 0 && s8 > 0 && s2 > 0);
  CHECK(qlora_quant_sizes_dq(INT64_MAX, QLORA_DQ_FP8_MEAN, &c, &s8, &s2, &w) == QLORA_OK);
  CHECK(c > 0 && s8 > 0 && s2 > 0 && w > 0);
  CHECK(qlora_quant_sizes_dq(16384, QLORA_DQ_INT8_MEAN, &c, &s8, &s2, &w) == QLORA_OK);
  CHECK(s2 == 8 && w == 256);
  CHECK(qlora_quant_sizes_dq(16, 3, NULL, NULL, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_quant_sizes_dq(-3, 0, NULL, NULL, NULL, NULL) == QLORA_E_INVALID);

  float tab[16];
  for (int f = 0; f < 4; ++f) {
    CHECK(qlora_codebook(f, tab) == QLORA_OK);
    CHECK(tab[0] <= -1.0f && tab[15] == 1.0f);   /* int4 reaches -8/7 */
    for (int k = 1; k < 16; ++k) CHECK(tab[k - 1] <= tab[k]);
  }
  CHECK(qlora_codebook(4, tab) == QLORA_E_INVALID);
  CHECK(qlora_codebook(-1, tab) == QLORA_E_INVALID);
  CHECK(qlora_codebook(0, NULL) == QLORA_E_INVALID);

  /* workspace sizes: the block shapes, zero sizes, and sizes no call accepts */
  CHECK(qlora_workspace_bytes(QLORA_OP_BWD, 2048, 8192, 22016, 64) > 0);
  CHECK(qlora_workspace_bytes(QLORA_OP_FWD, 4096, 4096, 4096, 0) == 0);
  CHECK(qlora_workspace_bytes(QLORA_OP_FWD, 1, 64, 8, 512) == 0);
  CHECK(qlora_workspace_bytes(7, 1, 64, 8, 8) == 0);
  for (int op = 0; op < 2; ++op) {
    (void)qlora_workspace_bytes(op, 0, 0, 0, 0);
    CHECK(qlora_workspace_bytes(op, INT64_MAX, 4096, 4096, 64) == 0);
    CHECK(qlora_workspace_bytes(op, 4096, INT64_MAX, 4096, 64) == 0);
    CHECK(qlora_workspace_bytes(op, 4096, 4096, INT64_MAX, 64) == 0);
    CHECK(qlora_workspace_bytes(op, -1, 4096, 4096, 64) == 0);
  }

  for (int st = -2; st < 12; ++st) {
    const char* s = qlora_strerror(st);
    CHECK(s != NULL && strlen(s) > 0);
  }
  CHECK(strstr(qlora_strerror(QLORA_E_SHAPE), "o % 8") != NULL);
  CHECK(strstr(qlora_strerror(QLORA_E_SHAPE), "r % 8") != NULL);
  CHECK(strstr(qlora_version(), "gfx950") != NULL);
}

static void linear_validation(void) {
  qlora_nf4dq v = view(128 * 128, 0, 0);
  const size_t big_ws = (size_t)1 << 30;
  qlora_nf4dq v100 = view(128 * 100, 0, 0);
  CHECK(fwd(&v100, A16, 8, 100, 128, A16, 8, big_ws) == QLORA_E_SHAPE);   /* d % 64 */
  qlora_nf4dq vo = view(100 * 128, 0, 0);
  CHECK(fwd(&vo, A16, 8, 128, 100, A16, 8, big_ws) == QLORA_E_SHAPE);     /* o % 8 */
  CHECK(fwd(&v, A16, 8, 128, 128, A16, 12, big_ws) == QLORA_E_SHAPE);     /* r % 8 */
  CHECK(fwd(&v, A16, 8, 128, 128, A16, 264, big_ws) == QLORA_E_SHAPE);    /* r > 256 */
  CHECK(fwd(&v, A16, 8, 128, 128, A16, -8, big_ws) == QLORA_E_SHAPE);
  CHECK(fwd(&v, A16, -1, 128, 128, A16, 8, big_ws) == QLORA_E_SHAPE);
  CHECK(fwd(&v, A16, INT64_MAX, 128, 128, A16, 8, big_ws) == QLORA_E_SHAPE);
  qlora_nf4dq vn = view(128 * 127, 0, 0);
  CHECK(fwd(&vn, A16, 8, 128, 128, A16, 8, big_ws) == QLORA_E_SHAPE);     /* n != o*d */
  qlora_nf4dq vbig = view(INT64_MAX, 0, 0);
  CHECK(fwd(&vbig, A16, 8, INT64_MAX - 63, INT64_MAX - 7, A16, 8, big_ws) == QLORA_E_SHAPE);
  CHECK(fwd(&vbig, A16, 8, (int64_t)1 << 20, (int64_t)1 << 20, A16, 8, big_ws) == QLORA_E_SHAPE);
  CHECK(fwd(&v, MIS(2), 8, 128, 128, A16, 8, big_ws) == QLORA_E_ALIGN);
  qlora_nf4dq va = view(128 * 128, 0, 0);
  va.codes = (uint8_t*)MIS(4);
  CHECK(fwd(&va, A16, 8, 128, 128, A16, 8, big_ws) == QLORA_E_ALIGN);
  CHECK(fwd(&v, A16, 8, 128, 128, A16, 8, 16) == QLORA_E_WORKSPACE);
  CHECK(fwd(&v, A16, 8, 128, 128, NULL, 8, big_ws) == QLORA_E_INVALID);
  CHECK(fwd(NULL, A16, 8, 128, 128, A16, 8, big_ws) == QLORA_E_INVALID);
  for (int bad = -1; bad <= 4; bad += 5) {
    qlora_nf4dq vf = view(128 * 128, bad, 0);
    CHECK(fwd(&vf, A16, 8, 128, 128, A16, 8, big_ws) == QLORA_E_INVALID);
  }
  qlora_nf4dq vd = view(128 * 128, 0, 1);                                   /* dq variant */
  CHECK(fwd(&vd, A16, 8, 128, 128, A16, 8, big_ws) == QLORA_E_INVALID);

  /* backward */
  const qlora_bf16* b = (const qlora_bf16*)A16;
  qlora_bf16* w = (qlora_bf16*)A16;
  CHECK(qlora_linear_bwd(b, b, NULL, 8, 128, &v, 128, b, b, 8, 2.0f, w, NULL, w, A16, big_ws,
                         NULL) == QLORA_E_INVALID);                         /* dA missing */
  CHECK(qlora_linear_bwd(b, b, NULL, 8, 128, &v, 128, b, b, 12, 2.0f, w, w, w, A16, big_ws,
                         NULL) == QLORA_E_SHAPE);
  CHECK(qlora_linear_bwd(b, b, NULL, 8, 128, &v, 128, b, b, 8, 2.0f, w, w, w, A16, 16, NULL) ==
        QLORA_E_WORKSPACE);
  CHECK(qlora_linear_bwd(b, b, NULL, INT64_MAX, 128, &v, 128, b, b, 8, 2.0f, w, w, w, A16, big_ws,
                         NULL) == QLORA_E_SHAPE);
  /* allocation-free backward: sizes beyond its scratch, then shape errors */
  qlora_nf4dq v7 = view((int64_t)11008 * 11008, 0, 0);
  CHECK(qlora_linear_bwd_noalloc(b, b, NULL, 4096, 11008, &v7, 11008, b, b, 64, 2.0f, w, w, w,
                                 NULL) == QLORA_E_SCRATCH);
  CHECK(qlora_linear_bwd_noalloc(b, b, NULL, 8, 100, &v100, 128, b, b, 8, 2.0f, w, w, w, NULL) ==
        QLORA_E_SHAPE);
  CHECK(qlora_linear_bwd_noalloc(b, b, NULL, INT64_MAX, 128, &v, 128, b, b, 8, 2.0f, w, w, w,
                                 NULL) == QLORA_E_SHAPE);

  /* several adapters over one base */
  float s[64];
  for (int i = 0; i < 64; ++i) s[i] = 1.0f;
  const int32_t* ad = (const int32_t*)A16;
  CHECK(qlora_linear_fwd_multi(b, 17, 128, &v, 128, b, b, 3, 16, s, ad, w, NULL, A16, big_ws,
                               NULL) == QLORA_E_SHAPE);
  CHECK(qlora_linear_fwd_multi(b, 4, 128, &v, 128, b, b, 0, 16, s, ad, w, NULL, A16, big_ws,
                               NULL) == QLORA_E_SHAPE);
  CHECK(qlora_linear_fwd_multi(b, 4, 128, &v, 128, b, b, 65, 16, s, ad, w, NULL, A16, big_ws,
                               NULL) == QLORA_E_SHAPE);
  CHECK(qlora_linear_fwd_multi(b, 4, 128, &v, 128, b, b, 3, 12, s, ad, w, NULL, A16, big_ws,
                               NULL) == QLORA_E_SHAPE);
  CHECK(qlora_linear_fwd_multi(b, 4, 128, &v, 128, b, b, 3, 16, NULL, ad, w, NULL, A16, big_ws,
                               NULL) == QLORA_E_INVALID);
  CHECK(qlora_linear_fwd_multi(b, 4, 128, &v, 128, b, b, 3, 16, s, (const int32_t*)MIS(2), w,
                               NULL, A16, big_ws, NULL) == QLORA_E_ALIGN);
}

static void other_validation(void) {
  qlora_nf4dq v = view(128 * 128, 0, 0);
  const float* f = (const float*)A16;
  /* quantize / dequant */
  qlora_nf4dq v0 = view(0, 0, 0), v99 = view(99, 0, 0), v100 = view(100, 0, 0);
  CHECK(qlora_quantize_nf4_dq(f, -5, &v0, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_quantize_nf4_dq(f, 100, &v99, NULL, NULL) == QLORA_E_SHAPE);
  CHECK(qlora_quantize_nf4_dq((const float*)MIS(8), 100, &v100, NULL, NULL) == QLORA_E_ALIGN);
  CHECK(qlora_quantize_nf4_dq(f, 100, NULL, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_quantize_nf4_dq(NULL, 100, &v100, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_quantize_nf4_dq(f, 0, &v0, NULL, NULL) == QLORA_OK);        /* empty: no-op */
  CHECK(qlora_dequant(&v100, 5, A16, NULL) == QLORA_E_INVALID);
  CHECK(qlora_dequant(NULL, 0, A16, NULL) == QLORA_E_INVALID);
  qlora_nf4dq vf = view(100, 7, 0);
  CHECK(qlora_quantize_nf4_dq(f, 100, &vf, NULL, NULL) == QLORA_E_INVALID);
  qlora_nf4dq vd = view(128 * 128, 0, 1);
  CHECK(qlora_quantize_nf4_dq(f, 128 * 128, &vd, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_quantize_nf4_dq_ws(f, 128 * 128, &vd, NULL, NULL, 0, NULL) == QLORA_E_WORKSPACE);
  vd.dq = 7;
  CHECK(qlora_dequant(&vd, 0, A16, NULL) == QLORA_E_INVALID);
  qlora_nf4dq vmax = view(INT64_MAX, 0, 0);
  CHECK(qlora_quantize_nf4_dq(f, INT64_MAX, &vmax, NULL, NULL) == QLORA_E_SHAPE);
  CHECK(qlora_dequant(&vmax, 0, A16, NULL) == QLORA_E_SHAPE);

  /* grouped quantizer */
  {
    const float* Wg[3] = {f, f, NULL};
    qlora_nf4dq vg[3] = {view(128, 0, 0), view(64, 0, 0), view(0, 0, 0)};
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vg, 0, NULL, NULL) == QLORA_OK);
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vg, -1, NULL, NULL) == QLORA_E_INVALID);
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vg, QLORA_MAX_GROUPED + 1, NULL, NULL) == QLORA_E_INVALID);
    CHECK(qlora_quantize_nf4_dq_grouped(NULL, vg, 3, NULL, NULL) == QLORA_E_INVALID);
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, NULL, 3, NULL, NULL) == QLORA_E_INVALID);
    const float* Wm[2] = {f, (const float*)MIS(4)};
    CHECK(qlora_quantize_nf4_dq_grouped(Wm, vg, 2, NULL, NULL) == QLORA_E_ALIGN);
    qlora_nf4dq vmix[2] = {view(128, 0, 0), view(64, 2, 0)};
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vmix, 2, NULL, NULL) == QLORA_E_INVALID);
    qlora_nf4dq vbig[2] = {view(128, 0, 0), view(INT64_MAX, 0, 0)};
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vbig, 2, NULL, NULL) == QLORA_E_SHAPE);
    qlora_nf4dq vdq[1] = {view(128, 0, 1)};          /* the default second level only */
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vdq, 1, NULL, NULL) == QLORA_E_INVALID);
  }

  /* merge */
  const qlora_bf16* b = (const qlora_bf16*)A16;
  float* out = (float*)A16;
  CHECK(qlora_merge_adapter(&v, 128, 128, b, b, 16, 2.0f, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_merge_adapter(&v, 128, 128, NULL, b, 16, 2.0f, out, NULL) == QLORA_E_INVALID);
  CHECK(qlora_merge_adapter(&v, 128, 100, b, b, 16, 2.0f, out, NULL) == QLORA_E_SHAPE);
  CHECK(qlora_merge_adapter(&v, 128, 128, b, b, 12, 2.0f, out, NULL) == QLORA_E_SHAPE);
  CHECK(qlora_merge_adapter(&v, 128, 128, b, b, 16, 2.0f, (float*)MIS(4), NULL) == QLORA_E_ALIGN);
  CHECK(qlora_merge_adapter(&v, INT64_MAX, INT64_MAX - 63, b, b, 16, 2.0f, out, NULL) ==
        QLORA_E_SHAPE);

  /* AdamW */
  qlora_adamw h = {1e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, 1};
  qlora_adamw h0 = h;
  h0.step = 0;
  float* p = (float*)A16;
  qlora_bf16* g = (qlora_bf16*)A16;
  CHECK(qlora_adamw_step(p, NULL, g, p, p, 100, NULL, NULL) == QLORA_E_INVALID);
  CHECK(qlora_adamw_step(p, NULL, g, p, p, 100, &h0, NULL) == QLORA_E_INVALID);
  CHECK(qlora_adamw_step(NULL, NULL, g, p, p, 100, &h, NULL) == QLORA_E_INVALID);
  CHECK(qlora_adamw_step((float*)MIS(4), NULL, g, p, p, 100, &h, NULL) == QLORA_E_ALIGN);
  CHECK(qlora_adamw_step(p, NULL, g, p, p, 0, &h, NULL) == QLORA_OK);
  CHECK(qlora_adamw_step(p, NULL, g, p, p, -1, &h, NULL) == QLORA_E_INVALID);
  CHECK(qlora_paged_adamw_step(p, NULL, g, p, p, 100, &h, A16, 4096, NULL) == QLORA_E_WORKSPACE);
  CHECK(qlora_paged_adamw_step(p, NULL, g, p, p, 100, &h, NULL, (size_t)1 << 20, NULL) ==
        QLORA_E_WORKSPACE);
  CHECK(qlora_paged_adamw_step(p, NULL, g, p, p, INT64_MAX, &h, A16, (size_t)1 << 20, NULL) ==
        QLORA_E_SHAPE);
  CHECK(qlora_adamw_step(p, NULL, g, p, p, QLORA_MAX_ELEMENTS + 1, &h, NULL) == QLORA_E_SHAPE);
}

static void no_device(void) {
  /* valid calls reach the device probe; with no device visible it answers */
  qlora_nf4dq v = view(128 * 128, 0, 0);
  const qlora_bf16* b = (const qlora_bf16*)A16;
  qlora_bf16* w = (qlora_bf16*)A16;
  CHECK(qlora_quantize_nf4_dq((const float*)A16, 128 * 128, &v, NULL, NULL) == QLORA_E_NO_DEVICE);
  CHECK(qlora_dequant(&v, 0, A16, NULL) == QLORA_E_NO_DEVICE);
  {
    const float* Wg[2] = {(const float*)A16, (const float*)A16};
    qlora_nf4dq vg[2] = {view(128 * 128, 0, 0), view(100, 0, 0)};
    CHECK(qlora_quantize_nf4_dq_grouped(Wg, vg, 2, NULL, NULL) == QLORA_E_NO_DEVICE);
  }
  CHECK(fwd(&v, A16, 8, 128, 128, A16, 8, (size_t)1 << 30) == QLORA_E_NO_DEVICE);
  CHECK(qlora_linear_bwd_noalloc(b, b, NULL, 8, 128, &v, 128, b, b, 8, 2.0f, w, w, w, NULL) ==
        QLORA_E_NO_DEVICE);
  /* the timing diagnostics with nothing timed */
  double ms = -1.0;
  int64_t n = -1;
  CHECK(qlora_timing_begin(0x3f) == QLORA_OK);
  CHECK(fwd(&v, A16, 8, 128, 128, A16, 8, (size_t)1 << 30) == QLORA_E_NO_DEVICE);
  CHECK(qlora_timing_end() == QLORA_OK);
  for (int k = 0; k < QLORA_K_COUNT; ++k) {
    CHECK(qlora_timing_read(k, &ms, &n) == QLORA_OK);
    CHECK(ms == 0.0 && n == 0);
  }
  CHECK(qlora_timing_read(QLORA_K_COUNT, &ms, &n) == QLORA_E_INVALID);
  CHECK(qlora_timing_read(-1, NULL, NULL) == QLORA_E_INVALID);
}

int main(int argc, char** argv) {
  /* argv[1] == "nodevice": the process sees no HIP device */
  const int nodevice = argc > 1 && strcmp(argv[1], "nodevice") == 0;
  sizes();
  linear_validation();
  other_validation();
  if (nodevice) no_device();
  printf("abi_host_check: %d checks, %d failed\n", g_checks, g_fail);
  return g_fail != 0;
}
