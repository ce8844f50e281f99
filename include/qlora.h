/*
 * qlora.h -- C ABI of the NF4 + double-quantization QLoRA linear layer,
 *            hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * Source of the method (cited by page title and section):
 *   [QLoRA-074] "074｜QLoRA：把大模型放进显存，再用小适配器改变它"
 *               (wq-win.github.io/llm/074-qlora.html), a summary of Dettmers
 *               et al., "QLoRA: Efficient Finetuning of Quantized LLMs", 2023.
 *
 * The layer (QLoRA-074 §一, problem setting):
 *     Y = X·Ŵ + s·X·A·B,   Ŵ = Dequant(W4bit, scales),
 *     X ∈ R^{M×d}, Ŵ ∈ R^{d×o}, A ∈ R^{d×r}, B ∈ R^{r×o}.
 * The 4-bit weight is frozen: training updates A and B only, but the input
 * gradient still multiplies by Ŵᵀ (QLoRA-074, note on what the backward pass
 * still needs).  There is deliberately no weight gradient in this ABI.
 *
 * Storage conventions shared by every entry point
 *   - The weight is stored as nn.Linear stores it, Wq[o][d] row-major, so
 *     Ŵ = Wqᵀ.  Quantization sees it as a flat array of n = o·d fp32 values,
 *     element i = row·d + col.
 *   - Block b = i / 64 has one first-level constant (absmax), group
 *     g = b / 256 one fp32 second-level constant (QLoRA-074 §二).  For the
 *     linear entry points d must be a multiple of 64, so blocks run along d.
 *   - codes: 4 bits per weight, 8 consecutive codes per little-endian 32-bit
 *     word: byte j (0..3) holds code j in bits 3:0 and code j+4 in bits 7:4.
 *     Codes past n are padded with 7 (NF4's zero code; 7 for every table),
 *     so the buffer is 4·ceil(n/8) bytes (n/2 when 8 divides n).
 *   - scale8: ceil(n/64) bytes, unsigned linear code q of the block absmax:
 *     ĉ_b = fl32(q_b · step_g).
 *   - scale2: ceil(n/16384) fp32 values, step_g = fl32(max c1 in g / 255).
 *   - Dequantized weight ŵ_i = fl32(V[k_i] · ĉ_b) with V the 16-value table
 *     of the view's fmt, NF4 by default (qlora_codebook); the linear layer
 *     uses RNE_bf16(ŵ_i).
 *   - bf16 tensors are raw bfloat16 bit patterns (uint16_t), row-major,
 *     contiguous.
 *
 * Memory and execution
 *   - Every tensor pointer is caller-allocated DEVICE memory, 16-byte aligned,
 *     unless stated otherwise.  The library never allocates or frees device
 *     memory; scratch comes from the caller's workspace (qlora_workspace_bytes).
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *     the null stream).  Nothing synchronizes the host.
 *   - Calls that share a workspace must be ordered (same stream); calls with
 *     separate workspaces are independent.  No kernel uses atomics; split
 *     planes are summed in plane order, so every result is bitwise
 *     reproducible run to run.
 *
 * Errors: every entry point returns a qlora_status.  Argument checks happen
 * before anything is launched; on error nothing was enqueued.
 */
#ifndef QLORA_H_
#define QLORA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_BLOCK 64      /* weights per first-level (absmax) block        */
#define QLORA_GROUP 256     /* first-level constants per second-level step   */
#define QLORA_MAX_RANK 256  /* largest LoRA rank r accepted                  */
#define QLORA_MAX_DIM (1LL << 20)       /* largest d and o of a linear layer  */
#define QLORA_MAX_WEIGHTS (1LL << 31)   /* largest o*d of a linear layer      */
#define QLORA_MAX_TOKENS (1LL << 26)    /* largest M of a linear layer        */
#define QLORA_MAX_ELEMENTS (1LL << 40)  /* largest n of the elementwise calls */
#define QLORA_MAX_MULTI_TOKENS 16       /* largest M of qlora_linear_fwd_multi */
#define QLORA_MAX_GROUPED 16            /* most tensors of qlora_quantize_nf4_dq_grouped */
#define QLORA_MAX_ADAPTERS 64           /* largest adapter count of the same   */
#define QLORA_NOALLOC_SCRATCH_BYTES (64LL << 20)  /* static scratch of qlora_linear_bwd_noalloc */

typedef enum {
  QLORA_OK = 0,
  QLORA_E_INVALID = 1,    /* null pointer where one is required, bad enum, n < 0 */
  QLORA_E_SHAPE = 2,      /* d % 64 != 0, o % 8 != 0, r out of range or not a
                             multiple of 8, negative sizes, n != o*d, d or o
                             above QLORA_MAX_DIM, o*d above QLORA_MAX_WEIGHTS,
                             M above QLORA_MAX_TOKENS, n of the quantizer,
                             dequantizer or optimizer above QLORA_MAX_ELEMENTS */
  QLORA_E_ALIGN = 3,      /* a tensor pointer is not 16-byte aligned          */
  QLORA_E_WORKSPACE = 4,  /* ws_bytes below qlora_workspace_bytes()          */
  QLORA_E_NO_DEVICE = 5,  /* no HIP device visible to the process            */
  QLORA_E_HIP = 6,        /* a HIP launch or runtime call failed             */
  QLORA_E_NONFINITE = 7,  /* reserved for bindings: a flag word had bit 0 set */
  QLORA_E_SCRATCH = 8     /* the sizes need more scratch than the static buffer
                             of qlora_linear_bwd_noalloc holds               */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

typedef enum {
  QLORA_OP_FWD = 0,       /* workspace of qlora_linear_fwd */
  QLORA_OP_BWD = 1        /* workspace of qlora_linear_bwd */
} qlora_op;

typedef uint16_t qlora_bf16; /* raw bfloat16 bits */

/* The 16-entry table the 4-bit codes index.  NF4 is the method's format
 * (QLoRA-074 §二); the others are the comparison formats of QLoRA-074 §四
 * (Table 2), run through the same kernels (see qlora_codebook). */
typedef enum {
  QLORA_FMT_NF4 = 0,
  QLORA_FMT_INT4 = 1,
  QLORA_FMT_FP4_E2M1 = 2,
  QLORA_FMT_FP4_E3M0 = 3
} qlora_fmt;

/* The code of the first-level constants (the double quantization).  UINT8 is
 * this library's reading of the method (QLoRA-074 §二: 8-bit constants, one
 * fp32 per 256): an unsigned linear code with no offset.  The variants centre
 * the constants on their tensor mean first (the page notes that offsets
 * exist beside the 8-bit constants) and code them as symmetric int8 or as
 * FP8 E4M3; scale2 then holds the steps followed by the mean.  Only the
 * quantizer with a workspace (qlora_quantize_nf4_dq_ws) and qlora_dequant
 * accept the variants. */
typedef enum {
  QLORA_DQ_UINT8 = 0,
  QLORA_DQ_INT8_MEAN = 1,
  QLORA_DQ_FP8_MEAN = 2
} qlora_dq;

/* Non-owning view of a quantized tensor (QLoRA-074 §三: the frozen W4 codes
 * plus the 8-bit first-level and fp32 second-level constants).  All three
 * buffers are device memory sized by qlora_quant_sizes(n) (qlora_quant_sizes_dq
 * for a dq variant).  fmt selects the table of the codes and dq the code of
 * the constants (0 = NF4 and UINT8, so a zero-initialised view is the
 * default); unknown values make every entry point return QLORA_E_INVALID,
 * and so does a dq variant passed to an entry point other than
 * qlora_quantize_nf4_dq_ws and qlora_dequant. */
typedef struct qlora_nf4dq {
  uint8_t* codes;   /* 4*ceil(n/8) bytes      */
  uint8_t* scale8;  /* ceil(n/64) bytes       */
  float* scale2;    /* ceil(n/16384) floats   */
  int64_t n;        /* number of weights      */
  int32_t fmt;      /* a qlora_fmt            */
  int32_t dq;       /* a qlora_dq             */
} qlora_nf4dq;

/* ---------------------------------------------------------------- host helpers */

/* Byte sizes of the three buffers of n weights (QLoRA-074, boxed note on the
 * compression ratio: 16384 weights -> 8192 code bytes + 256 + 4 bytes of
 * constants).  Any output pointer may be NULL.  Pure host code. */
int qlora_quant_sizes(int64_t n, int64_t* codes_bytes, int64_t* scale8_bytes,
                      int64_t* scale2_bytes);

/* The 16 values of table `fmt` as fp32, ascending; `out` is host memory for
 * 16 floats.  QLORA_FMT_NF4 is generated on the host at load time from
 * normal quantiles (QLoRA-074 §二): 8 positive values Φ⁻¹(1/2 + j(p−1/2)/8),
 * 7 negative −Φ⁻¹(1/2 + j(p−1/2)/7), and 0, all over Φ⁻¹(p),
 * p = 1 − (1/32 + 1/30)/2.  The comparison tables (readings of the format
 * names of QLoRA-074 §四; the pages give no tables): INT4 = (i−8)/7 (the
 * absmax maps to 7, −8/7 is never nearest); FP4_E2M1 = sign, 2 exponent
 * bits (bias 1, subnormals), 1 mantissa bit, over 6; FP4_E3M0 = sign and 3
 * exponent bits, field 0 = zero, field e = 2^(e−7).  Both FP4 tables keep −0
 * (index 7) and +0 (index 8). */
int qlora_codebook(int fmt, float* out);

/* Sizes for second-level variant dq: scale2 gains one float (the tensor mean)
 * when dq != QLORA_DQ_UINT8, and *ws_bytes is the workspace of
 * qlora_quantize_nf4_dq_ws (8 bytes per 16384-weight group).  Any output
 * pointer may be NULL.  Pure host code. */
int qlora_quant_sizes_dq(int64_t n, int dq, int64_t* codes_bytes, int64_t* scale8_bytes,
                         int64_t* scale2_bytes, int64_t* ws_bytes);

/* Workspace in bytes needed by qlora_linear_fwd (op = QLORA_OP_FWD) or
 * qlora_linear_bwd (op = QLORA_OP_BWD) for these sizes.  Returns 0 for
 * invalid sizes.  Pure host code. */
size_t qlora_workspace_bytes(int op, int64_t M, int64_t d, int64_t o, int64_t r);

const char* qlora_strerror(int status);
const char* qlora_version(void);

/* ------------------------------------------------------------ device entry points */

/* Blockwise NF4 quantization with double quantization of the constants
 * (QLoRA-074 §三 procedure: blockwise NF4 quantize with block 64, then
 * quantize the first-level constants with block 256; §二 NF4 and double
 * quantization).
 *   W      device fp32[n], any values; 0 <= n <= QLORA_MAX_ELEMENTS (n = 0
 *          is a no-op).
 *   out    view of caller buffers sized by qlora_quant_sizes(n); out->n must
 *          equal n.  Overwritten entirely.
 *   d_flags device int32 or NULL.  If any weight is NaN or ±Inf, bit 0 is set
 *          (the word is never cleared by the library; zero it first).  The
 *          outputs of a group holding a non-finite weight are unspecified.
 * Per block: c1 = max |w|; each weight gets the number of table midpoints
 * strictly below w/c1 (exact comparison): the nearest value, ties to the
 * lower index (with the duplicated zero of the FP4 tables a weight rounding
 * to zero keeps its sign, +0 only for w > 0); a zero block gets code 7.
 * The table is out->fmt (out->dq must be QLORA_DQ_UINT8; the variants need
 * qlora_quantize_nf4_dq_ws); codes past n are 7 for every table.  Per group:
 * step = fl32(max c1 / 255); q = the integer in 0..255 nearest to c1/step
 * (ties to the lower), 0 if step is 0. */
int qlora_quantize_nf4_dq(const float* W, int64_t n, const qlora_nf4dq* out,
                          int32_t* d_flags, void* stream);

/* The same quantization for several tensors in one launch (the procedure of
 * QLoRA-074 §三 applied to each tensor: blockwise NF4 with block 64, then the
 * constants with block 256).  Tensor k is W[k] (device fp32[outs[k].n]) and
 * its outputs are the buffers of outs[k], exactly as qlora_quantize_nf4_dq(
 * W[k], outs[k].n, &outs[k], d_flags, stream) would write them; groups never
 * span two tensors.  W and outs are host arrays of `count` entries,
 * 0 <= count <= QLORA_MAX_GROUPED (0 is a no-op); every view must use the
 * same table (fmt) and QLORA_DQ_UINT8; an entry with n = 0 is skipped.
 * d_flags as for qlora_quantize_nf4_dq (one word for all tensors).  Errors
 * as for qlora_quantize_nf4_dq, checked for every entry before any launch. */
int qlora_quantize_nf4_dq_grouped(const float* const* W, const qlora_nf4dq* outs, int count,
                                  int32_t* d_flags, void* stream);

/* The quantizer for any second-level variant out->dq (QLORA_DQ_UINT8 gives
 * exactly qlora_quantize_nf4_dq).  The codes are those of the default scheme
 * (encoded with the exact c1).  For the variants, per tensor:
 * μ = fl32(S/nb), S the fp64 sum of the block constants c1 (each group in
 * block order, then the groups in order); per block c' = fl32(c1 − μ); per
 * group step = fl32(max|c'| / 127) (INT8_MEAN) or fl32(max|c'| / 448)
 * (FP8_MEAN), 0 if max|c'| = 0; scale8[b] = the nearest int8 (two's
 * complement, ties to the smaller magnitude) or the nearest E4M3 value
 * (bias 7, subnormals, ties to the even mantissa, never −0) of c'/step;
 * scale2 = the steps, then μ.  ĉ = fl32(fl32(q·step) + μ).
 *   ws  device workspace of qlora_quant_sizes_dq(...)->ws_bytes bytes. */
int qlora_quantize_nf4_dq_ws(const float* W, int64_t n, const qlora_nf4dq* out,
                             int32_t* d_flags, void* ws, size_t ws_bytes, void* stream);

/* Dequantization Ŵ = Dequant(W4bit, scales) (QLoRA-074 §一; §三: the
 * weights a product needs are dequantized to BF16 on demand).
 *   q          quantized tensor (device buffers), q->n >= 0.
 *   out_dtype  QLORA_F32: out is fp32[n] with ŵ_i = fl32(V[k]·ĉ), ĉ = fl32(q8·step)
 *              (or the ĉ of the view's dq variant);
 *              QLORA_BF16: out is bf16[n] holding RNE_bf16(ŵ_i).
 * Bit-exact by construction: two IEEE fp32 products, nearest-even rounding. */
int qlora_dequant(const qlora_nf4dq* q, int out_dtype, void* out, void* stream);

/* Forward of the QLoRA linear layer (QLoRA-074 §一):
 *     T = X·A,   Y = X·Ŵ + s·T·B,   Ŵ = Wqᵀ.
 *   X      bf16[M][d]       A  bf16[d][r]      B  bf16[r][o]
 *   W      quantized Wq[o][d], W->n == o*d, d % 64 == 0
 *   s      adapter scale (α/r in LoRA); r == 0 or s == 0 runs the base only
 *   Y      bf16[M][o] (output, overwritten)
 *   T_out  fp32[M][r] or NULL: if given, receives T = X·A (for the backward)
 *   ws     device workspace of at least qlora_workspace_bytes(QLORA_OP_FWD,...)
 * Products use bf16 operands (the dequantized weight rounded to bf16) with
 * fp32 accumulation; Y is rounded to bf16 once.  M == 0 is a no-op.
 * 0 <= r <= 256, r % 8 == 0, o % 8 == 0 and M <= QLORA_MAX_TOKENS (eight
 * bf16 values are the 16-byte unit the kernels stream rows of A, B and Y
 * in); A and B may be NULL only if r == 0. */
int qlora_linear_fwd(const qlora_bf16* X, int64_t M, int64_t d,
                     const qlora_nf4dq* W, int64_t o,
                     const qlora_bf16* A, const qlora_bf16* B, int64_t r, float s,
                     qlora_bf16* Y, float* T_out,
                     void* ws, size_t ws_bytes, void* stream);

/* Few-token forward with one LoRA adapter per token over one shared frozen
 * base: several independent adapter pairs sit beside the 4-bit base and each
 * request picks one (LoRA-PyTorch page §四.5; the weimeta QLoRA glossary's
 * FAQ on serving customers from one unmerged 4-bit base).  For each row m:
 *     a = d_adapter[m],   T[m] = X[m]·A[a],   Y[m] = X[m]·Ŵ + s[a]·T[m]·B[a]
 * and an index outside [0, n_adapters) selects the base alone (T[m] = 0).
 *   X          bf16[M][d], 1 <= M <= QLORA_MAX_MULTI_TOKENS (M == 0: no-op)
 *   W          quantized Wq[o][d] as for qlora_linear_fwd
 *   A          bf16[n_adapters][d][r], B bf16[n_adapters][r][o] (device)
 *   s          host float[n_adapters]; 1 <= n_adapters <= QLORA_MAX_ADAPTERS
 *   d_adapter  device int32[M]
 *   Y          bf16[M][o] (overwritten); T_out fp32[M][r] or NULL
 *   ws         workspace of qlora_workspace_bytes(QLORA_OP_FWD, M, d, o, r)
 * 8 <= r <= 256, r % 8 == 0.  A row whose adapter is a gives bitwise the
 * result of qlora_linear_fwd with (A[a], B[a], s[a]).  QLORA_E_SHAPE also
 * when the few-token kernel cannot serve these sizes (d above 65536 with a
 * large M·r). */
int qlora_linear_fwd_multi(const qlora_bf16* X, int64_t M, int64_t d,
                           const qlora_nf4dq* W, int64_t o, const qlora_bf16* A,
                           const qlora_bf16* B, int64_t n_adapters, int64_t r,
                           const float* s, const int32_t* d_adapter, qlora_bf16* Y,
                           float* T_out, void* ws, size_t ws_bytes, void* stream);

/* Merge an adapter into the base weight, ahead of quantizing the merged layer
 * again (QLoRA-074 §五, §六: merging and re-quantizing can change outputs;
 * the weimeta QLoRA glossary FAQ: merge at 16-bit or better, not on the 4-bit
 * codes):
 *     W_out[n][k] = fl32( ŵ[n][k] + fl32(s · Δ[k][n]) ),   Δ = A·B,
 * with Δ accumulated by fp32 fused multiply-adds in increasing j (each bf16
 * product is exact in fp32, so each step rounds once) and ŵ the fp32
 * dequantized weight of qlora_dequant.  Pass W_out to qlora_quantize_nf4_dq
 * to obtain the merged 4-bit layer.
 *   W      quantized Wq[o][d] (shapes as for qlora_linear_fwd)
 *   A, B   bf16 [d][r], [r][o]; r == 0 (A, B may be NULL) gives W_out = ŵ
 *   W_out  device fp32 [o][d], overwritten */
int qlora_merge_adapter(const qlora_nf4dq* W, int64_t o, int64_t d, const qlora_bf16* A,
                        const qlora_bf16* B, int64_t r, float s, float* W_out, void* stream);

/* AdamW hyper-parameters of one step; step is t >= 1, the step being taken. */
typedef struct qlora_adamw {
  float lr, beta1, beta2, eps, weight_decay;
  int64_t step;
} qlora_adamw;

/* AdamW step of adapter parameters (QLoRA-074 §三: only the LoRA parameters
 * are updated).  Per element, each operation rounded to fp32 in this order
 * (sqrt and division correctly rounded, no contraction):
 *     m' = b1·m + c1·g,  v' = b2·v + c2·(g·g),  den = sqrt(v')·rs + eps,
 *     p' = p·keep − (lr1·m')/den
 * with c1 = 1−b1, c2 = 1−b2, rs = 1/sqrt(1−b2^t), keep = 1 − lr·wd and
 * lr1 = lr/(1−b1^t) formed in fp64 from the fp32 fields (b^t as t products)
 * and rounded once to fp32.
 *   p    device fp32[n] master parameters (updated in place)
 *   p16  device bf16[n] or NULL: receives RNE_bf16(p'), the copy the layer uses
 *   g    device bf16[n] gradient (dA or dB of qlora_linear_bwd)
 *   m, v device fp32[n] states (updated in place)
 * All pointers 16-byte aligned; n >= 0; h->step >= 1. */
int qlora_adamw_step(float* p, qlora_bf16* p16, const qlora_bf16* g, float* m, float* v,
                     int64_t n, const qlora_adamw* h, void* stream);

/* The same update with the optimizer states in host memory, paged through a
 * small device pool (QLoRA-074 §二 and the weimeta QLoRA glossary: the paged
 * optimizer keeps Adam's states in CPU memory and moves them to the GPU when
 * the update needs them).  m_host and v_host are pinned host memory
 * (hipHostMalloc); pool is device memory of pool_bytes >= 8192 split into four
 * slots of an m page and a v page.  One library copy stream moves pages in
 * while slots are free, `stream` updates each page, a second copy stream
 * moves it back out; `stream` waits for the last page, so later work on it
 * sees the new p, and a host synchronize of it makes m_host and v_host
 * current.  Results are bitwise those of
 * qlora_adamw_step.  Not for HIP-graph capture (it uses two more streams). */
int qlora_paged_adamw_step(float* p, qlora_bf16* p16, const qlora_bf16* g, float* m_host,
                           float* v_host, int64_t n, const qlora_adamw* h, void* pool,
                           size_t pool_bytes, void* stream);

/* Backward of the QLoRA linear layer (QLoRA-074 §一 and the note on what the
 * backward pass still needs): with U = dY·Bᵀ,
 *     dX = dY·Ŵᵀ + s·U·Aᵀ,   dA = s·Xᵀ·U,   dB = s·Tᵀ·dY,   T = X·A.
 * No gradient is produced for the frozen 4-bit weight.
 *   dY     bf16[M][o]        X bf16[M][d] (both may be NULL when M == 0)
 *   T      fp32[M][r] from qlora_linear_fwd's T_out, or NULL to recompute it
 *   W, A, B, s, r as in qlora_linear_fwd
 *   dX     bf16[M][d] or NULL (skip the input gradient)
 *   dA     bf16[d][r], dB bf16[r][o]: overwritten (not accumulated); may be
 *          NULL only if r == 0
 *   ws     device workspace of at least qlora_workspace_bytes(QLORA_OP_BWD,...)
 * M == 0 writes zeros to dA and dB. */
int qlora_linear_bwd(const qlora_bf16* dY, const qlora_bf16* X, const float* T,
                     int64_t M, int64_t d, const qlora_nf4dq* W, int64_t o,
                     const qlora_bf16* A, const qlora_bf16* B, int64_t r, float s,
                     qlora_bf16* dX, qlora_bf16* dA, qlora_bf16* dB,
                     void* ws, size_t ws_bytes, void* stream);

/* qlora_linear_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results (bitwise) and errors as qlora_linear_bwd, without
 * ws and ws_bytes: the scratch is a static device array of the library,
 * QLORA_NOALLOC_SCRATCH_BYTES (64 MiB) on each GPU it runs on, held from the
 * first call on that GPU until the process ends.  Sizes whose
 * qlora_workspace_bytes(QLORA_OP_BWD, M, d, o, r) exceeds it return
 * QLORA_E_SCRATCH before any launch (at r = 64 every projection of a
 * 7B-style block at 4096 tokens and of a 65B-style block at 2048 tokens fits:
 * at most 60.5 MiB).  No call
 * allocates or frees memory.  Every call on one GPU shares that GPU's array
 * and leaves its contents behind (each call overwrites the scratch it
 * reads): calls that overlap on one GPU (several streams or threads without
 * ordering between them) race and give undefined results. */
int qlora_linear_bwd_noalloc(const qlora_bf16* dY, const qlora_bf16* X, const float* T,
                             int64_t M, int64_t d, const qlora_nf4dq* W, int64_t o,
                             const qlora_bf16* A, const qlora_bf16* B, int64_t r, float s,
                             qlora_bf16* dX, qlora_bf16* dA, qlora_bf16* dB, void* stream);

/* ------------------------------------------------------------ diagnostics */

/* Kernel classes timed by the diagnostics below. */
typedef enum {
  QLORA_K_MAIN_GEMM = 0,  /* fused X·Ŵ (+adapter) and dY·Ŵᵀ (+adapter) products */
  QLORA_K_QUANTIZE = 1,   /* blockwise NF4 + double-quant kernel                  */
  QLORA_K_GEMV = 2,       /* few-token dequant-GEMV forward                       */
  QLORA_K_DEQUANT = 3,    /* standalone / transposed dequant kernels              */
  QLORA_K_ADAPTER = 4,    /* rank-r products T = X·A, U = dY·Bᵀ and their sums    */
  QLORA_K_GRADS = 5,      /* dA, dB products over the tokens and their sums       */
  QLORA_K_COUNT = 6
} qlora_kernel_class;

/* Launch timing for benchmarks (diagnostics only).  Between
 * qlora_timing_begin(mask) and qlora_timing_end(), every call whose kernel
 * class bit (1 << class) is set in `mask` launches its kernel(s) with a pair
 * of HIP events recorded at the first dispatch's begin and the last
 * dispatch's end (hipExtLaunchKernel), so the interval is kernel time, not
 * host or queue time.  qlora_timing_read() waits for the events and returns
 * the summed milliseconds and the number of calls of one class since the
 * last qlora_timing_begin().  Events come from a pool that grows only when a
 * pass needs more than any earlier pass did (run a warm-up pass first to
 * keep event creation out of a timed pass).  The state is process-wide and
 * not thread-safe: meant for single-threaded benchmark drivers; calls made
 * while timing is off launch plainly and touch none of it. */
int qlora_timing_begin(uint32_t mask);
int qlora_timing_end(void);
int qlora_timing_read(int kernel_class, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H_ */
