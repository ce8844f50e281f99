// extern "C" entry points declared in include/qlora.h: argument checks,
// workspace layout and the launch sequence of each operation.
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "kernels.h"
#include "qlora.h"


using namespace qlora;

namespace {

constexpr int64_t kAlign = 256;

// a >= 0, b > 0; no intermediate overflows, also for a = INT64_MAX
inline int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0); }
inline int64_t up(int64_t a) { return cdiv(a, kAlign) * kAlign; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline int64_t clampi(int64_t v, int64_t lo, int64_t hi) { return v < lo ? lo : (v > hi ? hi : v); }

struct FwdLayout {
  bool gemv;               // few-token path
  int64_t Tpart, sT, total;  // byte offsets into the workspace
  int64_t t_splits;
};
FwdLayout fwd_layout(int64_t M, int64_t d, int64_t o, int64_t r) {
  (void)o;
  FwdLayout L{};
  int64_t off = 0;
  L.gemv = M <= kGemvMaxTokens && gemv_fits(M, d, r);
  L.t_splits = L.gemv ? gemv_tsplits(d) : rank_down_splits(d);
  L.Tpart = off; off += up(4 * L.t_splits * M * r);
  if (!L.gemv) {
    L.sT = off;  off += up(2 * M * r);
  }
  L.total = off;
  return L;
}

struct BwdLayout {
  int64_t Tpart, sT, Upart, sU, dApart, dBpart, total;
  int64_t t_splits, u_splits, g_splits;
};
BwdLayout bwd_layout(int64_t M, int64_t d, int64_t o, int64_t r) {
  BwdLayout L{};
  int64_t off = 0;
  if (r > 0) {
    L.t_splits = rank_down_splits(d);
    L.u_splits = rank_down_splits(o);
    L.g_splits = rank_grad_splits(M);
  }
  L.Tpart = off;  off += up(4 * L.t_splits * M * r);
  L.sT = off;     off += up(2 * M * r);
  L.Upart = off;  off += up(4 * L.u_splits * M * r);
  L.sU = off;     off += up(2 * M * r);
  L.dApart = off; off += up(4 * L.g_splits * d * r);
  L.dBpart = off; off += up(4 * L.g_splits * r * o);
  L.total = off;
  return L;
}

int device_status() {
  static int cached = -1;
  if (cached < 0) {
    int n = 0;
    cached = (hipGetDeviceCount(&n) == hipSuccess && n > 0) ? QLORA_OK : QLORA_E_NO_DEVICE;
  }
  return cached;
}

// Launch timing (diagnostics only; process-wide state, not thread-safe: one
// benchmark driver thread).  While on, every call of a chosen kernel class
// arms one start/stop event pair from a pool, and launch() records the
// events at the dispatches' own begin and end.  The pool grows only when a
// pass needs more pairs than any earlier one, so a warm-up pass leaves the
// timed pass without event creation.
struct LaunchTimer {
  bool on = false;
  uint32_t mask = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
  size_t cursor = 0;
  std::vector<size_t> used[QLORA_K_COUNT];
  hipError_t next(size_t* idx) {
    if (cursor == pool.size()) {
      hipEvent_t a, b;
      hipError_t e = hipEventCreate(&a);
      if (e != hipSuccess) return e;
      if ((e = hipEventCreate(&b)) != hipSuccess) {
        (void)hipEventDestroy(a);   // diagnostics: nothing more to do on failure
        return e;
      }
      pool.push_back({a, b});
    }
    *idx = cursor++;
    return hipSuccess;
  }
};
LaunchTimer g_timer;

}  // namespace

namespace qlora {
LaunchEvents*& armed_launch_events() {
  static thread_local LaunchEvents* armed = nullptr;
  return armed;
}
}  // namespace qlora

namespace {

template <class F>
hipError_t timed(int cls, hipStream_t st, F&& f) {
  (void)st;
  if (!g_timer.on || !((g_timer.mask >> cls) & 1u)) return f();
  size_t idx = 0;
  hipError_t e = g_timer.next(&idx);
  if (e != hipSuccess) return e;
  LaunchEvents ev{g_timer.pool[idx].first, g_timer.pool[idx].second, false};
  armed_launch_events() = &ev;
  e = f();
  armed_launch_events() = nullptr;
  if (e == hipSuccess && ev.fired) g_timer.used[cls].push_back(idx);
  return e;
}

#define QL_TRY(expr)                                  \
  do {                                                \
    if ((expr) != hipSuccess) return QLORA_E_HIP;     \
  } while (0)

// Launch one kernel of class `cls` (timed while diagnostics are on).
#define QL_RUN(cls, st, expr) QL_TRY(timed((cls), (st), [&]() { return (expr); }))

// allow_dq: whether the entry point decodes the second-level variants (the
// standalone quantizer and dequantizer); the fused kernels decode only the
// default one.
int check_quant_view(const qlora_nf4dq* q, bool allow_dq = false) {
  if (q == nullptr) return QLORA_E_INVALID;
  if (q->n < 0) return QLORA_E_INVALID;
  if (q->fmt < QLORA_FMT_NF4 || q->fmt > QLORA_FMT_FP4_E3M0) return QLORA_E_INVALID;
  if (q->dq < QLORA_DQ_UINT8 || q->dq > QLORA_DQ_FP8_MEAN) return QLORA_E_INVALID;
  if (q->dq != QLORA_DQ_UINT8 && !allow_dq) return QLORA_E_INVALID;
  if (q->n > 0 && (q->codes == nullptr || q->scale8 == nullptr || q->scale2 == nullptr))
    return QLORA_E_INVALID;
  if (!aligned16(q->codes) || !aligned16(q->scale8) || !aligned16(q->scale2)) return QLORA_E_ALIGN;
  return QLORA_OK;
}

int check_linear_shapes(int64_t M, int64_t d, int64_t o, int64_t r, const qlora_nf4dq* W) {
  if (M < 0 || d <= 0 || o <= 0 || r < 0) return QLORA_E_SHAPE;
  if (M > QLORA_MAX_TOKENS) return QLORA_E_SHAPE;
  // the kernels address a weight tensor and a 512-row activation tile with
  // 32-bit offsets
  if (d > QLORA_MAX_DIM || o > QLORA_MAX_DIM || o * d > QLORA_MAX_WEIGHTS) return QLORA_E_SHAPE;
  if (d % QLORA_BLOCK != 0 || o % 8 != 0) return QLORA_E_SHAPE;
  if (r > QLORA_MAX_RANK || r % 8 != 0) return QLORA_E_SHAPE;
  int st = check_quant_view(W);
  if (st) return st;
  if (W->n != o * d) return QLORA_E_SHAPE;
  return QLORA_OK;
}

// Scratch of qlora_linear_bwd_noalloc: a static device array, one copy per
// GPU.  In host code `scratch` names a host-side stand-in, not the device
// array; its device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is handed to
// kernels.
static __device__ __align__(256) uint8_t scratch[QLORA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QLORA_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QLORA_E_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QLORA_E_HIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_quant_sizes(int64_t n, int64_t* codes_bytes, int64_t* scale8_bytes, int64_t* scale2_bytes) {
  if (n < 0) return QLORA_E_INVALID;
  const int64_t nb = cdiv(n, QLORA_BLOCK);
  if (codes_bytes) *codes_bytes = 4 * cdiv(n, 8);
  if (scale8_bytes) *scale8_bytes = nb;
  if (scale2_bytes) *scale2_bytes = 4 * cdiv(nb, QLORA_GROUP);
  return QLORA_OK;
}

int qlora_codebook(int fmt, float* out) {
  if (out == nullptr || fmt < QLORA_FMT_NF4 || fmt > QLORA_FMT_FP4_E3M0) return QLORA_E_INVALID;
  memcpy(out, host_codebook(fmt).v, sizeof(float) * 16);
  return QLORA_OK;
}

size_t qlora_workspace_bytes(int op, int64_t M, int64_t d, int64_t o, int64_t r) {
  if (M < 0 || d < 0 || o < 0 || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (M > QLORA_MAX_TOKENS || d > QLORA_MAX_DIM || o > QLORA_MAX_DIM) return 0;
  if (op == QLORA_OP_FWD) return (size_t)fwd_layout(M, d, o, r).total;
  if (op == QLORA_OP_BWD) return (size_t)bwd_layout(M, d, o, r).total;
  return 0;
}

const char* qlora_strerror(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_E_INVALID: return "invalid argument";
    case QLORA_E_SHAPE: return "unsupported shape (need d % 64 == 0, o % 8 == 0, 0 <= r <= 256, r % 8 == 0, n == o*d, d and o <= 2^20, o*d <= 2^31, M <= 2^26, n <= 2^40)";
    case QLORA_E_ALIGN: return "tensor pointer not 16-byte aligned";
    case QLORA_E_WORKSPACE: return "workspace too small";
    case QLORA_E_NO_DEVICE: return "no HIP device available";
    case QLORA_E_HIP: return "HIP runtime or launch failure";
    case QLORA_E_NONFINITE: return "non-finite weight in quantizer input";
    case QLORA_E_SCRATCH: return "sizes need more scratch than the 64 MiB static buffer of qlora_linear_bwd_noalloc";
    default: return "unknown status";
  }
}

const char* qlora_version(void) { return "qlora-mi355x 0.1.0 (gfx950)"; }

int qlora_timing_begin(uint32_t mask) {
  for (auto& u : g_timer.used) u.clear();
  g_timer.cursor = 0;
  g_timer.mask = mask;
  g_timer.on = true;
  return QLORA_OK;
}

int qlora_timing_end(void) {
  g_timer.on = false;
  return QLORA_OK;
}

int qlora_timing_read(int kernel_class, double* total_ms, int64_t* launches) {
  if (kernel_class < 0 || kernel_class >= QLORA_K_COUNT) return QLORA_E_INVALID;
  double sum = 0.0;
  for (size_t idx : g_timer.used[kernel_class]) {
    const auto& p = g_timer.pool[idx];
    if (hipEventSynchronize(p.second) != hipSuccess) return QLORA_E_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, p.first, p.second) != hipSuccess) return QLORA_E_HIP;
    sum += ms;
  }
  if (total_ms) *total_ms = sum;
  if (launches) *launches = (int64_t)g_timer.used[kernel_class].size();
  return QLORA_OK;
}

int qlora_quantize_nf4_dq(const float* W, int64_t n, const qlora_nf4dq* out, int32_t* d_flags,
                          void* stream) {
  if (n < 0 || out == nullptr) return QLORA_E_INVALID;
  if (n > 0 && W == nullptr) return QLORA_E_INVALID;
  int st = check_quant_view(out);
  if (st) return st;
  if (n > QLORA_MAX_ELEMENTS) return QLORA_E_SHAPE;
  if (out->n != n) return QLORA_E_SHAPE;
  if (!aligned16(W)) return QLORA_E_ALIGN;
  if (n == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  QL_RUN(QLORA_K_QUANTIZE, (hipStream_t)stream, launch_quantize(W, n, out->codes, out->scale8, out->scale2, d_flags,
                                                                   out->fmt, (hipStream_t)stream));
  return QLORA_OK;
}

int qlora_quantize_nf4_dq_grouped(const float* const* W, const qlora_nf4dq* outs, int count,
                                  int32_t* d_flags, void* stream) {
  if (count < 0 || count > QLORA_MAX_GROUPED) return QLORA_E_INVALID;
  if (count == 0) return QLORA_OK;
  if (W == nullptr || outs == nullptr) return QLORA_E_INVALID;
  QuantJobs jobs{};
  int64_t g0 = 0;
  for (int k = 0; k < count; ++k) {
    const qlora_nf4dq& o = outs[k];
    int st = check_quant_view(&o);
    if (st) return st;
    if (o.fmt != outs[0].fmt) return QLORA_E_INVALID;
    if (o.n > QLORA_MAX_ELEMENTS) return QLORA_E_SHAPE;
    if (o.n > 0 && W[k] == nullptr) return QLORA_E_INVALID;
    if (!aligned16(W[k])) return QLORA_E_ALIGN;
    jobs.j[k] = QuantJob{W[k], o.codes, o.scale8, o.scale2, o.n, g0};
    g0 += cdiv(o.n, QLORA_BLOCK * QLORA_GROUP);
  }
  if (g0 > 0x7FFFFFFF) return QLORA_E_SHAPE;
  jobs.count = count;
  if (g0 == 0) return QLORA_OK;
  int st = device_status();
  if (st) return st;
  QL_RUN(QLORA_K_QUANTIZE, (hipStream_t)stream,
         launch_quantize_grouped(jobs, d_flags, outs[0].fmt, (hipStream_t)stream));
  return QLORA_OK;
}

int qlora_quant_sizes_dq(int64_t n, int dq, int64_t* codes_bytes, int64_t* scale8_bytes,
                         int64_t* scale2_bytes, int64_t* ws_bytes) {
  if (n < 0 || dq < QLORA_DQ_UINT8 || dq > QLORA_DQ_FP8_MEAN) return QLORA_E_INVALID;
  int64_t c = 0, s8 = 0, s2 = 0;
  qlora_quant_sizes(n, &c, &s8, &s2);
  const int64_t ng = s2 / 4;
  if (codes_bytes) *codes_bytes = c;
  if (scale8_bytes) *scale8_bytes = s8;
  if (scale2_bytes) *scale2_bytes = s2 + (dq != QLORA_DQ_UINT8 && n > 0 ? 4 : 0);
  if (ws_bytes) *ws_bytes = dq != QLORA_DQ_UINT8 ? up(8 * ng) : 0;
  return QLORA_OK;
}

int qlora_quantize_nf4_dq_ws(const float* W, int64_t n, const qlora_nf4dq* out, int32_t* d_flags,
                             void* ws, size_t ws_bytes, void* stream) {
  if (n < 0 || out == nullptr) return QLORA_E_INVALID;
  if (n > 0 && W == nullptr) return QLORA_E_INVALID;
  int st = check_quant_view(out, true);
  if (st) return st;
  if (out->n != n || n > QLORA_MAX_ELEMENTS) return QLORA_E_SHAPE;
  if (!aligned16(W) || !aligned16(ws)) return QLORA_E_ALIGN;
  int64_t need = 0;
  qlora_quant_sizes_dq(n, out->dq, nullptr, nullptr, nullptr, &need);
  if (ws_bytes < (size_t)need || (need > 0 && ws == nullptr)) return QLORA_E_WORKSPACE;
  if (n == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  hipStream_t hs = (hipStream_t)stream;
  QL_RUN(QLORA_K_QUANTIZE, hs, launch_quantize(W, n, out->codes, out->scale8, out->scale2, d_flags,
                                               out->fmt, hs));
  QL_RUN(QLORA_K_QUANTIZE, hs, launch_dq_variant(W, n, out->scale8, out->scale2, out->dq,
                                                 static_cast<double*>(ws), hs));
  return QLORA_OK;
}

int qlora_dequant(const qlora_nf4dq* q, int out_dtype, void* out, void* stream) {
  int st = check_quant_view(q, true);
  if (st) return st;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_E_INVALID;
  if (q->n > QLORA_MAX_ELEMENTS) return QLORA_E_SHAPE;
  if (q->n > 0 && out == nullptr) return QLORA_E_INVALID;
  if (!aligned16(out)) return QLORA_E_ALIGN;
  if (q->n == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  QL_RUN(QLORA_K_DEQUANT, (hipStream_t)stream, launch_dequant(q->codes, q->scale8, q->scale2, q->n, out_dtype == QLORA_BF16, out,
                        host_codebook(q->fmt), (hipStream_t)stream, q->dq));
  return QLORA_OK;
}

int qlora_linear_fwd(const qlora_bf16* X, int64_t M, int64_t d, const qlora_nf4dq* W, int64_t o,
                     const qlora_bf16* A, const qlora_bf16* B, int64_t r, float s, qlora_bf16* Y,
                     float* T_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear_shapes(M, d, o, r, W);
  if (st) return st;
  if (M > 0 && (X == nullptr || Y == nullptr)) return QLORA_E_INVALID;
  if (r > 0 && (A == nullptr || B == nullptr)) return QLORA_E_INVALID;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(A) || !aligned16(B) || !aligned16(T_out) ||
      !aligned16(ws))
    return QLORA_E_ALIGN;
  const FwdLayout L = fwd_layout(M, d, o, r);
  if (ws_bytes < (size_t)L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && ws == nullptr) return QLORA_E_WORKSPACE;
  if (M == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  hipStream_t hs = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  float* Tpart = reinterpret_cast<float*>(w + L.Tpart);
  const bool lora = r > 0 && s != 0.0f;

  if (L.gemv) {
    // T planes (the adapter class), then the dequant-GEMV that sums them
    if (r > 0 && (lora || T_out != nullptr))
      QL_RUN(QLORA_K_ADAPTER, hs, launch_gemv_tdown(X, (int)M, d, A, (int)r, Tpart, hs));
    QL_RUN(QLORA_K_GEMV, hs,
           launch_gemv_fwd(X, (int)M, d, W->codes, W->scale8, W->scale2, o, A, B, (int)r, s, Y,
                           T_out, Tpart, host_codebook(W->fmt), hs, nullptr, 0, nullptr, false));
    return QLORA_OK;
  }
  uint16_t* sT = reinterpret_cast<uint16_t*>(w + L.sT);
  if (r > 0 && (lora || T_out != nullptr)) {
    // T = X·A as split-K planes, summed into T_out (fp32) and s·T (bf16)
    QL_RUN(QLORA_K_ADAPTER, hs, launch_rank_down(false, X, M, d, A, (int)r, Tpart, hs));
    QL_RUN(QLORA_K_ADAPTER, hs,
           launch_reduce_planes(ReduceJob{Tpart, (int)L.t_splits, M * r, M * r, T_out,
                                          lora ? sT : nullptr, s},
                                ReduceJob{}, hs));
  }
  QL_RUN(QLORA_K_MAIN_GEMM, hs,
         launch_qgemm(false, X, d, W->codes, W->scale8, W->scale2, d, sT, r, B, o, M, o, d,
                      lora ? r : 0, Y, o, host_codebook(W->fmt), hs));
  return QLORA_OK;
}

int qlora_linear_fwd_multi(const qlora_bf16* X, int64_t M, int64_t d, const qlora_nf4dq* W,
                           int64_t o, const qlora_bf16* A, const qlora_bf16* B, int64_t n_adapters,
                           int64_t r, const float* s, const int32_t* d_adapter, qlora_bf16* Y,
                           float* T_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_linear_shapes(M, d, o, r, W);
  if (st) return st;
  if (M > QLORA_MAX_MULTI_TOKENS || r < 8) return QLORA_E_SHAPE;
  if (n_adapters < 1 || n_adapters > QLORA_MAX_ADAPTERS) return QLORA_E_SHAPE;
  if (M > 0 && (X == nullptr || Y == nullptr || d_adapter == nullptr)) return QLORA_E_INVALID;
  if (A == nullptr || B == nullptr || s == nullptr) return QLORA_E_INVALID;
  if (!aligned16(X) || !aligned16(Y) || !aligned16(A) || !aligned16(B) || !aligned16(T_out) ||
      !aligned16(ws) || (reinterpret_cast<uintptr_t>(d_adapter) & 3) != 0)
    return QLORA_E_ALIGN;
  const FwdLayout L = fwd_layout(M, d, o, r);
  if (M > 0 && !L.gemv) return QLORA_E_SHAPE;
  if (ws_bytes < (size_t)L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && ws == nullptr) return QLORA_E_WORKSPACE;
  if (M == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  hipStream_t hs = (hipStream_t)stream;
  float* Tpart = reinterpret_cast<float*>(static_cast<char*>(ws) + L.Tpart);
  QL_RUN(QLORA_K_ADAPTER, hs,
         launch_gemv_tdown(X, (int)M, d, A, (int)r, Tpart, hs, d_adapter, (int)n_adapters));
  QL_RUN(QLORA_K_GEMV, hs,
         launch_gemv_fwd(X, (int)M, d, W->codes, W->scale8, W->scale2, o, A, B, (int)r, 0.0f, Y,
                         T_out, Tpart, host_codebook(W->fmt), hs, d_adapter, (int)n_adapters, s,
                         false));
  return QLORA_OK;
}

int qlora_merge_adapter(const qlora_nf4dq* W, int64_t o, int64_t d, const qlora_bf16* A,
                        const qlora_bf16* B, int64_t r, float s, float* W_out, void* stream) {
  int st = check_linear_shapes(1, d, o, r, W);
  if (st) return st;
  if (W_out == nullptr || (r > 0 && (A == nullptr || B == nullptr))) return QLORA_E_INVALID;
  if (!aligned16(A) || !aligned16(B) || !aligned16(W_out)) return QLORA_E_ALIGN;
  if ((st = device_status())) return st;
  hipStream_t hs = (hipStream_t)stream;
  QL_RUN(QLORA_K_DEQUANT, hs,
         launch_merge(W->codes, W->scale8, W->scale2, o, d, A, B, (int)r, s, W_out,
                      host_codebook(W->fmt), hs));
  return QLORA_OK;
}

namespace {
int check_adamw(const float* p, const qlora_bf16* p16, const qlora_bf16* g, const float* m,
                const float* v, int64_t n, const qlora_adamw* h) {
  if (h == nullptr || n < 0 || h->step < 1) return QLORA_E_INVALID;
  if (n > 0 && (p == nullptr || g == nullptr || m == nullptr || v == nullptr)) return QLORA_E_INVALID;
  if (!aligned16(p) || !aligned16(p16) || !aligned16(g) || !aligned16(m) || !aligned16(v))
    return QLORA_E_ALIGN;
  if (n > QLORA_MAX_ELEMENTS) return QLORA_E_SHAPE;
  return QLORA_OK;
}
}  // namespace

int qlora_adamw_step(float* p, qlora_bf16* p16, const qlora_bf16* g, float* m, float* v,
                     int64_t n, const qlora_adamw* h, void* stream) {
  int st = check_adamw(p, p16, g, m, v, n, h);
  if (st) return st;
  if (n == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  const AdamwConsts k = adamw_consts(h->lr, h->beta1, h->beta2, h->eps, h->weight_decay, h->step);
  QL_RUN(QLORA_K_GRADS, (hipStream_t)stream, launch_adamw(p, p16, g, m, v, n, k, (hipStream_t)stream));
  return QLORA_OK;
}

int qlora_paged_adamw_step(float* p, qlora_bf16* p16, const qlora_bf16* g, float* m_host,
                           float* v_host, int64_t n, const qlora_adamw* h, void* pool,
                           size_t pool_bytes, void* stream) {
  int st = check_adamw(p, p16, g, m_host, v_host, n, h);
  if (st) return st;
  if (!aligned16(pool)) return QLORA_E_ALIGN;
  if (n > 0 && (pool == nullptr || paged_adamw_page_elems(pool_bytes) <= 0)) return QLORA_E_WORKSPACE;
  if (n == 0) return QLORA_OK;
  if ((st = device_status())) return st;
  const AdamwConsts k = adamw_consts(h->lr, h->beta1, h->beta2, h->eps, h->weight_decay, h->step);
  if (launch_paged_adamw(p, p16, g, m_host, v_host, n, k, pool, pool_bytes, (hipStream_t)stream) !=
      hipSuccess)
    return QLORA_E_HIP;
  return QLORA_OK;
}

int qlora_linear_bwd(const qlora_bf16* dY, const qlora_bf16* X, const float* T, int64_t M, int64_t d,
                     const qlora_nf4dq* W, int64_t o, const qlora_bf16* A, const qlora_bf16* B,
                     int64_t r, float s, qlora_bf16* dX, qlora_bf16* dA, qlora_bf16* dB, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = check_linear_shapes(M, d, o, r, W);
  if (st) return st;
  if (M > 0 && dY == nullptr) return QLORA_E_INVALID;
  if (r > 0 && (A == nullptr || B == nullptr || dA == nullptr || dB == nullptr ||
                (M > 0 && X == nullptr)))
    return QLORA_E_INVALID;
  if (dX == nullptr && r == 0) return QLORA_OK;
  if (!aligned16(dY) || !aligned16(X) || !aligned16(T) || !aligned16(A) || !aligned16(B) ||
      !aligned16(dX) || !aligned16(dA) || !aligned16(dB) || !aligned16(ws))
    return QLORA_E_ALIGN;
  const BwdLayout L = bwd_layout(M, d, o, r);
  if (ws_bytes < (size_t)L.total) return QLORA_E_WORKSPACE;
  if (L.total > 0 && ws == nullptr) return QLORA_E_WORKSPACE;
  if ((st = device_status())) return st;
  hipStream_t hs = (hipStream_t)stream;
  if (M == 0) {
    if (r > 0) {
      QL_RUN(QLORA_K_GRADS, hs, launch_fill_zero_bf16(dA, d * r, hs));
      QL_RUN(QLORA_K_GRADS, hs, launch_fill_zero_bf16(dB, r * o, hs));
    }
    return QLORA_OK;
  }
  char* w = static_cast<char*>(ws);
  float* Tpart = reinterpret_cast<float*>(w + L.Tpart);
  uint16_t* sT = reinterpret_cast<uint16_t*>(w + L.sT);
  float* Upart = reinterpret_cast<float*>(w + L.Upart);
  uint16_t* sU = reinterpret_cast<uint16_t*>(w + L.sU);
  float* dApart = reinterpret_cast<float*>(w + L.dApart);
  float* dBpart = reinterpret_cast<float*>(w + L.dBpart);
  const bool lora = r > 0 && s != 0.0f;

  if (r > 0) {
    // U = dY·Bᵀ as split planes (B [r][o] is the K-major operand); T as
    // planes too when the caller did not keep it
    if (T == nullptr)
      QL_RUN(QLORA_K_ADAPTER, hs, launch_rank_down(false, X, M, d, A, (int)r, Tpart, hs));
    QL_RUN(QLORA_K_ADAPTER, hs, launch_rank_down(true, dY, M, o, B, (int)r, Upart, hs));
    // s·U and s·T in bf16 (a given T is one plane)
    QL_RUN(QLORA_K_ADAPTER, hs,
           launch_reduce_planes(
               ReduceJob{Upart, (int)L.u_splits, M * r, M * r, nullptr, sU, s},
               T != nullptr ? ReduceJob{T, 1, M * r, M * r, nullptr, sT, s}
                            : ReduceJob{Tpart, (int)L.t_splits, M * r, M * r, nullptr, sT, s},
               hs));
    // dA = Xᵀ·(s·U) [d][r] and dB = (s·T)ᵀ·dY [r][o], reductions over the
    // tokens, in one launch; then both sums in one launch
    QL_RUN(QLORA_K_GRADS, hs,
           launch_rank_grads(RankGradJob{X, d, sU, dApart, true, 0},
                             RankGradJob{dY, o, sT, dBpart, false, 0}, (int)r, M, hs));
  }
  // the sums of the dA and dB planes: at the end of the dX launch when there
  // is one (a launch fewer), else on their own
  const ReduceJob sum_dA = r > 0 ? ReduceJob{dApart, (int)L.g_splits, d * r, d * r, nullptr, dA, 1.0f}
                                 : ReduceJob{};
  const ReduceJob sum_dB = r > 0 ? ReduceJob{dBpart, (int)L.g_splits, r * o, r * o, nullptr, dB, 1.0f}
                                 : ReduceJob{};
  if (dX != nullptr) {
    QL_RUN(QLORA_K_MAIN_GEMM, hs,
           launch_qgemm(true, dY, o, W->codes, W->scale8, W->scale2, d, sU, r, A, r, M, d, o,
                        lora ? r : 0, dX, d, host_codebook(W->fmt), hs, sum_dA, sum_dB));
  } else if (r > 0) {
    QL_RUN(QLORA_K_GRADS, hs, launch_reduce_planes(sum_dA, sum_dB, hs));
  }
  return QLORA_OK;
}

int qlora_linear_bwd_noalloc(const qlora_bf16* dY, const qlora_bf16* X, const float* T, int64_t M,
                             int64_t d, const qlora_nf4dq* W, int64_t o, const qlora_bf16* A,
                             const qlora_bf16* B, int64_t r, float s, qlora_bf16* dX,
                             qlora_bf16* dA, qlora_bf16* dB, void* stream) {
  int st = check_linear_shapes(M, d, o, r, W);
  if (st) return st;
  if ((int64_t)bwd_layout(M, d, o, r).total > QLORA_NOALLOC_SCRATCH_BYTES) return QLORA_E_SCRATCH;
  if ((st = device_status())) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws))) return st;
  return qlora_linear_bwd(dY, X, T, M, d, W, o, A, B, r, s, dX, dA, dB, ws,
                          (size_t)QLORA_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
