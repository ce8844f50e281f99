// AdamW step of the adapter parameters, with the optimizer states either in
// device memory or paged from host memory ("074｜QLoRA：把大模型放进显存，再用
// 小适配器改变它" §三: only the LoRA parameters are updated, by a paged
// optimizer; §二 and the weimeta QLoRA glossary: the paged optimizer keeps
// Adam's states in CPU memory and moves them to the GPU when the update needs
// them, which avoids memory spikes at the cost of transfers).
//
// Per element, every operation rounded to fp32 in this order (no
// contraction; sqrt and division correctly rounded, the root by an exact
// midpoint test around the hardware root):
//     m' = b1·m + c1·g,  v' = b2·v + c2·(g·g),  den = sqrt(v')·rs + eps,
//     p' = p·keep − (lr1·m') / den,             p16 = RNE_bf16(p')
// with c1 = 1 − b1, c2 = 1 − b2, rs = 1/sqrt(1 − b2^t), keep = 1 − lr·wd,
// lr1 = lr/(1 − b1^t) computed on the host in fp64 (b^t by t products) and
// rounded once to fp32.
//
// The paged step streams the states through a caller device pool of four
// slots: one library copy stream brings pages in while slots are free, the
// caller's stream updates each page once it is in, a second copy stream takes
// it back out, freeing the slot; events order the three streams, and the
// caller's stream waits for the last page out.
#include <cmath>
#include <mutex>

#include "kernels.h"

namespace qlora {

// Correctly rounded fp32 square root of x >= 0.  The hardware root y is
// within an ulp; the nearest float to √x is the candidate c ∈ {y⁻, y, y⁺}
// with (c⁻ + c)/2 ≤ √x ≤ (c + c⁺)/2, tested on squares: the midpoints of two
// floats and their squares are exact in fp64 (25 and 50 significant bits),
// and √x never lies exactly on a midpoint.  Two rounds of the test.
__device__ __forceinline__ float sqrt_rn(float x) {
#pragma clang fp contract(off)
  float y = __builtin_sqrtf(x);
  if (!(x > 0.0f) || !(x < 3.0e38f)) return y;
  const double xd = (double)x;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const float dn = __int_as_float(__float_as_int(y) - 1);
    const float up = __int_as_float(__float_as_int(y) + 1);
    const double lo = 0.5 * ((double)dn + (double)y), hi = 0.5 * ((double)y + (double)up);
    if (xd < lo * lo) y = dn;
    else if (xd > hi * hi) y = up;
  }
  return y;
}

__device__ __forceinline__ void adamw_one(float& p, float& m, float& v, uint16_t g16,
                                          const AdamwConsts& k, uint16_t& p16) {
#pragma clang fp contract(off)
  const float g = bf16_to_f32(g16);
  const float m2 = k.b1 * m + k.c1 * g;
  const float v2 = k.b2 * v + k.c2 * (g * g);
  const float den = sqrt_rn(v2) * k.rs + k.eps;
  const float p2 = p * k.keep - __fdiv_rn(k.lr1 * m2, den);
  p = p2;
  m = m2;
  v = v2;
  p16 = bf16_bits(p2);
}

// Four consecutive elements per thread; the last partial quad element-wise.
__global__ __launch_bounds__(256) void k_adamw(float* __restrict__ p, uint16_t* __restrict__ p16,
                                               const uint16_t* __restrict__ g,
                                               float* __restrict__ m, float* __restrict__ v,
                                               int64_t n, AdamwConsts k) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t e = q * 4;
  if (e >= n) return;
  if (e + 4 <= n) {
    float4 pv = reinterpret_cast<float4*>(p)[q];
    float4 mv = reinterpret_cast<float4*>(m)[q];
    float4 vv = reinterpret_cast<float4*>(v)[q];
    const uint2 gv = reinterpret_cast<const uint2*>(g)[q];
    uint16_t o[4];
    adamw_one(pv.x, mv.x, vv.x, (uint16_t)(gv.x & 0xFFFF), k, o[0]);
    adamw_one(pv.y, mv.y, vv.y, (uint16_t)(gv.x >> 16), k, o[1]);
    adamw_one(pv.z, mv.z, vv.z, (uint16_t)(gv.y & 0xFFFF), k, o[2]);
    adamw_one(pv.w, mv.w, vv.w, (uint16_t)(gv.y >> 16), k, o[3]);
    reinterpret_cast<float4*>(p)[q] = pv;
    reinterpret_cast<float4*>(m)[q] = mv;
    reinterpret_cast<float4*>(v)[q] = vv;
    if (p16 != nullptr)
      reinterpret_cast<uint2*>(p16)[q] = make_uint2(o[0] | ((uint32_t)o[1] << 16), o[2] | ((uint32_t)o[3] << 16));
  } else {
    for (int64_t i = e; i < n; ++i) {
      float pp = p[i], mm = m[i], vv = v[i];
      uint16_t o;
      adamw_one(pp, mm, vv, g[i], k, o);
      p[i] = pp;
      m[i] = mm;
      v[i] = vv;
      if (p16 != nullptr) p16[i] = o;
    }
  }
}

AdamwConsts adamw_consts(float lr, float b1, float b2, float eps, float wd, int64_t t) {
  const double lrd = lr, b1d = b1, b2d = b2, wdd = wd;
  double p1 = 1.0, p2 = 1.0;
  for (int64_t i = 0; i < t; ++i) {
    p1 *= b1d;
    p2 *= b2d;
  }
  AdamwConsts k;
  k.b1 = b1;
  k.b2 = b2;
  k.c1 = (float)(1.0 - b1d);
  k.c2 = (float)(1.0 - b2d);
  k.rs = (float)(1.0 / std::sqrt(1.0 - p2));
  k.keep = (float)(1.0 - lrd * wdd);
  k.lr1 = (float)(lrd / (1.0 - p1));
  k.eps = eps;
  return k;
}

hipError_t launch_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m, float* v, int64_t n,
                        const AdamwConsts& k, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t quads = (n + 3) / 4;
  launch(k_adamw, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, p, p16, g, m,
                     v, n, k);
  return hipGetLastError();
}

namespace {
constexpr int kSlots = 4;   // pool slots, each an m page and a v page

// The copy streams (one per direction, so host-to-device and device-to-host
// transfers overlap) and events of the paged step, one set per device,
// created on first use and kept for the life of the process.  One mutex
// covers their creation and every call's whole enqueue, and a call's first
// pages wait for the previous call's write-back of the same pool slot, so
// calls from several threads or caller streams never overwrite a slot in
// use (when they pass the same pool).
struct PagedRes {
  hipStream_t in = nullptr, out = nullptr;
  hipEvent_t loaded[kSlots] = {}, done[kSlots] = {}, freed[kSlots] = {};
  hipEvent_t start = nullptr, finish = nullptr;
};
std::mutex g_paged_mu;
PagedRes g_paged[64];

hipError_t paged_res(PagedRes** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  PagedRes& r = g_paged[dev];   // the caller holds g_paged_mu
  if (r.in == nullptr) {
    if ((e = hipStreamCreateWithFlags(&r.in, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipStreamCreateWithFlags(&r.out, hipStreamNonBlocking)) != hipSuccess) return e;
    for (int i = 0; i < kSlots; ++i) {
      hipEvent_t* evs[3] = {&r.loaded[i], &r.done[i], &r.freed[i]};
      for (hipEvent_t* ev : evs)
        if ((e = hipEventCreateWithFlags(ev, hipEventDisableTiming)) != hipSuccess) return e;
    }
    if ((e = hipEventCreateWithFlags(&r.start, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&r.finish, hipEventDisableTiming)) != hipSuccess) return e;
  }
  *out = &r;
  return hipSuccess;
}
}  // namespace

int64_t paged_adamw_page_elems(size_t pool_bytes) {
  return (int64_t)(pool_bytes / (kSlots * 2 * sizeof(float))) / 256 * 256;
}

// Page i uses slot i % kSlots.  Stream `in` loads pages ahead while slots
// are free, the caller's stream updates page i once it is in, and stream
// `out` writes page i back once updated, which frees its slot for page
// i + kSlots.  Every event is recorded (in host order) before it is waited.
hipError_t launch_paged_adamw(float* p, uint16_t* p16, const uint16_t* g, float* m_host,
                              float* v_host, int64_t n, const AdamwConsts& k, void* pool,
                              size_t pool_bytes, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t page = paged_adamw_page_elems(pool_bytes);
  if (page <= 0) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_paged_mu);
  PagedRes* R = nullptr;
  hipError_t e = paged_res(&R);
  if (e != hipSuccess) return e;
  float* const base = static_cast<float*>(pool);
  auto slot_m = [&](int s) { return base + (int64_t)(2 * s) * page; };
  auto slot_v = [&](int s) { return base + (int64_t)(2 * s + 1) * page; };
  const int64_t pages = (n + page - 1) / page;
  auto count = [&](int64_t i) { return (i + 1) * page <= n ? page : n - i * page; };
#define QL_CK(x) do { if ((e = (x)) != hipSuccess) return e; } while (0)
  auto load = [&](int64_t i) -> hipError_t {
    const int s = (int)(i % kSlots);
    const size_t bytes = (size_t)count(i) * sizeof(float);
    hipError_t r;
    // the slot's last write-back: this call's page i - kSlots, or for the
    // first pages the previous call's (an event never recorded is complete)
    if ((r = hipStreamWaitEvent(R->in, R->freed[s], 0)) != hipSuccess) return r;
    if ((r = hipMemcpyAsync(slot_m(s), m_host + i * page, bytes, hipMemcpyHostToDevice, R->in)) != hipSuccess) return r;
    if ((r = hipMemcpyAsync(slot_v(s), v_host + i * page, bytes, hipMemcpyHostToDevice, R->in)) != hipSuccess) return r;
    return hipEventRecord(R->loaded[s], R->in);
  };
  // the pool and the host pages may still be in use by earlier work on the
  // caller's stream (the slots' use by the previous call is covered by
  // waiting for each slot's last write-back)
  QL_CK(hipEventRecord(R->start, st));
  QL_CK(hipStreamWaitEvent(R->in, R->start, 0));
  QL_CK(hipStreamWaitEvent(R->out, R->start, 0));
  for (int64_t i = 0; i < pages && i < kSlots; ++i) QL_CK(load(i));
  for (int64_t i = 0; i < pages; ++i) {
    const int s = (int)(i % kSlots);
    const int64_t off = i * page, c = count(i);
    QL_CK(hipStreamWaitEvent(st, R->loaded[s], 0));
    QL_CK(launch_adamw(p + off, p16 ? p16 + off : nullptr, g + off, slot_m(s), slot_v(s), c, k, st));
    QL_CK(hipEventRecord(R->done[s], st));
    QL_CK(hipStreamWaitEvent(R->out, R->done[s], 0));
    QL_CK(hipMemcpyAsync(m_host + off, slot_m(s), (size_t)c * sizeof(float), hipMemcpyDeviceToHost, R->out));
    QL_CK(hipMemcpyAsync(v_host + off, slot_v(s), (size_t)c * sizeof(float), hipMemcpyDeviceToHost, R->out));
    QL_CK(hipEventRecord(R->freed[s], R->out));
    if (i + kSlots < pages) QL_CK(load(i + kSlots));
  }
  QL_CK(hipEventRecord(R->finish, R->out));
  QL_CK(hipStreamWaitEvent(st, R->finish, 0));
#undef QL_CK
  return hipSuccess;
}

}  // namespace qlora
