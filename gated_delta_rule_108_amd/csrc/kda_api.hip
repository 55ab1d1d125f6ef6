// C ABI of libkda: argument validation, then dispatch to the kernels.
// Every check runs on the host before any launch; see include/kda.h for the
// contract of each entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other.  Only caches an immutable fact.
std::atomic<int> g_arch_ok[kMaxDevices];

kda_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_DEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KDA_ERR_HIP;
    st = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? KDA_OK : KDA_ERR_DEVICE;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Chunk length the kernels run for a requested C.  A 128-token chunk runs as
// two 64-token chunks: its C x C solve matrix, P and Y tiles do not fit the
// CU's 160 KiB of LDS beside the K, Q, V tiles, and by the chunk algebra two
// consecutive 64-token chunks give the same result up to rounding.
int chunk_run(int C) { return C == 128 ? 64 : C; }

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};
Span span(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}
bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

}  // namespace

extern "C" {

const char* kda_status_string(kda_status s) {
  switch (s) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range";
    case KDA_ERR_UNSUPPORTED: return "unsupported dk, dv, chunk size, dtype or q/k map";
    case KDA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KDA_ERR_ALIAS: return "an output overlaps an input";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_DEVICE: return "current device is not gfx950";
    case KDA_ERR_HIP: return "HIP runtime error";
    case KDA_ERR_SCRATCH:
      return "sizes need more device scratch than the library's fixed scratch array holds";
  }
  return "unknown status";
}

size_t kda_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int C, kda_dtype dt) {
  C = chunk_run(C);
  if (B < 1 || H < 1 || T < 0) return static_cast<size_t>(-1);
  if (dt != KDA_F32 && dt != KDA_BF16) return static_cast<size_t>(-1);
  if (!dim_ok(dk) || !dim_ok(dv)) return static_cast<size_t>(-1);
  if (!kda::prefill_supported(dk, dv, C, dt == KDA_BF16)) return static_cast<size_t>(-1);
  return kda::prefill_workspace(B, T, H, dk, dv, C, dt == KDA_BF16);
}

}  // extern "C"

// ----------------------------------------------------------------------------
// The device scratch of kda_prefill_chunked_noalloc, for callers that cannot
// allocate device memory: a file-scope device array, one copy per GPU, held
// until the process ends.  Host code never passes the array's name to a
// kernel or a copy (on the host the name only stands in for the symbol): the
// device address of each GPU's copy comes from hipGetSymbolAddress, looked up
// on the first call on that GPU with it current, and is kept per device.
// ----------------------------------------------------------------------------
static __device__ __align__(256) char scratch[kda::kNoallocScratchBytes];

namespace {

std::atomic<void*> g_scratch[kMaxDevices];   // device address of `scratch`, per device

// Device address of the current device's copy of `scratch`.
kda_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return KDA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KDA_ERR_DEVICE;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return KDA_ERR_HIP;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return KDA_OK;
}

}  // namespace

namespace {

// Bytes of the gate array per token and head for each way the gate arrives.
size_t gate_bytes(int gate_in, int dk, size_t esize) {
  switch (gate_in) {
    case kda::kGateLogit: return dk * esize;   // logits of the I/O type
    case kda::kGateScalar: return 4;           // one fp32 gate per token and head
  }
  return dk * 4;                               // fp32 alpha per key channel
}

// Shared by kda_prefill_chunked (alpha: fp32 gates per channel),
// kda_prefill_chunked_logits (gate logits of type dt, beta as logits) and
// kda_gdn_prefill_chunked (one gate per token and head, or none).
kda_status prefill_impl(const void* q, const void* k, const void* v, const void* alpha,
                        const float* beta, const float* S0, void* o, float* S_T, int B, int T,
                        int H, int dk, int dv, int C, kda_dtype dt, int gate_in, int qk_map,
                        void* workspace, size_t workspace_bytes, void* stream,
                        size_t segment_budget = 0, bool use_scratch = false) {
  C = chunk_run(C);
  if (B < 1 || H < 1 || T < 0) return KDA_ERR_SHAPE;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
  if (!kda::prefill_supported(dk, dv, C, dt == KDA_BF16)) return KDA_ERR_UNSUPPORTED;
  const bool has_tokens = T > 0;
  const bool gate_optional = gate_in == kda::kGateScalar;   // null: alpha = 1
  if (has_tokens && (!q || !k || !v || (!alpha && !gate_optional) || !beta || !o))
    return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, alpha, beta, S0, o, S_T, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const size_t ws_need =
      kda::prefill_workspace(B, T, H, dk, dv, C, dt == KDA_BF16, segment_budget);
  if (use_scratch) {
    if (ws_need > kda::kNoallocScratchBytes) return KDA_ERR_SCRATCH;
  } else if (ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need)) {
    return KDA_ERR_WORKSPACE;
  }

  const size_t e = (dt == KDA_BF16) ? 2 : 4;
  const size_t ntok = static_cast<size_t>(B) * T * H;
  const size_t ga = alpha ? ntok * gate_bytes(gate_in, dk, e) : 0;
  const size_t nst = static_cast<size_t>(B) * H * dk * dv * 4;
  if (has_tokens) {
    const Span so = span(o, ntok * dv * e);
    const Span ins[] = {span(q, ntok * dk * e), span(k, ntok * dk * e), span(v, ntok * dv * e),
                        span(alpha, ga), span(beta, ntok * 4),
                        S0 ? span(S0, nst) : Span{0, 0}, S_T ? span(S_T, nst) : Span{0, 0}};
    for (const Span& s : ins)
      if (overlap(so, s)) return KDA_ERR_ALIAS;
  }
  if (ws_need > 0 && !use_scratch) {   // the library's own scratch overlaps no caller buffer
    const Span sw = span(workspace, ws_need);
    const Span all[] = {span(q, ntok * dk * e), span(k, ntok * dk * e), span(v, ntok * dv * e),
                        span(alpha, ga), span(beta, ntok * 4), span(o, ntok * dv * e),
                        S0 ? span(S0, nst) : Span{0, 0}, S_T ? span(S_T, nst) : Span{0, 0}};
    for (const Span& s : all)
      if (overlap(sw, s)) return KDA_ERR_ALIAS;
  }
  if (S_T) {
    const Span st = span(S_T, nst);
    if (S0 && S0 != S_T && overlap(st, span(S0, nst))) return KDA_ERR_ALIAS;
    if (has_tokens) {
      const Span ins[] = {span(q, ntok * dk * e), span(k, ntok * dk * e), span(v, ntok * dv * e),
                          span(alpha, ga), span(beta, ntok * 4)};
      for (const Span& s : ins)
        if (overlap(st, s)) return KDA_ERR_ALIAS;
    }
  }
  const kda_status dev = check_device();
  if (dev != KDA_OK) return dev;
  if (!S_T && !has_tokens) return KDA_OK;  // nothing to compute or write
  if (use_scratch && ws_need > 0) {
    const kda_status st = scratch_address(&workspace);
    if (st != KDA_OK) return st;
    workspace_bytes = kda::kNoallocScratchBytes;
  }

  kda::PrefillArgs a{q,  k,  v,  alpha, beta, S0, o,  S_T,          B,         T,
                     H,  dk, dv, C,     dt == KDA_BF16,   stream, workspace, workspace_bytes,
                     gate_in, qk_map};
  a.segment_budget = segment_budget;
  if (kda::launch_prefill(a) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status decode_impl(const void* q, const void* k, const void* v, const void* alpha,
                       const float* beta, const float* S_in, void* o, float* S_out, int N, int H,
                       int dk, int dv, kda_dtype dt, int gate_in, int qk_map, void* stream) {
  if (N < 1 || H < 1) return KDA_ERR_SHAPE;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
  const bool gate_optional = gate_in == kda::kGateScalar;   // null: alpha = 1
  if (!q || !k || !v || (!alpha && !gate_optional) || !beta || !S_in || !o || !S_out)
    return KDA_ERR_NULL;
  const void* ptrs[] = {q, k, v, alpha, beta, S_in, o, S_out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const size_t e = (dt == KDA_BF16) ? 2 : 4;
  const size_t nh = static_cast<size_t>(N) * H;
  const size_t ga = alpha ? nh * gate_bytes(gate_in, dk, e) : 0;
  const size_t nst = nh * dk * dv * 4;
  const Span ins[] = {span(q, nh * dk * e), span(k, nh * dk * e), span(v, nh * dv * e),
                      span(alpha, ga), span(beta, nh * 4), span(S_in, nst)};
  const Span so = span(o, nh * dv * e), ss = span(S_out, nst);
  for (const Span& s : ins)
    if (overlap(so, s)) return KDA_ERR_ALIAS;
  for (int i = 0; i < 5; ++i)
    if (overlap(ss, ins[i])) return KDA_ERR_ALIAS;
  if (overlap(so, ss)) return KDA_ERR_ALIAS;
  if (S_out != S_in && overlap(ss, ins[5])) return KDA_ERR_ALIAS;  // equal is in place
  const kda_status dev = check_device();
  if (dev != KDA_OK) return dev;
  kda::DecodeArgs a{q, k, v, alpha, beta, S_in, o, S_out, N, H, dk, dv, dt == KDA_BF16, stream,
                    gate_in, qk_map};
  if (kda::launch_decode(a) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

bool qk_map_ok(kda_qk_map m) { return m == KDA_QK_AS_GIVEN || m == KDA_QK_L2 || m == KDA_QK_SILU_L2; }

}  // namespace

extern "C" {

kda_status kda_prefill_chunked(const void* q, const void* k, const void* v, const float* alpha,
                               const float* beta, const float* S0, void* o, float* S_T, int B,
                               int T, int H, int dk, int dv, int C, kda_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, alpha, beta, S0, o, S_T, B, T, H, dk, dv, C, dt, kda::kGateAlpha,
                      0, workspace, workspace_bytes, stream);
}

kda_status kda_prefill_chunked_logits(const void* q, const void* k, const void* v, const void* g,
                                      const float* b, const float* S0, void* o, float* S_T, int B,
                                      int T, int H, int dk, int dv, int C, kda_dtype dt,
                                      kda_qk_map qk_map, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  if (!qk_map_ok(qk_map)) return KDA_ERR_UNSUPPORTED;
  return prefill_impl(q, k, v, g, b, S0, o, S_T, B, T, H, dk, dv, C, dt, kda::kGateLogit,
                      static_cast<int>(qk_map), workspace, workspace_bytes, stream);
}

kda_status kda_gdn_prefill_chunked(const void* q, const void* k, const void* v, const float* a,
                                   const float* beta, const float* S0, void* o, float* S_T, int B,
                                   int T, int H, int dk, int dv, int C, kda_dtype dt,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(q, k, v, a, beta, S0, o, S_T, B, T, H, dk, dv, C, dt, kda::kGateScalar, 0,
                      workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const float* alpha,
                           const float* beta, const float* S_in, void* o, float* S_out, int N,
                           int H, int dk, int dv, kda_dtype dt, void* stream) {
  return decode_impl(q, k, v, alpha, beta, S_in, o, S_out, N, H, dk, dv, dt, kda::kGateAlpha, 0,
                     stream);
}

kda_status kda_decode_step_logits(const void* q, const void* k, const void* v, const void* g,
                                  const float* b, const float* S_in, void* o, float* S_out,
                                  int N, int H, int dk, int dv, kda_dtype dt, kda_qk_map qk_map,
                                  void* stream) {
  if (!qk_map_ok(qk_map)) return KDA_ERR_UNSUPPORTED;
  return decode_impl(q, k, v, g, b, S_in, o, S_out, N, H, dk, dv, dt, kda::kGateLogit,
                     static_cast<int>(qk_map), stream);
}

kda_status kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* a,
                               const float* beta, const float* S_in, void* o, float* S_out, int N,
                               int H, int dk, int dv, kda_dtype dt, void* stream) {
  return decode_impl(q, k, v, a, beta, S_in, o, S_out, N, H, dk, dv, dt, kda::kGateScalar, 0,
                     stream);
}

}  // extern "C"

namespace {

kda_status decode_backward_impl(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* S_in, const void* dO,
                                const float* dS_new, void* dq, void* dk, void* dv,
                                float* dalpha, float* dbeta, float* dS, int N, int H, int dk_,
                                int dv_, kda_dtype dt, void* stream, int gate_in) {
  if (N < 1 || H < 1) return KDA_ERR_SHAPE;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (!dim_ok(dk_) || !dim_ok(dv_)) return KDA_ERR_UNSUPPORTED;
  // the scalar gate is optional (NULL: 1, DeltaNet); then so is its gradient
  const bool scalar = gate_in == kda::kGateScalar;
  const void* ptrs[] = {q, k, v, alpha, beta, S_in, dO, dS_new, dq, dk, dv, dalpha, dbeta, dS};
  for (const void* p : ptrs) {
    const bool optional = scalar && (p == alpha || p == dalpha);
    if (!p && !optional) return KDA_ERR_NULL;
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  }
  const size_t e = (dt == KDA_BF16) ? 2 : 4;
  const size_t nh = static_cast<size_t>(N) * H;
  const size_t nst = nh * dk_ * dv_ * 4;
  auto sp = [](const void* p, size_t n) { return p ? span(p, n) : Span{0, 0}; };
  const Span ins[] = {span(q, nh * dk_ * e), span(k, nh * dk_ * e), span(v, nh * dv_ * e),
                      sp(alpha, nh * (scalar ? 1 : dk_) * 4), span(beta, nh * 4), span(S_in, nst),
                      span(dO, nh * dv_ * e), span(dS_new, nst)};
  const Span outs[] = {span(dq, nh * dk_ * e), span(dk, nh * dk_ * e), span(dv, nh * dv_ * e),
                       sp(dalpha, nh * (scalar ? 1 : dk_) * 4), span(dbeta, nh * 4), span(dS, nst)};
  constexpr int kIns = sizeof(ins) / sizeof(ins[0]), kOuts = sizeof(outs) / sizeof(outs[0]);
  for (int o = 0; o < kOuts; ++o) {
    for (int i = 0; i < kIns; ++i) {
      const bool in_place = (o == kOuts - 1) && (i == kIns - 1) && dS == dS_new;
      if (!in_place && overlap(outs[o], ins[i])) return KDA_ERR_ALIAS;
    }
    for (int p = 0; p < o; ++p)
      if (overlap(outs[o], outs[p])) return KDA_ERR_ALIAS;
  }
  const kda_status dev = check_device();
  if (dev != KDA_OK) return dev;
  kda::DecodeBwdArgs a{q,  k,  v,  alpha,  beta,  S_in, dO, dS_new, dq,  dk,
                       dv, dalpha, dbeta, dS, N, H, dk_, dv_, dt == KDA_BF16, stream};
  a.gate_in = gate_in;
  if (scalar && !alpha) a.g_alpha = nullptr;   // DeltaNet: no gate, no gate gradient
  if (kda::launch_decode_backward(a) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}


}  // namespace

extern "C" {

size_t kda_prefill_backward_workspace_bytes(int B, int T, int H, int dk, int dv) {
  if (B < 1 || H < 1 || T < 0 || !dim_ok(dk) || !dim_ok(dv)) return static_cast<size_t>(-1);
  return kda::prefill_backward_workspace(B, T, H, dk, dv);
}

kda_status kda_decode_step_backward(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta, const float* S_in,
                                    const void* dO, const float* dS_new, void* dq, void* dk,
                                    void* dv, float* dalpha, float* dbeta, float* dS, int N, int H,
                                    int dk_, int dv_, kda_dtype dt, void* stream) {
  return decode_backward_impl(q, k, v, alpha, beta, S_in, dO, dS_new, dq, dk, dv, dalpha, dbeta,
                              dS, N, H, dk_, dv_, dt, stream, kda::kGateAlpha);
}

kda_status kda_gdn_decode_step_backward(const void* q, const void* k, const void* v,
                                        const float* a, const float* beta, const float* S_in,
                                        const void* dO, const float* dS_new, void* dq, void* dk,
                                        void* dv, float* da, float* dbeta, float* dS, int N,
                                        int H, int dk_, int dv_, kda_dtype dt, void* stream) {
  return decode_backward_impl(q, k, v, a, beta, S_in, dO, dS_new, dq, dk, dv, a ? da : nullptr,
                              dbeta, dS, N, H, dk_, dv_, dt, stream, kda::kGateScalar);
}

}  // extern "C"

namespace {

kda_status prefill_backward_impl(const void* q, const void* k, const void* v, const float* alpha,
                                 const float* beta, const float* S0, const void* dO,
                                 const float* dS_T, float* dq, float* dk, float* dv,
                                 float* dalpha, float* dbeta, float* dS0, int B, int T, int H,
                                 int dk_, int dv_, kda_dtype dt, void* workspace,
                                 size_t workspace_bytes, void* stream, int gate_in,
                                 bool chunked = false) {
  if (B < 1 || H < 1 || T < 0) return KDA_ERR_SHAPE;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (!dim_ok(dk_) || !dim_ok(dv_)) return KDA_ERR_UNSUPPORTED;
  if (chunked && (dt != KDA_BF16 || dk_ != 128 || dv_ != 128)) return KDA_ERR_UNSUPPORTED;
  const bool has_tokens = T > 0;
  // the scalar gate is optional (NULL: 1, DeltaNet); then so is its gradient
  const bool scalar = gate_in == kda::kGateScalar;
  if (has_tokens && (!q || !k || !v || (!alpha && !scalar) || !beta || !dO || !dq || !dk ||
                     !dv || (!dalpha && !scalar) || !dbeta))
    return KDA_ERR_NULL;
  const void* ptrs[] = {q,  k,  v,      alpha, beta, S0,  dO,       dS_T,
                        dq, dk, dv, dalpha, dbeta, dS0, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return KDA_ERR_ALIGN;
  const size_t ws_need = chunked ? kda::prefill_backward_chunked_workspace(B, T, H, dk_, dv_)
                                 : kda::prefill_backward_workspace(B, T, H, dk_, dv_);
  if (ws_need > 0 && (workspace == nullptr || workspace_bytes < ws_need)) return KDA_ERR_WORKSPACE;

  const size_t e = (dt == KDA_BF16) ? 2 : 4;
  const size_t ntok = has_tokens ? static_cast<size_t>(B) * T * H : 0;
  const size_t nst = static_cast<size_t>(B) * H * dk_ * dv_ * 4;
  auto sp = [](const void* p, size_t n) { return p ? span(p, n) : Span{0, 0}; };
  const Span ins[] = {sp(q, ntok * dk_ * e),  sp(k, ntok * dk_ * e), sp(v, ntok * dv_ * e),
                      sp(alpha, ntok * (scalar ? 1 : dk_) * 4), sp(beta, ntok * 4), sp(S0, nst),
                      sp(dO, ntok * dv_ * e), sp(dS_T, nst)};
  const Span outs[] = {sp(dq, ntok * dk_ * 4), sp(dk, ntok * dk_ * 4), sp(dv, ntok * dv_ * 4),
                       sp(dalpha, ntok * (scalar ? 1 : dk_) * 4), sp(dbeta, ntok * 4),
                       sp(dS0, nst),
                       sp(workspace, ws_need)};
  constexpr int kIns = sizeof(ins) / sizeof(ins[0]), kOuts = sizeof(outs) / sizeof(outs[0]);
  for (int o = 0; o < kOuts; ++o) {
    for (int i = 0; i < kIns; ++i) {
      // dS0 may be dS_T itself: each element is read before it is written, by one lane.
      const bool in_place = (o == 5) && (i == 7) && dS0 == dS_T;
      if (!in_place && overlap(outs[o], ins[i])) return KDA_ERR_ALIAS;
    }
    for (int p = 0; p < o; ++p)
      if (overlap(outs[o], outs[p])) return KDA_ERR_ALIAS;
  }
  const kda_status dev = check_device();
  if (dev != KDA_OK) return dev;
  kda::PrefillBwdArgs a{q,  k,  v,      alpha, beta,      S0, dO, dS_T, dq, dk,
                        dv, dalpha, dbeta, dS0, workspace, B,  T,  H,    dk_, dv_,
                        dt == KDA_BF16, stream};
  a.gate_in = gate_in;
  if (scalar && !alpha) a.g_alpha = nullptr;   // DeltaNet: no gate, no gate gradient
  const hipError_t err =
      chunked ? kda::launch_prefill_backward_chunked(a) : kda::launch_prefill_backward(a);
  if (err != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prefill_backward(const void* q, const void* k, const void* v, const float* alpha,
                                const float* beta, const float* S0, const void* dO,
                                const float* dS_T, float* dq, float* dk, float* dv,
                                float* dalpha, float* dbeta, float* dS0, int B, int T, int H,
                                int dk_, int dv_, kda_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream) {
  return prefill_backward_impl(q, k, v, alpha, beta, S0, dO, dS_T, dq, dk, dv, dalpha, dbeta, dS0,
                               B, T, H, dk_, dv_, dt, workspace, workspace_bytes, stream,
                               kda::kGateAlpha);
}

size_t kda_prefill_backward_chunked_workspace_bytes(int B, int T, int H, int dk, int dv) {
  if (B < 1 || H < 1 || T < 0 || dk != 128 || dv != 128) return static_cast<size_t>(-1);
  return kda::prefill_backward_chunked_workspace(B, T, H, dk, dv);
}

kda_status kda_prefill_backward_chunked(const void* q, const void* k, const void* v,
                                        const float* alpha, const float* beta, const float* S0,
                                        const void* dO, const float* dS_T, float* dq, float* dk,
                                        float* dv, float* dalpha, float* dbeta, float* dS0,
                                        int B, int T, int H, int dk_, int dv_, kda_dtype dt,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_backward_impl(q, k, v, alpha, beta, S0, dO, dS_T, dq, dk, dv, dalpha, dbeta, dS0,
                               B, T, H, dk_, dv_, dt, workspace, workspace_bytes, stream,
                               kda::kGateAlpha, true);
}

kda_status kda_gdn_prefill_backward(const void* q, const void* k, const void* v, const float* a,
                                    const float* beta, const float* S0, const void* dO,
                                    const float* dS_T, float* dq, float* dk, float* dv,
                                    float* da, float* dbeta, float* dS0, int B, int T, int H,
                                    int dk_, int dv_, kda_dtype dt, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return prefill_backward_impl(q, k, v, a, beta, S0, dO, dS_T, dq, dk, dv, a ? da : nullptr,
                               dbeta, dS0, B, T, H, dk_, dv_, dt, workspace, workspace_bytes,
                               stream, kda::kGateScalar);
}

}  // extern "C"

namespace {

// Shared validation of the two prologue calls: rows >= 0, dk and dtype and
// map supported, every pointer present (when there are rows) and aligned,
// and no output overlapping an input or another output.
kda_status prologue_check(const void* const* ins, const size_t* in_bytes, int nin,
                          void* const* outs, const size_t* out_bytes, int nout, int rows, int dk,
                          kda_dtype dt, kda_qk_map qk_map) {
  if (rows < 0) return KDA_ERR_SHAPE;
  if (dt != KDA_F32 && dt != KDA_BF16) return KDA_ERR_UNSUPPORTED;
  if (!dim_ok(dk) || !qk_map_ok(qk_map)) return KDA_ERR_UNSUPPORTED;
  if (rows == 0) return KDA_OK;
  for (int i = 0; i < nin; ++i) {
    if (!ins[i]) return KDA_ERR_NULL;
    if (!aligned16(ins[i])) return KDA_ERR_ALIGN;
  }
  for (int o = 0; o < nout; ++o) {
    if (!outs[o]) return KDA_ERR_NULL;
    if (!aligned16(outs[o])) return KDA_ERR_ALIGN;
    const Span so = span(outs[o], out_bytes[o]);
    for (int i = 0; i < nin; ++i)
      if (overlap(so, span(ins[i], in_bytes[i]))) return KDA_ERR_ALIAS;
    for (int p = 0; p < o; ++p)
      if (overlap(so, span(outs[p], out_bytes[p]))) return KDA_ERR_ALIAS;
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_prologue_forward(const void* q, const void* k, const void* g, const float* b,
                                void* q_hat, void* k_hat, float* alpha, float* beta, int rows,
                                int dk, kda_dtype dt, kda_qk_map qk_map, void* stream) {
  const size_t e = (dt == KDA_BF16) ? 2 : 4;
  const size_t n = rows > 0 ? static_cast<size_t>(rows) : 0;
  const void* ins[] = {q, k, g, b};
  const size_t inb[] = {n * dk * e, n * dk * e, n * dk * e, n * 4};
  void* outs[] = {q_hat, k_hat, alpha, beta};
  const size_t outb[] = {n * dk * e, n * dk * e, n * dk * 4, n * 4};
  const kda_status st = prologue_check(ins, inb, 4, outs, outb, 4, rows, dk, dt, qk_map);
  if (st != KDA_OK || rows == 0) return st;
  const kda_status dev = check_device();
  if (dev != KDA_OK) return dev;
  kda::PrologueArgs a{};
  a.q = q; a.k = k; a.g = g; a.b = b;
  a.q_hat = q_hat; a.k_hat = k_hat; a.alpha = alpha; a.beta = beta;
  a.rows = rows; a.dk = dk; a.bf16 = dt == KDA_BF16; a.qk_map = static_cast<int>(qk_map);
  a.backward = false; a.stream = stream;
  if (kda::launch_prologue(a) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

kda_status kda_prologue_backward(const void* q, const void* k, const void* g, const float* b,
                                 const float* dq_hat, const float* dk_hat, const float* dalpha,
                                 const float* dbeta, float* dq, float* dk, float* dg, float* db,
                                 int rows, int dk_, kda_dtype dt, kda_qk_map qk_map,
                                 void* stream) {
  const size_t e = (dt == KDA_BF16) ? 2 : 4;
  const size_t n = rows > 0 ? static_cast<size_t>(rows) : 0;
  const size_t nk = n * (dk_ > 0 ? dk_ : 0);
  const void* ins[] = {q, k, g, b, dq_hat, dk_hat, dalpha, dbeta};
  const size_t inb[] = {nk * e, nk * e, nk * e, n * 4, nk * 4, nk * 4, nk * 4, n * 4};
  void* outs[] = {dq, dk, dg, db};
  const size_t outb[] = {nk * 4, nk * 4, nk * 4, n * 4};
  const kda_status st = prologue_check(ins, inb, 8, outs, outb, 4, rows, dk_, dt, qk_map);
  if (st != KDA_OK || rows == 0) return st;
  const kda_status dev = check_device();
  if (dev != KDA_OK) return dev;
  kda::PrologueArgs a{};
  a.q = q; a.k = k; a.g = g; a.b = b;
  a.dq_hat = dq_hat; a.dk_hat = dk_hat; a.dalpha = dalpha; a.dbeta = dbeta;
  a.d_q = dq; a.d_k = dk; a.d_g = dg; a.d_b = db;
  a.rows = rows; a.dk = dk_; a.bf16 = dt == KDA_BF16; a.qk_map = static_cast<int>(qk_map);
  a.backward = true; a.stream = stream;
  if (kda::launch_prologue(a) != hipSuccess) return KDA_ERR_HIP;
  return KDA_OK;
}

}  // extern "C"


extern "C" {

// Every call on a device shares that device's scratch array: the records of
// one segment and the carried state are overwritten before they are read, so
// nothing needs clearing between calls, but two calls in flight at once on
// one device (two streams, two threads) race on it.
kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta, const float* S0,
                                       void* o, float* S_T, int B, int T, int H, int dk, int dv,
                                       int C, kda_dtype dt, void* stream) {
  // Segments of records sized so that the records and the carried state fit
  // the scratch array: more segments than kda_prefill_chunked may use, with
  // bit-identical results (a segment boundary does not change the arithmetic).
  const size_t carry = (B > 0 && H > 0 && dk > 0 && dv > 0)
                           ? static_cast<size_t>(B) * H * dk * dv * 4 : 0;
  const size_t budget =
      carry < kda::kNoallocScratchBytes ? kda::kNoallocScratchBytes - carry : 1;
  return prefill_impl(q, k, v, alpha, beta, S0, o, S_T, B, T, H, dk, dv, C, dt, kda::kGateAlpha,
                      0, nullptr, 0, stream, budget, /*use_scratch=*/true);
}

}  // extern "C"
