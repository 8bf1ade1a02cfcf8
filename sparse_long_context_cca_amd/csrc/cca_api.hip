// C ABI of the CCA attention library: argument validation on the host, then
// kernel launches on the caller's stream.  Nothing here allocates memory or
// synchronises.  See include/cca.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdarg>
#include <mutex>
#include <string>

#include "../../include/cca.h"
#include "cca_device.hpp"
#include "cca_pool_group.hpp"
#include "cca_internal.hpp"

namespace cca {

hipError_t compute_units(int* out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int counts[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (counts[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    counts[dev] = n > 0 ? n : 1;
  }
  *out = counts[dev];
  return hipSuccess;
}

}  // namespace cca

namespace {

thread_local std::string g_last_error;

cca_status fail(cca_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cca_status ok() {
  g_last_error.clear();
  return CCA_OK;
}

cca_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CCA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const long long kMaxElems = 1LL << 40;

#define REQUIRE_PTR(p)                                                                  \
  do {                                                                                  \
    if ((p) == nullptr) return fail(CCA_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);     \
    if (!aligned16(p)) return fail(CCA_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

// Checks shared by every entry point that takes a head layout.
cca_status check_heads(const char* fn, int B, int Hq, int Hkv, int d, int dt) {
  if (B < 1 || Hq < 1 || Hkv < 1)
    return fail(CCA_ERR_INVALID_ARG, "%s: B=%d Hq=%d Hkv=%d must be >= 1", fn, B, Hq, Hkv);
  if (dt != CCA_F32 && dt != CCA_BF16)
    return fail(CCA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dt);
  if (Hq % Hkv != 0)
    return fail(CCA_ERR_UNSUPPORTED, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
  if (d != 64 && d != 128) return fail(CCA_ERR_UNSUPPORTED, "%s: head dim d=%d not in {64,128}", fn, d);
  return CCA_OK;
}

cca_status check_out_dt(const char* fn, int out_dt, int dt) {
  if (out_dt != CCA_F32 && out_dt != CCA_BF16)
    return fail(CCA_ERR_INVALID_ARG, "%s: unknown out dtype %d", fn, out_dt);
  if (out_dt != dt && out_dt != CCA_F32)
    return fail(CCA_ERR_UNSUPPORTED, "%s: out dtype must be the input dtype or fp32", fn);
  return CCA_OK;
}

// Sequence lengths, positions, g, w, R and m_cap stay below 2^30, so that
// the kernels' 32-bit sums of two of them (a position plus g or w, the end of
// a row block) cannot overflow.  Pass -1 for an extent that does not apply.
const int kMaxExtent = (1 << 30) - 1;
cca_status check_extents(const char* fn, int L, int g, int w, int other) {
  if (L > kMaxExtent || g > kMaxExtent || w > kMaxExtent || other > kMaxExtent)
    return fail(CCA_ERR_UNSUPPORTED, "%s: lengths, g, w, R and m_cap must be below 2^30", fn);
  return CCA_OK;
}

cca_status check_sizes(const char* fn, long long a, long long b, long long c) {
  if (a > kMaxElems || b > kMaxElems || c > kMaxElems)
    return fail(CCA_ERR_UNSUPPORTED, "%s: a buffer exceeds 2^40 elements", fn);
  return CCA_OK;
}

}  // namespace

extern "C" {

int cca_version(void) { return 20000; }

int cca_core_dtype(int dt) {
  if (dt == CCA_F32) return CCA_F32;
  if (dt == CCA_BF16) return CCA_F16;
  return -1;
}

const char* cca_status_string(int status) {
  switch (status) {
    case CCA_OK: return "CCA_OK";
    case CCA_ERR_INVALID_ARG: return "CCA_ERR_INVALID_ARG";
    case CCA_ERR_UNSUPPORTED: return "CCA_ERR_UNSUPPORTED";
    case CCA_ERR_CAPACITY: return "CCA_ERR_CAPACITY";
    case CCA_ERR_HIP: return "CCA_ERR_HIP";
    default: return "CCA_ERR_UNKNOWN";
  }
}

const char* cca_last_error(void) { return g_last_error.c_str(); }

cca_status cca_visibility_table(int L, int g, int w, int32_t* n_core, int32_t* win_lo,
                                int32_t* group_last, void* stream) {
  const char* fn = "cca_visibility_table";
  if (L < 1 || g < 1 || w < 1)
    return fail(CCA_ERR_INVALID_ARG, "%s: L=%d g=%d w=%d must be >= 1", fn, L, g, w);
  if (check_extents(fn, L, g, w, -1) != CCA_OK) return CCA_ERR_UNSUPPORTED;
  REQUIRE_PTR(n_core);
  REQUIRE_PTR(win_lo);
  if (L / g > 0) REQUIRE_PTR(group_last);
  return from_hip(cca::launch_visibility(L, g, w, n_core, win_lo, group_last,
                                         static_cast<hipStream_t>(stream)),
                  fn);
}

namespace {

// Pooling rule: a known mode, and at most kPoolHeadsMaxG heads per kv head for
// the per-head rule.
cca_status check_pool_mode(const char* fn, int mode, int Hq, int Hkv) {
  if (mode < CCA_POOL_SOFTMAX || mode > CCA_POOL_MAX)
    return fail(CCA_ERR_INVALID_ARG, "%s: unknown pooling mode %d", fn, mode);
  if (mode == CCA_POOL_SOFTMAX_HEADS && Hq / Hkv > cca::kPoolHeadsMaxG)
    return fail(CCA_ERR_UNSUPPORTED, "%s: per-head pooling needs G <= %d (G=%d)", fn,
                cca::kPoolHeadsMaxG, Hq / Hkv);
  return CCA_OK;
}

cca_status pool_core(const char* fn, const void* q, const void* k, const void* v, void* core_k,
                     void* core_v, int m_cap, float* weights, int B, int Hq, int Hkv, int L, int d,
                     int g, int dt, int mode, void* stream) {
  if (L < 1 || g < 1) return fail(CCA_ERR_INVALID_ARG, "%s: L=%d g=%d must be >= 1", fn, L, g);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_extents(fn, L, g, -1, m_cap);
  if (st != CCA_OK) return st;
  st = check_pool_mode(fn, mode, Hq, Hkv);
  if (st != CCA_OK) return st;
  if (mode == CCA_POOL_MAX && weights != nullptr)
    return fail(CCA_ERR_INVALID_ARG, "%s: max pooling has no weights (weights must be NULL)", fn);
  const bool reads_q = mode == CCA_POOL_SOFTMAX || mode == CCA_POOL_SOFTMAX_HEADS;
  if (reads_q) REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  const int m = L / g;
  if (m_cap < m) return fail(CCA_ERR_CAPACITY, "%s: m_cap=%d < L/g=%d", fn, m_cap, m);
  st = check_sizes(fn, (long long)B * Hq * L * d, (long long)B * Hkv * L * d,
                   (long long)B * Hkv * m_cap * d);
  if (st != CCA_OK) return st;
  if (m == 0) return ok();  // no complete group: nothing to write
  REQUIRE_PTR(core_k);
  REQUIRE_PTR(core_v);
  if (weights != nullptr && !aligned16(weights))
    return fail(CCA_ERR_INVALID_ARG, "%s: weights is not 16-byte aligned", fn);
  cca::Shape sh{B, Hq, Hkv, L, d, g, 1};
  cca::RowRange rr;
  rr.Lq = rr.Lk = L;
  return from_hip(cca::launch_pool(q, k, v, core_k, core_v, m_cap, weights, sh, rr, dt, mode,
                                   static_cast<hipStream_t>(stream)),
                  fn);
}

// Per-sequence row arrays of the chunked calls: device int32 [B], 4-byte aligned.
cca_status check_rows(const char* fn, const int32_t* q_start, const int32_t* q_len, int Lq, int Lk) {
  if (q_start == nullptr || q_len == nullptr)
    return fail(CCA_ERR_INVALID_ARG, "%s: q_start and q_len must not be NULL", fn);
  if ((reinterpret_cast<uintptr_t>(q_start) & 3u) != 0 || (reinterpret_cast<uintptr_t>(q_len) & 3u) != 0)
    return fail(CCA_ERR_INVALID_ARG, "%s: q_start / q_len are not 4-byte aligned", fn);
  if (Lq < 1 || Lk < 1) return fail(CCA_ERR_INVALID_ARG, "%s: Lq=%d Lk=%d must be >= 1", fn, Lq, Lk);
  return CCA_OK;
}

}  // namespace

cca_status cca_pool_core(const void* q, const void* k, const void* v, void* core_k, void* core_v,
                         int m_cap, float* weights, int B, int Hq, int Hkv, int L, int d, int g,
                         int dt, void* stream) {
  return pool_core("cca_pool_core", q, k, v, core_k, core_v, m_cap, weights, B, Hq, Hkv, L, d, g,
                   dt, CCA_POOL_SOFTMAX, stream);
}

cca_status cca_pool_core_ex(const void* q, const void* k, const void* v, void* core_k,
                            void* core_v, int m_cap, float* weights, int B, int Hq, int Hkv, int L,
                            int d, int g, int dt, int mode, void* stream) {
  return pool_core("cca_pool_core_ex", q, k, v, core_k, core_v, m_cap, weights, B, Hq, Hkv, L, d,
                   g, dt, mode, stream);
}

cca_status cca_pool_core_chunk(const void* q, const void* k, const void* v, void* core_k,
                               void* core_v, int m_cap, const int32_t* q_start,
                               const int32_t* q_len, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                               int g, int dt, int mode, void* stream) {
  const char* fn = "cca_pool_core_chunk";
  if (g < 1) return fail(CCA_ERR_INVALID_ARG, "%s: g=%d must be >= 1", fn, g);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_pool_mode(fn, mode, Hq, Hkv);
  if (st != CCA_OK) return st;
  st = check_rows(fn, q_start, q_len, Lq, Lk);
  if (st != CCA_OK) return st;
  st = check_extents(fn, Lq > Lk ? Lq : Lk, g, -1, m_cap);
  if (st != CCA_OK) return st;
  if (mode == CCA_POOL_SOFTMAX || mode == CCA_POOL_SOFTMAX_HEADS) REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  if (m_cap < 0) return fail(CCA_ERR_INVALID_ARG, "%s: m_cap=%d", fn, m_cap);
  st = check_sizes(fn, (long long)B * Hq * Lq * d, (long long)B * Hkv * Lk * d,
                   (long long)B * Hkv * m_cap * d);
  if (st != CCA_OK) return st;
  if (m_cap == 0) return ok();  // no core slot: nothing to write
  REQUIRE_PTR(core_k);
  REQUIRE_PTR(core_v);
  cca::Shape sh{B, Hq, Hkv, Lq, d, g, 1};
  cca::RowRange rr;
  rr.q_start = q_start;
  rr.q_len = q_len;
  rr.Lq = Lq;
  rr.Lk = Lk;
  return from_hip(cca::launch_pool(q, k, v, core_k, core_v, m_cap, nullptr, sh, rr, dt, mode,
                                   static_cast<hipStream_t>(stream)),
                  fn);
}

cca_status cca_attn_prefill_ex(const void* q, const void* k, const void* v, const void* core_k,
                               const void* core_v, int m_cap, void* out, int out_dt, int B,
                               int Hq, int Hkv, int L, int d, int g, int w, int dt,
                               int kernel, void* stream) {
  const char* fn = "cca_attn_prefill";
  if (L < 1 || g < 1 || w < 1)
    return fail(CCA_ERR_INVALID_ARG, "%s: L=%d g=%d w=%d must be >= 1", fn, L, g, w);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_extents(fn, L, g, w, m_cap);
  if (st != CCA_OK) return st;
  st = check_out_dt(fn, out_dt, dt);
  if (st != CCA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  const int m = L / g;
  if (m_cap < m) return fail(CCA_ERR_CAPACITY, "%s: m_cap=%d < L/g=%d", fn, m_cap, m);
  // Cores are read only when some query sees one: n_core(L-1) > 0.
  if (cca::n_core(L - 1, g, w) > 0) {
    REQUIRE_PTR(core_k);
    REQUIRE_PTR(core_v);
  }
  st = check_sizes(fn, (long long)B * Hq * L * d, (long long)B * Hkv * L * d,
                   (long long)B * Hkv * m_cap * d);
  if (st != CCA_OK) return st;
  if (kernel < 0 || kernel > 2) return fail(CCA_ERR_INVALID_ARG, "%s: kernel=%d", fn, kernel);
  if (kernel == 2 && dt != CCA_BF16)
    return fail(CCA_ERR_UNSUPPORTED, "%s: the matrix-core kernel takes bf16 inputs", fn);
  if (kernel == 0) kernel = (dt == CCA_BF16) ? 2 : 1;
  cca::Shape sh{B, Hq, Hkv, L, d, g, w};
  cca::RowRange rr;
  rr.Lq = rr.Lk = L;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kernel == 2)
    return from_hip(cca::launch_prefill_mfma(q, k, v, core_k, core_v, m_cap, out, out_dt, sh, rr, nullptr, s),
                    fn);
  return from_hip(
      cca::launch_prefill_valu(q, k, v, core_k, core_v, m_cap, out, out_dt, sh, rr, nullptr, dt, s), fn);
}

cca_status cca_attn_prefill_train(const void* q, const void* k, const void* v, const void* core_k,
                                  const void* core_v, int m_cap, void* out, int out_dt,
                                  float* lse, int B, int Hq, int Hkv, int L, int d, int g, int w,
                                  int dt, void* stream) {
  const char* fn = "cca_attn_prefill_train";
  if (lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(CCA_ERR_INVALID_ARG, "%s: lse is NULL or not 4-byte aligned", fn);
  if (L < 1 || g < 1 || w < 1)
    return fail(CCA_ERR_INVALID_ARG, "%s: L=%d g=%d w=%d must be >= 1", fn, L, g, w);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_extents(fn, L, g, w, m_cap);
  if (st != CCA_OK) return st;
  st = check_out_dt(fn, out_dt, dt);
  if (st != CCA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  const int m = L / g;
  if (m_cap < m) return fail(CCA_ERR_CAPACITY, "%s: m_cap=%d < L/g=%d", fn, m_cap, m);
  if (cca::n_core(L - 1, g, w) > 0) {
    REQUIRE_PTR(core_k);
    REQUIRE_PTR(core_v);
  }
  st = check_sizes(fn, (long long)B * Hq * L * d, (long long)B * Hkv * L * d,
                   (long long)B * Hkv * m_cap * d);
  if (st != CCA_OK) return st;
  cca::Shape sh{B, Hq, Hkv, L, d, g, w};
  cca::RowRange rr;
  rr.Lq = rr.Lk = L;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == CCA_BF16)
    return from_hip(cca::launch_prefill_mfma(q, k, v, core_k, core_v, m_cap, out, out_dt, sh, rr, lse, s),
                    fn);
  return from_hip(
      cca::launch_prefill_valu(q, k, v, core_k, core_v, m_cap, out, out_dt, sh, rr, lse, dt, s), fn);
}

size_t cca_attn_backward_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int g, int dt) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || d < 1 || g < 1) return 0;
  if (dt != CCA_F32 && dt != CCA_BF16) return 0;
  return cca::backward_workspace_bytes(B, Hq, Hkv, L, d, g, dt);
}

cca_status cca_attn_backward(const void* q, const void* k, const void* v, const void* core_k,
                             const void* core_v, int m_cap, const void* out, const float* lse,
                             const void* dout, float* dq, float* dk, float* dv, void* workspace,
                             size_t workspace_bytes, int B, int Hq, int Hkv, int L, int d, int g,
                             int w, int dt, int pool_mode, void* stream) {
  const char* fn = "cca_attn_backward";
  if (L < 1 || g < 1 || w < 1)
    return fail(CCA_ERR_INVALID_ARG, "%s: L=%d g=%d w=%d must be >= 1", fn, L, g, w);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_extents(fn, L, g, w, m_cap);
  if (st != CCA_OK) return st;
  st = check_pool_mode(fn, pool_mode, Hq, Hkv);
  if (st != CCA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  REQUIRE_PTR(lse);
  REQUIRE_PTR(dout);
  REQUIRE_PTR(dq);
  REQUIRE_PTR(dk);
  REQUIRE_PTR(dv);
  const int m = L / g;
  if (m_cap < m) return fail(CCA_ERR_CAPACITY, "%s: m_cap=%d < L/g=%d", fn, m_cap, m);
  if (m > 0) {
    REQUIRE_PTR(core_k);
    REQUIRE_PTR(core_v);
  }
  st = check_sizes(fn, (long long)B * Hq * L * d, (long long)B * Hkv * L * d,
                   (long long)B * Hkv * m_cap * d);
  if (st != CCA_OK) return st;
  if ((long long)B * Hkv > 65535 || (long long)Hq > 65535)
    return fail(CCA_ERR_UNSUPPORTED, "%s: B*Hkv or Hq exceeds 65535", fn);
  const size_t need = cca::backward_workspace_bytes(B, Hq, Hkv, L, d, g, dt);
  if (workspace_bytes < need)
    return fail(CCA_ERR_CAPACITY, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes, need);
  REQUIRE_PTR(workspace);
  cca::Shape sh{B, Hq, Hkv, L, d, g, w};
  return from_hip(cca::launch_backward(q, k, v, core_k, core_v, m_cap, out, lse, dout, dq, dk, dv,
                                       workspace, sh, dt, pool_mode, static_cast<hipStream_t>(stream)),
                  fn);
}

cca_status cca_attn_prefill_chunk(const void* q, const void* k, const void* v, const void* core_k,
                                  const void* core_v, int m_cap, void* out, int out_dt,
                                  const int32_t* q_start, const int32_t* q_len, int B, int Hq,
                                  int Hkv, int Lq, int Lk, int d, int g, int w, int dt,
                                  void* stream) {
  const char* fn = "cca_attn_prefill_chunk";
  if (g < 1 || w < 1) return fail(CCA_ERR_INVALID_ARG, "%s: g=%d w=%d must be >= 1", fn, g, w);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_out_dt(fn, out_dt, dt);
  if (st != CCA_OK) return st;
  st = check_rows(fn, q_start, q_len, Lq, Lk);
  if (st != CCA_OK) return st;
  st = check_extents(fn, Lq > Lk ? Lq : Lk, g, w, m_cap);
  if (st != CCA_OK) return st;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  if (m_cap < 0) return fail(CCA_ERR_INVALID_ARG, "%s: m_cap=%d", fn, m_cap);
  if (m_cap > 0) {
    REQUIRE_PTR(core_k);
    REQUIRE_PTR(core_v);
  }
  st = check_sizes(fn, (long long)B * Hq * Lq * d, (long long)B * Hkv * Lk * d,
                   (long long)B * Hkv * m_cap * d);
  if (st != CCA_OK) return st;
  cca::Shape sh{B, Hq, Hkv, Lq, d, g, w};
  cca::RowRange rr;
  rr.q_start = q_start;
  rr.q_len = q_len;
  rr.Lq = Lq;
  rr.Lk = Lk;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dt == CCA_BF16)
    return from_hip(cca::launch_prefill_mfma(q, k, v, core_k, core_v, m_cap, out, out_dt, sh, rr, nullptr, s),
                    fn);
  return from_hip(
      cca::launch_prefill_valu(q, k, v, core_k, core_v, m_cap, out, out_dt, sh, rr, nullptr, dt, s), fn);
}

cca_status cca_cache_fill_ring(const void* k, const void* v, void* ring_k, void* ring_v, int R,
                               const int32_t* seq_len, int B, int Hkv, int Lk, int d, int dt,
                               void* stream) {
  const char* fn = "cca_cache_fill_ring";
  cca_status st = check_heads(fn, B, Hkv, Hkv, d, dt);
  if (st != CCA_OK) return st;
  if (R < 1 || Lk < 1) return fail(CCA_ERR_INVALID_ARG, "%s: R=%d Lk=%d must be >= 1", fn, R, Lk);
  st = check_extents(fn, Lk, -1, -1, R);
  if (st != CCA_OK) return st;
  if (seq_len == nullptr || (reinterpret_cast<uintptr_t>(seq_len) & 3u) != 0)
    return fail(CCA_ERR_INVALID_ARG, "%s: seq_len is NULL or not 4-byte aligned", fn);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(ring_k);
  REQUIRE_PTR(ring_v);
  st = check_sizes(fn, (long long)B * Hkv * Lk * d, (long long)B * Hkv * R * d, 0);
  if (st != CCA_OK) return st;
  if ((long long)B * Hkv > 65535)
    return fail(CCA_ERR_UNSUPPORTED, "%s: B*Hkv=%lld exceeds 65535", fn, (long long)B * Hkv);
  return from_hip(cca::launch_fill_ring(k, v, ring_k, ring_v, R, seq_len, B, Hkv, Lk, d,
                                        dt == CCA_BF16 ? 2 : 4, static_cast<hipStream_t>(stream)),
                  fn);
}

cca_status cca_attn_prefill(const void* q, const void* k, const void* v, const void* core_k,
                            const void* core_v, int m_cap, void* out, int out_dt, int B,
                            int Hq, int Hkv, int L, int d, int g, int w, int dt,
                            void* stream) {
  return cca_attn_prefill_ex(q, k, v, core_k, core_v, m_cap, out, out_dt, B, Hq, Hkv, L, d, g, w,
                             dt, 0, stream);
}

size_t cca_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int m_cap, int g, int w) {
  if (B < 1 || Hq < 1 || Hkv < 1 || d < 1 || m_cap < 0 || g < 1 || w < 1) return 0;
  return cca::decode_plan(B, Hq, Hkv, d, m_cap, g, w).ws_bytes;
}

namespace {

cca_status attn_decode(const char* fn, const void* q_t, const void* k_t, const void* v_t,
                       void* ring_k, void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                       int32_t* pos, int advance_pos, void* out, int out_dt, void* workspace,
                       size_t workspace_bytes, int B, int Hq, int Hkv, int d, int g, int w,
                       int dt, int pool_mode, void* stream, bool use_scratch = false) {
  if (g < 1 || w < 1) return fail(CCA_ERR_INVALID_ARG, "%s: g=%d w=%d must be >= 1", fn, g, w);
  cca_status st = check_heads(fn, B, Hq, Hkv, d, dt);
  if (st != CCA_OK) return st;
  st = check_pool_mode(fn, pool_mode, Hq, Hkv);
  if (st != CCA_OK) return st;
  st = check_out_dt(fn, out_dt, dt);
  if (st != CCA_OK) return st;
  st = check_extents(fn, R, g, w, m_cap);
  if (st != CCA_OK) return st;
  REQUIRE_PTR(q_t);
  REQUIRE_PTR(k_t);
  REQUIRE_PTR(v_t);
  REQUIRE_PTR(ring_k);
  REQUIRE_PTR(ring_v);
  REQUIRE_PTR(out);
  if (m_cap < 0) return fail(CCA_ERR_INVALID_ARG, "%s: m_cap=%d", fn, m_cap);
  if (m_cap > 0) {
    REQUIRE_PTR(core_k);
    REQUIRE_PTR(core_v);
  }
  if (pos == nullptr) return fail(CCA_ERR_INVALID_ARG, "%s: pos is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(pos) & 3u) != 0)
    return fail(CCA_ERR_INVALID_ARG, "%s: pos is not 4-byte aligned", fn);
  const int need_r = w > g ? w : g;
  if (R < need_r) return fail(CCA_ERR_CAPACITY, "%s: ring R=%d < max(w,g)=%d", fn, R, need_r);
  st = check_sizes(fn, (long long)B * Hkv * R * d, (long long)B * Hkv * m_cap * d,
                   (long long)B * Hq * d);
  if (st != CCA_OK) return st;
  cca::DecodePlan plan = cca::decode_plan(B, Hq, Hkv, d, m_cap, g, w);
  if (use_scratch) {
    // the split states go to the library's fixed device scratch
    if (plan.ws_bytes > cca::kDecodeScratchBytes)
      return fail(CCA_ERR_CAPACITY, "%s: the split states need %zu bytes, beyond the %zu-byte scratch", fn,
                  plan.ws_bytes, cca::kDecodeScratchBytes);
    const hipError_t e = cca::decode_scratch(&workspace);
    if (e != hipSuccess) return from_hip(e, fn);
  } else {
    if (workspace_bytes < plan.ws_bytes)
      return fail(CCA_ERR_CAPACITY, "%s: workspace %zu bytes < %zu needed", fn, workspace_bytes,
                  plan.ws_bytes);
    if (plan.ws_bytes > 0) REQUIRE_PTR(workspace);
  }
  cca::Shape sh{B, Hq, Hkv, 0, d, g, w};
  return from_hip(cca::launch_decode(q_t, k_t, v_t, ring_k, ring_v, R, core_k, core_v, m_cap, pos,
                                     advance_pos, out, out_dt, workspace, plan, sh, dt, pool_mode,
                                     static_cast<hipStream_t>(stream)),
                  fn);
}

}  // namespace

cca_status cca_attn_decode(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                           void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                           int32_t* pos, int advance_pos, void* out, int out_dt,
                           void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int d,
                           int g, int w, int dt, void* stream) {
  return attn_decode("cca_attn_decode", q_t, k_t, v_t, ring_k, ring_v, R, core_k, core_v, m_cap,
                     pos, advance_pos, out, out_dt, workspace, workspace_bytes, B, Hq, Hkv, d, g, w,
                     dt, CCA_POOL_SOFTMAX, stream);
}

cca_status cca_attn_decode_ex(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                              void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                              int32_t* pos, int advance_pos, void* out, int out_dt,
                              void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                              int d, int g, int w, int dt, int pool_mode, void* stream) {
  return attn_decode("cca_attn_decode_ex", q_t, k_t, v_t, ring_k, ring_v, R, core_k, core_v, m_cap,
                     pos, advance_pos, out, out_dt, workspace, workspace_bytes, B, Hq, Hkv, d, g, w,
                     dt, pool_mode, stream);
}

cca_status cca_attn_decode_scratch(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                                   void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                                   int32_t* pos, int advance_pos, void* out, int out_dt, int B,
                                   int Hq, int Hkv, int d, int g, int w, int dt, int pool_mode,
                                   void* stream) {
  return attn_decode("cca_attn_decode_scratch", q_t, k_t, v_t, ring_k, ring_v, R, core_k, core_v,
                     m_cap, pos, advance_pos, out, out_dt, nullptr, 0, B, Hq, Hkv, d, g, w, dt,
                     pool_mode, stream, true);
}

size_t cca_decode_scratch_bytes(void) { return cca::kDecodeScratchBytes; }

}  // extern "C"
