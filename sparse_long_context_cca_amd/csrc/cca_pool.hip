// Global-aware pooling (and its variants) and the visibility-table export.
//
// Pooling (digest at digest.lyk-ai.com/posts/2412.12465, "Method", pooling
// formula; ICML 2025 article at changsha.jmyizhao.com, global-aware pooling
// paragraph: the last token's query scores every token of its group): for
// group j of kv head (b, hk),
//   qbar = mean_{h in heads of hk} Q[b, h, (j+1)g-1, :]
//   a    = softmax_tau(qbar . K[jg+tau] / sqrt(d))
//   CK_j = sum_tau a_tau K[jg+tau],  CV_j = sum_tau a_tau V[jg+tau].
// The other modes (mean of per-head softmaxes, mean, max) are described with
// the per-group routine in cca_pool_group.hpp.
//
// One wave64 per group.  Each lane owns a 16-byte slice of one key row, so a
// wave load covers 1 KB of the group's contiguous K (or V) rows and every byte
// of K and V is read exactly once (twice for K in the per-head mode).
// HBM-bound: reads K, V and the G query rows at group ends, writes CK and CV
// (fp16 for bf16 inputs, fp32 for fp32 inputs; rounded once, to nearest even).
#include "cca_device.hpp"
#include "cca_internal.hpp"
#include "cca_pool_group.hpp"

namespace cca {

__global__ void visibility_kernel(int L, int g, int w, int32_t* __restrict__ nc,
                                  int32_t* __restrict__ lo, int32_t* __restrict__ gl) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t < L) {
    nc[t] = n_core(t, g, w);
    lo[t] = win_lo(t, w);
  }
  if (gl != nullptr && t < L / g) gl[t] = group_last(t, g);
}

hipError_t launch_visibility(int L, int g, int w, int32_t* n_core_tab, int32_t* win_lo_tab,
                             int32_t* group_last_tab, hipStream_t s) {
  const int threads = 256;
  const int blocks = (L + threads - 1) / threads;
  hipLaunchKernelGGL(visibility_kernel, dim3(blocks), dim3(threads), 0, s, L, g, w, n_core_tab,
                     win_lo_tab, L / g > 0 ? group_last_tab : nullptr);
  return hipGetLastError();
}

namespace {

template <int DT, int D, int MODE>
__global__ __launch_bounds__(256) void pool_kernel(const void* __restrict__ q_,
                                                   const void* __restrict__ k_,
                                                   const void* __restrict__ v_,
                                                   void* __restrict__ ck_, void* __restrict__ cv_,
                                                   float* __restrict__ weights, int m_cap,
                                                   const int32_t* __restrict__ q_start,
                                                   const int32_t* __restrict__ q_len, int gpb,
                                                   int B, int Hq, int Hkv, int Lq, int Lk, int g,
                                                   float scale_log2) {
  typedef RowLanes<DT, D> RL;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // one wave per (b, kv head, group slot); gpb slots per (b, kv head)
  const long slot = (long)blockIdx.x * (blockDim.x >> 6) + wave;
  if (slot >= (long)B * Hkv * gpb) return;
  const int jl = (int)(slot % gpb);
  const long bh = slot / gpb;  // b * Hkv + hk
  const int hk = (int)(bh % Hkv);
  const int b = (int)(bh / Hkv);
  const int G = Hq / Hkv;
  // the groups whose last token lies among sequence b's rows qs .. qs+ql-1
  const SeqRows sr = seq_rows(q_start, q_len, b, Lq, Lk, g, 1, 0x7fffffff);
  if (!sr.ok) return;
  const int j = (sr.qs + g) / g - 1 + jl;  // first such group, plus jl
  if (j >= (sr.qs + sr.ql) / g || j >= m_cap) return;
  const int m = Lq / g;  // weights rows per (b, kv head) (full prefill only)
  const char* qb = static_cast<const char*>(q_);
  const char* kb = static_cast<const char*>(k_);
  const char* vb = static_cast<const char*>(v_);
  const long kv_row0 = (long)bh * Lk + (long)j * g;  // first token of the group
  const int last = group_last(j, g) - sr.qs;          // local row of its last token
  auto krow = [&](int tau) { return kb + (kv_row0 + tau) * D * RL::ES; };
  auto vrow = [&](int tau) { return vb + (kv_row0 + tau) * D * RL::ES; };
  auto qrow = [&](int h) { return qb + ((long)(b * Hq + hk * G + h) * Lq + last) * D * RL::ES; };
  float acck[RL::EPL], accv[RL::EPL];
  float* wout = weights != nullptr ? weights + ((long)bh * m + j) * g : nullptr;
  pool_group<DT, D, MODE>(krow, vrow, qrow, g, G, scale_log2, acck, accv, wout);
  if (lane < RL::LPK) {  // cores in the core dtype (same element size as the input)
    const long crow = ((long)bh * m_cap + j) * D + lane * RL::EPL;
    Row16<core_dt(DT)>::store(static_cast<char*>(ck_) + crow * RL::ES, acck);
    Row16<core_dt(DT)>::store(static_cast<char*>(cv_) + crow * RL::ES, accv);
  }
}

template <int DT, int D, int MODE>
void launch_pool_t(const void* q, const void* k, const void* v, void* ck, void* cv, int m_cap,
                   float* weights, const Shape& sh, const RowRange& rr, hipStream_t s) {
  // group slots per (b, kv head): every group of a full prefill; at most
  // Lq / g + 1 group ends fall among Lq consecutive rows of a chunk
  const int gpb = rr.q_start == nullptr ? rr.Lq / sh.g : rr.Lq / sh.g + 1;
  const long slots = (long)sh.B * sh.Hkv * gpb;
  const int waves = 4;
  const long blocks = (slots + waves - 1) / waves;
  if (blocks == 0) return;
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((pool_kernel<DT, D, MODE>), dim3((unsigned)blocks), dim3(64 * waves), 0, s, q, k,
                     v, ck, cv, weights, m_cap, rr.q_start, rr.q_len, gpb, sh.B, sh.Hq, sh.Hkv,
                     rr.Lq, rr.Lk, sh.g, scale_log2);
}

template <int DT, int D>
void launch_pool_mode(int mode, const void* q, const void* k, const void* v, void* ck, void* cv,
                      int m_cap, float* weights, const Shape& sh, const RowRange& rr,
                      hipStream_t s) {
  switch (mode) {
    case kPoolSoftmaxHeads: launch_pool_t<DT, D, kPoolSoftmaxHeads>(q, k, v, ck, cv, m_cap, weights, sh, rr, s); break;
    case kPoolMean: launch_pool_t<DT, D, kPoolMean>(q, k, v, ck, cv, m_cap, weights, sh, rr, s); break;
    case kPoolMax: launch_pool_t<DT, D, kPoolMax>(q, k, v, ck, cv, m_cap, weights, sh, rr, s); break;
    default: launch_pool_t<DT, D, kPoolSoftmax>(q, k, v, ck, cv, m_cap, weights, sh, rr, s); break;
  }
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, const void* v, void* ck, void* cv, int m_cap,
                       float* weights, const Shape& sh, const RowRange& rr, int dt, int mode,
                       hipStream_t s) {
  if (dt == 0) {
    if (sh.d == 64) launch_pool_mode<0, 64>(mode, q, k, v, ck, cv, m_cap, weights, sh, rr, s);
    else launch_pool_mode<0, 128>(mode, q, k, v, ck, cv, m_cap, weights, sh, rr, s);
  } else {
    if (sh.d == 64) launch_pool_mode<1, 64>(mode, q, k, v, ck, cv, m_cap, weights, sh, rr, s);
    else launch_pool_mode<1, 128>(mode, q, k, v, ck, cv, m_cap, weights, sh, rr, s);
  }
  return hipGetLastError();
}

}  // namespace cca
