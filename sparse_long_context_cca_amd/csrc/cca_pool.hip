// Global-aware pooling and the visibility-table export.
//
// Pooling (digest at digest.lyk-ai.com/posts/2412.12465, "Method", pooling
// formula; ICML 2025 article at changsha.jmyizhao.com, global-aware pooling
// paragraph: the last token's query scores every token of its group): for
// group j of kv head (b, hk),
//   qbar = mean_{h in heads of hk} Q[b, h, (j+1)g-1, :]
//   a    = softmax_tau(qbar . K[jg+tau] / sqrt(d))
//   CK_j = sum_tau a_tau K[jg+tau],  CV_j = sum_tau a_tau V[jg+tau].
//
// One wave64 per group.  Each lane owns a 16-byte slice of one key row, so a
// wave load covers 1 KB of the group's contiguous K (or V) rows and every byte
// of K and V is read exactly once.  The g keys are consumed in chunks of
// KPW keys (one per lane group); each lane group keeps its own online-softmax
// state (max, sum, weighted K and V slices) and the lane groups are merged at
// the end.  Works for any g >= 1.  HBM-bound: reads K, V and the G query rows
// at group ends, writes CK and CV.
#include "cca_device.hpp"
#include "cca_internal.hpp"

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

template <int DT>
struct Vec16;  // 16 bytes of a row as floats
template <>
struct Vec16<0> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void load(const void* p, float* x) {
    float4 v = *reinterpret_cast<const float4*>(p);
    x[0] = v.x; x[1] = v.y; x[2] = v.z; x[3] = v.w;
  }
  static __device__ __forceinline__ void store(void* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <>
struct Vec16<1> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void load(const void* p, float* x) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void store(void* p, const float* x) {
    uint4 v;
    v.x = pack_bf16x2(x[0], x[1]);
    v.y = pack_bf16x2(x[2], x[3]);
    v.z = pack_bf16x2(x[4], x[5]);
    v.w = pack_bf16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = v;
  }
};

template <int DT, int D>
__global__ __launch_bounds__(256) void pool_kernel(const void* __restrict__ q_,
                                                   const void* __restrict__ k_,
                                                   const void* __restrict__ v_,
                                                   void* __restrict__ ck_, void* __restrict__ cv_,
                                                   float* __restrict__ weights, int m_cap, int B,
                                                   int Hq, int Hkv, int L, int g, float scale_log2) {
  typedef Vec16<DT> V16;
  constexpr int ES = DT == 0 ? 4 : 2;      // element bytes
  constexpr int EPL = V16::N;              // elements per lane slice
  constexpr int LPK = D * ES / 16;         // lanes per key row
  constexpr int KPW = 64 / LPK;            // keys per wave load
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int m = L / g;
  const long group = (long)blockIdx.x * (blockDim.x >> 6) + wave;
  if (group >= (long)B * Hkv * m) return;
  const int j = (int)(group % m);
  const long bh = group / m;  // b * Hkv + hk
  const int hk = (int)(bh % Hkv);
  const int b = (int)(bh / Hkv);
  const int G = Hq / Hkv;
  const int ks = lane / LPK;   // key slot within a chunk
  const int piece = lane % LPK;
  const int d0 = piece * EPL;

  const char* qb = static_cast<const char*>(q_);
  const char* kb = static_cast<const char*>(k_);
  const char* vb = static_cast<const char*>(v_);

  // Pooling query: mean over the G query heads of kv head hk, at the group's last token.
  float qbar[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) qbar[e] = 0.f;
  const int last = group_last(j, g);
  for (int gh = 0; gh < G; ++gh) {
    const long row = ((long)(b * Hq + hk * G + gh) * L + last) * D + d0;
    float x[EPL];
    V16::load(qb + row * ES, x);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qbar[e] += x[e];
  }
  const float invG = 1.0f / (float)G;
#pragma unroll
  for (int e = 0; e < EPL; ++e) qbar[e] *= invG;

  const long kv_row0 = ((long)bh * L + (long)j * g) * D;  // first key of the group
  float mrun = -INFINITY, lrun = 0.f;
  float acck[EPL], accv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acck[e] = accv[e] = 0.f;

  for (int c0 = 0; c0 < g; c0 += KPW) {
    const int tau = c0 + ks;
    const bool valid = tau < g;
    float kx[EPL], vx[EPL];
    if (valid) {
      V16::load(kb + (kv_row0 + (long)tau * D + d0) * ES, kx);
      V16::load(vb + (kv_row0 + (long)tau * D + d0) * ES, vx);
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) kx[e] = vx[e] = 0.f;
    }
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) part = fmaf(qbar[e], kx[e], part);
#pragma unroll
    for (int o = LPK / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    const float s = valid ? part * scale_log2 : -INFINITY;  // log2-domain score
    const float mnew = fmaxf(mrun, s);
    if (mnew != -INFINITY) {
      const float alpha = exp2f(mrun - mnew);
      const float p = exp2f(s - mnew);
      lrun = lrun * alpha + p;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        acck[e] = fmaf(p, kx[e], acck[e] * alpha);
        accv[e] = fmaf(p, vx[e], accv[e] * alpha);
      }
      mrun = mnew;
    }
  }
  // Merge the KPW lane groups (lanes piece, piece+LPK, ...).
#pragma unroll
  for (int o = LPK; o < 64; o <<= 1) {
    const float mo = __shfl_xor(mrun, o, 64);
    const float lo = __shfl_xor(lrun, o, 64);
    const float mnew = fmaxf(mrun, mo);
    const float fa = mrun == -INFINITY ? 0.f : exp2f(mrun - mnew);
    const float fb = mo == -INFINITY ? 0.f : exp2f(mo - mnew);
    lrun = lrun * fa + lo * fb;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float ko = __shfl_xor(acck[e], o, 64);
      const float vo = __shfl_xor(accv[e], o, 64);
      acck[e] = acck[e] * fa + ko * fb;
      accv[e] = accv[e] * fa + vo * fb;
    }
    mrun = mnew;
  }
  const float inv = 1.0f / lrun;
  if (ks == 0) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acck[e] *= inv;
      accv[e] *= inv;
    }
    const long crow = ((long)bh * m_cap + j) * D + d0;
    V16::store(static_cast<char*>(ck_) + crow * ES, acck);
    V16::store(static_cast<char*>(cv_) + crow * ES, accv);
  }
  if (weights != nullptr) {
    // Test output: a_tau = exp2(s_tau - max) / sum, scores recomputed identically.
    for (int c0 = 0; c0 < g; c0 += KPW) {
      const int tau = c0 + ks;
      float kx[EPL];
      if (tau < g) {
        V16::load(kb + (kv_row0 + (long)tau * D + d0) * ES, kx);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kx[e] = 0.f;
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part = fmaf(qbar[e], kx[e], part);
#pragma unroll
      for (int o = LPK / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
      if (tau < g && piece == 0)
        weights[((long)bh * m + j) * g + tau] = exp2f(part * scale_log2 - mrun) * inv;
    }
  }
}

template <int DT, int D>
void launch_pool_t(const void* q, const void* k, const void* v, void* ck, void* cv, int m_cap,
                   float* weights, const Shape& sh, hipStream_t s) {
  const long groups = (long)sh.B * sh.Hkv * sh.m();
  const int waves = 4;
  const long blocks = (groups + waves - 1) / waves;
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((pool_kernel<DT, D>), dim3((unsigned)blocks), dim3(64 * waves), 0, s, q, k, v,
                     ck, cv, weights, m_cap, sh.B, sh.Hq, sh.Hkv, sh.L, sh.g, scale_log2);
}

}  // namespace

hipError_t launch_pool(const void* q, const void* k, const void* v, void* ck, void* cv, int m_cap,
                       float* weights, const Shape& sh, int dt, hipStream_t s) {
  if (dt == 0) {
    if (sh.d == 64) launch_pool_t<0, 64>(q, k, v, ck, cv, m_cap, weights, sh, s);
    else launch_pool_t<0, 128>(q, k, v, ck, cv, m_cap, weights, sh, s);
  } else {
    if (sh.d == 64) launch_pool_t<1, 64>(q, k, v, ck, cv, m_cap, weights, sh, s);
    else launch_pool_t<1, 128>(q, k, v, ck, cv, m_cap, weights, sh, s);
  }
  return hipGetLastError();
}

}  // namespace cca
