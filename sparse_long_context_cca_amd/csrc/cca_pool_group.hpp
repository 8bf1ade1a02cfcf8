// Pooling of one group of g tokens into one core key/value pair, by one wave.
//
// Global-aware pooling (digest at digest.lyk-ai.com/posts/2412.12465,
// "Method", pooling formula; ICML 2025 article at changsha.jmyizhao.com,
// global-aware pooling paragraph: the group's last-token query scores every
// token of the group) and the variants the pages name or leave open:
//   kPoolSoftmax      a = softmax_tau(qbar . K[tau] / sqrt(d)), qbar the mean
//                     of the G query heads' last-token queries (default);
//   kPoolSoftmaxHeads a = mean over the G heads of softmax_tau(q_h . K[tau] /
//                     sqrt(d)) (the other plain GQA rule; the rebuttal at
//                     paperhub.cn, answer on GQA, leaves the rule open);
//   kPoolMean         a = 1/g;                     (rebuttal, answer on
//   kPoolMax          element-wise max over tau    Table 3: the max- and
//                     of K and of V, separately.   mean-pooling ablations)
//   CK = sum_tau a_tau K[tau], CV = sum_tau a_tau V[tau] (kPoolMax: the maxima).
//
// Lane layout: each lane owns a 16-byte slice (EPL elements) of a row; LPK
// lanes cover a row, so a wave load covers KPW = 64 / LPK rows, and lane group
// ks = lane / LPK takes rows ks, ks + KPW, ...  Each lane group keeps its own
// partial state, and the groups are merged with shuffles at the end.  Works
// for any g >= 1.
#pragma once

#include "cca_device.hpp"

namespace cca {

enum PoolMode { kPoolSoftmax = 0, kPoolSoftmaxHeads = 1, kPoolMean = 2, kPoolMax = 3 };
constexpr int kPoolHeadsMaxG = 8;  // kPoolSoftmaxHeads keeps one state per head in registers

template <int DT>
struct Row16;  // a lane's 16-byte slice of a row, as floats (unpack: from its raw bits)
template <>
struct Row16<0> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float* x) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ void load(const void* p, float* x) {
    unpack(*reinterpret_cast<const uint4*>(p), x);
  }
  static __device__ __forceinline__ void store(void* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  }
};
template <>
struct Row16<1> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ void load(const void* p, float* x) {
    unpack(*reinterpret_cast<const uint4*>(p), x);
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

template <>
struct Row16<2> {  // fp16 (the core cache of bf16 inputs)
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* x) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = f16_to_f32((uint16_t)(w[i] & 0xffffu));
      x[2 * i + 1] = f16_to_f32((uint16_t)(w[i] >> 16));
    }
  }
  static __device__ __forceinline__ void load(const void* p, float* x) {
    unpack(*reinterpret_cast<const uint4*>(p), x);
  }
  static __device__ __forceinline__ void store(void* p, const float* x) {
    uint4 v;
    v.x = pack_f16x2(x[0], x[1]);
    v.y = pack_f16x2(x[2], x[3]);
    v.z = pack_f16x2(x[4], x[5]);
    v.w = pack_f16x2(x[6], x[7]);
    *reinterpret_cast<uint4*>(p) = v;
  }
};

template <int DT, int D>
struct RowLanes {
  static constexpr int ES = DT == 0 ? 4 : 2;   // element bytes
  static constexpr int EPL = Row16<DT>::N;     // elements per lane slice
  static constexpr int LPK = D * ES / 16;      // lanes per row
  static constexpr int KPW = 64 / LPK;         // rows per wave load
};

// Dot product of two lane slices, summed over the LPK lanes of a row.
template <int DT, int D>
__device__ __forceinline__ float row_dot(const float* a, const float* b) {
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < RowLanes<DT, D>::EPL; ++e) part = fmaf(a[e], b[e], part);
#pragma unroll
  for (int o = RowLanes<DT, D>::LPK / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
  return part;
}

// Merges the online-softmax states (m, l, acc) of the KPW lane groups.
template <int DT, int D>
__device__ __forceinline__ void merge_softmax_states(float& m, float& l, float* acck, float* accv) {
  typedef RowLanes<DT, D> RL;
#pragma unroll
  for (int o = RL::LPK; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m, o, 64);
    const float lo = __shfl_xor(l, o, 64);
    const float mnew = fmaxf(m, mo);
    const float fa = m == -INFINITY ? 0.f : exp2f(m - mnew);
    const float fb = mo == -INFINITY ? 0.f : exp2f(mo - mnew);
    l = l * fa + lo * fb;
#pragma unroll
    for (int e = 0; e < RL::EPL; ++e) {
      const float ko = __shfl_xor(acck[e], o, 64);
      const float vo = __shfl_xor(accv[e], o, 64);
      acck[e] = acck[e] * fa + ko * fb;
      accv[e] = accv[e] * fa + vo * fb;
    }
    m = mnew;
  }
}

// Pools one group.  krow(tau) / vrow(tau) give the byte address of token tau's
// K / V row (0 <= tau < g); qrow(h) that of the group's last-token query of
// head h (0 <= h < G; not read by kPoolMean and kPoolMax).  scale_log2 =
// log2(e) / sqrt(d).  On return the lanes of lane group 0 (lane < LPK) hold
// elements lane*EPL .. +EPL-1 of CK and CV in acck / accv (fp32, unrounded).
// If wout is not null, the weights a_tau are written to wout[tau] (fp32;
// kPoolMax has none and writes nothing).  kPoolSoftmaxHeads needs
// G <= kPoolHeadsMaxG.
template <int DT, int D, int MODE, class KRow, class VRow, class QRow>
__device__ __forceinline__ void pool_group(KRow krow, VRow vrow, QRow qrow, int g, int G,
                                           float scale_log2, float* acck, float* accv,
                                           float* wout) {
  typedef Row16<DT> R16;
  typedef RowLanes<DT, D> RL;
  constexpr int EPL = RL::EPL;
  const int lane = threadIdx.x & 63;
  const int ks = lane / RL::LPK;
  const int piece = lane % RL::LPK;
  const int d0 = piece * EPL;  // element offset of this lane's slice
  const int off = d0 * RL::ES;  // ... in bytes

  if constexpr (MODE == kPoolMean || MODE == kPoolMax) {
    const float init = MODE == kPoolMax ? -INFINITY : 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acck[e] = accv[e] = init;
    for (int tau = ks; tau < g; tau += RL::KPW) {
      float kx[EPL], vx[EPL];
      R16::load(krow(tau) + off, kx);
      R16::load(vrow(tau) + off, vx);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if (MODE == kPoolMax) {
          acck[e] = fmaxf(acck[e], kx[e]);
          accv[e] = fmaxf(accv[e], vx[e]);
        } else {
          acck[e] += kx[e];
          accv[e] += vx[e];
        }
      }
    }
#pragma unroll
    for (int o = RL::LPK; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ko = __shfl_xor(acck[e], o, 64);
        const float vo = __shfl_xor(accv[e], o, 64);
        acck[e] = MODE == kPoolMax ? fmaxf(acck[e], ko) : acck[e] + ko;
        accv[e] = MODE == kPoolMax ? fmaxf(accv[e], vo) : accv[e] + vo;
      }
    if constexpr (MODE == kPoolMean) {
      const float inv = 1.0f / (float)g;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        acck[e] *= inv;
        accv[e] *= inv;
      }
      if (wout != nullptr && lane == 0)
        for (int tau = 0; tau < g; ++tau) wout[tau] = inv;
    }
  } else if constexpr (MODE == kPoolSoftmax) {
    // The group's rows are read one round ahead of their use (raw 16-byte
    // slices), and the first round is requested before the query rows.  In
    // one process on one MI355X this took the GQA 128K pooling from 126-132
    // to 122-124 us; four rounds ahead (a group of 16 in flight at once)
    // took 155 us, its registers costing a wave per SIMD.
    auto fetch = [&](int c0, uint4& kr, uint4& vr) {
      const int tau = c0 + ks;
      if (tau < g) {
        kr = *reinterpret_cast<const uint4*>(krow(tau) + off);
        vr = *reinterpret_cast<const uint4*>(vrow(tau) + off);
      } else {
        kr = vr = make_uint4(0u, 0u, 0u, 0u);
      }
    };
    uint4 kr, vr;
    fetch(0, kr, vr);
    // pooling query: mean over the G heads of the last-token queries
    float qbar[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) qbar[e] = 0.f;
    for (int h = 0; h < G; ++h) {
      float x[EPL];
      R16::load(qrow(h) + off, x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qbar[e] += x[e];
    }
    const float invG = 1.0f / (float)G;
#pragma unroll
    for (int e = 0; e < EPL; ++e) qbar[e] *= invG;
    float m = -INFINITY, l = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acck[e] = accv[e] = 0.f;
    // every lane group runs the same number of rounds (the dot products
    // shuffle across the lanes of a row)
    for (int c0 = 0; c0 < g; c0 += RL::KPW) {
      const int tau = c0 + ks;
      const bool valid = tau < g;
      float kx[EPL], vx[EPL];
      R16::unpack(kr, kx);  // zeros past the group
      R16::unpack(vr, vx);
      if (c0 + RL::KPW < g) fetch(c0 + RL::KPW, kr, vr);
      const float part = row_dot<DT, D>(qbar, kx);
      const float s = valid ? part * scale_log2 : -INFINITY;  // log2-domain score
      const float mnew = fmaxf(m, s);
      if (mnew != -INFINITY) {
        const float alpha = exp2f(m - mnew);
        const float p = exp2f(s - mnew);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          acck[e] = fmaf(p, kx[e], acck[e] * alpha);
          accv[e] = fmaf(p, vx[e], accv[e] * alpha);
        }
        m = mnew;
      }
    }
    merge_softmax_states<DT, D>(m, l, acck, accv);
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      acck[e] *= inv;
      accv[e] *= inv;
    }
    if (wout != nullptr) {
      // scores recomputed identically; a_tau = exp2(s_tau - m) / l
      for (int c0 = 0; c0 < g; c0 += RL::KPW) {
        const int tau = c0 + ks;
        float kx[EPL];
        if (tau < g) {
          R16::load(krow(tau) + off, kx);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) kx[e] = 0.f;
        }
        const float part = row_dot<DT, D>(qbar, kx);
        if (tau < g && piece == 0) wout[tau] = exp2f(part * scale_log2 - m) * inv;
      }
    }
  } else {  // kPoolSoftmaxHeads
    static_assert(MODE == kPoolSoftmaxHeads, "pooling mode");
    constexpr int MG = kPoolHeadsMaxG;
    float qh[MG][EPL];
#pragma unroll
    for (int h = 0; h < MG; ++h)
      if (h < G) R16::load(qrow(h) + off, qh[h]);
    // pass 1: per head, the max and the sum of exp2(s - max) over the group
    float mh[MG], lh[MG];
#pragma unroll
    for (int h = 0; h < MG; ++h) {
      mh[h] = -INFINITY;
      lh[h] = 0.f;
    }
    for (int c0 = 0; c0 < g; c0 += RL::KPW) {
      const int tau = c0 + ks;
      const bool valid = tau < g;
      float kx[EPL];
      if (valid) {
        R16::load(krow(tau) + off, kx);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kx[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < MG; ++h) {
        if (h >= G) break;
        const float part = row_dot<DT, D>(qh[h], kx);
        const float s = valid ? part * scale_log2 : -INFINITY;
        const float mnew = fmaxf(mh[h], s);
        if (mnew != -INFINITY) {
          lh[h] = lh[h] * exp2f(mh[h] - mnew) + exp2f(s - mnew);
          mh[h] = mnew;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < MG; ++h) {
      if (h >= G) break;
#pragma unroll
      for (int o = RL::LPK; o < 64; o <<= 1) {
        const float mo = __shfl_xor(mh[h], o, 64);
        const float lo = __shfl_xor(lh[h], o, 64);
        const float mnew = fmaxf(mh[h], mo);
        const float fa = mh[h] == -INFINITY ? 0.f : exp2f(mh[h] - mnew);
        const float fb = mo == -INFINITY ? 0.f : exp2f(mo - mnew);
        lh[h] = lh[h] * fa + lo * fb;
        mh[h] = mnew;
      }
    }
    // pass 2: a_tau = mean_h exp2(s_h,tau - m_h) / l_h; accumulate a K, a V
#pragma unroll
    for (int e = 0; e < EPL; ++e) acck[e] = accv[e] = 0.f;
    const float invG = 1.0f / (float)G;
    for (int c0 = 0; c0 < g; c0 += RL::KPW) {
      const int tau = c0 + ks;
      const bool valid = tau < g;
      float kx[EPL], vx[EPL];
      if (valid) {
        R16::load(krow(tau) + off, kx);
        R16::load(vrow(tau) + off, vx);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kx[e] = vx[e] = 0.f;
      }
      float a = 0.f;
#pragma unroll
      for (int h = 0; h < MG; ++h) {
        if (h >= G) break;
        const float part = row_dot<DT, D>(qh[h], kx);
        a += exp2f(part * scale_log2 - mh[h]) / lh[h];
      }
      a = valid ? a * invG : 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        acck[e] = fmaf(a, kx[e], acck[e]);
        accv[e] = fmaf(a, vx[e], accv[e]);
      }
      if (wout != nullptr && valid && piece == 0) wout[tau] = a;
    }
#pragma unroll
    for (int o = RL::LPK; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        acck[e] += __shfl_xor(acck[e], o, 64);
        accv[e] += __shfl_xor(accv[e], o, 64);
      }
  }
}

}  // namespace cca
