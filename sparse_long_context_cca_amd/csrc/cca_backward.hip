// Backward pass of the CCA attention forward (pooling, then the fused softmax).
//
// The pages fine-tune models with CCA attention in place (paper card at
// atlas.scime.ai, summary and key results; rebuttal at paperhub.cn, answer on
// the fine-tuning setting); the gradients follow from the chain rule through
// the fusion formula and the pooling formula (digest at
// digest.lyk-ai.com/posts/2412.12465, "Method").  For row t with visible keys
// k (cores, then raw), P = softmax(S), S = q_t . key / sqrt(d), and upstream
// dO_t, with D_t = dO_t . o_t (= sum_k P_k dP_k):
//   dP_k = dO_t . value_k,  dS_k = P_k (dP_k - D_t),
//   dq_t = sum_k dS_k key_k / sqrt(d),
//   dkey_k += dS_k q_t / sqrt(d),  dvalue_k += P_k dO_t.
// The probabilities are recomputed from the row's log-sum-exp, which the
// forward writes.  Pooling then sends the core gradients to the group's keys,
// values and pooling query (see pool_backward_kernel).
//
// bf16 inputs take the matrix-core kernels of cca_backward_mfma.hip for steps
// 1-4 (step 4 folded into its key-parallel kernel).  fp32 inputs take the
// kernels below, in launch order (all arithmetic fp32 on the vector ALUs;
// gradients fp32):
//   1. row_dot_kernel       D_t = dO_t . o_t
//   2. dq_kernel            row-parallel over each row's visible keys
//   3. dkv_raw_kernel       key-parallel: raw key p is seen by rows p .. p+w-1
//   4. dcore_kernel         core-parallel: core j is seen by every row
//                           t >= (j+1)g + w - 1; rows are split over blocks
//                           and the partial sums meet by atomic adds in an
//                           fp32 workspace (cleared by fill_zero_kernel)
//   5. pool_backward_kernel one wave per group: adds the pooling share into
//                           dK, dV (the group's rows) and dQ (its last row)
#include <algorithm>

#include "cca_device.hpp"
#include "cca_internal.hpp"
#include "cca_pool_group.hpp"

namespace cca {
namespace {

constexpr int kTPR = 4;                      // threads per row (or key), each a quarter of d
constexpr int kRowsPerBlock = 256 / kTPR;    // rows (or keys) per block
constexpr int kTile = 32;           // staged rows / keys per LDS tile
constexpr int kCoreRowsPerSplit = 4096;

template <int DT>
using E = Elem<DT>;

// ---------------------------------------------------------------- 1. D = dO . O

template <int DT, int D>
__global__ __launch_bounds__(256) void row_dot_kernel(const void* __restrict__ out_,
                                                      const void* __restrict__ dout_,
                                                      float* __restrict__ Dv, long rows) {
  typedef typename E<DT>::T T;
  constexpr int LPR = 16;  // lanes per row
  const long row = ((long)blockIdx.x * blockDim.x + threadIdx.x) / LPR;
  const int part = threadIdx.x % LPR;
  const bool valid = row < rows;
  const T* o = static_cast<const T*>(out_);
  const T* g = static_cast<const T*>(dout_);
  float acc = 0.f;
  if (valid)
    for (int e = part; e < D; e += LPR) acc = fmaf(E<DT>::load(o, row * D + e), E<DT>::load(g, row * D + e), acc);
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (valid && part == 0) Dv[row] = acc;
}

// ------------------------------------------------------------------ 2. dQ

template <int DT, int D>
__global__ __launch_bounds__(256) void dq_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const void* __restrict__ ck_, const void* __restrict__ cv_, const void* __restrict__ dout_,
    const float* __restrict__ lse, const float* __restrict__ Dv, float* __restrict__ dq, int m_cap,
    int Hq, int Hkv, int L, int g, int w, float c, float scale) {
  typedef typename E<DT>::T T;
  constexpr int DH = D / kTPR;
  __shared__ float sk[kTile][D + 1];
  __shared__ float sv[kTile][D + 1];
  const int tid = threadIdx.x, part = tid % kTPR, r = tid / kTPR;  // part: which quarter of d
  const int h = blockIdx.y, b = blockIdx.z, G = Hq / Hkv, hk = h / G;
  const int t0 = blockIdx.x * kRowsPerBlock;
  const int t_hi = min(L - 1, t0 + kRowsPerBlock - 1);
  const int t = min(t0 + r, L - 1);  // rows past L compute a duplicate and store nothing
  const T* q = static_cast<const T*>(q_);
  const T* kk = static_cast<const T*>(k_);
  const T* vv = static_cast<const T*>(v_);
  const T* ck = static_cast<const T*>(ck_);
  const T* cv = static_cast<const T*>(cv_);
  const T* dout = static_cast<const T*>(dout_);
  const long row = (long)(b * Hq + h) * L + t;
  float qr[DH], gr[DH], acc[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    qr[e] = E<DT>::load(q, row * D + part * DH + e);
    gr[e] = E<DT>::load(dout, row * D + part * DH + e);
    acc[e] = 0.f;
  }
  const float lse2 = lse[row] * kLog2e, Dt = Dv[row];
  const int my_nc = n_core(t, g, w), my_lo = win_lo(t, w);
  const int nc_hi = n_core(t_hi, g, w);
  const int raw_lo = win_lo(t0, w);
  const int total = nc_hi + (t_hi - raw_lo + 1);
  const long kvb = (long)(b * Hkv + hk);
  for (int base = 0; base < total; base += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += 256) {
      const int i = idx / D, e = idx % D, f = base + i;
      float kx = 0.f, vx = 0.f;
      if (f < nc_hi) {
        kx = E<DT>::load(ck, (kvb * m_cap + f) * D + e);
        vx = E<DT>::load(cv, (kvb * m_cap + f) * D + e);
      } else if (f < total) {
        kx = E<DT>::load(kk, (kvb * L + raw_lo + (f - nc_hi)) * D + e);
        vx = E<DT>::load(vv, (kvb * L + raw_lo + (f - nc_hi)) * D + e);
      }
      sk[i][e] = kx;
      sv[i][e] = vx;
    }
    __syncthreads();
#pragma unroll 4
    for (int i = 0; i < kTile; ++i) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) {
        s = fmaf(qr[e], sk[i][part * DH + e], s);
        dp = fmaf(gr[e], sv[i][part * DH + e], dp);
      }
      s += __shfl_xor(s, 1, 64);
      dp += __shfl_xor(dp, 1, 64);
      s += __shfl_xor(s, 2, 64);
      dp += __shfl_xor(dp, 2, 64);
      const int f = base + i;
      const bool vis = f < nc_hi ? f < my_nc : (f < total && raw_lo + (f - nc_hi) >= my_lo && raw_lo + (f - nc_hi) <= t);
      const float p = vis ? exp2f(s * c - lse2) : 0.f;
      const float ds = p * (dp - Dt);
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = fmaf(ds, sk[i][part * DH + e], acc[e]);
    }
  }
  if (t0 + r < L) {
#pragma unroll
    for (int e = 0; e < DH; ++e) dq[row * D + part * DH + e] = acc[e] * scale;
  }
}

// ------------------------------------------------- 3. dK, dV of raw keys

template <int DT, int D>
__global__ __launch_bounds__(256) void dkv_raw_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const void* __restrict__ dout_, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ dk, float* __restrict__ dv, int Hq, int Hkv, int L, int w, float c,
    float scale) {
  typedef typename E<DT>::T T;
  constexpr int DH = D / kTPR;
  __shared__ float sq[kTile][D + 1];
  __shared__ float sg[kTile][D + 1];
  __shared__ float slse[kTile], sD[kTile];
  const int tid = threadIdx.x, part = tid % kTPR, r = tid / kTPR;  // part: which quarter of d
  const int hk = blockIdx.y, b = blockIdx.z, G = Hq / Hkv;
  const int p0 = blockIdx.x * kRowsPerBlock;
  const int p_hi = min(L - 1, p0 + kRowsPerBlock - 1);
  const int p = min(p0 + r, L - 1);
  const T* q = static_cast<const T*>(q_);
  const T* kk = static_cast<const T*>(k_);
  const T* vv = static_cast<const T*>(v_);
  const T* dout = static_cast<const T*>(dout_);
  const long krow = (long)(b * Hkv + hk) * L + p;
  float kr[DH], vr[DH], ak[DH], av[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    kr[e] = E<DT>::load(kk, krow * D + part * DH + e);
    vr[e] = E<DT>::load(vv, krow * D + part * DH + e);
    ak[e] = av[e] = 0.f;
  }
  // rows whose window holds a key of this block: p0 .. p_hi + w - 1
  const int t_end = min(L - 1, p_hi + w - 1);
  for (int hg = 0; hg < G; ++hg) {
    const int h = hk * G + hg;
    const long rbase = (long)(b * Hq + h) * L;
    for (int t0 = p0; t0 <= t_end; t0 += kTile) {
      __syncthreads();
      for (int idx = tid; idx < kTile * D; idx += 256) {
        const int i = idx / D, e = idx % D, t = t0 + i;
        sq[i][e] = t <= t_end ? E<DT>::load(q, (rbase + t) * D + e) : 0.f;
        sg[i][e] = t <= t_end ? E<DT>::load(dout, (rbase + t) * D + e) : 0.f;
      }
      if (tid < kTile) {
        const int t = t0 + tid;
        slse[tid] = t <= t_end ? lse[rbase + t] * kLog2e : 0.f;
        sD[tid] = t <= t_end ? Dv[rbase + t] : 0.f;
      }
      __syncthreads();
#pragma unroll 4
      for (int i = 0; i < kTile; ++i) {
        const int t = t0 + i;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < DH; ++e) {
          s = fmaf(kr[e], sq[i][part * DH + e], s);
          dp = fmaf(vr[e], sg[i][part * DH + e], dp);
        }
        s += __shfl_xor(s, 1, 64);
        dp += __shfl_xor(dp, 1, 64);
        s += __shfl_xor(s, 2, 64);
        dp += __shfl_xor(dp, 2, 64);
        const bool vis = t <= t_end && p <= t && p >= win_lo(t, w);
        const float pw = vis ? exp2f(s * c - slse[i]) : 0.f;
        const float ds = pw * (dp - sD[i]);
#pragma unroll
        for (int e = 0; e < DH; ++e) {
          ak[e] = fmaf(ds, sq[i][part * DH + e], ak[e]);
          av[e] = fmaf(pw, sg[i][part * DH + e], av[e]);
        }
      }
    }
  }
  if (p0 + r < L) {
#pragma unroll
    for (int e = 0; e < DH; ++e) {
      dk[krow * D + part * DH + e] = ak[e] * scale;
      dv[krow * D + part * DH + e] = av[e];
    }
  }
}

// --------------------------------------------- 4. dCK, dCV of the cores

__global__ void fill_zero_kernel(float* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

// grid = (core blocks, row splits, B * Hkv).  Core j is seen by rows
// t >= (j+1)g + w - 1 (n_core(t) > j).
template <int DT, int D>
__global__ __launch_bounds__(256) void dcore_kernel(
    const void* __restrict__ q_, const void* __restrict__ ck_, const void* __restrict__ cv_,
    const void* __restrict__ dout_, const float* __restrict__ lse, const float* __restrict__ Dv,
    float* __restrict__ dck, float* __restrict__ dcv, int m, int m_cap, int Hq, int Hkv, int L,
    int g, int w, float c, float scale) {
  typedef typename E<DT>::T T;
  constexpr int DH = D / kTPR;
  __shared__ float sq[kTile][D + 1];
  __shared__ float sg[kTile][D + 1];
  __shared__ float slse[kTile], sD[kTile];
  const int tid = threadIdx.x, part = tid % kTPR, r = tid / kTPR;  // part: which quarter of d
  const int bh = blockIdx.z, b = bh / Hkv, hk = bh % Hkv, G = Hq / Hkv;
  const int j0 = blockIdx.x * kRowsPerBlock;
  const int j = min(j0 + r, m - 1);
  const int t_first = (j0 + 1) * g + w - 1;  // first row that sees core j0
  const int t_lo = t_first + blockIdx.y * kCoreRowsPerSplit;
  const int t_hi = min(L - 1, t_lo + kCoreRowsPerSplit - 1);
  if (t_lo > t_hi) return;
  const T* q = static_cast<const T*>(q_);
  const T* ck = static_cast<const T*>(ck_);
  const T* cv = static_cast<const T*>(cv_);
  const T* dout = static_cast<const T*>(dout_);
  const long crow = (long)bh * m_cap + j;
  float kr[DH], vr[DH], ak[DH], av[DH];
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    kr[e] = E<DT>::load(ck, crow * D + part * DH + e);
    vr[e] = E<DT>::load(cv, crow * D + part * DH + e);
    ak[e] = av[e] = 0.f;
  }
  for (int hg = 0; hg < G; ++hg) {
    const int h = hk * G + hg;
    const long rbase = (long)(b * Hq + h) * L;
    for (int t0 = t_lo; t0 <= t_hi; t0 += kTile) {
      __syncthreads();
      for (int idx = tid; idx < kTile * D; idx += 256) {
        const int i = idx / D, e = idx % D, t = t0 + i;
        sq[i][e] = t <= t_hi ? E<DT>::load(q, (rbase + t) * D + e) : 0.f;
        sg[i][e] = t <= t_hi ? E<DT>::load(dout, (rbase + t) * D + e) : 0.f;
      }
      if (tid < kTile) {
        const int t = t0 + tid;
        slse[tid] = t <= t_hi ? lse[rbase + t] * kLog2e : 0.f;
        sD[tid] = t <= t_hi ? Dv[rbase + t] : 0.f;
      }
      __syncthreads();
#pragma unroll 4
      for (int i = 0; i < kTile; ++i) {
        const int t = t0 + i;
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < DH; ++e) {
          s = fmaf(kr[e], sq[i][part * DH + e], s);
          dp = fmaf(vr[e], sg[i][part * DH + e], dp);
        }
        s += __shfl_xor(s, 1, 64);
        dp += __shfl_xor(dp, 1, 64);
        s += __shfl_xor(s, 2, 64);
        dp += __shfl_xor(dp, 2, 64);
        const bool vis = t <= t_hi && j0 + r < m && j < n_core(t, g, w);
        const float pw = vis ? exp2f(s * c - slse[i]) : 0.f;
        const float ds = pw * (dp - sD[i]);
#pragma unroll
        for (int e = 0; e < DH; ++e) {
          ak[e] = fmaf(ds, sq[i][part * DH + e], ak[e]);
          av[e] = fmaf(pw, sg[i][part * DH + e], av[e]);
        }
      }
    }
  }
  if (j0 + r < m) {
    const long wrow = ((long)bh * m + j) * D + part * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) {
      atomicAdd(dck + wrow + e, ak[e] * scale);
      atomicAdd(dcv + wrow + e, av[e]);
    }
  }
}

// ------------------------------------------------ 5. pooling backward

// One wave per (b, kv head, group).  dK, dV, dQ hold the raw-key / row
// gradients already; this adds the pooling share (each group's rows and its
// last row belong to that group alone, so plain read-modify-writes suffice).
template <int DT, int D, int MODE>
__global__ __launch_bounds__(256) void pool_backward_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const float* __restrict__ dck, const float* __restrict__ dcv, float* __restrict__ dq,
    float* __restrict__ dk, float* __restrict__ dv, int B, int Hq, int Hkv, int L, int g,
    float scale_log2, float scale) {
  typedef RowLanes<DT, D> RL;
  typedef Row16<DT> R16;
  constexpr int EPL = RL::EPL;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int m = L / g;
  const long grp = (long)blockIdx.x * (blockDim.x >> 6) + wave;
  if (grp >= (long)B * Hkv * m) return;
  const int j = (int)(grp % m);
  const long bh = grp / m;
  const int hk = (int)(bh % Hkv), b = (int)(bh / Hkv), G = Hq / Hkv;
  const int ks = lane / RL::LPK, piece = lane % RL::LPK, d0 = piece * EPL;
  const char* qb = static_cast<const char*>(q_);
  const char* kb = static_cast<const char*>(k_);
  const char* vb = static_cast<const char*>(v_);
  const long row0 = bh * L + (long)j * g;  // first token of the group
  const int last = group_last(j, g);
  auto krow = [&](int tau) { return kb + ((row0 + tau) * D + d0) * RL::ES; };
  auto vrow = [&](int tau) { return vb + ((row0 + tau) * D + d0) * RL::ES; };
  auto qrow = [&](int hh) { return qb + (((long)(b * Hq + hk * G + hh) * L + last) * D + d0) * RL::ES; };
  float gk[EPL], gv[EPL];  // this lane's slice of dCK_j, dCV_j
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    gk[e] = dck[(bh * m + j) * D + d0 + e];
    gv[e] = dcv[(bh * m + j) * D + d0 + e];
  }
  auto add_row = [&](float* base, long row, const float* x) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) base[row * D + d0 + e] += x[e];
  };

  if constexpr (MODE == kPoolMean) {
    const float inv = 1.0f / (float)g;
    for (int tau = ks; tau < g; tau += RL::KPW) {
      float xk[EPL], xv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        xk[e] = gk[e] * inv;
        xv[e] = gv[e] * inv;
      }
      add_row(dk, row0 + tau, xk);
      add_row(dv, row0 + tau, xv);
    }
  } else if constexpr (MODE == kPoolMax) {
    // each component's gradient goes to the first token holding the maximum
    float mk[EPL], mv[EPL];
    int ik[EPL], iv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      mk[e] = mv[e] = -INFINITY;
      ik[e] = iv[e] = g;
    }
    for (int tau = ks; tau < g; tau += RL::KPW) {
      float xk[EPL], xv[EPL];
      R16::load(krow(tau), xk);
      R16::load(vrow(tau), xv);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        if (xk[e] > mk[e]) { mk[e] = xk[e]; ik[e] = tau; }
        if (xv[e] > mv[e]) { mv[e] = xv[e]; iv[e] = tau; }
      }
    }
#pragma unroll
    for (int o = RL::LPK; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float mko = __shfl_xor(mk[e], o, 64), mvo = __shfl_xor(mv[e], o, 64);
        const int iko = __shfl_xor(ik[e], o, 64), ivo = __shfl_xor(iv[e], o, 64);
        if (mko > mk[e] || (mko == mk[e] && iko < ik[e])) { mk[e] = mko; ik[e] = iko; }
        if (mvo > mv[e] || (mvo == mv[e] && ivo < iv[e])) { mv[e] = mvo; iv[e] = ivo; }
      }
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        dk[(row0 + ik[e]) * D + d0 + e] += gk[e];
        dv[(row0 + iv[e]) * D + d0 + e] += gv[e];
      }
    }
  } else {
    constexpr int MG = MODE == kPoolSoftmax ? 1 : kPoolHeadsMaxG;
    const int NH = MODE == kPoolSoftmax ? 1 : G;  // softmaxes over the group
    float qh[MG][EPL];
    if constexpr (MODE == kPoolSoftmax) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qh[0][e] = 0.f;
      for (int hh = 0; hh < G; ++hh) {
        float x[EPL];
        R16::load(qrow(hh), x);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qh[0][e] += x[e] / (float)G;
      }
    } else {
#pragma unroll
      for (int hh = 0; hh < MG; ++hh)
        if (hh < G) R16::load(qrow(hh), qh[hh]);
    }
    // pass 1: per softmax, max and sum of exp2(s - max)
    float mh[MG], lh[MG];
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      mh[i] = -INFINITY;
      lh[i] = 0.f;
    }
    for (int c0 = 0; c0 < g; c0 += RL::KPW) {
      const int tau = c0 + ks;
      const bool valid = tau < g;
      float xk[EPL];
      if (valid) R16::load(krow(tau), xk);
      else
#pragma unroll
        for (int e = 0; e < EPL; ++e) xk[e] = 0.f;
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        if (i >= NH) break;
        const float sd = row_dot<DT, D>(qh[i], xk);  // every lane: the dot shuffles across a row
        const float s = valid ? sd * scale_log2 : -INFINITY;
        const float mn = fmaxf(mh[i], s);
        if (mn != -INFINITY) {
          lh[i] = lh[i] * exp2f(mh[i] - mn) + exp2f(s - mn);
          mh[i] = mn;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      if (i >= NH) break;
#pragma unroll
      for (int o = RL::LPK; o < 64; o <<= 1) {
        const float mo = __shfl_xor(mh[i], o, 64), lo = __shfl_xor(lh[i], o, 64);
        const float mn = fmaxf(mh[i], mo);
        const float fa = mh[i] == -INFINITY ? 0.f : exp2f(mh[i] - mn);
        const float fb = mo == -INFINITY ? 0.f : exp2f(mo - mn);
        lh[i] = lh[i] * fa + lo * fb;
        mh[i] = mn;
      }
    }
    // pass 2: da_tau = dCK . K + dCV . V; per softmax, sum_tau a da
    float sad[MG];
#pragma unroll
    for (int i = 0; i < MG; ++i) sad[i] = 0.f;
    for (int c0 = 0; c0 < g; c0 += RL::KPW) {
      const int tau = c0 + ks;
      const bool valid = tau < g;
      float xk[EPL], xv[EPL];
      if (valid) {
        R16::load(krow(tau), xk);
        R16::load(vrow(tau), xv);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) xk[e] = xv[e] = 0.f;
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part = fmaf(gk[e], xk[e], fmaf(gv[e], xv[e], part));
#pragma unroll
      for (int o = RL::LPK / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        if (i >= NH) break;
        const float sd = row_dot<DT, D>(qh[i], xk);
        const float a = valid ? exp2f(sd * scale_log2 - mh[i]) / lh[i] : 0.f;
        sad[i] += a * part;
      }
    }
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      if (i >= NH) break;
#pragma unroll
      for (int o = RL::LPK; o < 64; o <<= 1) sad[i] += __shfl_xor(sad[i], o, 64);
    }
    // pass 3: dK += a dCK + sum_i ds_i q_i / sqrt(d); dV += a dCV; dq_i += ds_i K / sqrt(d)
    float dqh[MG][EPL];
#pragma unroll
    for (int i = 0; i < MG; ++i)
#pragma unroll
      for (int e = 0; e < EPL; ++e) dqh[i][e] = 0.f;
    const float wsum = MODE == kPoolSoftmax ? 1.0f : 1.0f / (float)G;  // weight of each softmax in a
    for (int c0 = 0; c0 < g; c0 += RL::KPW) {
      const int tau = c0 + ks;
      const bool valid = tau < g;
      float xk[EPL], xv[EPL];
      if (valid) {
        R16::load(krow(tau), xk);
        R16::load(vrow(tau), xv);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) xk[e] = xv[e] = 0.f;
      }
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) part = fmaf(gk[e], xk[e], fmaf(gv[e], xv[e], part));
#pragma unroll
      for (int o = RL::LPK / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
      float a_tot = 0.f;
      float addk[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) addk[e] = 0.f;
#pragma unroll
      for (int i = 0; i < MG; ++i) {
        if (i >= NH) break;
        const float sd = row_dot<DT, D>(qh[i], xk);
        const float a = valid ? exp2f(sd * scale_log2 - mh[i]) / lh[i] : 0.f;
        a_tot += a * wsum;
        const float ds = a * (part - sad[i]) * wsum;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          addk[e] = fmaf(ds * scale, qh[i][e], addk[e]);
          dqh[i][e] = fmaf(ds * scale, xk[e], dqh[i][e]);
        }
      }
      if (valid) {
        float addv[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          addk[e] = fmaf(a_tot, gk[e], addk[e]);
          addv[e] = a_tot * gv[e];
        }
        add_row(dk, row0 + tau, addk);
        add_row(dv, row0 + tau, addv);
      }
    }
    // query gradients: sum over the lane groups, then into the last row
#pragma unroll
    for (int i = 0; i < MG; ++i) {
      if (i >= NH) break;
#pragma unroll
      for (int o = RL::LPK; o < 64; o <<= 1)
#pragma unroll
        for (int e = 0; e < EPL; ++e) dqh[i][e] += __shfl_xor(dqh[i][e], o, 64);
    }
    if (ks == 0) {
      for (int hh = 0; hh < G; ++hh) {
        const int i = MODE == kPoolSoftmax ? 0 : hh;
        const float f = MODE == kPoolSoftmax ? 1.0f / (float)G : 1.0f;  // qbar = mean of the heads
        const long qr = (long)(b * Hq + hk * G + hh) * L + last;
#pragma unroll
        for (int e = 0; e < EPL; ++e) dq[qr * D + d0 + e] += dqh[i < MG ? i : 0][e] * f;
      }
    }
  }
}

// Workspace: row statistics (2 floats per row), dCK, dCV (fp32), then for
// bf16 inputs, from a 256-byte boundary, fp16 copies of q and dO.
size_t f32_part_bytes(const Shape& sh) {
  const size_t m = sh.g > 0 ? (size_t)(sh.L / sh.g) : 0;
  return (2 * (size_t)sh.B * sh.Hq * sh.L + 2 * (size_t)sh.B * sh.Hkv * m * sh.d) * sizeof(float);
}
size_t f16_copies_offset(const Shape& sh) { return (f32_part_bytes(sh) + 255) & ~(size_t)255; }

template <int DT, int D>
hipError_t launch_backward_t(const void* q, const void* k, const void* v, const void* ck,
                             const void* cv, int m_cap, const void* out, const float* lse,
                             const void* dout, float* dq, float* dk, float* dv, float* ws,
                             const Shape& sh, int pool_mode, hipStream_t s) {
  const int B = sh.B, Hq = sh.Hq, Hkv = sh.Hkv, L = sh.L, g = sh.g, w = sh.w;
  const int m = L / g;
  const float scale = 1.0f / sqrtf((float)D), c = kLog2e * scale;
  // workspace: row statistics (2 floats per row), then dCK, dCV
  const long rows = (long)B * Hq * L;
  float* dck = ws + 2 * (size_t)rows;
  float* dcv = dck + (size_t)B * Hkv * m * D;
  if (m > 0) {
    const long nws = 2L * B * Hkv * m * D;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<long>((nws + 255) / 256, 4096)), dim3(256),
                       0, s, dck, nws);
  }
  if constexpr (DT == 1) {
    // bf16: matrix-core kernels (cca_backward_mfma.hip)
    uint16_t* q16 = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(ws) + f16_copies_offset(sh));
    uint16_t* do16 = q16 + (size_t)rows * D;
    const hipError_t e = launch_backward_mfma(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv,
                                              reinterpret_cast<float2*>(ws), dck, dcv, q16, do16, sh, s);
    if (e != hipSuccess) return e;
  } else {
    float* Dv = ws;
    hipLaunchKernelGGL((row_dot_kernel<DT, D>), dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, s,
                       out, dout, Dv, rows);
    const int rb = (L + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL((dq_kernel<DT, D>), dim3(rb, Hq, B), dim3(256), 0, s, q, k, v, ck, cv, dout, lse,
                       Dv, dq, m_cap, Hq, Hkv, L, g, w, c, scale);
    hipLaunchKernelGGL((dkv_raw_kernel<DT, D>), dim3(rb, Hkv, B), dim3(256), 0, s, q, k, v, dout, lse,
                       Dv, dk, dv, Hq, Hkv, L, w, c, scale);
    if (m > 0) {
      const int cb = (m + kRowsPerBlock - 1) / kRowsPerBlock;
      const int splits = (L + kCoreRowsPerSplit - 1) / kCoreRowsPerSplit;
      hipLaunchKernelGGL((dcore_kernel<DT, D>), dim3(cb, splits, B * Hkv), dim3(256), 0, s, q, ck, cv, dout,
                         lse, Dv, dck, dcv, m, m_cap, Hq, Hkv, L, g, w, c, scale);
    }
  }
  if (m > 0) {
    const long groups = (long)B * Hkv * m;
    const dim3 pg((unsigned)((groups + 3) / 4));
    switch (pool_mode) {
      case kPoolSoftmaxHeads:
        hipLaunchKernelGGL((pool_backward_kernel<DT, D, kPoolSoftmaxHeads>), pg, dim3(256), 0, s, q, k, v, dck,
                           dcv, dq, dk, dv, B, Hq, Hkv, L, g, c, scale);
        break;
      case kPoolMean:
        hipLaunchKernelGGL((pool_backward_kernel<DT, D, kPoolMean>), pg, dim3(256), 0, s, q, k, v, dck, dcv,
                           dq, dk, dv, B, Hq, Hkv, L, g, c, scale);
        break;
      case kPoolMax:
        hipLaunchKernelGGL((pool_backward_kernel<DT, D, kPoolMax>), pg, dim3(256), 0, s, q, k, v, dck, dcv,
                           dq, dk, dv, B, Hq, Hkv, L, g, c, scale);
        break;
      default:
        hipLaunchKernelGGL((pool_backward_kernel<DT, D, kPoolSoftmax>), pg, dim3(256), 0, s, q, k, v, dck,
                           dcv, dq, dk, dv, B, Hq, Hkv, L, g, c, scale);
        break;
    }
  }
  return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int g, int dt) {
  const Shape sh{B, Hq, Hkv, L, d, g, 1};
  if (dt == 0) return f32_part_bytes(sh);
  return f16_copies_offset(sh) + 2 * (size_t)B * Hq * L * d * sizeof(uint16_t);
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* ck,
                           const void* cv, int m_cap, const void* out, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, void* ws,
                           const Shape& sh, int dt, int pool_mode, hipStream_t s) {
  float* w = static_cast<float*>(ws);
  if (dt == 0)
    return sh.d == 64 ? launch_backward_t<0, 64>(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv, w, sh, pool_mode, s)
                      : launch_backward_t<0, 128>(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv, w, sh, pool_mode, s);
  return sh.d == 64 ? launch_backward_t<1, 64>(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv, w, sh, pool_mode, s)
                    : launch_backward_t<1, 128>(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv, w, sh, pool_mode, s);
}

}  // namespace cca
