// KV-cached decode step of the fused CCA attention (the ICML 2025 article at
// changsha.jmyizhao.com says CCA supports a KV cache natively and decodes at
// FlashAttention-level speed; the digest at digest.lyk-ai.com/posts/2412.12465,
// "Method", fusion formula, defines the row computed).
//
// Per step and sequence b (new token at position t = pos[b]):
//   pass 1 (grid: splits x query-head groups x batch)
//     - one block per (b, kv head) appends k_t, v_t to ring slot t % R and,
//       when (t+1) % g == 0, pools group (t+1)/g-1 (positions t-g+1..t; the
//       pooling query is the mean over the kv head's G query heads of q_t) into
//       core slot (t+1)/g-1.  Neither location is read by this step: the ring
//       slot held position t-R <= t-w, and the new core is not visible to t.
//     - every block streams its share of the visible keys [cores 0..n_core(t)
//       ; raw win_lo(t)..t] once from HBM and keeps an online softmax state for
//       its query heads; position t itself is read from k_t/v_t.
//     - the partial states (max, sum, weighted values) go to the workspace.
//   pass 2 merges the split states per (b, query head), writes the output and
//   optionally advances pos[b].
// HBM-bound: every visible K/V byte is read once per step.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "cca_device.hpp"
#include "cca_internal.hpp"
#include "cca_pool_group.hpp"

namespace cca {
namespace {

constexpr int kThreads = 256;
// The max a split writes for a step whose position is invalid: a quiet NaN
// with a payload of its own, so that the combine tells it from a NaN the data
// produced (which must reach the output, with pos still advanced).
constexpr unsigned kInvalidState = 0x7fc00badu;
constexpr int kBatch = 4;  // keys per lane group per iteration

template <int DT>
using Slice = Row16<DT>;  // a lane's 16-byte slice of a row, as floats

// A step at position t runs when t >= 0, t + 1 does not overflow, and the
// group that t completes has a core slot: (t+1)/g <= m_cap (which also bounds
// every visible core, n_core(t) <= (t+1)/g).
__device__ __forceinline__ bool decode_valid(int t, int g, int m_cap) {
  return t >= 0 && t < 0x7fffffff && (t + 1) / g <= m_cap;
}

// Pools the group ending at t with one wave, in pooling mode `mode`: rows
// t-g+1..t-1 from the ring, row t from k_t/v_t; the pooling queries are q_t of
// the kv head's G heads (q_t points at the first of them).
template <int DT, int D>
__device__ __forceinline__ void pool_new_group(int mode, const char* q_t, const char* k_new,
                                               const char* v_new, const char* ring_k,
                                               const char* ring_v, char* ck, char* cv, int t,
                                               int R, int g, int G, float scale_log2) {
  typedef RowLanes<DT, D> RL;
  auto krow = [&](int tau) {
    const int p = t - g + 1 + tau;
    return p == t ? k_new : ring_k + (long)(p % R) * D * RL::ES;
  };
  auto vrow = [&](int tau) {
    const int p = t - g + 1 + tau;
    return p == t ? v_new : ring_v + (long)(p % R) * D * RL::ES;
  };
  auto qrow = [&](int h) { return q_t + (long)h * D * RL::ES; };
  float acck[RL::EPL], accv[RL::EPL];
  switch (mode) {
    case kPoolSoftmaxHeads:
      pool_group<DT, D, kPoolSoftmaxHeads>(krow, vrow, qrow, g, G, scale_log2, acck, accv, nullptr);
      break;
    case kPoolMean:
      pool_group<DT, D, kPoolMean>(krow, vrow, qrow, g, G, scale_log2, acck, accv, nullptr);
      break;
    case kPoolMax:
      pool_group<DT, D, kPoolMax>(krow, vrow, qrow, g, G, scale_log2, acck, accv, nullptr);
      break;
    default:
      pool_group<DT, D, kPoolSoftmax>(krow, vrow, qrow, g, G, scale_log2, acck, accv, nullptr);
      break;
  }
  const int lane = threadIdx.x & 63;
  if (lane < RL::LPK) {  // the core dtype has the input's element size
    Row16<core_dt(DT)>::store(ck + lane * RL::EPL * RL::ES, acck);
    Row16<core_dt(DT)>::store(cv + lane * RL::EPL * RL::ES, accv);
  }
}

// Pass 1.  grid = (splits, Hq / GT, B); the block serves GT query heads.
template <int DT, int D, int GT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const void* __restrict__ q_t_, const void* __restrict__ k_t_, const void* __restrict__ v_t_,
    void* __restrict__ ring_k_, void* __restrict__ ring_v_, int R, void* __restrict__ ck_,
    void* __restrict__ cv_, int m_cap, const int32_t* __restrict__ pos, float* __restrict__ ws_m,
    float* __restrict__ ws_l, float* __restrict__ ws_o, int Hq, int Hkv, int g, int w, int splits,
    float scale_log2, int pool_mode) {
  typedef Slice<DT> S;
  constexpr int ES = DT == 0 ? 4 : 2;
  constexpr int EPL = S::N;
  constexpr int LPK = D * ES / 16;   // lanes per key row
  constexpr int KPW = 64 / LPK;      // key rows per wave load
  constexpr int NW = kThreads / 64;

  const int split = blockIdx.x;
  const int hg = blockIdx.y;          // query-head group
  const int b = blockIdx.z;
  const int G = Hq / Hkv;
  const int h0 = hg * GT;
  const int hk = h0 / G;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ks = lane / LPK;
  const int d0 = (lane % LPK) * EPL;
  const int t = pos[b];
  const long bhk = (long)b * Hkv + hk;
  const long st_base = ((long)b * Hq + h0) * splits + split;  // partial state of head h0

  if (!decode_valid(t, g, m_cap)) {
    if (threadIdx.x < GT) ws_m[st_base + (long)threadIdx.x * splits] = __uint_as_float(kInvalidState);
    return;
  }

  const char* q_t = static_cast<const char*>(q_t_);
  const char* k_new = static_cast<const char*>(k_t_) + bhk * D * ES;
  const char* v_new = static_cast<const char*>(v_t_) + bhk * D * ES;
  char* ring_k = static_cast<char*>(ring_k_) + bhk * R * D * ES;
  char* ring_v = static_cast<char*>(ring_v_) + bhk * R * D * ES;
  char* ck = static_cast<char*>(ck_) + bhk * m_cap * D * ES;
  char* cv = static_cast<char*>(cv_) + bhk * m_cap * D * ES;

  // Cache maintenance by one block per (b, kv head).
  if (split == 0 && h0 % G == 0) {
    if (wave == 0) {
      // append k_t, v_t at slot t % R
      const long slot = (long)(t % R) * D * ES;
      for (int i = lane * 16; i < D * ES; i += 64 * 16) {
        *reinterpret_cast<uint4*>(ring_k + slot + i) = *reinterpret_cast<const uint4*>(k_new + i);
        *reinterpret_cast<uint4*>(ring_v + slot + i) = *reinterpret_cast<const uint4*>(v_new + i);
      }
    } else if (wave == 1 && (t + 1) % g == 0) {
      const int jn = (t + 1) / g - 1;
      pool_new_group<DT, D>(pool_mode, q_t + ((long)b * Hq + (long)hk * G) * D * ES, k_new, v_new, ring_k,
                            ring_v, ck + (long)jn * D * ES, cv + (long)jn * D * ES, t, R, g, G,
                            scale_log2);
    }
  }

  const int nc = n_core(t, g, w);
  const int lo = win_lo(t, w);
  const int nvis = nc + (t - lo + 1);
  const int chunk = (nvis + splits - 1) / splits;
  const int f_begin = min(nvis, split * chunk);
  const int f_end = min(nvis, f_begin + chunk);

  float qs[GT][EPL];
#pragma unroll
  for (int i = 0; i < GT; ++i) {
    S::load(q_t + (((long)b * Hq + h0 + i) * D + d0) * ES, qs[i]);
  }
  float mrun[GT], lrun[GT], acc[GT][EPL];
#pragma unroll
  for (int i = 0; i < GT; ++i) {
    mrun[i] = -INFINITY;
    lrun[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[i][e] = 0.f;
  }

  // Each iteration: every lane group of every wave takes kBatch keys.
  constexpr int kStep = NW * KPW * kBatch;
  for (int f0 = f_begin; f0 < f_end; f0 += kStep) {
    float kx[kBatch][EPL], vx[kBatch][EPL];
    bool ok[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int f = f0 + (j * NW + wave) * KPW + ks;
      ok[j] = f < f_end;
      const char* kr = nullptr;
      const char* vr = nullptr;
      if (ok[j]) {
        if (f < nc) {  // cores: the core dtype, same element size
          Slice<core_dt(DT)>::load(ck + ((long)f * D + d0) * ES, kx[j]);
          Slice<core_dt(DT)>::load(cv + ((long)f * D + d0) * ES, vx[j]);
        } else {
          const int p = lo + (f - nc);
          if (p == t) {
            kr = k_new;
            vr = v_new;
          } else {
            kr = ring_k + (long)(p % R) * D * ES;
            vr = ring_v + (long)(p % R) * D * ES;
          }
          S::load(kr + d0 * ES, kx[j]);
          S::load(vr + d0 * ES, vx[j]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kx[j][e] = vx[j][e] = 0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < GT; ++i) {
      float s[kBatch];
      float mb = -INFINITY;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(qs[i][e], kx[j][e], part);
#pragma unroll
        for (int o = LPK / 2; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
        s[j] = ok[j] ? part * scale_log2 : -INFINITY;
        mb = fmaxf(mb, s[j]);
      }
      const float mnew = fmaxf(mrun[i], mb);
      if (mnew != -INFINITY) {
        const float alpha = exp2f(mrun[i] - mnew);
        lrun[i] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[i][e] *= alpha;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          const float p = exp2f(s[j] - mnew);
          lrun[i] += p;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[i][e] = fmaf(p, vx[j][e], acc[i][e]);
        }
        mrun[i] = mnew;
      }
    }
  }

  // Merge lane groups within the wave, then the waves through LDS.
  __shared__ float red_m[NW][GT];
  __shared__ float red_l[NW][GT];
  __shared__ float red_o[NW][GT][D];
#pragma unroll
  for (int i = 0; i < GT; ++i) {
#pragma unroll
    for (int o = LPK; o < 64; o <<= 1) {
      const float mo = __shfl_xor(mrun[i], o, 64);
      const float lo2 = __shfl_xor(lrun[i], o, 64);
      const float mnew = fmaxf(mrun[i], mo);
      const float fa = mrun[i] == -INFINITY ? 0.f : exp2f(mrun[i] - mnew);
      const float fb = mo == -INFINITY ? 0.f : exp2f(mo - mnew);
      lrun[i] = lrun[i] * fa + lo2 * fb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[i][e], o, 64);
        acc[i][e] = acc[i][e] * fa + ao * fb;
      }
      mrun[i] = mnew;
    }
    if (ks == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][i][d0 + e] = acc[i][e];
      if (lane == 0) {
        red_m[wave][i] = mrun[i];
        red_l[wave][i] = lrun[i];
      }
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < GT * D; idx += kThreads) {
    const int i = idx / D, e = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < NW; ++wv) M = fmaxf(M, red_m[wv][i]);
    float lsum = 0.f, osum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < NW; ++wv) {
        const float f = red_m[wv][i] == -INFINITY ? 0.f : exp2f(red_m[wv][i] - M);
        lsum += red_l[wv][i] * f;
        osum += red_o[wv][i][e] * f;
      }
    }
    const long st = st_base + (long)i * splits;
    ws_o[st * D + e] = osum;
    if (e == 0) {
      ws_m[st] = M;
      ws_l[st] = lsum;
    }
  }
}

// Pass 1 on the matrix cores (bf16 inputs, G <= 8 query heads per kv head).
// grid = (splits, 1, B * Hkv); four waves per block.  Each wave streams its own
// 32-key tiles of the block's key range -- no block barrier in the main loop.
// The block's raw keys come first (bf16 operands), then its cores (fp16, the
// core cache's dtype; the Q fragments are converted once in registers), so no
// tile mixes the two:
//   S^T (32 keys x 32 columns) = K . Q^T with v_mfma_f32_32x32x16_{bf16,f16};
//   the columns are the kv head's G query heads, the rest zero (the matrix
//   cores have ample headroom here: the loop is bound by HBM);
//   K rows go straight from memory into the A operand registers;
//   V rows are transposed through a wave-private LDS tile into V^T, with the
//   key order permuted to match the score layout, so P^T is used in place as
//   the B operand of O^T += V^T . P^T.
// The four waves' online-softmax states are merged through LDS at the end.
constexpr int kDecBK = 32;     // keys per wave tile
constexpr int kDecVRow = 80;   // bytes per V^T row in LDS: 32 keys + 16 pad

template <int D>
__global__ __launch_bounds__(256, 2) void decode_mfma_kernel(
    const uint16_t* __restrict__ q_t, const uint16_t* __restrict__ k_t,
    const uint16_t* __restrict__ v_t, uint16_t* __restrict__ ring_k, uint16_t* __restrict__ ring_v,
    int R, uint16_t* __restrict__ ck, uint16_t* __restrict__ cv, int m_cap,
    const int32_t* __restrict__ pos, float* __restrict__ ws_m, float* __restrict__ ws_l,
    float* __restrict__ ws_o, int Hq, int Hkv, int g, int w, int splits, float c, int pool_mode) {
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x16 __attribute__((ext_vector_type(16)));
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int KS = D / 16;            // k-steps of K.Q^T
  constexpr int DB = D / 32;            // 32-dim blocks of O^T
  constexpr int VBytes = D * kDecVRow;  // one wave's V^T tile
  constexpr int NVP = (kDecBK / 4) * (D / 8) / 64;  // (key quad, dim octet) pairs per lane
  // the V^T tiles, reused after the loop for the merge of the waves' states
  constexpr int kMaxG = 8;
  static_assert(4 * kMaxG * D * 4 <= 4 * VBytes, "merge area fits in the V^T tiles");
  __shared__ __attribute__((aligned(16))) char lds[4 * VBytes];
  __shared__ float red_m[4][kMaxG], red_l[4][kMaxG];

  const int split = blockIdx.x;
  const int bk = blockIdx.z;               // b * Hkv + kv head
  const int b = bk / Hkv, hk = bk % Hkv;
  const int G = Hq / Hkv;
  const int h0 = hk * G;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31, hh = lane >> 5;
  const int t = pos[b];
  const long st_base = ((long)b * Hq + h0) * splits + split;  // state of head h0

  if (!decode_valid(t, g, m_cap)) {
    if ((int)threadIdx.x < G) ws_m[st_base + (long)threadIdx.x * splits] = __uint_as_float(kInvalidState);
    return;
  }
  const long bkl = bk;
  const uint16_t* k_new = k_t + bkl * D;
  const uint16_t* v_new = v_t + bkl * D;
  uint16_t* rk = ring_k + bkl * R * D;
  uint16_t* rv = ring_v + bkl * R * D;
  uint16_t* ckb = ck + bkl * m_cap * D;
  uint16_t* cvb = cv + bkl * m_cap * D;

  // cache maintenance by the split-0 block of each (b, kv head)
  if (split == 0) {
    if (wave == 0) {
      const long slot = (long)(t % R) * D;
      for (int i = lane * 8; i < D; i += 64 * 8) {
        *reinterpret_cast<uint4*>(rk + slot + i) = *reinterpret_cast<const uint4*>(k_new + i);
        *reinterpret_cast<uint4*>(rv + slot + i) = *reinterpret_cast<const uint4*>(v_new + i);
      }
    } else if (wave == 1 && (t + 1) % g == 0) {
      const int jn = (t + 1) / g - 1;
      pool_new_group<1, D>(pool_mode, reinterpret_cast<const char*>(q_t + ((long)b * Hq + h0) * D),
                           reinterpret_cast<const char*>(k_new), reinterpret_cast<const char*>(v_new),
                           reinterpret_cast<const char*>(rk), reinterpret_cast<const char*>(rv),
                           reinterpret_cast<char*>(ckb + (long)jn * D), reinterpret_cast<char*>(cvb + (long)jn * D),
                           t, R, g, G, c);
    }
  }

  const int nc = n_core(t, g, w);
  const int lo = win_lo(t, w);
  const int nvis = nc + (t - lo + 1);
  const int chunk = (nvis + splits - 1) / splits;
  const int f_begin = min(nvis, split * chunk);
  const int f_end = min(nvis, f_begin + chunk);

  // row pointer of visible key f (core, ring slot, or the new token)
  auto krow = [&](int f, bool values) -> const uint16_t* {
    if (f < nc) return (values ? cvb : ckb) + (long)f * D;
    const int p = lo + (f - nc);
    if (p == t) return values ? v_new : k_new;
    return (values ? rv : rk) + (long)(p % R) * D;
  };

  // B operand: column j = query head h0 + j (zero past G); dims 16ks + 8hh ..
  bf16x8 qb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (j < G) {
      qb[ks] = *reinterpret_cast<const bf16x8*>(q_t + ((long)b * Hq + h0 + j) * D + 16 * ks + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qb[ks][e] = static_cast<__bf16>(0.0f);
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  char* vt = lds + wave * VBytes;

  // The wave's tiles of keys fb .. fe-1, all raw (CORE false: bf16) or all
  // cores (CORE true: fp16).
  auto run = [&](int fb, int fe, auto core_tag) {
    constexpr bool CORE = decltype(core_tag)::value;
    auto mfma = [](const bf16x8& a, const bf16x8& bq, const f32x16& acc) {
      if constexpr (CORE)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, bq), acc, 0, 0, 0);
      else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq, acc, 0, 0, 0);
    };
    for (int f0 = fb + wave * kDecBK; f0 < fe; f0 += 4 * kDecBK) {
      // K rows -> A operand registers (zero past fe)
      u32x4 ka[KS];
      {
        const int f = f0 + j;
        const bool ok = f < fe;
        const uint16_t* kr = ok ? krow(f, false) : k_new;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          ka[ks] = ok ? *reinterpret_cast<const u32x4*>(kr + 16 * ks + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
      }
      // V rows: lane covers NVP (key quad, dim octet) pairs
      u32x4 va[NVP][4];
#pragma unroll
      for (int pi = 0; pi < NVP; ++pi) {
        const int pair = lane + 64 * pi;
        const int q = pair % (kDecBK / 4), oct = pair / (kDecBK / 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int f = f0 + 4 * q + i;
          va[pi][i] = f < fe ? *reinterpret_cast<const u32x4*>(krow(f, true) + 8 * oct)
                             : u32x4{0u, 0u, 0u, 0u};
        }
      }
      // S^T = K.Q^T
      f32x16 sx;
#pragma unroll
      for (int r = 0; r < 16; ++r) sx[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sx = mfma(__builtin_bit_cast(bf16x8, ka[ks]), qb[ks], sx);
      // V^T into the wave's LDS tile (keys permuted: bits 2 and 3 swapped)
#pragma unroll
      for (int pi = 0; pi < NVP; ++pi) {
        const int pair = lane + 64 * pi;
        const int q = pair % (kDecBK / 4), oct = pair / (kDecBK / 4);
        const int k0 = 4 * q;
        const int kpos0 = (k0 & ~15) | ((k0 & 4) << 1) | ((k0 & 8) >> 1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int dw = i >> 1;
          const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t lo2 = __builtin_amdgcn_perm(va[pi][1][dw], va[pi][0][dw], sel);
          const uint32_t hi2 = __builtin_amdgcn_perm(va[pi][3][dw], va[pi][2][dw], sel);
          *reinterpret_cast<uint2*>(vt + (8 * oct + i) * kDecVRow + 2 * kpos0) = make_uint2(lo2, hi2);
        }
      }
      // mask keys past the range; key of register r = 8(r/4) + 4hh + r%4
      if (f0 + kDecBK > fe) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 8 * (r >> 2) + 4 * hh + (r & 3);
          sx[r] = f0 + kk < fe ? sx[r] : -INFINITY;
        }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sx[r]);
      {
        auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(rr[0]), __uint_as_float(rr[1]));
      }
      const float mnew = fmaxf(m, mt);
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - mnew) * c);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      const float mc = (m == -INFINITY ? 0.f : m) * c;
      // probabilities rounded to the tile's operand type; the row sum adds
      // exactly the rounded values the P.V product uses
      u32x4 pw[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sx[r], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sx[r + 1], c, -mc));
        uint32_t pk;
        if constexpr (CORE) {
          typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
          pk = pack_f16x2(p0, p1);
          l = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pk), f16x2{(_Float16)1.0f, (_Float16)1.0f}, l, false);
        } else {
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          pk = pack_bf16x2(p0, p1);
          l = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk),
                                              bf16x2{static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)}, l, false);
        }
        pw[r >> 3][(r & 7) >> 1] = pk;
      }
      // O^T += V^T . P^T
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (32 * db + j) * kDecVRow + (16 * cc + 8 * hh) * 2);
          o[db] = mfma(a, __builtin_bit_cast(bf16x8, pw[cc]), o[db]);
        }
    }
  };
  // raw keys of this split (bf16), then its cores (fp16)
  run(max(f_begin, nc), f_end, std::false_type{});
  if (f_begin < nc) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(static_cast<float>(qb[ks][e]));
      qb[ks] = __builtin_bit_cast(bf16x8, h);
    }
    run(f_begin, min(f_end, nc), std::true_type{});
  }

  // merge the four waves: lane (column j, half hh) holds dims 32db + 8(r/4) + 4hh + r%4
  {
    auto rr = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    l = __uint_as_float(rr[0]) + __uint_as_float(rr[1]);
  }
  __syncthreads();  // every wave is done with its V^T tile
  float* red_o = reinterpret_cast<float*>(lds);   // [4 waves][kMaxG][D]
  if (j < G) {
    if (hh == 0) {
      red_m[wave][j] = m;
      red_l[wave][j] = l;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        red_o[(wave * kMaxG + j) * D + 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3)] = o[db][r];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int hcol = idx / D, e = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) M = fmaxf(M, red_m[wv][hcol]);
    float lsum = 0.f, osum = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) {
        const float f = red_m[wv][hcol] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((red_m[wv][hcol] - M) * c);
        lsum += red_l[wv][hcol] * f;
        osum += red_o[(wv * kMaxG + hcol) * D + e] * f;
      }
    }
    const long st = st_base + (long)hcol * splits;
    ws_o[st * D + e] = osum;
    if (e == 0) {
      ws_m[st] = M * c;   // the combine pass works in log2 units
      ws_l[st] = lsum;
    }
  }
}

// Pass 2.  One block of D threads per (b, query head).  The split states are
// staged in LDS first so that the weighted sum issues independent loads.  A
// valid step never has t = INT32_MAX (decode_valid), so the advance of pos
// cannot overflow.
constexpr int kMaxSplits = 128;

template <int OT, int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float* __restrict__ ws_m, const float* __restrict__ ws_l, const float* __restrict__ ws_o,
    void* __restrict__ out_, int32_t* __restrict__ pos, int advance_pos, int Hq, int splits) {
  typedef Elem<OT> EO;
  __shared__ float sm[kMaxSplits];
  __shared__ float sl[kMaxSplits];
  __shared__ float red[2];
  const long bh = blockIdx.x;
  const int e = threadIdx.x;
  const long st0 = bh * splits;
  for (int s = e; s < splits; s += D) {
    sm[s] = ws_m[st0 + s];
    sl[s] = ws_l[st0 + s];
  }
  __syncthreads();
  if (e < 64) {
    float M = -INFINITY;
    float bad = 0.f;
    for (int s = e; s < splits; s += 64) {
      M = fmaxf(M, sm[s]);
      bad += __float_as_uint(sm[s]) == kInvalidState ? 1.f : 0.f;
    }
    M = wave_max(M);
    bad = wave_sum(bad);
    if (e == 0) {
      red[0] = M;
      red[1] = bad;
    }
  }
  __syncthreads();
  const float M = red[0];
  for (int s = e; s < splits; s += D) {
    const float ms = sm[s];
    // weight of split s; a NaN max from the data stays NaN and reaches the output
    sm[s] = (ms == -INFINITY || __float_as_uint(ms) == kInvalidState) ? 0.f : exp2f(ms - M);
  }
  __syncthreads();
  float lsum = 0.f, osum = 0.f;
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float f = sm[s];
    lsum = fmaf(sl[s], f, lsum);
    osum = fmaf(ws_o[(st0 + s) * D + e], f, osum);
  }
  // an invalid step (every split marked kInvalidState: validity depends on t
  // alone) writes NaN and leaves pos where it is
  const bool invalid = red[1] != 0.f;
  const float r = invalid ? NAN : osum / lsum;
  EO::store(static_cast<typename EO::T*>(out_), bh * D + e, r);
  if (advance_pos && e == 0 && bh % Hq == 0 && !invalid) pos[bh / Hq] += 1;
}

int pick_gt(int G) {
  if (G % 8 == 0) return 8;
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

template <int DT, int D, int GT>
void launch_split(const void* q_t, const void* k_t, const void* v_t, void* ring_k, void* ring_v,
                  int R, void* ck, void* cv, int m_cap, const int32_t* pos, float* ws_m,
                  float* ws_l, float* ws_o, const Shape& sh, int splits, int pool_mode,
                  hipStream_t s) {
  dim3 grid(splits, sh.Hq / GT, sh.B);
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((decode_split_kernel<DT, D, GT>), grid, dim3(kThreads), 0, s, q_t, k_t, v_t,
                     ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh.Hq, sh.Hkv, sh.g,
                     sh.w, splits, scale_log2, pool_mode);
}

template <int DT, int D>
void launch_split_g(int GT, const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                    void* ring_v, int R, void* ck, void* cv, int m_cap, const int32_t* pos,
                    float* ws_m, float* ws_l, float* ws_o, const Shape& sh, int splits,
                    int pool_mode, hipStream_t s) {
  switch (GT) {
    case 8: launch_split<DT, D, 8>(q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, splits, pool_mode, s); break;
    case 4: launch_split<DT, D, 4>(q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, splits, pool_mode, s); break;
    case 2: launch_split<DT, D, 2>(q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, splits, pool_mode, s); break;
    default: launch_split<DT, D, 1>(q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, splits, pool_mode, s); break;
  }
}

// Prefill -> decode handoff: the last R positions of each sequence into its ring.
__global__ __launch_bounds__(256) void fill_ring_kernel(const char* __restrict__ k,
                                                        const char* __restrict__ v,
                                                        char* __restrict__ ring_k,
                                                        char* __restrict__ ring_v, int R,
                                                        const int32_t* __restrict__ seq_len, int Hkv,
                                                        int Lk, int row_bytes) {
  const int bh = blockIdx.y;  // b * Hkv + kv head
  const int len = seq_len[bh / Hkv];
  if (len < 0 || len > Lk) return;
  const int n = min(len, R);  // rows to copy: positions len-n .. len-1
  const int cpr = row_bytes / 16;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < (long)n * cpr;
       i += (long)gridDim.x * blockDim.x) {
    const int r = (int)(i / cpr), c = (int)(i % cpr);
    const int p = len - n + r;
    const long src = ((long)bh * Lk + p) * row_bytes + c * 16;
    const long dst = ((long)bh * R + p % R) * row_bytes + c * 16;
    *reinterpret_cast<uint4*>(ring_k + dst) = *reinterpret_cast<const uint4*>(k + src);
    *reinterpret_cast<uint4*>(ring_v + dst) = *reinterpret_cast<const uint4*>(v + src);
  }
}

}  // namespace

hipError_t launch_fill_ring(const void* k, const void* v, void* ring_k, void* ring_v, int R,
                            const int32_t* seq_len, int B, int Hkv, int Lk, int d, int elem_bytes,
                            hipStream_t s) {
  const int row_bytes = d * elem_bytes;
  const long chunks = (long)R * (row_bytes / 16);
  const int bx = (int)std::min<long>((chunks + 255) / 256, 64);
  hipLaunchKernelGGL(fill_ring_kernel, dim3(bx, B * Hkv), dim3(256), 0, s,
                     static_cast<const char*>(k), static_cast<const char*>(v),
                     static_cast<char*>(ring_k), static_cast<char*>(ring_v), R, seq_len, Hkv, Lk,
                     row_bytes);
  return hipGetLastError();
}

// ---- fixed device scratch for callers that cannot allocate
// The split states of cca_attn_decode_scratch live in this array: one copy
// per GPU, held until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is a stand-in, not a device address): the
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return hipSuccess;
}

DecodePlan decode_plan(int B, int Hq, int Hkv, int d, int m_cap, int g, int w) {
  (void)g;
  // Enough blocks to fill the GPU (about 512 for 256 CUs), but no split
  // shorter than 128 keys of the largest visible range (every core slot plus
  // the window).
  const long nvis_max = (long)m_cap + w;
  const long bk = (long)B * Hkv;
  long splits = (512 + bk - 1) / bk;
  const long by_len = (nvis_max + 127) / 128;
  if (splits > by_len) splits = by_len;
  if (splits < 1) splits = 1;
  if (splits > kMaxSplits) splits = kMaxSplits;
  DecodePlan p;
  p.splits = (int)splits;
  p.ws_bytes = (size_t)B * Hq * splits * (size_t)(d + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                         void* ring_v, int R, void* ck, void* cv, int m_cap, int32_t* pos,
                         int advance_pos, void* out, int out_dt, void* ws, const DecodePlan& plan,
                         const Shape& sh, int dt, int pool_mode, hipStream_t s) {
  const int S = plan.splits;
  float* ws_m = static_cast<float*>(ws);
  float* ws_l = ws_m + (size_t)sh.B * sh.Hq * S;
  float* ws_o = ws_l + (size_t)sh.B * sh.Hq * S;
  const int GT = pick_gt(sh.G());
  if (dt == 1 && sh.G() <= 8) {
    const float c = kLog2e / sqrtf((float)sh.d);
    dim3 grid(S, 1, sh.B * sh.Hkv);
    const uint16_t* q16 = static_cast<const uint16_t*>(q_t);
    const uint16_t* k16 = static_cast<const uint16_t*>(k_t);
    const uint16_t* v16 = static_cast<const uint16_t*>(v_t);
    uint16_t* rk16 = static_cast<uint16_t*>(ring_k);
    uint16_t* rv16 = static_cast<uint16_t*>(ring_v);
    uint16_t* ck16 = static_cast<uint16_t*>(ck);
    uint16_t* cv16 = static_cast<uint16_t*>(cv);
    if (sh.d == 64)
      hipLaunchKernelGGL((decode_mfma_kernel<64>), grid, dim3(256), 0, s, q16, k16, v16, rk16, rv16, R, ck16, cv16, m_cap, pos, ws_m, ws_l, ws_o, sh.Hq, sh.Hkv, sh.g, sh.w, S, c, pool_mode);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<128>), grid, dim3(256), 0, s, q16, k16, v16, rk16, rv16, R, ck16, cv16, m_cap, pos, ws_m, ws_l, ws_o, sh.Hq, sh.Hkv, sh.g, sh.w, S, c, pool_mode);
  } else if (dt == 0) {
    if (sh.d == 64) launch_split_g<0, 64>(GT, q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, S, pool_mode, s);
    else launch_split_g<0, 128>(GT, q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, S, pool_mode, s);
  } else {
    if (sh.d == 64) launch_split_g<1, 64>(GT, q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, S, pool_mode, s);
    else launch_split_g<1, 128>(GT, q_t, k_t, v_t, ring_k, ring_v, R, ck, cv, m_cap, pos, ws_m, ws_l, ws_o, sh, S, pool_mode, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(sh.B * sh.Hq));
  if (out_dt == 0) {
    if (sh.d == 64) hipLaunchKernelGGL((decode_combine_kernel<0, 64>), grid, dim3(64), 0, s, ws_m, ws_l, ws_o, out, pos, advance_pos, sh.Hq, S);
    else hipLaunchKernelGGL((decode_combine_kernel<0, 128>), grid, dim3(128), 0, s, ws_m, ws_l, ws_o, out, pos, advance_pos, sh.Hq, S);
  } else {
    if (sh.d == 64) hipLaunchKernelGGL((decode_combine_kernel<1, 64>), grid, dim3(64), 0, s, ws_m, ws_l, ws_o, out, pos, advance_pos, sh.Hq, S);
    else hipLaunchKernelGGL((decode_combine_kernel<1, 128>), grid, dim3(128), 0, s, ws_m, ws_l, ws_o, out, pos, advance_pos, sh.Hq, S);
  }
  return hipGetLastError();
}

}  // namespace cca
