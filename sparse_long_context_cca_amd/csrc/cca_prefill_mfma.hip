// Fused CCA prefill on the gfx950 matrix cores (bf16 operands, fp32 accumulate).
//
// Row t of head h computes one softmax over [cores 0..n_core(t) ; raw keys
// win_lo(t)..t] (digest at digest.lyk-ai.com/posts/2412.12465, "Method",
// fusion formula; paper card at atlas.scime.ai, "Approach": both contexts are
// fused in a single softmax).
//
// Work decomposition
//   * A workgroup (4 waves) owns 128 query rows that share one kv head: Hw
//     query heads x (128/Hw) consecutive positions, Hw = gcd(G, 4).  Each wave
//     owns 32 rows (one head, 32 consecutive positions).  With GQA the four
//     waves are four query heads at the same positions, so every K/V tile
//     staged in LDS serves all of them.
//   * The workgroup walks the union of its rows' visible keys: first the core
//     tiles 0..n_core(last row) (64 cores each), then the raw tiles covering
//     win_lo(first row)..last row (64 positions each, 64-aligned).  Tiles that
//     every row of a wave sees completely skip the mask; tiles no row of a
//     wave sees are skipped by that wave.
//   * Workgroups are issued longest-first (the last positions see the most
//     cores) and, when the kv heads divide evenly over the 8 XCDs, all
//     workgroups of one kv head run on one XCD so that its core K/V stay in
//     that XCD's L2.
// Per 64-key tile and wave
//   S^T (64 keys x 32 rows) = K_tile . Q^T with v_mfma_f32_32x32x16_bf16
//   (A = K rows from LDS, B = the wave's Q fragment kept in registers);
//   each lane then holds 32 scores of one query row, so the row max needs one
//   exchange with lane l^32 and the row sum is kept per lane until the end.
//   P (bf16) is used in place as the B operand of O^T += V^T . P^T; V is
//   stored transposed in LDS, its keys permuted to match the score layout.
// Online softmax in the log2 domain with fp32 state; K/V tiles are double
// buffered (global loads of tile i+1 are in flight while tile i computes).
#include "cca_device.hpp"
#include "cca_internal.hpp"

namespace cca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kBK = 64;       // keys per tile
constexpr int kVRow = 144;    // bytes per transposed-V row: 64 keys + 16 pad
constexpr float kLazyLog2 = 8.0f;  // rescale threshold of the running max, log2 units

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  void* out;
  int B, Hq, Hkv, L, g, w, m_cap;
  int G, Hw, RP;        // heads per workgroup, rows per head per workgroup
  int nPB, nHG, U;      // position blocks, head groups per kv head, units
  int xcd;              // 1 when units split evenly over 8 XCDs
  float c;              // softmax scale * log2(e)
};

// Lanes l and l^32 hold the two halves of one query row's scores.  One
// v_permlane32_swap of a register with itself leaves {x[l], x[l^32]} in the
// two results (in an order that differs between the lane halves), so the
// pair max and pair sum below are symmetric in them.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int OT>
// Two waves per SIMD (the accumulators stay in arch VGPRs, 256 per wave) so
// that one wave's softmax overlaps the other's matrix ops.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillParams P) {
  constexpr int KS = D / 16;            // k-steps of Q.K^T
  constexpr int DB = D / 32;            // 32-wide dim blocks of the output
  constexpr int KRow = D * 2 + 16;      // bytes per K row in LDS (padded)
  constexpr int KBytes = kBK * KRow;
  constexpr int VBytes = D * kVRow;
  constexpr int Stage = KBytes + VBytes;
  constexpr int LPR = D / 8;            // threads per key row (16 B each)
  constexpr int KPP = kThreads / LPR;   // key rows per load pass
  constexpr int NPK = kBK / KPP;        // load passes for a K tile
  constexpr int NVQ = (kBK / 4) * (D / 8);  // (key quad, dim octet) pairs in a V tile
  __shared__ __attribute__((aligned(16))) char lds[2 * Stage];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar, so that every per-wave quantity below (rows,
  // tile visibility) is known to be uniform and branches on it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int hh = lane >> 5;

  // ---- which rows: longest first, XCD-aware
  const long bid = blockIdx.x;
  int pb, u;
  if (P.xcd) {
    const int per = P.U / 8;
    const long slot = bid >> 3;
    const int x = (int)(bid & 7);
    pb = P.nPB - 1 - (int)(slot / per);
    u = x * per + (int)(slot % per);
  } else {
    pb = P.nPB - 1 - (int)(bid / P.U);
    u = (int)(bid % P.U);
  }
  const int kvp = u / P.nHG;  // b * Hkv + kv head
  const int hg = u % P.nHG;
  const int b = kvp / P.Hkv;
  const int kvh = kvp % P.Hkv;
  const int L = P.L, g = P.g, w = P.w;
  const int h = kvh * P.G + hg * P.Hw + (wave % P.Hw);
  const int P_lo = pb * P.RP;
  const int P_hi = min(L - 1, P_lo + P.RP - 1);
  const int p0 = P_lo + 32 * (wave / P.Hw);

  // ---- this lane's query row and the wave's row range
  const int t_raw = p0 + j;
  const int t = min(t_raw, L - 1);
  const int my_nc = n_core(t, g, w);
  const int my_lo = win_lo(t, w);
  const int w_lo = min(p0, L - 1);
  const int w_hi = min(p0 + 31, L - 1);
  const int wnc_lo = n_core(w_lo, g, w), wnc_hi = n_core(w_hi, g, w);
  const int wlo_lo = win_lo(w_lo, w), wlo_hi = win_lo(w_hi, w);

  // ---- workgroup key range
  const int nc_hi = n_core(P_hi, g, w);
  const int n_ct = (nc_hi + kBK - 1) / kBK;
  const int raw_lo = win_lo(P_lo, w);
  const int r0 = raw_lo & ~(kBK - 1);
  const int n_rt = (P_hi - r0) / kBK + 1;
  const int n_tiles = n_ct + n_rt;

  const long kvrow = (long)kvp;
  const uint16_t* kbase = P.k + kvrow * L * D;
  const uint16_t* vbase = P.v + kvrow * L * D;
  const uint16_t* ckbase = P.ck + kvrow * P.m_cap * D;
  const uint16_t* cvbase = P.cv + kvrow * P.m_cap * D;

  // ---- Q fragment: B operand, lane holds Q[row j][16ks + 8hh .. +7]
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = P.q + (((long)b * P.Hq + h) * L + t) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hh);
  }

  // ---- tile loaders (global -> registers -> LDS)
  // Buffer loads: the resource of each tile starts at the tile's first key and
  // spans only its valid keys, so rows past the end (beyond the last visible
  // core, or past the last row of the workgroup) read as zero in hardware.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  u32x4 kreg[NPK];
  u32x4 vreg[4];
  const int k_oct = tid % LPR;
  const int k_row0 = tid / LPR;
  const int v_oct = tid / 16;   // dim octet
  const int v_quad = tid % 16;  // key quad
  const bool v_act = tid < NVQ;
  int koff[NPK], voff[4];
#pragma unroll
  for (int i = 0; i < NPK; ++i) koff[i] = ((k_row0 + i * KPP) * D + 8 * k_oct) * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = ((4 * v_quad + i) * D + 8 * v_oct) * 2;

  auto load_tile = [&](int it) {
    const bool core = it < n_ct;
    const int base = core ? it * kBK : r0 + (it - n_ct) * kBK;
    const int lim = core ? nc_hi : P_hi + 1;  // keys < lim are valid
    const int nvalid = min(kBK, lim - base);
    const uint16_t* ks = (core ? ckbase : kbase) + (long)base * D;
    const uint16_t* vs = (core ? cvbase : vbase) + (long)base * D;
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ks), 0, nvalid * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vs), 0, nvalid * D * 2, 0x00020000);
#pragma unroll
    for (int i = 0; i < NPK; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[i], 0, 0);
    if (v_act) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vreg[i] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[i], 0, 0);
    }
  };
  auto store_tile = [&](int stage) {
    char* kt = lds + stage * Stage;
    char* vt = kt + KBytes;
#pragma unroll
    for (int i = 0; i < NPK; ++i)
      *reinterpret_cast<u32x4*>(kt + (k_row0 + i * KPP) * KRow + 16 * k_oct) = kreg[i];
    if (v_act) {
      // keys 4q..4q+3 land at permuted positions kpos0..kpos0+3 (bits 2,3 of the key swapped);
      // dim 8*v_oct+i of the four keys becomes one 8-byte row segment of V^T.
      const int q = v_quad;
      const int kpos0 = 16 * (q >> 2) + 8 * (q & 1) + 4 * ((q >> 1) & 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int dw = i >> 1;
        const unsigned sel = (i & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t lo = __builtin_amdgcn_perm(vreg[1][dw], vreg[0][dw], sel);
        const uint32_t hi = __builtin_amdgcn_perm(vreg[3][dw], vreg[2][dw], sel);
        *reinterpret_cast<uint2*>(vt + (8 * v_oct + i) * kVRow + 2 * kpos0) = make_uint2(lo, hi);
      }
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY, l = 0.f;
  const float c = P.c;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int stage = it & 1;
    if (it + 1 < n_tiles) load_tile(it + 1);

    const bool core = it < n_ct;
    const int base = core ? it * kBK : r0 + (it - n_ct) * kBK;
    // visibility of this tile for the wave's rows (wave-uniform)
    bool skip, full;
    if (core) {
      skip = base >= wnc_hi;
      full = base + kBK <= wnc_lo;
    } else {
      skip = base > w_hi || base + kBK - 1 < wlo_lo;
      full = base >= wlo_hi && base + kBK - 1 <= w_lo;
    }
    if (!skip) {
      const char* kt = lds + stage * Stage;
      const char* vt = kt + KBytes;
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(kt + (32 * kb + j) * KRow + (16 * ks + 8 * hh) * 2);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
        }
      }
      if (!full) {
        // (the empty asm keeps this a real branch: masks are needed on edge tiles only)
        asm volatile("" ::: "memory");
        // key kk of the tile is visible to this lane's row iff lo_rel <= kk <= hi_rel
        const int lo_rel = core ? 0 : my_lo - base;
        const int hi_rel = core ? my_nc - 1 - base : t - base;
        const unsigned span = (unsigned)(hi_rel - lo_rel);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool vis = hi_rel >= lo_rel && (unsigned)(kk - lo_rel) <= span;
            s[kb][r] = vis ? s[kb][r] : -INFINITY;
          }
      }
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = pair_max(mt);
      // Lazy rescale: the reference max m only moves when the row max grows by
      // more than kLazyLog2 (log2 units), so probabilities stay <= 2^kLazyLog2
      // and the accumulator rescale is skipped on almost every tile.  The
      // final normalisation divides by a sum taken against the same m.
      const float mnew = fmaxf(m, mt);
      const bool grow = (mnew - m) * c > kLazyLog2;  // false while both are -inf
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = grow ? __builtin_amdgcn_exp2f((m - mnew) * c) : 1.0f;
        m = grow ? mnew : m;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      const float mc = (m == -INFINITY ? 0.f : m) * c;
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], c, -mc));
          bf16x2 pk;
          pk[0] = static_cast<__bf16>(p0);
          pk[1] = static_cast<__bf16>(p1);
          // row sum of the rounded probabilities actually fed to P.V
          l = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, l, false);
          pb[2 * kb + (r >> 3)][r & 7] = pk[0];
          pb[2 * kb + (r >> 3)][(r & 7) + 1] = pk[1];
        }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(vt + (32 * db + j) * kVRow + (16 * cc + 8 * hh) * 2);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], o[db], 0, 0, 0);
        }
    }
    if (it + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- normalise and store: lane holds dims 32db + 8(r/4) + 4hh + r%4 of row j
  const float ltot = pair_sum(l);
  const float inv = 1.0f / ltot;
  if (t_raw < L) {
    const long orow = (((long)b * P.Hq + h) * L + t_raw) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * hh;
        const float x0 = o[db][4 * rr + 0] * inv, x1 = o[db][4 * rr + 1] * inv;
        const float x2 = o[db][4 * rr + 2] * inv, x3 = o[db][4 * rr + 3] * inv;
        if (OT == 1) {
          uint16_t* out = static_cast<uint16_t*>(P.out);
          *reinterpret_cast<uint2*>(out + orow + d0) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
        } else {
          float* out = static_cast<float*>(P.out);
          *reinterpret_cast<float4*>(out + orow + d0) = make_float4(x0, x1, x2, x3);
        }
      }
  }
}

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

}  // namespace

hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* ck,
                               const void* cv, int m_cap, void* out, int out_dt, const Shape& sh,
                               hipStream_t s) {
  PrefillParams P;
  P.q = static_cast<const uint16_t*>(q);
  P.k = static_cast<const uint16_t*>(k);
  P.v = static_cast<const uint16_t*>(v);
  P.ck = static_cast<const uint16_t*>(ck);
  P.cv = static_cast<const uint16_t*>(cv);
  P.out = out;
  P.B = sh.B;
  P.Hq = sh.Hq;
  P.Hkv = sh.Hkv;
  P.L = sh.L;
  P.g = sh.g;
  P.w = sh.w;
  P.m_cap = m_cap;
  P.G = sh.G();
  P.Hw = gcd_int(P.G, 4);
  P.RP = 32 * (4 / P.Hw);
  P.nPB = (sh.L + P.RP - 1) / P.RP;
  P.nHG = P.G / P.Hw;
  P.U = sh.B * sh.Hkv * P.nHG;
  P.xcd = (P.U % 8 == 0) ? 1 : 0;
  P.c = kLog2e / sqrtf((float)sh.d);
  const long blocks = (long)P.nPB * P.U;
  if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
  if (sh.d == 64) {
    if (out_dt == 1) hipLaunchKernelGGL((prefill_mfma_kernel<64, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, s, P);
    else hipLaunchKernelGGL((prefill_mfma_kernel<64, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, s, P);
  } else {
    if (out_dt == 1) hipLaunchKernelGGL((prefill_mfma_kernel<128, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, s, P);
    else hipLaunchKernelGGL((prefill_mfma_kernel<128, 0>), dim3((unsigned)blocks), dim3(kThreads), 0, s, P);
  }
  return hipGetLastError();
}

}  // namespace cca
