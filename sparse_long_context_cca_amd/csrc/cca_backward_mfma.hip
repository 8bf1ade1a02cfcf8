// Backward pass of the CCA attention prefill on the gfx950 matrix cores (bf16
// operands for the raw keys, fp16 for the cores, which are stored in fp16;
// fp32 accumulate and gradients).
//
// Gradients of the fused softmax (digest at digest.lyk-ai.com/posts/2412.12465,
// "Method", fusion formula; the pages fine-tune with CCA attention in place:
// paper card at atlas.scime.ai, summary; rebuttal at paperhub.cn, answer on the
// fine-tuning setting).  For row t with visible keys k (cores, then raw), score
// S = q_t . key_k / sqrt(d), P = softmax(S) recomputed from the row's
// log-sum-exp, dP = dO_t . value_k and D_t = dO_t . o_t:
//   dS = P (dP - D_t)
//   dq_t = sum_k dS key_k / sqrt(d)                      (dq_mfma_kernel)
//   dkey_k = sum_t dS q_t / sqrt(d), dvalue_k = sum_t P dO_t   (dkv_mfma_kernel)
// Kernels, in launch order:
//   1. dq_mfma_kernel    row-parallel, the forward's work decomposition: per
//                        64-key tile S^T = K.Q^T and dP^T = V.dO^T (K, V rows
//                        from LDS, Q and dO fragments in registers), and
//                        dQ^T += K^T.dS^T with K^T through transposing reads;
//                        the dQ product of tile i-1 is interleaved with tile
//                        i's exponentials, as in the forward
//   2. dkv_mfma_kernel   key-parallel: a workgroup owns 128 keys (raw
//                        positions, or cores) of one kv head and walks the
//                        rows that see them for every query head of the
//                        group.  A pair of waves shares 32 keys (K fragments
//                        in registers, V fragments in LDS) and splits each
//                        tile's rows: S = Q.K^T, dP = dO.V^T (Q, dO rows from
//                        LDS), dV^T += dO^T.P and dK^T += Q^T.dS (dO^T, Q^T
//                        through transposing reads) for all head dims; the
//                        pair's partial sums meet in LDS at the end.  Raw keys
//                        get plain stores; core rows are split over workgroups
//                        and meet by atomic adds in an fp32 workspace.
// The pooling share of the gradients is added afterwards by the pooling
// backward of cca_backward.hip.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "cca_device.hpp"
#include "cca_internal.hpp"
#include "cca_lds.hpp"
#include "cca_queue.hpp"

namespace cca {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTileRows = 64;    // keys per tile (dQ), rows per tile (dK dV)
constexpr int kKeysPerUnit = 128;  // keys per dK dV workgroup (4 wave pairs x 32)
constexpr int kCoreSplit = 8192;   // rows per core unit (absolute, aligned splits)

// A wave-uniform value held in a scalar register.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ------------------------------------------------------------------ 1. dQ

struct DqParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  const uint16_t* dout;
  const uint16_t* out;
  const float* lse;
  float2* stats;     // written here: per row {lse * log2(e), dO . O}
  uint16_t* q16;     // written here: fp16 copies of q and dout, for the dK dV kernel
  uint16_t* do16;
  float* dq;
  int B, Hq, Hkv, L, g, w, m_cap;
  int G, Hw, RP;     // heads per workgroup, rows per head per workgroup
  int nPB, nHG, U;   // position blocks, head groups per kv head, units
  int xcd;
  float c, scale;
  int total;         // items (position block x unit) in all
  int n_static;      // items 0 .. n_static-1 go one to a workgroup, in block order
  int qslot;         // work-queue slot of this launch (for the items after them)
};

// work-queue counters of the dQ launches in flight, one 16-word slot each
__device__ unsigned g_dq_queue[kQueueSlots * 16];

template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_mfma_kernel(DqParams P) {
  constexpr int NW = 8, kThreads = 64 * NW;
  constexpr int KS = D / 16, DB = D / 32, CPR = D / 8;
  typedef BothWaysTile<D> KT;          // K: row reads (S) and transposing reads (dQ)
  constexpr int VRow = D * 2 + 16;     // V: row reads only; one chunk of padding per row
  constexpr int VBytes = kTileRows * VRow;
  static_assert(VBytes % 1024 == 0, "V tile is a whole number of wave loads");
  constexpr int NKI = KT::kLoads, NVI = VBytes / 1024, NL = NKI + NVI;
  constexpr int NLW = (NL + NW - 1) / NW, NLMIN = NL / NW;
  // K: a ring of four slots (a tile's K is read once more, by the dQ product
  // deferred to the next iteration); V: a ring of three
  __shared__ __attribute__((aligned(16))) char lds[4 * KT::kBytes + 3 * VBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int j = lane & 31, hh = lane >> 5;

  // ---- rows: longest first, all units of one kv head on one XCD when possible
  auto item_body = [&](const long bid) {
  const auto* const A = kernel_args<DqParams>();
  int pb, u;
  if (A->xcd) {
    const int per = A->U / 8;
    const long slot = bid >> 3;
    const int x = (int)(bid & 7);
    pb = A->nPB - 1 - (int)(slot / per);
    u = x * per + (int)(slot % per);
  } else {
    pb = A->nPB - 1 - (int)(bid / A->U);
    u = (int)(bid % A->U);
  }
  const int kvp = u / A->nHG, hg = u % A->nHG;
  const int b = kvp / A->Hkv;
  const int g = A->g, w = A->w, L = A->L;
  const int h = (kvp % A->Hkv) * A->G + hg * A->Hw + (wave % A->Hw);
  const int row0 = pb * A->RP + 32 * (wave / A->Hw);
  const int P_lo = pb * A->RP;
  const int P_hi = min(L - 1, P_lo + A->RP - 1);
  const int t_raw = row0 + j;
  const int t = min(t_raw, L - 1);
  const int w_lo = uni(min(row0, L - 1)), w_hi = uni(min(row0 + 31, L - 1));
  const int wnc_lo = uni(n_core(w_lo, g, w));
  const int wlo_hi = uni(win_lo(w_hi, w));
  // key tiles: raw tiles 0 .. n_rt-1 (bf16 operands), then core tiles (fp16)
  const int nc_hi = uni(n_core(P_hi, g, w));
  const int n_ct = uni((nc_hi + kTileRows - 1) / kTileRows);
  const int r0 = win_lo(P_lo, w) & ~(kTileRows - 1);
  const int n_rt = uni((P_hi - r0) / kTileRows + 1);
  const int n_tiles = uni(n_ct + n_rt);

  const uint16_t* kbase = A->k + (long)kvp * L * D;
  const uint16_t* vbase = A->v + (long)kvp * L * D;
  const uint16_t* ckbase = A->ck + (long)kvp * A->m_cap * D;
  const uint16_t* cvbase = A->cv + (long)kvp * A->m_cap * D;

  // ---- this lane's row: Q and dO fragments (B operands), statistics
  const long grow = ((long)b * A->Hq + h) * L + t;
  // The row's statistics are made here: D_t = dO_t . o_t (the lane's half
  // of the dims, plus its partner lane's), lse in base 2.  The lane that owns
  // row t (lanes past the sequence end repeat row L-1) also stores them, with
  // fp16 copies of its q and dO fragments, for the dK dV kernel.
  bf16x8 qf[KS], gf[KS];
  float dacc = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const long e0 = grow * D + 16 * ks + 8 * hh;
    qf[ks] = *reinterpret_cast<const bf16x8*>(A->q + e0);
    gf[ks] = *reinterpret_cast<const bf16x8*>(A->dout + e0);
    const bf16x8 of = *reinterpret_cast<const bf16x8*>(A->out + e0);
#pragma unroll
    for (int e = 0; e < 8; ++e) dacc = fmaf(static_cast<float>(of[e]), static_cast<float>(gf[ks][e]), dacc);
  }
  const float Dt = dacc + __shfl_xor(dacc, 32, 64);
  const float lse2 = A->lse[grow] * kLog2e;
  if (t_raw < L) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const long e0 = grow * D + 16 * ks + 8 * hh;
      *reinterpret_cast<bf16x8*>(A->q16 + e0) = bf16_frag_to_f16(qf[ks]);
      *reinterpret_cast<bf16x8*>(A->do16 + e0) = bf16_frag_to_f16(gf[ks]);
    }
    if (hh == 0) A->stats[grow] = make_float2(lse2, Dt);
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]), "v"(gf[ks]));
  asm volatile("" ::"v"(lse2), "v"(Dt));

  // ---- tile loaders: load index li < NKI fills the K tile, the rest the V tile
  int soff[NLW];
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int li = wave + NW * i;
    if (li < NKI) {
      soff[i] = KT::src_offset(li * 64 + lane);
    } else {
      const int slot = (li - NKI) * 64 + lane;
      const int row = slot / (CPR + 1), chunk = slot % (CPR + 1);
      soff[i] = chunk < CPR ? (row * D + 8 * chunk) * 2 : 0x40000000;
    }
  }
  auto tile_core = [&](int it) { return it >= n_rt; };
  auto tile_base = [&](int it) { return it >= n_rt ? (it - n_rt) * kTileRows : r0 + it * kTileRows; };
  auto kbuf = [&](int s) { return lds + s * KT::kBytes; };
  auto vbuf = [&](int s) { return lds + 4 * KT::kBytes + s * VBytes; };
  auto load_tile = [&](int kslot, int vslot, int it) {
    const bool core = tile_core(it);
    const int base = tile_base(it);
    const int lim = core ? nc_hi : P_hi + 1;
    const int nbytes = max(0, min(kTileRows, lim - base)) * D * 2;
    const long off = (long)base * D;
    const u32x4 rk = buffer_desc((core ? ckbase : kbase) + off, nbytes);
    const u32x4 rv = buffer_desc((core ? cvbase : vbase) + off, nbytes);
    const uint32_t kb = lds_addr(kbuf(kslot)), vb = lds_addr(vbuf(vslot));
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int li = wave + NW * i;
      if (li < NKI) lds_dma16(rk, kb + li * 1024, soff[i]);
      else if (li < NL) lds_dma16(rv, vb + (li - NKI) * 1024, soff[i]);
    }
  };
  auto sync_stage = [&]() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NLMIN) : "memory");
  };

  // LDS addresses: row read of K row 32kb + j (A operand of S^T), of V row;
  // transposing read of K (A operand of dQ^T): lane s of a 16-lane group at
  // row 16cc + 8x + 4hh + s/4, dims 32db + 16((lane/16)%2) + 4(s%4) .. +3
  const int krow_off = KT::row_off(j) + 16 * hh;
  const int vrow_off = j * VRow + 16 * hh;
  const int s16 = lane & 15;
  const int ktr_off = hh * KT::kGroup + (s16 >> 2) * KT::kRow + 2 * (16 * ((lane >> 4) & 1) + 4 * (s16 & 3));

  auto tile_full = [&](int it, bool core) {
    const int base = tile_base(it);
    return core ? base + kTileRows <= wnc_lo : (base >= wlo_hi && base + kTileRows - 1 <= w_lo);
  };

  f32x16 dqt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[db][r] = 0.f;
  const float c = A->c;
  // dQ^T += K^T . dS^T for chunk cc (16 keys) and dim block db of a tile
  // (F16: a core tile)
  auto dq_mfma = [&](const char* kt, int cc, int db, const bf16x8& dsf, auto core_tag) {
    const char* p0 = kt + ktr_off + (4 * cc) * KT::kGroup + 64 * db;
    const bf16x4 x0 = lds_read_tr16(p0);
    const bf16x4 x1 = lds_read_tr16(p0 + 2 * KT::kGroup);
    const bf16x8 a = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    dqt[db] = mfma32<decltype(core_tag)::value>(a, dsf, dqt[db]);
  };

  // prologue: tiles 0 and 1; K slot 3 (read as "tile -1" with dS = 0) cleared
  load_tile(0, 0, 0);
  load_tile(1, 1, 1);
  for (int i = tid; i < KT::kBytes / 16; i += kThreads)
    *reinterpret_cast<u32x4*>(kbuf(3) + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NLMIN) : "memory");
  // dS of the previous tile (zeros before the first), bf16 B operands
  bf16x8 dsb[4];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) dsb[cc][e] = static_cast<__bf16>(0.0f);
  // Iteration it: K(it) in K slot it%4, V(it) in V slot it%3, K(it-1) still in
  // K slot (it-1)%4.  It loads tile it+2 (K slot (it+2)%4, V slot (it+2)%3),
  // computes S^T and dP^T of tile it, then runs the dQ product of tile it-1
  // interleaved with tile it's P and dS (the forward's P.V / exponential
  // interleave): chunk cc of dsb is consumed by the product just before tile
  // it's chunk cc overwrites it.  CUR and PREV say whether tiles it and it-1
  // are core tiles (fp16 operands) or raw tiles (bf16).
  int kslot = 0, vslot = 0;
  // key_lo .. key_hi: the keys of this phase (raw positions, or cores) that
  // this lane's row sees
  auto iteration = [&](int it, auto cur_tag, auto prev_tag, int key_lo, int key_hi) {
    constexpr bool CUR = decltype(cur_tag)::value;
    const int kprev = (kslot + 3) & 3;
    load_tile((kslot + 2) & 3, vslot == 0 ? 2 : vslot - 1, it + 2);
    const char* kt = kbuf(kslot);
    const char* vt = vbuf(vslot);
    const char* kt_prev = kbuf(kprev);
    f32x16 sx[2], dpx[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sx[kb][r] = dpx[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + krow_off + kb * 8 * KT::kGroup + 32 * ks);
        sx[kb] = mfma32<CUR>(a, qf[ks], sx[kb]);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(vt + vrow_off + kb * 32 * VRow + 32 * ks);
        dpx[kb] = mfma32<CUR>(av, gf[ks], dpx[kb]);
      }
    if (!tile_full(it, CUR)) {
      // key kk = 32kb + 8(r/4) + 4hh + r%4 of the tile is visible to this
      // lane's row iff lo_rel <= kk <= hi_rel; hidden keys get P = 0
      asm volatile("" ::: "memory");  // keeps this a real (scalar) branch
      const int base = tile_base(it);
      const int lo_rel = key_lo - base;
      const int hi_rel = key_hi - base;
      const unsigned span = (unsigned)(hi_rel - lo_rel);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool vis = hi_rel >= lo_rel && (unsigned)(kk - lo_rel) <= span;
          sx[kb][r] = vis ? sx[kb][r] : -INFINITY;
        }
    }
    // dQ of tile it-1 interleaved with P = exp2(S c - lse2), dS = P (dP - D)
    // of tile it: after each MFMA come the scores it can hide
    constexpr int NDQ = 4 * DB;     // dQ MFMAs per tile
    constexpr int PPM = 32 / NDQ;   // scores per MFMA slot
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      u32x4 dnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dq_mfma(kt_prev, cc, db, dsb[cc], prev_tag);
#pragma unroll
        for (int e = db * PPM; e < db * PPM + PPM; e += 2) {
          const int r = (cc & 1) * 8 + e;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sx[cc >> 1][r], c, -lse2));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sx[cc >> 1][r + 1], c, -lse2));
          dnew[e >> 1] = pack_op<CUR>(p0 * (dpx[cc >> 1][r] - Dt), p1 * (dpx[cc >> 1][r + 1] - Dt));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      dsb[cc] = __builtin_bit_cast(bf16x8, dnew);
    }
    kslot = (kslot + 1) & 3;
    vslot = vslot == 2 ? 0 : vslot + 1;
    sync_stage();
  };
  // raw tiles on bf16 Q and dO fragments, then the core tiles on fp16 ones
  // (the conversion is one-way: no fp16 value is converted back; the other
  // order's round trip spilled registers inside this kernel's loops)
  {
    const int my_lo = win_lo(t, w);
    for (int it = 0; it < n_rt; ++it) iteration(it, RawTile{}, RawTile{}, my_lo, t);
  }
  if (n_ct > 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // converted again rather than kept from the prologue's stores, which
      // would hold 16 more fragments live through the raw tiles
      asm volatile("" : "+v"(qf[ks]), "+v"(gf[ks]));
      qf[ks] = bf16_frag_to_f16(qf[ks]);
      gf[ks] = bf16_frag_to_f16(gf[ks]);
    }
    const int my_nc = n_core(t, g, w);
    iteration(n_rt, CoreTile{}, RawTile{}, 0, my_nc - 1);
    for (int it = n_rt + 1; it < n_tiles; ++it) iteration(it, CoreTile{}, CoreTile{}, 0, my_nc - 1);
  }
  // dQ of the last tile (K slot (n_tiles-1)%4)
  auto last_tile = [&](auto core_tag) {
    const char* kt_last = kbuf((kslot + 3) & 3);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int db = 0; db < DB; ++db) dq_mfma(kt_last, cc, db, dsb[cc], core_tag);
  };
  if (n_ct > 0) last_tile(CoreTile{});
  else last_tile(RawTile{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane holds dims 32db + 8(r/4) + 4hh + r%4 of row j
  if (t_raw < L) {
    float* out = A->dq + (((long)b * A->Hq + h) * L + t_raw) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hh;
        *reinterpret_cast<float4*>(out + d0) =
            make_float4(dqt[db][4 * q4] * A->scale, dqt[db][4 * q4 + 1] * A->scale,
                        dqt[db][4 * q4 + 2] * A->scale, dqt[db][4 * q4 + 3] * A->scale);
      }
  }
  };

  // ---- blocks below n_static run item blockIdx.x; the others take the tail
  // from the queues.  One loop, so the item code has a single call site.
  const bool queue_wg = (int)blockIdx.x >= P.n_static;
  unsigned* const qs = g_dq_queue + 16 * P.qslot;
  __shared__ int claimed;
  int cq = tail_home_queue(), dead = 0;
  for (;;) {
    int item = (int)blockIdx.x;
    if (queue_wg) {
      if (tid == 0) claimed = tail_claim(qs, cq, dead, P.n_static, P.total - P.n_static);
      __syncthreads();  // also: every wave is done with the previous item's LDS
      item = __builtin_amdgcn_readfirstlane(claimed);
      __syncthreads();  // every wave has read it before it is written again
      if (item < 0) break;
    }
    item_body(item);
    if (!queue_wg) break;
  }
  if (queue_wg && tid == 0) tail_done(qs, gridDim.x - P.n_static);
}

// --------------------------------------------------------------- 2. dK, dV

struct DkvParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  const uint16_t* dout;
  const uint16_t* q16;   // fp16 copies of q and dout (written by the dQ kernel), read by core units
  const uint16_t* do16;
  const float2* stats;
  float* dk;   // raw-key gradients [B,Hkv,L,d]
  float* dv;
  float* dck;  // core gradients [B,Hkv,m,d], accumulated with atomic adds
  float* dcv;
  int B, Hq, Hkv, L, g, w, m, m_cap, G;
  int nCB, nSplit, nRB, UP;  // core blocks, row splits, raw blocks, units per (b, kv head)
  int xcd;
  float c, scale;
  int total;     // units in all
  int n_static;  // units 0 .. n_static-1 go one to a workgroup, in block order
  int qslot;     // work-queue slot of this launch (the raw units after them)
};

// work-queue counters of the dK/dV launches in flight, one 16-word slot each
__device__ unsigned g_dkv_queue[kQueueSlots * 16];

// A workgroup of 8 waves owns 128 keys.  Waves 2p and 2p+1 share keys
// 32p .. 32p+31 and split each 64-row tile: each computes S, dP, P and dS for
// its 32 rows and accumulates dV^T and dK^T over them for all head dims; the
// two partial sums meet once, through LDS, when the unit is done.  The K
// fragments of the wave's keys stay in registers, the V fragments sit in LDS
// (registers for both would take a wave past 256, and one wave per SIMD
// left the compiler shuttling accumulators between register files).
template <int D>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkv_mfma_kernel(DkvParams P) {
  constexpr int NW = 8;
  constexpr int KS = D / 16, DB = D / 32;
  typedef BothWaysTile<D> RT;  // Q and dO tiles: row reads and transposing reads
  // The row statistics of a tile (64 x 8 bytes) sit in the Q tile's unused tail.
  static_assert(RT::kBytes - RT::kBytesUsed >= 512, "room for the row statistics");
  constexpr int QTailLanes = (RT::kBytesUsed - (RT::kLoads - 1) * 1024) / 16;  // live lanes of Q's last load
  constexpr int SlotBytes = 2 * RT::kBytes;
  constexpr int VFBytes = (NW / 2) * KS * 1024;  // per wave pair: V fragments [ks][lane]
  static_assert((NW / 2) * 2 * DB * 4 * 1024 <= 3 * SlotBytes + VFBytes, "partial sums fit in LDS");
  constexpr int NL = 2 * RT::kLoads + 1;
  constexpr int NLW = (NL + NW - 1) / NW, NLMIN = NL / NW;
  __shared__ __attribute__((aligned(16))) char lds[3 * SlotBytes + VFBytes];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int pair = wave >> 1, half = wave & 1;
  const int i32 = lane & 31, hh = lane >> 5;
  const int g = P.g, w = P.w, L = P.L;

  // ---- unit: core units (split-major) first, then raw-key units; the queue
  // workgroups only ever take raw-key units (RAW_ONLY)
  auto item = [&](const long bid, auto raw_only_tag) {
  constexpr bool RAW_ONLY = decltype(raw_only_tag)::value;
  const auto* const A = kernel_args<DkvParams>();
  const int BH = A->B * A->Hkv;
  int kvp, u;
  if (A->xcd) {
    const int hpx = BH / 8;
    const long q = bid >> 3;
    kvp = (int)(bid & 7) * hpx + (int)(q % hpx);
    u = (int)(q / hpx);
  } else {
    kvp = (int)(bid % BH);
    u = (int)(bid / BH);
  }
  const int b = kvp / A->Hkv;
  // core units meet fp16 cores: every product runs on fp16 operands, with Q
  // and dO from their fp16 copies; raw units run on bf16 operands
  auto unit = [&](auto core_tag) {
  constexpr bool core = decltype(core_tag)::value;
  const uint16_t* qsrc = core ? A->q16 : A->q;
  const uint16_t* gsrc = core ? A->do16 : A->dout;
  int key_lo, key_lim, t_lo, t_end;
  if (core) {
    const int split = u / A->nCB, cb = u % A->nCB;
    key_lo = cb * kKeysPerUnit;
    key_lim = A->m;
    t_lo = max((key_lo + 1) * g + w - 1, split * kCoreSplit);
    t_end = min(L, (split + 1) * kCoreSplit) - 1;
  } else {
    const int rb = u - A->nCB * A->nSplit;
    key_lo = rb * kKeysPerUnit;
    key_lim = L;
    t_lo = key_lo;
    t_end = min(L - 1, key_lo + kKeysPerUnit - 1 + w - 1);
  }
  t_lo = uni(t_lo);
  t_end = uni(t_end);
  if (t_lo > t_end) return;  // nothing sees these keys in this split
  const int n_rt = (t_end - t_lo) / kTileRows + 1;
  const int n_it = A->G * n_rt;

  // ---- this pair's keys k0 .. k0+31 and this lane's key
  const int k0 = key_lo + 32 * pair;
  const int key = k0 + i32;
  const bool key_ok = key < key_lim;
  // rows that see this lane's key: [lo, hi] (empty when hi < lo)
  int lo, hi;
  if (core) {
    lo = (key + 1) * g + w - 1;
    hi = key_ok ? t_end : lo - 1;
  } else {
    lo = key;
    hi = key_ok ? min(key + w - 1, t_end) : lo - 1;
  }
  const bool wave_keys_ok = k0 + 31 < key_lim;
  const int lo_max = core ? (k0 + 32) * g + w - 1 : k0 + 31;
  const int hi_min = core ? t_end : min(k0 + w - 1, t_end);

  const long kvrow = (long)kvp;
  const uint16_t* kb_ = core ? A->ck + kvrow * A->m_cap * D : A->k + kvrow * L * D;
  const uint16_t* vb_ = core ? A->cv + kvrow * A->m_cap * D : A->v + kvrow * L * D;
  char* vfrag = lds + 3 * SlotBytes + pair * KS * 1024 + 16 * lane;  // V fragment ks at + 1024 ks
  bf16x8 kf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8 vx;
    if (key_ok) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(kb_ + (long)key * D + 16 * ks + 8 * hh);
      vx = *reinterpret_cast<const bf16x8*>(vb_ + (long)key * D + 16 * ks + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) kf[ks][e] = vx[e] = static_cast<__bf16>(0.0f);
    }
    if (half == 0) *reinterpret_cast<bf16x8*>(vfrag + 1024 * ks) = vx;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(kf[ks]));

  // ---- tile loaders: load index li < RT::kLoads fills Q, then dO, then the statistics
  int soff[NLW];
#pragma unroll
  for (int i = 0; i < NLW; ++i) {
    const int li = wave + NW * i;
    if (li < RT::kLoads) soff[i] = RT::src_offset(li * 64 + lane);
    else if (li < 2 * RT::kLoads) soff[i] = RT::src_offset((li - RT::kLoads) * 64 + lane);
    else soff[i] = 16 * lane;
  }
  auto qbuf = [&](int s) { return lds + s * SlotBytes; };
  auto gbuf = [&](int s) { return lds + s * SlotBytes + RT::kBytes; };
  auto sbuf = [&](int s) { return lds + s * SlotBytes + RT::kBytesUsed; };
  auto load_tile = [&](int slot, int it) {
    const int hg = it / n_rt, tile = it % n_rt;
    const int t0 = t_lo + tile * kTileRows;
    const int nr = it < n_it ? max(0, min(kTileRows, t_end + 1 - t0)) : 0;
    const long row = ((long)b * A->Hq + (long)(kvp % A->Hkv) * A->G + hg) * L + t0;
    const u32x4 rq = buffer_desc(qsrc + row * D, nr * D * 2);
    const u32x4 rg = buffer_desc(gsrc + row * D, nr * D * 2);
    const u32x4 rs = buffer_desc(A->stats + row, nr * 8);
    const uint32_t qa = lds_addr(qbuf(slot)), ga = lds_addr(gbuf(slot)), sa = lds_addr(sbuf(slot));
    // load li = wave + NW i: which array it fills is uniform (a scalar select).
    // Q's last load leaves the tail (the statistics' place) alone; the
    // statistics load writes 512 bytes.
#pragma unroll
    for (int i = 0; i < NLW; ++i) {
      const int li = wave + NW * i;
      if (NW * i + NW <= RT::kLoads - 1) {
        lds_dma16(rq, qa + li * 1024, soff[i]);
      } else if (NW * i >= RT::kLoads && NW * i + NW <= 2 * RT::kLoads) {
        lds_dma16(rg, ga + (li - RT::kLoads) * 1024, soff[i]);
      } else if (li < NL) {
        const bool isq = li < RT::kLoads, isg = li < 2 * RT::kLoads;
        const u32x4 r = isq ? rq : (isg ? rg : rs);
        const uint32_t dst = isq ? qa + li * 1024 : (isg ? ga + (li - RT::kLoads) * 1024 : sa);
        const int live = li == RT::kLoads - 1 ? QTailLanes : (isg ? 64 : 32);
        if (lane < live) lds_dma16(r, dst, soff[i]);
      }
    }
  };
  auto sync_stage = [&]() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NLMIN) : "memory");
  };

  // LDS addresses: row read of Q / dO row 32 half + i32 (A operand of S, dP);
  // transposing read (A operand of dV^T, dK^T): lane s of a 16-lane group at
  // row 16cc + 8x + 4hh + s/4, dims 32db + 16((lane/16)%2) + 4(s%4) .. +3
  const int rrow_off = RT::row_off(32 * half + i32) + 16 * hh;
  const int s16 = lane & 15;
  const int rtr_off = hh * RT::kGroup + (s16 >> 2) * RT::kRow + 2 * (16 * ((lane >> 4) & 1) + 4 * (s16 & 3));

  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkt[db][r] = dvt[db][r] = 0.f;
  const float c = A->c;

  load_tile(0, 0);
  load_tile(1, 1);
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NLMIN) : "memory");
  int slot = 0;
  int tile = 0;  // it % n_rt
  for (int it = 0; it < n_it; ++it) {
    const int nslot = slot == 0 ? 2 : slot - 1;
    load_tile(nslot, it + 2);
    const int t0 = t_lo + tile * kTileRows;
    const int tw = t0 + 32 * half;  // first row of this wave's half
    const char* qt = qbuf(slot);
    const char* gt = gbuf(slot);
    const char* sta = sbuf(slot);
    // S, dP over this wave's 32 rows; register r is row tw + 8(r/4) + 4hh + r%4
    f32x16 sx, dpx;
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[r] = dpx[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qt + rrow_off + 32 * ks);
      sx = mfma32<core>(a, kf[ks], sx);
      const bf16x8 ag = *reinterpret_cast<const bf16x8*>(gt + rrow_off + 32 * ks);
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(vfrag + 1024 * ks);
      dpx = mfma32<core>(ag, vf, dpx);
    }
    // P and dS (fragments of k-steps 2 half and 2 half + 1, in the unit's
    // operand type)
    const bool full = wave_keys_ok && tw >= lo_max && tw + 31 <= hi_min;
    u32x4 pw[2], dsw[2];
    auto probs = [&](auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const unsigned span = (unsigned)(hi - lo);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int rr = 32 * half + 8 * q4 + 4 * hh;  // tile row of this lane's first of 4
        const float4 s01 = *reinterpret_cast<const float4*>(sta + rr * 8);
        const float4 s23 = *reinterpret_cast<const float4*>(sta + rr * 8 + 16);
        const float l2[4] = {s01.x, s01.z, s23.x, s23.z};
        const float dd[4] = {s01.y, s01.w, s23.y, s23.w};
        float p[4], ds[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * q4 + x;
          p[x] = __builtin_amdgcn_exp2f(fmaf(sx[r], c, -l2[x]));
          if (MASK) {
            const bool vis = hi >= lo && (unsigned)(t0 + rr + x - lo) <= span;
            p[x] = vis ? p[x] : 0.f;
          }
          ds[x] = p[x] * (dpx[r] - dd[x]);
        }
#pragma unroll
        for (int x = 0; x < 4; x += 2) {
          pw[q4 >> 1][2 * (q4 & 1) + x / 2] = pack_op<core>(p[x], p[x + 1]);
          dsw[q4 >> 1][2 * (q4 & 1) + x / 2] = pack_op<core>(ds[x], ds[x + 1]);
        }
      }
    };
    if (full) probs(std::false_type{});
    else probs(std::true_type{});
    // dV^T += dO^T . P and dK^T += Q^T . dS over this wave's 32 rows, all dims
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int cc = 2 * half + h2;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int o = rtr_off + (4 * cc) * RT::kGroup + 64 * db;
        const bf16x4 g0 = lds_read_tr16(gt + o), g1 = lds_read_tr16(gt + o + 2 * RT::kGroup);
        const bf16x8 ag = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
        dvt[db] = mfma32<core>(ag, __builtin_bit_cast(bf16x8, pw[h2]), dvt[db]);
        const bf16x4 q0 = lds_read_tr16(qt + o), q1 = lds_read_tr16(qt + o + 2 * RT::kGroup);
        const bf16x8 aq = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
        dkt[db] = mfma32<core>(aq, __builtin_bit_cast(bf16x8, dsw[h2]), dkt[db]);
      }
    }
    slot = slot == 2 ? 0 : slot + 1;
    tile = tile + 1 == n_rt ? 0 : tile + 1;
    sync_stage();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // the pair's two partial sums meet in LDS (the ring is idle now): the
  // second wave writes its accumulators, the first adds them and stores
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  float4* part = reinterpret_cast<float4*>(lds) + (size_t)pair * (2 * DB * 4 * 64) + lane;
  if (half == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        part[((0 * DB + db) * 4 + q4) * 64] = make_float4(dkt[db][4 * q4], dkt[db][4 * q4 + 1], dkt[db][4 * q4 + 2], dkt[db][4 * q4 + 3]);
        part[((1 * DB + db) * 4 + q4) * 64] = make_float4(dvt[db][4 * q4], dvt[db][4 * q4 + 1], dvt[db][4 * q4 + 2], dvt[db][4 * q4 + 3]);
      }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (half == 1 || !key_ok) return;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 a = part[((0 * DB + db) * 4 + q4) * 64];
      const float4 v = part[((1 * DB + db) * 4 + q4) * 64];
      dkt[db][4 * q4] += a.x;
      dkt[db][4 * q4 + 1] += a.y;
      dkt[db][4 * q4 + 2] += a.z;
      dkt[db][4 * q4 + 3] += a.w;
      dvt[db][4 * q4] += v.x;
      dvt[db][4 * q4 + 1] += v.y;
      dvt[db][4 * q4 + 2] += v.z;
      dvt[db][4 * q4 + 3] += v.w;
    }

  // lane holds dims 32db + 8(r/4) + 4hh + r%4 of its key
  if constexpr (!core) {
    const long orow = ((long)kvp * L + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * hh;
        *reinterpret_cast<float4*>(A->dk + orow + d0) =
            make_float4(dkt[db][4 * q4] * A->scale, dkt[db][4 * q4 + 1] * A->scale,
                        dkt[db][4 * q4 + 2] * A->scale, dkt[db][4 * q4 + 3] * A->scale);
        *reinterpret_cast<float4*>(A->dv + orow + d0) =
            make_float4(dvt[db][4 * q4], dvt[db][4 * q4 + 1], dvt[db][4 * q4 + 2], dvt[db][4 * q4 + 3]);
      }
  } else {
    const long orow = ((long)kvp * A->m + key) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
        atomicAdd(A->dck + orow + d, dkt[db][r] * A->scale);
        atomicAdd(A->dcv + orow + d, dvt[db][r]);
      }
  }
  };
  if constexpr (RAW_ONLY) {
    unit(RawTile{});
  } else {
    if (u < A->nCB * A->nSplit) unit(CoreTile{});
    else unit(RawTile{});
  }
  };

  // ---- blocks below n_static run unit blockIdx.x; the others take the tail
  if ((int)blockIdx.x < P.n_static) {
    item(blockIdx.x, std::false_type{});
    return;
  }
  unsigned* const qslot = g_dkv_queue + 16 * P.qslot;
  __shared__ int claimed;
  int cq = tail_home_queue(), dead = 0;
  for (;;) {
    if (tid == 0) claimed = tail_claim(qslot, cq, dead, P.n_static, P.total - P.n_static);
    __syncthreads();  // also: every wave is done with the previous unit's LDS
    const int next = __builtin_amdgcn_readfirstlane(claimed);
    __syncthreads();  // every wave has read it before it is written again
    if (next < 0) break;
    item(next, std::true_type{});
  }
  if (tid == 0) tail_done(qslot, gridDim.x - P.n_static);
}

constexpr int kDqWaves = 8;

int gcd_int(int a, int b) {
  while (b) {
    const int t = a % b;
    a = b;
    b = t;
  }
  return a;
}

template <int D>
hipError_t launch_t(const void* q, const void* k, const void* v, const void* ck, const void* cv,
                    int m_cap, const void* out, const float* lse, const void* dout, float* dq,
                    float* dk, float* dv, float2* stats, float* dck, float* dcv, uint16_t* q16,
                    uint16_t* do16, const Shape& sh, hipStream_t s) {
  const int B = sh.B, Hq = sh.Hq, Hkv = sh.Hkv, L = sh.L, g = sh.g, w = sh.w;
  const int m = L / g;
  const float scale = 1.0f / sqrtf((float)D), c = kLog2e * scale;

  DqParams Q;
  Q.q = static_cast<const uint16_t*>(q);
  Q.k = static_cast<const uint16_t*>(k);
  Q.v = static_cast<const uint16_t*>(v);
  Q.ck = static_cast<const uint16_t*>(ck);
  Q.cv = static_cast<const uint16_t*>(cv);
  Q.dout = static_cast<const uint16_t*>(dout);
  Q.out = static_cast<const uint16_t*>(out);
  Q.lse = lse;
  Q.stats = stats;
  Q.q16 = q16;
  Q.do16 = do16;
  Q.dq = dq;
  Q.B = B;
  Q.Hq = Hq;
  Q.Hkv = Hkv;
  Q.L = L;
  Q.g = g;
  Q.w = w;
  Q.m_cap = m_cap;
  Q.G = sh.G();
  Q.Hw = gcd_int(Q.G, kDqWaves);
  Q.RP = 32 * (kDqWaves / Q.Hw);
  Q.nPB = (L + Q.RP - 1) / Q.RP;
  Q.nHG = Q.G / Q.Hw;
  Q.U = B * Hkv * Q.nHG;
  Q.xcd = (Q.U % 8 == 0) ? 1 : 0;
  Q.c = c;
  Q.scale = scale;
  const long qblocks = (long)Q.nPB * Q.U;
  if (qblocks > 0x7fffffffL / 2) return hipErrorInvalidConfiguration;
  int cus = 0;
  const hipError_t ce = compute_units(&cus);
  if (ce != hipSuccess) return ce;
  const int q_tail = tail_items(qblocks, cus);
  Q.total = (int)qblocks;
  Q.n_static = Q.total - q_tail;
  static std::atomic<unsigned> dq_launches{0};
  Q.qslot = (int)(dq_launches.fetch_add(1, std::memory_order_relaxed) % kQueueSlots);
  const long dq_grid = (long)Q.n_static + std::min(q_tail, cus);
  hipLaunchKernelGGL((dq_mfma_kernel<D>), dim3((unsigned)dq_grid), dim3(64 * kDqWaves), 0, s, Q);

  DkvParams K;
  K.q = Q.q;
  K.k = Q.k;
  K.v = Q.v;
  K.ck = Q.ck;
  K.cv = Q.cv;
  K.dout = Q.dout;
  K.q16 = q16;
  K.do16 = do16;
  K.stats = stats;
  K.dk = dk;
  K.dv = dv;
  K.dck = dck;
  K.dcv = dcv;
  K.B = B;
  K.Hq = Hq;
  K.Hkv = Hkv;
  K.L = L;
  K.g = g;
  K.w = w;
  K.m = m;
  K.m_cap = m_cap;
  K.G = sh.G();
  K.nCB = (m + kKeysPerUnit - 1) / kKeysPerUnit;
  K.nSplit = (L + kCoreSplit - 1) / kCoreSplit;
  K.nRB = (L + kKeysPerUnit - 1) / kKeysPerUnit;
  K.UP = K.nCB * K.nSplit + K.nRB;
  K.xcd = ((B * Hkv) % 8 == 0) ? 1 : 0;
  K.c = c;
  K.scale = scale;
  const long kblocks = (long)K.UP * B * Hkv;
  if (kblocks > 0x7fffffffL / 2) return hipErrorInvalidConfiguration;
  // the raw-key units come last in block order: the queues take the last of
  // them (never a core unit)
  const long raw_units = (long)K.nRB * B * Hkv;
  const int n_tail = (int)std::min<long>(tail_items(kblocks, cus), raw_units & ~7L);
  K.total = (int)kblocks;
  K.n_static = K.total - n_tail;
  static std::atomic<unsigned> launches{0};
  K.qslot = (int)(launches.fetch_add(1, std::memory_order_relaxed) % kQueueSlots);
  const long dkv_grid = (long)K.n_static + std::min(n_tail, cus);
  hipLaunchKernelGGL((dkv_mfma_kernel<D>), dim3((unsigned)dkv_grid), dim3(512), 0, s, K);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_mfma(const void* q, const void* k, const void* v, const void* ck,
                                const void* cv, int m_cap, const void* out, const float* lse,
                                const void* dout, float* dq, float* dk, float* dv, float2* stats,
                                float* dck, float* dcv, uint16_t* q16, uint16_t* do16,
                                const Shape& sh, hipStream_t s) {
  if (sh.d == 64)
    return launch_t<64>(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv, stats, dck, dcv, q16, do16, sh, s);
  return launch_t<128>(q, k, v, ck, cv, m_cap, out, lse, dout, dq, dk, dv, stats, dck, dcv, q16, do16, sh, s);
}

}  // namespace cca
