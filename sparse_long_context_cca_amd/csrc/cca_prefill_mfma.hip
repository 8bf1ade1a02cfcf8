// Fused CCA prefill on the gfx950 matrix cores (bf16 raw and fp16 core operands, fp32 accumulate).
//
// Row t of head h computes one softmax over [cores 0..n_core(t) ; raw keys
// win_lo(t)..t] (digest at digest.lyk-ai.com/posts/2412.12465, "Method",
// fusion formula; paper card at atlas.scime.ai, "Approach": both contexts are
// fused in a single softmax).
//
// Work decomposition
//   * A workgroup (8 waves) owns 256 query rows that share one kv head: Hw
//     query heads x (256/Hw) consecutive positions, Hw = gcd(G, 8).  Each wave
//     owns 32 rows (one head, 32 consecutive positions).  With GQA several
//     waves are query heads at the same positions, and every K/V tile staged
//     in LDS serves all eight waves.
//   * The workgroup walks the union of its rows' visible keys: first the raw
//     tiles covering win_lo(first row)..last row (64 positions each,
//     64-aligned), then the core tiles 0..n_core(last row) (64 cores each).
//     Tiles that every row of a wave sees completely skip the mask; tiles no
//     row of a wave sees are fully masked.
//   * Raw tiles run on bf16 MFMAs (the inputs' dtype).  The cores are stored
//     in fp16 (three more mantissa bits than bf16: a core is a weighted mean
//     of keys that can be large), so core tiles run on fp16 MFMAs: when the
//     walk reaches them, each wave converts its Q fragments to fp16 once, in
//     registers, and the probabilities of core tiles are rounded to fp16.
//   * Workgroups are issued longest-first (the last positions see the most
//     cores) and, when the kv heads divide evenly over the 8 XCDs, all
//     workgroups of one kv head run on one XCD so that its core K/V stay in
//     that XCD's L2.  An XCD that holds several kv heads runs them one after
//     another (each longest-first), so the cores being read at any time are
//     those of one head.
// Per 64-key tile and wave
//   S^T (64 keys x 32 rows) = K_tile . Q^T with v_mfma_f32_32x32x16_{bf16,f16}
//   (A = K rows from LDS, B = the wave's Q fragments, held in registers);
//   each lane then holds 32 scores of one query row, so the row max needs one
//   exchange with lane l^32.  The row sum of the rounded probabilities is
//   taken on the matrix cores too: one 16x16x32 MFMA per P chunk whose A
//   operand selects, for output rows 0 and 1, the lanes that hold query rows
//   0..15 and 16..31 (the sum does not depend on the key order).
//   P (bf16 or fp16) is used in place as the B operand of O^T += V^T . P^T; the V^T
//   operand comes from a row-major V tile through transposing LDS reads that
//   follow the key order of the score layout.  The P.V product of tile i-1
//   is interleaved with the exponentials of tile i, so the matrix cores work
//   while the vector ALUs compute the softmax.
// Online softmax in the log2 domain with fp32 state and a lazy rescale.  K
// and V tiles are loaded straight from memory into three-slot LDS rings, two
// tiles ahead (buffer loads whose range check zero-fills keys past the end).
#include <algorithm>
#include <atomic>
#include <mutex>

#include "cca_device.hpp"
#include "cca_internal.hpp"
#include "cca_lds.hpp"
#include "cca_queue.hpp"

namespace cca {
namespace {

constexpr int kBK = 64;       // keys per tile
constexpr float kLazyLog2 = 8.0f;  // rescale threshold of the running max, log2 units

struct PrefillParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* ck;
  const uint16_t* cv;
  void* out;
  float* lse;  // null, or the natural-log log-sum-exp of each row's scores [B,Hq,Lq]
  const int32_t* q_start;  // per-sequence query rows (RowRange); null: every row
  const int32_t* q_len;
  int B, Hq, Hkv, Lq, Lk, g, w, m_cap;
  int G, Hw, RP;        // heads per workgroup, rows per head per workgroup
  int nPB, nHG, U;      // position blocks, head groups per kv head, units
  int xcd;              // 1 when units split evenly over 8 XCDs
  int total;            // items (a workgroup's worth of rows each): nPB * U
  int n_static;         // items 0 .. n_static-1 go one to a workgroup, in block order
  int qslot;            // work-queue slot of this launch (for the items after them)
  float c;              // softmax scale * log2(e)
};

// the tail queues' counters (cca_queue.hpp)
__device__ unsigned g_prefill_queue[kQueueSlots * 16];

// Lanes l and l^32 hold the two halves of one query row's scores.  One
// v_permlane32_swap of a register with itself leaves {x[l], x[l^32]} in the
// two results (in an order that differs between the lane halves), so the
// pair max below is symmetric in them.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Two waves per SIMD (the accumulators stay in arch VGPRs, 256 per wave) so
// that one wave's softmax overlaps the other's matrix ops.  OFF > 0 (a
// workgroup of one head's 256 consecutive rows): the second half of the waves
// walks the raw window up to OFF tiles ahead of the first half, so that each
// half steps only through the window it needs (about 18 tiles at w = 1024)
// instead of the union of all rows' windows (20).
template <int D, int OT, int NW, int OFF>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_mfma_kernel(PrefillParams P) {
  constexpr int kThreads = 64 * NW;
  constexpr int KS = D / 16;            // k-steps of Q.K^T
  constexpr int DB = D / 32;            // 32-wide dim blocks of the output
  constexpr int CPR = D / 8;            // 16-byte chunks per K row
  constexpr int KRow = D * 2 + 16;      // bytes per K row in LDS (one chunk of padding)
  constexpr int KBytes = kBK * KRow;
  constexpr int NKI = KBytes / 1024;    // 1 KB wave loads per K tile
  static_assert(KBytes % 1024 == 0, "K tile is a whole number of wave loads");
  constexpr int NKW = (NKI + NW - 1) / NW;  // K wave loads per wave (at most)
  constexpr int NKMIN = NKI / NW;           // ... issued by every wave
  constexpr int VBytes = kBK * D * 2;   // V tile: row-major, 64-byte blocks swizzled
  constexpr int NVI = VBytes / 1024;    // 1 KB wave loads per V tile
  static_assert(NVI % NW == 0, "V wave loads split evenly over the waves");
  constexpr int NVW = NVI / NW;
  // LDS: rings of K and V tiles, K(q) in slot q % NSK and V(q) in q % NSV
  // for tile q of the walk.  OFF = 0: three K slots (K loaded two tiles
  // ahead) and three V slots (V one tile ahead of its scores).  OFF > 0: the
  // leading half may be OFF tiles ahead, so OFF + 3 K slots, and OFF + 2 V
  // slots with V loaded in the stage that computes the leading half's scores
  // of its tile.
  constexpr int NSK = OFF + 3;
  constexpr int NSV = OFF == 0 ? 3 : OFF + 2;
  __shared__ __attribute__((aligned(16))) char lds[NSK * KBytes + NSV * VBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave index as a scalar, so that every per-wave quantity below (rows,
  // tile visibility) is known to be uniform and branches on it stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31;
  const int hh = lane >> 5;

  // One item: the rows of one workgroup, start to end (the LDS rings are
  // idle again when it returns).
  auto item_body = [&](const long bid) {
  const auto* const A = kernel_args<PrefillParams>();
  // ---- which rows: longest first, XCD-aware.  Item ids are dealt round
  // robin over the XCDs; on XCD x the slots walk unit x*per's position blocks
  // from the last down, then unit x*per+1's, and so on.
  int pb, u;
  if (A->xcd) {
    const int per = A->U / 8;
    const long slot = bid >> 3;
    const int x = (int)(bid & 7);
    pb = A->nPB - 1 - (int)(slot % A->nPB);
    u = x * per + (int)(slot / A->nPB);
  } else {
    pb = A->nPB - 1 - (int)(bid / A->U);
    u = (int)(bid % A->U);
  }
  const int kvp = u / A->nHG;  // b * Hkv + kv head
  const int hg = u % A->nHG;
  const int b = kvp / A->Hkv;
  const int kvh = kvp % A->Hkv;
  const int g = A->g, w = A->w;
  const int h = kvh * A->G + hg * A->Hw + (wave % A->Hw);
  const int row0 = pb * A->RP + 32 * (wave / A->Hw);  // local row of the wave's first row
  // sequence b's rows: positions qs .. qs + ql - 1 at local rows 0 .. ql - 1
  const SeqRows sr = seq_rows(A->q_start, A->q_len, b, A->Lq, A->Lk, g, w, A->m_cap);
  if (!sr.ok) {  // rows that do not fit the buffers: NaN, nothing read
    if (row0 + j < A->Lq) {
      const long orow = (((long)b * A->Hq + h) * A->Lq + row0 + j) * D;
#pragma unroll 1
      for (int e = hh; e < D; e += 2) {
        if (OT == 1) static_cast<uint16_t*>(A->out)[orow + e] = 0x7fc0;
        else static_cast<float*>(A->out)[orow + e] = NAN;
      }
    }
    return;
  }
  const int qs = sr.qs, Le = sr.qs + sr.ql;  // first position, one past the last
  if (pb * A->RP >= sr.ql) return;             // the whole workgroup lies past the end
  const int P_lo = qs + pb * A->RP;
  const int P_hi = min(Le - 1, P_lo + A->RP - 1);
  const int p0 = qs + row0;

  // ---- this lane's query row and the wave's row range
  const int t_raw = p0 + j;
  const int t = min(t_raw, Le - 1);
  const int my_nc = n_core(t, g, w);
  const int my_lo = win_lo(t, w);
  // Per-wave and per-workgroup bounds are uniform; readfirstlane keeps them in
  // scalar registers (the integer divisions inside n_core run on the vector
  // ALUs), so that the tile branches below stay scalar branches.
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  const int w_lo = uni(min(p0, Le - 1));
  const int w_hi = uni(min(p0 + 31, Le - 1));
  const int wnc_lo = uni(n_core(w_lo, g, w));
  const int wlo_hi = uni(win_lo(w_hi, w));

  // ---- workgroup key range: raw tiles 0 .. n_rt-1, then core tiles
  const int nc_hi = uni(n_core(P_hi, g, w));
  const int n_ct = uni((nc_hi + kBK - 1) / kBK);
  const int raw_lo = win_lo(P_lo, w);
  const int r0 = raw_lo & ~(kBK - 1);
  const int n_rt = uni((P_hi - r0) / kBK + 1);
  const int n_tiles = uni(n_ct + n_rt);
  // ---- the halves (OFF > 0): waves 0 .. NW/2-1 hold rows P_lo .. mid-1 and
  // need raw tiles 0 .. a_last; the leading half (the other waves) needs raw
  // tiles from b_first on and walks them off_b tiles ahead, so the raw walk
  // takes n_rt - off_b steps (off_b <= b_first keeps every tile the leading
  // half needs in its walk, off_b <= n_rt-1-a_last every tile of the other).
  // Both halves then walk the same core tiles, tile s + off_b at step s.
  int off_b = 0;
  if constexpr (OFF > 0) {
    const int mid = P_lo + A->RP / 2;
    const int a_last = (min(mid - 1, Le - 1) - r0) / kBK;
    const int b_first = (win_lo(min(mid, Le - 1), w) - r0) / kBK;
    off_b = uni(max(0, min(min(OFF, b_first), n_rt - 1 - a_last)));
  }
  const int lead_off = (OFF > 0 && wave >= NW / 2) ? off_b : 0;
  const int n_raw_steps = n_rt - off_b;

  const long kvrow = (long)kvp;
  const uint16_t* kbase = A->k + kvrow * A->Lk * D;
  const uint16_t* vbase = A->v + kvrow * A->Lk * D;
  const uint16_t* ckbase = A->ck + kvrow * A->m_cap * D;
  const uint16_t* cvbase = A->cv + kvrow * A->m_cap * D;

  // ---- Q fragment: B operand, lane holds Q[row j][16ks + 8hh .. +7]
  bf16x8 qf[KS];
  {
    const uint16_t* qrow = A->q + (((long)b * A->Hq + h) * A->Lq + (t - qs)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hh);
    // Use the fragments here, so that the compiler waits for these loads now:
    // a wait placed at their first use inside the loop would also wait for the
    // tile loads in flight there.
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qf[ks]));
  }

  // ---- tile loaders: buffer loads straight into LDS
  // The resource of each tile starts at the tile's first key and spans only
  // its valid keys, so rows past the end (beyond the last visible core, or
  // past the last row of the workgroup) read as zero.  A wave load writes lane
  // i's 16 bytes at base + 16 i, so the LDS layout is chosen by which chunk of
  // the tile each lane fetches:
  //   K: rows of D*2 bytes plus one 16-byte chunk of padding (the lanes that
  //      land on it get an offset past the range and write zeros);
  //   V: unpadded rows whose 64-byte blocks (32 dims) are XOR-swizzled by
  //      vswz(row), so that the transposing reads below hit distinct banks.
  auto vswz = [](int row) { return D == 128 ? (row & 3) : ((row >> 1) & 1); };
  int koff[NKW], voff[NVW];
#pragma unroll
  for (int i = 0; i < NKW; ++i) {
    const int slot = (wave + NW * i) * 64 + lane;  // 16-byte slot of the LDS tile
    const int row = slot / (CPR + 1), chunk = slot % (CPR + 1);
    koff[i] = chunk < CPR ? (row * D + 8 * chunk) * 2 : 0x40000000;
  }
#pragma unroll
  for (int i = 0; i < NVW; ++i) {
    const int slot = (wave + NW * i) * 64 + lane;
    const int row = slot / CPR, pos = (slot % CPR) >> 2, sub = slot & 3;
    voff[i] = row * D * 2 + ((pos ^ vswz(row)) * 4 + sub) * 16;
  }

  auto tile_core = [&](int it) { return it >= n_rt; };
  auto tile_base = [&](int it) { return it >= n_rt ? (it - n_rt) * kBK : r0 + it * kBK; };
  auto rsrc = [&](int it, bool values) {
    const bool core = tile_core(it);
    const int base = tile_base(it);
    const int lim = core ? nc_hi : P_hi + 1;  // keys < lim are valid
    const int nbytes = max(0, min(kBK, lim - base)) * D * 2;  // 0 past the last tile
    const uint16_t* src = (core ? (values ? cvbase : ckbase) : (values ? vbase : kbase)) + (long)base * D;
    return buffer_desc(src, nbytes);
  };
  // LDS: [K ring slots 0 .. NSK-1 | V ring slots 0 .. NSV-1]
  auto kbuf = [&](int i) { return lds + i * KBytes; };
  auto vbuf = [&](int i) { return lds + NSK * KBytes + i * VBytes; };
  auto load_k = [&](int slot, int it) {  // K(it) -> K ring slot (wave-uniform)
    const u32x4 r = rsrc(it, false);
    const uint32_t base = lds_addr(kbuf(slot));
#pragma unroll
    for (int i = 0; i < NKMIN; ++i) lds_dma16(r, base + (wave + NW * i) * 1024, koff[i]);
    if (NKW > NKMIN && wave < NKI - NW * NKMIN) lds_dma16(r, base + (wave + NW * NKMIN) * 1024, koff[NKW - 1]);
  };
  auto load_v = [&](int slot, int it) {  // V(it) -> V ring slot
    const u32x4 r = rsrc(it, true);
    const uint32_t base = lds_addr(vbuf(slot));
#pragma unroll
    for (int i = 0; i < NVW; ++i) lds_dma16(r, base + (wave + NW * i) * 1024, voff[i]);
  };
  // V^T fragment for P.V MFMA (k-step cc, dim block db): lane (i, hh) needs
  // V[key][dim 32 db + i] for the 8 keys 16cc + 8(e/4) + 4hh + e%4 (the key
  // order of the score layout), i.e. two runs of 4 consecutive keys.  Each
  // run is one transposing read in which lane s of a 16-lane group points at
  // row 16cc + 8x + 4hh + s/4, dims 32db + 16((lane/16)%2) + 4(s%4) .. +3.
  const int vs = lane & 15;
  int vaddr[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    vaddr[db] = (4 * hh + (vs >> 2)) * D * 2 + ((db ^ vswz(vs >> 2)) * 32 + 16 * ((lane >> 4) & 1) + 4 * (vs & 3)) * 2;
  auto vfrag_at = [&](const char* vt, int cc, int db) {
    const bf16x4 x0 = lds_read_tr16(vt + vaddr[db] + (16 * cc) * D * 2);
    const bf16x4 x1 = lds_read_tr16(vt + vaddr[db] + (16 * cc + 8) * D * 2);
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
  };
  // Does tile it need a mask for this wave's rows?  (wave-uniform)  A tile
  // none of the wave's rows can see is simply fully masked.
  auto tile_full = [&](int it, bool core) {
    const int base = tile_base(it);
    return core ? base + kBK <= wnc_lo : (base >= wlo_hi && base + kBK - 1 <= w_lo);
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m = -INFINITY;
  // Row sums: a 16x16x32 MFMA reads its B operand as B[k = 8(l/16) + e][l%16]
  // for lane l, so with A[0][k] = 1 on k in [0,8) u [16,24) (lanes 0 and 32
  // of the A operand) and A[1][k] = 1 on [8,16) u [24,32) (lanes 17 and 49),
  // C[0][c] adds lanes c and c+32 of a P chunk (query row c) and C[1][c] lanes
  // c+16 and c+48 (query row c+16).  Lane c < 16 holds C[0][c] and C[1][c]
  // in lsum[0] and lsum[1]; the other rows of C stay zero.
  f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  // The selector holds ones in the operand type of the probabilities it sums:
  // bf16 through the raw tiles, fp16 through the core tiles.
  const bool sel_on = lane == 0 || lane == 32 || lane == 17 || lane == 49;
  auto selector = [&](auto core_tag) {
    bf16x8 s;
    if constexpr (decltype(core_tag)::value) {
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(sel_on ? 1.0f : 0.0f);
      s = __builtin_bit_cast(bf16x8, h);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = static_cast<__bf16>(sel_on ? 1.0f : 0.0f);
    }
    return s;
  };
  bf16x8 sel = selector(RawTile{});
  // rescale the row sums by their rows' factors (lane c < 16 needs those of
  // rows c and c+16, held by lanes c and c+16)
  auto rescale_sums = [&](float a) {
    const float a_hi = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & 15) + 16) * 4, __float_as_int(a)));
    lsum[0] *= a;
    lsum[1] *= a_hi;
  };
  const float c = A->c;

  // End of a pipeline stage: this wave's loads of the previous stage (K(it+1),
  // V(it)) have landed in LDS, then the workgroup meets.  Loads finish in
  // issue order, so allowing this stage's loads (K(it+2): at least NKMIN wave
  // loads; V(it+1): NVW) to stay in flight is enough.  OFF > 0: a stage
  // issues its V tile before its K tile, and the V tile must land in it.
  constexpr int kInFlight = OFF == 0 ? NKMIN + NVW : NKMIN;
  auto sync_stage = [&]() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kInFlight) : "memory");
  };

  // prologue: K(0), K(1) into K slots 0, 1 and V(0) into V slot 0; V slot 2
  // (read as "tile -1", with zero probabilities) cleared so it holds no NaN
  // OFF > 0: K(0 .. off_b) and V(0 .. off_b-1) land before the walk and
  // K(off_b+1) in its first stage; V slot NSV-1 is tile -1's.
  if constexpr (OFF == 0) {
    load_k(0, 0);
    load_k(1, 1);
    load_v(0, 0);
  } else {
#pragma unroll 1
    for (int x = 0; x <= off_b; ++x) load_k(x, x);
#pragma unroll 1
    for (int x = 0; x < off_b; ++x) load_v(x, x);
    load_k(off_b + 1, off_b + 1);
  }
  for (int i = tid; i < VBytes / 16; i += kThreads)
    *reinterpret_cast<u32x4*>(vbuf(NSV - 1) + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(OFF == 0 ? NKMIN + NVW : NKMIN) : "memory");
  // probabilities of the previous tile, the B operands of its P.V: bf16 for
  // a raw tile (pr), fp16 for a core tile (prh); each walk starts them at zero
  bf16x8 pr[4];
  f16x8 prh[4];

  // Iteration it: LDS holds K(it) (K slot it%3) and V(it-1) (V slot
  // (it+2)%3); K(it+1) and V(it) are landing.  It issues the loads of K(it+2)
  // and V(it+1) into the slots freed by tiles it-1 and it-2.  CUR and PREV say
  // whether tiles it and it-1 are core tiles (fp16 operands) or raw tiles
  // (bf16).  S = Q.K^T(it) on the matrix cores;
  // then tile it's softmax on the vector ALUs while the matrix cores run P.V
  // of tile it-1.  Chunk cc of pr is consumed by that P.V just before tile
  // it's chunk cc overwrites it.  The rescale a new max demands (alpha) is
  // applied to the accumulators at the top of the next iteration, i.e. after
  // the P.V of tile it-1 and before that of tile it.  The loop body is kept
  // free of branches between the max and the barrier so that the P.V MFMAs
  // and the exponentials share one scheduling region.
  bool grow_pending = false;
  float alpha_pending = 1.0f;
  int kslot = 0;  // it % 3 (OFF = 0)
  // Step st, this wave's tile it (it = st unless the wave's half is ahead).
  auto iteration = [&](int st, int it, auto cur_tag, auto prev_tag) {
    constexpr bool CUR = decltype(cur_tag)::value, PREV = decltype(prev_tag)::value;
    int k_cur, v_prev, k_next = 0;  // K slot of tile it, V slot of tile it-1
    if constexpr (OFF == 0) {
      (void)st;
      const int prev = kslot == 0 ? 2 : kslot - 1, next = kslot == 2 ? 0 : kslot + 1;
      load_k(prev, it + 2);  // empty (zeros) past the last tile
      load_v(next, it + 1);
      k_cur = kslot;
      v_prev = prev;
      k_next = next;
    } else {
      const int ql = st + off_b;  // the leading half's tile
      load_v(ql % NSV, ql);
      load_k((ql + 2) % NSK, ql + 2);
      k_cur = it % NSK;
      v_prev = (it + NSV - 1) % NSV;
    }
    if (grow_pending) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha_pending;
      rescale_sums(alpha_pending);
    }
    const char* kt = kbuf(k_cur);
    const char* vt_prev = vbuf(v_prev);
    f32x16 sx[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sx[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 qb = qf[ks];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kt + (32 * kb + j) * KRow + (16 * ks + 8 * hh) * 2);
        sx[kb] = mfma32<CUR>(a, qb, sx[kb]);
      }
    }
    if (!tile_full(it, CUR)) {
      // key kk of the tile is visible to this lane's row iff lo_rel <= kk <= hi_rel
      asm volatile("" ::: "memory");  // keeps this a real (scalar) branch
      const int base = tile_base(it);
      const int lo_rel = CUR ? 0 : my_lo - base;
      const int hi_rel = CUR ? my_nc - 1 - base : t - base;
      const unsigned span = (unsigned)(hi_rel - lo_rel);
      // key offsets from one per-lane value made here (hidden from the
      // compiler, which would otherwise keep all 32 live across the loop)
      int off = 4 * hh - lo_rel;
      asm volatile("" : "+v"(off));
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = 32 * kb + 8 * (r >> 2) + (r & 3);
          const bool vis = hi_rel >= lo_rel && (unsigned)(kk + off) <= span;
          sx[kb][r] = vis ? sx[kb][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sx[kb][r]);
    mt = pair_max(mt);
    // Lazy rescale: the reference max m only moves when the row max grows by
    // more than kLazyLog2 (log2 units), so probabilities stay <= 2^kLazyLog2
    // and the accumulator rescale is skipped on almost every tile.  The final
    // normalisation divides by a sum taken against the same m.
    const float mnew = fmaxf(m, mt);
    const bool grow = (mnew - m) * c > kLazyLog2;  // false while both are -inf
    const float ex = __builtin_amdgcn_exp2f((m - mnew) * c);  // NaN while both are -inf; unused then
    const float alpha = grow ? ex : 1.0f;
    m = grow ? mnew : m;
    const float mc = (m == -INFINITY ? 0.f : m) * c;
    // P.V of tile it-1 interleaved by hand with tile it's exponentials: after
    // each MFMA (32 cycles on the matrix core) come the probabilities it can
    // hide (2 fma, 2 exp, 1 convert per pair).  sched_barrier freezes
    // that order; V^T fragments are read two MFMAs ahead through a ring of 3.
    // The P.V and row-sum MFMAs take tile it-1's operand type, the new
    // probabilities tile it's.
    static_assert(DB == 2 || DB == 4, "head dim 64 or 128");
    constexpr int PPM = 8 / DB;  // probabilities per MFMA slot
    constexpr int NPV = 4 * DB;  // P.V MFMAs per tile
    auto vfrag = [&](int n) { return vfrag_at(vt_prev, n / DB, n % DB); };
    bf16x8 ring[3];
    ring[0] = vfrag(0);
    ring[1] = vfrag(1);
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      // the new chunk is built element-wise in its own type (vector bit-casts
      // of packed dwords here made the compiler copy the fragments around)
      bf16x8 pnew;
      f16x8 pnew_h;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int n = cc * DB + db;
        if (n + 2 < NPV) ring[(n + 2) % 3] = vfrag(n + 2);
        if constexpr (PREV) o[db] = mfma32<true>(ring[n % 3], prh[cc], o[db]);
        else o[db] = mfma32<false>(ring[n % 3], pr[cc], o[db]);
#pragma unroll
        for (int e = db * PPM; e < db * PPM + PPM; e += 2) {
          const int r = (cc & 1) * 8 + e;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sx[cc >> 1][r], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sx[cc >> 1][r + 1], c, -mc));
          if constexpr (CUR) {
            pnew_h[e] = static_cast<_Float16>(p0);
            pnew_h[e + 1] = static_cast<_Float16>(p1);
          } else {
            pnew[e] = static_cast<__bf16>(p0);
            pnew[e + 1] = static_cast<__bf16>(p1);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // tile it-1's chunk cc into the row sums, then replaced by tile it's
      if constexpr (PREV) lsum = mfma16<true>(sel, prh[cc], lsum);
      else lsum = mfma16<false>(sel, pr[cc], lsum);
      if constexpr (CUR) prh[cc] = pnew_h;
      else pr[cc] = pnew;
    }
    grow_pending = __builtin_amdgcn_ballot_w64(grow) != 0;
    alpha_pending = alpha;
    if constexpr (OFF == 0) kslot = k_next;
    sync_stage();
  };
  // the rescale the last tile's new max asked for, before a P.V that runs
  // outside the pipeline
  auto apply_pending_rescale = [&]() {
    if (grow_pending) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha_pending;
      rescale_sums(alpha_pending);
    }
    grow_pending = false;
  };
  // The P.V of a walk's last tile (this wave's tile last), outside the
  // pipeline.  OFF = 0: V(last) sits in the V slot before the next load slot.
  auto flush_tile = [&](int last, auto core_tag) {
    constexpr bool CORE = decltype(core_tag)::value;
    apply_pending_rescale();
    const char* vt;
    if constexpr (OFF == 0) {
      (void)last;
      vt = vbuf(kslot == 0 ? 2 : kslot - 1);
    } else {
      vt = vbuf(last % NSV);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (CORE) o[db] = mfma32<true>(vfrag_at(vt, cc, db), prh[cc], o[db]);
        else o[db] = mfma32<false>(vfrag_at(vt, cc, db), pr[cc], o[db]);
      }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      if constexpr (CORE) lsum = mfma16<true>(sel, prh[cc], lsum);
      else lsum = mfma16<false>(sel, pr[cc], lsum);
    }
  };
  // Raw tiles on bf16 Q fragments, then the core tiles on fp16 ones (converted
  // once, in registers; no value goes back).  Each walk starts with zero
  // probabilities standing for "tile -1" (whose V slot holds finite values),
  // and the raw walk ends with its last tile's P.V flushed.  In a
  // same-process comparison this order and the flush ran faster than the
  // core walk first with a transition tile, whose loop carried 16 register
  // copies of the probabilities per tile.
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[cc][e] = static_cast<__bf16>(0.0f);
  for (int st = 0; st < n_raw_steps; ++st) iteration(st, st + lead_off, RawTile{}, RawTile{});
  if (n_ct > 0) {
    flush_tile(n_raw_steps - 1 + lead_off, RawTile{});
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = bf16_frag_to_f16(qf[ks]);
    sel = selector(CoreTile{});
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int e = 0; e < 8; ++e) prh[cc][e] = static_cast<_Float16>(0.0f);
    for (int st = n_raw_steps; st < n_tiles - off_b; ++st) iteration(st, st + off_b, CoreTile{}, CoreTile{});
  }
  // the loads issued for tiles past the end must land before the workgroup's
  // LDS can be handed to another
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (n_ct > 0) flush_tile(n_tiles - 1, CoreTile{});  // the walk's last tile
  else flush_tile(n_raw_steps - 1 + lead_off, RawTile{});

  // ---- normalise and store: lane holds dims 32db + 8(r/4) + 4hh + r%4 of row j
  // row j's sum: lane j%16 holds it, in lsum[0] for j < 16 and lsum[1] above
  const float l_lo = __int_as_float(__builtin_amdgcn_ds_bpermute((j & 15) * 4, __float_as_int(lsum[0])));
  const float l_hi = __int_as_float(__builtin_amdgcn_ds_bpermute((j & 15) * 4, __float_as_int(lsum[1])));
  const float ltot = j < 16 ? l_lo : l_hi;
  const float inv = 1.0f / ltot;
  if (t_raw < Le) {
    const long orow = (((long)b * A->Hq + h) * A->Lq + (t_raw - qs)) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d0 = 32 * db + 8 * rr + 4 * hh;
        const float x0 = o[db][4 * rr + 0] * inv, x1 = o[db][4 * rr + 1] * inv;
        const float x2 = o[db][4 * rr + 2] * inv, x3 = o[db][4 * rr + 3] * inv;
        if (OT == 1) {
          uint16_t* out = static_cast<uint16_t*>(A->out);
          *reinterpret_cast<uint2*>(out + orow + d0) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
        } else {
          float* out = static_cast<float*>(A->out);
          *reinterpret_cast<float4*>(out + orow + d0) = make_float4(x0, x1, x2, x3);
        }
      }
    // the softmax's normaliser for a backward pass: probabilities are
    // exp2(s c - m c) / ltot, so log-sum-exp (natural log) = (m c + log2 ltot) ln 2
    if (A->lse != nullptr && hh == 0)
      A->lse[((long)b * A->Hq + h) * A->Lq + (t_raw - qs)] = (m * c + log2f(ltot)) * kLn2;
  }
  };

  // ---- blocks below n_static run item blockIdx.x; the others take the tail
  // items from the queues (cca_queue.hpp)
  if ((int)blockIdx.x < P.n_static) {
    item_body(blockIdx.x);
    return;
  }
  unsigned* const slot = g_prefill_queue + 16 * P.qslot;
  __shared__ int claimed;
  int cq = tail_home_queue(), dead = 0;
  for (;;) {
    if (tid == 0) claimed = tail_claim(slot, cq, dead, P.n_static, P.total - P.n_static);
    __syncthreads();  // also: every wave is done with the previous item's LDS
    const int item = __builtin_amdgcn_readfirstlane(claimed);
    __syncthreads();  // every wave has read it before it is written again
    if (item < 0) break;
    item_body(item);
  }
  if (tid == 0) tail_done(slot, gridDim.x - P.n_static);
}

constexpr int kWaves = 8;  // waves per workgroup

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
                               const RowRange& rr, float* lse, hipStream_t s) {
  PrefillParams P;
  P.q = static_cast<const uint16_t*>(q);
  P.k = static_cast<const uint16_t*>(k);
  P.v = static_cast<const uint16_t*>(v);
  P.ck = static_cast<const uint16_t*>(ck);
  P.cv = static_cast<const uint16_t*>(cv);
  P.out = out;
  P.lse = lse;
  P.B = sh.B;
  P.Hq = sh.Hq;
  P.Hkv = sh.Hkv;
  P.q_start = rr.q_start;
  P.q_len = rr.q_len;
  P.Lq = rr.Lq;
  P.Lk = rr.Lk;
  P.g = sh.g;
  P.w = sh.w;
  P.m_cap = m_cap;
  P.G = sh.G();
  P.Hw = gcd_int(P.G, kWaves);
  P.RP = 32 * (kWaves / P.Hw);
  P.nPB = (rr.Lq + P.RP - 1) / P.RP;
  P.nHG = P.G / P.Hw;
  P.U = sh.B * sh.Hkv * P.nHG;
  P.xcd = (P.U % 8 == 0) ? 1 : 0;
  P.c = kLog2e / sqrtf((float)sh.d);
  const long items = (long)P.nPB * P.U;
  if (items > 0x7fffffffL / 2) return hipErrorInvalidConfiguration;
  if (items == 0) return hipSuccess;
  P.total = (int)items;
  // The shortest quarter of the items (a multiple of 8, so that each keeps
  // its XCD) goes to one queue workgroup per compute unit, when there are
  // enough items for the XCDs to drift apart.
  int cus = 0;
  const hipError_t ce = compute_units(&cus);
  if (ce != hipSuccess) return ce;
  const int n_tail = tail_items(items, cus);
  P.n_static = P.total - n_tail;
  const long blocks = (long)P.n_static + std::min(n_tail, cus);
  static std::atomic<unsigned> launches{0};
  P.qslot = (int)(launches.fetch_add(1, std::memory_order_relaxed) % kQueueSlots);
  // one head per workgroup (256 consecutive rows): the halves walk the raw
  // window apart
  const dim3 grid((unsigned)blocks), block(64 * kWaves);
  const bool halves = P.Hw == 1;
  if (sh.d == 64) {
    if (out_dt == 1) {
      if (halves) hipLaunchKernelGGL((prefill_mfma_kernel<64, 1, kWaves, 2>), grid, block, 0, s, P);
      else hipLaunchKernelGGL((prefill_mfma_kernel<64, 1, kWaves, 0>), grid, block, 0, s, P);
    } else {
      if (halves) hipLaunchKernelGGL((prefill_mfma_kernel<64, 0, kWaves, 2>), grid, block, 0, s, P);
      else hipLaunchKernelGGL((prefill_mfma_kernel<64, 0, kWaves, 0>), grid, block, 0, s, P);
    }
  } else {
    if (out_dt == 1) {
      if (halves) hipLaunchKernelGGL((prefill_mfma_kernel<128, 1, kWaves, 2>), grid, block, 0, s, P);
      else hipLaunchKernelGGL((prefill_mfma_kernel<128, 1, kWaves, 0>), grid, block, 0, s, P);
    } else {
      if (halves) hipLaunchKernelGGL((prefill_mfma_kernel<128, 0, kWaves, 2>), grid, block, 0, s, P);
      else hipLaunchKernelGGL((prefill_mfma_kernel<128, 0, kWaves, 0>), grid, block, 0, s, P);
    }
  }
  return hipGetLastError();
}

}  // namespace cca
