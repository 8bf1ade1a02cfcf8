// Fused CCA prefill on the vector ALUs, fp32 arithmetic throughout.
//
// Computes, for every (b, h, t), one softmax over [cores 0..n_core(t)) ;
// raw keys win_lo(t)..t] (digest at digest.lyk-ai.com/posts/2412.12465,
// "Method", fusion formula).  This is the kernel for fp32 inputs and the
// plain-arithmetic cross-check of the bf16 matrix-core kernel.
//
// A block owns 128 consecutive query rows of one query head; two threads share
// a row, each holding half of the head dimension of q and of the output
// accumulator.  The block walks the union of its rows' visible keys (cores
// first, then the raw window) in tiles of 32 keys staged in LDS as fp32, and
// applies each row's own visibility mask inside the tile.  Online softmax in
// the log2 domain; one rescale per tile.
#include "cca_device.hpp"
#include "cca_internal.hpp"

namespace cca {
namespace {

constexpr int kRows = 128;
constexpr int kTile = 32;

template <int DT, int OT, int D>
__global__ __launch_bounds__(256) void prefill_valu_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const void* __restrict__ ck_, const void* __restrict__ cv_, void* __restrict__ out_, int m_cap,
    const int32_t* __restrict__ q_start, const int32_t* __restrict__ q_len, float* __restrict__ lse,
    int Hq, int Hkv, int Lq, int Lk, int g, int w, float scale_log2) {
  typedef Elem<DT> E;
  typedef typename E::T T;
  constexpr int DH = D / 2;
  __shared__ float sk[kTile][D + 1];
  __shared__ float sv[kTile][D + 1];

  const int tid = threadIdx.x;
  const int half = tid & 1;
  const int r = tid >> 1;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int G = Hq / Hkv;
  const int hk = h / G;
  // sequence b's rows: positions qs .. qs + ql - 1 at local rows 0 .. ql - 1
  const SeqRows sr = seq_rows(q_start, q_len, b, Lq, Lk, g, w, m_cap);
  const int r0 = blockIdx.x * kRows;  // local row of the block's first row
  typedef Elem<OT> EO;
  typename EO::T* out = static_cast<typename EO::T*>(out_);
  if (!sr.ok) {  // rows that do not fit the buffers: NaN, nothing read
    if (r0 + r < Lq) {
      const long orow = ((long)(b * Hq + h) * Lq + r0 + r) * D + half * DH;
      for (int e = 0; e < DH; ++e) EO::store(out, orow + e, NAN);
    }
    return;
  }
  if (r0 >= sr.ql) return;
  const int qs = sr.qs, Le = sr.qs + sr.ql;
  const int t0 = qs + r0;
  const int t_hi = min(Le - 1, t0 + kRows - 1);
  const int t = min(t0 + r, Le - 1);  // rows past the end compute a duplicate and store nothing

  const T* q = static_cast<const T*>(q_);
  const T* kk = static_cast<const T*>(k_);
  const T* vv = static_cast<const T*>(v_);
  // the core cache: fp32 for fp32 inputs, fp16 for bf16 inputs
  typedef Elem<core_dt(DT)> EC;
  const typename EC::T* ck = static_cast<const typename EC::T*>(ck_);
  const typename EC::T* cv = static_cast<const typename EC::T*>(cv_);

  float qr[DH], acc[DH];
  const long qrow = ((long)(b * Hq + h) * Lq + (t - qs)) * D + half * DH;
#pragma unroll
  for (int e = 0; e < DH; ++e) {
    qr[e] = E::load(q, qrow + e);
    acc[e] = 0.f;
  }
  const int my_nc = n_core(t, g, w);
  const int my_lo = win_lo(t, w);

  // Union of visible keys of this block's rows, as one flat index space:
  // [0, nc_hi) are cores, [nc_hi, nc_hi + nraw) are raw positions raw_lo.. .
  const int nc_hi = n_core(t_hi, g, w);
  const int raw_lo = win_lo(t0, w);
  const int nraw = t_hi - raw_lo + 1;
  const int total = nc_hi + nraw;
  const long kv_base = (long)(b * Hkv + hk);

  float mrun = -INFINITY, lrun = 0.f;
  for (int base = 0; base < total; base += kTile) {
    __syncthreads();
    for (int idx = tid; idx < kTile * D; idx += 256) {
      const int i = idx / D, e = idx % D;
      const int f = base + i;
      float kx = 0.f, vx = 0.f;
      if (f < nc_hi) {
        const long off = (kv_base * m_cap + f) * D + e;
        kx = EC::load(ck, off);
        vx = EC::load(cv, off);
      } else if (f < total) {
        const long off = (kv_base * Lk + raw_lo + (f - nc_hi)) * D + e;
        kx = E::load(kk, off);
        vx = E::load(vv, off);
      }
      sk[i][e] = kx;
      sv[i][e] = vx;
    }
    __syncthreads();
    float s[kTile];
    float mt = -INFINITY;
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DH; ++e) part = fmaf(qr[e], sk[i][half * DH + e], part);
      part += __shfl_xor(part, 1, 64);
      const int f = base + i;
      bool vis;
      if (f < nc_hi) {
        vis = f < my_nc;
      } else {
        const int pos = raw_lo + (f - nc_hi);
        vis = f < total && pos >= my_lo && pos <= t;
      }
      s[i] = vis ? part * scale_log2 : -INFINITY;
      mt = fmaxf(mt, s[i]);
    }
    const float mnew = fmaxf(mrun, mt);
    if (mnew == -INFINITY) continue;  // nothing visible to this row yet
    const float alpha = exp2f(mrun - mnew);
    lrun *= alpha;
#pragma unroll
    for (int e = 0; e < DH; ++e) acc[e] *= alpha;
#pragma unroll
    for (int i = 0; i < kTile; ++i) {
      const float p = exp2f(s[i] - mnew);
      lrun += p;
#pragma unroll
      for (int e = 0; e < DH; ++e) acc[e] = fmaf(p, sv[i][half * DH + e], acc[e]);
    }
    mrun = mnew;
  }
  if (t0 + r < Le) {
    const float inv = 1.0f / lrun;
    const long orow = ((long)(b * Hq + h) * Lq + (t - qs)) * D + half * DH;
#pragma unroll
    for (int e = 0; e < DH; ++e) EO::store(out, orow + e, acc[e] * inv);
    // natural-log log-sum-exp of the row's scores, for a backward pass
    if (lse != nullptr && half == 0)
      lse[(long)(b * Hq + h) * Lq + (t - qs)] = (mrun + log2f(lrun)) * kLn2;
  }
}

template <int DT, int OT, int D>
void launch_t(const void* q, const void* k, const void* v, const void* ck, const void* cv,
              int m_cap, void* out, const Shape& sh, const RowRange& rr, float* lse,
              hipStream_t s) {
  dim3 grid((rr.Lq + kRows - 1) / kRows, sh.Hq, sh.B);
  const float scale_log2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((prefill_valu_kernel<DT, OT, D>), grid, dim3(256), 0, s, q, k, v, ck, cv, out,
                     m_cap, rr.q_start, rr.q_len, lse, sh.Hq, sh.Hkv, rr.Lq, rr.Lk, sh.g, sh.w,
                     scale_log2);
}

}  // namespace

hipError_t launch_prefill_valu(const void* q, const void* k, const void* v, const void* ck,
                               const void* cv, int m_cap, void* out, int out_dt, const Shape& sh,
                               const RowRange& rr, float* lse, int dt, hipStream_t s) {
  if (dt == 0) {
    if (sh.d == 64) launch_t<0, 0, 64>(q, k, v, ck, cv, m_cap, out, sh, rr, lse, s);
    else launch_t<0, 0, 128>(q, k, v, ck, cv, m_cap, out, sh, rr, lse, s);
  } else if (out_dt == 1) {
    if (sh.d == 64) launch_t<1, 1, 64>(q, k, v, ck, cv, m_cap, out, sh, rr, lse, s);
    else launch_t<1, 1, 128>(q, k, v, ck, cv, m_cap, out, sh, rr, lse, s);
  } else {
    if (sh.d == 64) launch_t<1, 0, 64>(q, k, v, ck, cv, m_cap, out, sh, rr, lse, s);
    else launch_t<1, 0, 128>(q, k, v, ck, cv, m_cap, out, sh, rr, lse, s);
  }
  return hipGetLastError();
}

}  // namespace cca
