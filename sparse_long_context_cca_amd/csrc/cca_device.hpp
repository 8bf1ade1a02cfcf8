// Device-side helpers shared by the CCA kernels (gfx950, wave64).
//
// Index functions implement the visibility rule of the fused softmax (digest
// at digest.lyk-ai.com/posts/2412.12465, "Method", fusion formula; the pages
// name the core set T_i and the window set U_i without defining them):
//   window of query t : raw positions win_lo(t) = max(0, t-w+1) .. t
//   cores of query t  : groups j with (j+1)g-1 < t-w+1, i.e. j < n_core(t)
// Every kernel and the table export call these same functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cca {

__host__ __device__ __forceinline__ int win_lo(int t, int w) {
  int lo = t - w + 1;
  return lo > 0 ? lo : 0;
}

__host__ __device__ __forceinline__ int n_core(int t, int g, int w) {
  int u = t - w + 1;
  return u > 0 ? u / g : 0;
}

__host__ __device__ __forceinline__ int group_last(int j, int g) { return (j + 1) * g - 1; }

// Query rows of sequence b in a chunked / variable-length call (see RowRange):
// q_start and q_len from device arrays, or 0 and Lq when there are none.  ok
// is false when the range does not fit the buffers (q_start < 0, q_len < 0,
// q_len > Lq, q_start + q_len > Lk) or sees a core beyond m_cap; such a
// sequence gets NaN rows and nothing is read for it.
struct SeqRows {
  int qs, ql;
  bool ok;
};
__device__ __forceinline__ SeqRows seq_rows(const int32_t* q_start, const int32_t* q_len, int b,
                                            int Lq, int Lk, int g, int w, int m_cap) {
  SeqRows r;
  r.qs = 0;
  r.ql = Lq;
  if (q_start != nullptr) {
    r.qs = __builtin_amdgcn_readfirstlane(q_start[b]);
    r.ql = __builtin_amdgcn_readfirstlane(q_len[b]);
  }
  r.ok = r.qs >= 0 && r.ql >= 0 && r.ql <= Lq && (long)r.qs + r.ql <= Lk &&
         (r.ql == 0 || n_core(r.qs + r.ql - 1, g, w) <= m_cap);
  return r;
}

typedef uint16_t bf16_bits;

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest even via the
// hardware conversion.
__device__ __forceinline__ float bf16_to_f32(bf16_bits h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ bf16_bits f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(bf16_bits, b);
}
// Two floats -> packed bf16x2 in one dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  bf2 v;
  v[0] = static_cast<__bf16>(a);
  v[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// fp16 <-> fp32 (the core cache of bf16 inputs).  Widening is exact;
// narrowing rounds to nearest even.
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
// Two floats -> packed fp16x2 in one dword (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef _Float16 f2 __attribute__((ext_vector_type(2)));
  f2 v;
  v[0] = static_cast<_Float16>(a);
  v[1] = static_cast<_Float16>(b);
  return __builtin_bit_cast(uint32_t, v);
}

// Storage dtype of the core cache for input dtype DT: fp32 cores for fp32
// inputs, fp16 cores for bf16 inputs.  A core is a convex combination of the
// group's keys (values), so it needs their range but more precision than bf16
// gives: with keys of magnitude ~15 the bf16 rounding of the cores alone moves
// attention outputs by ~0.03, the fp16 rounding by ~0.003.
constexpr int core_dt(int dt) { return dt == 0 ? 0 : 2; }

// Element access by dtype (0 = fp32, 1 = bf16, 2 = fp16).
template <int DT>
struct Elem;
template <>
struct Elem<0> {
  typedef float T;
  static __device__ __forceinline__ float load(const T* p, long i) { return p[i]; }
  static __device__ __forceinline__ void store(T* p, long i, float x) { p[i] = x; }
};
template <>
struct Elem<1> {
  typedef bf16_bits T;
  static __device__ __forceinline__ float load(const T* p, long i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(T* p, long i, float x) { p[i] = f32_to_bf16(x); }
};
template <>
struct Elem<2> {
  typedef uint16_t T;
  static __device__ __forceinline__ float load(const T* p, long i) { return f16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(T* p, long i, float x) { p[i] = f32_to_f16(x); }
};

// Wave64 reductions.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace cca
