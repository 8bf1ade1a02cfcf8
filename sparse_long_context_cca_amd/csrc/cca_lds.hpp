// LDS and buffer-load helpers shared by the matrix-core kernels (gfx950).
//
// Tiles of bf16 rows are moved from memory straight into LDS by buffer loads
// with the LDS bit (each lane's 16 bytes land at M0 + 16 * lane), and read
// back either as rows (16 bytes per lane, the A/B operand of an MFMA whose
// contraction runs along the row) or through the transposing read
// ds_read_b64_tr_b16 (the operand of an MFMA whose contraction runs across
// rows).  gfx950's LDS has 64 banks of 4 bytes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "cca_device.hpp"

namespace cca {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- typed matrix-core operations on 16-bit operands
// Fragments are held as bf16x8 whatever their type: bf16 for the raw keys and
// values (the inputs' dtype), fp16 (the same bits reinterpreted) for the
// cores, which are stored in fp16.  F16 selects the instruction.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef std::integral_constant<bool, true> CoreTile;   // fp16 operands
typedef std::integral_constant<bool, false> RawTile;   // bf16 operands

// The B operand may also come typed as f16x8 (no reinterpretation).
__device__ __forceinline__ f16x8 as_f16(const bf16x8& x) { return __builtin_bit_cast(f16x8, x); }
__device__ __forceinline__ f16x8 as_f16(const f16x8& x) { return x; }
template <bool F16, class BT>
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const BT& b, const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16(a), as_f16(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16, class BT>
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const BT& b, const f32x4& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16(a), as_f16(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Two values rounded (nearest even) to the operand type, packed in a dword.
template <bool F16>
__device__ __forceinline__ uint32_t pack_op(float a, float b) {
  if constexpr (F16) return pack_f16x2(a, b);
  else return pack_bf16x2(a, b);
}
// bf16 fragment -> fp16 fragment (exact for 2^-17 <= |x| < 65504; a
// smaller bf16 value is rounded to fp16's subnormal grid of 2^-24).
__device__ __forceinline__ bf16x8 bf16_frag_to_f16(const bf16x8& x) {
  f16x8 h;
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(static_cast<float>(x[e]));
  return __builtin_bit_cast(bf16x8, h);
}
// The way back, fp16 fragment -> bf16 fragment: exact for a fragment that
// came from bf16_frag_to_f16, except for the values below 2^-17 that it
// rounded, which stay within 2^-25 of the original.
__device__ __forceinline__ bf16x8 f16_frag_to_bf16(const bf16x8& x) {
  const f16x8 h = __builtin_bit_cast(f16x8, x);
  bf16x8 b;
#pragma unroll
  for (int e = 0; e < 8; ++e) b[e] = static_cast<__bf16>(static_cast<float>(h[e]));
  return b;
}

// 32-bit LDS address of a pointer into a __shared__ array.  (Address-space
// casts live in plain functions: inside a kernel template they have no host
// form and would drop the host-side launch stub.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane s points at 4 consecutive 16-bit elements X_s[0..3]; lane i receives
// X_{4e + (i%16)/4}[i % 4] for e = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
}

// Buffer resource over `nbytes` bytes from `base` (raw, no stride); reads past
// the range return zeros.  Every word is uniform (scalar registers).
__device__ __forceinline__ u32x4 buffer_desc(const void* base, int nbytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu;
  r[2] = __builtin_amdgcn_readfirstlane((uint32_t)nbytes);
  r[3] = 0x00020000u;
  return r;
}

// One wave load from a buffer straight into LDS: lane i's 16 bytes (from byte
// voffset of the buffer) land at LDS address m0 + 16 i; m0 is uniform.  Issued
// as inline assembly so that the compiler does not see an LDS write: it would
// otherwise make every later LDS read wait for all such loads in flight.  The
// caller therefore orders these loads itself (a vmcnt wait and a barrier
// before the data are read, and before the kernel ends).
__device__ __forceinline__ void lds_dma16(u32x4 rsrc, uint32_t m0, int voffset) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(m0));
}

// Row layout of a 64-row bf16 tile read both ways (rows of D elements).
// Rows come in groups of four: row r starts at byte (r/4)*kGroup + (r%4)*kRow,
// kRow = 2D + 64 and kGroup = 4 kRow + 16.  Then
//   * a row read (16 lanes = 16 consecutive rows, one 16-byte chunk each) hits
//     16 distinct 16-byte bank slots: (r%4)*kRow moves the row by a quarter of
//     the 256-byte bank line, (r/4)*kGroup by one slot;
//   * a transposing read (32 lanes = 4 aligned consecutive rows x 64 bytes)
//     hits 4 disjoint quarters of the bank line;
// and both addresses are affine in the row, so a lane's address for any
// row block is its base plus an immediate offset.  The 16-byte slots of the
// padding are filled with zeros by the tile loader.
template <int D>
struct BothWaysTile {
  static constexpr int kRow = 2 * D + 64;
  static constexpr int kGroup = 4 * kRow + 16;
  static constexpr int kSlotsPerRow = kRow / 16;      // 16-byte slots per row (with padding)
  static constexpr int kSlotsPerGroup = kGroup / 16;
  static constexpr int kRows = 64;
  static constexpr int kBytesUsed = (kRows / 4) * kGroup;
  static constexpr int kLoads = (kBytesUsed + 1023) / 1024;  // 1 KB wave loads per tile
  static constexpr int kBytes = kLoads * 1024;
  __host__ __device__ static constexpr int row_off(int r) { return (r >> 2) * kGroup + (r & 3) * kRow; }
  // Byte offset in global memory (relative to the tile's first row) of the
  // 16 bytes that land in LDS slot `slot`, or a value past any buffer range
  // (which loads zeros) for a padding slot.
  __device__ static int src_offset(int slot) {
    const int grp = slot / kSlotsPerGroup, in = slot % kSlotsPerGroup;
    const int rr = in / kSlotsPerRow, chunk = in % kSlotsPerRow;
    if (rr >= 4 || chunk >= D / 8 || grp >= kRows / 4) return 0x40000000;
    return ((4 * grp + rr) * D + 8 * chunk) * 2;
  }
};

}  // namespace cca
