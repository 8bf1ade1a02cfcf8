// Matrix-core probe (libcca_probe.so): back-to-back bf16 MFMAs on random
// register operands, the rate the matrix cores sustain on this chip with
// nothing else running beside them.  Measurement infrastructure, not part of
// the CCA path; declared in cca_probe.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/cca_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// a bf16 in [-2, 2): random sign, exponent 126 or 127, random mantissa
__device__ __forceinline__ __bf16 random_bf16(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  const uint16_t bits = (uint16_t)((x & 0x807fu) | ((x & 0x80u) ? 0x3f80u : 0x3f00u));
  return __builtin_bit_cast(__bf16, bits);
}

template <int NSET>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void probe_mfma_kernel(float* out, int iters, uint32_t seed) {
  const uint32_t gid = blockIdx.x * 512u + threadIdx.x;
  bf16x8 a[NSET], b[NSET];
#pragma unroll
  for (int s = 0; s < NSET; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[s][e] = random_bf16(seed ^ (gid * 64u + s * 16u + e));
      b[s][e] = random_bf16(seed ^ (gid * 64u + s * 16u + 8u + e) ^ 0x9e3779b9u);
    }
  f32x16 c0 = {}, c1 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 16; k += 2) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k % NSET], b[k % NSET], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(k + 1) % NSET], b[(k + 1) % NSET], c1, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r];
  out[gid] = s;
}

}  // namespace

extern "C" int cca_probe_mfma(float* out, int blocks, int iters, int operand_sets, unsigned seed, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1 || operand_sets < 1 || operand_sets > 4) return 1;
  const dim3 grid((unsigned)blocks), block(512);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // an error left by an earlier call is not this launch's
  switch (operand_sets) {
    case 1: hipLaunchKernelGGL(probe_mfma_kernel<1>, grid, block, 0, s, out, iters, seed); break;
    case 2: hipLaunchKernelGGL(probe_mfma_kernel<2>, grid, block, 0, s, out, iters, seed); break;
    case 3: hipLaunchKernelGGL(probe_mfma_kernel<3>, grid, block, 0, s, out, iters, seed); break;
    default: hipLaunchKernelGGL(probe_mfma_kernel<4>, grid, block, 0, s, out, iters, seed); break;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : 1000 + (int)e;
}
