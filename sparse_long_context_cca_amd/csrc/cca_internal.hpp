// Host-side launchers of the CCA kernels (internal; the public ABI is cca.h).
// Arguments reaching these functions have been validated by cca_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cca {

struct Shape {
  int B, Hq, Hkv, L, d, g, w;
  int G() const { return Hq / Hkv; }
  int m() const { return L / g; }
};

hipError_t launch_visibility(int L, int g, int w, int32_t* n_core, int32_t* win_lo,
                             int32_t* group_last, hipStream_t s);

// mode: PoolMode (cca_pool_group.hpp), equal to the cca_pool_mode values.
hipError_t launch_pool(const void* q, const void* k, const void* v, void* ck, void* cv, int m_cap,
                       float* weights, const Shape& sh, int dt, int mode, hipStream_t s);

// Vector-ALU prefill (fp32 math, any input dtype).
hipError_t launch_prefill_valu(const void* q, const void* k, const void* v, const void* ck,
                               const void* cv, int m_cap, void* out, int out_dt, const Shape& sh,
                               int dt, hipStream_t s);

// bf16 matrix-core prefill.
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* ck,
                               const void* cv, int m_cap, void* out, int out_dt, const Shape& sh,
                               hipStream_t s);

struct DecodePlan {
  int splits;         // key-range splits per (b, kv head)
  size_t ws_bytes;    // workspace bytes
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int d, int m_cap, int g, int w);

hipError_t launch_decode(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                         void* ring_v, int R, void* ck, void* cv, int m_cap, int32_t* pos,
                         int advance_pos, void* out, int out_dt, void* ws, const DecodePlan& plan,
                         const Shape& sh, int dt, int pool_mode, hipStream_t s);

}  // namespace cca
