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

// The query rows a prefill or pooling call covers.  Sequence b's rows are
// positions q_start[b] .. q_start[b] + q_len[b] - 1, stored at local rows 0..
// of Q and of the output (Lq rows per sequence); its K and V hold positions
// 0 .. Lk - 1 (only those below q_start[b] + q_len[b] are read).  Null arrays
// (both or neither) mean q_start = 0 and q_len = Lq: every row of a full
// prefill, with Lq = Lk = L.
struct RowRange {
  const int32_t* q_start = nullptr;
  const int32_t* q_len = nullptr;
  int Lq = 0;
  int Lk = 0;
};

hipError_t launch_visibility(int L, int g, int w, int32_t* n_core, int32_t* win_lo,
                             int32_t* group_last, hipStream_t s);

// mode: PoolMode (cca_pool_group.hpp), equal to the cca_pool_mode values.
// Pools the groups whose last token lies among the covered rows (all complete
// groups of a full prefill); the pooling queries come from Q's local rows.
hipError_t launch_pool(const void* q, const void* k, const void* v, void* ck, void* cv, int m_cap,
                       float* weights, const Shape& sh, const RowRange& rr, int dt, int mode,
                       hipStream_t s);

// Vector-ALU prefill (fp32 math, any input dtype).
// lse: null, or fp32 [B,Hq,Lq] receiving each row's natural-log log-sum-exp
// of its scores (the statistic a backward pass needs).
hipError_t launch_prefill_valu(const void* q, const void* k, const void* v, const void* ck,
                               const void* cv, int m_cap, void* out, int out_dt, const Shape& sh,
                               const RowRange& rr, float* lse, int dt, hipStream_t s);

// bf16 matrix-core prefill.
hipError_t launch_prefill_mfma(const void* q, const void* k, const void* v, const void* ck,
                               const void* cv, int m_cap, void* out, int out_dt, const Shape& sh,
                               const RowRange& rr, float* lse, hipStream_t s);

// Compute units of the current device (looked up once per device).
hipError_t compute_units(int* out);

struct DecodePlan {
  int splits;         // key-range splits per (b, kv head)
  size_t ws_bytes;    // workspace bytes
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int d, int m_cap, int g, int w);

// Device scratch of cca_attn_decode_scratch (a fixed array in cca_decode.hip,
// one per GPU): its device address on the current device, looked up once per
// device.  Calls that overlap on one GPU share it and race.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
hipError_t decode_scratch(void** ptr);

hipError_t launch_decode(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                         void* ring_v, int R, void* ck, void* cv, int m_cap, int32_t* pos,
                         int advance_pos, void* out, int out_dt, void* ws, const DecodePlan& plan,
                         const Shape& sh, int dt, int pool_mode, hipStream_t s);

// Backward pass (cca_backward.hip).  Workspace: two fp32 row statistics per
// row [B,Hq,L,2], the core gradients dCK, dCV [B,Hkv,L/g,d] (fp32), and for
// bf16 inputs (from a 256-byte boundary) fp16 copies of q and dO [B,Hq,L,d].
size_t backward_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int g, int dt);
hipError_t launch_backward(const void* q, const void* k, const void* v, const void* ck,
                           const void* cv, int m_cap, const void* out, const float* lse,
                           const void* dout, float* dq, float* dk, float* dv, void* ws,
                           const Shape& sh, int dt, int pool_mode, hipStream_t s);

// bf16 matrix-core part of the backward (cca_backward_mfma.hip): row
// statistics {lse log2(e), dO.O} into stats [B,Hq,L] and fp16 copies of q and
// dO into q16, do16 [B,Hq,L,d], dq (fully written), the raw-key dk, dv (fully
// written) and the core gradients added into dck, dcv ([B,Hkv,L/g,d], zeroed
// by the caller).
hipError_t launch_backward_mfma(const void* q, const void* k, const void* v, const void* ck,
                                const void* cv, int m_cap, const void* out, const float* lse,
                                const void* dout, float* dq, float* dk, float* dv, float2* stats,
                                float* dck, float* dcv, uint16_t* q16, uint16_t* do16,
                                const Shape& sh, hipStream_t s);

// Copies positions max(0, len-R) .. len-1 of sequence b's K and V (len =
// seq_len[b], device) into ring slot p % R; a len outside 0 .. Lk copies nothing.
hipError_t launch_fill_ring(const void* k, const void* v, void* ring_k, void* ring_v, int R,
                            const int32_t* seq_len, int B, int Hkv, int Lk, int d, int elem_bytes,
                            hipStream_t s);

}  // namespace cca
