/*
 * cca.h - C ABI of the Core Context Aware (CCA) attention forward on AMD
 * MI355X (gfx950).
 *
 * The method (Core Context Aware Transformers for Long Context Language
 * Modeling):
 *   - global-aware pooling: tokens are cut into non-overlapping groups of g;
 *     each group becomes one core key/value pair, weighted by a softmax of the
 *     group's last query against the group's keys (digest at
 *     digest.lyk-ai.com/posts/2412.12465, "Method", pooling formula; ICML 2025
 *     article at changsha.jmyizhao.com, global-aware pooling paragraph);
 *   - locality-preserving module: each token also sees the raw keys of its last
 *     w tokens (same article, locality-preserving module paragraph);
 *   - fusion: one softmax over [visible core tokens ; raw window] (digest,
 *     "Method", fusion formula; paper card at atlas.scime.ai, "Approach").
 *
 * Visibility (the pages name the index sets but do not define them; this
 * library fixes them as): query t sees raw positions max(0, t-w+1) .. t and the
 * core of every group j whose last token (j+1)g-1 < t-w+1, i.e.
 *   n_core(t) = max(0, floor((t-w+1)/g)),  win_lo(t) = max(0, t-w+1).
 * Groups start at token 0; a trailing partial group has no core.
 * GQA: one core pair per (kv head, group); its pooling query is the mean over
 * the G = Hq/Hkv query heads of that kv head of their last-token queries.
 * Query head h reads kv head h / G.  Softmax scale is 1/sqrt(d) everywhere.
 *
 * Conventions shared by every entry point:
 *   - Layouts are row-major with the head dimension d contiguous:
 *       Q, O        [B, Hq, L, d]      K, V          [B, Hkv, L, d]
 *       core K/V    [B, Hkv, m_cap, d] (slot j = group j)
 *   - Every pointer argument except `stream` is a DEVICE pointer, 16-byte
 *     aligned.  The caller allocates and frees all memory (including the decode
 *     workspace) and owns the stream; the library never allocates, frees or
 *     synchronises.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously; results are valid once the stream has been synchronised.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is enqueued and a status other than CCA_OK is returned,
 *     with a message available from cca_last_error() (per thread).
 *   - Input dtype `dt` applies to q, k, v, the new token and the decode ring.
 *     Supported: d in {64, 128}; dt in {CCA_F32, CCA_BF16}; out_dt in
 *     {dt, CCA_F32}.  Every buffer must hold at most 2^40 elements (offsets are
 *     64-bit); sequence lengths, g, w, the ring size R and m_cap are below
 *     2^30 (positions are 32-bit).  Beyond either: CCA_ERR_UNSUPPORTED.
 *   - Core cache dtype: cca_core_dtype(dt), i.e. fp32 cores for fp32 inputs
 *     and FP16 cores for bf16 inputs (same element size as the inputs).  A
 *     core is a weighted mean of its group's keys (values); with keys of
 *     magnitude ~15 the bf16 rounding of the cores alone moves attention
 *     outputs by ~0.03, fp16 rounding by ~0.003.  For bf16 inputs the products
 *     with cores therefore run on fp16 operands: q (and in the backward dout)
 *     is converted to fp16 for them, so q, k, v and dout must stay below
 *     fp16's range limit (|x| < 65504); beyond it results are undefined.
 *   - Rounding: accumulation is fp32; core K/V and outputs are rounded to their
 *     storage dtype once, to nearest even.  bf16 attention feeds the matrix
 *     cores bf16 operands for raw keys and fp16 operands for cores; the
 *     probabilities are rounded to that operand type before P*V.
 *   - Concurrency: a bf16 prefill launch (cca_attn_prefill, _ex, _chunk,
 *     _train) that has many row blocks hands its shortest ones out through
 *     work-queue counters held in library-owned device memory, 64 slots per
 *     GPU taken round robin, one per launch, and cleared by the launch itself;
 *     so do the two main kernels of a bf16 cca_attn_backward with many row or
 *     key blocks (64 slots each of their own).  At most 64 calls of each kind
 *     may be in flight on one GPU at once (across all streams).  A launch captured into a graph keeps the slot it took at
 *     capture for every replay, so replays that overlap in time (of one graph,
 *     or of graphs captured with such launches) can share counters and must
 *     not be run concurrently; sequential replays are safe.
 */
#ifndef CCA_H
#define CCA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cca_status {
  CCA_OK = 0,
  CCA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, non-positive size, bad enum */
  CCA_ERR_UNSUPPORTED = 2, /* d not in {64,128}, dtype combination, Hq % Hkv != 0, size limits */
  CCA_ERR_CAPACITY = 3,    /* m_cap < L/g, ring R < max(w, g), workspace too small */
  CCA_ERR_HIP = 4          /* a HIP launch failed; see cca_last_error() */
} cca_status;

/* Element types.  CCA_F16 names the core cache of bf16 inputs only; it is not
 * accepted as an input or output dtype.  Entry points take dtypes as int, so
 * that any value a caller passes is checked rather than undefined. */
typedef enum cca_dtype { CCA_F32 = 0, CCA_BF16 = 1, CCA_F16 = 2 } cca_dtype;

/*
 * Pooling rule for the core token of a group (used by cca_pool_core_ex and
 * cca_attn_decode_ex; the other entry points use CCA_POOL_SOFTMAX):
 *   CCA_POOL_SOFTMAX        global-aware pooling: a = softmax(qbar . K / sqrt(d))
 *                           with qbar the mean over the G query heads of the
 *                           group's last-token query (digest, "Method",
 *                           pooling formula; one query per kv head).
 *   CCA_POOL_SOFTMAX_HEADS  a = mean over the G heads of softmax(q_h . K /
 *                           sqrt(d)); the rebuttal's GQA answer leaves this
 *                           rule open.  Needs G <= 8.
 *   CCA_POOL_MEAN           a = 1/g (the mean-pooling ablation the rebuttal
 *   CCA_POOL_MAX            names, answer on Table 3); element-wise maximum
 *                           over the group of K and of V (max-pooling
 *                           ablation), which has no weights.
 */
typedef enum cca_pool_mode {
  CCA_POOL_SOFTMAX = 0,
  CCA_POOL_SOFTMAX_HEADS = 1,
  CCA_POOL_MEAN = 2,
  CCA_POOL_MAX = 3
} cca_pool_mode;

/* Library version (major*10000 + minor*100 + patch). */
int cca_version(void);

/* Static string for a status code. */
const char* cca_status_string(int status);

/* Message of the last error returned on the calling thread ("" if none). */
const char* cca_last_error(void);

/* Dtype of the core cache (core_k, core_v) for input dtype dt: CCA_F32 for
 * CCA_F32, CCA_F16 for CCA_BF16; -1 for any other value. */
int cca_core_dtype(int dt);

/*
 * cca_visibility_table - integer index tables of the visibility rule above.
 *   n_core[t] and win_lo[t] for t < L (int32 [L]); group_last[j] = (j+1)g-1
 *   for j < L/g (int32 [L/g]; may be NULL when L < g).
 * Bit-exact by construction; the kernels use the same device index functions.
 */
cca_status cca_visibility_table(int L, int g, int w, int32_t* n_core, int32_t* win_lo,
                                int32_t* group_last, void* stream);

/*
 * cca_pool_core - global-aware pooling (digest, "Method", pooling formula).
 *   For every (b, kv head, group j < m = L/g):
 *     qbar = mean over the G query heads of Q[b, h, (j+1)g-1, :]
 *     a    = softmax_tau(qbar . K[b, kv, jg+tau, :] / sqrt(d)), tau < g
 *     core_k[b, kv, j, :] = sum_tau a_tau K[b, kv, jg+tau, :]   (same for V)
 *   q [B,Hq,L,d], k/v [B,Hkv,L,d] (dt); core_k/core_v [B,Hkv,m_cap,d]
 *   (cca_core_dtype(dt)), slots j < m written, others untouched.  weights: NULL, or fp32
 *   [B,Hkv,m,g] receiving a (for tests).
 * Errors: INVALID_ARG (null, L<1, g<1, B/Hq/Hkv<1), UNSUPPORTED (d, dt,
 *   Hq % Hkv), CAPACITY (m_cap < m).
 */
cca_status cca_pool_core(const void* q, const void* k, const void* v, void* core_k, void* core_v,
                         int m_cap, float* weights, int B, int Hq, int Hkv, int L, int d, int g,
                         int dt, void* stream);

/*
 * cca_pool_core_ex - cca_pool_core with a pooling rule (cca_pool_mode above).
 *   weights receives the a of the rule; it must be NULL for CCA_POOL_MAX.
 *   q is not read by CCA_POOL_MEAN and CCA_POOL_MAX (it may be NULL there).
 * Errors: as cca_pool_core; INVALID_ARG for an unknown mode or weights with
 *   CCA_POOL_MAX; UNSUPPORTED for CCA_POOL_SOFTMAX_HEADS with G > 8.
 */
cca_status cca_pool_core_ex(const void* q, const void* k, const void* v, void* core_k,
                            void* core_v, int m_cap, float* weights, int B, int Hq, int Hkv, int L,
                            int d, int g, int dt, int mode, void* stream);

/*
 * cca_attn_prefill - causal prefill of the fused CCA attention (digest,
 * "Method", fusion formula): for every (b, h, t < L)
 *     keys   = [core_k[0 .. n_core(t)) ; K[win_lo(t) .. t]]   (values alike)
 *     out[b,h,t,:] = softmax(q_t . keys^T / sqrt(d)) . values
 *   core_k/core_v: [B,Hkv,m_cap,d] as written by cca_pool_core (slots < L/g
 *   are read).  out: [B,Hq,L,d] in out_dt.
 * Errors: as cca_pool_core, plus INVALID_ARG for w < 1 or a bad out_dt.
 */
cca_status cca_attn_prefill(const void* q, const void* k, const void* v, const void* core_k,
                            const void* core_v, int m_cap, void* out, int out_dt, int B,
                            int Hq, int Hkv, int L, int d, int g, int w, int dt,
                            void* stream);

/*
 * cca_attn_prefill_ex - cca_attn_prefill with an explicit kernel choice, for
 * tests: kernel 0 = automatic (bf16: matrix-core kernel; fp32: vector
 * kernel), 1 = fp32 vector kernel (any dt), 2 = bf16 matrix-core kernel.
 * UNSUPPORTED if the choice does not fit dt.
 */
cca_status cca_attn_prefill_ex(const void* q, const void* k, const void* v, const void* core_k,
                               const void* core_v, int m_cap, void* out, int out_dt, int B,
                               int Hq, int Hkv, int L, int d, int g, int w, int dt,
                               int kernel, void* stream);

/*
 * Training: the forward with its softmax statistic, and the backward pass.
 * The pages fine-tune pretrained models with CCA attention in place (paper
 * card, summary and key results; rebuttal, answer on the fine-tuning
 * setting); the gradients follow from the chain rule through the fusion and
 * pooling formulas (digest, "Method").
 *
 * cca_attn_prefill_train - cca_attn_prefill (automatic kernel) that also
 *   writes lse: fp32 [B,Hq,L], each row's natural-log log-sum-exp of its
 *   scores q_t . key / sqrt(d) over its visible keys.
 */
cca_status cca_attn_prefill_train(const void* q, const void* k, const void* v, const void* core_k,
                                  const void* core_v, int m_cap, void* out, int out_dt,
                                  float* lse, int B, int Hq, int Hkv, int L, int d, int g, int w,
                                  int dt, void* stream);

/*
 * cca_attn_backward_workspace_bytes - device workspace cca_attn_backward needs
 *   for input dtype dt: two fp32 row statistics per row, [B,Hq,L,2], the core
 *   gradients 2 x [B,Hkv,L/g,d] fp32, and for bf16 inputs fp16 copies of q and
 *   dout (2 x [B,Hq,L,d], from a 256-byte boundary), which the products with
 *   the fp16 cores read; 0 for sizes below 1 or an unknown dt.
 */
size_t cca_attn_backward_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int g,
                                         int dt);

/*
 * cca_attn_backward - gradients of the whole forward (pooling with rule
 *   pool_mode, then the fused prefill) w.r.t. q, k and v, given the upstream
 *   gradient dout of out:
 *     q, k, v, out, dout in dt, core_k, core_v in cca_core_dtype(dt) (out and
 *     dout [B,Hq,L,d]; out and the cores as the forward wrote them); lse fp32 [B,Hq,L] from
 *     cca_attn_prefill_train; dq [B,Hq,L,d], dk, dv [B,Hkv,L,d] fp32, fully
 *     overwritten.  Per row: dS = P (dP - dout . out); dq, and the raw and
 *     core key/value gradients, as in the chain rule; the core gradients then
 *     flow through pooling into the group's k, v and the pooling query rows.
 *     Max pooling routes each component's gradient to the first token holding
 *     the maximum.  workspace: device memory of at least
 *     cca_attn_backward_workspace_bytes bytes; no initialisation needed.
 * Errors: INVALID_ARG (null/misaligned pointers, sizes, unknown mode),
 *   UNSUPPORTED (d, dt, Hq % Hkv, per-head pooling with G > 8, B*Hkv or Hq >
 *   65535), CAPACITY (m_cap < L/g, workspace too small).
 */
cca_status cca_attn_backward(const void* q, const void* k, const void* v, const void* core_k,
                             const void* core_v, int m_cap, const void* out, const float* lse,
                             const void* dout, float* dq, float* dk, float* dv, void* workspace,
                             size_t workspace_bytes, int B, int Hq, int Hkv, int L, int d, int g,
                             int w, int dt, int pool_mode, void* stream);

/*
 * Chunked and variable-length prefill.  The article notes that CCA generates
 * with token counts that are not multiples of g; a long prompt is processed in
 * chunks, and sequences of one batch have their own lengths.  Each sequence b
 * covers the query positions q_start[b] .. q_start[b] + q_len[b] - 1 (q_start,
 * q_len: device int32 [B], 4-byte aligned; q_len[b] may be 0), stored at local
 * rows 0 .. q_len[b]-1 of q and out ([B,Hq,Lq,d], rows >= q_len[b] untouched);
 * its k/v ([B,Hkv,Lk,d]) hold positions 0 .. q_start[b] + q_len[b] - 1 (the
 * cached prefix and the chunk).  A chunked pass is the same computation as one
 * full prefill: chunk after chunk, cca_pool_core_chunk then
 * cca_attn_prefill_chunk give exactly the rows cca_pool_core + cca_attn_prefill
 * give over the whole sequence (up to summation order).  A sequence whose
 * range does not fit (q_start < 0, q_len < 0 or > Lq, q_start + q_len > Lk,
 * or a visible core beyond m_cap) gets NaN in its Lq output rows and no cache
 * writes; the arrays live on the device, so this is not a status.
 *
 * cca_pool_core_chunk - pools, with rule `mode`, every group j < m_cap whose
 *   last token (j+1)g-1 lies among the covered positions of its sequence; the
 *   pooling query is that row of q (groups may start before q_start: their
 *   tokens come from k/v).  Writes core slots j of core_k/core_v
 *   ([B,Hkv,m_cap,d]).  q is not read by CCA_POOL_MEAN / CCA_POOL_MAX.
 */
cca_status cca_pool_core_chunk(const void* q, const void* k, const void* v, void* core_k,
                               void* core_v, int m_cap, const int32_t* q_start,
                               const int32_t* q_len, int B, int Hq, int Hkv, int Lq, int Lk, int d,
                               int g, int dt, int mode, void* stream);

/*
 * cca_attn_prefill_chunk - the fused attention rows of the covered positions
 *   (digest, "Method", fusion formula), each row t over cores 0 .. n_core(t)-1
 *   (core_k/core_v [B,Hkv,m_cap,d], pooled by earlier chunk calls) and raw
 *   positions win_lo(t) .. t of k/v.  out [B,Hq,Lq,d] in out_dt.  bf16 inputs
 *   run on the matrix cores, fp32 inputs on the vector ALUs.
 * Errors: INVALID_ARG (null or misaligned pointers, Lq or Lk < 1, g or w < 1,
 *   m_cap < 0), UNSUPPORTED as cca_attn_prefill.
 */
cca_status cca_attn_prefill_chunk(const void* q, const void* k, const void* v, const void* core_k,
                                  const void* core_v, int m_cap, void* out, int out_dt,
                                  const int32_t* q_start, const int32_t* q_len, int B, int Hq,
                                  int Hkv, int Lq, int Lk, int d, int g, int w, int dt,
                                  void* stream);

/*
 * cca_cache_fill_ring - prefill -> decode handoff: copies positions
 *   max(0, len-R) .. len-1 of k/v ([B,Hkv,Lk,d]), len = seq_len[b] (device
 *   int32 [B]), into ring slot p % R of ring_k/ring_v ([B,Hkv,R,d]).  With the
 *   cores pooled up to len and pos[b] = len, cca_attn_decode then continues
 *   the sequence.  A len outside 0 .. Lk copies nothing.
 * Errors: INVALID_ARG (null or misaligned pointers, R or Lk < 1), UNSUPPORTED
 *   (d, dt, B*Hkv > 65535).
 */
cca_status cca_cache_fill_ring(const void* k, const void* v, void* ring_k, void* ring_v, int R,
                               const int32_t* seq_len, int B, int Hkv, int Lk, int d, int dt,
                               void* stream);

/*
 * cca_decode_workspace_bytes - size of the workspace cca_attn_decode needs for
 * these shapes (fp32 partial softmax states of its split-K pass).  It takes
 * Hkv and the core capacity m_cap rather than a maximal context length: the
 * split plan depends on the longest visible range, m_cap + w, and on how many
 * (b, kv head) pairs share the GPU.
 */
size_t cca_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int m_cap, int g, int w);

/*
 * cca_attn_decode - one KV-cached decode step for a batch (CCA supports a KV
 * cache natively, per the article).  For batch b the new token has position
 * t = pos[b] (tokens already cached); every sequence may sit at its own t.
 *   q_t [B,Hq,d], k_t/v_t [B,Hkv,d] (dt): the new token's projections.
 *   ring_k/ring_v [B,Hkv,R,d] (dt): raw keys/values, position p in slot p % R;
 *     must hold positions max(0, t-R+1) .. t-1.  R >= max(w, g).
 *   core_k/core_v [B,Hkv,m_cap,d] (cca_core_dtype(dt)): cores of every
 *     completed group.
 *   Enqueued work: (1) k_t/v_t are written to slot t % R; (2) when (t+1) % g
 *   == 0, group (t+1)/g-1 is pooled from positions t-g+1 .. t with the mean
 *   over its G heads of q_t and written to core slot (t+1)/g-1 (it is not yet
 *   visible to t); (3) out[b,h,:] = softmax over the n_core(t) cores and the
 *   raw window win_lo(t) .. t (the same row prefill computes for position t).
 *   out: [B,Hq,d] in out_dt.  workspace: device memory of at least
 *   cca_decode_workspace_bytes(...) bytes, contents need no initialisation.
 *   pos: int32 [B] device array; read, and, when advance_pos != 0,
 *   incremented by one after a valid step, so that a loop of steps needs no
 *   host work and can be captured in a graph.  With advance_pos = 0 pos is
 *   read-only and the caller advances it.  (A read-only pos is the plain
 *   form; the device-side advance is an addition for replayed loops.)
 *   A sequence with t < 0, t = INT32_MAX or floor((t+1)/g) > m_cap (no core
 *   slot left) gets NaN outputs, no cache writes and keeps its pos (pos lives
 *   on the device, so this cannot be reported as a status).  Validity depends
 *   on t alone: NaN inputs at a valid t give NaN outputs and still advance pos.
 * Errors: INVALID_ARG, UNSUPPORTED as above; CAPACITY when R < max(w, g) or
 *   the workspace is too small.
 */
cca_status cca_attn_decode(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                           void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                           int32_t* pos, int advance_pos, void* out, int out_dt,
                           void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int d,
                           int g, int w, int dt, void* stream);

/*
 * cca_attn_decode_ex - cca_attn_decode whose on-completion pooling (step 2)
 * follows the rule `pool_mode` (cca_pool_mode above), so that a decode loop
 * continues a cache built by cca_pool_core_ex with the same rule.
 * Errors: as cca_attn_decode; INVALID_ARG for an unknown mode; UNSUPPORTED
 *   for CCA_POOL_SOFTMAX_HEADS with G > 8.
 */
cca_status cca_attn_decode_ex(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                              void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                              int32_t* pos, int advance_pos, void* out, int out_dt,
                              void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv,
                              int d, int g, int w, int dt, int pool_mode, void* stream);

/*
 * cca_attn_decode_scratch - cca_attn_decode_ex for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * must not call hipMalloc, harnesses that forbid it): the same step, with the
 * split-K states in a fixed device array of the library (cca_decode_scratch_bytes()
 * bytes, 16 MiB) instead of a caller workspace.  Nothing is allocated or freed
 * by this call or by the library.  Each GPU holds its own copy of the array
 * from its first use until the process ends; its address is looked up once
 * per device (the calling thread's current device).  Every call on one GPU
 * shares that array, so calls that overlap on one GPU (other streams, other
 * threads) race: the caller orders them.  The states need no clearing (every
 * call writes all it reads).  q_t .. out, the sizes, dt and pool_mode as
 * cca_attn_decode_ex.
 * Errors: as cca_attn_decode_ex; CAPACITY when the split states of these
 *   shapes (cca_decode_workspace_bytes) exceed the array; HIP when the array's
 *   address cannot be found on the current device.
 */
cca_status cca_attn_decode_scratch(const void* q_t, const void* k_t, const void* v_t, void* ring_k,
                                   void* ring_v, int R, void* core_k, void* core_v, int m_cap,
                                   int32_t* pos, int advance_pos, void* out, int out_dt, int B,
                                   int Hq, int Hkv, int d, int g, int w, int dt, int pool_mode,
                                   void* stream);

/* Size in bytes of the fixed device array cca_attn_decode_scratch uses. */
size_t cca_decode_scratch_bytes(void);

#ifdef __cplusplus
}
#endif

#endif /* CCA_H */
