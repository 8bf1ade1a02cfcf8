"""fp64 CPU oracle of CCA attention: visibility, global-aware pooling, fused softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

What it computes, in the pages' order:

1. Grouping.  Tokens 0..L-1 are cut into non-overlapping groups of ``g``
   consecutive tokens, group ``i`` holding tokens ig..ig+g-1 ([article],
   global-aware pooling paragraph: the sequence is split into non-overlapping
   groups; [digest], Method, pooling formula: index set I_i).  Only complete
   groups exist, m = floor(L/g) of them.

2. Global-aware pooling ([digest], Method, pooling formula; [article]: the
   importance scores come from the query of the group's *last* token against
   all keys of the group; [card], Approach).  For group i:
       s_tau = q_last . K[ig+tau] / sqrt(d),   a = softmax(s),
       core key   CK_i = sum_tau a_tau K[ig+tau],
       core value CV_i = sum_tau a_tau V[ig+tau].
   The pages pool the token representations X and then apply the key/value
   projections, which are shared with the local module ([article]: the two
   modules share the linear transformation parameters).  Because the weights
   sum to one, pooling X and then projecting equals pooling the projected keys
   and values, for any affine projection; the oracle pools the given
   (already projected) K and V.

3. Fusion ([digest], Method, fusion formula; [card], Approach: one softmax over
   both; [article]: the local module guarantees every token attends to at least
   the previous w raw tokens).  Query t attends, with ONE softmax, to the
   concatenation [visible core tokens ; raw keys of the local window]:
       o_t = softmax(q_t [CK_T ; K_U]^T / sqrt(d)) [CV_T ; V_U].

Readings of what the pages leave open (each is a choice, stated once here):
  R-1  Groups start at token 0; a trailing partial group (L mod g != 0) has no
       core token; its tokens are reached only through the window.
  R-2  Visibility sets (the fusion formula names them but never defines them):
       U_t = raw positions max(0, t-w+1) .. t (w tokens including t itself);
       T_t = cores j whose last token (j+1)g-1 < t-w+1, i.e. groups lying
       wholly before the window.  Hence n_core(t) = max(0, floor((t-w+1)/g)).
       Up to g-1 tokens between the last visible core and the window are seen
       by neither module; nothing is seen twice.
  R-3  "Last token of group i" is 0-indexed row (i+1)g-1.
  R-4  d is the head dimension; both softmaxes scale by 1/sqrt(d).
  R-5  K and V are pooled after projection and rotation (they arrive that way).
  R-7  g >= 1 and w >= 1; the visible set always holds t itself.
  R-8  GQA (the rebuttal, answer on GQA, says pooling "may need adjusting";
       no rule is given): one core pair per (kv head, group); the pooling
       query is the mean of the group's last-token queries over the G query
       heads that share the kv head.  PARITY UNPINNED by the pages: pinned
       only by the G = 1 reduction and by "G identical heads == one head".
  R-9  Query head h reads kv head floor(h / G).
  R-13 Pooling variants.  The rebuttal (answer on Table 3) names max pooling
       and mean pooling as ablation alternatives to global-aware pooling,
       without formulas.  Plainest reading: over the g tokens of a group, the
       element-wise maximum (mode "max") or the arithmetic mean (mode
       "mean") of K and of V, each taken separately.  The rebuttal's GQA
       answer leaves the rule open; besides R-8 (mode "softmax", the default)
       the oracle offers the other plain rule, the mean over the G query heads
       of each head's own pooling softmax (mode "softmax_heads").  These
       modes are pinned by brute force, by their reductions to one another
       and by invariants; the pages fix none of their values (PARITY
       UNPINNED by the pages, like R-8).
  R-10 Decode row t is prefill row t of the sequence extended to t+1 tokens;
       the core of a group that completes at t is pooled with q_t and is not
       visible to t itself.

Arithmetic: every value is widened to float64 (bf16 and fp32 widen exactly)
and nothing is rounded back.  Each output row is computed on its own from its
own index sets; numpy matrix-vector products and reductions are the only
library primitives.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------- visibility


def win_lo(t: int, w: int) -> int:
    """First raw position of the local window of query t (reading R-2)."""
    return max(0, t - w + 1)


def n_core(t: int, g: int, w: int) -> int:
    """Number of cores visible to query t: groups wholly before the window (R-2)."""
    return max(0, (t - w + 1) // g) if t - w + 1 > 0 else 0


def group_last(j: int, g: int) -> int:
    """Index of the last token of group j, whose query scores the group (R-3)."""
    return (j + 1) * g - 1


def visibility(L: int, g: int, w: int):
    """Integer tables: n_core[L], win_lo[L], group_last[floor(L/g)] (int64)."""
    t = np.arange(L, dtype=np.int64)
    lo = np.maximum(0, t - w + 1)
    nc = np.where(t - w + 1 > 0, (t - w + 1) // g, 0)
    gl = (np.arange(L // g, dtype=np.int64) + 1) * g - 1
    return nc, lo, gl


def visible_pairs_total(L: int, g: int, w: int) -> int:
    """Sum over queries t < L of the number of visible keys (cores + window)."""
    nc, lo, _ = visibility(L, g, w)
    return int(nc.sum() + (np.arange(L) - lo + 1).sum())


def cache_tokens(L: int, g: int, w: int) -> int:
    """Tokens a decoder must keep after L tokens: every complete core plus the
    last w raw tokens ([rebuttal], answer on 128K contexts, gives the KV cache
    of LLaMA2-7B at 128K as 4.5 GB against 64 GB for full attention)."""
    return L // g + min(w, L)


# ----------------------------------------------------------------- helpers


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Max-subtracted softmax along ``axis`` (masked entries are -inf)."""
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


# ------------------------------------------------------------------- pooling


POOL_MODES = ("softmax", "softmax_heads", "mean", "max")


def pool_core(Q, K, V, g: int, mode: str = "softmax"):
    """Global-aware pooling ([digest], Method, pooling formula) and the
    variants of R-13 (``mode``).

    Q [B,Hq,L,d]; K, V [B,Hkv,L,d] (any float dtype; widened to fp64).
    Returns CK, CV [B,Hkv,m,d] and the pooling weights A [B,Hkv,m,g], m = L//g
    (NaN for mode "max", which has no weights).
    """
    B, Hq, L, d = Q.shape
    m = L // g
    last = np.array([group_last(j, g) for j in range(m)], dtype=np.int64)
    # query of each group's last token, one per query head: [B,Hq,m,d]
    return pool_from_last(Q[:, :, last, :], K, V, g, mode)


def pool_from_last(q_last, K, V, g: int, mode: str = "softmax"):
    """Pooling given the last-token query rows: q_last[:, h, j] is the query of
    head h at token (j+1)g-1.  Same outputs as ``pool_core``."""
    if mode not in POOL_MODES:
        raise ValueError(f"unknown pooling mode {mode!r}")
    B, Hq, m, d = q_last.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    if m == 0:
        z = np.zeros((B, Hkv, 0, d))
        return z, z.copy(), np.zeros((B, Hkv, 0, g))
    CK = np.empty((B, Hkv, m, d))
    CV = np.empty((B, Hkv, m, d))
    A = np.empty((B, Hkv, m, g))
    for b in range(B):
        for hk in range(Hkv):
            # R-8: one pooling query per kv head = mean over its G query heads
            q_bar = _f64(q_last[b, hk * G : hk * G + G]).mean(axis=0)         # [m, d]
            Kg = _f64(K[b, hk, : m * g, :]).reshape(m, g, d)                  # group i = rows ig..ig+g-1
            Vg = _f64(V[b, hk, : m * g, :]).reshape(m, g, d)
            if mode == "max":                                                 # R-13
                A[b, hk] = np.nan
                CK[b, hk] = Kg.max(axis=1)
                CV[b, hk] = Vg.max(axis=1)
                continue
            if mode == "softmax":
                s = (Kg * q_bar[:, None, :]).sum(axis=-1) / math.sqrt(d)      # [m, g]
                a = _softmax(s, axis=-1)
            elif mode == "softmax_heads":                                     # R-13: mean of per-head softmaxes
                qs = _f64(q_last[b, hk * G : hk * G + G])                     # [G, m, d]
                s = (Kg[None] * qs[:, :, None, :]).sum(axis=-1) / math.sqrt(d)  # [G, m, g]
                a = _softmax(s, axis=-1).mean(axis=0)
            else:                                                             # "mean"
                a = np.full((m, g), 1.0 / g)
            A[b, hk] = a
            CK[b, hk] = (a[:, :, None] * Kg).sum(axis=1)
            CV[b, hk] = (a[:, :, None] * Vg).sum(axis=1)
    return CK, CV, A


# ------------------------------------------------------------------- fusion


def attn_rows(Q, K, V, CK, CV, g: int, w: int, ts):
    """Fused attention rows ([digest], Method, fusion formula) for positions ts.

    Q [B,Hq,L,d]; K, V [B,Hkv,L,d]; CK, CV [B,Hkv,>=n_core(max ts),d].
    Returns O [B,Hq,len(ts),d] in fp64.
    """
    ts = list(ts)
    return attn_rows_q(Q[:, :, ts, :], K, V, CK, CV, g, w, ts)


def attn_rows_q(qrows, K, V, CK, CV, g: int, w: int, ts):
    """As ``attn_rows`` with the query rows given: qrows[:, :, i] sits at ts[i].

    Each row t uses its own index sets: cores 0..n_core(t)-1 and raw positions
    win_lo(t)..t; the scores of both parts are concatenated and go through ONE
    softmax, and the output is the probability-weighted sum of both parts'
    values.
    """
    B, Hq, _, d = qrows.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    out = np.empty((B, Hq, len(ts), d))
    scale = 1.0 / math.sqrt(d)
    for i, t in enumerate(ts):
        nc, lo = n_core(t, g, w), win_lo(t, w)
        q = _f64(qrows[:, :, i, :]).reshape(B, Hkv, G, d)       # R-9: head h -> kv head h//G
        ck, cv = _f64(CK[:, :, :nc, :]), _f64(CV[:, :, :nc, :])
        kw, vw = _f64(K[:, :, lo : t + 1, :]), _f64(V[:, :, lo : t + 1, :])
        s = np.concatenate([q @ ck.transpose(0, 1, 3, 2), q @ kw.transpose(0, 1, 3, 2)], axis=-1) * scale
        p = _softmax(s, axis=-1)                                  # one softmax over [cores ; window]
        o = p[..., :nc] @ cv + p[..., nc:] @ vw
        out[:, :, i, :] = o.reshape(B, Hq, d)
    return out


def attn_rows_masked(Q, K, V, CK, CV, g: int, w: int, t0: int, t1: int):
    """Rows t0..t1-1 (consecutive) of ``attn_rows`` evaluated together.

    The same definition written with a mask, for checking many rows at once:
    every row of the range is scored against the cores 0..n_core(t1-1)-1 and
    the raw positions win_lo(t0)..t1-1 (the union of the rows' visible sets),
    the scores of keys outside the row's own sets (core j >= n_core(t); raw
    position p < win_lo(t) or p > t) are set to -inf, and ONE softmax over
    [cores ; raw] weights the matching values.  Masked keys get probability
    exactly zero, so each row equals ``attn_rows`` for that row.
    Returns O [B,Hq,t1-t0,d] in fp64.
    """
    B, Hq, _, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    ts = np.arange(t0, t1)
    nc = np.array([n_core(int(t), g, w) for t in ts])
    lo = np.array([win_lo(int(t), w) for t in ts])
    NC, LO = int(nc.max()), int(lo.min())
    q = _f64(Q[:, :, t0:t1, :]).reshape(B, Hkv, G, len(ts), d)      # R-9: head h -> kv head h//G
    ck, cv = _f64(CK[:, :, None, :NC, :]), _f64(CV[:, :, None, :NC, :])
    kw, vw = _f64(K[:, :, None, LO:t1, :]), _f64(V[:, :, None, LO:t1, :])
    scale = 1.0 / math.sqrt(d)
    sc = (q @ np.swapaxes(ck, -1, -2)) * scale                      # [B,Hkv,G,n,NC]
    sr = (q @ np.swapaxes(kw, -1, -2)) * scale                      # [B,Hkv,G,n,t1-LO]
    core_vis = np.arange(NC)[None, :] < nc[:, None]
    raw_pos = np.arange(LO, t1)[None, :]
    raw_vis = (raw_pos >= lo[:, None]) & (raw_pos <= ts[:, None])
    s = np.concatenate([np.where(core_vis, sc, -np.inf), np.where(raw_vis, sr, -np.inf)], axis=-1)
    p = _softmax(s, axis=-1)                                          # one softmax over [cores ; window]
    o = p[..., :NC] @ cv + p[..., NC:] @ vw
    return o.reshape(B, Hq, len(ts), d)


def attn_prefill(Q, K, V, CK, CV, g: int, w: int):
    """All L rows of causal prefill (see ``attn_rows``)."""
    return attn_rows(Q, K, V, CK, CV, g, w, range(Q.shape[2]))


def attn_row(Q, K, V, CK, CV, g: int, w: int, t: int):
    """Row t for every (batch, query head): O [B,Hq,d]."""
    return attn_rows(Q, K, V, CK, CV, g, w, [t])[:, :, 0, :]


def attn_decode(q_t, K_seq, V_seq, CK, CV, pos, g: int, w: int):
    """One decode step (R-10): for batch b the new token sits at position pos[b].

    q_t [B,Hq,d]; K_seq, V_seq [B,Hkv,T,d] hold every token up to and including
    pos[b] for each b; CK, CV [B,Hkv,>=n_core(pos[b]),d] are the cores of the
    completed groups of that sequence.  Row pos[b] of prefill over the extended
    sequence is exactly this; returns [B,Hq,d] in fp64.
    """
    B, Hq, d = q_t.shape
    out = np.empty((B, Hq, d))
    for b in range(B):
        t = int(pos[b])
        out[b] = attn_rows_q(q_t[b : b + 1, :, None, :], K_seq[b : b + 1], V_seq[b : b + 1],
                             CK[b : b + 1], CV[b : b + 1], g, w, [t])[0, :, 0, :]
    return out
