"""fp64 CPU oracle of the CCA attention backward pass (gradients of the forward
in ``cca_oracle``).

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path imports this module.

The pages fine-tune pretrained models with CCA attention in place (paper
card, summary and key results: full and partial fine-tuning; rebuttal, answer
on the fine-tuning setting), which needs the gradients of the two steps of the
forward; they print none.  The oracle takes them from the
chain rule, step by step, in the forward's order reversed:

1. Fusion ([digest], Method, fusion formula).  Row t has scores
   S_k = q_t . key_k / sqrt(d) over its visible keys (cores CK_0..CK_{n-1},
   then raw K_lo..K_t), P = softmax(S) and o_t = sum_k P_k value_k.  With an
   upstream gradient dO_t:
       dP_k     = dO_t . value_k
       dS_k     = P_k (dP_k - sum_k' P_k' dP_k')            (softmax Jacobian)
       dq_t     = sum_k dS_k key_k / sqrt(d)
       dkey_k  += dS_k q_t / sqrt(d),   dvalue_k += P_k dO_t
   summed over every row (and query head) that sees key k; a core's
   gradient goes to dCK / dCV.

2. Global-aware pooling ([digest], Method, pooling formula; modes of reading
   R-13).  For group j with weights a (over its g tokens), CK_j = sum a K and
   CV_j = sum a V:
       dK[tau] += a_tau dCK_j,   dV[tau] += a_tau dCV_j
       da_tau   = dCK_j . K[tau] + dCV_j . V[tau]
   and for the softmax rules, a = softmax(s) with s_tau = q . K[tau] / sqrt(d):
       ds_tau   = a_tau (da_tau - sum a da)
       dK[tau] += ds_tau q / sqrt(d),   dq = sum_tau ds_tau K[tau] / sqrt(d),
   where q is the mean of the G heads' last-token queries (rule "softmax":
   each head's query row gets dq / G) or each head's own query with its own
   softmax, averaged over the heads (rule "softmax_heads": the head's a is
   that head's softmax, and its da is divided by G).  Rule "mean" has fixed
   weights 1/g; rule "max" routes each component's gradient to the token that
   holds the maximum (the first one on ties, a reading: R-15).

Each function below computes its row or group on its own, with numpy
products and sums as the only library primitives.
"""
from __future__ import annotations

import math

import numpy as np

from .cca_oracle import _f64, _softmax, group_last, n_core, pool_core, win_lo, attn_prefill


def _scale(d: int) -> float:
    """Score scale of both softmaxes, 1/sqrt(d) (reading R-4)."""
    return 1.0 / math.sqrt(d)


def _softmax_backward(p, dp):
    """Gradient through p = softmax(s) along the last axis: p * (dp - sum p dp)."""
    return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))


def attn_backward(Q, K, V, CK, CV, g: int, w: int, dO):
    """Gradients of the fused prefill (step 1) for upstream dO [B,Hq,L,d].

    Returns dQ [B,Hq,L,d], dK, dV [B,Hkv,L,d] (raw keys/values) and dCK, dCV
    [B,Hkv,m,d] (cores), all fp64; m = CK.shape[2].
    """
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Q, K, V, CK, CV, dO = (_f64(x) for x in (Q, K, V, CK, CV, dO))
    scale = _scale(d)
    dQ = np.zeros_like(Q)
    dK, dV = np.zeros_like(K), np.zeros_like(V)
    dCK, dCV = np.zeros_like(CK), np.zeros_like(CV)
    for t in range(L):
        nc, lo = n_core(t, g, w), win_lo(t, w)
        for h in range(Hq):
            hk = h // G
            for b in range(B):
                keys = np.concatenate([CK[b, hk, :nc], K[b, hk, lo : t + 1]], axis=0)
                vals = np.concatenate([CV[b, hk, :nc], V[b, hk, lo : t + 1]], axis=0)
                q = Q[b, h, t]
                p = _softmax(keys @ q * scale)
                dp = vals @ dO[b, h, t]
                ds = _softmax_backward(p, dp)
                dQ[b, h, t] = ds @ keys * scale
                dkeys = np.outer(ds, q) * scale
                dvals = np.outer(p, dO[b, h, t])
                dCK[b, hk, :nc] += dkeys[:nc]
                dCV[b, hk, :nc] += dvals[:nc]
                dK[b, hk, lo : t + 1] += dkeys[nc:]
                dV[b, hk, lo : t + 1] += dvals[nc:]
    return dQ, dK, dV, dCK, dCV


def attn_backward_rows(Q, K, V, CK, CV, g: int, w: int, dO, rows):
    """Step 1 restricted to the query rows ``rows`` (every batch and head).

    The same chain rule as ``attn_backward``, with the G query heads of a kv
    head handled together by small matrix products, for long sequences where
    only some rows are wanted.  Returns dQ [B,Hq,len(rows),d] of those rows
    and the contributions of those rows alone to dK, dV [B,Hkv,L,d] and dCK,
    dCV [B,Hkv,m,d] (fp64); over all rows it is ``attn_backward``.
    """
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    K, V, CK, CV = (_f64(x) for x in (K, V, CK, CV))
    scale = _scale(d)
    rows = list(rows)
    dQ = np.zeros((B, Hq, len(rows), d))
    dK, dV = np.zeros_like(K), np.zeros_like(V)
    dCK, dCV = np.zeros_like(CK), np.zeros_like(CV)
    T = (0, 1, 3, 2)
    for i, t in enumerate(rows):
        nc, lo = n_core(t, g, w), win_lo(t, w)
        q = _f64(Q[:, :, t]).reshape(B, Hkv, G, d)       # head h -> kv head h // G
        go = _f64(dO[:, :, t]).reshape(B, Hkv, G, d)
        ck, cv = CK[:, :, :nc], CV[:, :, :nc]
        kw, vw = K[:, :, lo : t + 1], V[:, :, lo : t + 1]
        p = _softmax(np.concatenate([q @ ck.transpose(T), q @ kw.transpose(T)], axis=-1) * scale)
        dp = np.concatenate([go @ cv.transpose(T), go @ vw.transpose(T)], axis=-1)
        ds = _softmax_backward(p, dp)                      # [B,Hkv,G,nc + window]
        dQ[:, :, i] = ((ds[..., :nc] @ ck + ds[..., nc:] @ kw) * scale).reshape(B, Hq, d)
        dCK[:, :, :nc] += ds[..., :nc].transpose(T) @ q * scale   # summed over the G heads
        dCV[:, :, :nc] += p[..., :nc].transpose(T) @ go
        dK[:, :, lo : t + 1] += ds[..., nc:].transpose(T) @ q * scale
        dV[:, :, lo : t + 1] += p[..., nc:].transpose(T) @ go
    return dQ, dK, dV, dCK, dCV


def attn_backward_rows_masked(Q, K, V, CK, CV, g: int, w: int, dO, t0: int, t1: int):
    """Step 1 for the consecutive rows t0..t1-1, evaluated together.

    The chain rule of ``attn_backward_rows`` written with a mask, for checking
    every row of a long sequence: each row of the range is scored against the
    cores 0..NC-1 and the raw positions LO..t1-1 (the union of the rows'
    visible sets); keys outside a row's own sets get score -inf, hence P = 0
    and dS = 0, so they neither give to dq nor receive from the row.  Returns
    dQ [B,Hq,t1-t0,d] of the rows, their contributions to the raw keys
    LO..t1-1, dK, dV [B,Hkv,t1-LO,d], and to the cores 0..NC-1, dCK, dCV
    [B,Hkv,NC,d] (summed over the G query heads of each kv head), and LO; fp64.
    """
    B, Hq, _, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    ts = np.arange(t0, t1)
    n = len(ts)
    nc = np.array([n_core(int(t), g, w) for t in ts])
    lo = np.array([win_lo(int(t), w) for t in ts])
    NC, LO = int(nc.max()), int(lo.min())
    scale = _scale(d)
    q = _f64(Q[:, :, t0:t1]).reshape(B, Hkv, G, n, d)      # head h -> kv head h // G
    go = _f64(dO[:, :, t0:t1]).reshape(B, Hkv, G, n, d)
    ck, cv = _f64(CK[:, :, None, :NC]), _f64(CV[:, :, None, :NC])
    kw, vw = _f64(K[:, :, None, LO:t1]), _f64(V[:, :, None, LO:t1])
    sw = lambda x: np.swapaxes(x, -1, -2)
    raw_pos = np.arange(LO, t1)[None, :]
    vis = np.concatenate([np.arange(NC)[None, :] < nc[:, None],
                          (raw_pos >= lo[:, None]) & (raw_pos <= ts[:, None])], axis=-1)
    s = np.concatenate([q @ sw(ck), q @ sw(kw)], axis=-1) * scale
    p = _softmax(np.where(vis, s, -np.inf))                   # one softmax over [cores ; window]
    dp = np.concatenate([go @ sw(cv), go @ sw(vw)], axis=-1)
    ds = _softmax_backward(p, dp)                             # [B,Hkv,G,n,NC + window]
    dQ = ((ds[..., :NC] @ ck + ds[..., NC:] @ kw) * scale).reshape(B, Hq, n, d)
    dCK = (sw(ds[..., :NC]) @ q).sum(axis=2) * scale
    dCV = (sw(p[..., :NC]) @ go).sum(axis=2)
    dK = (sw(ds[..., NC:]) @ q).sum(axis=2) * scale
    dV = (sw(p[..., NC:]) @ go).sum(axis=2)
    return dQ, dK, dV, dCK, dCV, LO


def pool_backward(Q, K, V, g: int, dCK, dCV, mode: str = "softmax"):
    """Gradients of pooling (step 2) for upstream dCK, dCV [B,Hkv,m,d].

    Returns dQ [B,Hq,L,d] (non-zero only at group-end rows of the softmax
    rules), dK, dV [B,Hkv,L,d]; fp64.
    """
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    m = dCK.shape[2]
    Q, K, V, dCK, dCV = (_f64(x) for x in (Q, K, V, dCK, dCV))
    scale = _scale(d)
    dQ = np.zeros_like(Q)
    dK, dV = np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        for hk in range(Hkv):
            heads = range(hk * G, hk * G + G)
            for j in range(m):
                rows = slice(j * g, j * g + g)
                Kg, Vg = K[b, hk, rows], V[b, hk, rows]
                dck, dcv = dCK[b, hk, j], dCV[b, hk, j]
                last = group_last(j, g)
                if mode == "max":
                    # R-15: each component's gradient goes to the first token holding the maximum
                    for e in range(d):
                        dK[b, hk, j * g + int(np.argmax(Kg[:, e])), e] += dck[e]
                        dV[b, hk, j * g + int(np.argmax(Vg[:, e])), e] += dcv[e]
                    continue
                if mode == "mean":
                    dK[b, hk, rows] += dck / g
                    dV[b, hk, rows] += dcv / g
                    continue
                da = Kg @ dck + Vg @ dcv                                      # [g]
                if mode == "softmax":
                    qbar = np.mean([Q[b, h, last] for h in heads], axis=0)
                    a = _softmax(Kg @ qbar * scale)
                    ds = _softmax_backward(a, da)
                    dK[b, hk, rows] += np.outer(a, dck) + np.outer(ds, qbar) * scale
                    dV[b, hk, rows] += np.outer(a, dcv)
                    dq = ds @ Kg * scale
                    for h in heads:
                        dQ[b, h, last] += dq / G
                elif mode == "softmax_heads":
                    a_sum = np.zeros(g)
                    for h in heads:
                        ah = _softmax(Kg @ Q[b, h, last] * scale)
                        a_sum += ah / G
                        dsh = _softmax_backward(ah, da) / G
                        dK[b, hk, rows] += np.outer(dsh, Q[b, h, last]) * scale
                        dQ[b, h, last] += dsh @ Kg * scale
                    dK[b, hk, rows] += np.outer(a_sum, dck)
                    dV[b, hk, rows] += np.outer(a_sum, dcv)
                else:
                    raise ValueError(f"unknown pooling mode {mode!r}")
    return dQ, dK, dV


def backward(Q, K, V, g: int, w: int, dO, mode: str = "softmax"):
    """Gradients of the whole forward (pooling, then fused prefill) w.r.t. Q,
    K and V, for upstream dO: step 1, then step 2 on step 1's core gradients.
    Returns dQ [B,Hq,L,d], dK, dV [B,Hkv,L,d] in fp64."""
    CK, CV, _ = pool_core(Q, K, V, g, mode)
    dQ, dK, dV, dCK, dCV = attn_backward(Q, K, V, CK, CV, g, w, dO)
    pQ, pK, pV = pool_backward(Q, K, V, g, dCK, dCV, mode)
    return dQ + pQ, dK + pK, dV + pV


def loss(Q, K, V, g: int, w: int, dO, mode: str = "softmax") -> float:
    """The scalar whose gradient ``backward`` returns: sum(O * dO)."""
    CK, CV, _ = pool_core(Q, K, V, g, mode)
    return float(np.sum(attn_prefill(Q, K, V, CK, CV, g, w) * _f64(dO)))


def row_lse(Q, K, CK, g: int, w: int):
    """Natural-log log-sum-exp of each row's scores, [B,Hq,L] (the statistic a
    forward pass hands to the backward)."""
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    Q, K, CK = _f64(Q), _f64(K), _f64(CK)
    out = np.empty((B, Hq, L))
    for t in range(L):
        nc, lo = n_core(t, g, w), win_lo(t, w)
        for h in range(Hq):
            keys = np.concatenate([CK[:, h // G, :nc], K[:, h // G, lo : t + 1]], axis=1)
            s = np.einsum("bkd,bd->bk", keys, Q[:, h, t]) / math.sqrt(d)
            mx = s.max(axis=1)
            out[:, h, t] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    return out


__all__ = ["attn_backward", "attn_backward_rows", "pool_backward", "backward", "loss", "row_lse"]
