"""Scalar brute-force form of the CCA oracle, for tiny inputs only.

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over explicit index lists and
``math.exp``, written straight from the set definitions so that it shares no
formula shortcuts with ``cca_oracle`` (which uses the closed form of n_core and
numpy reductions).  The two forms must agree to rounding on every tiny case.

Definitions used (same readings as ``cca_oracle``):
  * group j = tokens jg .. jg+g-1; it exists when all its tokens are < L;
  * query t sees raw positions s with 0 <= s <= t and t - s < w, and every
    group all of whose tokens precede the first raw position it sees
    ([digest], Method, fusion formula; [article], locality-preserving module);
  * a group is scored by the query at its last token, averaged over the query
    heads sharing its kv head ([digest], Method, pooling formula).
"""
from __future__ import annotations

import math


def visible_sets(L: int, g: int, w: int):
    """For each t: (list of visible core indices, list of visible raw positions)."""
    groups = [list(range(j * g, j * g + g)) for j in range(L) if j * g + g <= L]
    out = []
    for t in range(L):
        raw = [s for s in range(0, t + 1) if t - s < w]
        first_raw = raw[0]
        cores = [j for j, members in enumerate(groups) if all(i < first_raw for i in members)]
        out.append((cores, raw))
    return out


def _dot(a, b):
    acc = 0.0
    for x, y in zip(a, b):
        acc += float(x) * float(y)
    return acc


def _softmax_list(s):
    mx = max(s)
    e = [math.exp(x - mx) for x in s]
    tot = sum(e)
    return [x / tot for x in e]


def pool(Q, K, V, g: int, mode: str = "softmax"):
    """Nested lists / arrays indexed [b][h][t][e]; returns CK, CV, A as lists.

    mode "softmax": weights from the softmax of the mean last-token query;
    "softmax_heads": mean over the heads of each head's own softmax;
    "mean": equal weights; "max": element-wise maximum (A holds None)."""
    B, Hq, L, d = len(Q), len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    Hkv = len(K[0])
    G = Hq // Hkv
    CK, CV, A = [], [], []
    for b in range(B):
        ck_b, cv_b, a_b = [], [], []
        for hk in range(Hkv):
            ck_h, cv_h, a_h = [], [], []
            j = 0
            while (j + 1) * g <= L:
                last = (j + 1) * g - 1
                members = list(range(j * g, j * g + g))
                heads = list(range(hk * G, hk * G + G))
                if mode == "max":
                    ck = [max(float(K[b][hk][i][e]) for i in members) for e in range(d)]
                    cv = [max(float(V[b][hk][i][e]) for i in members) for e in range(d)]
                    ck_h.append(ck)
                    cv_h.append(cv)
                    a_h.append(None)
                    j += 1
                    continue
                if mode == "softmax":
                    qbar = [0.0] * d
                    for hq in heads:
                        for e in range(d):
                            qbar[e] += float(Q[b][hq][last][e]) / G
                    a = _softmax_list([_dot(qbar, K[b][hk][i]) / math.sqrt(d) for i in members])
                elif mode == "softmax_heads":
                    a = [0.0] * g
                    for hq in heads:
                        ah = _softmax_list([_dot(Q[b][hq][last], K[b][hk][i]) / math.sqrt(d) for i in members])
                        for n in range(g):
                            a[n] += ah[n] / G
                elif mode == "mean":
                    a = [1.0 / g] * g
                else:
                    raise ValueError(mode)
                ck = [sum(a[n] * float(K[b][hk][i][e]) for n, i in enumerate(members)) for e in range(d)]
                cv = [sum(a[n] * float(V[b][hk][i][e]) for n, i in enumerate(members)) for e in range(d)]
                ck_h.append(ck)
                cv_h.append(cv)
                a_h.append(a)
                j += 1
            ck_b.append(ck_h)
            cv_b.append(cv_h)
            a_b.append(a_h)
        CK.append(ck_b)
        CV.append(cv_b)
        A.append(a_b)
    return CK, CV, A


def attention(Q, K, V, CK, CV, g: int, w: int):
    """O[b][h][t] over the explicit visible sets of ``visible_sets``."""
    B, Hq, L, d = len(Q), len(Q[0]), len(Q[0][0]), len(Q[0][0][0])
    Hkv = len(K[0])
    G = Hq // Hkv
    sets = visible_sets(L, g, w)
    O = []
    for b in range(B):
        o_b = []
        for h in range(Hq):
            hk = h // G
            o_h = []
            for t in range(L):
                cores, raw = sets[t]
                keys = [CK[b][hk][j] for j in cores] + [K[b][hk][s] for s in raw]
                vals = [CV[b][hk][j] for j in cores] + [V[b][hk][s] for s in raw]
                p = _softmax_list([_dot(Q[b][h][t], k) / math.sqrt(d) for k in keys])
                o_h.append([sum(p[n] * float(vals[n][e]) for n in range(len(vals))) for e in range(d)])
            o_b.append(o_h)
        O.append(o_b)
    return O
