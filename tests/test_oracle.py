"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

CPU only.  Each pin is a plain function returning a list of failure strings
(empty = pass), so that ``test_planted_mistakes_are_caught`` can re-run every
pin against copies of the oracle with one plausible mistake planted in each
and show that some pin fails for every one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest
import torch

import cca_inputs
import oracle.cca_oracle as orc
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, shape, scale=1.0):
    return cca_inputs.normal_f32(seed, shape, scale).astype(np.float64)


def _close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return f"shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    return None if err <= tol else f"max abs err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ pins


def pin_visibility_vs_sets(o):
    """Closed-form n_core / win_lo equal the explicit set definitions."""
    fails = []
    for L, g, w in [(1, 1, 1), (7, 2, 3), (40, 3, 5), (64, 4, 4), (53, 5, 9), (33, 16, 1),
                    (50, 1, 7), (20, 7, 30), (45, 6, 2)]:
        sets = brute.visible_sets(L, g, w)
        nc, lo, gl = o.visibility(L, g, w)
        for t in range(L):
            cores, raw = sets[t]
            if nc[t] != len(cores) or cores != list(range(len(cores))):
                fails.append(f"n_core L={L} g={g} w={w} t={t}: {nc[t]} vs {len(cores)}")
            if lo[t] != raw[0] or len(raw) != t - lo[t] + 1:
                fails.append(f"win_lo L={L} g={g} w={w} t={t}: {lo[t]} vs {raw[0]}")
            if o.n_core(t, g, w) != nc[t] or o.win_lo(t, w) != lo[t]:
                fails.append(f"scalar/table mismatch at t={t}")
        if list(gl) != [j * g + g - 1 for j in range(L // g)]:
            fails.append(f"group_last L={L} g={g}")
    return fails


def _pairs_closed_form(L, g, w):
    # window: min(w, t+1) keys per row; cores: sum_{u=0}^{L-w} floor(u/g)
    win = sum(min(w, t + 1) for t in range(min(L, w))) + max(0, L - w) * w
    N = L - w
    core = 0
    if N >= 0:
        q, r = divmod(N + 1, g)
        core = g * q * (q - 1) // 2 + r * q
    return win + core


def pin_pair_counts(o):
    """Total visible pairs: table sum == arithmetic-series closed form, and the
    per-head totals of the five workloads."""
    fails = []
    expect = {(1024, 16, 64): 91_900, (32768, 16, 1024): 64_506_816, (131072, 16, 1024): 662_152_128}
    for (L, g, w), n in expect.items():
        got = o.visible_pairs_total(L, g, w)
        cf = _pairs_closed_form(L, g, w)
        if got != n or cf != n:
            fails.append(f"pairs L={L}: table {got}, closed form {cf}, expected {n}")
    for L, g, w in [(1, 1, 1), (10, 3, 4), (100, 7, 13), (5, 16, 64)]:
        if o.visible_pairs_total(L, g, w) != _pairs_closed_form(L, g, w):
            fails.append(f"pairs L={L} g={g} w={w}")
    return fails


def pin_kv_cache_size(o):
    """The rebuttal's 128K KV-cache figure (4.5 GB vs 64 GB, LLaMA2-7B) and the
    article's 'up to 93%' follow from 'every complete core + w raw tokens'."""
    with open(os.path.join(GOLDEN, "kv_cache_128k.json")) as f:
        gold = json.load(f)
    per_tok = gold["layers"] * gold["heads"] * gold["head_dim"] * 2 * gold["bytes_per_value"]
    L = gold["context_tokens"]
    cca = o.cache_tokens(L, gold["g"], gold["w"]) * per_tok / 2**30
    full = L * per_tok / 2**30
    fails = []
    if abs(cca - gold["cca_kv_cache_GB"]) > 1e-9 or abs(full - gold["vanilla_kv_cache_GB"]) > 1e-9:
        fails.append(f"cache {cca} GiB vs {gold['cca_kv_cache_GB']}, full {full}")
    if round(100 * (1 - cca / full)) != gold["kv_reduction_percent_up_to"]:
        fails.append("reduction percent")
    return fails


def pin_pool_worked_example(o):
    """Hand-computed: d=4, g=2, q=(2,0,0,0), k0=(1,0,0,0), k1=0 ->
    scores (2*1/sqrt(4), 0) = (1, 0), weights (e/(e+1), 1/(e+1))."""
    Q = np.zeros((1, 1, 2, 4))
    Q[0, 0, 1] = [2, 0, 0, 0]              # last token of group 0 scores the group
    Q[0, 0, 0] = [-50, 3, 0, 0]            # first token must not matter
    K = np.zeros((1, 1, 2, 4))
    K[0, 0, 0] = [1, 0, 0, 0]
    V = np.zeros((1, 1, 2, 4))
    V[0, 0, 0] = [1, 0, 0, 0]
    V[0, 0, 1] = [0, 1, 0, 0]
    CK, CV, A = o.pool_core(Q, K, V, 2)
    a0 = math.e / (math.e + 1.0)
    fails = []
    for name, got, want in [("A", A[0, 0, 0], [a0, 1 - a0]), ("CK", CK[0, 0, 0], [a0, 0, 0, 0]),
                            ("CV", CV[0, 0, 0], [a0, 1 - a0, 0, 0])]:
        e = _close(got, want, 1e-15)
        if e:
            fails.append(f"worked example {name}: {e}")
    return fails


def pin_pool_invariants(o):
    """Weights sum to 1; identical keys -> that key; zero query -> group mean;
    joint permutation inside a group; g=1 -> CK=K; the last token's query
    selects; pooling commutes with any affine projection (pages: X is pooled,
    then projected with the shared W^K/W^V)."""
    fails = []
    B, Hq, Hkv, L, d, g = 2, 4, 2, 48, 8, 4
    Q, K, V = _rand(11, (B, Hq, L, d)), _rand(12, (B, Hkv, L, d)), _rand(13, (B, Hkv, L, d))
    CK, CV, A = o.pool_core(Q, K, V, g)
    if A.shape != (B, Hkv, L // g, g):
        return [f"weights shape {A.shape}"]
    if np.max(np.abs(A.sum(-1) - 1)) > 1e-12 or A.min() < 0:
        fails.append("weights do not sum to 1")
    # identical keys in a group -> CK equals that key (uniform weights)
    K2 = K.copy()
    K2[:, :, 4:8] = K2[:, :, 4:5]
    CK2, _, A2 = o.pool_core(Q, K2, V, g)
    e = _close(CK2[:, :, 1], K2[:, :, 4], 1e-12) or _close(A2[:, :, 1], np.full((B, Hkv, g), 0.25), 1e-12)
    if e:
        fails.append(f"identical keys: {e}")
    # zero pooling query -> mean pooling
    Qz = Q.copy()
    Qz[:, :, g - 1 :: g] = 0
    CKz, CVz, _ = o.pool_core(Qz, K, V, g)
    e = _close(CKz, K.reshape(B, Hkv, L // g, g, d).mean(3), 1e-12) or \
        _close(CVz, V.reshape(B, Hkv, L // g, g, d).mean(3), 1e-12)
    if e:
        fails.append(f"zero query mean pooling: {e}")
    # joint permutation of (k, v) inside each group
    perm = np.concatenate([np.random.default_rng(5).permutation(g) + j * g for j in range(L // g)])
    CKp, CVp, _ = o.pool_core(Q, K[:, :, perm], V[:, :, perm], g)
    e = _close(CKp, CK, 1e-12) or _close(CVp, CV, 1e-12)
    if e:
        fails.append(f"permutation: {e}")
    # g = 1 -> cores are the tokens themselves
    CK1, CV1, _ = o.pool_core(Q, K, V, 1)
    e = _close(CK1, K, 1e-12) or _close(CV1, V, 1e-12)
    if e:
        fails.append(f"g=1: {e}")
    # the LAST token's query selects: set it to 40 * k_tau* for one group
    Qs, tau = Q.copy(), 2
    for h in range(Hq):
        Qs[:, h, 2 * g + g - 1] = 40.0 * K[:, h // (Hq // Hkv), 2 * g + tau]
    CKs, CVs, As = o.pool_core(Qs, K, V, g)
    if np.min(As[:, :, 2, tau]) < 0.999:
        fails.append(f"last-token query does not select key tau: {As[:, :, 2]}")
    e = _close(CVs[:, :, 2], V[:, :, 2 * g + tau], 2e-2)
    if e:
        fails.append(f"selected value: {e}")
    # only the last token's query matters
    Qn = Q.copy()
    Qn[:, :, 0 : L : g] += 5.0
    CKn, _, _ = o.pool_core(Qn, K, V, g)
    if _close(CKn, CK, 1e-12):
        fails.append("pooling reads a query other than the group's last")
    # affine projection commutes with pooling
    W = _rand(14, (d, d))
    bias = _rand(15, (d,))
    X = _rand(16, (B, Hkv, L, d))
    Kx = X @ W + bias
    CKx, CVx, Ax = o.pool_core(Q, Kx, X, g)
    e = _close(CKx, CVx @ W + bias, 1e-10)
    if e:
        fails.append(f"pooling then projection: {e}")
    # trailing partial group has no core
    CKt, _, _ = o.pool_core(Q[:, :, : L - 3], K[:, :, : L - 3], V[:, :, : L - 3], g)
    if CKt.shape[2] != (L - 3) // g:
        fails.append("partial group produced a core")
    return fails


def pin_pool_gqa(o):
    """GQA reading: with G identical query heads the cores equal those of one
    head (MHA); the pooling query is the mean of the G heads' queries."""
    fails = []
    B, Hkv, L, d, g, G = 1, 2, 32, 8, 4, 3
    Q1 = _rand(21, (B, Hkv, L, d))
    K, V = _rand(22, (B, Hkv, L, d)), _rand(23, (B, Hkv, L, d))
    Qg = np.repeat(Q1, G, axis=1)
    a = o.pool_core(Q1, K, V, g)
    b = o.pool_core(Qg, K, V, g)
    for x, y in zip(a, b):
        e = _close(x, y, 1e-12)
        if e:
            fails.append(f"identical heads: {e}")
    # mean of queries: heads (q + r, q - r) pool like a single head q
    R = _rand(24, (B, Hkv, L, d))
    Qpm = np.stack([Q1 + R, Q1 - R], axis=2).reshape(B, 2 * Hkv, L, d)
    c = o.pool_core(Qpm, K, V, g)
    for x, y in zip(a, c):
        e = _close(x, y, 1e-12)
        if e:
            fails.append(f"mean query: {e}")
    return fails


def _sdpa_causal(Q, K, V):
    G = Q.shape[1] // K.shape[1]
    q = torch.from_numpy(Q)
    k = torch.from_numpy(K).repeat_interleave(G, dim=1)
    v = torch.from_numpy(V).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).numpy()


def pin_reduces_to_full_causal(o):
    """g=1 or w>=L: exactly full causal softmax attention (torch's SDPA, fp64)."""
    fails = []
    for B, Hq, Hkv, L, d, g, w in [(1, 2, 2, 37, 8, 1, 5), (2, 4, 2, 50, 16, 1, 1), (1, 2, 1, 40, 8, 3, 40),
                                   (1, 3, 3, 29, 4, 16, 64), (1, 2, 2, 64, 8, 1, 64)]:
        Q = _rand(31, (B, Hq, L, d))
        K, V = _rand(32, (B, Hkv, L, d)), _rand(33, (B, Hkv, L, d))
        CK, CV, _ = o.pool_core(Q, K, V, g)
        O = o.attn_prefill(Q, K, V, CK, CV, g, w)
        e = _close(O, _sdpa_causal(Q, K, V), 1e-12)
        if e:
            fails.append(f"full causal g={g} w={w} L={L}: {e}")
    return fails


def pin_visible_set_one_hot(o):
    """With q = 0 every visible key gets weight 1/n_vis; one-hot values then
    reveal exactly which cores and raw tokens each row sees."""
    fails = []
    for L, g, w in [(30, 4, 5), (25, 3, 1), (40, 5, 12), (17, 2, 2)]:
        m = L // g
        D = L + m
        Q = np.zeros((1, 1, L, D))
        K = _rand(41, (1, 1, L, D))
        V = np.zeros((1, 1, L, D))
        V[0, 0, np.arange(L), np.arange(L)] = 1.0
        CK = _rand(42, (1, 1, m, D))
        CV = np.zeros((1, 1, m, D))
        CV[0, 0, np.arange(m), L + np.arange(m)] = 1.0
        O = o.attn_prefill(Q, K, V, CK, CV, g, w)
        sets = brute.visible_sets(L, g, w)
        for t in range(L):
            cores, raw = sets[t]
            want = np.zeros(D)
            n = len(cores) + len(raw)
            want[raw] = 1.0 / n
            want[[L + j for j in cores]] = 1.0 / n
            e = _close(O[0, 0, t], want, 1e-14)
            if e:
                fails.append(f"one-hot L={L} g={g} w={w} t={t}: {e}")
                break
    return fails


def pin_brute_force(o):
    """Oracle == pure-Python brute force on tiny grids (incl. ragged L, GQA)."""
    fails = []
    cases = [(1, 1, 1, 1, 4, 1, 1), (1, 2, 1, 23, 4, 3, 5), (2, 4, 2, 19, 8, 4, 4), (1, 2, 2, 40, 4, 16, 6),
             (1, 3, 1, 33, 6, 2, 1), (1, 1, 1, 26, 5, 5, 30)]
    for B, Hq, Hkv, L, d, g, w in cases:
        Q = _rand(51 + L, (B, Hq, L, d))
        K, V = _rand(52 + L, (B, Hkv, L, d)), _rand(53 + L, (B, Hkv, L, d))
        CK, CV, A = o.pool_core(Q, K, V, g)
        bk, bv, ba = brute.pool(Q.tolist(), K.tolist(), V.tolist(), g)
        m = L // g
        if m:
            for x, y, name in [(CK, bk, "CK"), (CV, bv, "CV"), (A, ba, "A")]:
                e = _close(x, np.array(y), 1e-12)
                if e:
                    fails.append(f"pool {name} {B, Hq, Hkv, L, d, g, w}: {e}")
        O = o.attn_prefill(Q, K, V, CK, CV, g, w)
        bo = brute.attention(Q.tolist(), K.tolist(), V.tolist(),
                             CK.tolist() if m else [[[] for _ in range(Hkv)] for _ in range(B)],
                             CV.tolist() if m else [[[] for _ in range(Hkv)] for _ in range(B)], g, w)
        e = _close(O, np.array(bo), 1e-12)
        if e:
            fails.append(f"attention {B, Hq, Hkv, L, d, g, w}: {e}")
    return fails


def pin_convex_hull(o):
    """Each output lies inside the componentwise hull of the visible values."""
    fails = []
    B, Hq, Hkv, L, d, g, w = 1, 2, 1, 60, 8, 4, 9
    Q = _rand(61, (B, Hq, L, d), 3.0)
    K, V = _rand(62, (B, Hkv, L, d)), _rand(63, (B, Hkv, L, d))
    CK, CV, _ = o.pool_core(Q, K, V, g)
    O = o.attn_prefill(Q, K, V, CK, CV, g, w)
    for t in range(L):
        nc, lo = o.n_core(t, g, w), o.win_lo(t, w)
        vals = np.concatenate([CV[0, 0, :nc], V[0, 0, lo : t + 1]], 0)
        for h in range(Hq):
            if np.any(O[0, h, t] < vals.min(0) - 1e-12) or np.any(O[0, h, t] > vals.max(0) + 1e-12):
                fails.append(f"hull t={t} h={h}")
    return fails


def pin_decode_is_prefill_row(o):
    """A decode step at position t equals prefill row t of the extended
    sequence, with cores pooled by each group's last query (incl. groups that
    complete at the step itself, which are not yet visible)."""
    fails = []
    B, Hq, Hkv, d, g, w, T = 3, 4, 2, 8, 4, 6, 45
    Q = _rand(71, (B, Hq, T, d))
    K, V = _rand(72, (B, Hkv, T, d)), _rand(73, (B, Hkv, T, d))
    CK, CV, _ = o.pool_core(Q, K, V, g)
    O = o.attn_prefill(Q, K, V, CK, CV, g, w)
    for pos in ([10, 11, 12], [44, 7, 23], [0, 5, 39]):
        dec = o.attn_decode(Q[np.arange(B), :, pos], K, V, CK, CV, np.array(pos), g, w)
        e = _close(dec, O[np.arange(B), :, pos], 1e-12)
        if e:
            fails.append(f"decode pos={pos}: {e}")
    return fails


def pin_pool_modes(o):
    """Pooling variants (reading R-13): each mode against the scalar brute
    force; their reductions to one another; and invariants that fix them."""
    fails = []
    B, Hq, Hkv, L, d, g = 2, 6, 2, 22, 5, 4
    Q = _rand(81, (B, Hq, L, d), 2.0)
    K, V = _rand(82, (B, Hkv, L, d)), _rand(83, (B, Hkv, L, d))
    m = L // g
    for mode in ("softmax", "softmax_heads", "mean", "max"):
        ck, cv, a = o.pool_core(Q, K, V, g, mode)
        bk, bv, ba = brute.pool(Q, K, V, g, mode)
        for name, x, y in (("CK", ck, bk), ("CV", cv, bv)):
            e = _close(x, np.array(y), 1e-12)
            if e:
                fails.append(f"{mode} {name} vs brute force: {e}")
        if mode != "max":
            e = _close(a, np.array(ba), 1e-12)
            if e:
                fails.append(f"{mode} weights vs brute force: {e}")
            if np.any(a < 0) or _close(a.sum(-1), np.ones((B, Hkv, m)), 1e-12):
                fails.append(f"{mode} weights are not a distribution")
    # mean pooling is softmax pooling with a zero query (equal scores)
    e = _close(o.pool_core(Q, K, V, g, "mean")[0], o.pool_core(np.zeros_like(Q), K, V, g, "softmax")[0], 1e-12)
    if e:
        fails.append(f"mean != softmax with zero query: {e}")
    # one query head per kv head: the two softmax rules coincide
    Q1 = Q[:, :Hkv]
    e = _close(o.pool_core(Q1, K, V, g, "softmax_heads")[0], o.pool_core(Q1, K, V, g, "softmax")[0], 1e-12)
    if e:
        fails.append(f"softmax_heads != softmax at G=1: {e}")
    # G identical heads: both rules equal the single-head pooling
    Qrep = np.repeat(Q1, 3, axis=1)
    for mode in ("softmax", "softmax_heads"):
        e = _close(o.pool_core(Qrep, K, V, g, mode)[0], o.pool_core(Q1, K, V, g, "softmax")[0], 1e-12)
        if e:
            fails.append(f"{mode} with identical heads: {e}")
    # different heads: the two rules differ (softmax is not linear in its logits)
    if _close(o.pool_core(Q, K, V, g, "softmax_heads")[0], o.pool_core(Q, K, V, g, "softmax")[0], 1e-6) is None:
        fails.append("softmax_heads equals softmax for distinct heads")
    # max: every member is below the result, and each component is attained
    ck, cv, _ = o.pool_core(Q, K, V, g, "max")
    Kg = K[:, :, : m * g].reshape(B, Hkv, m, g, d)
    Vg = V[:, :, : m * g].reshape(B, Hkv, m, g, d)
    for name, x, grp in (("CK", ck, Kg), ("CV", cv, Vg)):
        if np.any(grp > x[:, :, :, None, :]):
            fails.append(f"max {name}: a member exceeds the pooled value")
        if not np.all(np.any(grp == x[:, :, :, None, :], axis=3)):
            fails.append(f"max {name}: a pooled component is not attained")
    # a group of identical tokens pools to that token in every mode; a joint
    # permutation of the tokens inside each group changes nothing
    Kc = np.repeat(K[:, :, ::g][:, :, :m], g, axis=2)
    Vc = np.repeat(V[:, :, ::g][:, :, :m], g, axis=2)
    perm = np.concatenate([j * g + np.roll(np.arange(g), 1) for j in range(m)] + [np.arange(m * g, L)])
    Qp = Q.copy()
    Qp[:, :, perm] = Q  # keep each group's last-token query where the pooling looks for it
    Qp[:, :, [j * g + g - 1 for j in range(m)]] = Q[:, :, [j * g + g - 1 for j in range(m)]]
    for mode in ("softmax", "softmax_heads", "mean", "max"):
        e = _close(o.pool_core(Q[:, :, : m * g], Kc, Vc, g, mode)[0], Kc[:, :, ::g], 1e-12)
        if e:
            fails.append(f"{mode}: identical tokens: {e}")
        base = o.pool_core(Q, K, V, g, mode)
        permd = o.pool_core(Q, K[:, :, perm], V[:, :, perm], g, mode)
        for x, y in zip(base[:2], permd[:2]):
            e = _close(x, y, 1e-12)
            if e:
                fails.append(f"{mode}: permutation inside groups: {e}")
    return fails


def pin_masked_rows_form(o):
    """The masked multi-row form (used to check consecutive rows at full
    size) equals the per-row form on every row, for ranges that start and end
    anywhere: GQA, MHA, g = 1, g > w, w >= L, rows before the first core."""
    fails = []
    cases = [(2, 4, 2, 70, 8, 3, 5, 13), (1, 8, 2, 64, 16, 4, 16, 9), (1, 2, 2, 40, 8, 1, 7, 6),
             (1, 3, 1, 33, 8, 40, 60, 33), (1, 4, 1, 90, 8, 5, 12, 128), (1, 2, 1, 50, 8, 6, 2, 7)]
    for i, (B, Hq, Hkv, L, d, g, w, n) in enumerate(cases):
        Q, K, V = _rand(900 + i, (B, Hq, L, d)), _rand(910 + i, (B, Hkv, L, d)), _rand(920 + i, (B, Hkv, L, d))
        CK, CV, _ = o.pool_core(Q, K, V, g)
        ref = o.attn_rows(Q, K, V, CK, CV, g, w, range(L))
        got = np.concatenate([o.attn_rows_masked(Q, K, V, CK, CV, g, w, t0, min(L, t0 + n))
                              for t0 in range(0, L, n)], axis=2)
        e = _close(got, ref, 1e-12)
        if e:
            fails.append(f"B={B} Hq={Hq} Hkv={Hkv} L={L} g={g} w={w} rows of {n}: {e}")
    return fails


PINS = [pin_visibility_vs_sets, pin_pair_counts, pin_kv_cache_size, pin_pool_worked_example,
        pin_pool_invariants, pin_pool_gqa, pin_reduces_to_full_causal, pin_visible_set_one_hot,
        pin_brute_force, pin_convex_hull, pin_decode_is_prefill_row, pin_pool_modes, pin_masked_rows_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    fails = pin(orc)
    assert not fails, "\n".join(fails[:10])


# ---------------------------------------------------- planted mistakes (CPU)


MUTATIONS = {
    "pool query = first token of group": ("group_last", lambda j, g: j * g),
    "pool query = token after the group": ("group_last", lambda j, g: (j + 1) * g),
    "n_core one too many": ("n_core", lambda t, g, w: max(0, (t - w + 1) // g + 1) if t - w + 1 > 0 else 0),
    "n_core one too few": ("n_core", lambda t, g, w: max(0, (t - w + 1) // g - 1)),
    "n_core uses <= (group ending at window start)": ("n_core", lambda t, g, w: max(0, (t - w + 2) // g)),
    "window one token short": ("win_lo", lambda t, w: max(0, t - w + 2) if t - w + 2 <= t else t),
    "window one token long": ("win_lo", lambda t, w: max(0, t - w)),
    "softmax sign flipped": ("_softmax", lambda s, axis=-1: np.exp(-s - np.max(-s, axis=axis, keepdims=True)) /
                             np.sum(np.exp(-s - np.max(-s, axis=axis, keepdims=True)), axis=axis, keepdims=True)),
    "softmax without normalisation": ("_softmax", lambda s, axis=-1: np.exp(s - np.max(s, axis=axis, keepdims=True))),
}


def _pool_no_scale(Q, K, V, g, mode="softmax"):
    B, Hq, L, d = Q.shape
    return _ORIG_POOL(Q * math.sqrt(d), K, V, g, mode)


def _pool_swapped_kv(Q, K, V, g, mode="softmax"):
    ck, cv, a = _ORIG_POOL(Q, K, V, g, mode)
    return cv, ck, a


def _pool_first_head_only(Q, K, V, g, mode="softmax"):
    G = Q.shape[1] // K.shape[1]
    return _ORIG_POOL(np.repeat(Q[:, ::G], G, axis=1), K, V, g, mode)


def _pool_max_is_min(Q, K, V, g, mode="softmax"):
    if mode != "max":
        return _ORIG_POOL(Q, K, V, g, mode)
    ck, cv, a = _ORIG_POOL(-Q, -K, -V, g, mode)
    return -ck, -cv, a


def _pool_heads_average_logits(Q, K, V, g, mode="softmax"):
    # mean of the per-head scores instead of the mean of the per-head softmaxes
    return _ORIG_POOL(Q, K, V, g, "softmax" if mode == "softmax_heads" else mode)


def _pool_mean_over_g_minus_1(Q, K, V, g, mode="softmax"):
    ck, cv, a = _ORIG_POOL(Q, K, V, g, mode)
    if mode == "mean" and g > 1:
        return ck * g / (g - 1), cv * g / (g - 1), a * g / (g - 1)
    return ck, cv, a


def _rows_transposed_heads(Q, K, V, CK, CV, g, w, ts):
    # kv head taken as h % Hkv instead of h // G
    Hq, Hkv = Q.shape[1], K.shape[1]
    G = Hq // Hkv
    perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)]) if G > 1 else np.arange(Hq)
    out = _ORIG_ROWS(Q[:, perm], K, V, CK, CV, g, w, ts)
    inv = np.argsort(perm)
    return out[:, inv]


def _masked_window_one_long(Q, K, V, CK, CV, g, w, t0, t1):
    return _ORIG_MASKED(Q, K, V, CK, CV, g, w + 1, t0, t1)


def _masked_rows_shifted(Q, K, V, CK, CV, g, w, t0, t1):
    # rows of the range computed one position late (the last one early)
    L = Q.shape[2]
    a, b = min(t0 + 1, L - 1), min(t1 + 1, L)
    out = _ORIG_MASKED(Q, K, V, CK, CV, g, w, a, b)
    if out.shape[2] < t1 - t0:
        out = np.concatenate([out, _ORIG_MASKED(Q, K, V, CK, CV, g, w, L - 1, L)], axis=2)
    return out[:, :, : t1 - t0]


_ORIG_POOL = orc.pool_core
_ORIG_ROWS = orc.attn_rows
_ORIG_MASKED = orc.attn_rows_masked

FN_MUTATIONS = {
    "pooling scores not scaled by 1/sqrt(d)": ("pool_core", _pool_no_scale),
    "core K and V swapped": ("pool_core", _pool_swapped_kv),
    "GQA pooling query from first head only": ("pool_core", _pool_first_head_only),
    "max pooling takes the minimum": ("pool_core", _pool_max_is_min),
    "per-head softmax rule averages logits": ("pool_core", _pool_heads_average_logits),
    "mean pooling divides by g-1": ("pool_core", _pool_mean_over_g_minus_1),
    "query head -> kv head map transposed": ("attn_rows", _rows_transposed_heads),
    "masked rows: window one token long": ("attn_rows_masked", _masked_window_one_long),
    "masked rows: rows shifted by one": ("attn_rows_masked", _masked_rows_shifted),
}


@pytest.mark.parametrize("label", list(MUTATIONS) + list(FN_MUTATIONS))
def test_planted_mistakes_are_caught(label, monkeypatch):
    name, fn = MUTATIONS.get(label) or FN_MUTATIONS[label]
    monkeypatch.setattr(orc, name, fn)
    caught = []
    for pin in PINS:
        try:
            if pin(orc):
                caught.append(pin.__name__)
        except Exception as exc:  # a crash also counts as caught
            caught.append(f"{pin.__name__} raised {type(exc).__name__}")
    assert caught, f"no pin catches the planted mistake: {label}"
