"""Pins of the fp64 backward oracle (oracle/cca_backward.py), CPU only.

The gradients are pinned by things other than the chain rule they restate:
central finite differences of the forward oracle's scalar loss on tiny inputs
(every entry of dQ, dK, dV, for every pooling rule), and the reduction to
textbook causal attention, whose gradients torch's autograd of SDPA gives in
fp64.  As in test_oracle, each pin returns failure strings, and plausible
mistakes planted in the oracle must each be caught by some pin.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import cca_inputs
import oracle.cca_backward as bwd
import oracle.cca_oracle as orc


def _rand(seed, shape, scale=1.0):
    return cca_inputs.normal_f32(seed, shape, scale).astype(np.float64)


def _close(a, b, tol):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    return None if err <= tol else f"max abs err {err:.3e} > {tol:.1e}"


FD_CASES = [
    # B, Hq, Hkv, L, d, g, w  (tiny: every entry is differenced)
    (1, 2, 1, 14, 3, 3, 4),
    (1, 4, 2, 11, 2, 2, 3),
    (2, 1, 1, 9, 2, 4, 2),
]


def pin_finite_differences(b):
    """Every entry of dQ, dK, dV equals the central difference of
    sum(O * dO) (h = 1e-6, fp64), for every pooling rule."""
    fails = []
    h = 1e-6
    for ci, (B, Hq, Hkv, L, d, g, w) in enumerate(FD_CASES):
        Q = _rand(200 + ci, (B, Hq, L, d), 1.5)
        K, V = _rand(210 + ci, (B, Hkv, L, d), 1.5), _rand(220 + ci, (B, Hkv, L, d))
        dO = _rand(230 + ci, (B, Hq, L, d))
        for mode in orc.POOL_MODES:
            grads = b.backward(Q, K, V, g, w, dO, mode)
            for name, X, G in zip("QKV", (Q, K, V), grads):
                num = np.empty_like(X)
                for idx in np.ndindex(X.shape):
                    keep = X[idx]
                    X[idx] = keep + h
                    up = b.loss(Q, K, V, g, w, dO, mode)
                    X[idx] = keep - h
                    dn = b.loss(Q, K, V, g, w, dO, mode)
                    X[idx] = keep
                    num[idx] = (up - dn) / (2 * h)
                e = _close(G, num, 2e-6)
                if e:
                    fails.append(f"case {ci} {mode} d{name}: {e}")
    return fails


def _sdpa_grads(Q, K, V, dO):
    """Textbook causal attention and its gradients (torch autograd, fp64);
    GQA by repeating each kv head over its G query heads."""
    G = Q.shape[1] // K.shape[1]
    q = torch.tensor(Q, requires_grad=True)
    k = torch.tensor(K, requires_grad=True)
    v = torch.tensor(V, requires_grad=True)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(G, dim=1), v.repeat_interleave(G, dim=1), is_causal=True)
    (o * torch.tensor(dO)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def pin_reduces_to_causal_attention(b):
    """w >= L (no core visible) or g = 1 (each token its own core, weight 1):
    the gradients of textbook causal attention."""
    fails = []
    for ci, (B, Hq, Hkv, L, d, g, w) in enumerate([(1, 2, 2, 20, 4, 4, 20), (2, 4, 2, 17, 3, 3, 40),
                                                   (1, 2, 1, 23, 4, 1, 3), (1, 3, 3, 16, 2, 1, 1)]):
        Q = _rand(300 + ci, (B, Hq, L, d))
        K, V, dO = _rand(310 + ci, (B, Hkv, L, d)), _rand(320 + ci, (B, Hkv, L, d)), _rand(330 + ci, (B, Hq, L, d))
        for mode in orc.POOL_MODES:
            if g > 1 and mode != "softmax":
                continue
            got = b.backward(Q, K, V, g, w, dO, mode)
            for name, x, y in zip("QKV", got, _sdpa_grads(Q, K, V, dO)):
                e = _close(x, y, 1e-11)
                if e:
                    fails.append(f"case {ci} {mode} d{name}: {e}")
    return fails


def pin_row_lse(b):
    """The row statistic equals torch's logsumexp of the masked causal scores
    when every key is raw (w >= L)."""
    fails = []
    B, Hq, Hkv, L, d, g, w = 1, 2, 1, 19, 4, 3, 19
    Q, K = _rand(401, (B, Hq, L, d)), _rand(402, (B, Hkv, L, d))
    CK, _, _ = orc.pool_core(Q, K, K, g)
    lse = b.row_lse(Q, K, CK, g, w)
    s = torch.tensor(Q) @ torch.tensor(K).repeat_interleave(Hq // Hkv, 1).transpose(-1, -2) / math.sqrt(d)
    s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), float("-inf"))
    e = _close(lse, torch.logsumexp(s, dim=-1).numpy(), 1e-12)
    if e:
        fails.append(f"row lse: {e}")
    return fails


def pin_rows_form(b):
    """The row-restricted form equals the per-head loop: over all rows every
    output, over a subset the dQ rows (and the contributions of those rows,
    against the loop run on inputs whose other rows' upstream gradient is 0)."""
    fails = []
    for ci, (B, Hq, Hkv, L, d, g, w) in enumerate([(1, 4, 2, 37, 8, 3, 7), (2, 2, 2, 29, 4, 4, 5),
                                                   (1, 3, 1, 20, 4, 1, 2)]):
        Q, K, V = _rand(500 + ci, (B, Hq, L, d)), _rand(510 + ci, (B, Hkv, L, d)), _rand(520 + ci, (B, Hkv, L, d))
        dO = _rand(530 + ci, (B, Hq, L, d))
        CK, CV, _ = orc.pool_core(Q, K, V, g)
        full = b.attn_backward(Q, K, V, CK, CV, g, w, dO)
        got = b.attn_backward_rows(Q, K, V, CK, CV, g, w, dO, range(L))
        for name, x, y in zip(("dQ", "dK", "dV", "dCK", "dCV"), got, full):
            e = _close(x, y, 1e-12)
            if e:
                fails.append(f"case {ci} all rows {name}: {e}")
        rows = [t for t in range(L) if t % 3 != 1]
        dO_sub = dO.copy()
        dO_sub[:, :, [t for t in range(L) if t % 3 == 1]] = 0.0
        sub = b.attn_backward(Q, K, V, CK, CV, g, w, dO_sub)
        got = b.attn_backward_rows(Q, K, V, CK, CV, g, w, dO, rows)
        e = _close(got[0], full[0][:, :, rows], 1e-12)
        if e:
            fails.append(f"case {ci} row subset dQ: {e}")
        for name, x, y in zip(("dK", "dV", "dCK", "dCV"), got[1:], sub[1:]):
            e = _close(x, y, 1e-12)
            if e:
                fails.append(f"case {ci} row subset {name}: {e}")
    return fails


def pin_masked_rows_form(b):
    """The masked multi-row form, its contributions summed over runs of rows
    that start and end anywhere, equals the per-row form over all rows."""
    fails = []
    for ci, (B, Hq, Hkv, L, d, g, w, n) in enumerate([(1, 4, 2, 37, 8, 3, 7, 5), (2, 2, 2, 29, 4, 4, 5, 8),
                                                      (1, 3, 1, 20, 4, 1, 2, 20), (1, 2, 1, 45, 4, 6, 30, 7)]):
        Q, K, V = _rand(540 + ci, (B, Hq, L, d)), _rand(550 + ci, (B, Hkv, L, d)), _rand(560 + ci, (B, Hkv, L, d))
        dO = _rand(570 + ci, (B, Hq, L, d))
        CK, CV, _ = orc.pool_core(Q, K, V, g)
        ref = b.attn_backward_rows(Q, K, V, CK, CV, g, w, dO, range(L))
        dQ = np.zeros_like(ref[0])
        dK, dV, dCK, dCV = (np.zeros_like(x) for x in ref[1:])
        for t0 in range(0, L, n):
            t1 = min(L, t0 + n)
            q_, k_, v_, ck_, cv_, LO = b.attn_backward_rows_masked(Q, K, V, CK, CV, g, w, dO, t0, t1)
            dQ[:, :, t0:t1] = q_
            dK[:, :, LO:t1] += k_
            dV[:, :, LO:t1] += v_
            dCK[:, :, : ck_.shape[2]] += ck_
            dCV[:, :, : cv_.shape[2]] += cv_
        for name, x, y in zip(("dQ", "dK", "dV", "dCK", "dCV"), (dQ, dK, dV, dCK, dCV), ref):
            e = _close(x, y, 1e-12)
            if e:
                fails.append(f"case {ci} {name}: {e}")
    return fails


PINS = [pin_finite_differences, pin_reduces_to_causal_attention, pin_row_lse, pin_rows_form,
        pin_masked_rows_form]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_pin(pin):
    fails = pin(bwd)
    assert not fails, "\n".join(fails[:10])


# ---------------------------------------------------- planted mistakes

_ORIG_ATTN = bwd.attn_backward
_ORIG_POOL = bwd.pool_backward


def _no_core_grad(Q, K, V, CK, CV, g, w, dO):
    dQ, dK, dV, dCK, dCV = _ORIG_ATTN(Q, K, V, CK, CV, g, w, dO)
    return dQ, dK, dV, 0 * dCK, dCV


def _pool_no_query_grad(Q, K, V, g, dCK, dCV, mode="softmax"):
    dQ, dK, dV = _ORIG_POOL(Q, K, V, g, dCK, dCV, mode)
    return 0 * dQ, dK, dV


def _pool_max_routes_to_min(Q, K, V, g, dCK, dCV, mode="softmax"):
    if mode != "max":
        return _ORIG_POOL(Q, K, V, g, dCK, dCV, mode)
    return _ORIG_POOL(Q, -K, -V, g, dCK, dCV, mode)


def _pool_mean_over_g_minus_1(Q, K, V, g, dCK, dCV, mode="softmax"):
    dQ, dK, dV = _ORIG_POOL(Q, K, V, g, dCK, dCV, mode)
    if mode == "mean" and g > 1:
        return dQ, dK * g / (g - 1), dV * g / (g - 1)
    return dQ, dK, dV


def _attn_dv_from_ds(Q, K, V, CK, CV, g, w, dO):
    # dV accumulated with the raw-score gradient path's weights swapped: dV -> dK
    dQ, dK, dV, dCK, dCV = _ORIG_ATTN(Q, K, V, CK, CV, g, w, dO)
    return dQ, dV, dK, dCK, dCV


_ORIG_MASKED = bwd.attn_backward_rows_masked


def _masked_window_one_long(Q, K, V, CK, CV, g, w, dO, t0, t1):
    return _ORIG_MASKED(Q, K, V, CK, CV, g, w + 1, dO, t0, t1)


def _masked_dv_from_ds(Q, K, V, CK, CV, g, w, dO, t0, t1):
    dQ, dK, dV, dCK, dCV, LO = _ORIG_MASKED(Q, K, V, CK, CV, g, w, dO, t0, t1)
    return dQ, dV, dK, dCK, dCV, LO


MUTATIONS = {
    "softmax Jacobian without the row correction": ("_softmax_backward", lambda p, dp: p * dp),
    "backward scores not scaled by 1/sqrt(d)": ("_scale", lambda d: 1.0),
    "core gradients dropped": ("attn_backward", _no_core_grad),
    "pooling query gradient dropped": ("pool_backward", _pool_no_query_grad),
    "max-pooling gradient routed to the minimum": ("pool_backward", _pool_max_routes_to_min),
    "mean-pooling gradient divided by g-1": ("pool_backward", _pool_mean_over_g_minus_1),
    "raw dK and dV swapped": ("attn_backward", _attn_dv_from_ds),
    "masked rows: window one token long": ("attn_backward_rows_masked", _masked_window_one_long),
    "masked rows: raw dK and dV swapped": ("attn_backward_rows_masked", _masked_dv_from_ds),
}


@pytest.mark.parametrize("label", list(MUTATIONS))
def test_planted_backward_mistakes_are_caught(label, monkeypatch):
    name, fn = MUTATIONS[label]
    monkeypatch.setattr(bwd, name, fn)
    caught = []
    for pin in PINS:
        try:
            if pin(bwd):
                caught.append(pin.__name__)
        except Exception as exc:  # a crash also counts as caught
            caught.append(f"{pin.__name__} raised {type(exc).__name__}")
    assert caught, f"no pin catches the planted mistake: {label}"
