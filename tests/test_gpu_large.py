"""GPU check at buffer sizes past 2^31 elements (64-bit offsets in every kernel).

B = 260 sequences of 2 query heads / 1 kv head, L = 32768, d = 128 (bf16): Q and
the output hold 2.18e9 elements each, so the last sequence's rows lie beyond
2^31 elements from the start of their buffers.  Only three sequences (the
first, one in the middle, the last) carry seeded inputs; the others are zeros
(and, for the backward, a zero upstream gradient), which keeps the input
generation small.  The oracle checks pooling, sampled prefill rows and the
backward (as in the full-size backward test: dq over the last w + 3g rows, dk
and dv at positions of the last groups) of the last sequence, and the output of
the first one.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cca_inputs
import oracle.cca_backward as bwd
import oracle.cca_oracle as orc
import sparse_long_context_cca_amd as cca

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg: str) -> None:
    print(msg, flush=True)


def f32np(t):
    return t.detach().to("cpu", torch.float32).numpy()


def test_offsets_beyond_2_31_elements():
    B, Hq, Hkv, L, d, g, w = 260, 2, 1, 32768, 128, 16, 1024
    assert B * Hq * L * d > 2 ** 31
    filled = [0, B // 2, B - 1]
    say(f"large buffers: B={B} Hq={Hq} L={L} d={d}: {B * Hq * L * d / 2 ** 31:.3f} x 2^31 query elements")
    bf = torch.bfloat16
    q = torch.zeros((B, Hq, L, d), dtype=bf, device=DEV)
    k = torch.zeros((B, Hkv, L, d), dtype=bf, device=DEV)
    v = torch.zeros_like(k)
    dO = torch.zeros_like(q)
    host = {}
    for i, b in enumerate(filled):
        qs = cca_inputs.to_storage(cca_inputs.normal_f32(8100 + i, (1, Hq, L, d)), "bf16")
        ks = cca_inputs.to_storage(cca_inputs.normal_f32(8200 + i, (1, Hkv, L, d)), "bf16")
        vs = cca_inputs.to_storage(cca_inputs.normal_f32(8300 + i, (1, Hkv, L, d)), "bf16")
        gs = cca_inputs.to_storage(cca_inputs.normal_f32(8400 + i, (1, Hq, L, d)), "bf16")
        q[b : b + 1].copy_(qs.to(DEV))
        k[b : b + 1].copy_(ks.to(DEV))
        v[b : b + 1].copy_(vs.to(DEV))
        dO[b : b + 1].copy_(gs.to(DEV))
        host[b] = (f32np(qs), f32np(ks), f32np(vs), f32np(gs))
    m = L // g
    ck = torch.empty((B, Hkv, m, d), dtype=cca.core_dtype(bf), device=DEV)
    cv = torch.empty_like(ck)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    say("  pool, forward with statistics, backward on GPU")
    cca.cca_pool_core(q, k, v, ck, cv, g)
    cca.cca_attn_prefill_train(q, k, v, ck, cv, out, lse, g, w)
    dq = torch.empty((B, Hq, L, d), dtype=torch.float32, device=DEV)
    dk = torch.empty((B, Hkv, L, d), dtype=torch.float32, device=DEV)
    dv = torch.empty_like(dk)
    ws = torch.empty(cca.cca_attn_backward_workspace_bytes(B, Hq, Hkv, L, d, g, bf), dtype=torch.uint8, device=DEV)
    cca.cca_attn_backward(q, k, v, ck, cv, out, lse, dO, dq, dk, dv, ws, g, w)
    torch.cuda.synchronize()

    r0 = L - w - 3 * g
    rows = list(range(r0, L))
    sample = sorted({0, 1, w - 1, w, w + g - 1, L // 2, L // 2 + 5, L - 1} | set(range(r0, r0 + 4)))
    pos = [r0, r0 + g - 1, L - w - 1, L - w, L - 2, L - 1]
    for b in filled:
        Q, K, V, G = host[b]
        say(f"  oracle, sequence {b}")
        CK, CV, _ = orc.pool_core(Q, K, V, g)
        e_ck = float(np.abs(ck[b : b + 1].double().cpu().numpy() - CK).max())
        o_ref = orc.attn_rows(Q, K, V, CK, CV, g, w, sample)
        e_o = float(np.abs(out[b : b + 1, :, sample].double().cpu().numpy() - o_ref).max())
        say(f"    cores max abs err {e_ck:.3e}; output rows max abs err {e_o:.3e}")
        assert e_ck <= 2e-2 and e_o <= 2e-2
        if b != B - 1:
            continue
        dQr, dKf, dVf, dCK, dCV = bwd.attn_backward_rows(Q, K, V, CK, CV, g, w, G, rows)
        j0 = r0 // g
        pQ, pK, pV = bwd.pool_backward(Q[:, :, j0 * g :], K[:, :, j0 * g :], V[:, :, j0 * g :], g,
                                       dCK[:, :, j0:], dCV[:, :, j0:], "softmax")
        dq_ref = dQr + pQ[:, :, [t - j0 * g for t in rows]]
        dk_ref = dKf[:, :, pos] + pK[:, :, [p - j0 * g for p in pos]]
        dv_ref = dVf[:, :, pos] + pV[:, :, [p - j0 * g for p in pos]]
        got = (dq[b : b + 1, :, rows], dk[b : b + 1, :, pos], dv[b : b + 1, :, pos])
        for name, x, y in zip(("dq", "dk", "dv"), got, (dq_ref, dk_ref, dv_ref)):
            e = float(np.abs(x.double().cpu().numpy() - y).max()) / max(1.0, float(np.abs(y).max()))
            say(f"    {name} max err / scale {e:.3e}")
            assert e <= 2e-2, name
    # a zero sequence: zero output (uniform weights over zero values)
    assert float(out[1].float().abs().max()) == 0.0
