"""The decode entry point that allocates nothing (cca_attn_decode_scratch:
its split states live in the library's fixed device array) against the one
that takes a caller workspace (cca_attn_decode_ex), through the C ABI.

Two calls in a row, the second with smaller shapes: each runs a few decode
steps (one of them completing a group, so a core is appended) from identical
copies of a seeded cache state, and the outputs, the caches and pos must be
bit-identical between the two entry points (same kernels, same split plan).
"""
from __future__ import annotations

import pytest
import torch

import cca_inputs
import sparse_long_context_cca_amd as cca

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def state(B, Hq, Hkv, d, g, w, R, m_cap, pos0, steps, seed):
    """A decode state after pos0[b] tokens (cores pooled on the GPU, ring
    filled) and the projections of every token the steps will read."""
    T = max(pos0) + steps
    cfg = cca_inputs.make_config(seed, "scratch", B, Hq, Hkv, T, d, g, w, "bf16")
    q, k, v = (x.to(DEV) for x in cca_inputs.prefill_inputs(cfg))
    Lh = max(pos0)
    ck = torch.zeros((B, Hkv, m_cap, d), dtype=cca.core_dtype(q.dtype), device=DEV)
    cv = torch.zeros_like(ck)
    ck_h = torch.empty((B, Hkv, max(Lh // g, 1), d), dtype=ck.dtype, device=DEV)
    cv_h = torch.empty_like(ck_h)
    cca.cca_pool_core(q[:, :, :Lh].contiguous(), k[:, :, :Lh].contiguous(), v[:, :, :Lh].contiguous(),
                      ck_h, cv_h, g)
    n = min(m_cap, Lh // g)
    ck[:, :, :n] = ck_h[:, :, :n]
    cv[:, :, :n] = cv_h[:, :, :n]
    rk = torch.zeros((B, Hkv, R, d), dtype=q.dtype, device=DEV)
    rv = torch.zeros_like(rk)
    for b in range(B):
        for p in range(max(0, pos0[b] - R), pos0[b]):
            rk[b, :, p % R] = k[b, :, p]
            rv[b, :, p % R] = v[b, :, p]
    pos = torch.tensor(pos0, dtype=torch.int32, device=DEV)
    return (q, k, v), [ck, cv, rk, rv, pos]


def run_both(B, Hq, Hkv, d, g, w, R, m_cap, pos0, steps, seed):
    print(f"scratch decode B={B} Hq={Hq} Hkv={Hkv} d={d} g={g} w={w} pos0={pos0} steps={steps}", flush=True)
    (q, k, v), st = state(B, Hq, Hkv, d, g, w, R, m_cap, pos0, steps, seed)
    assert max(pos0) + steps - 1 < q.shape[2], "every step's token must exist in the inputs"
    a = [x.clone() for x in st]
    b = [x.clone() for x in st]
    ws = torch.empty(cca.cca_decode_workspace_bytes(B, Hq, Hkv, d, m_cap, g, w), dtype=torch.uint8, device=DEV)
    assert ws.numel() <= cca.cca_decode_scratch_bytes()
    bidx = torch.arange(B, device=DEV)
    for i in range(steps):
        t = torch.tensor([p + i for p in pos0], device=DEV)
        q_t, k_t, v_t = (x[bidx, :, t].contiguous() for x in (q, k, v))
        out_a = torch.full((B, Hq, d), float("nan"), dtype=q.dtype, device=DEV)
        out_b = torch.full_like(out_a, float("nan"))
        cca.cca_attn_decode(q_t, k_t, v_t, a[2], a[3], a[0], a[1], a[4], out_a, ws, g, w, advance_pos=True)
        cca.cca_attn_decode_scratch(q_t, k_t, v_t, b[2], b[3], b[0], b[1], b[4], out_b, g, w, advance_pos=True)
        torch.cuda.synchronize()
        assert torch.isfinite(out_a.float()).all()
        assert torch.equal(out_a, out_b), f"step {i}: outputs differ"
    for name, x, y in zip(("core_k", "core_v", "ring_k", "ring_v", "pos"), a, b):
        assert torch.equal(x, y), f"{name} differs"
    assert b[4].tolist() == [p + steps for p in pos0]


def test_scratch_decode_matches_workspace_decode():
    # a group completes at t = 15 mod 16 during the steps; then a smaller call
    run_both(4, 16, 4, 128, 16, 64, 64, 64, [300, 645, 90, 733], 12, seed=901)
    run_both(2, 8, 2, 64, 4, 16, 16, 40, [33, 60], 5, seed=902)
