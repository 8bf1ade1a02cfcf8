"""GPU parity of chunked and variable-length prefill and of the prefill -> decode
handoff, through the C ABI, against the fp64 CPU oracle.

A chunked pass computes exactly the rows one full prefill computes (the pages'
method has no notion of chunks; a row depends only on its own visible sets), so
the oracle is the full-sequence oracle restricted to each chunk's rows, and
the cores are the full-sequence cores.  Bars as in test_gpu_parity.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cca_inputs
import oracle.cca_oracle as orc
import sparse_long_context_cca_amd as cca

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}
MODES = {cca.CCA_POOL_SOFTMAX: "softmax", cca.CCA_POOL_SOFTMAX_HEADS: "softmax_heads",
         cca.CCA_POOL_MEAN: "mean", cca.CCA_POOL_MAX: "max"}


def say(msg: str) -> None:
    print(msg, flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def f32np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def inputs(dt, B, Hq, Hkv, L, d, g, w, seed):
    cfg = cca_inputs.make_config(seed, "chunk", B, Hq, Hkv, L, d, g, w, dt,
                                 scale=1.0 if dt == "bf16" else d ** -0.5)
    return cca_inputs.prefill_inputs(cfg)


def i32(x):
    return torch.tensor(x, dtype=torch.int32, device=DEV)


def check_cores(dt, got, ref, mode):
    """Cores in the core dtype (fp16 for bf16 inputs): max pooling equals the
    oracle's maximum rounded to it, the other rules lie within half an ulp."""
    if mode == cca.CCA_POOL_MAX:
        cdt = torch.float32 if dt == "f32" else torch.float16
        assert np.array_equal(host(got), torch.from_numpy(ref).to(cdt).to(torch.float64).numpy())
    elif dt == "f32":
        assert float(np.abs(host(got) - ref).max()) <= 1e-5
    else:
        assert np.all(np.abs(host(got) - ref) <= np.abs(ref) * 2.0 ** -11 * 1.01 + 1e-6)


CHUNK_CASES = [
    # dt, B, Hq, Hkv, L, d, g, w, chunk sizes, pooling rule
    ("f32", 1, 2, 1, 300, 64, 16, 32, [1, 7, 40, 100, 152], cca.CCA_POOL_SOFTMAX),
    ("bf16", 2, 8, 2, 1100, 128, 16, 64, [5, 300, 64, 731], cca.CCA_POOL_SOFTMAX),
    ("bf16", 1, 4, 4, 2000, 128, 16, 1024, [1024, 976], cca.CCA_POOL_SOFTMAX),
    ("bf16", 1, 4, 1, 517, 64, 3, 20, [517], cca.CCA_POOL_SOFTMAX),
    ("bf16", 1, 8, 2, 700, 128, 16, 48, [129, 200, 371], cca.CCA_POOL_MAX),
    ("f32", 2, 4, 2, 450, 128, 5, 30, [64, 64, 64, 258], cca.CCA_POOL_SOFTMAX_HEADS),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: f"{c[0]}-L{c[4]}-g{c[6]}-w{c[7]}-{len(c[8])}chunks-{MODES[c[9]]}")
def test_chunked_prefill_equals_full_prefill(case):
    dt, B, Hq, Hkv, L, d, g, w, chunks, mode = case
    assert sum(chunks) == L
    say(f"chunked prefill {case}")
    q, k, v = inputs(dt, B, Hq, Hkv, L, d, g, w, seed=700 + L)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    m_cap = L // g + 2
    ck = torch.full((B, Hkv, m_cap, d), float("nan"), dtype=cca.core_dtype(q.dtype), device=DEV)
    cv = torch.full_like(ck, float("nan"))
    out = torch.full((B, Hq, L, d), float("nan"), dtype=q.dtype, device=DEV)
    start = 0
    for C in chunks:
        qc = qd[:, :, start:start + C].contiguous()
        qs, ql = i32([start] * B), i32([C] * B)
        oc = torch.full((B, Hq, C, d), float("nan"), dtype=q.dtype, device=DEV)
        # K/V: a cache buffer holding every position (only those below start + C are read)
        cca.cca_pool_core_chunk(qc, kd, vd, ck, cv, g, qs, ql, mode=mode)
        cca.cca_attn_prefill_chunk(qc, kd, vd, ck, cv, oc, g, w, qs, ql)
        out[:, :, start:start + C] = oc
        start += C
    torch.cuda.synchronize()
    Q, K, V = f32np(q), f32np(k), f32np(v)
    CK, CV, _ = orc.pool_core(Q, K, V, g, MODES[mode])
    ref = orc.attn_prefill(Q, K, V, CK, CV, g, w)
    e = float(np.abs(host(out) - ref).max())
    say(f"  max abs err {e:.3e}")
    assert e <= TOL[dt]
    m = L // g
    check_cores(dt, ck[:, :, :m], CK, mode)
    check_cores(dt, cv[:, :, :m], CV, mode)
    assert torch.isnan(ck[:, :, m:]).all(), "no core beyond the completed groups"


@pytest.mark.parametrize("heads,w", [((8, 2), 64), ((4, 4), 300)], ids=["G4-w64", "G1-w300"])
def test_variable_length_batch(heads, w):
    """One call per step for a batch whose sequences sit at their own offsets
    and lengths (one of them empty in the first step); output rows past each
    sequence's length stay untouched.  With one query head per kv head the
    workgroups' halves walk the raw window apart, from offsets that start
    mid-tile."""
    (Hq, Hkv), dt, B, d, g = heads, "bf16", 3, 128, 16
    L = 600
    say(f"variable-length batch Hq={Hq} Hkv={Hkv} w={w}")
    q, k, v = inputs(dt, B, Hq, Hkv, L, d, g, w, seed=811)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    m_cap = L // g
    ck = torch.full((B, Hkv, m_cap, d), float("nan"), dtype=cca.core_dtype(q.dtype), device=DEV)
    cv = torch.full_like(ck, float("nan"))
    steps = [([0, 0, 0], [100, 250, 0]), ([100, 250, 0], [200, 50, 300]), ([300, 300, 300], [0, 277, 3])]
    got = {b: [] for b in range(B)}
    for starts, lens in steps:
        Lq = max(max(lens), 1)
        qc = torch.zeros((B, Hq, Lq, d), dtype=q.dtype, device=DEV)
        for b in range(B):
            qc[b, :, : lens[b]] = qd[b, :, starts[b] : starts[b] + lens[b]]
        oc = torch.full((B, Hq, Lq, d), 7.0, dtype=q.dtype, device=DEV)
        cca.cca_pool_core_chunk(qc, kd, vd, ck, cv, g, i32(starts), i32(lens))
        cca.cca_attn_prefill_chunk(qc, kd, vd, ck, cv, oc, g, w, i32(starts), i32(lens))
        torch.cuda.synchronize()
        for b in range(B):
            assert bool((oc[b, :, lens[b]:] == 7.0).all()), "rows past q_len must stay untouched"
            got[b].append(oc[b, :, : lens[b]])
    Q, K, V = f32np(q), f32np(k), f32np(v)
    worst = 0.0
    for b in range(B):
        n = sum(lens[b] for _, lens in steps)
        rows = torch.cat(got[b], dim=1)
        CK, CV, _ = orc.pool_core(Q[b : b + 1, :, :n], K[b : b + 1, :, :n], V[b : b + 1, :, :n], g)
        ref = orc.attn_prefill(Q[b : b + 1, :, :n], K[b : b + 1, :, :n], V[b : b + 1, :, :n], CK, CV, g, w)
        worst = max(worst, float(np.abs(host(rows)[None] - ref).max()))
        check_cores(dt, ck[b, :, : n // g], CK[0], cca.CCA_POOL_SOFTMAX)
    say(f"  max abs err {worst:.3e}")
    assert worst <= TOL[dt]


def test_ranges_that_do_not_fit_give_nan_and_no_writes():
    B, Hq, Hkv, d, g, w, Lq, Lk, m_cap = 4, 4, 2, 128, 16, 32, 64, 256, 8
    say("chunk ranges that do not fit")
    mk = lambda *s: torch.ones(s, dtype=torch.bfloat16, device=DEV)
    q, k, v = mk(B, Hq, Lq, d), mk(B, Hkv, Lk, d), mk(B, Hkv, Lk, d)
    ck, cv = torch.zeros((B, Hkv, m_cap, d), dtype=torch.float16, device=DEV), torch.zeros((B, Hkv, m_cap, d), dtype=torch.float16, device=DEV)
    out = torch.zeros((B, Hq, Lq, d), dtype=torch.bfloat16, device=DEV)
    # b0 fits; b1 q_len > Lq; b2 q_start + q_len > Lk; b3 sees a core beyond m_cap
    qs, ql = i32([0, 0, 250, 192]), i32([64, 65, 10, 64])
    cca.cca_pool_core_chunk(q, k, v, ck, cv, g, qs, ql)
    cca.cca_attn_prefill_chunk(q, k, v, ck, cv, out, g, w, qs, ql)
    torch.cuda.synchronize()
    assert torch.isfinite(out[0].float()).all()
    for b in (1, 2, 3):
        assert torch.isnan(out[b].float()).all(), f"sequence {b} must read NaN"
    assert bool((ck[1:3] == 0).all()), "no core written for a range that does not fit"
    assert bool((ck[0, :, :4] != 0).all()), "the fitting sequence's groups are pooled"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_decode_handoff(dt):
    """Chunked prefill of two sequences of different lengths, ring filled by the
    library, then decode steps continuing both: every step equals the oracle."""
    B, Hq, Hkv, d, g, w, R = 2, 8, 2, 128, 16, 64, 64
    lens = [333, 200]
    steps = 40
    T = max(lens) + steps
    say(f"prefill -> decode handoff {dt}")
    q, k, v = inputs(dt, B, Hq, Hkv, T, d, g, w, seed=919)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    m_cap = T // g + 1
    ck = torch.zeros((B, Hkv, m_cap, d), dtype=cca.core_dtype(q.dtype), device=DEV)
    cv = torch.zeros_like(ck)
    # prefill in two chunks per sequence: 128 rows, then the rest
    for starts, ln in (([0, 0], [128, 128]), ([128, 128], [lens[0] - 128, lens[1] - 128])):
        Lq = max(ln)
        qc = torch.zeros((B, Hq, Lq, d), dtype=q.dtype, device=DEV)
        for b in range(B):
            qc[b, :, : ln[b]] = qd[b, :, starts[b] : starts[b] + ln[b]]
        oc = torch.empty((B, Hq, Lq, d), dtype=q.dtype, device=DEV)
        cca.cca_pool_core_chunk(qc, kd, vd, ck, cv, g, i32(starts), i32(ln))
        cca.cca_attn_prefill_chunk(qc, kd, vd, ck, cv, oc, g, w, i32(starts), i32(ln))
    rk = torch.zeros((B, Hkv, R, d), dtype=q.dtype, device=DEV)
    rv = torch.zeros_like(rk)
    seq_len = i32(lens)
    cca.cca_cache_fill_ring(kd, vd, rk, rv, seq_len)
    pos = seq_len.clone()
    ws = torch.empty(cca.cca_decode_workspace_bytes(B, Hq, Hkv, d, m_cap, g, w), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, Hq, d), dtype=q.dtype, device=DEV)
    Q, K, V = f32np(q), f32np(k), f32np(v)
    CK, CV, _ = orc.pool_core(Q, K, V, g)
    bidx = torch.arange(B, device=DEV)
    worst = 0.0
    for i in range(steps):
        t = torch.tensor([p + i for p in lens], device=DEV)
        cca.cca_attn_decode(qd[bidx, :, t].contiguous(), kd[bidx, :, t].contiguous(),
                            vd[bidx, :, t].contiguous(), rk, rv, ck, cv, pos, out, ws, g, w,
                            advance_pos=True)
        torch.cuda.synchronize()
        tt = np.array([p + i for p in lens])
        ref = orc.attn_decode(Q[np.arange(B), :, tt], K, V, CK, CV, tt, g, w)
        worst = max(worst, float(np.abs(host(out) - ref).max()))
    say(f"  max abs err over steps {worst:.3e}")
    assert worst <= TOL[dt]
    assert pos.tolist() == [p + steps for p in lens]


def test_chunked_full_size_is_bit_identical_to_full_prefill():
    """The 128K GQA workload in five ragged chunks (boundaries off every tile
    and group edge) gives the one-shot prefill's outputs and cores bit for bit:
    a row's result depends only on the keys it sees, the key tiles sit at
    absolute 64-key boundaries in both runs, and a key outside a row's sets
    adds exact zeros.  (The one-shot prefill itself is checked against the
    oracle at this size in test_gpu_parity.)"""
    cfg = cca_inputs.CONFIGS[4]
    chunks = [1, 20000, 32768, 45679, 32624]
    assert sum(chunks) == cfg.L
    say(f"chunked vs one-shot prefill at full size {cfg.name}, chunks {chunks}")
    q, k, v = cca_inputs.prefill_inputs(cfg)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    del q, k, v
    B, Hkv, d, g, w = cfg.B, cfg.Hkv, cfg.d, cfg.g, cfg.w
    m = cfg.L // g
    ck_full = torch.empty((B, Hkv, m, d), dtype=cca.core_dtype(qd.dtype), device=DEV)
    cv_full = torch.empty_like(ck_full)
    out_full = torch.empty_like(qd)
    cca.cca_pool_core(qd, kd, vd, ck_full, cv_full, g)
    cca.cca_attn_prefill(qd, kd, vd, ck_full, cv_full, out_full, g, w)
    ck = torch.full_like(ck_full, float("nan"))
    cv = torch.full_like(ck_full, float("nan"))
    out = torch.full_like(qd, float("nan"))
    start = 0
    for C in chunks:
        qc = qd[:, :, start:start + C].contiguous()
        qs, ql = i32([start] * B), i32([C] * B)
        oc = torch.empty((B, cfg.Hq, C, d), dtype=qd.dtype, device=DEV)
        cca.cca_pool_core_chunk(qc, kd, vd, ck, cv, g, qs, ql)
        cca.cca_attn_prefill_chunk(qc, kd, vd, ck, cv, oc, g, w, qs, ql)
        out[:, :, start:start + C] = oc
        start += C
    torch.cuda.synchronize()
    assert torch.equal(ck, ck_full) and torch.equal(cv, cv_full), "cores differ"
    same = out == out_full
    assert bool(same.all()), f"{int((~same).sum())} output values differ"
