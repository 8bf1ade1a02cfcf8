#!/usr/bin/env python3
"""Benchmark of the CCA attention hot path on one MI355X.

A step is one pass of the prefill hot path over the LLaMA-3.1-8B GQA workload
(batch 1, 32 query / 8 kv heads, head dim 128, L = 131072, g = 16, w = 1024,
bf16): cca_pool_core then cca_attn_prefill, inputs already resident in HBM.
In the same run, under "prefill_configs": the other prefill workloads (tiny
fp32 L = 1024; LLaMA-2-7B MHA at 32K; LLaMA-2-7B MHA at 128K with spiky keys)
and the headline one again, each as pool + prefill steps timed with events;
under "backward": the backward pass over the headline workload; under
"decode": the decode workload (batch 8, 32/8 heads, 65536 cached tokens, 256
single-token steps).  A large bf16 GEMM, a device-to-device copy and a
read-only reduction give measured ceilings ("reference_rates") next to the
spec peaks, and so does a kernel that runs nothing but matrix-core work on
random operands (libcca_probe.so): the rate the matrix cores sustain on this
chip, at the clock its power limit allows.

Prints ONE JSON line.  Flags: --gpus N (only 1 is supported), --steps K,
--warmup W, --no-cpu (skip the CPU-oracle baseline), --no-decode, --no-backward,
--no-configs (skip the other prefill workloads).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import cca_inputs  # noqa: E402

METRIC = "CCA prefill tokens/s + MFMA util at 128K (8B GQA shape, 1 GPU); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_VALU_TFLOPS = 157.3  # MI355X fp32 vector peak (the fp32 prefill runs on the vector ALUs)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak


def profile_fields(filename):
    """The `key: value` lines of a committed counter summary under profiles/,
    or None when the summary is missing or its kernel has changed since the
    counters were taken (the summary carries a digest of the kernel's sources
    and build flags; a figure for other code describes nothing here)."""
    path = os.path.join(ROOT, "profiles", filename)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if line.startswith("#") or ":" not in line:
            continue
        key, val = line.split(":", 1)
        fields[key.strip()] = val.strip()
    try:
        digest = code_digest(fields.get("sources", "").split())
    except OSError:
        return None
    return fields if digest == fields.get("kernel_sha256") else None


def measured_traffic(name):
    """HBM bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    each scaled by what the same counter reads for a device copy of known
    size (profiles/traffic_<name>.txt)."""
    fields = profile_fields(f"traffic_{name}.txt")
    return int(fields["traffic_bytes"]) if fields else None


def measured_mfma_busy(name, kernel="mfma_busy_fraction"):
    """Fraction of SIMD cycles with the matrix cores busy, from the shader
    counters in profiles/counters_<name>.txt (it includes masked and
    recomputed work, unlike the algorithmic fraction)."""
    fields = profile_fields(f"counters_{name}.txt")
    return float(fields[kernel]) if fields and kernel in fields else None


def code_digest(sources):
    """SHA-256 over the code lines of the given sources (// comments and blank
    lines dropped, so that editing a comment keeps a counter figure valid).  Of
    the build script only its compiler-flag block counts (the lines between
    its "---- compiler flags" and "---- end of compiler flags" markers): the
    rest of the script does not change what a kernel executes."""
    h = hashlib.sha256()
    for src in sources:
        lines = open(os.path.join(ROOT, src), encoding="utf-8").read().splitlines(True)
        if src.endswith("build.py"):
            start = next(i for i, ln in enumerate(lines) if "---- compiler flags" in ln)
            end = next(i for i, ln in enumerate(lines) if "---- end of compiler flags" in ln)
            lines = lines[start:end + 1]
        for line in lines:
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def visible_pairs(L, g, w):
    t = np.arange(L, dtype=np.int64)
    nc = np.where(t - w + 1 > 0, (t - w + 1) // g, 0)
    lo = np.maximum(0, t - w + 1)
    return int(nc.sum() + (t - lo + 1).sum())


def prefill_flops(cfg):
    """Algorithmic FLOPs: 4*d per visible (query head, key) pair (Q.K and P.V)."""
    return 4.0 * cfg.d * cfg.B * cfg.Hq * visible_pairs(cfg.L, cfg.g, cfg.w)


def pool_bytes(cfg):
    """Algorithmic bytes of pooling: K and V read once, the G query rows at
    each group end, core K and V written."""
    es = 2 if cfg.dtype == "bf16" else 4
    m = cfg.L // cfg.g
    return es * cfg.B * (2 * cfg.Hkv * m * cfg.g * cfg.d + cfg.Hq * m * cfg.d + 2 * cfg.Hkv * m * cfg.d)


def decode_step_bytes(cfg, t):
    """Algorithmic bytes of one decode step at position t for every sequence:
    visible core + window K/V, q, out, k_t/v_t read and appended, and on a
    group boundary the g-1 ring rows pooled plus the core written."""
    es = 2
    B, Hq, Hkv, d, g, w = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.g, cfg.w
    nc = max(0, (t - w + 1) // g) if t - w + 1 > 0 else 0
    nvis = nc + (t - max(0, t - w + 1) + 1)
    by = B * Hkv * nvis * 2 * d * es          # K and V of visible keys
    by += 2 * B * Hq * d * es                 # q_t in, out
    by += 2 * 2 * B * Hkv * d * es            # k_t, v_t read + written to the ring
    if (t + 1) % g == 0:
        by += B * Hkv * ((g - 1) * 2 * d * es + 2 * d * es)
    return by


def cpu_oracle_baseline(cfg, q, k, v, budget_s=20.0):
    """Times the fp64 CPU oracle (as it stands) on a bounded sample of the
    prefill workload: pooling of one kv head over all L tokens (scaled to all
    kv heads) plus the attention rows of the last S positions for every query
    head; S doubles until one sample costs more than budget_s/4, so the timed
    (last) sample takes budget_s/4 to budget_s/2 and all samples together
    about twice that."""
    import oracle.cca_oracle as orc
    try:
        from threadpoolctl import threadpool_limits
        cores = len(os.sched_getaffinity(0))
        limiter = threadpool_limits(limits=cores)
    except Exception:  # pragma: no cover
        cores, limiter = os.cpu_count(), None
    Q = q.to(torch.float32).numpy()
    K = k.to(torch.float32).numpy()
    V = v.to(torch.float32).numpy()
    G = cfg.Hq // cfg.Hkv
    # cores of every kv head are needed by the attention rows; the first one is timed
    CKs = np.empty((cfg.B, cfg.Hkv, cfg.L // cfg.g, cfg.d))
    CVs = np.empty_like(CKs)
    t_pool_one = 0.0
    for hk in range(cfg.Hkv):
        t0 = time.perf_counter()
        a, b_, _ = orc.pool_core(Q[:, hk * G:(hk + 1) * G], K[:, hk:hk + 1], V[:, hk:hk + 1], cfg.g)
        if hk == 0:
            t_pool_one = time.perf_counter() - t0
        CKs[:, hk], CVs[:, hk] = a[:, 0], b_[:, 0]
    t_pool = t_pool_one * cfg.Hkv
    S, t_rows = 4, 0.0
    while True:
        rows = list(range(cfg.L - S, cfg.L))
        t0 = time.perf_counter()
        orc.attn_rows(Q, K, V, CKs, CVs, cfg.g, cfg.w, rows)
        t_rows = time.perf_counter() - t0
        if t_rows > budget_s / 4 or S >= 4096:
            break
        S *= 2
    if limiter is not None and hasattr(limiter, "unregister"):
        limiter.unregister()
    per_token = t_rows / S + t_pool / cfg.L
    return {
        "value": 1.0 / per_token,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 numpy oracle: pooling of 1 of {cfg.Hkv} kv heads over all {cfg.L} tokens "
                   f"({t_pool_one:.2f} s, scaled x{cfg.Hkv}) + attention rows of the last {S} positions "
                   f"for all {cfg.Hq} query heads ({t_rows:.2f} s); last positions see the most keys, "
                   f"so this rate is a lower bound for the whole sequence"),
    }


def bench_prefill(cca, cfg, steps, warmup, inputs=None, min_warmup_s=0.0):
    """Pool + prefill steps over one prefill workload (inputs resident on the
    GPU), timed with events on the launch stream: the whole step and the
    prefill launch alone.  The untimed warm-up is `warmup` steps, continued
    until `min_warmup_s` seconds have passed: the chip's clock climbs back
    over tens of milliseconds after the seconds of host-side input generation,
    longer than three short launches.  Returns the per-config record and the
    device tensors (so the caller can reuse them)."""
    dev = "cuda:0"
    if inputs is None:
        q, k, v = cca_inputs.prefill_inputs(cfg)
        inputs = (q.to(dev), k.to(dev), v.to(dev))
    qd, kd, vd = inputs
    m = cfg.L // cfg.g
    ck = torch.empty((cfg.B, cfg.Hkv, max(m, 1), cfg.d), dtype=cca.core_dtype(qd.dtype), device=dev)
    cv = torch.empty_like(ck)
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[2].record(stream)
        cca.cca_pool_core(qd, kd, vd, ck, cv, cfg.g)
        if ev is not None:
            ev[0].record(stream)
        cca.cca_attn_prefill(qd, kd, vd, ck, cv, out, cfg.g, cfg.w)
        if ev is not None:
            ev[1].record(stream)

    t0 = time.perf_counter()
    n_warm = 0
    while n_warm < warmup or time.perf_counter() - t0 < min_warmup_s:
        step()
        n_warm += 1
        if n_warm % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # per step: prefill start (= pooling end), prefill end, pooling start
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(steps):
        step(evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    prefill_ms = [e[0].elapsed_time(e[1]) for e in evs]
    pool_each = [e[2].elapsed_time(e[0]) for e in evs]
    ms_step = total_ms / steps
    prefill_avg = sum(prefill_ms) / len(prefill_ms)
    pool_ms = sum(pool_each) / len(pool_each)
    assert torch.isfinite(out[0, :, -4:].float()).all()
    flops = prefill_flops(cfg)
    tflops = flops / (prefill_avg * 1e-3) / 1e12
    bf16 = cfg.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_VALU_TFLOPS
    rec = {
        "workload": cfg.name, "dtype": cfg.dtype, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
        "seq_len": cfg.L, "head_dim": cfg.d, "group": cfg.g, "window": cfg.w, "steps": steps,
        "warmup_steps": n_warm,
        "ms_per_step": ms_step, "tokens_per_s": cfg.B * cfg.L / (ms_step * 1e-3),
        "prefill_ms": prefill_avg, "pool_ms": pool_ms,
        "algorithmic_flops": flops, "achieved_TFLOP_per_s": tflops,
        "bound": "mfma" if bf16 else "alu", "peak": peak, "frac": tflops / peak,
        "kernel": "prefill_mfma_kernel" if bf16 else "prefill_valu_kernel",
        "pool_GB_per_s": pool_bytes(cfg) / (pool_ms * 1e-3) / 1e9 if pool_ms > 0 else None,
    }
    return rec, (qd, kd, vd), (ck, cv, out)


def bench_backward(cca, cfg, qd, kd, vd, steps=2, warmup=1):
    """Backward pass over the prefill workload: forward with row statistics,
    then cca_attn_backward timed with events over `steps` calls.  Algorithmic
    FLOPs: 10*d per visible (query head, key) pair (the five products of a
    flash-style backward: Q.K recomputed, dO.V, dS.K, dS^T.Q, P^T.dO).  The
    bf16 kernels execute 14*d per pair: the row-parallel dQ kernel recomputes
    Q.K and dO.V (6d with dS.K), the key-parallel dK dV kernel does 8d."""
    B, Hq, Hkv, L, d, g, w = cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, cfg.g, cfg.w
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(4242)
    dout = torch.randn((B, Hq, L, d), generator=gen, device=dev).to(torch.bfloat16)
    m = L // g
    ck = torch.empty((B, Hkv, m, d), dtype=cca.core_dtype(qd.dtype), device=dev)
    cv = torch.empty_like(ck)
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=dev)
    cca.cca_pool_core(qd, kd, vd, ck, cv, g)
    cca.cca_attn_prefill_train(qd, kd, vd, ck, cv, out, lse, g, w)
    dq = torch.empty((B, Hq, L, d), dtype=torch.float32, device=dev)
    dk = torch.empty((B, Hkv, L, d), dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws = torch.empty(cca.cca_attn_backward_workspace_bytes(B, Hq, Hkv, L, d, g, qd.dtype), dtype=torch.uint8,
                     device=dev)
    for _ in range(warmup):
        cca.cca_attn_backward(qd, kd, vd, ck, cv, out, lse, dout, dq, dk, dv, ws, g, w)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        cca.cca_attn_backward(qd, kd, vd, ck, cv, out, lse, dout, dq, dk, dv, ws, g, w)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert torch.isfinite(dq[0, :, -4:]).all() and torch.isfinite(dk[0, :, -4:]).all()
    pairs = B * Hq * visible_pairs(L, g, w)
    flops = 10.0 * d * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": cfg.name, "steps": steps, "ms_per_call": ms, "algorithmic_flops": flops,
            "achieved_TFLOP_per_s": tflops, "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
            "frac": tflops / PEAK_BF16_TFLOPS, "executed_mfma_flops": 14.0 * d * pairs,
            "mfma_busy": {k: measured_mfma_busy("backward_mfma_gqa_L131072", f"{k}_mfma_busy_fraction")
                          for k in ("dq", "dkv")},
            "note": "matrix-core kernels: bf16 operands for raw keys, fp16 for the cores (fp32 accumulate); "
                    "gradients fp32"}


def reference_rates(dev="cuda:0", n=16384, copy_bytes=1 << 30, read_rows=65536, reps=10):
    """Measured ceilings on this GPU next to the spec peaks, each timed with
    events over `reps` runs after one warm-up: a large dense bf16 GEMM through
    torch (hipBLASLt), a device-to-device copy (read + write), and two
    read-only streams -- the ceiling for kernels that only read, like decode:
    a bf16 matrix-vector product through torch (reads the [read_rows, n]
    matrix once, writes read_rows values) and torch's sum over a fp32 buffer
    of the same size (reads every byte once, writes one value).  The faster
    of the two is the read ceiling."""
    a = torch.randn((n, n), device=dev).to(torch.bfloat16)
    b = torch.randn((n, n), device=dev).to(torch.bfloat16)
    c = a @ b
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    mat = torch.empty((read_rows, n), dtype=torch.bfloat16, device=dev).uniform_(-1, 1)
    vec = torch.empty((n, 1), dtype=torch.bfloat16, device=dev).uniform_(-1, 1)
    y = mat @ vec
    read_bytes = mat.numel() * mat.element_size()
    rd = torch.ones(read_bytes // 4, dtype=torch.float32, device=dev)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    torch.sum(rd, dim=0, out=acc)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    e[0].record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e[1].record()
    for _ in range(reps):
        dst.copy_(src)
    e[2].record()
    for _ in range(reps):
        torch.matmul(mat, vec, out=y)
    e[3].record()
    for _ in range(reps):
        torch.sum(rd, dim=0, out=acc)
    e[4].record()
    torch.cuda.synchronize()
    gemm_ms = e[0].elapsed_time(e[1]) / reps
    copy_ms = e[1].elapsed_time(e[2]) / reps
    gemv_ms = e[2].elapsed_time(e[3]) / reps
    sum_ms = e[3].elapsed_time(e[4]) / reps
    del a, b, c, src, dst, mat, vec, y, rd, acc
    torch.cuda.empty_cache()
    gemv_gbs = read_bytes / (gemv_ms * 1e-3) / 1e9
    sum_gbs = read_bytes / (sum_ms * 1e-3) / 1e9
    return {"bf16_gemm_TFLOP_per_s": 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12, "gemm_shape": f"{n}x{n}x{n}",
            "d2d_copy_GB_per_s": 2.0 * copy_bytes / (copy_ms * 1e-3) / 1e9,
            "copy_bytes": copy_bytes, "copy_note": "read + write bytes per copy",
            "read_only_GB_per_s": max(gemv_gbs, sum_gbs), "read_bytes": read_bytes,
            "gemv_read_GB_per_s": gemv_gbs, "sum_read_GB_per_s": sum_gbs,
            "read_note": f"faster of a bf16 [{read_rows}x{n}] matrix-vector product and a fp32 sum, "
                         "bytes read per pass"}


def mfma_ceiling(dev="cuda:0", iters=50000, reps=3, operand_sets=4):
    """The rate the matrix cores sustain on this chip doing nothing else:
    libcca_probe.so's kernel (one 8-wave workgroup per compute unit, back-to-back
    32x32x16 bf16 MFMAs on random register operands that rotate over four sets),
    timed with events on torch's stream after one short warm-up launch.  The
    operands are random because the chip's power, and with it the clock, depends
    on the bits the multipliers see: constant operands run much faster than any
    real kernel can."""
    import ctypes
    path = os.path.join(ROOT, "sparse_long_context_cca_amd", "libcca_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.cca_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                   ctypes.c_void_p]
    blocks = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.cca_probe_mfma(out.data_ptr(), blocks, iters // 10, operand_sets, 1, stream) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        assert lib.cca_probe_mfma(out.data_ptr(), blocks, iters, operand_sets, 2 + r, stream) == 0
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = blocks * 8.0 * iters * 16 * 32768
    return {"mfma_random_TFLOP_per_s": flops / (ms * 1e-3) / 1e12, "mfma_probe_ms": ms,
            "mfma_note": f"{blocks} workgroups x 8 waves, back-to-back v_mfma_f32_32x32x16_bf16 on random "
                         f"register operands rotating over {operand_sets} sets (libcca_probe.so)"}


def bench_decode(cca, cfg, steps_timed=True):
    """256 sequential decode steps over a 65536-token cache; one timed region."""
    B, Hq, Hkv, d, g, w, L, S = cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.g, cfg.w, cfg.L, cfg.decode_steps
    dev = "cuda:0"
    x = cca_inputs.decode_inputs(cfg)
    R, m_cap = w, (L + S) // g
    kd, vd = x["k"].to(dev), x["v"].to(dev)
    qfull = torch.zeros((B, Hq, L, d), dtype=torch.bfloat16, device=dev)
    qfull[:, :, g - 1::g] = x["q_ends"].to(dev)
    ck = torch.zeros((B, Hkv, m_cap, d), dtype=cca.core_dtype(torch.bfloat16), device=dev)
    cv = torch.zeros_like(ck)
    cca.cca_pool_core(qfull, kd[:, :, :L].contiguous(), vd[:, :, :L].contiguous(), ck, cv, g)
    del qfull
    rk = torch.empty((B, Hkv, R, d), dtype=torch.bfloat16, device=dev)
    rv = torch.empty_like(rk)
    slots = torch.arange(L - R, L, device=dev) % R
    rk[:, :, slots] = kd[:, :, L - R:L]
    rv[:, :, slots] = vd[:, :, L - R:L]
    ring0 = (rk.clone(), rv.clone())
    pos = torch.full((B,), L, dtype=torch.int32, device=dev)
    ws = torch.empty(cca.cca_decode_workspace_bytes(B, Hq, Hkv, d, m_cap, g, w), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    qs = x["q_steps"].to(dev).permute(2, 0, 1, 3).contiguous()     # [S, B, Hq, d]
    ks = kd[:, :, L:L + S].permute(2, 0, 1, 3).contiguous()         # [S, B, Hkv, d]
    vs = vd[:, :, L:L + S].permute(2, 0, 1, 3).contiguous()

    def run_all():
        for i in range(S):
            cca.cca_attn_decode(qs[i], ks[i], vs[i], rk, rv, ck, cv, pos, out, ws, g, w, advance_pos=True)

    def reset():
        pos.fill_(L)
        rk.copy_(ring0[0])
        rv.copy_(ring0[1])

    run_all()          # warm-up pass
    reset()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run_all()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    assert pos.tolist() == [L + S] * B
    assert torch.isfinite(out.float()).all()
    out_eager = out.clone()
    total_bytes = sum(decode_step_bytes(cfg, L + i) for i in range(S))
    gbs = total_bytes / (ms * 1e-3) / 1e9

    # the same 256 steps captured once in a HIP graph and replayed (no host
    # launch work between steps; pos advances on the device)
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_all()
    reset()
    torch.cuda.synchronize()
    graph.replay()                      # warm replay
    reset()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_g = e0.elapsed_time(e1)
    assert pos.tolist() == [L + S] * B
    assert torch.equal(out, out_eager), "graph replay differs from eager decode"
    gbs_g = total_bytes / (ms_g * 1e-3) / 1e9
    return {
        "workload": cfg.name,
        "steps": S,
        "us_per_step": ms * 1e3 / S,
        "GB_per_s": gbs,
        "hbm_frac": gbs / PEAK_HBM_GBS,
        "us_per_step_graph": ms_g * 1e3 / S,
        "GB_per_s_graph": gbs_g,
        "hbm_frac_graph": gbs_g / PEAK_HBM_GBS,
        "algorithmic_bytes_per_step": total_bytes / S,
        "traffic_per_step": measured_traffic("decode_mfma_b8_ctx65536"),
        "launches_per_step": 2,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="first run one device-to-device copy of this many bytes (a counter "
                         "calibration reference for FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only (it has no sharding or collectives); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import sparse_long_context_cca_amd as cca
    cca.load()
    dev = "cuda:0"
    if args.copy_bytes:
        n = args.copy_bytes // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = cca_inputs.CONFIGS[4]
    print(f"[bench] generating {cfg.name}", file=sys.stderr, flush=True)
    q, k, v = cca_inputs.prefill_inputs(cfg)
    print(f"[bench] {cfg.name}: warmup {args.warmup}, timing {args.steps} steps", file=sys.stderr, flush=True)
    head, (qd, kd, vd), (ck, cv, out) = bench_prefill(cca, cfg, args.steps, args.warmup,
                                                      (q.to(dev), k.to(dev), v.to(dev)))
    ms_step, prefill_avg, pool_ms = head["ms_per_step"], head["prefill_ms"], head["pool_ms"]
    flops, tflops = head["algorithmic_flops"], head["achieved_TFLOP_per_s"]
    tokens = cfg.B * cfg.L
    result = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. normal Q/K/V, bf16)",
        "config": {"workload": cfg.name, "batch": cfg.B, "q_heads": cfg.Hq, "kv_heads": cfg.Hkv,
                   "seq_len": cfg.L, "head_dim": cfg.d, "group": cfg.g, "window": cfg.w},
        "roofline": {
            "bound": "mfma",
            "kernel": "prefill_mfma_kernel<128,1,8,0>",
            "achieved": tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / PEAK_BF16_TFLOPS,
            "traffic": measured_traffic("prefill_mfma_gqa_L131072"),
            "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "mfma_busy": measured_mfma_busy("prefill_mfma_gqa_L131072"),
            "algorithmic_flops_per_launch": flops,
            "avg_launch_ms": prefill_avg,
        },
        "pool": {"ms": pool_ms, "algorithmic_bytes": pool_bytes(cfg),
                 "traffic": measured_traffic("pool_gqa_L131072"),
                 "GB_per_s": pool_bytes(cfg) / (pool_ms * 1e-3) / 1e9 if pool_ms > 0 else None},
    }
    del out, ck, cv
    torch.cuda.empty_cache()
    # The other prefill workloads, each warmed up for at least 0.3 s: with
    # three warm-up steps the MHA 32K prefill's timed launches still ran
    # 1.56 -> 1.23 ms while the clock climbed back after the input generation.
    if not args.no_configs:
        # every prefill workload, the headline one included, in one list
        recs = []
        torch.cuda.empty_cache()
        for number in (1, 2, 3):
            c = cca_inputs.CONFIGS[number]
            print(f"[bench] prefill workload {c.name}", file=sys.stderr, flush=True)
            rec, dev_in, dev_out = bench_prefill(cca, c, steps=10 if number > 1 else 20, warmup=3,
                                                 min_warmup_s=0.3)
            recs.append(rec)
            del dev_in, dev_out
            torch.cuda.empty_cache()
        recs.append(head)
        result["prefill_configs"] = recs
    if not args.no_backward:
        print("[bench] backward", file=sys.stderr, flush=True)
        result["backward"] = bench_backward(cca, cfg, qd, kd, vd)
    if not args.no_decode:
        qd = kd = vd = None
        torch.cuda.empty_cache()
        print("[bench] decode", file=sys.stderr, flush=True)
        result["decode"] = bench_decode(cca, cca_inputs.CONFIGS[5])
    # measured ceilings: the prefill against a large bf16 GEMM, pooling and
    # decode against a device-to-device copy
    print("[bench] reference rates", file=sys.stderr, flush=True)
    ref = reference_rates()
    ceiling = mfma_ceiling()
    if ceiling is not None:
        ref.update(ceiling)
    result["reference_rates"] = ref
    result["roofline"]["frac_of_measured_gemm"] = tflops / ref["bf16_gemm_TFLOP_per_s"]
    if ceiling is not None:
        result["roofline"]["frac_of_mfma_ceiling"] = tflops / ceiling["mfma_random_TFLOP_per_s"]
    if result["pool"]["GB_per_s"]:
        result["pool"]["frac_of_measured_copy"] = result["pool"]["GB_per_s"] / ref["d2d_copy_GB_per_s"]
    if "decode" in result:
        result["decode"]["frac_of_measured_copy"] = result["decode"]["GB_per_s"] / ref["d2d_copy_GB_per_s"]
        result["decode"]["frac_of_measured_read"] = result["decode"]["GB_per_s"] / ref["read_only_GB_per_s"]
    if not args.no_cpu:
        print("[bench] cpu oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_oracle_baseline(cfg, q, k, v)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
