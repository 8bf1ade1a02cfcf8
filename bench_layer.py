#!/usr/bin/env python3
"""Layer-level timing of one CCA attention block on one MI355X (context only).

The pages report end-to-end first-token latency (FTL) of whole models on an
A800 (paper card, "Key results"; rebuttal, answer on 128K context); nothing of
that is a kernel number.  This script relates the CCA kernels to that metric:
it times the attention block of one layer at a model's head shapes,

    x [L, hidden] --(fused QKV GEMM)--> Q, K, V --(RoPE)--> cca_pool_core +
    cca_attn_prefill --(O projection GEMM)--> y [L, hidden]

with synthetic bf16 weights (no checkpoints) and synthetic activations.  The
GEMMs run through torch (hipBLASLt); RoPE (rotate-half form) and the head
layout changes are torch elementwise/copy kernels; the CCA steps are this
library's kernels.  The MLP and norms of a full layer are not included.

Prints ONE JSON line with per-component times.  Flags: --model
{llama3_1_8b,llama2_7b}, --seq-len L, --steps K, --warmup W.
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MODELS = {
    # hidden, query heads, kv heads, head dim, RoPE base
    "llama3_1_8b": dict(hidden=4096, Hq=32, Hkv=8, d=128, rope_base=500000.0),
    "llama2_7b": dict(hidden=4096, Hq=32, Hkv=32, d=128, rope_base=10000.0),
}


def make_weights(spec, seed=0, device="cuda:0"):
    """Synthetic bf16 projection weights, N(0, 1/hidden) (no trained weights exist here)."""
    gen = torch.Generator(device="cpu").manual_seed(seed)
    h, Hq, Hkv, d = spec["hidden"], spec["Hq"], spec["Hkv"], spec["d"]
    std = h ** -0.5
    wqkv = (torch.randn(h, (Hq + 2 * Hkv) * d, generator=gen) * std).to(torch.bfloat16)
    wo = (torch.randn(Hq * d, h, generator=gen) * (Hq * d) ** -0.5).to(torch.bfloat16)
    return wqkv.to(device), wo.to(device)


def rope_tables(L, d, base, device):
    inv = 1.0 / (base ** (torch.arange(0, d, 2, dtype=torch.float64) / d))
    ang = torch.arange(L, dtype=torch.float64)[:, None] * inv[None, :]
    return torch.cos(ang).float().to(device), torch.sin(ang).float().to(device)


def apply_rope(x, cos, sin):
    """Rotate-half RoPE on x [B, H, L, d] (fp32 math, result in x's dtype)."""
    d2 = x.shape[-1] // 2
    xf = x.float()
    x1, x2 = xf[..., :d2], xf[..., d2:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1).to(x.dtype)


def attention_block(x, wqkv, wo, spec, g, w, cos, sin, cca, events=None):
    """y = O-proj(CCA(RoPE(QKV(x)))) for x [L, hidden] (batch 1).  When
    `events` is a list, CUDA events are recorded between the stages."""
    L = x.shape[0]
    Hq, Hkv, d = spec["Hq"], spec["Hkv"], spec["d"]
    rec = (lambda: events.append(torch.cuda.Event(enable_timing=True)) or events[-1].record()) \
        if events is not None else (lambda: None)
    rec()
    qkv = x @ wqkv                                                        # [L, (Hq+2Hkv) d]
    rec()
    q = qkv[:, : Hq * d].view(L, Hq, d).transpose(0, 1).unsqueeze(0)
    k = qkv[:, Hq * d : (Hq + Hkv) * d].view(L, Hkv, d).transpose(0, 1).unsqueeze(0)
    v = qkv[:, (Hq + Hkv) * d :].view(L, Hkv, d).transpose(0, 1).unsqueeze(0).contiguous()
    q = apply_rope(q, cos, sin).contiguous()
    k = apply_rope(k, cos, sin).contiguous()
    rec()
    m = L // g
    ck = torch.empty((1, Hkv, max(m, 1), d), dtype=cca.core_dtype(x.dtype), device=x.device)
    cv = torch.empty_like(ck)
    o = torch.empty((1, Hq, L, d), dtype=x.dtype, device=x.device)
    cca.cca_pool_core(q, k, v, ck, cv, g)
    rec()
    cca.cca_attn_prefill(q, k, v, ck, cv, o, g, w)
    rec()
    y = o[0].transpose(0, 1).reshape(L, Hq * d) @ wo                      # [L, hidden]
    rec()
    return y, (qkv, q, k, v, ck, cv, o)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--model", default="llama3_1_8b", choices=sorted(MODELS))
    ap.add_argument("--seq-len", type=int, default=131072)
    ap.add_argument("--group", type=int, default=16)
    ap.add_argument("--window", type=int, default=1024)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    args = ap.parse_args()

    import sparse_long_context_cca_amd as cca
    cca.load()
    dev = "cuda:0"
    spec = MODELS[args.model]
    L, g, w = args.seq_len, args.group, args.window
    wqkv, wo = make_weights(spec, device=dev)
    gen = torch.Generator(device="cpu").manual_seed(1)
    x = torch.randn(L, spec["hidden"], generator=gen).to(torch.bfloat16).to(dev)
    cos, sin = rope_tables(L, spec["d"], spec["rope_base"], dev)
    for _ in range(args.warmup):
        attention_block(x, wqkv, wo, spec, g, w, cos, sin, cca)
    torch.cuda.synchronize()
    names = ["qkv_gemm", "layout_rope", "cca_pool", "cca_prefill", "o_proj_gemm"]
    acc = {n: 0.0 for n in names}
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        ev = []
        attention_block(x, wqkv, wo, spec, g, w, cos, sin, cca, events=ev)
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n] += ev[i].elapsed_time(ev[i + 1])
    t1.record()
    torch.cuda.synchronize()
    comp = {n: acc[n] / args.steps for n in names}
    block = sum(comp.values())
    h, Hq, Hkv, d = spec["hidden"], spec["Hq"], spec["Hkv"], spec["d"]
    gemm_flops = 2.0 * L * h * (Hq + 2 * Hkv) * d + 2.0 * L * Hq * d * h
    print(json.dumps({
        "metric": "attention-block latency per layer (QKV GEMM + RoPE + CCA + O-proj), context for FTL",
        "value": block, "unit": "ms", "higher_is_better": False, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "dtype": "bf16", "data": "synthetic activations and random-init weights",
        "config": {"workload": f"{args.model}_attention_block_L{L}", "seq_len": L, "hidden": h, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "group": g, "window": w},
        "components_ms": comp,
        "cca_share": (comp["cca_pool"] + comp["cca_prefill"]) / block,
        "gemm_TFLOP_per_s": gemm_flops / ((comp["qkv_gemm"] + comp["o_proj_gemm"]) * 1e-3) / 1e12,
        "note": "context only: the pages' FTL is a whole-model figure on another GPU; MLP and norms excluded",
    }), flush=True)


if __name__ == "__main__":
    main()
