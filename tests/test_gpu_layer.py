"""GPU check of the layer-level bench's attention block (bench_layer.py) at a
small length: each stage against a CPU reference of its own.

  * Q, K, V after the QKV GEMM and RoPE: RoPE written here as a complex
    rotation of the pairs (i, i + d/2) in fp64, applied to the GPU's own QKV
    GEMM output;
  * the CCA output: the fp64 oracle on the GPU's Q, K, V (2e-2, as the parity
    tests);
  * the output projection: an fp32 GEMM of the GPU's CCA output.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import bench_layer
import oracle.cca_oracle as orc
import sparse_long_context_cca_amd as cca

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("model", ["llama3_1_8b", "llama2_7b"])
def test_attention_block_stages(model):
    print(f"attention block {model}", flush=True)
    spec = bench_layer.MODELS[model]
    L, g, w = 640, 16, 64
    wqkv, wo = bench_layer.make_weights(spec, seed=3, device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(4)
    x = torch.randn(L, spec["hidden"], generator=gen).to(torch.bfloat16).to(DEV)
    cos, sin = bench_layer.rope_tables(L, spec["d"], spec["rope_base"], DEV)
    y, (qkv_gpu, q, k, v, ck, cv, o) = bench_layer.attention_block(x, wqkv, wo, spec, g, w, cos, sin, cca)
    torch.cuda.synchronize()
    Hq, Hkv, d = spec["Hq"], spec["Hkv"], spec["d"]

    # RoPE of the GPU's QKV GEMM output, as a complex rotation in fp64
    assert float((qkv_gpu.float() - (x.float() @ wqkv.float())).abs().max()) <= 0.05, "QKV GEMM"
    qkv = qkv_gpu.double().cpu().numpy()
    pos = np.arange(L, dtype=np.float64)[:, None]
    theta = pos * spec["rope_base"] ** (-np.arange(0, d, 2, dtype=np.float64) / d)[None, :]
    rot = np.exp(1j * theta)                                                  # [L, d/2]

    def rope_ref(block, H):
        z = block.reshape(L, H, d)
        c = (z[..., : d // 2] + 1j * z[..., d // 2 :]) * rot[:, None, :]
        return np.concatenate([c.real, c.imag], axis=-1).transpose(1, 0, 2)   # [H, L, d]

    q_ref = rope_ref(qkv[:, : Hq * d], Hq)
    k_ref = rope_ref(qkv[:, Hq * d : (Hq + Hkv) * d], Hkv)
    v_ref = qkv[:, (Hq + Hkv) * d :].reshape(L, Hkv, d).transpose(1, 0, 2)
    for name, got, ref in (("q", q, q_ref), ("k", k, k_ref), ("v", v, v_ref)):
        g64 = got[0].double().cpu().numpy()
        bound = np.abs(ref) * 2.0 ** -7 + 1e-5    # bf16 rounding of the fp32 RoPE result
        assert np.all(np.abs(g64 - ref) <= bound), f"{name} after RoPE"

    # CCA on the GPU's Q, K, V against the oracle
    Q, K, V = (t.float().cpu().numpy() for t in (q, k, v))
    CK, CV, _ = orc.pool_core(Q, K, V, g)
    ref = orc.attn_prefill(Q, K, V, CK, CV, g, w)
    e = float(np.abs(o.double().cpu().numpy() - ref).max())
    print(f"  CCA max abs err {e:.3e}", flush=True)
    assert e <= 2e-2

    # output projection: fp32 GEMM of the GPU's attention output
    o2 = o[0].transpose(0, 1).reshape(L, Hq * d).float().cpu()
    y_ref = (o2 @ wo.float().cpu()).numpy()
    y64 = y.double().cpu().numpy()
    assert np.all(np.abs(y64 - y_ref) <= np.abs(y_ref) * 2.0 ** -7 + 1e-3)
