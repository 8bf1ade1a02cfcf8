"""The Python binding refuses tensors that do not match the sizes it passes
to the C ABI (CPU only: every check fires before the library is called, so no
kernel is launched).  Shapes and dtypes are checked before the device, which
lets host tensors exercise those checks here."""
from __future__ import annotations

import pytest
import torch

import sparse_long_context_cca_amd as cca
from sparse_long_context_cca_amd import _lib

INV = _lib.CCA_ERR_INVALID_ARG


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


F16 = torch.float16  # the core cache of bf16 inputs


def prefill_args(B=1, Hq=4, Hkv=2, L=64, d=64, m_cap=4):
    return dict(q=t(B, Hq, L, d), k=t(B, Hkv, L, d), v=t(B, Hkv, L, d), core_k=t(B, Hkv, m_cap, d, dtype=F16),
                core_v=t(B, Hkv, m_cap, d, dtype=F16), out=t(B, Hq, L, d))


def raises(fn, match, **kw):
    with pytest.raises(cca.CCAError, match=match) as ei:
        fn(**kw)
    assert ei.value.status == INV


@pytest.mark.parametrize("change,match", [
    (dict(k=t(1, 2, 63, 64)), "k has shape"),             # k shorter than q's L
    (dict(v=t(1, 2, 64, 128)), "v has shape"),            # head dim differs
    (dict(out=t(1, 4, 32, 64)), "out has shape"),         # output too small
    (dict(core_v=t(1, 2, 3, 64, dtype=F16)), "core_v has shape"),  # cores of different capacity
    (dict(core_k=t(1, 2, 4, 64), core_v=t(1, 2, 4, 64)), "core_k has dtype"),  # bf16 cores: fp16 expected
    (dict(k=t(1, 2, 64, 64, dtype=torch.float32), v=t(1, 2, 64, 64, dtype=torch.float32)), "k has dtype"),
    (dict(out=t(1, 4, 64, 64, dtype=torch.float16)), "out has dtype"),
    (dict(q=t(4, 64, 64)), "q must be a 4-d tensor"),
])
def test_prefill_refuses_mismatched_tensors(change, match):
    a = prefill_args()
    a.update(change)
    raises(lambda **kw: cca.cca_attn_prefill(g=16, w=8, **kw), match, **a)


def test_host_tensors_are_refused():
    raises(lambda **kw: cca.cca_attn_prefill(g=16, w=8, **kw), "not a GPU tensor", **prefill_args())


def test_pool_refuses_mismatched_tensors():
    a = prefill_args()
    raises(lambda: cca.cca_pool_core(a["q"], a["k"], t(1, 2, 60, 64), a["core_k"], a["core_v"], 16),
           "v has shape")
    raises(lambda: cca.cca_pool_core(a["q"], a["k"], a["v"], a["core_k"], a["core_v"], 16,
                                     weights=t(1, 2, 4, 8, dtype=torch.float32)), "weights has shape")


def test_decode_refuses_mismatched_tensors():
    B, Hq, Hkv, d, R, m = 2, 4, 2, 64, 16, 8
    base = dict(q_t=t(B, Hq, d), k_t=t(B, Hkv, d), v_t=t(B, Hkv, d), ring_k=t(B, Hkv, R, d),
                ring_v=t(B, Hkv, R, d), core_k=t(B, Hkv, m, d, dtype=F16), core_v=t(B, Hkv, m, d, dtype=F16),
                pos=torch.zeros(B, dtype=torch.int32), out=t(B, Hq, d), workspace=t(64, dtype=torch.uint8))
    run = lambda **kw: cca.cca_attn_decode(g=4, w=8, **kw)
    raises(run, "pos has dtype", **{**base, "pos": torch.zeros(B, dtype=torch.int64)})
    raises(run, "pos has shape", **{**base, "pos": torch.zeros(B + 1, dtype=torch.int32)})
    raises(run, "ring_v has shape", **{**base, "ring_v": t(B, Hkv, R - 1, d)})
    raises(run, "core_v has dtype", **{**base, "core_v": t(B, Hkv, m, d)})
    raises(run, "not a GPU tensor", **base)


def test_backward_refuses_mismatched_tensors():
    a = prefill_args()
    B, Hq, Hkv, L, d = 1, 4, 2, 64, 64
    f32 = torch.float32
    kw = dict(q=a["q"], k=a["k"], v=a["v"], core_k=a["core_k"], core_v=a["core_v"], out=a["out"],
              lse=t(B, Hq, L, dtype=f32), dout=t(B, Hq, L, d), dq=t(B, Hq, L, d, dtype=f32),
              dk=t(B, Hkv, L, d, dtype=f32), dv=t(B, Hkv, L, d, dtype=f32), workspace=t(16, dtype=torch.uint8))
    run = lambda **x: cca.cca_attn_backward(g=16, w=8, **x)
    raises(run, "dq has dtype", **{**kw, "dq": t(B, Hq, L, d)})
    raises(run, "out has dtype", **{**kw, "out": t(B, Hq, L, d, dtype=f32)})
    raises(run, "lse has shape", **{**kw, "lse": t(B, Hq, L - 1, dtype=f32)})


def test_chunk_and_ring_refuse_mismatched_tensors():
    a = prefill_args()
    i32 = torch.int32
    raises(lambda: cca.cca_attn_prefill_chunk(a["q"], a["k"], a["v"], a["core_k"], a["core_v"], a["out"], 16, 8,
                                              torch.zeros(2, dtype=i32), torch.zeros(1, dtype=i32)),
           "q_start has shape")
    raises(lambda: cca.cca_cache_fill_ring(a["k"], a["v"], t(1, 2, 8, 64), t(1, 2, 8, 32),
                                           torch.zeros(1, dtype=i32)), "ring_v has shape")


def test_core_dtype():
    """The core cache holds fp32 cores for fp32 inputs and fp16 cores for bf16 inputs."""
    assert cca.core_dtype(torch.float32) == torch.float32
    assert cca.core_dtype(torch.bfloat16) == torch.float16
    with pytest.raises(cca.CCAError):
        cca.core_dtype(torch.float16)
