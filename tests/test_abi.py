"""C-ABI checks that need no GPU: the library loads, exports every function
include/cca.h declares, and rejects invalid arguments on the host before any
HIP call (so no pointer below is ever dereferenced)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from sparse_long_context_cca_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cca.h")
FAKE = 0x10000       # 16-byte aligned, never dereferenced: every call below fails validation
MIS = 0x10008        # misaligned
OK, INV, UNS, CAP = (_lib.CCA_OK, _lib.CCA_ERR_INVALID_ARG, _lib.CCA_ERR_UNSUPPORTED,
                     _lib.CCA_ERR_CAPACITY)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cca_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["cca_pool_core", "cca_attn_prefill", "cca_attn_decode", "cca_visibility_table",
              "cca_decode_workspace_bytes", "cca_status_string", "cca_last_error", "cca_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(cca_lib):
    for name in declared_functions():
        assert hasattr(cca_lib, name), f"libcca.so does not export {name}"
    assert sorted(_lib.EXPORTS) == declared_functions()


def test_version_and_status_strings(cca_lib):
    assert cca_lib.cca_version() >= 100
    assert cca_lib.cca_status_string(OK) == b"CCA_OK"
    assert cca_lib.cca_status_string(CAP) == b"CCA_ERR_CAPACITY"
    assert cca_lib.cca_status_string(99) == b"CCA_ERR_UNKNOWN"


P = ctypes.c_void_p


def pool(lib, q=FAKE, k=FAKE, v=FAKE, ck=FAKE, cv=FAKE, m_cap=64, wts=None, B=1, Hq=4, Hkv=2, L=1024,
         d=128, g=16, dt=1):
    return lib.cca_pool_core(P(q), P(k), P(v), P(ck), P(cv), m_cap, P(wts), B, Hq, Hkv, L, d, g, dt, None)


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, ck=FAKE, cv=FAKE, m_cap=64, out=FAKE, out_dt=1, B=1, Hq=4,
            Hkv=2, L=1024, d=128, g=16, w=64, dt=1, kernel=0):
    return lib.cca_attn_prefill_ex(P(q), P(k), P(v), P(ck), P(cv), m_cap, P(out), out_dt, B, Hq, Hkv,
                                   L, d, g, w, dt, kernel, None)


def decode(lib, q=FAKE, kt=FAKE, vt=FAKE, rk=FAKE, rv=FAKE, R=1024, ck=FAKE, cv=FAKE, m_cap=4096,
           pos=FAKE, adv=0, out=FAKE, out_dt=1, ws=FAKE, ws_bytes=1 << 30, B=2, Hq=8, Hkv=2, d=128,
           g=16, w=1024, dt=1):
    return lib.cca_attn_decode(P(q), P(kt), P(vt), P(rk), P(rv), R, P(ck), P(cv), m_cap, P(pos), adv,
                               P(out), out_dt, P(ws), ws_bytes, B, Hq, Hkv, d, g, w, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(k=0), INV), (dict(v=MIS), INV), (dict(L=0), INV), (dict(g=0), INV),
    (dict(B=0), INV), (dict(Hq=0), INV), (dict(dt=7), INV), (dict(d=96), UNS), (dict(Hq=3), UNS),
    (dict(m_cap=63), CAP), (dict(ck=None), INV), (dict(wts=MIS), INV),
    (dict(B=1 << 16, Hq=1 << 10, Hkv=1 << 10, L=1 << 12, m_cap=256), UNS),
    (dict(g=1 << 30), UNS), (dict(L=(1 << 30) + 1, d=64, Hq=2, Hkv=1, m_cap=1 << 30), UNS),
])
def test_pool_validation(cca_lib, kw, code):
    assert pool(cca_lib, **kw) == code
    assert cca_lib.cca_last_error() != b""


def test_pool_without_complete_group_is_a_no_op(cca_lib):
    # L < g: nothing to pool, nothing enqueued, even with NULL core buffers
    assert pool(cca_lib, L=15, ck=None, cv=None, m_cap=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(out=None), INV), (dict(w=0), INV), (dict(out_dt=5), INV), (dict(dt=0, out_dt=1), UNS),
    (dict(kernel=3), INV), (dict(dt=0, out_dt=0, kernel=2), UNS), (dict(d=32), UNS),
    (dict(Hkv=3), UNS), (dict(m_cap=10), CAP), (dict(cv=None), INV), (dict(q=MIS), INV),
    (dict(w=(1 << 30) + 1), UNS), (dict(g=(1 << 30) + 1), UNS),
])
def test_prefill_validation(cca_lib, kw, code):
    assert prefill(cca_lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(R=1023), CAP), (dict(R=8, w=4, g=16), CAP), (dict(ws_bytes=16), CAP), (dict(pos=None), INV),
    (dict(pos=FAKE + 2), INV), (dict(g=0), INV), (dict(w=0), INV), (dict(rk=None), INV),
    (dict(out_dt=0, dt=0, d=80), UNS), (dict(Hq=6, Hkv=4), UNS), (dict(m_cap=-1), INV),
    (dict(ck=None), INV), (dict(ws=None), INV), (dict(R=(1 << 30) + 1), UNS), (dict(g=(1 << 30) + 1), UNS),
    (dict(m_cap=(1 << 30) + 1), UNS),
])
def test_decode_validation(cca_lib, kw, code):
    assert decode(cca_lib, **kw) == code


def pool_ex(lib, mode, q=FAKE, k=FAKE, v=FAKE, ck=FAKE, cv=FAKE, m_cap=64, wts=None, B=1, Hq=4, Hkv=2,
            L=1024, d=128, g=16, dt=1):
    return lib.cca_pool_core_ex(P(q), P(k), P(v), P(ck), P(cv), m_cap, P(wts), B, Hq, Hkv, L, d, g, dt,
                                mode, None)


def decode_ex(lib, mode, **kw):
    a = dict(q=FAKE, kt=FAKE, vt=FAKE, rk=FAKE, rv=FAKE, R=1024, ck=FAKE, cv=FAKE, m_cap=4096, pos=FAKE,
             adv=0, out=FAKE, out_dt=1, ws=FAKE, ws_bytes=1 << 30, B=2, Hq=8, Hkv=2, d=128, g=16, w=1024,
             dt=1)
    a.update(kw)
    return lib.cca_attn_decode_ex(P(a["q"]), P(a["kt"]), P(a["vt"]), P(a["rk"]), P(a["rv"]), a["R"],
                                  P(a["ck"]), P(a["cv"]), a["m_cap"], P(a["pos"]), a["adv"], P(a["out"]),
                                  a["out_dt"], P(a["ws"]), a["ws_bytes"], a["B"], a["Hq"], a["Hkv"],
                                  a["d"], a["g"], a["w"], a["dt"], mode, None)


@pytest.mark.parametrize("mode,kw,code", [
    (-1, {}, INV), (4, {}, INV),                               # unknown rule
    (_lib.CCA_POOL_MAX, dict(wts=FAKE), INV),                  # max pooling has no weights
    (_lib.CCA_POOL_SOFTMAX_HEADS, dict(Hq=18, Hkv=2), UNS),    # per-head rule needs G <= 8
    (_lib.CCA_POOL_SOFTMAX, dict(q=None), INV),                # the softmax rules read q
    (_lib.CCA_POOL_SOFTMAX_HEADS, dict(q=None), INV),
    (_lib.CCA_POOL_MEAN, dict(q=None, L=15, ck=None, cv=None, m_cap=0), OK),  # q unread, nothing to pool
    (_lib.CCA_POOL_MAX, dict(q=None, m_cap=63), CAP),          # q unread: the next check speaks
])
def test_pool_mode_validation(cca_lib, mode, kw, code):
    assert pool_ex(cca_lib, mode, **kw) == code


@pytest.mark.parametrize("mode,kw,code", [
    (-1, {}, INV), (9, {}, INV), (_lib.CCA_POOL_SOFTMAX_HEADS, dict(Hq=18, Hkv=2), UNS),
    (_lib.CCA_POOL_MAX, dict(R=1023), CAP),
])
def test_decode_mode_validation(cca_lib, mode, kw, code):
    assert decode_ex(cca_lib, mode, **kw) == code


def pool_chunk(lib, q=FAKE, k=FAKE, v=FAKE, ck=FAKE, cv=FAKE, m_cap=64, qs=FAKE, ql=FAKE, B=2, Hq=4,
               Hkv=2, Lq=256, Lk=1024, d=128, g=16, dt=1, mode=0):
    return lib.cca_pool_core_chunk(P(q), P(k), P(v), P(ck), P(cv), m_cap, P(qs), P(ql), B, Hq, Hkv, Lq,
                                   Lk, d, g, dt, mode, None)


def prefill_chunk(lib, q=FAKE, k=FAKE, v=FAKE, ck=FAKE, cv=FAKE, m_cap=64, out=FAKE, out_dt=1, qs=FAKE,
                  ql=FAKE, B=2, Hq=4, Hkv=2, Lq=256, Lk=1024, d=128, g=16, w=64, dt=1):
    return lib.cca_attn_prefill_chunk(P(q), P(k), P(v), P(ck), P(cv), m_cap, P(out), out_dt, P(qs), P(ql),
                                      B, Hq, Hkv, Lq, Lk, d, g, w, dt, None)


def fill_ring(lib, k=FAKE, v=FAKE, rk=FAKE, rv=FAKE, R=1024, sl=FAKE, B=2, Hkv=2, Lk=4096, d=128, dt=1):
    return lib.cca_cache_fill_ring(P(k), P(v), P(rk), P(rv), R, P(sl), B, Hkv, Lk, d, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), INV), (dict(ql=FAKE + 2), INV), (dict(Lq=0), INV), (dict(Lk=0), INV), (dict(g=0), INV),
    (dict(mode=7), INV), (dict(q=None), INV), (dict(k=None), INV), (dict(m_cap=-1), INV),
    (dict(ck=None), INV), (dict(d=96), UNS), (dict(mode=1, Hq=18, Hkv=2), UNS),
    (dict(m_cap=0, ck=None, cv=None), OK),  # no core slot: nothing to do
    (dict(q=None, mode=_lib.CCA_POOL_MAX, m_cap=0), OK),
    (dict(g=(1 << 30) + 1), UNS), (dict(Lk=(1 << 30) + 1, d=64, B=1, Hq=1, Hkv=1), UNS),
])
def test_pool_chunk_validation(cca_lib, kw, code):
    assert pool_chunk(cca_lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(qs=None), INV), (dict(ql=None), INV), (dict(qs=FAKE + 1), INV), (dict(Lq=0), INV), (dict(w=0), INV),
    (dict(out=None), INV), (dict(m_cap=-1), INV), (dict(cv=None), INV), (dict(dt=0, out_dt=1), UNS),
    (dict(Hkv=3), UNS), (dict(out_dt=4), INV), (dict(w=(1 << 30) + 1), UNS),
])
def test_prefill_chunk_validation(cca_lib, kw, code):
    assert prefill_chunk(cca_lib, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), INV), (dict(Lk=0), INV), (dict(sl=None), INV), (dict(sl=FAKE + 2), INV), (dict(rk=None), INV),
    (dict(d=32), UNS), (dict(B=1 << 9, Hkv=1 << 8), UNS), (dict(R=(1 << 30) + 1, B=1, Hkv=1), UNS),
])
def test_fill_ring_validation(cca_lib, kw, code):
    assert fill_ring(cca_lib, **kw) == code


def test_decode_workspace_size(cca_lib):
    f = cca_lib.cca_decode_workspace_bytes
    n = f(8, 32, 8, 128, 4112, 16, 1024)
    assert n > 0 and n % 4 == 0
    assert n == f(8, 32, 8, 128, 4112, 16, 1024)     # deterministic
    for B in (1, 8, 16):  # whole split states: B * Hq * splits * (d + 2) floats
        nb = f(B, 32, 8, 128, 4112, 16, 1024)
        assert nb > 0 and nb % (B * 32 * 130 * 4) == 0
    assert f(0, 32, 8, 128, 4112, 16, 1024) == 0


@pytest.mark.parametrize("args,code", [((0, 16, 4), INV), ((10, 0, 4), INV), ((10, 4, 0), INV),
                                       ((10, 4, (1 << 30) + 1), UNS)])
def test_visibility_validation(cca_lib, args, code):
    assert cca_lib.cca_visibility_table(*args, P(FAKE), P(FAKE), P(FAKE), None) == code
    assert cca_lib.cca_visibility_table(10, 4, 4, P(None), P(FAKE), P(FAKE), None) == INV


def test_core_dtype_export(cca_lib):
    """fp32 inputs keep fp32 cores; bf16 inputs get fp16 cores; anything else is -1."""
    assert cca_lib.cca_core_dtype(0) == 0
    assert cca_lib.cca_core_dtype(1) == 2
    assert cca_lib.cca_core_dtype(2) == -1 and cca_lib.cca_core_dtype(-1) == -1


def test_backward_workspace_size(cca_lib):
    """fp32: row statistics + fp32 core gradients; bf16 adds fp16 copies of q and
    dout from a 256-byte boundary."""
    f = cca_lib.cca_attn_backward_workspace_bytes
    B, Hq, Hkv, L, d, g = 1, 32, 8, 1001, 128, 16
    f32_part = (2 * B * Hq * L + 2 * B * Hkv * (L // g) * d) * 4
    assert f(B, Hq, Hkv, L, d, g, 0) == f32_part
    assert f(B, Hq, Hkv, L, d, g, 1) == (f32_part + 255) // 256 * 256 + 2 * B * Hq * L * d * 2
    assert f(B, Hq, Hkv, L, d, g, 2) == 0 and f(0, Hq, Hkv, L, d, g, 1) == 0


def test_decode_scratch_rejects_states_beyond_its_array(cca_lib):
    """The allocation-free decode refuses shapes whose split states exceed its
    fixed array, before anything touches the GPU."""
    cap = cca_lib.cca_decode_scratch_bytes()
    assert cap == 16 << 20
    f = cca_lib.cca_decode_workspace_bytes
    B, Hq, Hkv, d, m_cap, g, w = 512, 64, 8, 128, 64, 16, 64
    assert f(B, Hq, Hkv, d, m_cap, g, w) > cap
    st = cca_lib.cca_attn_decode_scratch(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 64, P(FAKE), P(FAKE), m_cap,
                                         P(FAKE), 1, P(FAKE), 1, B, Hq, Hkv, d, g, w, 1, 0, None)
    assert st == CAP
    assert b"scratch" in cca_lib.cca_last_error()
