"""ctypes binding of libcca.so (declared in include/cca.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's HIP
kernels.  There is no fallback: if libcca.so is missing or does not load,
importing the entry points raises.

The C ABI sees pointers and sizes only, so the binding checks what it cannot:
every tensor's shape against the sizes passed, its dtype, that it is
contiguous and that it lives on the same GPU as the others.  A mismatch raises
CCAError before anything reaches the library.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# CCA_LIB_PATH selects another build of the same library (the CPU tests point
# it at the host-sanitized build); there is no fallback either way.
LIB_PATH = os.environ.get("CCA_LIB_PATH") or os.path.join(_PKG, "libcca.so")

CCA_OK, CCA_ERR_INVALID_ARG, CCA_ERR_UNSUPPORTED, CCA_ERR_CAPACITY, CCA_ERR_HIP = range(5)
CCA_F32, CCA_BF16, CCA_F16 = 0, 1, 2
CCA_POOL_SOFTMAX, CCA_POOL_SOFTMAX_HEADS, CCA_POOL_MEAN, CCA_POOL_MAX = range(4)

EXPORTS = ["cca_version", "cca_status_string", "cca_last_error", "cca_core_dtype", "cca_visibility_table",
           "cca_pool_core", "cca_pool_core_ex", "cca_attn_prefill", "cca_attn_prefill_ex",
           "cca_decode_workspace_bytes", "cca_attn_decode", "cca_attn_decode_ex",
           "cca_pool_core_chunk", "cca_attn_prefill_chunk", "cca_cache_fill_ring",
           "cca_attn_prefill_train", "cca_attn_backward_workspace_bytes", "cca_attn_backward",
           "cca_attn_decode_scratch", "cca_decode_scratch_bytes"]


class CCAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Loads libcca.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m sparse_long_context_cca_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "cca_version": ([], I),
        "cca_status_string": ([I], ctypes.c_char_p),
        "cca_last_error": ([], ctypes.c_char_p),
        "cca_core_dtype": ([I], I),
        "cca_visibility_table": ([I, I, I, P, P, P, P], I),
        "cca_pool_core": ([P, P, P, P, P, I, P, I, I, I, I, I, I, I, P], I),
        "cca_pool_core_ex": ([P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, P], I),
        "cca_attn_prefill": ([P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, I, P], I),
        "cca_attn_prefill_ex": ([P, P, P, P, P, I, P, I, I, I, I, I, I, I, I, I, I, P], I),
        "cca_decode_workspace_bytes": ([I, I, I, I, I, I, I], S),
        "cca_attn_decode": ([P, P, P, P, P, I, P, P, I, P, I, P, I, P, S, I, I, I, I, I, I, I, P], I),
        "cca_attn_decode_ex": ([P, P, P, P, P, I, P, P, I, P, I, P, I, P, S, I, I, I, I, I, I, I, I, P], I),
        "cca_pool_core_chunk": ([P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, I, I, P], I),
        "cca_attn_prefill_chunk": ([P, P, P, P, P, I, P, I, P, P, I, I, I, I, I, I, I, I, I, P], I),
        "cca_cache_fill_ring": ([P, P, P, P, I, P, I, I, I, I, I, P], I),
        "cca_attn_prefill_train": ([P, P, P, P, P, I, P, I, P, I, I, I, I, I, I, I, I, P], I),
        "cca_attn_backward_workspace_bytes": ([I, I, I, I, I, I, I], S),
        "cca_attn_backward": ([P, P, P, P, P, I, P, P, P, P, P, P, P, S, I, I, I, I, I, I, I, I, I, P], I),
        "cca_attn_decode_scratch": ([P, P, P, P, P, I, P, P, I, P, I, P, I, I, I, I, I, I, I, I, I, P], I),
        "cca_decode_scratch_bytes": ([], S),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load().cca_status_string(status).decode()


def _check(status: int) -> None:
    if status != CCA_OK:
        raise CCAError(status, load().cca_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CCA_F32
    if t.dtype == torch.bfloat16:
        return CCA_BF16
    raise CCAError(CCA_ERR_UNSUPPORTED, f"dtype {t.dtype} not supported")


def _ptr(t):
    if t is None:
        return None
    if not t.is_contiguous():
        raise CCAError(CCA_ERR_INVALID_ARG, "tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


_FLOAT = (torch.float32, torch.bfloat16)
_TORCH_OF = {CCA_F32: torch.float32, CCA_BF16: torch.bfloat16, CCA_F16: torch.float16}


def core_dtype(dtype: torch.dtype) -> torch.dtype:
    """torch dtype of the core cache for inputs of ``dtype`` (cca_core_dtype: fp32 for fp32,
    fp16 for bf16)."""
    if dtype not in _FLOAT:
        raise CCAError(CCA_ERR_UNSUPPORTED, f"dtype {dtype} not supported")
    return _TORCH_OF[load().cca_core_dtype(CCA_F32 if dtype == torch.float32 else CCA_BF16)]


def _expect(tensors) -> None:
    """tensors: (name, tensor or None, shape, allowed dtypes or None) per argument.  Shapes
    and dtypes are checked first, then that every tensor is a contiguous tensor on one GPU."""
    dev = None
    for name, t, shape, dtypes in tensors:
        if t is None:
            raise CCAError(CCA_ERR_INVALID_ARG, f"{name} is missing")
        if tuple(t.shape) != tuple(shape):
            raise CCAError(CCA_ERR_INVALID_ARG, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtypes is not None and t.dtype not in dtypes:
            raise CCAError(CCA_ERR_INVALID_ARG, f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    for name, t, _, _ in tensors:
        if t.device.type != "cuda":
            raise CCAError(CCA_ERR_INVALID_ARG, f"{name} is not a GPU tensor ({t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise CCAError(CCA_ERR_INVALID_ARG, f"{name} is on {t.device}, the others on {dev}")
        if not t.is_contiguous():
            raise CCAError(CCA_ERR_INVALID_ARG, f"{name} is not contiguous")


def _dims(t, n, name):
    if t is None or t.dim() != n:
        raise CCAError(CCA_ERR_INVALID_ARG, f"{name} must be a {n}-d tensor")
    return tuple(t.shape)


def _workspace(name, t):
    if t is None:
        return []
    return [(name, t, tuple(t.shape), None)]


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------ entry points


def cca_version() -> int:
    return load().cca_version()


def cca_visibility_table(L: int, g: int, w: int, n_core: torch.Tensor, win_lo: torch.Tensor,
                         group_last: torch.Tensor | None, stream=None) -> None:
    i32 = (torch.int32,)
    spec = [("n_core", n_core, (L,), i32), ("win_lo", win_lo, (L,), i32)]
    if g > 0 and L // g > 0:  # group_last is not written (and may be None) when L < g
        spec.append(("group_last", group_last, (L // g,), i32))
    _expect(spec)
    _check(load().cca_visibility_table(L, g, w, _ptr(n_core), _ptr(win_lo), _ptr(group_last),
                                       _stream(stream)))


def cca_pool_core(q, k, v, core_k, core_v, g: int, weights=None, mode: int = CCA_POOL_SOFTMAX,
                  stream=None) -> None:
    """q [B,Hq,L,d]; k, v [B,Hkv,L,d]; core_k, core_v [B,Hkv,m_cap,d] in core_dtype(k.dtype);
    weights fp32 [B,Hkv,L//g,g];
    mode: one of the CCA_POOL_* rules (q gives the shapes; the mean and max rules do not read it)."""
    B, Hq, L, d = _dims(q, 4, "q")
    Hkv = _dims(k, 4, "k")[1]
    m_cap = core_k.shape[2] if core_k is not None else 0
    dt = (k.dtype,)
    spec = [("q", q, (B, Hq, L, d), dt), ("k", k, (B, Hkv, L, d), _FLOAT), ("v", v, (B, Hkv, L, d), dt)]
    if core_k is not None or core_v is not None:
        ct = (core_dtype(k.dtype),)
        spec += [("core_k", core_k, (B, Hkv, m_cap, d), ct), ("core_v", core_v, (B, Hkv, m_cap, d), ct)]
    if weights is not None:
        spec.append(("weights", weights, (B, Hkv, L // g if g > 0 else 0, g), (torch.float32,)))
    _expect(spec)
    _check(load().cca_pool_core_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(core_k), _ptr(core_v), m_cap,
                                   _ptr(weights), B, Hq, Hkv, L, d, g, _dt(k), mode, _stream(stream)))


def cca_attn_prefill(q, k, v, core_k, core_v, out, g: int, w: int, kernel: int = 0,
                     stream=None) -> None:
    """out [B,Hq,L,d] in q's dtype or fp32; kernel: 0 auto, 1 vector-ALU, 2 matrix-core."""
    B, Hq, L, d = _dims(q, 4, "q")
    Hkv = _dims(k, 4, "k")[1]
    m_cap = core_k.shape[2] if core_k is not None else 0
    _expect(_attn_spec(q, k, v, core_k, core_v, out, B, Hq, Hkv, L, L, d, m_cap))
    _check(load().cca_attn_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(core_k), _ptr(core_v), m_cap,
                                      _ptr(out), _dt(out), B, Hq, Hkv, L, d, g, w, _dt(q), kernel,
                                      _stream(stream)))


def _attn_spec(q, k, v, core_k, core_v, out, B, Hq, Hkv, Lq, Lk, d, m_cap):
    dt = (q.dtype,)
    spec = [("q", q, (B, Hq, Lq, d), _FLOAT), ("k", k, (B, Hkv, Lk, d), dt), ("v", v, (B, Hkv, Lk, d), dt),
            ("out", out, (B, Hq, Lq, d), (q.dtype, torch.float32))]
    if core_k is not None or core_v is not None:
        ct = (core_dtype(q.dtype),)
        spec += [("core_k", core_k, (B, Hkv, m_cap, d), ct), ("core_v", core_v, (B, Hkv, m_cap, d), ct)]
    return spec


def cca_decode_workspace_bytes(B: int, Hq: int, Hkv: int, d: int, m_cap: int, g: int, w: int) -> int:
    return int(load().cca_decode_workspace_bytes(B, Hq, Hkv, d, m_cap, g, w))


def cca_attn_decode(q_t, k_t, v_t, ring_k, ring_v, core_k, core_v, pos, out, workspace, g: int,
                    w: int, advance_pos: bool = False, pool_mode: int = CCA_POOL_SOFTMAX,
                    stream=None) -> None:
    """q_t [B,Hq,d]; k_t, v_t [B,Hkv,d]; ring_* [B,Hkv,R,d]; core_* [B,Hkv,m_cap,d];
    pos int32 [B]; out [B,Hq,d]; workspace uint8 of cca_decode_workspace_bytes bytes;
    pool_mode: the CCA_POOL_* rule for the core appended when a group completes."""
    B, Hq, d = _dims(q_t, 3, "q_t")
    Hkv = _dims(k_t, 3, "k_t")[1]
    R = _dims(ring_k, 4, "ring_k")[2]
    m_cap = core_k.shape[2] if core_k is not None else 0
    dt = (q_t.dtype,)
    spec = [("q_t", q_t, (B, Hq, d), _FLOAT), ("k_t", k_t, (B, Hkv, d), dt), ("v_t", v_t, (B, Hkv, d), dt),
            ("ring_k", ring_k, (B, Hkv, R, d), dt), ("ring_v", ring_v, (B, Hkv, R, d), dt),
            ("pos", pos, (B,), (torch.int32,)), ("out", out, (B, Hq, d), (q_t.dtype, torch.float32))]
    if core_k is not None or core_v is not None:
        ct = (core_dtype(q_t.dtype),)
        spec += [("core_k", core_k, (B, Hkv, m_cap, d), ct), ("core_v", core_v, (B, Hkv, m_cap, d), ct)]
    _expect(spec + _workspace("workspace", workspace))
    _check(load().cca_attn_decode_ex(_ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(ring_k), _ptr(ring_v), R,
                                     _ptr(core_k), _ptr(core_v), m_cap, _ptr(pos), int(advance_pos),
                                     _ptr(out), _dt(out), _ptr(workspace),
                                     workspace.numel() * workspace.element_size(), B, Hq, Hkv, d, g,
                                     w, _dt(q_t), pool_mode, _stream(stream)))


def cca_decode_scratch_bytes() -> int:
    return int(load().cca_decode_scratch_bytes())


def cca_attn_decode_scratch(q_t, k_t, v_t, ring_k, ring_v, core_k, core_v, pos, out, g: int, w: int,
                            advance_pos: bool = False, pool_mode: int = CCA_POOL_SOFTMAX,
                            stream=None) -> None:
    """cca_attn_decode without a workspace: the split states live in the library's fixed device
    array (for callers that cannot allocate; calls that overlap on one GPU race)."""
    B, Hq, d = _dims(q_t, 3, "q_t")
    Hkv = _dims(k_t, 3, "k_t")[1]
    R = _dims(ring_k, 4, "ring_k")[2]
    m_cap = core_k.shape[2] if core_k is not None else 0
    dt = (q_t.dtype,)
    spec = [("q_t", q_t, (B, Hq, d), _FLOAT), ("k_t", k_t, (B, Hkv, d), dt), ("v_t", v_t, (B, Hkv, d), dt),
            ("ring_k", ring_k, (B, Hkv, R, d), dt), ("ring_v", ring_v, (B, Hkv, R, d), dt),
            ("pos", pos, (B,), (torch.int32,)), ("out", out, (B, Hq, d), (q_t.dtype, torch.float32))]
    if core_k is not None or core_v is not None:
        ct = (core_dtype(q_t.dtype),)
        spec += [("core_k", core_k, (B, Hkv, m_cap, d), ct), ("core_v", core_v, (B, Hkv, m_cap, d), ct)]
    _expect(spec)
    _check(load().cca_attn_decode_scratch(_ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(ring_k), _ptr(ring_v), R,
                                          _ptr(core_k), _ptr(core_v), m_cap, _ptr(pos), int(advance_pos),
                                          _ptr(out), _dt(out), B, Hq, Hkv, d, g, w, _dt(q_t), pool_mode,
                                          _stream(stream)))


def _rows(t):
    if t is None or t.dtype != torch.int32:
        raise CCAError(CCA_ERR_INVALID_ARG, "q_start / q_len / seq_len must be int32 device tensors")
    return _ptr(t)


def cca_pool_core_chunk(q, k, v, core_k, core_v, g: int, q_start, q_len,
                        mode: int = CCA_POOL_SOFTMAX, stream=None) -> None:
    """Pools the groups completed by each sequence's chunk.  q [B,Hq,Lq,d] holds the chunk rows
    (local row i = position q_start[b] + i); k, v [B,Hkv,Lk,d] hold positions 0..; q_start, q_len
    int32 [B] on the device; core_k, core_v [B,Hkv,m_cap,d]."""
    B, Hq, Lq, d = _dims(q, 4, "q")
    _, Hkv, Lk, _ = _dims(k, 4, "k")
    m_cap = core_k.shape[2] if core_k is not None else 0
    dt = (k.dtype,)
    spec = [("q", q, (B, Hq, Lq, d), dt), ("k", k, (B, Hkv, Lk, d), _FLOAT), ("v", v, (B, Hkv, Lk, d), dt),
            ("q_start", q_start, (B,), (torch.int32,)), ("q_len", q_len, (B,), (torch.int32,))]
    if core_k is not None or core_v is not None:
        ct = (core_dtype(k.dtype),)
        spec += [("core_k", core_k, (B, Hkv, m_cap, d), ct), ("core_v", core_v, (B, Hkv, m_cap, d), ct)]
    _expect(spec)
    _check(load().cca_pool_core_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(core_k), _ptr(core_v), m_cap,
                                      _rows(q_start), _rows(q_len), B, Hq, Hkv, Lq, Lk, d, g, _dt(k),
                                      mode, _stream(stream)))


def cca_attn_prefill_chunk(q, k, v, core_k, core_v, out, g: int, w: int, q_start, q_len,
                           stream=None) -> None:
    """Fused attention rows of each sequence's chunk (see cca_pool_core_chunk for the layout);
    out [B,Hq,Lq,d] in q's dtype or fp32."""
    B, Hq, Lq, d = _dims(q, 4, "q")
    _, Hkv, Lk, _ = _dims(k, 4, "k")
    m_cap = core_k.shape[2] if core_k is not None else 0
    _expect(_attn_spec(q, k, v, core_k, core_v, out, B, Hq, Hkv, Lq, Lk, d, m_cap) +
            [("q_start", q_start, (B,), (torch.int32,)), ("q_len", q_len, (B,), (torch.int32,))])
    _check(load().cca_attn_prefill_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(core_k), _ptr(core_v), m_cap,
                                         _ptr(out), _dt(out), _rows(q_start), _rows(q_len), B, Hq, Hkv,
                                         Lq, Lk, d, g, w, _dt(q), _stream(stream)))


def cca_cache_fill_ring(k, v, ring_k, ring_v, seq_len, stream=None) -> None:
    """Copies the last R positions below seq_len[b] of k, v [B,Hkv,Lk,d] into ring slot p % R
    of ring_k, ring_v [B,Hkv,R,d]."""
    B, Hkv, Lk, d = _dims(k, 4, "k")
    R = _dims(ring_k, 4, "ring_k")[2]
    dt = (k.dtype,)
    _expect([("k", k, (B, Hkv, Lk, d), _FLOAT), ("v", v, (B, Hkv, Lk, d), dt),
             ("ring_k", ring_k, (B, Hkv, R, d), dt), ("ring_v", ring_v, (B, Hkv, R, d), dt),
             ("seq_len", seq_len, (B,), (torch.int32,))])
    _check(load().cca_cache_fill_ring(_ptr(k), _ptr(v), _ptr(ring_k), _ptr(ring_v), R, _rows(seq_len),
                                      B, Hkv, Lk, d, _dt(k), _stream(stream)))


def cca_attn_prefill_train(q, k, v, core_k, core_v, out, lse, g: int, w: int, stream=None) -> None:
    """cca_attn_prefill that also writes lse fp32 [B,Hq,L], each row's log-sum-exp of its scores."""
    B, Hq, L, d = _dims(q, 4, "q")
    Hkv = _dims(k, 4, "k")[1]
    m_cap = core_k.shape[2] if core_k is not None else 0
    _expect(_attn_spec(q, k, v, core_k, core_v, out, B, Hq, Hkv, L, L, d, m_cap) +
            [("lse", lse, (B, Hq, L), (torch.float32,))])
    _check(load().cca_attn_prefill_train(_ptr(q), _ptr(k), _ptr(v), _ptr(core_k), _ptr(core_v), m_cap,
                                         _ptr(out), _dt(out), _ptr(lse), B, Hq, Hkv, L, d, g, w, _dt(q),
                                         _stream(stream)))


def cca_attn_backward_workspace_bytes(B: int, Hq: int, Hkv: int, L: int, d: int, g: int,
                                      dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace bytes of cca_attn_backward for inputs of ``dtype`` (bf16 also holds fp16
    copies of q and dout)."""
    dt = CCA_F32 if dtype == torch.float32 else CCA_BF16
    return int(load().cca_attn_backward_workspace_bytes(B, Hq, Hkv, L, d, g, dt))


def cca_attn_backward(q, k, v, core_k, core_v, out, lse, dout, dq, dk, dv, workspace, g: int, w: int,
                      pool_mode: int = CCA_POOL_SOFTMAX, stream=None) -> None:
    """Gradients dq [B,Hq,L,d], dk, dv [B,Hkv,L,d] (fp32, overwritten) of the forward (pooling with
    rule pool_mode, then the fused prefill) for the upstream gradient dout of out."""
    B, Hq, L, d = _dims(q, 4, "q")
    Hkv = _dims(k, 4, "k")[1]
    m_cap = core_k.shape[2] if core_k is not None else 0
    f32 = (torch.float32,)
    spec = _attn_spec(q, k, v, core_k, core_v, out, B, Hq, Hkv, L, L, d, m_cap)
    spec[3] = ("out", out, (B, Hq, L, d), (q.dtype,))
    _expect(spec + [("lse", lse, (B, Hq, L), f32), ("dout", dout, (B, Hq, L, d), (q.dtype,)),
                    ("dq", dq, (B, Hq, L, d), f32), ("dk", dk, (B, Hkv, L, d), f32),
                    ("dv", dv, (B, Hkv, L, d), f32)] + _workspace("workspace", workspace))
    _check(load().cca_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(core_k), _ptr(core_v), m_cap, _ptr(out),
                                    _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), B, Hq, Hkv, L, d, g, w,
                                    _dt(q), pool_mode, _stream(stream)))
