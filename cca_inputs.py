"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and rounds them to the storage dtype; it holds
none of the attention method's arithmetic.  Both the CPU oracle (``oracle/``)
and the GPU library's tests and benchmark take their inputs from here, so that
the two sides always see the same bits.

Recipe (all configs):
  * Normals come from numpy's PCG64 generator.  A tensor with seed ``s`` is cut
    into fixed chunks of ``CHUNK`` elements of its flattened (row-major) form;
    chunk ``i`` is drawn from ``PCG64(SeedSequence(s, spawn_key=(i,)))``.  The
    result therefore does not depend on how many threads draw it.
  * bf16 tensors are the float32 draws rounded to nearest-even by torch on the
    CPU; fp32 tensors keep the float32 draws.
  * Seeds: Q = 1000 + c, K = 2000 + c, V = 3000 + c, spike mask = 4000 + c for
    config number c (1..5).

The five workloads stand in for the pages' long-context evaluation (LongBench-E
at up to 32K tokens, multi-document QA at 64K/128K); they take the context
lengths of those evaluations and the LLaMA-2-7B / LLaMA-3.1-8B attention head
shapes, with i.i.d. normal projections in place of real activations.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def normal_f32(seed: int, shape, scale: float = 1.0) -> np.ndarray:
    """Standard normals (times ``scale``) as float32, chunked as described above."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def draw(i: int) -> None:
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(i,))))
        rng.standard_normal(out=out[lo:hi], dtype=np.float32)

    if nchunks <= 1:
        for i in range(nchunks):
            draw(i)
    else:
        with ThreadPoolExecutor(min(_threads(), nchunks)) as ex:
            list(ex.map(draw, range(nchunks)))
    if scale != 1.0:
        out *= np.float32(scale)
    return out.reshape(shape)


def to_storage(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> CPU torch tensor in the storage dtype ('f32' or 'bf16', RNE)."""
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t.clone() if not t.is_contiguous() else t
    raise ValueError(f"unknown dtype {dtype!r}")


def seeded(seed: int, shape, dtype: str, scale: float = 1.0) -> torch.Tensor:
    return to_storage(normal_f32(seed, shape, scale), dtype)


def spike_mask(seed: int, shape, p: float = 0.01) -> np.ndarray:
    """Independent Bernoulli(p) flags, one per (batch, kv head, token)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return rng.random(size=shape) < p


@dataclass(frozen=True)
class Config:
    """One workload: attention head shapes, grouping g, window w, storage dtype."""
    number: int
    name: str
    B: int
    Hq: int
    Hkv: int
    L: int            # prefill tokens; for decode, tokens already cached before the first step
    d: int
    g: int
    w: int
    dtype: str        # 'f32' or 'bf16'
    scale: float = 1.0   # normals are multiplied by this before rounding
    spiky: bool = False  # 1% of keys (per token, per kv head) scaled by 4
    decode_steps: int = 0
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def m(self) -> int:
        return self.L // self.g

    def seeds(self):
        c = self.number
        return 1000 + c, 2000 + c, 3000 + c, 4000 + c


CONFIGS = {
    1: Config(1, "tiny_f32_L1024_d64", 1, 1, 1, 1024, 64, 16, 64, "f32", scale=1.0 / math.sqrt(64)),
    2: Config(2, "llama2_7b_mha_L32768", 1, 32, 32, 32768, 128, 16, 1024, "bf16"),
    3: Config(3, "llama2_7b_mha_L131072_spiky", 1, 32, 32, 131072, 128, 16, 1024, "bf16", spiky=True),
    4: Config(4, "llama3_1_8b_gqa_L131072", 1, 32, 8, 131072, 128, 16, 1024, "bf16"),
    5: Config(5, "decode_b8_gqa_ctx65536", 8, 32, 8, 65536, 128, 16, 1024, "bf16", decode_steps=256),
}


def make_config(number: int, name: str, B: int, Hq: int, Hkv: int, L: int, d: int, g: int, w: int,
                dtype: str, scale: float = 1.0, spiky: bool = False, decode_steps: int = 0) -> Config:
    """An ad-hoc workload (tests use these for small and ragged shapes)."""
    return Config(number, name, B, Hq, Hkv, L, d, g, w, dtype, scale, spiky, decode_steps)


def prefill_inputs(cfg: Config):
    """Q [B,Hq,L,d], K, V [B,Hkv,L,d] as CPU torch tensors in the storage dtype."""
    sq, sk, sv, sm = cfg.seeds()
    q = normal_f32(sq, (cfg.B, cfg.Hq, cfg.L, cfg.d), cfg.scale)
    k = normal_f32(sk, (cfg.B, cfg.Hkv, cfg.L, cfg.d), cfg.scale)
    v = normal_f32(sv, (cfg.B, cfg.Hkv, cfg.L, cfg.d), cfg.scale)
    if cfg.spiky:
        mask = spike_mask(sm, (cfg.B, cfg.Hkv, cfg.L))
        k[mask] *= np.float32(4.0)
    return to_storage(q, cfg.dtype), to_storage(k, cfg.dtype), to_storage(v, cfg.dtype)


def decode_inputs(cfg: Config):
    """Inputs of a decode run: a cached history of ``cfg.L`` tokens, then steps.

    Returns a dict of CPU torch tensors in the storage dtype:
      q_ends  [B,Hq,L//g,d]  query rows at the last token of each history group
                             (the only history query rows the decode path reads)
      k, v    [B,Hkv,L+S,d]  keys/values of the history followed by the S steps
      q_steps [B,Hq,S,d]     the query of each decode step
    Query rows of the history that are not group ends are never drawn; a full
    history query buffer holds zeros there.
    """
    sq, sk, sv, sm = cfg.seeds()
    S = cfg.decode_steps
    n_ends = cfg.L // cfg.g
    qall = normal_f32(sq, (cfg.B, cfg.Hq, n_ends + S, cfg.d), cfg.scale)
    k = normal_f32(sk, (cfg.B, cfg.Hkv, cfg.L + S, cfg.d), cfg.scale)
    v = normal_f32(sv, (cfg.B, cfg.Hkv, cfg.L + S, cfg.d), cfg.scale)
    if cfg.spiky:
        mask = spike_mask(sm, (cfg.B, cfg.Hkv, cfg.L + S))
        k[mask] *= np.float32(4.0)
    return {
        "q_ends": to_storage(np.ascontiguousarray(qall[:, :, :n_ends]), cfg.dtype),
        "q_steps": to_storage(np.ascontiguousarray(qall[:, :, n_ends:]), cfg.dtype),
        "k": to_storage(k, cfg.dtype),
        "v": to_storage(v, cfg.dtype),
    }


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a storage tensor to a float64 numpy array."""
    return t.to(torch.float64).numpy()
