"""The matrix-core prefill gives most items (a workgroup's worth of rows each)
one to a workgroup by block id and the shortest quarter, when there are at
least 8 per compute unit, to one workgroup per compute unit that takes them
from per-XCD work queues in device memory: one queue slot per launch, which
the launch's last queue workgroup clears.  These cases check what the queues
add: slots reused across more launches than there are slots, launches on two
streams at once, and launches replayed from a HIP graph all give the same
outputs, bit for bit, as one eager launch (every row's arithmetic is the same
whichever workgroup computes it), and every row is written.

The backward's kernels hand out their last items the same way (the dQ kernel
its shortest position blocks, the key-parallel kernel its last raw-key
units); the gradients also take the cores' contributions through fp32 atomic
adds, whose order varies, so there the repeated calls must agree to a few
ulps and leave no gradient row unwritten.
"""
from __future__ import annotations

import pytest
import torch

import cca_inputs
import sparse_long_context_cca_amd as cca

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MFMA = 2  # kernel selector of cca_attn_prefill: the matrix-core path


def say(msg: str) -> None:
    print(msg, flush=True)


def case(name, B, Hq, Hkv, L, d, g, w, seed):
    """Inputs on the GPU, cores pooled, and an output buffer filled with NaN."""
    cfg = cca_inputs.make_config(seed, name, B, Hq, Hkv, L, d, g, w, "bf16")
    q, k, v = (x.to(DEV) for x in cca_inputs.prefill_inputs(cfg))
    m = max(L // g, 1)
    ck = torch.zeros((B, Hkv, m, d), dtype=cca.core_dtype(q.dtype), device=DEV)
    cv = torch.zeros_like(ck)
    cca.cca_pool_core(q, k, v, ck, cv, g)
    out = torch.full_like(q, float("nan"))
    return dict(q=q, k=k, v=v, ck=ck, cv=cv, out=out, g=g, w=w)


def run(c, stream=None):
    cca.cca_attn_prefill(c["q"], c["k"], c["v"], c["ck"], c["cv"], c["out"], c["g"], c["w"], kernel=MFMA,
                         stream=stream)


def eager(c):
    c["out"].fill_(float("nan"))
    run(c)
    torch.cuda.synchronize()
    ref = c["out"].clone()
    assert torch.isfinite(ref.float()).all(), "every row written"
    return ref


# GQA, 4 heads per kv head: 64-row items, 1024 position blocks x 2 kv heads =
# 2048 items (512 through the queues); MHA: 256-row items, 4 x 16 x 40 = 2560
# items (640 through the queues); a small case with no queue at all.
BIG = ("gqa", 1, 8, 2, 65536, 128, 16, 256)
MHA = ("mha", 4, 16, 16, 10240, 64, 16, 512)
SMALL = ("small", 1, 4, 4, 512, 64, 8, 64)


def test_queue_slots_reused_across_launches():
    """More launches than queue slots, alternating shapes with and without a
    queue: each output stays identical."""
    say("prefill queues: 150 launches over the queue slots")
    big = case(*BIG, seed=71)
    small = case(*SMALL, seed=72)
    ref_big, ref_small = eager(big), eager(small)
    for i in range(75):
        run(big)
        run(small)
        if i % 25 == 24:
            torch.cuda.synchronize()
            assert torch.equal(big["out"], ref_big), f"launch pair {i}"
            assert torch.equal(small["out"], ref_small), f"launch pair {i}"


def test_two_streams_at_once():
    """Two launches in flight on two streams (different queue slots)."""
    say("prefill queues: two streams")
    a = case(*BIG, seed=73)
    b = case(*MHA, seed=74)
    ref_a, ref_b = eager(a), eager(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for rep in range(4):
        a["out"].fill_(float("nan"))
        b["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            run(a, stream=s1)
        with torch.cuda.stream(s2):
            run(b, stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(a["out"], ref_a), f"stream 1, round {rep}"
        assert torch.equal(b["out"], ref_b), f"stream 2, round {rep}"


def test_graph_replay_matches_eager():
    """A prefill captured in a HIP graph: every replay, with eager launches and
    synchronisation in between, reproduces the eager output bit for bit."""
    say("prefill queues: graph replay")
    c = case(*MHA, seed=75)
    other = case(*BIG, seed=76)
    ref, ref_other = eager(c), eager(other)
    graph = torch.cuda.CUDAGraph()
    c["out"].fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run(c, stream=torch.cuda.current_stream())
    for rep in range(3):
        c["out"].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(c["out"], ref), f"replay {rep}"
        run(other)
        torch.cuda.synchronize()
        assert torch.equal(other["out"], ref_other), f"eager launch after replay {rep}"


# ------------------------------------------------------------------ backward
# The key-parallel kernel: 8 kv heads x (32 core blocks x 8 row splits + 512
# raw blocks) = 6144 units, 1536 of them through the queues; the row-parallel
# dQ kernel: 256 position blocks x 8 heads = 2048 items, 512 through its
# queues.  A small shape with no queue.
BW_BIG = ("bw", 1, 8, 8, 65536, 128, 16, 1024)
BW_SMALL = ("bw_small", 1, 4, 2, 700, 64, 8, 64)


def bw_case(name, B, Hq, Hkv, L, d, g, w, seed):
    c = case(name, B, Hq, Hkv, L, d, g, w, seed)
    c["lse"] = torch.empty((B, Hq, L), dtype=torch.float32, device=DEV)
    cca.cca_attn_prefill_train(c["q"], c["k"], c["v"], c["ck"], c["cv"], c["out"], c["lse"], g, w)
    gen = torch.Generator(device=DEV).manual_seed(seed)
    c["dout"] = torch.randn(c["q"].shape, generator=gen, device=DEV).to(c["q"].dtype)
    c["ws"] = torch.empty(cca.cca_attn_backward_workspace_bytes(B, Hq, Hkv, L, d, g, c["q"].dtype),
                          dtype=torch.uint8, device=DEV)
    c["grads"] = [torch.empty((B, Hq, L, d), device=DEV), torch.empty((B, Hkv, L, d), device=DEV),
                  torch.empty((B, Hkv, L, d), device=DEV)]
    return c


def bw_run(c, stream=None):
    for t in c["grads"]:
        t.fill_(float("nan"))
    dq, dk, dv = c["grads"]
    cca.cca_attn_backward(c["q"], c["k"], c["v"], c["ck"], c["cv"], c["out"], c["lse"], c["dout"],
                          dq, dk, dv, c["ws"], c["g"], c["w"], stream=stream)


def bw_check(c, ref, what):
    for name, got, r in zip(("dq", "dk", "dv"), c["grads"], ref):
        assert torch.isfinite(got).all(), f"{what}: {name} has unwritten rows"
        tol = 1e-5 * max(1.0, float(r.abs().max()))
        assert float((got - r).abs().max()) <= tol, f"{what}: {name} differs"


def bw_eager(c):
    bw_run(c)
    torch.cuda.synchronize()
    ref = [t.clone() for t in c["grads"]]
    bw_check(c, ref, "eager")
    return ref


def test_backward_queue_slots_reused_across_calls():
    """More backward calls than queue slots, alternating shapes with and
    without a queue: every call writes every gradient row and agrees with the
    first."""
    say("backward queues: 140 calls over the queue slots")
    big = bw_case(*BW_BIG, seed=81)
    small = bw_case(*BW_SMALL, seed=82)
    ref_big, ref_small = bw_eager(big), bw_eager(small)
    for i in range(70):
        bw_run(big)
        if i % 10 == 9:
            torch.cuda.synchronize()
            bw_check(big, ref_big, f"call {i}")
        bw_run(small)
        if i % 10 == 9:
            torch.cuda.synchronize()
            bw_check(small, ref_small, f"call {i}")


def test_backward_two_streams_at_once():
    """Two backward calls in flight on two streams (different queue slots)."""
    say("backward queues: two streams")
    a = bw_case(*BW_BIG, seed=83)
    b = bw_case(*BW_BIG, seed=84)
    ref_a, ref_b = bw_eager(a), bw_eager(b)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(5):
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            bw_run(a, stream=s1)
        with torch.cuda.stream(s2):
            bw_run(b, stream=s2)
        torch.cuda.synchronize()
        bw_check(a, ref_a, f"stream 1, round {rep}")
        bw_check(b, ref_b, f"stream 2, round {rep}")


def test_backward_graph_replay_matches_eager():
    """A backward call captured in a HIP graph (it clears its core partial sums
    with a fill kernel, so the clear replays too): every replay, with eager
    calls and synchronisation in between, writes every gradient row and agrees
    with the eager call."""
    say("backward queues: graph replay")
    c = bw_case(*BW_BIG, seed=85)
    other = bw_case(*BW_SMALL, seed=86)
    ref, ref_other = bw_eager(c), bw_eager(other)
    dq, dk, dv = c["grads"]
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        cca.cca_attn_backward(c["q"], c["k"], c["v"], c["ck"], c["cv"], c["out"], c["lse"], c["dout"],
                              dq, dk, dv, c["ws"], c["g"], c["w"], stream=torch.cuda.current_stream())
    for rep in range(3):
        for t in c["grads"]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bw_check(c, ref, f"replay {rep}")
        bw_run(other)
        torch.cuda.synchronize()
        bw_check(other, ref_other, f"eager call after replay {rep}")
