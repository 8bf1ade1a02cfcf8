"""The matrix-core probe (libcca_probe.so, include/cca_probe.h) that bench.py
times beside the kernels: its export and argument checks on the CPU, one small
launch on the GPU."""
from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch  # before the probe library: it must bind to the HIP runtime torch loads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cca_probe.h")
LIB = os.path.join(ROOT, "sparse_long_context_cca_amd", "libcca_probe.so")


@pytest.fixture(scope="module")
def probe():
    if not os.path.exists(LIB):
        from sparse_long_context_cca_amd import build
        build.build(verbose=False)
    lib = ctypes.CDLL(LIB)
    lib.cca_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                   ctypes.c_void_p]
    return lib


def test_probe_exports_what_its_header_declares(probe):
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(cca_[a-z_0-9]+)\s*\(", text)))
    assert names == ["cca_probe_mfma"]
    for n in names:
        assert hasattr(probe, n)


@pytest.mark.parametrize("args", [(None, 4, 1, 4), (0x10000, 0, 1, 4), (0x10000, 4, 0, 4), (0x10000, 4, 1, 0),
                                  (0x10000, 4, 1, 5)])
def test_probe_rejects_bad_arguments_before_launching(probe, args):
    out, blocks, iters, sets = args
    assert probe.cca_probe_mfma(out, blocks, iters, sets, 1, None) == 1


@pytest.mark.gpu
def test_probe_runs_and_writes_finite_sums(probe):
    out = torch.full((4 * 512,), float("nan"), device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for sets in (1, 4):
        rc = probe.cca_probe_mfma(out.data_ptr(), 4, 3, sets, 7, stream)
        assert rc == 0, f"launch failed: hipError {rc - 1000}"
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out).all())
