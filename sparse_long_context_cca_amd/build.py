"""Builds libcca.so (HIP, gfx950 only) in-tree with hipcc.

Usage: python -m sparse_long_context_cca_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcca.so")

SOURCES = ["cca_api.hip", "cca_pool.hip", "cca_prefill_valu.hip", "cca_prefill_mfma.hip",
           "cca_decode.hip", "cca_backward.hip", "cca_backward_mfma.hip"]

# the matrix-core probe that bench.py times beside the kernels (a library of its own)
PROBE_SOURCES = ["cca_probe.hip"]
PROBE_LIB = os.path.join(PKG, "libcca_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# ---- compiler flags (the lines up to the end marker are what a counter
# summary's digest covers of this script; see bench.py's code_digest)
ARCH = "gfx950"
# Packed fp32 VALU ops are disabled: only scalar fp32 arithmetic is emitted.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"),
          "-Wall", "-Wno-unused-function"]
# Per-source flags.  The prefill kernel's main loop is scheduled with the
# backend's iterative ILP strategy: measured in one process on one MI355X it
# is about 2 % faster on the GQA 128K prefill and 3 % on the MHA 32K one (the
# same strategy slows the backward kernels, which keep the default).
SOURCE_FLAGS = {
    "cca_prefill_mfma.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}
# ---- end of compiler flags


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


# Host-side checking build: the argument validation of the C ABI (cca_api.hip)
# compiled with AddressSanitizer and UndefinedBehaviorSanitizer on its host
# code only (each -fsanitize follows -Xarch_host; device code is built as
# usual) and linked with the regular kernel objects into a separate library.
# The CPU tests load it with the sanitizer runtime preloaded.
SAN_LIB = os.path.join(OBJ, "libcca_asan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_RUNTIME = os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang")


def sanitizer_runtime() -> str:
    """Path of clang's shared ASan runtime (to preload into an uninstrumented Python)."""
    for root, _, files in os.walk(SAN_RUNTIME):
        if "libclang_rt.asan-x86_64.so" in files:
            return os.path.join(root, "libclang_rt.asan-x86_64.so")
    raise RuntimeError(f"libclang_rt.asan-x86_64.so not found under {SAN_RUNTIME}")


def build_sanitized(objs=None) -> str:
    """Builds _build/libcca_asan.so: cca_api.hip with host sanitizers, the
    other sources as in build().  Returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    san_obj = os.path.join(OBJ, "cca_api_asan.o")
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *SAN_FLAGS, "-c", os.path.join(CSRC, "cca_api.hip"), "-o", san_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for the sanitized cca_api.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if objs is None:
        objs = [_compile(s) for s in SOURCES if s != "cca_api.hip"]
    objs = [o for o in objs if not o.endswith("cca_api.o")]
    tmp = SAN_LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan", *SAN_FLAGS, san_obj, *objs,
           "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, SAN_LIB)
    return SAN_LIB


def build(verbose: bool = True) -> str:
    """Compiles every source for gfx950 and links libcca.so, the matrix-core
    probe libcca_probe.so and the host-sanitized libcca_asan.so for the CPU
    tests; returns libcca.so's path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(OBJ, exist_ok=True)
    srcs = [s for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    with ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, LIB)
    probe_objs = [_compile(s) for s in PROBE_SOURCES]
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *probe_objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, PROBE_LIB)
    build_sanitized(objs)
    if verbose:
        print(f"built {LIB} from {len(objs)} sources (and {SAN_LIB})", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
