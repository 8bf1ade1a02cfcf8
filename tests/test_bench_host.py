"""Host-side behaviour of bench.py that needs no GPU: the one-GPU refusal and
the digest gate on figures read from committed counter summaries."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, env=env, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_a_distributed_launch_is_refused():
    r = _run_bench([], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def _summary(tmp_path, src_text, digest_of):
    """A source file and a counter summary whose digest covers `digest_of`."""
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_text(src_text)
    (tmp_path / "ref.hip").write_text(digest_of)
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        digest = bench.code_digest(["ref.hip"])
    finally:
        bench.ROOT = old
    (tmp_path / "profiles" / "counters_x.txt").write_text(
        "# header line: ignored\n"
        "mfma_busy_fraction: 0.5\n"
        "sources: k.hip\n"
        f"kernel_sha256: {digest}\n")
    (tmp_path / "profiles" / "traffic_x.txt").write_text(
        "traffic_bytes: 1234\nsources: k.hip\n" f"kernel_sha256: {digest}\n")


def _with_root(tmp_path, fn):
    old = bench.ROOT
    bench.ROOT = str(tmp_path)
    try:
        return fn()
    finally:
        bench.ROOT = old


def test_figures_are_reported_while_the_kernel_is_unchanged(tmp_path):
    code = "__global__ void k(float* x) {\n  x[0] = 1.f;\n}\n"
    _summary(tmp_path, code, code)
    assert _with_root(tmp_path, lambda: bench.measured_mfma_busy("x")) == 0.5
    assert _with_root(tmp_path, lambda: bench.measured_traffic("x")) == 1234


def test_comment_and_blank_line_edits_keep_the_figures(tmp_path):
    code = "__global__ void k(float* x) {\n  x[0] = 1.f;\n}\n"
    edited = "// a new comment\n\n__global__ void k(float* x) {\n  // and another\n  x[0] = 1.f;\n}\n"
    _summary(tmp_path, edited, code)
    assert _with_root(tmp_path, lambda: bench.measured_mfma_busy("x")) == 0.5


def test_a_changed_kernel_drops_the_figures(tmp_path):
    code = "__global__ void k(float* x) {\n  x[0] = 1.f;\n}\n"
    changed = "__global__ void k(float* x) {\n  x[0] = 2.f;\n}\n"
    _summary(tmp_path, changed, code)
    assert _with_root(tmp_path, lambda: bench.measured_mfma_busy("x")) is None
    assert _with_root(tmp_path, lambda: bench.measured_traffic("x")) is None


def test_a_missing_summary_gives_no_figure(tmp_path):
    (tmp_path / "profiles").mkdir()
    assert _with_root(tmp_path, lambda: bench.measured_traffic("absent")) is None


def _build_script(flags_line, other_line):
    return ("import os\n" + other_line + "\n# ---- compiler flags (covered)\nARCH = 'gfx950'\n" + flags_line +
            "\n# ---- end of compiler flags\n\ndef build():\n    pass\n")


def test_build_script_digest_covers_its_flag_block_only(tmp_path):
    """Of a build script only the compiler-flag block enters the digest: a
    change elsewhere in it (a new library to link, say) keeps the counter
    figures, a changed flag drops them."""
    def digest(text):
        (tmp_path / "build.py").write_text(text)
        return _with_root(tmp_path, lambda: bench.code_digest(["build.py"]))
    base = digest(_build_script("COMMON = ['-O3']", "X = 1"))
    assert digest(_build_script("COMMON = ['-O3']", "X = 2  # another library")) == base
    assert digest(_build_script("COMMON = ['-O2']", "X = 1")) != base

