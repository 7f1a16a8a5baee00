"""Host sanitizers over the CPU code: the library's HIP-free host sources (packer, encoders,
error text) built with clang++ and the C oracle built with gcc, each under AddressSanitizer +
UndefinedBehaviorSanitizer (any report aborts the run) and under ThreadSanitizer, driven by
tests/sanitize/*_driver.*.  A canary run that writes one element past a buffer must be
reported, which shows the instrumentation reaches the code under test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "weight_only_quant_amd", "csrc")
HOST_SOURCES = [os.path.join(HERE, "sanitize", "host_driver.cpp")] + [
    os.path.join(CSRC, f) for f in ("qmat_host.cpp", "qmat_pack.cpp", "qmat_encode.cpp")]
ORACLE_SOURCES = [os.path.join(HERE, "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "qmat_oracle.c")]
ASAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
TSAN = ["-fsanitize=thread"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
           TSAN_OPTIONS="halt_on_error=1")


def _clangxx():
    # the encoders use _Float16, which this image's g++ lacks; ROCm's clang has it and ships
    # the x86-64 sanitizer runtimes
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no clang++ for the host sanitizer build")


def _build(tmp_path, name, cmd):
    exe = str(tmp_path / name)
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return exe


def _run(exe, *args):
    return subprocess.run([exe, *args], capture_output=True, text=True, timeout=300, env=ENV)


def _host_cmd(flags):
    return [_clangxx(), "-std=c++17", "-O1", "-g", *flags, *HOST_SOURCES, "-lpthread"]


def _oracle_cmd(flags):
    return ["gcc", "-std=c11", "-O1", "-g", "-fno-fast-math", "-ffp-contract=off", *flags, *ORACLE_SOURCES,
            "-lm", "-lpthread"]


@pytest.mark.parametrize("kind", ["asan_ubsan", "tsan"])
def test_host_sources_sanitized(tmp_path, kind):
    exe = _build(tmp_path, "host_" + kind, _host_cmd(ASAN if kind == "asan_ubsan" else TSAN))
    r = _run(exe)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr, r.stderr
    if kind == "asan_ubsan":
        c = _run(exe, "--canary")
        assert c.returncode != 0 and "heap-buffer-overflow" in c.stderr and "pack_tile" in c.stderr, c.stdout + c.stderr


@pytest.mark.parametrize("kind", ["asan_ubsan", "tsan"])
def test_oracle_sanitized(tmp_path, kind):
    exe = _build(tmp_path, "oracle_" + kind, _oracle_cmd(ASAN if kind == "asan_ubsan" else TSAN))
    r = _run(exe)
    assert r.returncode == 0 and "all checks passed" in r.stdout, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr, r.stderr
    if kind == "asan_ubsan":
        c = _run(exe, "--canary")
        assert c.returncode != 0 and "heap-buffer-overflow" in c.stderr and "qo_dequant_groupwise" in c.stderr, \
            c.stdout + c.stderr
