"""Build the qmat shared library (libqmat.so) and the read-stream probe used by the benchmark
(libqmat_probe.so) for gfx950 with hipcc, in place."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqmat.so")
SOURCES = [os.path.join(CSRC, "qmat_host.cpp"), os.path.join(CSRC, "qmat_pack.cpp"),
           os.path.join(CSRC, "qmat_api.cpp"), os.path.join(CSRC, "qmat_encode.cpp"),
           os.path.join(CSRC, "qmat_kernels.hip"), os.path.join(CSRC, "qmat_gemm.hip"),
           os.path.join(CSRC, "qmat_logits.hip")]
PROBE_LIB = os.path.join(HERE, "libqmat_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "qmat_probe.hip")]

# -packed-fp32-ops: keep the compiler from emitting packed fp32 (v_pk_*_f32) instructions.
HIPCC_FLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compile both libraries (two hipcc processes side by side); returns libqmat.so's path."""
    jobs = []
    for lib, sources in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        cmd = [hipcc(), *HIPCC_FLAGS, "-o", lib + ".tmp", *sources]
        jobs.append((lib, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
    errors = []
    for lib, cmd, proc in jobs:
        out, err = proc.communicate()
        if proc.returncode != 0:
            errors.append(f"hipcc failed for {os.path.basename(lib)}:\n{out}{err}")
        elif verbose:
            print(" ".join(cmd))
    if errors:
        raise RuntimeError("\n".join(errors))
    for lib, _, _ in jobs:
        os.replace(lib + ".tmp", lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
