"""Build libqmm.so (all HIP kernels + the C ABI) and libqmm_probe.so (the
measurement probes) for gfx950 with hipcc.

Flags: -O3; -ffp-contract=off so no multiply and add are fused unless the
source asks for fmaf (the quantizers are bit-exact only without contraction);
f32 denormals kept; packed-FP32 instructions disabled.  Each source compiles
to an object in its own hipcc process (in parallel), then one hipcc links the
shared library.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libqmm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


PROBE_LIB = os.path.join(HERE, "libqmm_probe.so")
PROBE_SOURCES = ("peaks.hip",)      # the measurement probes: a library of their own


def sources():
    """The product library's sources."""
    return sorted(f for f in glob.glob(os.path.join(HERE, "csrc", "*.hip"))
                  if os.path.basename(f) not in PROBE_SOURCES)


def probe_sources():
    return [os.path.join(HERE, "csrc", f) for f in PROBE_SOURCES]


def _filtered(text: str) -> str:
    # hipcc's host pass does not know the packed-FP32 target feature; harmless
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libqmm.so and libqmm_probe.so (always
    recompiles)."""
    _build(sources(), LIB, verbose)
    _build(probe_sources(), PROBE_LIB, verbose)
    return LIB


def _build(srcs, lib_path: str, verbose: bool) -> None:
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    tmpdir = tempfile.mkdtemp(prefix="qmm_build_", dir=HERE)
    try:
        jobs = []
        for src in srcs:
            obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
            cmd = [HIPCC] + FLAGS + inc + ["-c", "-o", obj, src]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                                    text=True)))
        failed = False
        for src, _, proc in jobs:
            out = _filtered(proc.communicate()[0])
            if proc.returncode != 0:
                failed = True
                sys.stderr.write(f"{src}:\n{out}\n")
            elif verbose and out.strip():
                print(out)
        if failed:
            raise RuntimeError("hipcc failed building " + os.path.basename(lib_path))
        tmp = lib_path + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [obj for _, obj, _ in jobs]
        proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if proc.returncode != 0:
            sys.stderr.write(_filtered(proc.stdout) + "\n")
            raise RuntimeError("hipcc failed linking " + os.path.basename(lib_path))
        os.replace(tmp, lib_path)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose=True))
