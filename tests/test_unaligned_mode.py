"""The 32-value prefill kernels copy 16-byte chunks of 34-, 22- and 18-byte
blocks with buffer loads into LDS.  When a row holds an even number of
blocks every chunk address is a multiple of 4; with an odd count every other
row starts 2 bytes past one, and those loads depend on the unaligned access
mode of the memory pipeline.

That mode is part of the HSA target the library is built for, not a property
of one machine: hipcc's gfx950 (amdhsa) target turns the
`unaligned-access-mode` feature on by default and then itself compiles an
under-aligned 16-byte load into one `global_load_dwordx4`; with the feature
off it falls back to byte loads.  This CPU test checks both on the toolchain
in use, so the kernels' assumption is the compiler's own.  The GPU parity
tests run rows of 3, 5, 65 and 129 blocks through the same kernels."""
from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

HIPCC = shutil.which("hipcc") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else None)

SRC = r"""
#include <hip/hip_runtime.h>
#include <cstdint>
struct __attribute__((packed, aligned(1))) Chunk { uint32_t a, b, c, d; };
__global__ void k(const unsigned char* p, uint4* o, int off) {
  const Chunk* q = reinterpret_cast<const Chunk*>(p + off + threadIdx.x * 18);
  Chunk v = *q;
  o[threadIdx.x] = make_uint4(v.a, v.b, v.c, v.d);
}
"""


def _loads(tmp_path, extra):
    src = tmp_path / "chunk.hip"
    src.write_text(SRC)
    asm = tmp_path / f"chunk{len(extra)}.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "--cuda-device-only", "-S", "-o", str(asm), str(src),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"] + extra
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return re.findall(r"^\s*(global_load_\w+)", asm.read_text(), re.M)


@pytest.mark.skipif(HIPCC is None, reason="hipcc not found")
def test_gfx950_hsa_target_assumes_unaligned_access(tmp_path):
    loads = _loads(tmp_path, [])
    assert loads == ["global_load_dwordx4"], loads
    off = _loads(tmp_path, ["-Xclang", "-target-feature", "-Xclang", "-unaligned-access-mode"])
    assert "global_load_dwordx4" not in off and len(off) >= 4, off
