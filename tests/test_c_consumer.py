"""The boundary as a C caller sees it: include/qmm.h compiles as strict C99
and as C++17, a plain C program links libqmm.so by name and gets the
documented status codes back for arguments the library must refuse (those
checks come before any device call, so this runs without a GPU)."""
import os
import shutil
import subprocess

import pytest

from conftest import ROOT

INC = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "matmul_quantize_q8_amd")

C_PROGRAM = r"""
#include <stdint.h>
#include <stdio.h>
#include "qmm.h"

/* a 16-byte aligned address that is never dereferenced */
#define A ((void *)(uintptr_t)(1u << 20))
#define AT(off) ((void *)((uintptr_t)(1u << 20) + (off)))

static int fails = 0;
static void expect(const char *what, qmm_status got, qmm_status want) {
    if (got != want) {
        printf("FAIL %s: %d (%s), want %d\n", what, (int)got, qmm_status_string(got), (int)want);
        ++fails;
    }
}

int main(void) {
    int s;
    if (qmm_abi_version() != 1) { printf("FAIL version\n"); ++fails; }
    for (s = QMM_OK; s <= QMM_E_LAUNCH; ++s)
        if (qmm_status_string((qmm_status)s) == NULL) { printf("FAIL string %d\n", s); ++fails; }
    expect("K % 32", qmm_quantize_q8_0((const float *)A, A, 1, 48, NULL), QMM_E_SHAPE);
    expect("K % 256", qmm_quantize_q8_k((const float *)A, A, 1, 96, NULL), QMM_E_SHAPE);
    expect("NULL x", qmm_quantize_q8_0(NULL, A, 1, 32, NULL), QMM_E_NULL);
    expect("misaligned x", qmm_quantize_q8_0((const float *)AT(4), A, 1, 32, NULL), QMM_E_ALIGN);
    expect("NULL y", qmm_matvec_q4_0(A, A, NULL, 8, 64, NULL), QMM_E_NULL);
    expect("misaligned xq", qmm_matvec_q4_0(A, AT(8), (float *)A, 8, 64, NULL), QMM_E_ALIGN);
    expect("q2_k K", qmm_matvec_q2_k(A, A, (float *)A, 8, 128, NULL), QMM_E_SHAPE);
    expect("matmul K", qmm_matmul_q4_0(A, A, (float *)A, 4, 8, 33, NULL), QMM_E_SHAPE);
    expect("matmul M", qmm_matmul_q4_0(A, A, (float *)A, (int64_t)1 << 31, 8, 32, NULL), QMM_E_SHAPE);
    expect("fused K", qmm_quantize_matvec_q4_0(A, (const float *)A, A, (float *)A, 8, 48, NULL), QMM_E_SHAPE);
    expect("fused K-quant K", qmm_quantize_matvec_q4_k(A, (const float *)A, A, (float *)A, 8, 288, NULL), QMM_E_SHAPE);
    expect("matmul M = 0", qmm_matmul_q4_0(NULL, NULL, NULL, 0, 8, 32, NULL), QMM_E_SHAPE);
    expect("matmul N = 0", qmm_matmul_q4_0(NULL, NULL, NULL, 4, 0, 32, NULL), QMM_E_SHAPE);
    expect("matvec N = 0", qmm_matvec_q8_0(NULL, NULL, NULL, 0, 32, NULL), QMM_E_SHAPE);
    expect("quantize M = 0", qmm_quantize_q8_0(NULL, NULL, 0, 32, NULL), QMM_E_SHAPE);
    printf(fails ? "failed\n" : "ok\n");
    return fails != 0;
}
"""

CXX_PROGRAM = r"""
#include "qmm.h"
int main() { return qmm_abi_version() == 1 ? 0 : 1; }
"""


def _lib():
    path = os.path.join(PKG, "libqmm.so")
    if not os.path.exists(path):
        pytest.skip("libqmm.so is not built")
    return path


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_program_links_and_gets_status_codes(tmp_path):
    _lib()
    src = tmp_path / "consumer.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "consumer"
    cc = ["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", INC, str(src), "-o", str(exe),
          "-L", PKG, "-lqmm", "-Wl,-rpath," + PKG]
    out = subprocess.run(cc, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), (run.stdout, run.stderr)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_header_compiles_as_cxx(tmp_path):
    _lib()
    src = tmp_path / "consumer.cpp"
    src.write_text(CXX_PROGRAM)
    exe = tmp_path / "consumer_cxx"
    cc = ["g++", "-std=c++17", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", INC, str(src), "-o", str(exe),
          "-L", PKG, "-lqmm", "-Wl,-rpath," + PKG]
    out = subprocess.run(cc, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, (run.stdout, run.stderr)
