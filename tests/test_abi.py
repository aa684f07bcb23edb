"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments before touching any device."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qmm.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def q():
    import matmul_quantize_q8_amd as q
    q.lib()
    return q


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("qmm_quantize_q8_0", "qmm_quantize_q8_k", "qmm_matvec_q8_0", "qmm_matvec_q4_0",
              "qmm_matvec_q2_k", "qmm_matmul_q4_0", "qmm_matmul_q2_k"):
        assert n in names


def test_library_exports_every_declared_symbol(q):
    lib = ctypes.CDLL(q.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(_declared()) == set(q.EXPORTS)
    for n in q.EXPORTS:
        assert callable(getattr(q, n, None)) or n in ("qmm_status_string", "qmm_abi_version")


def test_library_is_gfx950_code(q):
    data = open(q.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings_and_version(q):
    L = q.lib()
    assert L.qmm_abi_version() == 1
    for code in range(6):
        assert L.qmm_status_string(code).decode().startswith(q.STATUS[code])


# Argument checks happen before any device call, so they run without a GPU.
A = 1 << 20          # a 16-byte aligned fake device address (never dereferenced)


@pytest.mark.parametrize("call,code", [
    (lambda L: L.qmm_quantize_q8_0(A, A, 1, 48, None), 1),        # K % 32
    (lambda L: L.qmm_quantize_q8_0(A, A, 1, 0, None), 1),         # K = 0
    (lambda L: L.qmm_quantize_q8_0(A, A, -1, 32, None), 1),       # M < 0
    (lambda L: L.qmm_quantize_q8_k(A, A, 1, 32 * 3, None), 1),    # K % 256
    (lambda L: L.qmm_quantize_q8_0(None, A, 1, 32, None), 2),     # NULL
    (lambda L: L.qmm_quantize_q8_0(A + 4, A, 1, 32, None), 3),    # misaligned
    (lambda L: L.qmm_matvec_q4_0(A, A, None, 8, 64, None), 2),
    (lambda L: L.qmm_matvec_q4_0(A, A + 8, A, 8, 64, None), 3),
    (lambda L: L.qmm_matvec_q2_k(A, A, A, 8, 128, None), 1),
    (lambda L: L.qmm_matmul_q4_0(A, A, A, 4, 8, 33, None), 1),
    (lambda L: L.qmm_matmul_q4_0(A, A, A, 1 << 31, 8, 32, None), 1),   # M >= 2^31
    (lambda L: L.qmm_matmul_q2_k(A, A, A, 4, 8, 256 * 3 + 32, None), 1),
    (lambda L: L.qmm_matmul_q4_0(A, A, A, 1 << 30, 1 << 30, 32, None), 1),   # output bytes overflow
    (lambda L: L.qmm_quantize_matvec_q4_0(A, A, A, A, 8, 48, None), 1),      # K % 32
    (lambda L: L.qmm_quantize_matvec_q4_0(A, None, A, A, 8, 64, None), 2),   # x NULL
    (lambda L: L.qmm_quantize_matvec_q8_0(A, A, A, None, 8, 64, None), 2),   # y NULL
    (lambda L: L.qmm_quantize_matvec_q8_0(A, A, A + 2, A, 8, 64, None), 3),  # xq misaligned
    (lambda L: L.qmm_quantize_matvec_q4_0(A, A + 4, None, A, 8, 64, None), 3),
    (lambda L: L.qmm_quantize_matvec_q2_k(A, A, A, A, 8, 32 * 9, None), 1),   # K % 256
    (lambda L: L.qmm_quantize_matvec_q4_k(A, A, A + 4, A, 8, 256, None), 3),  # xq8k misaligned
    (lambda L: L.qmm_quantize_matvec_q6_k(None, A, A, A, 8, 256, None), 2),   # w NULL
    (lambda L: L.qmm_matvec_q4_k(A, A, A, 8, 32 * 9, None), 1),                # K % 256
    (lambda L: L.qmm_matmul_q6_k(A, A, A, 2, 8, 256 + 32, None), 1),
    (lambda L: L.qmm_quantize_q6_k(A, A, 1, 128, None), 1),
    (lambda L: L.qmm_matvec_q6_k(A, None, A, 8, 256, None), 2),
    (lambda L: L.qmm_get_rows_q4_0(A, A, A, 4, 8, 48, None), 1),
    (lambda L: L.qmm_get_rows_q4_k(A, A + 4, A, 4, 8, 256, None), 3),
    (lambda L: L.qmm_get_rows_q8_0(A, None, A, 4, 8, 64, None), 2),
    # the smallest K whose 128-row activation tile (Q8_0 or Q8_K) exceeds the
    # 32-bit buffer offsets of the MFMA prefill kernels
    (lambda L: L.qmm_matmul_q4_0(A, A, A, 4, 8, 32 * ((2**31 - 1) // (128 * 34) + 1), None), 1),
    (lambda L: L.qmm_matmul_q8_0(A, A, A, 4, 8, 32 * ((2**31 - 1) // (128 * 34) + 1), None), 1),
    (lambda L: L.qmm_matmul_q5_0(A, A, A, 4, 8, 32 * ((2**31 - 1) // (128 * 34) + 1), None), 1),
    (lambda L: L.qmm_matmul_q4_1(A, A, A, 4, 8, 32 * ((2**31 - 1) // (128 * 34) + 1), None), 1),
    (lambda L: L.qmm_matmul_q5_1(A, A, A, 4, 8, 32 * ((2**31 - 1) // (128 * 34) + 1), None), 1),
    (lambda L: L.qmm_matmul_q2_k(A, A, A, 4, 8, 256 * ((2**31 - 1) // (128 * 292) + 1), None), 1),
    (lambda L: L.qmm_matmul_q4_k(A, A, A, 4, 8, 256 * ((2**31 - 1) // (128 * 292) + 1), None), 1),
    (lambda L: L.qmm_matmul_q6_k(A, A, A, 4, 8, 256 * ((2**31 - 1) // (128 * 292) + 1), None), 1),
])
def test_argument_errors_without_device(q, call, code):
    assert call(q.lib()) == code


# ---------------------------------------------------------------------------
# The measurement probes: a library and header of their own (qmm_probe.h,
# libqmm_probe.so); the product library does not export them.
# ---------------------------------------------------------------------------
PROBE_HEADER = os.path.join(ROOT, "include", "qmm_probe.h")


def _probe_declared():
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(qmm_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def probe():
    from matmul_quantize_q8_amd import probe
    probe.lib()
    return probe


def test_probe_library_exports_its_header_and_product_does_not(q, probe):
    plib = ctypes.CDLL(probe.LIB_PATH)
    assert set(_probe_declared()) == set(probe.EXPORTS)
    for n in _probe_declared():
        assert hasattr(plib, n), n
    prod = ctypes.CDLL(q.LIB_PATH)
    for n in _probe_declared():
        assert not hasattr(prod, n), n
    assert not set(_probe_declared()) & set(_declared())


def test_probe_read_span(probe):
    assert probe.read_span(4, 4) == 16384
    assert probe.read_span(16, 16) == 262144
    assert probe.read_span(3, 4) == 0 and probe.read_span(4, 5) == 0


@pytest.mark.parametrize("call,code", [
    (lambda L: L.qmm_peak_read(A, 0, A, 4, 4, 1, None), 1),
    (lambda L: L.qmm_peak_read(A, 24, A, 4, 4, 1, None), 1),            # not a multiple of 16
    (lambda L: L.qmm_peak_read(A, 32, A, 3, 4, 1, None), 1),            # unsupported loads per lane
    (lambda L: L.qmm_peak_read(A, 32, A, 4, 2, 0, None), 1),            # unsupported waves
    (lambda L: L.qmm_peak_read(None, 32, A, 4, 4, 1, None), 2),
    (lambda L: L.qmm_peak_read(A, 32, None, 4, 4, 1, None), 2),
    (lambda L: L.qmm_peak_read(A + 8, 32, A, 4, 4, 1, None), 3),
    (lambda L: L.qmm_peak_read(A, 32, A + 2, 4, 4, 1, None), 3),
    (lambda L: L.qmm_peak_mfma_i8(A, 0, 10, None), 1),
    (lambda L: L.qmm_peak_mfma_i8(A, 8, 1000001, None), 1),      # out would pass 2^31
    (lambda L: L.qmm_peak_mfma_i8(A, (1 << 20) + 1, 10, None), 1),
    (lambda L: L.qmm_peak_mfma_i8(None, 8, 10, None), 2),
    (lambda L: L.qmm_peak_mfma_i8(A + 4, 8, 10, None), 3),
    (lambda L: L.qmm_probe_issue(4, 2, 10, A, A, None), 1),        # no mode 4
    (lambda L: L.qmm_probe_issue(0, 4, 10, A, A, None), 1),        # 1 or 2 waves per SIMD
    (lambda L: L.qmm_probe_issue(2, 2, 0, A, A, None), 1),
    (lambda L: L.qmm_probe_issue(2, 2, 1000001, A, A, None), 1),
    (lambda L: L.qmm_probe_issue(1, 1, 10, None, A, None), 2),
    (lambda L: L.qmm_probe_issue(1, 1, 10, A, None, None), 2),
    (lambda L: L.qmm_probe_issue(1, 1, 10, A + 2, A, None), 3),
])
def test_probe_argument_errors_without_device(probe, call, code):
    assert call(probe.lib()) == code


def test_empty_problem_is_a_shape_error(q):
    """M < 1 or N < 1 is QMM_E_SHAPE (the header's size rule), reported before
    any pointer is looked at."""
    L = q.lib()
    assert L.qmm_matmul_q4_0(None, None, None, 0, 8, 32, None) == 1
    assert L.qmm_matmul_q4_0(None, None, None, 4, 0, 32, None) == 1
    assert L.qmm_matmul_q2_k(None, None, None, -1, 8, 256, None) == 1
    assert L.qmm_matvec_q8_0(None, None, None, 0, 32, None) == 1
    assert L.qmm_quantize_q8_0(None, None, 0, 64, None) == 1
    assert L.qmm_quantize_q8_k(None, None, 0, 256, None) == 1
    assert L.qmm_quantize_matvec_q4_0(None, None, None, None, 0, 64, None) == 1
    assert L.qmm_quantize_matvec_q6_k(None, None, None, None, 0, 256, None) == 1
    assert L.qmm_get_rows_q4_0(None, None, None, 0, 8, 32, None) == 1
    assert L.qmm_get_rows_q4_0(None, None, None, 4, 0, 32, None) == 1


def test_python_binding_raises(q):
    with pytest.raises(q.QmmError) as e:
        q.qmm_quantize_q8_0(A, A, 1, 33, stream=0)
    assert e.value.code == "QMM_E_SHAPE"


def test_missing_library_fails_loudly(tmp_path):
    """Without libqmm.so the binding raises instead of computing anything
    (there is no CPU fallback)."""
    import subprocess
    import sys
    code = ("import matmul_quantize_q8_amd as q\n"
            "q.LIB_PATH = q.os.path.join(%r, 'libqmm.so')\n"
            "q._lib = None\n"
            "try:\n"
            "    q.qmm_quantize_q8_0(1 << 20, 1 << 20, 1, 32, stream=0)\n"
            "except ImportError as e:\n"
            "    print('raised', 'no fallback' in str(e))\n" % str(tmp_path))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert out.stdout.strip() == "raised True", (out.stdout, out.stderr)


def test_product_path_has_no_oracle_dependency():
    """The package never imports or loads the oracle."""
    pkg = os.path.join(ROOT, "matmul_quantize_q8_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                for bad in ("import oracle", "from oracle", "liboracle", "qmm_oracle"):
                    assert bad not in text, (f, bad)
