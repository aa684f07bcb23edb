"""Binding of libqmm_probe.so (include/qmm_probe.h): the attainable-peak
probes the benchmark reports the product kernels against.  Measurement
only; the product binding in this package neither loads nor needs it."""
from __future__ import annotations

import ctypes
import os

from . import QmmError, _addr, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm_probe.so")
EXPORTS = ("qmm_probe_read_span", "qmm_peak_read", "qmm_peak_mfma_i8", "qmm_probe_issue")
LOADS_PER_LANE = (1, 2, 4, 8, 16)
WAVES_PER_WG = (4, 8, 16)
_STATUS = {0: "QMM_PROBE_OK", 1: "QMM_PROBE_E_SHAPE", 2: "QMM_PROBE_E_NULL", 3: "QMM_PROBE_E_ALIGN",
           4: "QMM_PROBE_E_DEVICE", 5: "QMM_PROBE_E_LAUNCH"}
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with matmul_quantize_q8_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.qmm_probe_read_span.argtypes = [I32, I32]
        L.qmm_probe_read_span.restype = I64
        L.qmm_peak_read.argtypes = [P, I64, P, I32, I32, I32, P]
        L.qmm_peak_read.restype = I32
        L.qmm_peak_mfma_i8.argtypes = [P, I64, I64, P]
        L.qmm_peak_mfma_i8.restype = I32
        L.qmm_probe_issue.argtypes = [I32, I32, I64, P, P, P]
        L.qmm_probe_issue.restype = I32
        _lib = L
    return _lib


def _check(name: str, st: int) -> None:
    if st != 0:
        raise QmmError(st, name, _STATUS.get(st, str(st)))


def read_span(loads_per_lane: int, waves_per_wg: int) -> int:
    """Bytes one workgroup of the read probe covers (0 for unsupported parameters)."""
    return int(lib().qmm_probe_read_span(loads_per_lane, waves_per_wg))


def qmm_peak_read(buf, nbytes: int, sink, loads_per_lane: int = 4, waves_per_wg: int = 4, nontemporal: bool = True,
                  stream=None) -> None:
    """Stream nbytes of buf once; sink[b] = XOR of the words of workgroup b's span."""
    _check("qmm_peak_read", lib().qmm_peak_read(_addr(buf), nbytes, _addr(sink), loads_per_lane, waves_per_wg,
                                                int(bool(nontemporal)), _stream(stream)))


def qmm_peak_mfma_i8(out, workgroups: int, iters: int, stream=None) -> None:
    """workgroups x 4 waves x 4 chains of iters int8 MFMAs; out[t] = 2048 * iters."""
    _check("qmm_peak_mfma_i8", lib().qmm_peak_mfma_i8(_addr(out), workgroups, iters, _stream(stream)))


ISSUE_MODES = {"fma": 0, "mfma": 1, "mixed": 2, "fma_sgpr": 3}


def qmm_probe_issue(mode: str, waves_per_simd: int, iters: int, out, outi, stream=None) -> None:
    """Issue-rate loop on every SIMD: per wave and iteration 128 f32 FMAs with
    vector-register operands ("fma"), 4 int8 MFMAs ("mfma"), both interleaved
    ("mixed"), or the FMAs with one scalar-register operand ("fma_sgpr");
    outi[t] = 2048 * iters when MFMAs run."""
    _check("qmm_probe_issue", lib().qmm_probe_issue(ISSUE_MODES[mode], waves_per_simd, iters, _addr(out), _addr(outi),
                                                    _stream(stream)))
