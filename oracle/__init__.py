"""qmm oracle -- TEST INFRASTRUCTURE ONLY.

Python access (numpy in, numpy out) to the plain scalar C oracle in
``qmm_oracle.c``.  Only the tests, the smoke check and the CPU-baseline leg of
the benchmark may import this package; the product path (the HIP library and
its binding) never does.

Every function here marshals arguments only; all arithmetic is in the C file,
which cites the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmm_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

Q4_0, Q8_0, Q2_K, Q4_K, Q6_K, Q4_1, Q5_0, Q5_1 = 0, 1, 2, 3, 4, 5, 6, 7
BLOCK_BYTES = {"q4_0": 18, "q8_0": 34, "q2_k": 84, "q8_k": 292, "q4_k": 144, "q6_k": 210,
               "q4_1": 20, "q5_0": 22, "q5_1": 24}
BLOCK_VALUES = {"q4_0": 32, "q8_0": 32, "q2_k": 256, "q8_k": 256, "q4_k": 256, "q6_k": 256,
                "q4_1": 32, "q5_0": 32, "q5_1": 32}
FMT_ID = {"q4_0": Q4_0, "q8_0": Q8_0, "q2_k": Q2_K, "q4_k": Q4_K, "q6_k": Q6_K, "q4_1": Q4_1, "q5_0": Q5_0,
          "q5_1": Q5_1}
K_QUANTS = ("q2_k", "q4_k", "q6_k")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2 -ffp-contract=off, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                               "-pthread", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P, I64, I32, U16 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_f16.restype = U16
        L.orc_f16_to_f32.argtypes = [U16]
        L.orc_f16_to_f32.restype = ctypes.c_float
        for name in ("orc_quantize_q8_0", "orc_quantize_q8_k", "orc_quantize_q4_0_w", "orc_quantize_q2_k_w",
                     "orc_quantize_q4_k_w", "orc_quantize_q6_k_w", "orc_quantize_q4_1_w", "orc_quantize_q5_0_w",
                     "orc_quantize_q5_1_w", "orc_dequantize_q4_1", "orc_dequantize_q5_0", "orc_dequantize_q5_1",
                     "orc_dequantize_q8_0", "orc_dequantize_q4_0", "orc_dequantize_q2_k", "orc_dequantize_q8_k",
                     "orc_dequantize_q4_k", "orc_dequantize_q6_k"):
            getattr(L, name).argtypes = [P, P, I64, I64]
            getattr(L, name).restype = None
        L.orc_matmul.argtypes = [I32, P, P, P, P, P, I64, I64, I64, I32]
        L.orc_matmul.restype = I32
        L.orc_matmul_sampled.argtypes = [I32, P, P, P, P, I64, P, P, I64]
        L.orc_matmul_sampled.restype = I32
        L.orc_f32_to_f16_array.argtypes = [P, P, I64]
        L.orc_f32_to_f16_array.restype = None
        L.orc_f16_to_f32_array.argtypes = [P, P, I64]
        L.orc_f16_to_f32_array.restype = None
        L.orc_get_rows.argtypes = [I32, P, P, I64, I64, I64, P]
        L.orc_get_rows.restype = I32
        L.orc_block_isum.argtypes = [I32, P, P]
        L.orc_block_isum.restype = ctypes.c_int32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f32(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32)


def _u8(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.uint8)


def row_bytes(fmt: str, K: int) -> int:
    return K // BLOCK_VALUES[fmt] * BLOCK_BYTES[fmt]


# -- fp16 -------------------------------------------------------------------
def f32_to_f16_bits(v: float) -> int:
    return int(lib().orc_f32_to_f16(float(v)))


def f16_bits_to_f32(h: int) -> float:
    return float(lib().orc_f16_to_f32(int(h)))


def f32_to_f16_array(x) -> np.ndarray:
    x = _f32(x).ravel()
    h = np.zeros(x.size, dtype=np.uint16)
    lib().orc_f32_to_f16_array(_ptr(x), _ptr(h), x.size)
    return h


def f16_to_f32_array(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16).ravel()
    x = np.zeros(h.size, dtype=np.float32)
    lib().orc_f16_to_f32_array(_ptr(h), _ptr(x), h.size)
    return x


# -- quantizers ---------------------------------------------------------------
def _quant(name: str, fmt: str, x) -> np.ndarray:
    x = _f32(x)
    if x.ndim == 1:
        x = x[None, :]
    rows, K = x.shape
    assert K % BLOCK_VALUES[fmt] == 0
    out = np.zeros((rows, row_bytes(fmt, K)), dtype=np.uint8)
    getattr(lib(), name)(_ptr(x), _ptr(out), rows, K)
    return out


def quantize_q8_0(x) -> np.ndarray:
    """f32 [M][K] -> Q8_0 bytes [M][K/32*34]."""
    return _quant("orc_quantize_q8_0", "q8_0", x)


def quantize_q8_k(x) -> np.ndarray:
    """f32 [M][K] -> Q8_K bytes [M][K/256*292]."""
    return _quant("orc_quantize_q8_k", "q8_k", x)


def quantize_q4_0_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q4_0 bytes [N][K/32*18]."""
    return _quant("orc_quantize_q4_0_w", "q4_0", w)


def quantize_q2_k_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q2_K bytes [N][K/256*84]."""
    return _quant("orc_quantize_q2_k_w", "q2_k", w)


def quantize_q4_k_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q4_K bytes [N][K/256*144]."""
    return _quant("orc_quantize_q4_k_w", "q4_k", w)


def quantize_q6_k_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q6_K bytes [N][K/256*210]."""
    return _quant("orc_quantize_q6_k_w", "q6_k", w)


def quantize_q4_1_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q4_1 bytes [N][K/32*20]."""
    return _quant("orc_quantize_q4_1_w", "q4_1", w)


def quantize_q5_0_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q5_0 bytes [N][K/32*22]."""
    return _quant("orc_quantize_q5_0_w", "q5_0", w)


def quantize_q5_1_w(w) -> np.ndarray:
    """f32 weights [N][K] -> Q5_1 bytes [N][K/32*24]."""
    return _quant("orc_quantize_q5_1_w", "q5_1", w)


def quantize_w(fmt: str, w) -> np.ndarray:
    return {"q4_0": quantize_q4_0_w, "q8_0": quantize_q8_0, "q2_k": quantize_q2_k_w,
            "q4_k": quantize_q4_k_w, "q6_k": quantize_q6_k_w, "q4_1": quantize_q4_1_w,
            "q5_0": quantize_q5_0_w, "q5_1": quantize_q5_1_w}[fmt](w)


def act_format(fmt: str) -> str:
    """Activation format paired with weight format `fmt` (Q8_K for the K-quants, else Q8_0)."""
    return "q8_k" if fmt in K_QUANTS else "q8_0"


def quantize_x(fmt: str, x) -> np.ndarray:
    """Activation quantizer paired with weight format `fmt`."""
    return quantize_q8_k(x) if fmt in K_QUANTS else quantize_q8_0(x)


def dequantize(fmt: str, blocks, K: int) -> np.ndarray:
    """Block bytes [rows][row_bytes] -> float64 values [rows][K] (each exact)."""
    b = _u8(blocks)
    rows = b.size // row_bytes(fmt, K)
    out = np.zeros((rows, K), dtype=np.float64)
    getattr(lib(), "orc_dequantize_" + fmt)(_ptr(b), _ptr(out), rows, K)
    return out


# -- products -----------------------------------------------------------------
def matmul(fmt: str, w, xq, M: int, N: int, K: int, threads: int = 1, want=("y",)):
    """Y[M][N] for weights `w` (format fmt) and quantized activations `xq`.

    Returns a dict with any of: 'y' (f32), 'y64' (double, before the final
    rounding), 'mag' (double, sum of |term| per output, the tolerance base)."""
    w = _u8(w)
    xq = _u8(xq)
    assert w.size == N * row_bytes(fmt, K)
    assert xq.size == M * row_bytes(act_format(fmt), K)
    res = {}
    y = np.zeros((M, N), dtype=np.float32) if "y" in want else None
    y64 = np.zeros((M, N), dtype=np.float64) if "y64" in want else None
    mag = np.zeros((M, N), dtype=np.float64) if "mag" in want else None
    lib().orc_matmul(FMT_ID[fmt], _ptr(w), _ptr(xq),
                     _ptr(y) if y is not None else None,
                     _ptr(y64) if y64 is not None else None,
                     _ptr(mag) if mag is not None else None, M, N, K, int(threads))
    for k, v in (("y", y), ("y64", y64), ("mag", mag)):
        if v is not None:
            res[k] = v
    return res


def matmul_sampled(fmt: str, w, xq, mi, ni, K: int):
    """(y64, mag) for the outputs (mi[c], ni[c]) only."""
    w = _u8(w)
    xq = _u8(xq)
    mi = np.ascontiguousarray(mi, dtype=np.int64)
    ni = np.ascontiguousarray(ni, dtype=np.int64)
    y64 = np.zeros(mi.size, dtype=np.float64)
    mag = np.zeros(mi.size, dtype=np.float64)
    lib().orc_matmul_sampled(FMT_ID[fmt], _ptr(w), _ptr(xq), _ptr(mi), _ptr(ni), mi.size,
                             _ptr(y64), _ptr(mag), K)
    return y64, mag


def get_rows(fmt: str, w, ids, N: int, K: int) -> np.ndarray:
    """f32 [len(ids)][K]: the decoded rows ids of the [N][K] table `w` (NaN rows for ids outside [0, N))."""
    w = _u8(w)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    assert w.size == N * row_bytes(fmt, K)
    out = np.zeros((ids.size, K), dtype=np.float32)
    assert lib().orc_get_rows(FMT_ID[fmt], _ptr(w), _ptr(ids), ids.size, N, K, _ptr(out)) == 0
    return out


def block_isum(fmt: str, wblock, xblock) -> int:
    """Exact integer sum of one Q4_0 (or Q8_0) x Q8_0 block pair."""
    w = _u8(wblock)
    x = _u8(xblock)
    return int(lib().orc_block_isum(FMT_ID[fmt], _ptr(w), _ptr(x)))
