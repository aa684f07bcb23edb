"""matmul_quantize_q8_amd -- block-quantized weight x Q8_0/Q8_K activation
products on MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libqmm.so`` (declared in
``include/qmm.h``).  Every function has the name of its C entry point and
only marshals arguments: device pointers come from torch tensors (PyTorch
supplies device memory and the current stream), every step of the
computation runs in the library's HIP kernels.  There is no CPU fallback: if
the library is missing or refuses a call, an exception is raised.

Byte layouts (see the header): Q8_0 34 B / 32 values, Q4_0 18 B / 32,
Q2_K 84 B / 256, Q8_K 292 B / 256.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmm.so")

BLOCK_BYTES = {"q4_0": 18, "q8_0": 34, "q2_k": 84, "q8_k": 292, "q4_k": 144, "q6_k": 210,
               "q4_1": 20, "q5_0": 22, "q5_1": 24}
BLOCK_VALUES = {"q4_0": 32, "q8_0": 32, "q2_k": 256, "q8_k": 256, "q4_k": 256, "q6_k": 256,
                "q4_1": 32, "q5_0": 32, "q5_1": 32}
ACT_FORMAT = {"q4_0": "q8_0", "q8_0": "q8_0", "q2_k": "q8_k", "q4_k": "q8_k", "q6_k": "q8_k",
              "q4_1": "q8_0", "q5_0": "q8_0", "q5_1": "q8_0"}
WEIGHT_FORMATS = ("q4_0", "q8_0", "q4_1", "q5_0", "q5_1", "q2_k", "q4_k", "q6_k")
# Weight formats with a fused quantize + matvec decode entry point.
FUSED_FORMATS = ("q4_0", "q8_0", "q2_k", "q4_k", "q6_k")

STATUS = {0: "QMM_OK", 1: "QMM_E_SHAPE", 2: "QMM_E_NULL", 3: "QMM_E_ALIGN", 4: "QMM_E_DEVICE", 5: "QMM_E_LAUNCH"}


class QmmError(RuntimeError):
    """A libqmm entry point returned a status other than QMM_OK."""

    def __init__(self, status: int, name: str, text: str):
        super().__init__(f"{name}: {text}")
        self.status = status
        self.code = STATUS.get(status, str(status))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libqmm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with matmul_quantize_q8_amd/build.py "
                              "(or __graft_entry__.build()); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.qmm_status_string.argtypes = [ctypes.c_int]
        L.qmm_status_string.restype = ctypes.c_char_p
        L.qmm_abi_version.argtypes = []
        L.qmm_abi_version.restype = ctypes.c_int
        for name in ["qmm_quantize_q8_k"] + ["qmm_quantize_" + f for f in WEIGHT_FORMATS]:
            getattr(L, name).argtypes = [P, P, I64, I64, P]
            getattr(L, name).restype = ctypes.c_int
        for name in ["qmm_matvec_" + f for f in WEIGHT_FORMATS]:
            getattr(L, name).argtypes = [P, P, P, I64, I64, P]
            getattr(L, name).restype = ctypes.c_int
        for name in ["qmm_quantize_matvec_" + f for f in FUSED_FORMATS]:
            getattr(L, name).argtypes = [P, P, P, P, I64, I64, P]
            getattr(L, name).restype = ctypes.c_int
        for name in ["qmm_get_rows_" + f for f in WEIGHT_FORMATS]:
            getattr(L, name).argtypes = [P, P, P, I64, I64, I64, P]
            getattr(L, name).restype = ctypes.c_int
        for name in ["qmm_matmul_" + f for f in WEIGHT_FORMATS]:
            getattr(L, name).argtypes = [P, P, P, I64, I64, I64, P]
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


EXPORTS = tuple(["qmm_status_string", "qmm_abi_version", "qmm_quantize_q8_k"] +
                ["qmm_quantize_matvec_" + f for f in FUSED_FORMATS] +
                [p + f for p in ("qmm_quantize_", "qmm_matvec_", "qmm_matmul_", "qmm_get_rows_")
                 for f in WEIGHT_FORMATS])


def row_bytes(fmt: str, K: int) -> int:
    """Bytes of one row of K values in block format `fmt`."""
    return K // BLOCK_VALUES[fmt] * BLOCK_BYTES[fmt]


def _addr(t) -> int | None:
    """Device address of a tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name: str, st: int) -> None:
    if st != 0:
        raise QmmError(st, name, lib().qmm_status_string(st).decode())


def _call(name: str, *args) -> None:
    _check(name, getattr(lib(), name)(*args))


# -- quantizers -----------------------------------------------------------------
def qmm_quantize_q8_0(x, xq, M: int, K: int, stream=None) -> None:
    """f32 [M][K] -> Q8_0 blocks (activations, or Q8_0 weight rows)."""
    _call("qmm_quantize_q8_0", _addr(x), _addr(xq), M, K, _stream(stream))


def qmm_quantize_q8_k(x, xq, M: int, K: int, stream=None) -> None:
    """f32 [M][K] -> Q8_K blocks (activations paired with Q2_K weights)."""
    _call("qmm_quantize_q8_k", _addr(x), _addr(xq), M, K, _stream(stream))


def qmm_quantize_q4_0(w, wq, N: int, K: int, stream=None) -> None:
    """f32 weights [N][K] -> Q4_0 blocks."""
    _call("qmm_quantize_q4_0", _addr(w), _addr(wq), N, K, _stream(stream))


def qmm_quantize_q2_k(w, wq, N: int, K: int, stream=None) -> None:
    """f32 weights [N][K] -> Q2_K blocks."""
    _call("qmm_quantize_q2_k", _addr(w), _addr(wq), N, K, _stream(stream))


def qmm_quantize_q4_k(w, wq, N: int, K: int, stream=None) -> None:
    """f32 weights [N][K] -> Q4_K blocks."""
    _call("qmm_quantize_q4_k", _addr(w), _addr(wq), N, K, _stream(stream))


def qmm_quantize_q6_k(w, wq, N: int, K: int, stream=None) -> None:
    """f32 weights [N][K] -> Q6_K blocks."""
    _call("qmm_quantize_q6_k", _addr(w), _addr(wq), N, K, _stream(stream))


# -- products -------------------------------------------------------------------
def qmm_matvec_q8_0(w, xq, y, N: int, K: int, stream=None) -> None:
    _call("qmm_matvec_q8_0", _addr(w), _addr(xq), _addr(y), N, K, _stream(stream))


def qmm_matvec_q4_0(w, xq, y, N: int, K: int, stream=None) -> None:
    _call("qmm_matvec_q4_0", _addr(w), _addr(xq), _addr(y), N, K, _stream(stream))


def qmm_matvec_q2_k(w, xq8k, y, N: int, K: int, stream=None) -> None:
    _call("qmm_matvec_q2_k", _addr(w), _addr(xq8k), _addr(y), N, K, _stream(stream))


def qmm_matvec_q4_k(w, xq8k, y, N: int, K: int, stream=None) -> None:
    _call("qmm_matvec_q4_k", _addr(w), _addr(xq8k), _addr(y), N, K, _stream(stream))


def qmm_matvec_q6_k(w, xq8k, y, N: int, K: int, stream=None) -> None:
    _call("qmm_matvec_q6_k", _addr(w), _addr(xq8k), _addr(y), N, K, _stream(stream))


def qmm_quantize_matvec_q4_0(w, x, xq, y, N: int, K: int, stream=None) -> None:
    """Fused decode step: quantize f32 x [K] to Q8_0 (written to xq unless it
    is None) and y = W x for Q4_0 weights, in one launch."""
    _call("qmm_quantize_matvec_q4_0", _addr(w), _addr(x), _addr(xq), _addr(y), N, K, _stream(stream))


def qmm_quantize_matvec_q8_0(w, x, xq, y, N: int, K: int, stream=None) -> None:
    """As qmm_quantize_matvec_q4_0, for Q8_0 weights."""
    _call("qmm_quantize_matvec_q8_0", _addr(w), _addr(x), _addr(xq), _addr(y), N, K, _stream(stream))


def qmm_quantize_matvec_q2_k(w, x, xq8k, y, N: int, K: int, stream=None) -> None:
    """Fused decode step for Q2_K weights: quantize f32 x [K] to Q8_K (written
    to xq8k unless it is None) and y = W x, in one launch."""
    _call("qmm_quantize_matvec_q2_k", _addr(w), _addr(x), _addr(xq8k), _addr(y), N, K, _stream(stream))


def qmm_quantize_matvec_q4_k(w, x, xq8k, y, N: int, K: int, stream=None) -> None:
    """As qmm_quantize_matvec_q2_k, for Q4_K weights."""
    _call("qmm_quantize_matvec_q4_k", _addr(w), _addr(x), _addr(xq8k), _addr(y), N, K, _stream(stream))


def qmm_quantize_matvec_q6_k(w, x, xq8k, y, N: int, K: int, stream=None) -> None:
    """As qmm_quantize_matvec_q2_k, for Q6_K weights."""
    _call("qmm_quantize_matvec_q6_k", _addr(w), _addr(x), _addr(xq8k), _addr(y), N, K, _stream(stream))


def qmm_matmul_q4_0(w, xq, y, M: int, N: int, K: int, stream=None) -> None:
    _call("qmm_matmul_q4_0", _addr(w), _addr(xq), _addr(y), M, N, K, _stream(stream))


def qmm_matmul_q8_0(w, xq, y, M: int, N: int, K: int, stream=None) -> None:
    _call("qmm_matmul_q8_0", _addr(w), _addr(xq), _addr(y), M, N, K, _stream(stream))


def qmm_matmul_q2_k(w, xq8k, y, M: int, N: int, K: int, stream=None) -> None:
    _call("qmm_matmul_q2_k", _addr(w), _addr(xq8k), _addr(y), M, N, K, _stream(stream))


def qmm_matmul_q4_k(w, xq8k, y, M: int, N: int, K: int, stream=None) -> None:
    _call("qmm_matmul_q4_k", _addr(w), _addr(xq8k), _addr(y), M, N, K, _stream(stream))


def qmm_matmul_q6_k(w, xq8k, y, M: int, N: int, K: int, stream=None) -> None:
    _call("qmm_matmul_q6_k", _addr(w), _addr(xq8k), _addr(y), M, N, K, _stream(stream))


def _quantize_w(fmt):
    name = "qmm_quantize_" + fmt

    def quantize(w, wq, N: int, K: int, stream=None) -> None:
        _call(name, _addr(w), _addr(wq), N, K, _stream(stream))
    quantize.__name__ = name
    quantize.__doc__ = f"f32 weights [N][K] -> {fmt.upper()} blocks."
    return quantize


def _matvec(fmt):
    name = "qmm_matvec_" + fmt

    def matvec(w, xq, y, N: int, K: int, stream=None) -> None:
        _call(name, _addr(w), _addr(xq), _addr(y), N, K, _stream(stream))
    matvec.__name__ = name
    return matvec


def _matmul(fmt):
    name = "qmm_matmul_" + fmt

    def matmul(w, xq, y, M: int, N: int, K: int, stream=None) -> None:
        _call(name, _addr(w), _addr(xq), _addr(y), M, N, K, _stream(stream))
    matmul.__name__ = name
    return matmul


qmm_quantize_q4_1, qmm_quantize_q5_0, qmm_quantize_q5_1 = (_quantize_w(f) for f in ("q4_1", "q5_0", "q5_1"))
qmm_matvec_q4_1, qmm_matvec_q5_0, qmm_matvec_q5_1 = (_matvec(f) for f in ("q4_1", "q5_0", "q5_1"))
qmm_matmul_q4_1, qmm_matmul_q5_0, qmm_matmul_q5_1 = (_matmul(f) for f in ("q4_1", "q5_0", "q5_1"))


def _get_rows(fmt):
    name = "qmm_get_rows_" + fmt

    def get_rows(w, ids, out, n_ids: int, N: int, K: int, stream=None) -> None:
        """out[t][:] = decoded row ids[t] of the table w (f32; NaN rows for ids outside [0, N))."""
        _call(name, _addr(w), _addr(ids), _addr(out), n_ids, N, K, _stream(stream))
    get_rows.__name__ = name
    return get_rows


qmm_get_rows_q4_0 = _get_rows("q4_0")
qmm_get_rows_q8_0 = _get_rows("q8_0")
qmm_get_rows_q2_k = _get_rows("q2_k")
qmm_get_rows_q4_k = _get_rows("q4_k")
qmm_get_rows_q6_k = _get_rows("q6_k")
qmm_get_rows_q4_1 = _get_rows("q4_1")
qmm_get_rows_q5_0 = _get_rows("q5_0")
qmm_get_rows_q5_1 = _get_rows("q5_1")



QUANTIZE_W = {f: globals()["qmm_quantize_" + f] for f in WEIGHT_FORMATS}
QUANTIZE_X = {f: (qmm_quantize_q8_k if ACT_FORMAT[f] == "q8_k" else qmm_quantize_q8_0) for f in WEIGHT_FORMATS}
MATVEC = {f: globals()["qmm_matvec_" + f] for f in WEIGHT_FORMATS}
MATMUL = {f: globals()["qmm_matmul_" + f] for f in WEIGHT_FORMATS}
QUANTIZE_MATVEC = {"q4_0": qmm_quantize_matvec_q4_0, "q8_0": qmm_quantize_matvec_q8_0,
                   "q2_k": qmm_quantize_matvec_q2_k, "q4_k": qmm_quantize_matvec_q4_k,
                   "q6_k": qmm_quantize_matvec_q6_k}
GET_ROWS = {f: globals()["qmm_get_rows_" + f] for f in WEIGHT_FORMATS}
