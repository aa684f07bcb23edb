"""Seeded synthetic inputs, shared by the oracle side and the HIP side.

This module holds no arithmetic of the quantized-product method: it only
draws f32 arrays (Gaussian weights and activations, optional outliers) from
a fully specified counter-based stream, so both sides of a parity test see
the same bytes on any machine.

Stream definition
-----------------
* ``splitmix64``: output i (0-based) of the generator seeded with ``s`` is
  ``mix(s + (i + 1) * 0x9E3779B97F4A7C15)`` where ``mix`` is the SplitMix64
  finaliser (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
  z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31`` (all mod 2**64).
  Because output i depends only on (s, i), any slice can be drawn directly.
* uniform in (0, 1): ``((z >> 11) + 0.5) * 2**-53`` (never 0 or 1).
* standard normal: Box-Muller, cosine branch only, in double:
  normal j uses outputs 2j and 2j+1 as (u1, u2):
  ``sqrt(-2 ln u1) * cos(2 pi u2)``.
* a normal of std ``sigma`` is ``float32(sigma * z)`` (one rounding).

Seeds: ``seed_for(config, stream) = 0x514D4D00 + 16 * config + stream`` with
stream 0 = weights, 1 = activations, 2 = outlier picks, 3+ = extra matrices.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
# Entries are drawn in cache-sized chunks, several chunks at a time on host
# threads (numpy releases the interpreter lock inside its array loops).  Each
# entry depends only on (seed, index), so the bytes do not depend on either.
_CHUNK = 1 << 18
_THREADS = max(1, min(16, os.cpu_count() or 1))

SEED_BASE = 0x514D4D00


def seed_for(config: int, stream: int) -> int:
    """Seed of `stream` (0 weights, 1 activations, 2 outliers, 3+ extra) of a workload id."""
    return (SEED_BASE + 16 * int(config) + int(stream)) & 0xFFFFFFFFFFFFFFFF


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Outputs start .. start+count-1 of SplitMix64 seeded with `seed` (uint64 array)."""
    i = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + i * GAMMA
        z ^= z >> np.uint64(30)
        z *= _M1
        z ^= z >> np.uint64(27)
        z *= _M2
        z ^= z >> np.uint64(31)
    return z


def uniform01(seed: int, start: int, count: int) -> np.ndarray:
    """Doubles in the open interval (0, 1) from outputs start.. of the stream."""
    z = splitmix64(seed, start, count)
    return ((z >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def normal(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Standard normals start .. start+count-1 of the stream, in double."""
    out = np.empty(count, dtype=np.float64)
    for c0 in range(0, count, _CHUNK):
        c1 = min(count, c0 + _CHUNK)
        u = uniform01(seed, 2 * (start + c0), 2 * (c1 - c0))
        u1 = u[0::2]
        u2 = u[1::2]
        out[c0:c1] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    return out


def gaussian_f32(shape, sigma: float, seed: int) -> np.ndarray:
    """float32 array of the given shape, entries float32(sigma * N(0,1)) in C order."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)

    def fill(c0):
        c1 = min(n, c0 + _CHUNK)
        out[c0:c1] = (sigma * normal(seed, c1 - c0, start=c0)).astype(np.float32)

    starts = range(0, n, _CHUNK)
    if len(starts) <= 1 or _THREADS == 1:
        for c0 in starts:
            fill(c0)
    else:
        with ThreadPoolExecutor(max_workers=_THREADS) as ex:
            list(ex.map(fill, starts))
    return out.reshape(shape)


def pick_without_replacement(seed: int, population: int, count: int) -> np.ndarray:
    """`count` distinct indices of range(population): the ones with the smallest stream keys.

    Ties in the 64-bit keys are broken by index (stable sort), so the pick is
    fully determined by (seed, population, count)."""
    keys = splitmix64(seed, 0, population)
    order = np.argsort(keys, kind="stable")
    return np.sort(order[:count]).astype(np.int64)


def with_outliers(x: np.ndarray, frac: float, factor: float, seed: int) -> np.ndarray:
    """Copy of 1-D or 2-D `x` with round(frac * row_len) entries per row multiplied by `factor`.

    The picked indices are the same for every row (drawn once from `seed`)."""
    x = np.array(x, dtype=np.float32, copy=True)
    k = x.shape[-1]
    count = int(round(frac * k))
    if count == 0:
        return x
    idx = pick_without_replacement(seed, k, count)
    x[..., idx] = (x[..., idx].astype(np.float64) * factor).astype(np.float32)
    return x


# ---------------------------------------------------------------------------
# Named workloads.  Shapes and distributions follow the five benchmark
# configurations of the quantized product: Gaussian weights of std 0.02 and
# Gaussian activations of std 1, quantized by whichever side consumes them.
# ---------------------------------------------------------------------------
WORKLOADS = {
    "q4_0_matvec_512x1024": dict(id=0, fmt="q4_0", M=1, N=512, K=1024),
    "q4_0_matvec_12288x4096": dict(id=1, fmt="q4_0", M=1, N=12288, K=4096,
                                   outlier_frac=0.01, outlier_factor=20.0),
    "q8_0_matvec_layer7b": dict(id=2, fmt="q8_0", M=1,
                                shapes=[(12288, 4096), (22016, 4096), (4096, 11008)]),
    "q2_k_matvec_12288x4096": dict(id=3, fmt="q2_k", M=1, N=12288, K=4096),
    "q4_0_matmul_2048x12288x4096": dict(id=4, fmt="q4_0", M=2048, N=12288, K=4096),
}


def weights(n: int, k: int, config: int, stream: int = 0) -> np.ndarray:
    """f32 [n][k] weights ~ N(0, 0.02) for workload `config`."""
    return gaussian_f32((n, k), 0.02, seed_for(config, stream))


def activations(m: int, k: int, config: int, stream: int = 1,
                outlier_frac: float = 0.0, outlier_factor: float = 1.0) -> np.ndarray:
    """f32 [m][k] activations ~ N(0, 1) for workload `config`, optional outliers."""
    x = gaussian_f32((m, k), 1.0, seed_for(config, stream))
    if outlier_frac > 0.0:
        x = with_outliers(x, outlier_frac, outlier_factor, seed_for(config, 2))
    return x
