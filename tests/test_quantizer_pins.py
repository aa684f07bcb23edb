"""Hand-computed blocks for the weight quantizers whose rules are readings of
our own.

The pages give the Q2_K, Q4_K, Q6_K, Q4_1, Q5_0 and Q5_1 formats (ggml "Q4_0
vec_dot Walkthrough" section 1.2 for Q2_K's fields; minfer's block sizes; the
d*q + m form of the _1 formats in ggml section 1.1) but print no quantizer for
them; the only printed quantizer fact is Q4_0's signed maximum (kvad "The
scale that wasted a code"), pinned elsewhere.  The rules the oracle follows
are stated in its source.  Here each rule is pinned by blocks whose every
intermediate (lo, hi, s, mn, d, dmin, sc, m, q) was worked out by hand from
that statement: the inputs are multiples of a power of two, so each
operation is exact or far from a rounding boundary, except where a boundary
is the point of the case (ties, and cases where f16(d) differs from d).

The expected values are literals in this file, each group with its working.
`test_mutants_fail_a_pin` compiles altered copies of the oracle (on the CPU)
and checks that each plausible mistake -- dividing by the unrounded d,
clamping one code short, truncating instead of rounding half to even,
swapping the scale and min fields, taking the last index on magnitude ties
-- fails at least one of these blocks.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

from conftest import ROOT

ORACLE_SRC = os.path.join(ROOT, "oracle", "qmm_oracle.c")
T = 2.0 ** -6      # dyadic step of the exact cases
U = 2.0 ** -10


def f32(v):
    return np.float32(v)


def u16(b, off):
    return int(b[off]) | (int(b[off + 1]) << 8)


# ---------------------------------------------------------------------------
# field readers (the byte layouts are readings pinned by the decode tests)
# ---------------------------------------------------------------------------
def q2k_fields(b):
    sc = [int(b[g]) & 15 for g in range(16)]
    m = [int(b[g]) >> 4 for g in range(16)]
    q = [(int(b[16 + 32 * (i // 128) + i % 32]) >> (2 * ((i % 128) // 32))) & 3 for i in range(256)]
    return u16(b, 80), u16(b, 82), sc, m, q


def q4k_fields(b):
    s12 = [int(v) for v in b[4:16]]
    sc, m = [], []
    for s in range(8):
        if s < 4:
            sc.append(s12[s] & 63)
            m.append(s12[s + 4] & 63)
        else:
            sc.append((s12[s + 4] & 15) | ((s12[s - 4] >> 6) << 4))
            m.append((s12[s + 4] >> 4) | ((s12[s] >> 6) << 4))
    q = []
    for i in range(256):
        byte = int(b[16 + 32 * (i // 64) + i % 32])
        q.append(byte >> 4 if (i % 64) >= 32 else byte & 15)
    return u16(b, 0), u16(b, 2), sc, m, q


def q6k_fields(b):
    sc = [int(np.int8(np.uint8(b[192 + g]))) for g in range(16)]
    q = []
    for i in range(256):
        h, k, l = i // 128, (i % 128) // 32, i % 32
        lb = int(b[64 * h + l + 32 * (k & 1)])
        lo = (lb & 15) if k < 2 else (lb >> 4)
        q.append(lo | (((int(b[128 + 32 * h + l]) >> (2 * k)) & 3) << 4))
    return u16(b, 208), sc, q


def q32_fields(fmt, b):
    """d bits, m bits (None for Q5_0) and the 32 codes of a Q4_1 / Q5_0 / Q5_1 block."""
    qs0 = {"q4_1": 4, "q5_0": 6, "q5_1": 8}[fmt]
    qh = 0
    if fmt != "q4_1":
        o = 2 if fmt == "q5_0" else 4
        qh = int(b[o]) | (int(b[o + 1]) << 8) | (int(b[o + 2]) << 16) | (int(b[o + 3]) << 24)
    codes = []
    for j in range(32):
        byte = int(b[qs0 + (j & 15)])
        lo = byte & 15 if j < 16 else byte >> 4
        codes.append(lo | (((qh >> j) & 1) << 4))
    return u16(b, 0), (None if fmt == "q5_0" else u16(b, 2)), codes


# ---------------------------------------------------------------------------
# the hand blocks
# ---------------------------------------------------------------------------
def q2k_block_a():
    """Sixteen groups of 16 (value j of a group, p = j % 4); T = 2^-6.
    Per group: lo = min(0, min x), hi = max x, s = (hi - lo)/3, mn = -lo.
    Group 2 has the largest s (15T) and group 3 the largest mn (15T), so
    d = 15T/15 = T and dmin = 15T/15 = T exactly (f16 0x2400 both)."""
    pat = [
        [0, 1, 2, 3],              # g0: lo 0, hi 3T, s T -> sc 1, m 0; q = x/T
        [-2, -1, 0, 1],            # g1: lo -2T, hi T, s T, mn 2T -> sc 1, m 2; q = (x+2T)/T
        [0, 15, 30, 45],           # g2: s 15T -> sc 15, m 0; q = x/15T
        [-15, -10, -5, 0],         # g3: s 5T, mn 15T -> sc 5, m 15; q = (x+15T)/5T
        [0.75, 1.75, 2.25, 2.75],  # g4: lo 0, s 2.75T/3 = 0.917T -> sc 1; q = rne(0.75, 1.75, 2.25, 2.75)
        [0, 2.5, 3, 1],            # g5: s T -> sc 1; 2.5 is a tie -> 2
        [-0.5, 0, 1.25, 2.5],      # g6: s 3T/3 = T, mn 0.5T -> m = rne(0.5) = 0 (tie); q = rne(-0.5, 0, 1.25, 2.5)
        [-1.5, 0, 1.5, 3],         # g7: s 4.5T/3 = 1.5T -> sc = rne(1.5) = 2, m = rne(1.5) = 2;
                                   #     q = rne((x+2T)/2T) = rne(0.25, 1, 1.75, 2.5)
        [0, 1.4, 2.8, 4.2],        # g8: s 1.4T -> sc 1; q = rne(0, 1.4, 2.8, 4.2) = 0, 1, 3, 4 -> clamp 3
        [-12, -13, -14, -15],      # g9: all negative: lo -15T, hi -12T, s T, mn 15T -> sc 1, m 15;
                                   #     q = (x+15T)/T (hi = 0 instead would give s 5T -> sc 5)
    ] + [[0, 0, 0, 0]] * 6         # g10..g15: zero groups -> sc 0, m 0, divisor 0 -> q 0
    x = np.zeros(256, dtype=np.float32)
    for g, p in enumerate(pat):
        for j in range(16):
            x[16 * g + j] = f32(p[j % 4]) * f32(T)
    sc = [1, 1, 15, 5, 1, 1, 1, 2, 1, 1] + [0] * 6
    m = [0, 2, 0, 15, 0, 0, 0, 2, 0, 15] + [0] * 6
    qp = [[0, 1, 2, 3], [0, 1, 2, 3], [0, 1, 2, 3], [0, 1, 2, 3], [1, 2, 2, 3], [0, 2, 3, 1], [0, 0, 1, 2],
          [0, 1, 2, 2], [0, 1, 3, 3], [3, 2, 1, 0]] + [[0, 0, 0, 0]] * 6
    q = [qp[i // 16][i % 4] for i in range(256)]
    return x, (0x2400, 0x2400, sc, m, q)


def q2k_block_b():
    """f16(d) and f16(dmin) differ from d and dmin.  b = 0.4999.
    g0 = 0, 1, 2, 3 (s = 1): d = 1/15, stored f16 0x2C44 = 0.066650390625
    (1/15 = 2^-4 * 1.0667; 0.0667 * 1024 = 68.27 -> 68); sc = rne(15.004) = 15.
    g1 = p * b: s = b, sc = rne(b / 0.066650390625) = rne(7.50033) = 8, where
    b / (1/15) = 7.4985 would give 7; q = rne(p * b / 0.533203125) =
    rne(0.93754 p) = p.
    g2 = -1 then zeros: lo = -1, hi = 0, s = 1/3, mn = 1 (the largest, so dmin
    = 1/15, f16 0x2C44 like d); sc = rne(5.0012) = 5, m = rne(15.004) = 15;
    q = rne((x + 15 * 0.066650390625) / (5 * 0.066650390625)):
    -1 -> rne(-0.0007) = 0, 0 -> 0.999755859375 / 0.333251953125 = 3 exactly.
    g3 = -b, 0.1, then zeros: s = 0.5999/3 = 0.19997 -> sc = rne(3.0002) = 3;
    mn = b -> m = rne(7.50033) = 8, where b / (1/15) would give 7;
    q = rne((x + 0.533203125) / 0.199951171875): -b -> rne(0.167) = 0,
    0.1 -> rne(3.167) = 3, 0 -> rne(2.667) = 3.
    The rest is zero."""
    x = np.zeros(256, dtype=np.float32)
    b = f32(0.4999)
    for j in range(16):
        x[j] = f32(j % 4)
        x[16 + j] = f32(j % 4) * b
    x[32] = f32(-1.0)
    x[48], x[49] = -b, f32(0.1)
    sc = [15, 8, 5, 3] + [0] * 12
    m = [0, 0, 15, 8] + [0] * 12
    q = [(i % 4) if i < 32 else 0 for i in range(256)]
    for i in range(33, 48):
        q[i] = 3
    for i in range(49, 64):
        q[i] = 3
    return x, (0x2C44, 0x2C44, sc, m, q)


def q4k_block_a():
    """Eight sub-blocks of 32 (value j, k = j % 16); T = 2^-6.
    s = (hi - lo)/15; sub-block 5 has the largest s (63T) and sub-block 6
    the largest mn (63T): d = dmin = 63T/63 = T (f16 0x2400)."""
    x = np.zeros(256, dtype=np.float32)
    q = [0] * 256
    for j in range(32):
        k = j % 16
        x[j] = f32(k) * f32(T)                      # s0: s = T -> sc 1, m 0, q = k
        q[j] = k
        x[32 + j] = f32(k - 3) * f32(T)             # s1: lo -3T, hi 12T, s T, mn 3T -> sc 1, m 3, q = k
        q[32 + j] = k
        x[64 + j] = f32((j % 15) + 0.75) * f32(T)   # s2: lo 0, hi 14.75T, s 0.983T -> sc 1; q = rne(v + 0.75) = v + 1
        q[64 + j] = (j % 15) + 1
        x[96 + j] = f32(k + 0.5) * f32(T)           # s3: hi 15.5T, s 1.033T -> sc 1; q = rne(k + 0.5): ties to even,
        q[96 + j] = min(15, k + (k & 1))            #     15.5 -> 16 -> clamp 15
        x[128 + j] = f32(k - 40) * f32(T)           # s4: lo -40T, hi -25T, s T, mn 40T -> sc 1, m 40 (high bits used)
        q[128 + j] = k
        x[160 + j] = f32(63 * k) * f32(T)           # s5: s 945T/15 = 63T -> sc 63, q = k
        q[160 + j] = k
        x[192 + j] = f32(k - 63) * f32(T)           # s6: lo -63T, mn 63T -> sc 1, m 63, q = k
        q[192 + j] = k
    # s7 zero -> sc 0, m 0, q 0
    return x, (0x2400, 0x2400, [1, 1, 1, 1, 1, 63, 1, 0], [0, 3, 0, 0, 40, 0, 63, 0], q)


def q4k_block_b():
    """f16(d) differs from d.  s0 = 0..15 (s = 1): d = 1/63, f16 0x2410 =
    0.015869140625 (1/63 = 2^-6 * 1.01587; 0.01587 * 1024 = 16.25 -> 16);
    sc0 = rne(63.015) = 63.  s1 = k * 0.4999: sc1 = rne(0.4999 / 0.015869140625)
    = rne(31.5014) = 32, where 0.4999 * 63 = 31.494 would give 31; q = rne(k *
    0.4999 / 0.5078125) = rne(0.98442 k) = k."""
    x = np.zeros(256, dtype=np.float32)
    b = f32(0.4999)
    q = [0] * 256
    for j in range(32):
        k = j % 16
        x[j] = f32(k)
        x[32 + j] = f32(k) * b
        q[j] = q[32 + j] = k
    return x, (0x2410, 0x0000, [63, 32, 0, 0, 0, 0, 0, 0], [0] * 8, q)


def q6k_block_a():
    """Sixteen groups of 16 (value j); U = 2^-10.  Per group the value of
    largest magnitude mx (first on ties) gives s = mx/-32; group 0 has the
    largest |s| (127U), so d = 127U/127 = U (f16 0x1400)."""
    x = np.zeros(256, dtype=np.float32)
    q = [32] * 256
    for j in range(16):
        x[j] = f32(254 * (j - 16)) * f32(U)     # g0: mx = -4064U, s = 127U -> sc 127; q = 2(j-16) + 32 = 2j
        q[j] = 2 * j
        x[16 + j] = f32(128 * (16 - j)) * f32(U)  # g1: mx = +2048U, s = -64U -> sc -64; q = -2(16-j) + 32 = 2j
        q[16 + j] = 2 * j
    # g2: mx = -128U, s = 4U -> sc 4; others 4U(j + 0.75): q = rne(j + 0.75) + 32 = j + 33
    # g3: as g2 with 4U(j + 0.5): ties to even
    x[32] = x[48] = f32(-128) * f32(U)
    q[32] = q[48] = 0
    for j in range(1, 16):
        x[32 + j] = f32(4 * (j + 0.75)) * f32(U)
        q[32 + j] = j + 33
        x[48 + j] = f32(4 * (j + 0.5)) * f32(U)
        q[48 + j] = (j + (j & 1)) + 32
    # g4: -128U then +128U: the first wins (s = 4U, sc 4), +128U -> rne(32) + 32 = 64 -> clamp 63
    x[64] = f32(-128) * f32(U)
    x[65] = f32(128) * f32(U)
    q[64], q[65] = 0, 63
    # g5..g15 zero: s = -0 -> sc 0 -> divisor 0 -> q 32
    return x, (0x1400, [127, -64, 4, 4, 4] + [0] * 11, q)


def q6k_block_b():
    """f16(d) differs from d.  g0 = -32 then zeros: s = 1, d = 1/127, f16
    0x2008 = 0.00787353515625 (1/127 = 2^-7 * 1.00787; 0.00787 * 1024 = 8.06
    -> 8); sc0 = rne(127.008) = 127.  g1 = -32 * 0.7913 then zeros: s = 0.7913,
    sc1 = rne(0.7913 / 0.00787353515625) = rne(100.5012) = 101, where
    0.7913 * 127 = 100.495 would give 100; q of the first value:
    rne(-25.3216 / (101 * 0.00787353515625)) + 32 = rne(-31.84) + 32 = 0."""
    x = np.zeros(256, dtype=np.float32)
    x[0] = f32(-32.0)
    x[16] = f32(-25.3216)
    q = [32] * 256
    q[0] = q[16] = 0
    return x, (0x2008, [127, 101] + [0] * 14, q)


def q32_blocks(fmt):
    """(x, expected) pairs of one 32-value format; T = 2^-6."""
    L = 15 if fmt == "q4_1" else 31
    out = []
    if fmt == "q5_0":
        # A: x_j = T (j - 16) for j < 31 and x_31 = +16T: -16T (j = 0) and +16T tie in magnitude and the
        #    first wins: d = -16T / -16 = T (f16 0x2400); q = rne(x/T) + 16 = j, and x_31: 32 -> clamp 31
        xa = np.array([f32(j - 16) * f32(T) for j in range(31)] + [f32(16) * f32(T)], dtype=np.float32)
        out.append((xa, (0x2400, None, list(range(32)))))
        # B: x_0 = -16T, then T (k + 0.75) for j = 1..15 (k = j - 1) -> q = k + 1 + 16 = j + 16,
        #    then T (k + 0.5) for j = 16 + k -> q = rne(k + 0.5) + 16 (15.5 -> 16 -> 32 -> clamp 31)
        xb = np.zeros(32, dtype=np.float32)
        qb = [0] * 32
        xb[0] = f32(-16) * f32(T)
        for j in range(1, 16):
            xb[j] = f32((j - 1) + 0.75) * f32(T)
            qb[j] = j + 16
        for k in range(16):
            xb[16 + k] = f32(k + 0.5) * f32(T)
            qb[16 + k] = min(31, k + (k & 1) + 16)
        out.append((xb, (0x2400, None, qb)))
        # C: codes from the f32 d: x_0 = -1.1 gives d = -1.1 / -16 = 0.06875 (f16 0x2C66 = 0.0687255859375,
        #    1.1: 0.1 * 1024 = 102.4 -> 102); x_1 = 0.5155: rne(0.5155 / 0.06875) = rne(7.498) = 7 -> 23,
        #    where the f16 d would give rne(7.5008) = 8 -> 24
        xc = np.zeros(32, dtype=np.float32)
        xc[0], xc[1] = f32(-1.1), f32(0.5155)
        out.append((xc, (0x2C66, None, [0, 23] + [16] * 30)))
        return out
    # Q4_1 / Q5_1: lo = min x, hi = max x, d = (hi - lo)/L, m = lo, q = rne((x - m)/d)
    # A: x_j = T ((j % 16) - 3) (Q4_1) or T (j - 3) (Q5_1): d = T (0x2400), m = -3T = -0.046875 (0xAA00)
    xa = np.array([f32((j % 16 if L == 15 else j) - 3) * f32(T) for j in range(32)], dtype=np.float32)
    out.append((xa, (0x2400, 0xAA00, [j % 16 if L == 15 else j for j in range(32)])))
    # B: x_0 = 0, x_1 = L T, T (k + 0.75) at j = 2 + k (k < 15), T (k + 0.5) at j = 17 + k (k < 15):
    #    d = T, m = 0; q = 0, L, k + 1, rne(k + 0.5) (ties to even)
    xb = np.zeros(32, dtype=np.float32)
    qb = [0] * 32
    xb[1] = f32(L) * f32(T)
    qb[1] = L
    for k in range(15):
        xb[2 + k] = f32(k + 0.75) * f32(T)
        qb[2 + k] = k + 1
        xb[17 + k] = f32(k + 0.5) * f32(T)
        qb[17 + k] = k + (k & 1)
    out.append((xb, (0x2400, 0x0000, qb)))
    # C: f16(d) differs from d.  x_0 = 0, x_1 = 1, one value v, rest 0: d = 1/L.
    #    Q4_1: f16(1/15) = 0x2C44 = 0.066650390625; v = 0.4999: rne(7.50033) = 8 (1/15 would give 7.4985 -> 7);
    #          x_1: rne(1 / 0.06665) = rne(15.004) = 15.
    #    Q5_1: f16(1/31) = 0x2821 = 0.032257080078125 (1/31 = 2^-5 * 1.03226; 0.03226 * 1024 = 33.03 -> 33);
    #          v = 0.49999: rne(15.50025) = 16 (1/31 would give 15.4997 -> 15); x_1: rne(31.0009) = 31.
    xc = np.zeros(32, dtype=np.float32)
    xc[1] = f32(1.0)
    xc[2] = f32(0.4999) if L == 15 else f32(0.49999)
    out.append((xc, (0x2C44 if L == 15 else 0x2821, 0x0000, [0, L, 8 if L == 15 else 16] + [0] * 29)))
    return out


# ---------------------------------------------------------------------------
# checks against any library exporting the oracle's quantizers
# ---------------------------------------------------------------------------
BYTES = {"q2_k": 84, "q4_k": 144, "q6_k": 210, "q4_1": 20, "q5_0": 22, "q5_1": 24}
VALUES = {"q2_k": 256, "q4_k": 256, "q6_k": 256, "q4_1": 32, "q5_0": 32, "q5_1": 32}


def quantize_with(L, fmt, x):
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(1, -1)
    out = np.zeros(BYTES[fmt] * (x.shape[1] // VALUES[fmt]), dtype=np.uint8)
    fn = getattr(L, f"orc_quantize_{fmt}_w")
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64]
    fn.restype = None
    fn(x.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p), 1, x.shape[1])
    return out


def failures(L, fmt):
    """Names of the hand blocks of `fmt` whose quantized fields differ."""
    bad = []
    if fmt == "q2_k":
        cases = [("A", *q2k_block_a()), ("B", *q2k_block_b())]
        for name, x, want in cases:
            got = q2k_fields(quantize_with(L, fmt, x))
            if tuple(got) != want:
                bad.append(name)
    elif fmt == "q4_k":
        for name, x, want in [("A", *q4k_block_a()), ("B", *q4k_block_b())]:
            if tuple(q4k_fields(quantize_with(L, fmt, x))) != want:
                bad.append(name)
    elif fmt == "q6_k":
        for name, x, want in [("A", *q6k_block_a()), ("B", *q6k_block_b())]:
            if tuple(q6k_fields(quantize_with(L, fmt, x))) != want:
                bad.append(name)
    else:
        for name, (x, want) in zip("ABC", q32_blocks(fmt)):
            if tuple(q32_fields(fmt, quantize_with(L, fmt, x))) != want:
                bad.append(name)
    return bad


FORMATS = ["q2_k", "q4_k", "q6_k", "q4_1", "q5_0", "q5_1"]


@pytest.mark.parametrize("fmt", FORMATS)
def test_hand_blocks(orc, fmt):
    L = orc.lib()
    assert failures(L, fmt) == []


@pytest.mark.parametrize("fmt", FORMATS)
def test_hand_block_fields_in_detail(orc, fmt):
    """The same blocks field by field, so that a failure names the field."""
    L = orc.lib()
    if fmt == "q2_k":
        for x, (d, dmin, sc, m, q) in (q2k_block_a(), q2k_block_b()):
            gd, gdmin, gsc, gm, gq = q2k_fields(quantize_with(L, fmt, x))
            assert (gd, gdmin) == (d, dmin)
            assert gsc == sc and gm == m
            assert gq == q
    elif fmt == "q4_k":
        for x, (d, dmin, sc, m, q) in (q4k_block_a(), q4k_block_b()):
            gd, gdmin, gsc, gm, gq = q4k_fields(quantize_with(L, fmt, x))
            assert (gd, gdmin) == (d, dmin)
            assert gsc == sc and gm == m
            assert gq == q
    elif fmt == "q6_k":
        for x, (d, sc, q) in (q6k_block_a(), q6k_block_b()):
            gd, gsc, gq = q6k_fields(quantize_with(L, fmt, x))
            assert gd == d and gsc == sc
            assert gq == q
    else:
        for x, (d, m, codes) in q32_blocks(fmt):
            gd, gm, gcodes = q32_fields(fmt, quantize_with(L, fmt, x))
            assert (gd, gm) == (d, m)
            assert gcodes == codes


# ---------------------------------------------------------------------------
# mutants: each plausible mistake in a rule must fail at least one hand block
# ---------------------------------------------------------------------------
def _body(src, signature):
    """(start, end) of the body of the function whose definition starts with `signature`."""
    s = src.index(signature)
    return s, src.index("\n}\n", s) + 3


def _in_function(signature, old, new, count=None):
    def apply(src):
        s, e = _body(src, signature)
        body = src[s:e]
        n = body.count(old)
        assert n >= 1 and (count is None or n == count), (signature, old, n)
        return src[:s] + body.replace(old, new) + src[e:]
    return apply


Q2K = "void orc_quantize_q2_k_w("
Q4K = "void orc_quantize_q4_k_w("
Q6K = "void orc_quantize_q6_k_w("
B32 = "static void quant_block32("

MUTANTS = {
    # Q2_K
    "q2_k unrounded d": ("q2_k", _in_function(Q2K, "rne(s[g] / dh)", "rne(s[g] / d)", 1)),
    "q2_k unrounded dmin": ("q2_k", _in_function(Q2K, "rne(mn[g] / dminh)", "rne(mn[g] / dmin)", 1)),
    "q2_k clamp 0..2": ("q2_k", _in_function(Q2K, "(c > 3 ? 3 : c)", "(c > 2 ? 2 : c)", 1)),
    "q2_k trunc": ("q2_k", _in_function(Q2K, "rne(", "truncf(")),
    "q2_k sc/m nibble swap": ("q2_k", _in_function(Q2K, "(sc[g] | (mm[g] << 4))", "(mm[g] | (sc[g] << 4))", 1)),
    "q2_k hi = max(0, x)": ("q2_k", _in_function(Q2K, "float lo = 0.0f, hi = xb[16 * g];",
                                                 "float lo = 0.0f, hi = 0.0f;", 1)),
    # Q4_K
    "q4_k unrounded d": ("q4_k", _in_function(Q4K, "rne(sv[t] / dh)", "rne(sv[t] / (smax / 63.0f))", 1)),
    "q4_k clamp 0..14": ("q4_k", _in_function(Q4K, "(c > 15 ? 15 : c)", "(c > 14 ? 14 : c)", 1)),
    "q4_k trunc": ("q4_k", _in_function(Q4K, "rne(", "truncf(")),
    "q4_k sc/m swap": ("q4_k", _in_function(Q4K, "q4k_pack_scale_min(ob + 4, sc, mm)",
                                            "q4k_pack_scale_min(ob + 4, mm, sc)", 1)),
    # Q6_K
    "q6_k unrounded d": ("q6_k", _in_function(Q6K, "rne(sv[g] / dh)", "rne(sv[g] / (smax / 127.0f))", 1)),
    "q6_k clamp 0..62": ("q6_k", _in_function(Q6K, "(c > 63 ? 63 : c)", "(c > 62 ? 62 : c)", 1)),
    "q6_k trunc": ("q6_k", _in_function(Q6K, "rne(", "truncf(")),
    "q6_k last index on ties": ("q6_k", _in_function(Q6K, "if (a > amax)", "if (a >= amax)", 1)),
    # Q4_1 / Q5_1 (shared rule)
    "q4_1 unrounded d": ("q4_1", _in_function(B32, "rne((xb[j] - mh) / dh)", "rne((xb[j] - mh) / ((hi - lo) / (float)L))", 1)),
    "q5_1 unrounded d": ("q5_1", _in_function(B32, "rne((xb[j] - mh) / dh)", "rne((xb[j] - mh) / ((hi - lo) / (float)L))", 1)),
    "q4_1 clamp 0..L-1": ("q4_1", _in_function(B32, "(c > L ? L : c)", "(c > L - 1 ? L - 1 : c)", 1)),
    "q5_1 clamp 0..L-1": ("q5_1", _in_function(B32, "(c > L ? L : c)", "(c > L - 1 ? L - 1 : c)", 1)),
    "q4_1 trunc": ("q4_1", _in_function(B32, "rne(", "truncf(")),
    "q5_1 trunc": ("q5_1", _in_function(B32, "rne(", "truncf(")),
    "q4_1 d/m swap": ("q4_1", _in_function(B32, "wr_f16(ob, (hi - lo) / (float)L);\n        wr_f16(ob + 2, lo);",
                                           "wr_f16(ob, lo);\n        wr_f16(ob + 2, (hi - lo) / (float)L);", 1)),
    "q5_1 d/m swap": ("q5_1", _in_function(B32, "wr_f16(ob, (hi - lo) / (float)L);\n        wr_f16(ob + 2, lo);",
                                           "wr_f16(ob, lo);\n        wr_f16(ob + 2, (hi - lo) / (float)L);", 1)),
    # Q5_0
    "q5_0 codes from f16 d": ("q5_0", _in_function(B32, "rne(xb[j] / d) + 16", "rne(xb[j] / rd_f16(ob)) + 16", 1)),
    "q5_0 clamp 0..30": ("q5_0", _in_function(B32, "(c > 31 ? 31 : c)", "(c > 30 ? 30 : c)", 1)),
    "q5_0 trunc": ("q5_0", _in_function(B32, "rne(", "truncf(")),
    "q5_0 last index on ties": ("q5_0", _in_function(B32, "if (a > amax)", "if (a >= amax)", 1)),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutants_fail_a_pin(tmp_path, name):
    fmt, mutate = MUTANTS[name]
    src = open(ORACLE_SRC).read()
    msrc = mutate(src)
    assert msrc != src
    cfile = tmp_path / "mutant.c"
    cfile.write_text(msrc)
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
                           "-o", str(so), str(cfile), "-lm"], timeout=120)
    L = ctypes.CDLL(str(so))
    assert failures(L, fmt) != [], f"mutant '{name}' passes every hand block of {fmt}"
