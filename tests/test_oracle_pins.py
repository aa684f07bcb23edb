"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden, cited there), closed forms and invariants of the
method, special cases that reduce to a library routine (numpy's binary16
conversion, numpy's float64 matrix product on exactly decoded values), and
brute force on tiny inputs.  A plausible mistake anywhere in the oracle (a
dropped term, a wrong sign, a swapped nibble, a transposed output) fails at
least one of them.
"""
import numpy as np
import pytest

import synth
from conftest import golden


# ---------------------------------------------------------------------------
# binary16 conversion: library routine (numpy.float16), exhaustive decode
# ---------------------------------------------------------------------------
def test_f16_decode_exhaustive_matches_numpy(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = orc.f16_to_f32_array(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _f16_encode_cases():
    finite = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = finite.view(np.float16).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2.0).astype(np.float32)        # exact ties
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    top = np.array([65504, 65519.996, 65520, 65536, 1e30, 2.0 ** -25, 2.0 ** -24, 2.0 ** -26,
                    3 * 2.0 ** -26, 0.0], dtype=np.float32)
    rng = synth.splitmix64(0x12345, 0, 10_000_000)
    rnd = (rng & np.uint64(0x7FFFFFFF)).astype(np.uint32)
    rnd = rnd[rnd < 0x7F800000].view(np.float32)
    base = np.concatenate([vals.astype(np.float32), mids, up, dn, top, rnd])
    return np.concatenate([base, -base])


def test_f16_encode_matches_numpy(orc):
    x = _f16_encode_cases()
    assert x.size > 10_000_000
    ours = orc.f32_to_f16_array(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(ours[i]), hex(ref[i])) for i in bad[:5]]


# ---------------------------------------------------------------------------
# Q8_0 activation quantizer
# ---------------------------------------------------------------------------
def _q8_0_fields(q):
    q = q.reshape(-1, 34)
    d = q[:, :2].copy().view(np.uint16).ravel()
    codes = q[:, 2:].view(np.int8)
    return d, codes


def _mixed_activations(rows, K, seed):
    x = synth.gaussian_f32((rows, K), 1.0, seed)
    x = synth.with_outliers(x, 0.01, 20.0, seed + 1)
    x[0, :32] = 0.0                       # a zero block
    x[0, 32:64] = 0.0
    x[0, 40] = -3.25                      # a block with one nonzero value
    x[1, 64:96] *= 1e-30                  # tiny but normal values (amax >= 127 * FLT_MIN)
    x[1, 96:128] *= 1e4
    return x


def test_q8_0_invariants_and_special_cases(orc):
    x = _mixed_activations(8, 1024, 11)
    q = orc.quantize_q8_0(x)
    assert q.shape == (8, 1024 // 32 * 34)
    d, codes = _q8_0_fields(q)
    xb = x.reshape(-1, 32)
    amax = np.abs(xb).max(axis=1)
    # codes within [-127, 127]; the element of largest magnitude maps to +-127
    assert codes.min() >= -127 and codes.max() <= 127
    nz = amax > 0
    arg = np.abs(xb).argmax(axis=1)
    top = codes[np.arange(codes.shape[0]), arg]
    assert np.all(np.abs(top[nz]) == 127)
    assert np.all(np.sign(top[nz]) == np.sign(xb[np.arange(xb.shape[0]), arg][nz]))
    # zero block -> d = 0 and every code 0 (the zero-block guard)
    assert d[0] == 0 and np.all(codes[0] == 0)
    # one nonzero value -> d = f16(|v| / 127), code -127 at it and 0 elsewhere
    assert codes[1, 40 - 32] == -127 and np.count_nonzero(codes[1]) == 1
    assert d[1] == np.float16(np.float32(3.25) / np.float32(127)).view(np.uint16)
    # stored scale is the binary16 of the f32 quotient amax / 127
    ref_d = (amax.astype(np.float32) / np.float32(127)).astype(np.float16).view(np.uint16)
    assert np.array_equal(d, ref_d)


def test_q8_0_ties_to_even(orc):
    # amax = 127 gives an inverse scale of exactly 1, so x * id = x and the
    # rounding rule alone decides the code (_MM_ROUND_NEAREST: ties to even).
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :8] = [127.0, 2.5, 3.5, -0.5, -1.5, 126.5, 0.49999997, -2.5]
    q = orc.quantize_q8_0(x)
    _, codes = _q8_0_fields(q)
    assert list(codes[0, :8]) == [127, 2, 4, 0, -2, 126, 0, -2]


def test_q8_0_reconstruction_bound(orc):
    # |x - q * f16(d)| <= 0.5 d (1 + 1e-4) + 127 |f16(d) - d|: half a scale
    # step ("The error is bounded by half a scale step per value") plus the
    # storage rounding of d; the 1e-4 covers the two f32 roundings of id.
    x = _mixed_activations(16, 4096, 21)
    q = orc.quantize_q8_0(x)
    dbits, codes = _q8_0_fields(q)
    dh = dbits.view(np.float16).astype(np.float64)
    xb = x.reshape(-1, 32).astype(np.float64)
    d = np.abs(xb).max(axis=1) / 127.0
    err = np.abs(xb - codes * dh[:, None]).max(axis=1)
    bound = 0.5 * d * (1 + 1e-4) + 127 * np.abs(dh - d)
    assert np.all(err <= bound)


def test_q8_0_matches_float32_restatement(orc):
    """Algebra check (not a pin of the reading): numpy float32 arithmetic in
    the same order gives the same bytes."""
    x = _mixed_activations(4, 2048, 31)
    q = orc.quantize_q8_0(x)
    xb = x.reshape(-1, 32)
    amax = np.abs(xb).max(axis=1)
    with np.errstate(divide="ignore"):
        idv = np.where(amax != 0, np.float32(127) / amax, np.float32(0)).astype(np.float32)
    codes = np.rint(xb * idv[:, None]).astype(np.int8)
    d = (amax / np.float32(127)).astype(np.float16)
    ref = np.concatenate([d.view(np.uint8).reshape(-1, 2), codes.view(np.uint8)], axis=1)
    assert np.array_equal(q.reshape(-1, 34), ref)


# ---------------------------------------------------------------------------
# Q8_K activation quantizer
# ---------------------------------------------------------------------------
def _q8_k_fields(q):
    q = q.reshape(-1, 292)
    d = q[:, :4].copy().view(np.float32).ravel()
    codes = q[:, 4:260].view(np.int8)
    bsums = q[:, 260:292].copy().view(np.int16)
    return d, codes, bsums


def test_q8_k_invariants(orc):
    x = _mixed_activations(6, 1024, 41)
    x[2, 256:512] = 0.0
    q = orc.quantize_q8_k(x)
    assert q.shape == (6, 4 * 292)
    d, codes, bsums = _q8_k_fields(q)
    xb = x.reshape(-1, 256)
    amax = np.abs(xb).max(axis=1)
    assert np.array_equal(d, amax / np.float32(127))                  # f32 d
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.array_equal(bsums, codes.reshape(-1, 16, 16).astype(np.int32).sum(axis=2))
    zero = 2 * 4 + 1
    assert d[zero] == 0 and not codes[zero].any() and not bsums[zero].any()
    # an all-positive ramp: code i equals round(i * 127 / 255), checkable by hand
    ramp = np.arange(256, dtype=np.float32)[None, :]
    _, c, _ = _q8_k_fields(orc.quantize_q8_k(ramp))
    assert c[0, 255] == 127 and c[0, 0] == 0 and c[0, 1] == 0 and c[0, 2] == 1


# ---------------------------------------------------------------------------
# Q4_0 weight quantizer and decoder
# ---------------------------------------------------------------------------
def _q4_0_fields(q):
    q = q.reshape(-1, 18)
    d = q[:, :2].copy().view(np.uint16).ravel()
    qs = q[:, 2:]
    codes = np.concatenate([qs & 0x0F, qs >> 4], axis=1)   # elements 0..15, 16..31
    return d, codes


def test_worked_byte_0x21(orc):
    g = golden("worked_byte.json")
    blk = np.full(18, 0x88, dtype=np.uint8)
    blk[:2] = np.array([orc.f32_to_f16_bits(g["scale_w"])], dtype=np.uint16).view(np.uint8)
    blk[2] = g["byte"]
    vals = orc.dequantize("q4_0", blk, 32)[0]
    assert vals[0] == g["element_j"] and vals[16] == g["element_j_plus_16"]
    assert np.all(np.delete(vals, [0, 16]) == 0)
    # the same two values through the integer block dot: activation codes
    # 1 at element 0 and 10 at element 16 give -7 + 10 * (-6)
    xb = np.zeros(34, dtype=np.uint8)
    xb[2 + 0] = 1
    xb[2 + 16] = 10
    assert orc.block_isum("q4_0", blk, xb) == g["element_j"] + 10 * g["element_j_plus_16"]


def test_block_sizes(orc):
    g = golden("block_sizes.json")
    assert orc.BLOCK_BYTES["q4_0"] == g["q4_0_bytes"]
    assert orc.BLOCK_BYTES["q8_0"] == g["q8_0_bytes"]
    assert orc.BLOCK_BYTES["q2_k"] == g["q2_k_bytes"]
    assert orc.BLOCK_BYTES["q4_k"] == g["q4_k_bytes"]
    assert orc.BLOCK_BYTES["q6_k"] == g["q6_k_bytes"]
    assert orc.BLOCK_BYTES["q5_0"] == g["q5_0_bytes"]
    assert orc.BLOCK_BYTES["q5_1"] == g["q5_1_bytes"]
    w = synth.gaussian_f32((2, 512), 0.02, 6)
    assert orc.quantize_q5_0_w(w).shape == (2, 16 * g["q5_0_bytes"])
    assert orc.quantize_q5_1_w(w).shape == (2, 16 * g["q5_1_bytes"])
    assert orc.quantize_q4_k_w(w).shape == (2, 2 * g["q4_k_bytes"])
    assert orc.quantize_q6_k_w(w).shape == (2, 2 * g["q6_k_bytes"])
    assert orc.BLOCK_BYTES["q4_0"] / 32 == g["q4_0_bytes_per_weight"]
    assert orc.BLOCK_BYTES["q2_k"] * 8 / 256 == g["q2_k_bits_per_weight"]
    ex = g["row_example"]
    assert ex["K"] // 32 == ex["blocks"]
    assert orc.row_bytes("q4_0", ex["K"]) == ex["q4_0_row_bytes"]
    w = synth.gaussian_f32((3, ex["K"]), 0.02, 5)
    assert orc.quantize_q4_0_w(w).shape == (3, ex["q4_0_row_bytes"])


def test_q4_0_max_magnitude_element_is_code_0(orc):
    w = synth.gaussian_f32((64, 1024), 0.02, 51)
    w[0, :32] = 0.0                                   # zero block
    w[1, :32] = 0.01
    w[1, 3] = -0.5                                    # magnitude tie: first index wins
    w[1, 10] = 0.5
    q = orc.quantize_q4_0_w(w)
    d, codes = _q4_0_fields(q)
    assert codes.min() >= 0 and codes.max() <= 15
    vals = orc.dequantize("q4_0", q, 1024).reshape(-1, 32)
    wb = w.reshape(-1, 32)
    dh = d.view(np.float16).astype(np.float64)
    first = np.argmax(np.abs(wb), axis=1)            # numpy: first index on ties
    nz = np.abs(wb).max(axis=1) > 0
    rows = np.arange(wb.shape[0])
    assert np.all(codes[rows, first][nz] == 0)
    assert np.all(vals[rows, first][nz] == -8.0 * dh[nz])
    # zero block: d = 0 and every code 8
    assert d[0] == 0 and np.all(codes[0] == 8)
    # tie block: index 3 takes code 0, the opposite extreme clips to code 15 (7/8 of its value)
    b = 32
    assert codes[b, 3] == 0 and codes[b, 10] == 15
    assert vals[b, 10] == 7 * dh[b]


def test_q4_0_mean_relative_error_matches_page(orc):
    g = golden("q4_quantizer_error.json")
    x = synth.gaussian_f32((4096, 32 * 64), 1.0, 61).reshape(-1, 32)
    q = orc.quantize_q4_0_w(x)
    xh = orc.dequantize("q4_0", q, 32).reshape(-1, 32)
    rel = np.linalg.norm(x - xh, axis=1) / np.linalg.norm(x.astype(np.float64), axis=1)
    pct = 100.0 * rel.mean()
    assert round(pct, g["printed_digits"]) == g["mean_relative_error_signed_over_minus_8_percent"], pct


# ---------------------------------------------------------------------------
# Q2_K decoder (closed forms) and the qs bit-order reading
# ---------------------------------------------------------------------------
def _q2k_block(d, dmin, scales, qs):
    blk = np.zeros(84, dtype=np.uint8)
    blk[:16] = scales
    blk[16:80] = qs
    blk[80:82] = np.array([np.float16(d)], dtype=np.float16).view(np.uint8)
    blk[82:84] = np.array([np.float16(dmin)], dtype=np.float16).view(np.uint8)
    return blk


def test_q2_k_decode_closed_forms(orc):
    rng = synth.splitmix64(71, 0, 80)
    qs = (rng[:64] & np.uint64(0xFF)).astype(np.uint8)
    scales = (rng[64:80] & np.uint64(0xFF)).astype(np.uint8)
    scales[0] = 15 | (0 << 4)        # sc = 15, m = 0  -> 15 * d * q
    scales[1] = 0 | (7 << 4)         # sc = 0,  m = 7  -> -dmin * 7
    blk = _q2k_block(0.5, 0.25, scales, qs)
    vals = orc.dequantize("q2_k", blk, 256)[0]
    # group 0 = weights 0..15: byte l (h = 0), shift 0
    q0 = qs[:16] & 3
    assert np.array_equal(vals[:16], 15 * 0.5 * q0)
    assert np.all(vals[16:32] == -0.25 * 7)
    # general form d * sc * q - dmin * m for every weight
    sc = scales & 0x0F
    m = scales >> 4
    for i in range(256):
        h, s, l = i // 128, (i % 128) // 32, i % 32
        q = (int(qs[32 * h + l]) >> (2 * s)) & 3
        g = i // 16
        assert vals[i] == 0.5 * sc[g] * q - 0.25 * m[g]


@pytest.mark.parametrize("h,s,l", [(0, 0, 0), (0, 3, 31), (1, 1, 5), (1, 2, 16)])
def test_q2_k_bit_order_reading(orc, h, s, l):
    scales = np.full(16, 1, dtype=np.uint8)         # sc = 1, m = 0
    qs = np.zeros(64, dtype=np.uint8)
    qs[32 * h + l] = 3 << (2 * s)
    vals = orc.dequantize("q2_k", _q2k_block(1.0, 0.0, scales, qs), 256)[0]
    nz = np.nonzero(vals)[0]
    assert list(nz) == [128 * h + 32 * s + l] and vals[nz[0]] == 3.0


def test_q2_k_quantizer_format_invariants(orc):
    """The Q2_K weight quantizer's rule is not on the pages (parity unpinned);
    only the format it must fill and a sanity bound are checked."""
    w = synth.gaussian_f32((8, 1024), 0.02, 81)
    q = orc.quantize_q2_k_w(w)
    assert q.shape == (8, 4 * 84)
    vals = orc.dequantize("q2_k", q, 1024)
    err = np.linalg.norm(vals - w) / np.linalg.norm(w)
    assert err < 0.6
    corr = np.corrcoef(vals.ravel(), w.ravel())[0, 1]
    assert corr > 0.8


# ---------------------------------------------------------------------------
# Q4_K: the chunk order and the two-term dot are the pages' (minfer "The
# payoff: a K-quant dot kernel, walked"); the 12-byte packing of the 6-bit
# scales and mins is a reading (GGUF's), checked here only for consistency.
# ---------------------------------------------------------------------------
def _q4k_block(d, dmin, sc, m, qs):
    """A Q4_K block from 8 scales, 8 mins (6 bits each) and 128 nibble bytes,
    the scales packed as the reading says (s < 4: low 6 bits of bytes s and
    s + 4; s >= 4: low / high nibble of byte s + 4 and the top 2 bits of bytes
    s - 4 and s)."""
    blk = np.zeros(144, dtype=np.uint8)
    blk[0:2] = np.array([np.float16(d)], dtype=np.float16).view(np.uint8)
    blk[2:4] = np.array([np.float16(dmin)], dtype=np.float16).view(np.uint8)
    b = np.zeros(12, dtype=np.int64)
    for s in range(4):
        b[s] = sc[s] | (sc[s + 4] >> 4) << 6
        b[s + 4] = m[s] | (m[s + 4] >> 4) << 6
        b[s + 8] = (sc[s + 4] & 15) | (m[s + 4] & 15) << 4
    blk[4:16] = b.astype(np.uint8)
    blk[16:144] = qs
    return blk


@pytest.mark.parametrize("j,l,hi", [(0, 0, 0), (0, 31, 1), (1, 7, 0), (2, 16, 1), (3, 31, 0), (3, 0, 1)])
def test_q4_k_chunk_order_is_the_pages(orc, j, l, hi):
    """Byte l of 32-byte chunk j: its low nibble is value 64j + l, its high
    nibble value 64j + 32 + l (the kernel's q8 offsets q8off + l and
    q8off + 32 + l)."""
    qs = np.zeros(128, dtype=np.uint8)
    qs[32 * j + l] = (5 << 4) if hi else 5
    vals = orc.dequantize("q4_k", _q4k_block(1.0, 0.0, [1] * 8, [0] * 8, qs), 256)[0]
    nz = np.nonzero(vals)[0]
    assert list(nz) == [64 * j + 32 * hi + l] and vals[nz[0]] == 5.0


def test_q4_k_decode_closed_form_and_scale_packing(orc):
    """value = d * sc_s * q - dmin * m_s with s = i / 32, for scales and mins
    that use all six bits (so every packed bit is exercised)."""
    rng = synth.splitmix64(131, 0, 160)
    sc = [int(v) for v in (rng[:8] % np.uint64(64))]
    m = [int(v) for v in (rng[8:16] % np.uint64(64))]
    sc[4], m[7] = 63, 63
    qs = (rng[16:144] & np.uint64(0xFF)).astype(np.uint8)
    vals = orc.dequantize("q4_k", _q4k_block(0.5, 0.25, sc, m, qs), 256)[0]
    for i in range(256):
        j, hi, l = i // 64, (i % 64) // 32, i % 32
        q = (int(qs[32 * j + l]) >> 4) if hi else (int(qs[32 * j + l]) & 15)
        assert vals[i] == 0.5 * sc[i // 32] * q - 0.25 * m[i // 32], i


def test_q4_k_min_term_pairs_two_bsum_groups(orc):
    """All codes zero: the product is the min term alone, -dmin * d8 *
    sum_s m_s * (bsums[2s] + bsums[2s+1]), which equals -dmin * sum over each
    sub-block of its decoded activations."""
    m = [1, 2, 3, 4, 5, 6, 7, 8]
    wq = _q4k_block(0.0, 0.5, [0] * 8, m, np.zeros(128, dtype=np.uint8))
    x = synth.gaussian_f32((1, 256), 1.0, 141)
    xq = orc.quantize_q8_k(x)
    X = orc.dequantize("q8_k", xq, 256)[0]
    y = orc.matmul("q4_k", wq, xq, 1, 1, 256, want=("y64",))["y64"][0, 0]
    expect = -0.5 * sum(m[s] * X[32 * s:32 * s + 32].sum() for s in range(8))
    assert abs(y - expect) <= 1e-12 * np.abs(X).sum() * 8


def test_q4_k_quantizer_format_invariants(orc):
    """The Q4_K weight quantizer's rule is not on the pages (parity unpinned)."""
    w = synth.gaussian_f32((8, 1024), 0.02, 151)
    q = orc.quantize_q4_k_w(w)
    vals = orc.dequantize("q4_k", q, 1024)
    assert np.linalg.norm(vals - w) / np.linalg.norm(w) < 0.12
    assert np.corrcoef(vals.ravel(), w.ravel())[0, 1] > 0.99
    d = q.reshape(-1, 144)[:, 0:2].copy().view(np.float16).astype(np.float64)
    assert np.all(d >= 0)


# ---------------------------------------------------------------------------
# Q6_K: the pages give the block size only; the layout is a reading (GGUF's).
# ---------------------------------------------------------------------------
def _q6k_block(d, scales, ql, qh):
    blk = np.zeros(210, dtype=np.uint8)
    blk[0:128] = ql
    blk[128:192] = qh
    blk[192:208] = np.asarray(scales, dtype=np.int8).view(np.uint8)
    blk[208:210] = np.array([np.float16(d)], dtype=np.float16).view(np.uint8)
    return blk


@pytest.mark.parametrize("i", [0, 17, 40, 70, 100, 127, 128, 161, 200, 255])
def test_q6_k_layout_reading(orc, i):
    """Value i's six bits: low four in ql[64h + l + 32 (k & 1)] (low nibble for
    k < 2, high for k >= 2), high two at bit 2k of qh[32h + l], with h = i / 128,
    k = (i % 128) / 32, l = i % 32; the code 32 decodes to zero."""
    h, k, l = i // 128, (i % 128) // 32, i % 32
    ql = np.zeros(128, dtype=np.uint8)
    qh = np.zeros(64, dtype=np.uint8)
    # every value at code 32 (= 0 after the offset) except value i at code 45
    for v in range(256):
        hv, kv, lv = v // 128, (v % 128) // 32, v % 32
        c = 45 if v == i else 32
        ql[64 * hv + lv + 32 * (kv & 1)] |= (c & 15) << (4 if kv >= 2 else 0)
        qh[32 * hv + lv] |= (c >> 4) << (2 * kv)
    vals = orc.dequantize("q6_k", _q6k_block(1.0, [1] * 16, ql, qh), 256)[0]
    nz = np.nonzero(vals)[0]
    assert list(nz) == [i] and vals[i] == 13.0


def test_q6_k_decode_closed_form(orc):
    """value = d * sc_g * (q - 32), g = i / 16, signed int8 scales."""
    rng = synth.splitmix64(161, 0, 208)
    ql = (rng[:128] & np.uint64(0xFF)).astype(np.uint8)
    qh = (rng[128:192] & np.uint64(0xFF)).astype(np.uint8)
    sc = ((rng[192:208] % np.uint64(256)).astype(np.int64) - 128).astype(np.int8)
    vals = orc.dequantize("q6_k", _q6k_block(0.25, sc, ql, qh), 256)[0]
    for i in range(256):
        h, k, l = i // 128, (i % 128) // 32, i % 32
        lb = int(ql[64 * h + l + 32 * (k & 1)])
        q = ((lb & 15) if k < 2 else (lb >> 4)) | (((int(qh[32 * h + l]) >> (2 * k)) & 3) << 4)
        assert vals[i] == 0.25 * int(sc[i // 16]) * (q - 32), i


def test_q6_k_quantizer_format_invariants(orc):
    """The Q6_K weight quantizer's rule is not on the pages (parity unpinned)."""
    w = synth.gaussian_f32((8, 1024), 0.02, 171)
    q = orc.quantize_q6_k_w(w)
    vals = orc.dequantize("q6_k", q, 1024)
    assert np.linalg.norm(vals - w) / np.linalg.norm(w) < 0.03
    # a group's largest magnitude lands near code 0 (value -32 * d * sc)
    wg = w.reshape(-1, 16)
    vg = vals.reshape(-1, 16)
    first = np.argmax(np.abs(wg), axis=1)
    rows = np.arange(wg.shape[0])
    assert np.all(np.abs(vg[rows, first] - wg[rows, first]) <= 0.05 * np.abs(wg[rows, first]))


# ---------------------------------------------------------------------------
# Q4_1 / Q5_0 / Q5_1: the _1 formats decode as d*q + m (ggml section 1.1), the
# Q5 formats carry a fifth bit per value (minfer: high-bit planes); field and
# bit order are readings (GGUF's), checked for consistency.
# ---------------------------------------------------------------------------
def _blk32(fmt, d, m, codes):
    """A block of `fmt` from f16 d, f16 m (ignored by Q5_0) and 32 codes, laid
    out as the reading says."""
    nbytes = {"q4_1": 20, "q5_0": 22, "q5_1": 24}[fmt]
    blk = np.zeros(nbytes, dtype=np.uint8)
    blk[0:2] = np.array([np.float16(d)], dtype=np.float16).view(np.uint8)
    if fmt != "q5_0":
        blk[2:4] = np.array([np.float16(m)], dtype=np.float16).view(np.uint8)
    qs0 = {"q4_1": 4, "q5_0": 6, "q5_1": 8}[fmt]
    c = np.asarray(codes, dtype=np.int64)
    blk[qs0:qs0 + 16] = ((c[:16] & 15) | ((c[16:] & 15) << 4)).astype(np.uint8)
    if fmt != "q4_1":
        qh = int(sum(((int(c[j]) >> 4) & 1) << j for j in range(32)))
        o = 2 if fmt == "q5_0" else 4
        blk[o:o + 4] = np.array([qh], dtype="<u4").view(np.uint8)
    return blk


@pytest.mark.parametrize("fmt", ["q4_1", "q5_0", "q5_1"])
def test_32_value_offset_formats_closed_form(orc, fmt):
    """Q4_1 / Q5_1: value = d * q + m (the per-block offset); Q5_0: value =
    d * (q - 16); codes use all their bits."""
    rng = synth.splitmix64(191, 0, 32)
    L = 15 if fmt == "q4_1" else 31
    codes = (rng % np.uint64(L + 1)).astype(np.int64)
    codes[0], codes[31] = L, 0
    vals = orc.dequantize(fmt, _blk32(fmt, 0.5, -0.25, codes), 32)[0]
    if fmt == "q5_0":
        assert np.array_equal(vals, 0.5 * (codes - 16))
    else:
        assert np.array_equal(vals, 0.5 * codes - 0.25)


@pytest.mark.parametrize("fmt", ["q5_0", "q5_1"])
@pytest.mark.parametrize("j", [0, 7, 15, 16, 31])
def test_q5_fifth_bit_position(orc, fmt, j):
    """Bit j of qh is value j's fifth bit (reading): all nibbles 0, only that
    bit set, so only value j moves by 16 d."""
    codes = np.zeros(32, dtype=np.int64)
    codes[j] = 16
    vals = orc.dequantize(fmt, _blk32(fmt, 1.0, 0.0, codes), 32)[0]
    base = -16.0 if fmt == "q5_0" else 0.0
    assert vals[j] == base + 16.0
    assert np.all(np.delete(vals, j) == base)


@pytest.mark.parametrize("fmt,tol", [("q4_1", 0.12), ("q5_0", 0.06), ("q5_1", 0.05)])
def test_32_value_quantizers_format_invariants(orc, fmt, tol):
    """The weight quantizers' rules are not on the pages (parity unpinned)."""
    w = synth.gaussian_f32((8, 1024), 0.02, 201)
    vals = orc.dequantize(fmt, orc.quantize_w(fmt, w), 1024)
    assert np.linalg.norm(vals - w) / np.linalg.norm(w) < tol


# ---------------------------------------------------------------------------
# Products: brute force on decoded values, layout, thread invariance
# ---------------------------------------------------------------------------
def _case(fmt, M, N, K, seed):
    w = synth.gaussian_f32((N, K), 0.02, seed)
    x = synth.with_outliers(synth.gaussian_f32((M, K), 1.0, seed + 1), 0.02, 20.0, seed + 2)
    import oracle
    return oracle.quantize_w(fmt, w), oracle.quantize_x(fmt, x)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0"])
def test_single_block_dot_is_exact(orc, fmt):
    wq, xq = _case(fmt, 1, 7, 32, 91)
    r = orc.matmul(fmt, wq, xq, 1, 7, 32, want=("y64",))
    W = orc.dequantize(fmt, wq, 32)
    X = orc.dequantize("q8_0", xq, 32)
    brute = np.array([sum(float(a) * float(b) for a, b in zip(W[n], X[0])) for n in range(7)])
    assert np.array_equal(r["y64"][0], brute)


@pytest.mark.parametrize("fmt,K", [("q4_0", 96), ("q8_0", 160), ("q2_k", 512), ("q4_0", 4096), ("q4_k", 512),
                                   ("q6_k", 768), ("q4_1", 96), ("q5_0", 160), ("q5_1", 128)])
def test_matmul_matches_decoded_float64_product(orc, fmt, K):
    M, N = 3, 5
    wq, xq = _case(fmt, M, N, K, 101)
    r = orc.matmul(fmt, wq, xq, M, N, K, want=("y", "y64", "mag"))
    W = orc.dequantize(fmt, wq, K)
    X = orc.dequantize(orc.act_format(fmt), xq, K)
    ref = X @ W.T                                       # [M][N]: token-major output
    assert r["y64"].shape == (M, N)
    assert np.all(np.abs(r["y64"] - ref) <= 1e-12 * r["mag"])
    assert np.array_equal(r["y"], r["y64"].astype(np.float32))
    absprod = np.abs(X) @ np.abs(W).T
    if fmt in ("q2_k", "q4_k"):                       # |d sc q| + |dmin m| >= |d sc q - dmin m|
        assert np.all(r["mag"] >= absprod * (1 - 1e-12))
    elif fmt in ("q4_1", "q5_1"):                     # sum |(dq + m) x|, in double
        assert np.all(np.abs(r["mag"] - absprod) <= 1e-12 * absprod)
    else:
        assert np.all(np.abs(r["mag"] - absprod) <= 1e-12 * absprod)


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q2_k", "q4_k", "q6_k", "q4_1", "q5_0", "q5_1"])
def test_matmul_rows_equal_matvec_and_threads_invariant(orc, fmt):
    M, N, K = 4, 37, 512
    wq, xq = _case(fmt, M, N, K, 111)
    r1 = orc.matmul(fmt, wq, xq, M, N, K, threads=1, want=("y64",))["y64"]
    r7 = orc.matmul(fmt, wq, xq, M, N, K, threads=7, want=("y64",))["y64"]
    assert np.array_equal(r1, r7)
    xr = xq.reshape(M, -1)
    for m in range(M):
        v = orc.matmul(fmt, wq, xr[m], 1, N, K, want=("y64",))["y64"][0]
        assert np.array_equal(v, r1[m])
    mi = np.array([0, 3, 2, 1])
    ni = np.array([36, 0, 17, 5])
    ys, _ = orc.matmul_sampled(fmt, wq, xq, mi, ni, K)
    assert np.array_equal(ys, r1[mi, ni])


# ---------------------------------------------------------------------------
# Embedding rows (minfer "The embedding matmul")
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt,K", [("q4_0", 96), ("q8_0", 64), ("q2_k", 512), ("q4_k", 256), ("q6_k", 768),
                                   ("q4_1", 64), ("q5_0", 96), ("q5_1", 32)])
def test_get_rows_is_the_decoded_row(orc, fmt, K):
    """Row t of the output is row ids[t] of the table, every value the exactly
    decoded one rounded once to f32; repeated ids repeat the row; ids outside
    the table give NaN rows."""
    N = 7
    w = orc.quantize_w(fmt, synth.gaussian_f32((N, K), 0.02, 181))
    ids = np.array([3, 0, 6, 3, -1, 7], dtype=np.int32)
    out = orc.get_rows(fmt, w, ids, N, K)
    dec = orc.dequantize(fmt, w, K)
    for t, i in enumerate(ids):
        if 0 <= i < N:
            assert np.array_equal(out[t], dec[i].astype(np.float32))
            assert np.array_equal(out[t].astype(np.float64), dec[i]) or fmt in ("q2_k", "q4_k", "q4_1", "q5_1")
        else:
            assert np.all(np.isnan(out[t]))
    assert np.array_equal(out[0], out[3])


def test_get_rows_worked_byte(orc):
    """The worked Q4_0 byte 0x21 (minfer section 3.2) through the row getter:
    scale 1.0 gives -7 at element j and -6 at element j + 16."""
    g = golden("worked_byte.json")
    blk = np.zeros(18, dtype=np.uint8)
    blk[0:2] = np.array([np.float16(1.0)], dtype=np.float16).view(np.uint8)
    blk[2:18] = 0x88                                  # every other element decodes to 0
    blk[2 + 5] = g["byte"]
    row = orc.get_rows("q4_0", blk, np.array([0], dtype=np.int32), 1, 32)[0] * g["scale_w"]
    assert row[5] == g["element_j"] and row[5 + 16] == g["element_j_plus_16"]
    assert np.count_nonzero(row) == 2


# ---------------------------------------------------------------------------
# The seeded input stream
# ---------------------------------------------------------------------------
def test_splitmix64_counter_form_equals_sequential_definition():
    mask = (1 << 64) - 1

    def sequential(seed, n):
        state, out = seed, []
        for _ in range(n):
            state = (state + 0x9E3779B97F4A7C15) & mask
            z = state
            z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
            z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
            out.append(z ^ (z >> 31))
        return out

    for seed in (0, 1, synth.seed_for(1, 0), mask):
        ref = sequential(seed, 40)
        assert [int(v) for v in synth.splitmix64(seed, 0, 40)] == ref
        assert [int(v) for v in synth.splitmix64(seed, 17, 5)] == ref[17:22]
    assert int(synth.splitmix64(0, 0, 1)[0]) == 0xE220A8397B1DCDAF


def test_normal_stream_moments_and_outliers():
    z = synth.normal(synth.seed_for(0, 1), 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    x = synth.activations(2, 4096, 1, outlier_frac=0.01, outlier_factor=20.0)
    base = synth.activations(2, 4096, 1)
    changed = np.nonzero(x[0] != base[0])[0]
    assert len(changed) == 41
    assert np.allclose(x[:, changed], base[:, changed] * 20.0)
