"""Parity of the HIP path with the oracle, through the C ABI, on an MI355X.

Quantizers must be bit-exact.  Products must satisfy, per output,
    |y_gpu - y_exact| <= 1e-5 * sum_i |d_w w_i d_x q_i|
(the krafla "Numerics" bound: integer block sums are exact, only the f32
accumulation order differs), where y_exact is the oracle's double result.

Every input is seeded (synth) and every expected value comes from the oracle.
"""
import numpy as np
import pytest

import synth
from conftest import golden

pytestmark = pytest.mark.gpu

TOL = golden("tolerance.json")["relative_to_magnitude"]


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import matmul_quantize_q8_amd as q
    import oracle
    q.lib()
    oracle.lib()
    return torch, q, oracle


def _dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _say(*a):
    print("[case]", *a, flush=True)


def _gpu_quant(env, fmt, x, weights=False):
    """Quantize f32 rows on the GPU with the format's product-side quantizer."""
    torch, q, _ = env
    rows, K = x.shape
    out = torch.zeros(rows * q.row_bytes(fmt, K), dtype=torch.uint8, device="cuda")
    fn = dict(q.QUANTIZE_W, q8_k=q.qmm_quantize_q8_k)[fmt]
    fn(_dev(torch, x), out, rows, K)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(rows, -1)


def _edge_rows(rows, K, seed):
    x = synth.with_outliers(synth.gaussian_f32((rows, K), 1.0, seed), 0.01, 20.0, seed + 1)
    x[0, :32] = 0.0                                   # zero block
    if K >= 64:
        x[0, 32:64] = 0.0
        x[0, 37] = -2.75                              # one nonzero value
    if rows > 1 and K >= 96:
        x[1, 64:96] *= 1e-30                          # tiny but inside the contract
        x[1, :32] = np.arange(32, dtype=np.float32) - 15.5    # x * id lands exactly on .5: ties
        x[1, 0] = 127.0                                        # amax 127, so id = 1 exactly
    return x


# ---------------------------------------------------------------------------
# Quantizers: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("rows,K", [(1, 32), (1, 1024), (3, 4096), (7, 96), (2048, 4096), (5, 11008)])
def test_quantize_q8_0_bit_exact(env, rows, K):
    _, _, orc = env
    _say("quantize_q8_0", rows, K)
    x = _edge_rows(rows, K, 1000 + rows + K)
    assert np.array_equal(_gpu_quant(env, "q8_0", x), orc.quantize_q8_0(x))


@pytest.mark.parametrize("rows,K", [(1, 256), (1, 4096), (9, 768), (64, 4096)])
def test_quantize_q8_k_bit_exact(env, rows, K):
    _, _, orc = env
    _say("quantize_q8_k", rows, K)
    x = _edge_rows(rows, K, 2000 + rows + K)
    if rows > 2:
        x[2, 256:512] = 0.0
    assert np.array_equal(_gpu_quant(env, "q8_k", x), orc.quantize_q8_k(x))


@pytest.mark.parametrize("rows,K", [(1, 32), (512, 1024), (33, 96), (12288, 4096)])
def test_quantize_q4_0_weights_bit_exact(env, rows, K):
    _, _, orc = env
    _say("quantize_q4_0", rows, K)
    w = synth.gaussian_f32((rows, K), 0.02, 3000 + rows)
    w[0, :32] = 0.0
    if rows > 1 and K >= 32:
        w[1, :32] = 0.01
        w[1, 3] = -0.5
        w[1, 10] = 0.5
    assert np.array_equal(_gpu_quant(env, "q4_0", w), orc.quantize_q4_0_w(w))


@pytest.mark.parametrize("rows,K", [(1, 256), (16, 1024), (12288, 4096)])
def test_quantize_q2_k_weights_bit_exact(env, rows, K):
    _, _, orc = env
    _say("quantize_q2_k", rows, K)
    w = synth.gaussian_f32((rows, K), 0.02, 4000 + rows)
    w[0, :256] = 0.0
    if rows > 1:
        w[1, :16] = np.abs(w[1, :16])                 # a group with no negative value
    assert np.array_equal(_gpu_quant(env, "q2_k", w), orc.quantize_q2_k_w(w))


@pytest.mark.parametrize("fmt", ["q4_k", "q6_k"])
@pytest.mark.parametrize("rows,K", [(1, 256), (16, 1024), (12288, 4096), (3, 1280)])
def test_quantize_k_weights_bit_exact(env, fmt, rows, K):
    _, _, orc = env
    _say("quantize", fmt, rows, K)
    w = synth.gaussian_f32((rows, K), 0.02, 4100 + rows + K)
    w[0, :256] = 0.0                                  # zero super-block
    if rows > 1:
        w[1, :32] = np.abs(w[1, :32])                 # a sub-block with no negative value
        w[1, 40] = -0.5                               # magnitude tie inside a group: first index wins
        w[1, 44] = 0.5
    assert np.array_equal(_gpu_quant(env, fmt, w), orc.quantize_w(fmt, w))


@pytest.mark.parametrize("fmt", ["q4_1", "q5_0", "q5_1"])
@pytest.mark.parametrize("rows,K", [(1, 32), (16, 1024), (12288, 4096), (3, 96)])
def test_quantize_32_value_offset_weights_bit_exact(env, fmt, rows, K):
    _, _, orc = env
    _say("quantize", fmt, rows, K)
    w = synth.gaussian_f32((rows, K), 0.02, 4200 + rows + K)
    w[0, :32] = 0.0                                   # zero block
    if rows > 1:
        w[1, :32] = np.abs(w[1, :32])                 # no negative value
        w[1, 3] = -0.5                                # magnitude tie: first index wins
        w[1, 10] = 0.5
    assert np.array_equal(_gpu_quant(env, fmt, w), orc.quantize_w(fmt, w))


# ---------------------------------------------------------------------------
# Products
# ---------------------------------------------------------------------------
def _inputs(fmt, M, N, K, seed, outliers=True):
    import oracle
    w = synth.gaussian_f32((N, K), 0.02, seed)
    x = synth.gaussian_f32((M, K), 1.0, seed + 1)
    if outliers:
        x = synth.with_outliers(x, 0.01, 20.0, seed + 2)
    return oracle.quantize_w(fmt, w), oracle.quantize_x(fmt, x)


def _check(y, ref, mag, what):
    y = np.asarray(y, dtype=np.float64).reshape(ref.shape)
    err = np.abs(y - ref)
    bound = TOL * mag
    bad = np.nonzero(err > bound)
    assert bad[0].size == 0, (what, bad[0].size, [(tuple(int(i) for i in ix), float(y[ix]), float(ref[ix]),
                                                    float(bound[ix])) for ix in zip(*bad)][:5])


def _run_matvec(env, fmt, wq, xq, N, K):
    torch, q, _ = env
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    q.MATVEC[fmt](_dev(torch, wq), _dev(torch, xq), y, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run_matmul(env, fmt, wq, xq, M, N, K):
    torch, q, _ = env
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    q.MATMUL[fmt](_dev(torch, wq), _dev(torch, xq), y, M, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy()


MATVEC_CASES = [
    ("q4_0", 512, 1024),     # 512 x 1024 decode (L2-resident)
    ("q4_0", 12288, 4096),   # FFN-gate decode
    ("q4_0", 1, 32), ("q4_0", 3, 96), ("q4_0", 17, 160), ("q4_0", 5, 2080), ("q4_0", 7, 8192),
    ("q4_0", 9, 20480),      # two row segments
    ("q4_0", 45, 1024), ("q8_0", 37, 256), ("q8_0", 3, 64),     # small N: one row per wave
    ("q4_0", 13, 2048), ("q4_0", 7, 4000),                       # one row x 1 unit; one row x 4 single units
    # rows per wave past the 2048-wave floor, ragged last wave: 8 rows (K <= 1024
    # at N >= 16384), 4 rows, 2 rows x 4 single units (odd block count)
    ("q4_0", 16389, 1024), ("q4_0", 8197, 2048), ("q4_0", 4099, 4000), ("q8_0", 16411, 256),
    ("q2_k", 16390, 256), ("q4_k", 16391, 512), ("q6_k", 16387, 512), ("q4_1", 16389, 512),
    ("q5_0", 16389, 1024),
    ("q8_0", 5, 16384), ("q8_0", 3, 40960),                      # > 64 KB of LDS; paired segments
    ("q8_0", 12288, 4096), ("q8_0", 22016, 4096), ("q8_0", 4096, 11008),   # one 7B-style layer
    ("q8_0", 1, 32), ("q8_0", 5, 96), ("q8_0", 11, 4128), ("q8_0", 3, 20000),
    ("q2_k", 12288, 4096),
    ("q2_k", 1, 256), ("q2_k", 3, 768), ("q2_k", 13, 9216), ("q2_k", 2, 40960),
    ("q4_k", 12288, 4096), ("q4_k", 1, 256), ("q4_k", 3, 768), ("q4_k", 45, 512),   # 8 rows per wave
    ("q4_k", 13, 9216), ("q4_k", 2, 40960), ("q4_k", 7, 1280),                      # 4 units per lane; segments
    ("q6_k", 12288, 4096), ("q6_k", 1, 256), ("q6_k", 3, 768), ("q6_k", 37, 512),
    ("q6_k", 13, 9216), ("q6_k", 2, 40960), ("q6_k", 5, 1280),   # odd super-block count: rows 2 mod 4
] + [(f, N, K) for f in ("q4_1", "q5_0", "q5_1")
     for N, K in ((12288, 4096), (1, 32), (3, 96), (17, 160), (5, 2080), (7, 8192), (9, 20480), (45, 1024))]


@pytest.mark.parametrize("fmt,N,K", MATVEC_CASES)
def test_matvec_matches_oracle(env, fmt, N, K):
    _, _, orc = env
    _say("matvec", fmt, N, K)
    wq, xq = _inputs(fmt, 1, N, K, 5000 + N + K)
    ref = orc.matmul(fmt, wq, xq, 1, N, K, threads=8, want=("y64", "mag"))
    y = _run_matvec(env, fmt, wq, xq, N, K)
    _check(y, ref["y64"][0], ref["mag"][0], (fmt, N, K))


FUSED_CASES = [
    ("q4_0", 512, 1024), ("q4_0", 12288, 4096),
    ("q4_0", 1, 32), ("q4_0", 3, 96), ("q4_0", 17, 160), ("q4_0", 5, 2080), ("q4_0", 7, 8192),
    ("q4_0", 9, 20480), ("q4_0", 45, 1024), ("q4_0", 13, 2048), ("q4_0", 7, 4000),
    ("q4_0", 16389, 1024), ("q4_0", 8197, 2048),                # 8 and 4 rows per wave
    ("q8_0", 37, 256), ("q8_0", 3, 64), ("q8_0", 5, 16384), ("q8_0", 3, 40960), ("q8_0", 16411, 256),
    ("q8_0", 12288, 4096), ("q8_0", 22016, 4096), ("q8_0", 4096, 11008),
    ("q8_0", 1, 32), ("q8_0", 11, 4128), ("q8_0", 3, 20000),
    # K-quant weights with Q8_K activations: one segment (up to 16 super-blocks,
    # 2 per wave of eight), 8 rows per wave, ragged waves; longer rows run the
    # quantizer and the plain kernel when xq is requested
    ("q2_k", 12288, 4096), ("q4_k", 12288, 4096), ("q6_k", 12288, 4096),
    ("q2_k", 1, 256), ("q4_k", 3, 768), ("q6_k", 5, 1280), ("q4_k", 45, 512), ("q6_k", 37, 512),
    ("q2_k", 16390, 256), ("q4_k", 16391, 512), ("q6_k", 4099, 3840),
    ("q2_k", 13, 9216), ("q4_k", 2, 40960), ("q6_k", 13, 9216),
]


def _run_fused(env, fmt, wq, x, N, K, want_xq=True):
    torch, q, _ = env
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    xq = torch.full((q.row_bytes(q.ACT_FORMAT[fmt], K),), 0xA5, dtype=torch.uint8, device="cuda") if want_xq else None
    q.QUANTIZE_MATVEC[fmt](_dev(torch, wq), _dev(torch, x), xq, y, N, K)
    torch.cuda.synchronize()
    return y.cpu().numpy(), (xq.cpu().numpy() if want_xq else None)


@pytest.mark.parametrize("fmt,N,K", FUSED_CASES)
def test_fused_quantize_matvec_matches_oracle(env, fmt, N, K):
    """One launch quantizes the f32 activation and applies the weights: the
    Q8_0 (Q8_K) row it writes is the oracle's byte for byte, the output is
    within the bound of the oracle's product on that row."""
    _, _, orc = env
    _say("quantize_matvec", fmt, N, K)
    seed = 9000 + N + K
    wq = orc.quantize_w(fmt, synth.gaussian_f32((N, K), 0.02, seed))
    x = synth.with_outliers(synth.gaussian_f32((1, K), 1.0, seed + 1), 0.01, 20.0, seed + 2)
    x[0, :32] = 0.0                                   # zero block
    if K >= 64:
        x[0, 32:64] = 0.0
        x[0, 37] = -2.75                              # one nonzero value
    if K >= 96:
        x[0, 64:96] = np.arange(32, dtype=np.float32) - 15.5   # ties at .5
        x[0, 64] = 127.0
    if K >= 128:
        x[0, 96:128] *= 1e-30                         # tiny but inside the contract
    if K >= 512:
        x[0, 256:512] = 0.0                           # zero super-block
    if K >= 768:
        x[0, 512:768] = np.arange(256, dtype=np.float32) - 128.0   # amax 128: x * 127/128 ties at .5
    xq_ref = orc.quantize_x(fmt, x)
    y, xq = _run_fused(env, fmt, wq, x, N, K)
    assert np.array_equal(xq, xq_ref.reshape(-1))
    ref = orc.matmul(fmt, wq, xq_ref, 1, N, K, threads=8, want=("y64", "mag"))
    _check(y, ref["y64"][0], ref["mag"][0], ("fused", fmt, N, K))


@pytest.mark.parametrize("fmt,N,K", [("q4_0", 1000, 4096), ("q4_0", 37, 8192), ("q4_0", 9, 20480),
                                     ("q4_0", 5, 2080), ("q4_0", 45, 1024), ("q8_0", 300, 4096),
                                     ("q8_0", 3, 40960), ("q8_0", 11, 4128),
                                     ("q2_k", 300, 4096), ("q4_k", 37, 8192), ("q6_k", 9, 20480),
                                     ("q2_k", 13, 9216), ("q4_k", 5, 40960), ("q6_k", 45, 1280)])
def test_fused_without_xq_output_equals_two_launches(env, fmt, N, K):
    """xq = NULL (always the single fused launch, also for long rows): y is
    within the bound of the oracle and bit-identical to the two-launch path
    (same codes, same per-row summation order)."""
    torch, q, orc = env
    _say("quantize_matvec no xq", fmt, N, K)
    wq = orc.quantize_w(fmt, synth.gaussian_f32((N, K), 0.02, 9500 + K))
    x = synth.with_outliers(synth.gaussian_f32((1, K), 1.0, 9501 + K), 0.01, 20.0, 9502 + K)
    y, _ = _run_fused(env, fmt, wq, x, N, K, want_xq=False)
    act = q.ACT_FORMAT[fmt]
    xq_d = torch.empty(q.row_bytes(act, K), dtype=torch.uint8, device="cuda")
    getattr(q, "qmm_quantize_" + act)(_dev(torch, x), xq_d, 1, K)
    y2 = torch.empty(N, dtype=torch.float32, device="cuda")
    q.MATVEC[fmt](_dev(torch, wq), xq_d, y2, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(y, y2.cpu().numpy())
    ref = orc.matmul(fmt, wq, orc.quantize_x(fmt, x), 1, N, K, threads=8, want=("y64", "mag"))
    _check(y, ref["y64"][0], ref["mag"][0], ("fused no xq", fmt, N, K))


@pytest.mark.parametrize("fmt,N,K", [("q4_0", 151, 896), ("q8_0", 64, 1024), ("q2_k", 33, 512),
                                     ("q4_k", 40, 4096), ("q6_k", 17, 1280), ("q4_0", 3000, 4096),
                                     ("q4_1", 20, 96), ("q5_0", 31, 160), ("q5_1", 9, 4096)])
def test_get_rows_bit_exact(env, fmt, N, K):
    """Embedding rows are byte-for-byte the oracle's (minfer "The embedding
    matmul"), repeated ids included; ids outside the table give NaN rows."""
    torch, q, orc = env
    _say("get_rows", fmt, N, K)
    w = orc.quantize_w(fmt, synth.gaussian_f32((N, K), 0.02, 9700 + N))
    ids = np.array([0, N - 1, 5 % N, 0, -1, N, 2 % N, N - 1], dtype=np.int32)
    ref = orc.get_rows(fmt, w, ids, N, K)
    out = torch.full((ids.size, K), 1.0, dtype=torch.float32, device="cuda")
    q.GET_ROWS[fmt](_dev(torch, w), _dev(torch, ids), out, ids.size, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


MATMUL_CASES = [
    ("q4_0", 1, 8, 32), ("q4_0", 37, 200, 1024), ("q4_0", 128, 128, 4096), ("q4_0", 130, 129, 160),
    ("q4_0", 64, 512, 1024), ("q4_0", 5, 3, 96), ("q4_0", 256, 384, 4128), ("q4_0", 300, 700, 2080),
    ("q4_0", 129, 257, 64),
    # even block counts (the dword-plane kernel): 1..7 stages, ragged tiles
    ("q4_0", 1, 129, 64), ("q4_0", 131, 255, 128), ("q4_0", 70, 130, 192), ("q4_0", 257, 129, 256),
    ("q4_0", 3, 300, 320), ("q4_0", 200, 100, 448),
    # token counts one past and one short of 64: the last on the 32-token
    # tile and the first on the 128-token tile
    ("q4_0", 65, 130, 96), ("q4_0", 63, 127, 2048), ("q8_0", 65, 129, 160), ("q8_0", 63, 255, 2048),
    ("q8_0", 1, 8, 32), ("q8_0", 37, 200, 1024), ("q8_0", 128, 128, 4096), ("q8_0", 130, 129, 160),
    ("q8_0", 5, 3, 96), ("q8_0", 131, 255, 128), ("q8_0", 257, 129, 256), ("q8_0", 300, 700, 2080),
    ("q8_0", 3, 300, 320), ("q8_0", 129, 257, 64),
    ("q2_k", 1, 8, 256), ("q2_k", 9, 70, 1024), ("q2_k", 33, 130, 4096),
    ("q2_k", 128, 128, 256), ("q2_k", 130, 257, 512), ("q2_k", 257, 129, 2304), ("q2_k", 3, 300, 7936),
    ("q4_k", 1, 8, 256), ("q4_k", 9, 70, 1024), ("q4_k", 33, 130, 4096),
    ("q4_k", 128, 256, 256), ("q4_k", 130, 257, 512), ("q4_k", 257, 300, 2304), ("q4_k", 3, 520, 7936),
    ("q6_k", 1, 8, 256), ("q6_k", 9, 70, 1024), ("q6_k", 5, 33, 1280),
    ("q6_k", 128, 128, 256), ("q6_k", 130, 257, 512), ("q6_k", 257, 129, 2304), ("q6_k", 65, 300, 7936),
    # the K-quants' 32-token tile: two K groups per workgroup (uneven
    # super-block counts, one super-block per group, 64 tokens in two tiles),
    # one group with K split in two (2 super-blocks) or whole (1, or a grid of
    # more than 256 tiles)
    ("q4_k", 50, 129, 1280), ("q2_k", 17, 129, 1024), ("q6_k", 64, 257, 4096), ("q6_k", 12, 130, 2304),
    ("q6_k", 40, 200, 512), ("q2_k", 20, 70, 256), ("q4_k", 64, 300, 256), ("q2_k", 40, 16641, 512),
    ("q4_k", 45, 16390, 768), ("q2_k", 31, 260, 8192),
    # 65-128 tokens: the K-quants' 32-token tiles (Q2_K, Q4_K: three or four
    # token tiles, two K groups, a split without groups, no split) and the
    # 128-token tile (Q4_0, Q5_0: two K groups, one part)
    ("q4_0", 96, 4100, 1024), ("q4_0", 100, 130, 4096), ("q5_0", 120, 16500, 512), ("q5_0", 70, 257, 2080),
    ("q2_k", 100, 8200, 1024), ("q2_k", 65, 129, 512), ("q4_k", 127, 300, 2304), ("q4_k", 128, 16390, 256),
    # Q4_1 and Q5_1 on the same kernel, the offset term on an f32 MFMA
    ("q4_1", 1, 8, 32), ("q4_1", 9, 70, 1024), ("q4_1", 5, 3, 96), ("q4_1", 130, 129, 160),
    ("q4_1", 131, 255, 128), ("q4_1", 65, 130, 96), ("q4_1", 63, 127, 2048), ("q4_1", 129, 257, 64),
    ("q5_1", 1, 8, 32), ("q5_1", 9, 70, 1024), ("q5_1", 5, 3, 96), ("q5_1", 130, 129, 160),
    ("q5_1", 131, 255, 128), ("q5_1", 65, 130, 96), ("q5_1", 63, 127, 2048), ("q5_1", 300, 700, 2080),
    # Q5_0 on the Q4_0 MFMA kernel: one block, odd and even block counts, ragged tiles
    ("q5_0", 1, 8, 32), ("q5_0", 9, 70, 1024), ("q5_0", 5, 3, 96), ("q5_0", 130, 129, 160),
    ("q5_0", 131, 255, 128), ("q5_0", 65, 130, 96), ("q5_0", 63, 127, 2048), ("q5_0", 300, 700, 2080),
    ("q5_0", 129, 257, 64), ("q5_0", 128, 128, 4096),
    # long rows: 1025 blocks (an odd count), 128 super-blocks
    ("q4_0", 129, 65, 32800), ("q5_1", 65, 33, 32800), ("q2_k", 65, 129, 32768), ("q6_k", 33, 65, 32768),
    # 17-64 tokens on the 32-token tile; odd block counts, K split in two and
    # in one part (fewer than 4 blocks, or more than 256 tiles), ragged M and N
    ("q4_0", 17, 300, 160), ("q4_0", 33, 129, 96), ("q4_0", 64, 16577, 256), ("q4_0", 32, 12288, 4096),
    ("q8_0", 50, 260, 4128), ("q8_0", 64, 16512, 128), ("q5_0", 20, 130, 2080), ("q4_1", 45, 257, 1024),
    ("q5_1", 32, 128, 4096), ("q5_1", 17, 16641, 160),
    # more than 256 output tiles (128 x 128; 128 x 256 for Q2_K and Q4_K):
    # K in one part, the kernels the 2048-token prefill runs (the cases above
    # with 4 blocks or more have at most 256 tiles and split K in two); per
    # format an odd block or super-block count (the last stage shifted back
    # one block, or a last stage of one super-block) and an even one, with
    # ragged M and N
    ("q4_0", 129, 16640, 160), ("q4_0", 257, 16577, 256),
    ("q8_0", 130, 16512, 128), ("q8_0", 257, 16640, 160),
    ("q5_0", 257, 16640, 160), ("q5_0", 129, 16577, 256),
    ("q4_1", 257, 16640, 160), ("q4_1", 129, 16577, 256),
    ("q5_1", 257, 16640, 160), ("q5_1", 129, 16577, 256),
    ("q2_k", 257, 33024, 768), ("q2_k", 129, 33025, 512),
    ("q4_k", 257, 33024, 768), ("q4_k", 129, 33025, 512),
    ("q6_k", 257, 16640, 768), ("q6_k", 129, 16577, 512),
    # exactly 256 tiles (1 x 256): the largest launch that still splits K
    ("q5_1", 100, 32768, 128),
    # 128-token tiles with K split in two: one group of four waves (130 and
    # 256 tiles), two K groups (fewer than 128 tiles; 16 and 17 blocks, an
    # uneven group step, ragged M and N)
    ("q4_1", 130, 8200, 1024), ("q8_0", 200, 16384, 544), ("q8_0", 100, 130, 512), ("q5_1", 70, 257, 544),
    ("q4_0", 150, 200, 1056), ("q5_0", 255, 300, 4096),
    # the edge of K groups per workgroup: 127 tiles (four groups for the
    # 32-value formats' 32-token tile, two elsewhere) and 128 (one group, K
    # split in two), on the 32-token tile, the 128-token tile and the
    # K-quants' 32-token tile
    ("q4_0", 20, 16256, 512), ("q4_0", 20, 16384, 512), ("q8_0", 100, 16256, 512), ("q8_0", 100, 16384, 512),
    ("q4_k", 20, 16256, 1024), ("q4_k", 20, 16384, 1024),
]


# Few tokens: up to 2, 4 or 8 by format on the decode kernel with 2, 4 or 8
# tokens per weight pass (ragged token groups, odd block counts: unpaired
# units, rows walked in segments: K = 8192 and 11008), and the counts just
# past that on the 32-token MFMA tiles, every format.
SMALL_M_CASES = [
    ("q4_0", 2, 130, 4096), ("q4_0", 3, 77, 4128), ("q4_0", 8, 12288, 4096), ("q4_0", 9, 65, 8192),
    ("q4_0", 15, 33, 11008), ("q4_0", 16, 129, 1024), ("q4_0", 5, 9, 32), ("q4_0", 17, 65, 4096),
    ("q8_0", 4, 257, 4096), ("q8_0", 7, 70, 11008), ("q8_0", 16, 33, 2080), ("q8_0", 13, 64, 96),
    ("q4_1", 6, 130, 4096), ("q4_1", 12, 17, 4128), ("q5_0", 6, 130, 4096), ("q5_0", 14, 9, 8192),
    ("q5_1", 6, 130, 4096), ("q5_1", 2, 31, 160),
    ("q2_k", 2, 130, 4096), ("q2_k", 11, 70, 2304), ("q2_k", 16, 33, 11008),
    ("q4_k", 3, 130, 4096), ("q4_k", 8, 12288, 4096), ("q4_k", 10, 31, 11008), ("q4_k", 32, 65, 2304),
    ("q4_k", 25, 129, 4096), ("q4_k", 33, 33, 4096),
    ("q6_k", 5, 130, 4096), ("q6_k", 16, 65, 2304), ("q6_k", 9, 33, 11008),
    # the largest token counts on the decode kernel (8 for Q4_0, 2 for Q2_K,
    # 4 for the other formats), and the first past them on the MFMA kernels;
    # the cases above past those counts run on the MFMA kernels
    ("q6_k", 8, 65, 2304), ("q6_k", 7, 33, 11008), ("q8_0", 10, 70, 11008), ("q8_0", 9, 257, 4096),
    ("q5_0", 10, 9, 8192), ("q2_k", 10, 33, 11008), ("q2_k", 9, 130, 4096),
    ("q5_0", 4, 130, 4096), ("q5_0", 3, 70, 11008), ("q4_1", 4, 130, 4096), ("q5_1", 4, 33, 4128),
    ("q8_0", 3, 70, 11008), ("q4_0", 7, 65, 8192), ("q4_1", 5, 70, 4128), ("q5_1", 5, 130, 8192),
    ("q2_k", 3, 70, 4096), ("q4_k", 4, 33, 11008), ("q4_k", 5, 130, 2304), ("q6_k", 4, 65, 4096),
    ("q6_k", 5, 70, 2304),
    # the first counts on the 32-token MFMA tile, with two K groups per
    # workgroup (K of 16 and 17 blocks: two stages per group, and an odd
    # last stage) and without (K of 3 blocks, no split)
    ("q4_0", 9, 130, 512), ("q8_0", 9, 257, 544), ("q5_0", 5, 9, 544), ("q4_1", 9, 33, 96),
    ("q5_1", 12, 200, 512),
    # rows per wave past the 2048-wave floor over the grid's token rows: 8 rows
    # (one pass of 8 tokens), 4 rows (4 tokens, Q8_0 and Q4_K)
    ("q4_0", 8, 16389, 1024), ("q8_0", 4, 8197, 1024), ("q4_k", 4, 8203, 512),
    # the 32-token tile on a ragged 4101 rows
    ("q4_k", 16, 4101, 512),
]


@pytest.mark.parametrize("fmt,M,N,K", SMALL_M_CASES)
def test_matmul_few_tokens_matches_oracle(env, fmt, M, N, K):
    _, _, orc = env
    _say("matmul few tokens", fmt, M, N, K)
    wq, xq = _inputs(fmt, M, N, K, 9000 + M + N + K)
    ref = orc.matmul(fmt, wq, xq, M, N, K, threads=8, want=("y64", "mag"))
    y = _run_matmul(env, fmt, wq, xq, M, N, K)
    _check(y, ref["y64"], ref["mag"], (fmt, M, N, K))


@pytest.mark.parametrize("fmt,M,N,K", MATMUL_CASES)
def test_matmul_matches_oracle(env, fmt, M, N, K):
    _, _, orc = env
    _say("matmul", fmt, M, N, K)
    wq, xq = _inputs(fmt, M, N, K, 6000 + M + N + K)
    ref = orc.matmul(fmt, wq, xq, M, N, K, threads=8, want=("y64", "mag"))
    y = _run_matmul(env, fmt, wq, xq, M, N, K)
    _check(y, ref["y64"], ref["mag"], (fmt, M, N, K))


def test_matmul_prefill_full_size_every_output(env):
    """The 2048 x 12288 x 4096 prefill with the bench's weights and
    activations, every one of its 25.2 million outputs against the oracle
    (run on 16 host threads)."""
    torch, q, orc = env
    M, N, K = 2048, 12288, 4096
    _say("matmul q4_0 full, every output", M, N, K)
    w = synth.weights(N, K, config=1)
    x = synth.activations(M, K, config=4)
    wq = orc.quantize_q4_0_w(w)
    xq = orc.quantize_q8_0(x)
    y = _run_matmul(env, "q4_0", wq, xq, M, N, K)
    assert np.isfinite(y).all()
    ref = orc.matmul("q4_0", wq, xq, M, N, K, threads=16, want=("y64", "mag"))
    _check(y, ref["y64"], ref["mag"], "prefill, every output")


def test_matmul_q8_0_full_size_sampled(env):
    """A 2048 x 4096 x 4096 Q8_0 prefill, checked on sampled outputs and whole
    rows and columns at the tile edges."""
    torch, q, orc = env
    M, N, K = 2048, 4096, 4096
    _say("matmul q8_0 full", M, N, K)
    wq = orc.quantize_q8_0(synth.weights(N, K, config=8))
    xq = orc.quantize_q8_0(synth.activations(M, K, config=8))
    y = _run_matmul(env, "q8_0", wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(78, 0, 20000)
    mi = (rng[:10000] % np.uint64(M)).astype(np.int64)
    ni = (rng[10000:] % np.uint64(N)).astype(np.int64)
    edge_m = np.array([0, 127, 128, 2047])
    edge_n = np.array([0, 31, 32, 127, 128, 4095])
    mi = np.concatenate([mi, np.repeat(edge_m, N // 16), np.tile(np.arange(0, M, 5), len(edge_n))])
    ni = np.concatenate([ni, np.tile(np.arange(0, N, 16), len(edge_m)), np.repeat(edge_n, len(range(0, M, 5)))])
    ref, mag = orc.matmul_sampled("q8_0", wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, "q8_0 prefill sampled")


def test_matmul_q5_0_full_size_sampled(env):
    """The 2048 x 12288 x 4096 prefill with Q5_0 weights, checked on sampled
    outputs and whole rows and columns at the tile edges."""
    torch, q, orc = env
    M, N, K = 2048, 12288, 4096
    _say("matmul q5_0 full", M, N, K)
    wq = orc.quantize_q5_0_w(synth.weights(N, K, config=10))
    xq = orc.quantize_q8_0(synth.activations(M, K, config=10))
    y = _run_matmul(env, "q5_0", wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(97, 0, 20000)
    mi = (rng[:10000] % np.uint64(M)).astype(np.int64)
    ni = (rng[10000:] % np.uint64(N)).astype(np.int64)
    edge_m = np.array([0, 63, 64, 127, 128, 2047])
    edge_n = np.array([0, 31, 32, 127, 128, 12287])
    mi = np.concatenate([mi, np.repeat(edge_m, N // 64), np.tile(np.arange(0, M, 7), len(edge_n))])
    ni = np.concatenate([ni, np.tile(np.arange(0, N, 64), len(edge_m)), np.repeat(edge_n, len(range(0, M, 7)))])
    ref, mag = orc.matmul_sampled("q5_0", wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, "q5_0 prefill sampled")


@pytest.mark.parametrize("fmt,cfg,seed", [("q4_1", 9, 98), ("q5_1", 11, 99)])
def test_matmul_offset_formats_full_size_sampled(env, fmt, cfg, seed):
    """The 2048 x 12288 x 4096 prefill with Q4_1 / Q5_1 weights (int8 MFMA
    plus the offset term on an f32 MFMA), checked on sampled outputs and whole
    rows and columns at the tile edges."""
    torch, q, orc = env
    M, N, K = 2048, 12288, 4096
    _say("matmul", fmt, "full", M, N, K)
    wq = orc.quantize_w(fmt, synth.weights(N, K, config=cfg))
    xq = orc.quantize_q8_0(synth.activations(M, K, config=cfg))
    y = _run_matmul(env, fmt, wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(seed, 0, 20000)
    mi = (rng[:10000] % np.uint64(M)).astype(np.int64)
    ni = (rng[10000:] % np.uint64(N)).astype(np.int64)
    edge_m = np.array([0, 63, 64, 127, 128, 2047])
    edge_n = np.array([0, 31, 32, 127, 128, 12287])
    mi = np.concatenate([mi, np.repeat(edge_m, N // 64), np.tile(np.arange(0, M, 7), len(edge_n))])
    ni = np.concatenate([ni, np.tile(np.arange(0, N, 64), len(edge_m)), np.repeat(edge_n, len(range(0, M, 7)))])
    ref, mag = orc.matmul_sampled(fmt, wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, fmt + " prefill sampled")


def test_matmul_q2_k_full_size_sampled(env):
    """The 2048 x 12288 x 4096 prefill with Q2_K weights (int8 + f16 MFMA),
    checked on sampled outputs and whole rows and columns at the tile edges."""
    torch, q, orc = env
    M, N, K = 2048, 12288, 4096
    _say("matmul q2_k full", M, N, K)
    wq = orc.quantize_q2_k_w(synth.weights(N, K, config=3))
    xq = orc.quantize_q8_k(synth.activations(M, K, config=3))
    y = _run_matmul(env, "q2_k", wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(79, 0, 20000)
    mi = (rng[:10000] % np.uint64(M)).astype(np.int64)
    ni = (rng[10000:] % np.uint64(N)).astype(np.int64)
    edge_m = np.array([0, 127, 128, 2047])
    edge_n = np.array([0, 31, 32, 127, 128, 12287])
    mi = np.concatenate([mi, np.repeat(edge_m, N // 64), np.tile(np.arange(0, M, 7), len(edge_n))])
    ni = np.concatenate([ni, np.tile(np.arange(0, N, 64), len(edge_m)), np.repeat(edge_n, len(range(0, M, 7)))])
    ref, mag = orc.matmul_sampled("q2_k", wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, "q2_k prefill sampled")


def test_matmul_q4_k_full_size_sampled(env):
    """The 2048 x 12288 x 4096 prefill with Q4_K weights (one int8 MFMA tile
    per sub-block, scales applied in int32, f16 MFMA min term), checked on
    sampled outputs and whole rows and columns at the tile edges."""
    torch, q, orc = env
    M, N, K = 2048, 12288, 4096
    _say("matmul q4_k full", M, N, K)
    wq = orc.quantize_q4_k_w(synth.weights(N, K, config=5))
    xq = orc.quantize_q8_k(synth.activations(M, K, config=5))
    y = _run_matmul(env, "q4_k", wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(83, 0, 20000)
    mi = (rng[:10000] % np.uint64(M)).astype(np.int64)
    ni = (rng[10000:] % np.uint64(N)).astype(np.int64)
    edge_m = np.array([0, 127, 128, 2047])
    edge_n = np.array([0, 31, 32, 255, 256, 12287])
    mi = np.concatenate([mi, np.repeat(edge_m, N // 64), np.tile(np.arange(0, M, 7), len(edge_n))])
    ni = np.concatenate([ni, np.tile(np.arange(0, N, 64), len(edge_m)), np.repeat(edge_n, len(range(0, M, 7)))])
    ref, mag = orc.matmul_sampled("q4_k", wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, "q4_k prefill sampled")


@pytest.mark.parametrize("fmt,cfg,M", [("q4_0", 1, 32), ("q4_0", 1, 128), ("q4_k", 5, 64), ("q4_k", 5, 128),
                                       ("q6_k", 6, 100)])
def test_matmul_bench_few_token_shapes_sampled(env, fmt, cfg, M):
    """The few-token products the bench times on the MFMA kernels (12288 x
    4096): the 32-token tiles (Q4_0 M = 32: four K groups per workgroup;
    Q4_K M = 64: K split in two; Q4_K M = 128: K in one part), Q4_0's
    128-token tile with two K groups at M = 128 and Q6_K's with K split in
    two, checked on whole rows and sampled outputs."""
    torch, q, orc = env
    N, K = 12288, 4096
    _say("matmul few-token bench shape", fmt, M, N, K)
    wq = orc.quantize_w(fmt, synth.weights(N, K, config=cfg))
    xq = orc.quantize_x(fmt, synth.activations(M, K, config=cfg))
    y = _run_matmul(env, fmt, wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(97 + M, 0, 8000)
    mi = (rng[:4000] % np.uint64(M)).astype(np.int64)
    ni = (rng[4000:] % np.uint64(N)).astype(np.int64)
    rows = np.array([0, M - 1])
    mi = np.concatenate([mi, np.repeat(rows, N)])
    ni = np.concatenate([ni, np.tile(np.arange(N), len(rows))])
    ref, mag = orc.matmul_sampled(fmt, wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, (fmt, M, "few-token sampled"))


def test_matmul_q6_k_full_size_sampled(env):
    """The 2048 x 12288 x 4096 prefill with Q6_K weights (one int8 MFMA tile
    per 16-value group on the unsigned codes, signed scales applied in int32,
    the offset of 32 from an f16 MFMA over the block sums), checked on
    sampled outputs and whole rows and columns at the tile edges."""
    torch, q, orc = env
    M, N, K = 2048, 12288, 4096
    _say("matmul q6_k full", M, N, K)
    wq = orc.quantize_q6_k_w(synth.weights(N, K, config=6))
    xq = orc.quantize_q8_k(synth.activations(M, K, config=6))
    y = _run_matmul(env, "q6_k", wq, xq, M, N, K)
    assert np.isfinite(y).all()
    rng = synth.splitmix64(89, 0, 20000)
    mi = (rng[:10000] % np.uint64(M)).astype(np.int64)
    ni = (rng[10000:] % np.uint64(N)).astype(np.int64)
    edge_m = np.array([0, 63, 64, 127, 128, 2047])
    edge_n = np.array([0, 31, 32, 127, 128, 12287])
    mi = np.concatenate([mi, np.repeat(edge_m, N // 64), np.tile(np.arange(0, M, 7), len(edge_n))])
    ni = np.concatenate([ni, np.tile(np.arange(0, N, 64), len(edge_m)), np.repeat(edge_n, len(range(0, M, 7)))])
    ref, mag = orc.matmul_sampled("q6_k", wq, xq, mi, ni, K)
    _check(y[mi, ni], ref, mag, "q6_k prefill sampled")


def _degenerate_weights(N, K, seed):
    """Weight rows that hit the formats' corner cases, then Gaussian rows."""
    w = synth.gaussian_f32((N, K), 0.02, seed)
    w[0] = 0.0                                        # all-zero blocks (d = 0)
    w[1] = 0.05                                       # constant: the extreme code in every block
    w[2] = -0.05
    w[3] = 0.0
    w[3, ::32] = 0.7                                  # one nonzero per 32 values
    w[4] *= 1e-4                                      # f16 scales in the subnormal range
    w[5] *= 5e4                                       # large values
    w[6, : K // 2] = 0.0                              # half a row zero
    return w


def _degenerate_activations(M, K, seed):
    """Activation rows that hit the quantizer's corner cases, then Gaussian rows."""
    x = synth.with_outliers(synth.gaussian_f32((M, K), 1.0, seed), 0.01, 20.0, seed + 1)
    x[0] = 0.0                                        # zero blocks: d = 0, codes 0
    x[1] = 1.0                                        # every code +127
    x[2] = -1.0                                       # every code -127
    x[3, 0::2], x[3, 1::2] = 1.0, -1.0                # alternating signs: block sums 0
    x[4] *= 1e-7                                      # d rounds to 0 in f16, codes do not
    x[5] *= 1e4                                       # large scales
    x[6, :32] = np.arange(32, dtype=np.float32) - 15.5   # exact ties in x * id
    x[6, 0] = 127.0
    return x


@pytest.mark.parametrize("fmt", ["q4_0", "q8_0", "q4_1", "q5_0", "q5_1", "q2_k", "q4_k", "q6_k"])
def test_products_on_degenerate_inputs(env, fmt):
    """Matvec and matmul on corner-case weights and activations: zero and
    constant rows, extreme codes (|I| at its largest), f16 scales that are
    subnormal or round to zero, large scales, exact rounding ties."""
    torch, q, orc = env
    K = 768 if fmt in orc.K_QUANTS else 288          # 3 super-blocks, or 9 blocks (an odd count)
    M, N = 130, 70
    _say("degenerate", fmt, M, N, K)
    wq = orc.quantize_w(fmt, _degenerate_weights(N, K, 7100 + K))
    xq = orc.quantize_x(fmt, _degenerate_activations(M, K, 7200 + K))
    ref = orc.matmul(fmt, wq, xq, M, N, K, threads=8, want=("y64", "mag"))
    y = _run_matmul(env, fmt, wq, xq, M, N, K)
    _check(y, ref["y64"], ref["mag"], (fmt, "matmul"))
    assert np.all(y[0] == 0.0) and np.all(y[:, 0] == 0.0)   # a zero row or column gives exact zeros
    for m in range(8):
        yv = _run_matvec(env, fmt, wq, xq[m], N, K)
        _check(yv, ref["y64"][m], ref["mag"][m], (fmt, "matvec", m))


@pytest.mark.parametrize("M,N,K", [(40, 300, 2048), (40, 33000, 1024)])
def test_matmul_rows_equal_matvec(env, M, N, K):
    """Row m of the prefill product and the decode product of token m are two
    evaluations of the same outputs, each within the bound of the oracle.  M
    is past the few-token switch, so the rows come from the 32-token MFMA
    tiles: four K groups per workgroup at N = 300, one group and K in one
    part at N = 33000 (516 tiles)."""
    torch, q, orc = env
    _say("matmul rows vs matvec", M, N, K)
    wq, xq = _inputs("q4_0", M, N, K, 7000 + N)
    ref = orc.matmul("q4_0", wq, xq, M, N, K, threads=8, want=("y64", "mag"))
    y = _run_matmul(env, "q4_0", wq, xq, M, N, K)
    xr = xq.reshape(M, -1)
    for m in range(M):
        yv = _run_matvec(env, "q4_0", wq, xr[m], N, K)
        _check(yv, ref["y64"][m], ref["mag"][m], ("matvec row", m))
        _check(y[m], ref["y64"][m], ref["mag"][m], ("matmul row", m))
        # two values within TOL * mag of the exact one differ by at most twice that
        assert np.all(np.abs(y[m].astype(np.float64) - yv) <= 2 * TOL * ref["mag"][m])


def test_end_to_end_decode_gpu_quantized(env):
    """Decode as deployed: f32 activation quantized on the GPU, then the matvec;
    the activation bytes equal the oracle's, the output is within the bound."""
    torch, q, orc = env
    N, K = 12288, 4096
    w = synth.weights(N, K, config=1)
    x = synth.activations(1, K, config=1, outlier_frac=0.01, outlier_factor=20.0)
    wq_d = torch.zeros(N * q.row_bytes("q4_0", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q4_0(_dev(torch, w), wq_d, N, K)
    xq_d = torch.zeros(q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    q.qmm_quantize_q8_0(_dev(torch, x), xq_d, 1, K)
    y = torch.empty(N, dtype=torch.float32, device="cuda")
    q.qmm_matvec_q4_0(wq_d, xq_d, y, N, K)
    torch.cuda.synchronize()
    wq = orc.quantize_q4_0_w(w)
    xq = orc.quantize_q8_0(x)
    assert np.array_equal(wq_d.cpu().numpy().reshape(wq.shape), wq)
    assert np.array_equal(xq_d.cpu().numpy().reshape(xq.shape), xq)
    ref = orc.matmul("q4_0", wq, xq, 1, N, K, threads=8, want=("y64", "mag"))
    _check(y.cpu().numpy(), ref["y64"][0], ref["mag"][0], "decode e2e")


def test_outputs_are_overwritten_not_accumulated(env):
    torch, q, orc = env
    N, K = 64, 256
    wq, xq = _inputs("q4_0", 1, N, K, 8000)
    y1 = _run_matvec(env, "q4_0", wq, xq, N, K)
    wd, xd = _dev(torch, wq), _dev(torch, xq)
    y = torch.full((N,), 1e30, dtype=torch.float32, device="cuda")
    q.qmm_matvec_q4_0(wd, xd, y, N, K)
    q.qmm_matvec_q4_0(wd, xd, y, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy(), y1)


@pytest.mark.parametrize("M", [40, 200])
@pytest.mark.parametrize("fmt", ["q4_0", "q5_1", "q2_k", "q4_k", "q6_k"])
def test_split_k_matmul_overwrites_and_is_deterministic(env, fmt, M):
    """A prefill launch of few tiles splits K in two and adds the halves into
    a zeroed output: calling it twice on a garbage-filled output gives the
    same bits each time (two addends sum the same in either order).  M = 40
    runs the 32-token tiles (Q4_0, Q5_1: K whole in four groups per
    workgroup and plain stores; the K-quants: K split, two groups) and M =
    200 the 128-token tiles (two groups for Q4_0 and Q5_1); the groups' sums
    are handed over through LDS in a fixed order."""
    torch, q, orc = env
    N, K = 1000, 4096
    _say("split-k repeat", fmt, M, N, K)
    wq, xq = _inputs(fmt, M, N, K, 8100)
    wd, xd = _dev(torch, wq), _dev(torch, xq)
    y = torch.full((M, N), 1e30, dtype=torch.float32, device="cuda")
    q.MATMUL[fmt](wd, xd, y, M, N, K)
    torch.cuda.synchronize()
    first = y.clone()
    for _ in range(3):
        y.fill_(float("nan"))
        q.MATMUL[fmt](wd, xd, y, M, N, K)
        q.MATMUL[fmt](wd, xd, y, M, N, K)
        torch.cuda.synchronize()
        assert torch.equal(y, first)
    ref = orc.matmul(fmt, wq, xq, M, N, K, threads=8, want=("y64", "mag"))
    _check(first.cpu().numpy(), ref["y64"], ref["mag"], (fmt, M, N, K))


@pytest.mark.parametrize("lpl,nw,nt", [(1, 4, 0), (4, 4, 1), (16, 8, 1), (2, 16, 0), (8, 16, 1)])
@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1025, 1 << 20, (28311552 // 16 + 3) * 16])
def test_peak_read_probe_reads_every_word(env, nbytes, lpl, nw, nt):
    """The streaming-read probe XORs every 32-bit word of the buffer, each
    workgroup its own span, ragged tails included, and writes nothing past
    its last workgroup."""
    from matmul_quantize_q8_amd import probe
    torch, q, _ = env
    _say("peak_read", nbytes, lpl, nw, nt)
    words = synth.splitmix64(101, 0, nbytes // 4).astype(np.uint32)
    buf = _dev(torch, words.view(np.int32))
    span = probe.read_span(lpl, nw)
    nchunk = -(-nbytes // span)
    sink = torch.full((nchunk + 1,), -1, dtype=torch.int32, device="cuda")
    probe.qmm_peak_read(buf, nbytes, sink, lpl, nw, bool(nt))
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    padded = np.zeros(nchunk * (span // 4), dtype=np.uint32)
    padded[:words.size] = words
    assert np.array_equal(got[:nchunk], np.bitwise_xor.reduce(padded.reshape(nchunk, span // 4), axis=1))
    assert got[nchunk] == 0xFFFFFFFF   # nothing written past the last workgroup


@pytest.mark.parametrize("wg,iters", [(1, 1), (3, 17), (512, 100)])
def test_peak_mfma_probe_sums(env, wg, iters):
    """Every lane of the int8 MFMA probe ends with 4 chains x 16 results x 32 x iters."""
    from matmul_quantize_q8_amd import probe
    torch, q, _ = env
    _say("peak_mfma", wg, iters)
    out = torch.full((wg * 256,), -1, dtype=torch.int32, device="cuda")
    probe.qmm_peak_mfma_i8(out, wg, iters)
    torch.cuda.synchronize()
    assert bool((out == 2048 * iters).all())


@pytest.mark.parametrize("mode,wps", [("fma", 1), ("mfma", 2), ("mixed", 2), ("fma_sgpr", 2)])
def test_issue_probe_results(env, mode, wps):
    """The issue-rate probe runs every iteration: 2048 * iters per lane when
    MFMAs run, 0 otherwise; the FMA chains' sums are finite."""
    from matmul_quantize_q8_amd import probe
    torch, q, _ = env
    iters = 37
    _say("probe_issue", mode, wps, iters)
    n = 256 * 256 * wps
    out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    outi = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    probe.qmm_probe_issue(mode, wps, iters, out, outi)
    torch.cuda.synchronize()
    assert bool((outi == (0 if mode.startswith("fma") else 2048 * iters)).all())
    assert bool(torch.isfinite(out).all())


def test_device_errors_are_reported(env):
    torch, q, _ = env
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    with pytest.raises(q.QmmError) as e:
        q.qmm_matvec_q4_0(buf, buf[4:], buf, 4, 64)
    assert e.value.code == "QMM_E_ALIGN"
    with pytest.raises(q.QmmError) as e:
        q.qmm_matmul_q2_k(buf, buf, buf, 1, 1, 100)
    assert e.value.code == "QMM_E_SHAPE"
    with pytest.raises(q.QmmError) as e:
        q.qmm_quantize_matvec_q4_0(buf, buf, buf[2:], buf, 4, 64)
    assert e.value.code == "QMM_E_ALIGN"
    with pytest.raises(q.QmmError) as e:
        q.qmm_quantize_matvec_q8_0(buf, buf, None, buf, 4, 48)
    assert e.value.code == "QMM_E_SHAPE"


def test_concurrent_calls_from_host_threads(env):
    """Calls are thread-safe: four host threads, each on a stream of its own,
    quantize, run a decode matvec and a prefill matmul at the same time, five
    times over; every output equals the same calls made alone on one stream,
    bit for bit (the kernels are deterministic and keep no state)."""
    import threading
    torch, q, orc = env
    N, K, M, reps = 1024, 4096, 40, 5
    _say("threads", N, K, M)
    w = synth.weights(N, K, config=1)
    xd = _dev(torch, synth.activations(M, K, config=4))
    fmts = ("q4_0", "q8_0", "q2_k", "q4_k")
    wq = {f: _dev(torch, orc.quantize_w(f, w)) for f in fmts}

    def job(f):
        act = "q8_k" if f in ("q2_k", "q4_k") else "q8_0"
        rb = q.row_bytes(act, K)
        xq = torch.empty(M * rb, dtype=torch.uint8, device="cuda")
        yv = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
        ym = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        (q.qmm_quantize_q8_k if act == "q8_k" else q.qmm_quantize_q8_0)(xd, xq, M, K)
        q.MATVEC[f](wq[f], xq[:rb], yv, N, K)
        q.MATMUL[f](wq[f], xq, ym, M, N, K)
        return xq, yv, ym

    ref = {f: job(f) for f in fmts}
    torch.cuda.synchronize()
    got, errors = {}, []
    start = threading.Barrier(len(fmts))

    def worker(f):
        try:
            s = torch.cuda.Stream()
            start.wait()
            with torch.cuda.stream(s):
                got[f] = [job(f) for _ in range(reps)]
            s.synchronize()
        except Exception as e:          # reported by the main thread
            errors.append((f, repr(e)))

    threads = [threading.Thread(target=worker, args=(f,)) for f in fmts]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for f in fmts:
        for rep, outs in enumerate(got[f]):
            for name, a, b in zip(("xq", "matvec", "matmul"), outs, ref[f]):
                assert torch.equal(a, b), (f, rep, name)


def test_graph_replay_matches_eager(env):
    """Decode and prefill launches captured into a HIP graph: every replay, with
    eager work and synchronizations in between, equals the eager result bit for
    bit (the kernels are deterministic and keep no state).  The products reach
    the 32-token tiles with K groups (M = 64: four for Q4_0, two with K split
    for the K-quants), the 128-token tile with two K groups and K split (M =
    100) and the few-token decode kernel (M = 4), each split launch with its
    fill kernel."""
    torch, q, orc = env
    N, K, M, M2, M3 = 1024, 4096, 64, 100, 4
    w = synth.weights(N, K, config=1)
    x = synth.activations(M, K, config=4)
    wq = _dev(torch, orc.quantize_q4_0_w(w))
    xd = _dev(torch, x)
    xq = torch.empty(M * q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    xq1 = torch.empty(q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    yv = torch.empty(N, dtype=torch.float32, device="cuda")
    yf = torch.empty(N, dtype=torch.float32, device="cuda")
    ym = torch.empty((M, N), dtype=torch.float32, device="cuda")
    x2 = _dev(torch, synth.activations(M2, K, config=5))
    xq2 = torch.empty(M2 * q.row_bytes("q8_0", K), dtype=torch.uint8, device="cuda")
    ym2 = torch.empty((M2, N), dtype=torch.float32, device="cuda")
    ym3 = torch.empty((M3, N), dtype=torch.float32, device="cuda")
    # the K-quant prefill kernels (dynamic LDS of up to 153 KB) in the same graph
    wk = {f: _dev(torch, orc.quantize_w(f, w)) for f in ("q2_k", "q4_k", "q6_k")}
    x8k = torch.empty(M * q.row_bytes("q8_k", K), dtype=torch.uint8, device="cuda")
    yk = {f: torch.empty((M, N), dtype=torch.float32, device="cuda") for f in wk}

    def work():
        q.qmm_quantize_q8_0(xd, xq, M, K)
        q.qmm_matvec_q4_0(wq, xq, yv, N, K)
        q.qmm_quantize_matvec_q4_0(wq, xd[1], xq1, yf, N, K)
        q.qmm_matmul_q4_0(wq, xq, ym, M, N, K)
        q.qmm_quantize_q8_0(x2, xq2, M2, K)
        q.qmm_matmul_q4_0(wq, xq2, ym2, M2, N, K)
        q.qmm_matmul_q4_0(wq, xq, ym3, M3, N, K)
        q.qmm_quantize_q8_k(xd, x8k, M, K)
        for f in wk:
            q.MATMUL[f](wk[f], x8k, yk[f], M, N, K)

    work()
    torch.cuda.synchronize()
    ref_v, ref_m, ref_q, ref_f, ref_q1 = yv.clone(), ym.clone(), xq.clone(), yf.clone(), xq1.clone()
    ref_m2, ref_m3 = ym2.clone(), ym3.clone()
    ref_k = {f: yk[f].clone() for f in yk}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        yv.fill_(float("nan"))
        yf.fill_(float("nan"))
        ym.fill_(float("nan"))
        ym2.fill_(float("nan"))
        ym3.fill_(float("nan"))
        for f in yk:
            yk[f].fill_(float("nan"))
        xq.zero_()
        xq1.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xq, ref_q), rep
        assert torch.equal(yv, ref_v), rep
        assert torch.equal(ym, ref_m), rep
        assert torch.equal(ym2, ref_m2), rep
        assert torch.equal(ym3, ref_m3), rep
        assert torch.equal(yf, ref_f), rep
        assert torch.equal(xq1, ref_q1), rep
        for f in yk:
            assert torch.equal(yk[f], ref_k[f]), (f, rep)
        work()                      # eager work between replays
        torch.cuda.synchronize()
