"""Parity of q8_gemv (HIP, gfx950) with the CPU oracle.

Bit-exact where the mathematics makes the result exact (hand-built golden
blocks, unit vectors over every int8 value, subnormal scales and
activations, integer-valued data); otherwise every output within
1e-3 * sum|d*q*x| of the fp64 oracle. Also: N-invariance (token n's output
is bitwise the same for every N, the pages' verify == plain decode
contract), repeat-call determinism, ragged shapes spanning several row
groups, fp16 outputs, fp32 activations, multi-pass N > 8.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.golden_io import load_handbuilt
from tests.gpu_util import assert_parity, dev, host, note, require_gpu, threads, torch, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("case", load_handbuilt(), ids=lambda c: c["name"])
def test_golden_handbuilt_bitwise(case):
    note(f"golden {case['name']}")
    W = q8.pack(case["blocks"])
    y = host(q8.gemv(W, dev(case["x"])))
    assert np.array_equal(y.astype(np.float64), case["y"]), (case["why"], y)


@pytest.mark.parametrize("K,j", [(96, 0), (96, 31), (96, 95), (1024, 17), (5120, 5119), (768, 400)])
def test_unit_vector_every_int8_bitwise(K, j):
    note(f"unit vector K={K} j={j}")
    rng = np.random.default_rng(K + j)
    q = rng.integers(-128, 128, size=(256, K)).astype(np.int8)
    q[:, j] = np.arange(256) - 128
    d = np.full((256, K // 32), 1.0, np.float16)
    x = np.zeros((1, K), np.float16)
    x[0, j] = 1.0
    y = host(q8.gemv(upload(q, d), dev(x)))
    assert np.array_equal(y[0], (np.arange(256) - 128).astype(np.float32))


@pytest.mark.parametrize("M,N", [(256, 4), (256, 8), (40000, 4), (40000, 8)])
def test_unit_vectors_every_int8_batched_bitwise(M, N):
    """Every int8 value through the batched conversions: 5120-wide rows at
    4 and 8 tokens take the SDWA byte converts (the one-group kernel for 256
    rows, the persistent one for 40000). Token n reads column j_n alone, so
    y[n][m] = q[m][j_n] exactly, and column j_n holds all 256 values."""
    K = 5120
    note(f"unit vectors every int8 M={M} N={N}")
    rng = np.random.default_rng(M + N)
    q = np.tile(rng.integers(-128, 128, size=(251, K)).astype(np.int8), (M // 251 + 1, 1))[:M]
    cols = rng.choice(K, size=N, replace=False)
    x = np.zeros((N, K), np.float16)
    for n, j in enumerate(cols):
        q[:, j] = ((np.arange(M) + 37 * n) % 256 - 128).astype(np.int8)
        x[n, j] = 1.0
    d = np.full((M, K // 32), 1.0, np.float16)
    y = host(q8.gemv(upload(q, d), dev(x)))
    for n, j in enumerate(cols):
        assert np.array_equal(y[n], q[:, j].astype(np.float32)), f"token {n}"


def test_subnormal_scale_and_activation_bitwise():
    note("subnormals")
    K = 64
    q = np.zeros((3, K), np.int8)
    q[0, 40] = 127
    q[1, 3] = -128
    q[2, 7] = 100
    d = np.array([[0x3C00, 0x0001], [0x0001, 0x3C00], [0x03FF, 0x3C00]], np.uint16).view(np.float16)
    x = np.zeros((2, K), np.float16)
    x[0, 40] = 1.0
    x[0, 7] = np.uint16(0x0001).view(np.float16)
    x[1, 3] = np.uint16(0x0001).view(np.float16)
    y = host(q8.gemv(upload(q, d), dev(x)))
    ref, _ = oracle.gemv(q, d, x)
    assert y[0, 0] == np.float32(127 * 2.0 ** -24)
    assert y[0, 2] == np.float32(100 * 2.0 ** -24 * (1023 * 2.0 ** -24))
    assert np.array_equal(y.astype(np.float64), ref.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("M,K,N", [(24, 640, 3), (1000, 96, 2), (37, 5120, 8), (300, 768, 5),
                                   (64, 800, 1), (5, 32, 11)])
def test_integer_exact_bitwise(M, K, N):
    """x integer in [-8, 8], d = 2^e: every fp32 partial sum is exact."""
    note(f"integer exact M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 31 + K + N)
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    xi = rng.integers(-8, 9, size=(N, K))
    d = np.full((M, K // 32), 2.0 ** -5, np.float16)
    y = host(q8.gemv(upload(q, d), dev(xi.astype(np.float16))))
    ref = (q.astype(np.int64) @ xi.T.astype(np.int64)).T * 2.0 ** -5
    assert np.array_equal(y.astype(np.float64), ref)


SHAPES = [(1024, 1024, 1), (1000, 96, 3), (333, 2048, 4), (517, 768, 8), (64, 32, 2),
          (129, 800, 5), (2050, 5120, 2), (7, 160, 9), (1, 1024, 1), (600, 1024, 12),
          (300, 2048, 16)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_random_parity(M, K, N):
    note(f"random parity M={M} K={K} N={N}")
    c = synth.gemv_case(M, K, N, seed=M + K + N)
    y = host(q8.gemv(upload(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y, ref, A, what=f"{M}x{K} N={N}")


@pytest.mark.parametrize("M,K,N", [(300, 5120, 3), (1000, 768, 1), (64, 96, 8)])
def test_zero_blocks_in_random_rows(M, K, N):
    """Zero blocks inside random rows (scale 0, quants 0, or both) and an
    all-zero row: within the bound of the oracle, the zero row exactly 0,
    and the result does not depend on how a block is zero (each such block
    adds exactly nothing to its lane's sum), bitwise."""
    note(f"zero blocks {M}x{K} N={N}")
    rng = np.random.default_rng(M + K)
    q, d = synth.draw_weights(rng, M, K)
    x = synth.draw_x(rng, N, K)
    nb = K // 32
    zero = rng.random((M, nb)) < 0.25
    zero[M // 2] = True  # an all-zero row
    variants = []
    for how in ("d", "q", "both"):
        qv, dv = q.copy(), d.copy()
        for m, b in zip(*np.nonzero(zero)):
            if how in ("d", "both"):
                dv[m, b] = 0.0
            if how in ("q", "both"):
                qv[m, b * 32:(b + 1) * 32] = 0
        y = host(q8.gemv(upload(qv, dv), dev(x)))
        ref, A = oracle.gemv(qv, dv, x, threads())
        assert_parity(y, ref, A, what=f"zero blocks ({how})")
        assert np.all(y[:, M // 2] == 0)
        variants.append(y)
    assert np.array_equal(variants[0].view(np.uint32) & 0x7FFFFFFF, variants[1].view(np.uint32) & 0x7FFFFFFF)
    assert np.array_equal(variants[1].view(np.uint32), variants[2].view(np.uint32))


def test_config_5120_n1_full():
    note("5120x5120 N=1 full oracle")
    c = synth.gemv_case(5120, 5120, 1, seed=0)
    y = host(q8.gemv(upload(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    rel = assert_parity(y, ref, A, what="5120x5120")
    assert rel < 1e-4


def test_config_1024_n1_full():
    note("1024x1024 N=1 full oracle")
    c = synth.gemv_case(1024, 1024, 1, seed=0)
    y = host(q8.gemv(upload(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y, ref, A, what="1024x1024")


@pytest.mark.parametrize("M,K", [(700, 5120), (300, 768), (129, 96)])
def test_fp16_output(M, K):
    note(f"fp16 y M={M} K={K}")
    c = synth.gemv_case(M, K, 3, seed=5)
    W = upload(c.q, c.d)
    y16 = host(q8.gemv(W, dev(c.x), out_dtype=torch.float16))
    y32 = host(q8.gemv(W, dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y16, ref, A, out_dtype="f16", what="fp16 y")
    assert np.array_equal(y16, y32.astype(np.float16))  # fp16 y is RNE of the fp32 result


@pytest.mark.parametrize("M,K,N", [(300, 768, 3), (200, 5120, 1), (64, 96, 8)])
def test_fp32_activations(M, K, N):
    note(f"fp32 x M={M} K={K} N={N}")
    c = synth.gemv_case(M, K, 1, seed=9)
    x = np.random.default_rng(3).normal(0, 1, size=(N, K)).astype(np.float32)
    y = host(q8.gemv(upload(c.q, c.d), dev(x)))
    ref, A = oracle.gemv(c.q, c.d, x, threads())
    assert_parity(y, ref, A, what="fp32 x")


@pytest.mark.parametrize("K", [5120, 768, 96, 2048])
def test_n_invariance_bitwise(K):
    """Token n's output is bitwise the same whatever N and the other tokens."""
    note(f"N invariance K={K}")
    M = 777
    c = synth.gemv_case(M, K, 16, seed=K)
    W = upload(c.q, c.d)
    x = dev(c.x)
    solo = np.stack([host(q8.gemv(W, x[n:n + 1]))[0] for n in range(16)])
    for N in (2, 3, 4, 5, 6, 7, 8, 9, 16):
        yN = host(q8.gemv(W, x[:N].contiguous()))
        assert np.array_equal(yN.view(np.uint32), solo[:N].view(np.uint32)), f"N={N}"
    # other tokens' values do not leak into token 0
    x2 = x.clone()
    x2[1:] = -x2[1:]
    assert np.array_equal(host(q8.gemv(W, x2[:8].contiguous()))[0].view(np.uint32),
                          solo[0].view(np.uint32))


def test_repeat_calls_are_deterministic():
    note("determinism")
    c = synth.gemv_case(3000, 2048, 4, seed=1)
    W = upload(c.q, c.d)
    x = dev(c.x)
    first = host(q8.gemv(W, x))
    for _ in range(5):
        assert np.array_equal(host(q8.gemv(W, x)).view(np.uint32), first.view(np.uint32))


def test_outputs_fully_written_and_no_overrun():
    """Canary bands around y stay untouched; every output is written."""
    note("canary bands")
    c = synth.gemv_case(517, 768, 3, seed=2)
    W = upload(c.q, c.d)
    buf = torch.full((3 * 517 + 2048,), float("nan"), device="cuda")
    y = buf[1024:1024 + 3 * 517].view(3, 517)
    q8.gemv(W, dev(c.x), out=y)
    b = host(buf)
    assert np.all(np.isnan(b[:1024])) and np.all(np.isnan(b[1024 + 3 * 517:]))
    assert not np.any(np.isnan(b[1024:1024 + 3 * 517]))


def test_stream_argument_is_used():
    note("side stream")
    c = synth.gemv_case(256, 1024, 2, seed=4)
    W = upload(c.q, c.d)
    x = dev(c.x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = q8.gemv(W, x)
    s.synchronize()
    ref, A = oracle.gemv(c.q, c.d, c.x)
    assert_parity(host(y), ref, A, what="side stream")
