"""Parity of the Q4_0 GEMV (q8_gemv_q4_0) with the oracle.

Hand-built GGUF Q4_0 blocks (tests/golden/q4_0_handbuilt.txt) must come
out bitwise equal to their hand-derived results; random Q4_0 matrices
(q uniform in -8..7, d = |N(0, 0.02)|/8, x ~ N(0,1)) must be within
1e-3 * sum|d*q*x| of the fp64 oracle, over ragged shapes, every lane
width, fp16/fp32 activations, fp16 output and multi-pass N; token n's
result must be bitwise independent of N and of the other tokens.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.golden_io import load_handbuilt
from tests.gpu_util import assert_parity, dev, host, note, require_gpu, threads, torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def upload_q4(q, d):
    return q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q, d))


@pytest.mark.parametrize("case", load_handbuilt("q4_0_handbuilt.txt", 18), ids=lambda c: c["name"])
def test_golden_handbuilt_bitwise(case):
    note(f"q4 golden {case['name']}")
    y = host(q8.gemv_q4_0(q8.pack_q4_0(case["blocks"]), dev(case["x"])))
    assert np.array_equal(y.astype(np.float64), case["y"]), case["why"]


SHAPES = [(1024, 1024, 1), (1000, 96, 3), (333, 2048, 4), (517, 768, 8), (64, 32, 2),
          (129, 800, 5), (2050, 5120, 2), (7, 160, 9), (1, 1024, 1), (300, 4096, 16)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_random_parity(M, K, N):
    note(f"q4 random M={M} K={K} N={N}")
    c = synth.q4_0_case(M, K, N, seed=M + K + N)
    y = host(q8.gemv_q4_0(upload_q4(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y, ref, A, what=f"q4 {M}x{K} N={N}")


def test_full_5120_n1_and_pair_shape():
    note("q4 5120x5120 N=1 and 17408x5120 N=4 (sampled rows)")
    c = synth.q4_0_case(5120, 5120, 1, seed=0)
    y = host(q8.gemv_q4_0(upload_q4(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y, ref, A, what="q4 5120")
    c = synth.q4_0_case(17408, 5120, 4, seed=1)
    y = host(q8.gemv_q4_0(upload_q4(c.q, c.d), dev(c.x)))
    rows = np.unique(np.concatenate([[0, 17407], np.random.default_rng(0).choice(17408, 1500)]))
    ref, A = oracle.gemv_rows(c.q, c.d, c.x, rows, threads())
    assert_parity(y[:, rows], ref, A, what="q4 17408 N=4")


@pytest.mark.parametrize("M,K", [(513, 1024), (64, 96)])
def test_fp16_output_and_fp32_activations(M, K):
    note(f"q4 fp16 out / fp32 x M={M} K={K}")
    c = synth.q4_0_case(M, K, 3, seed=M)
    W = upload_q4(c.q, c.d)
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    y16 = host(q8.gemv_q4_0(W, dev(c.x), out_dtype=torch.float16))
    assert_parity(y16.astype(np.float64), ref, A, out_dtype="f16", what="q4 fp16 out")
    x32 = c.x.astype(np.float32)
    y = host(q8.gemv_q4_0(W, dev(x32)))
    ref32, A32 = oracle.gemv(c.q, c.d, x32, threads())
    assert_parity(y, ref32, A32, what="q4 fp32 x")


@pytest.mark.parametrize("K", [5120, 768, 96])
def test_n_invariance_bitwise(K):
    note(f"q4 N invariance K={K}")
    c = synth.q4_0_case(777, K, 16, seed=K)
    W = upload_q4(c.q, c.d)
    x = dev(c.x)
    solo = np.stack([host(q8.gemv_q4_0(W, x[n:n + 1]))[0] for n in range(16)])
    for N in (2, 3, 5, 8, 9, 16):
        yN = host(q8.gemv_q4_0(W, x[:N].contiguous()))
        assert np.array_equal(yN.view(np.uint32), solo[:N].view(np.uint32)), f"N={N}"


def test_extreme_nibbles_and_scales_bitwise():
    """Every weight -8 or 7 with d = 1 and integer activations: exact sums."""
    note("q4 extreme nibbles")
    K, M = 256, 64
    rng = np.random.default_rng(4)
    q = np.where(rng.random((M, K)) < 0.5, -8, 7).astype(np.int8)
    d = np.ones((M, K // 32), np.float16)
    x = rng.integers(-3, 4, size=(2, K)).astype(np.float16)
    y = host(q8.gemv_q4_0(upload_q4(q, d), dev(x)))
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ q.astype(np.float64).T)
