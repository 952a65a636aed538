"""Passes of 9 to 16 tokens (a verify step of up to 15 drafts plus one, or a
wider decode batch). For large Q8_0 matrices with fp16 activations (the
2 x 17408 x 5120 gate/up pair here) one weight stream serves all of them:
the wide kernels take the token count as a runtime value and keep the
per-(row, token) arithmetic of every other dense kernel. Smaller matrices,
Q4_0 and fp32 activations run passes of at most 8. Either way each token's
output is bitwise the one it gets when run alone.

Checked through the C ABI against the oracle and against the same tokens
run one at a time: the dense GEMV (Q8_0 and Q4_0, fp16 and fp32
activations, ragged row counts, 16/32/64-lane rows), the full-size gate+up
pair and SiLU pair (wide), a 12289 x 5120 matrix (wide, a ragged last row group),
fp16 output, and a K whose 16-token image does not fit the LDS.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import assert_parity, dev, host, note, require_gpu, threads, torch, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _bits(a):
    a = np.asarray(a)
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


@pytest.mark.parametrize("M,K,N,q4,xf32", [
    (5120, 5120, 9, False, False), (5120, 5120, 16, False, False), (12289, 5120, 13, False, False),
    (1001, 2048, 12, False, True), (300, 96, 16, False, False), (77, 768, 13, False, False), (4096, 4096, 16, True, False),
    (517, 1024, 11, True, True), (1, 5120, 16, False, False)])
def test_wide_gemv_parity_and_n_invariance(M, K, N, q4, xf32):
    note(f"wide gemv {M}x{K} N={N} q4={q4} xf32={xf32}")
    rng = np.random.default_rng(M + K + N)
    q, d = (synth.draw_weights_q4_0 if q4 else synth.draw_weights)(rng, M, K)
    x = synth.draw_x(rng, N, K)
    if xf32:
        x = x.astype(np.float32)
    W = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q, d)) if q4 else upload(q, d)
    y = host(q8.gemv(W, dev(x)))
    ref, A = oracle.gemv(q, d, x, threads())
    assert_parity(y, ref, A, what=f"wide N={N}")
    for n in range(N):
        y1 = host(q8.gemv(W, dev(x[n:n + 1])))
        assert np.array_equal(_bits(y1[0]), _bits(y[n])), f"token {n}"


def test_wide_fp16_output():
    note("wide gemv fp16 y")
    rng = np.random.default_rng(9)
    q, d = synth.draw_weights(rng, 700, 5120)
    x = synth.draw_x(rng, 10, 5120)
    W = upload(q, d)
    y = host(q8.gemv(W, dev(x), out_dtype=torch.float16))
    ref, A = oracle.gemv(q, d, x, threads())
    assert_parity(y, ref, A, out_dtype="f16", what="wide fp16")
    y32 = host(q8.gemv(W, dev(x)))
    assert np.array_equal(_bits(y), _bits(y32.astype(np.float16)))


def test_wide_pass_split_when_the_image_does_not_fit():
    """K = 12288 fp16: fewer than 16 tokens fit the LDS, so 16 tokens run as
    several passes; every token still equals its one-token result."""
    note("wide gemv K=12288 N=16")
    rng = np.random.default_rng(12)
    q, d = synth.draw_weights(rng, 256, 12288)
    x = synth.draw_x(rng, 16, 12288)
    W = upload(q, d)
    y = host(q8.gemv(W, dev(x)))
    ref, A = oracle.gemv(q, d, x, threads())
    assert_parity(y, ref, A, what="K=12288 N=16")
    for n in (0, 9, 15):
        assert np.array_equal(_bits(host(q8.gemv(W, dev(x[n:n + 1])))[0]), _bits(y[n]))


@pytest.fixture(scope="module")
def full_pair():
    c = synth.pair_case(17408, 5120, 16, seed=0)
    return c, upload(c.qa, c.da), upload(c.qb, c.db)


def _rows(seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, 17407], rng.choice(17408, 1500, replace=False)]))


@pytest.mark.parametrize("N", [9, 16])
def test_wide_full_pair(full_pair, N):
    note(f"wide pair 17408x5120 N={N}")
    c, Wa, Wb = full_pair
    x = c.x[:N]
    ya, yb = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x)))
    rows = _rows(N)
    for q, d, y in ((c.qa, c.da, ya), (c.qb, c.db, yb)):
        ref, A = oracle.gemv_rows(q, d, x, rows, threads())
        assert_parity(y[:, rows], ref, A, what=f"pair N={N}")
    for n in (0, N // 2, N - 1):
        a1, b1 = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x[n:n + 1])))
        assert np.array_equal(_bits(a1[0]), _bits(ya[n])), f"gate token {n}"
        assert np.array_equal(_bits(b1[0]), _bits(yb[n])), f"up token {n}"


@pytest.mark.parametrize("N", [9, 16])
def test_wide_full_silu_pair(full_pair, N):
    note(f"wide SiLU pair 17408x5120 N={N}")
    c, Wa, Wb = full_pair
    x = c.x[:N]
    h = host(q8.gemv_pair_silu(Wa, Wb, dev(x)))
    rows = _rows(100 + N)
    r = oracle.gate_up_silu(c.qa[rows], c.da[rows], c.qb[rows], c.db[rows], x, threads())
    bad = np.abs(h[:, rows] - r["h"]) > r["bh"]
    assert not bad.any(), f"{bad.sum()} outputs outside the propagated bound"
    for n in (0, N - 1):
        h1 = host(q8.gemv_pair_silu(Wa, Wb, dev(x[n:n + 1])))
        assert np.array_equal(_bits(h1[0]), _bits(h[n])), f"token {n}"


@pytest.mark.parametrize("M,K,N", [(129, 160, 16), (300, 768, 9), (1000, 2048, 14)])
def test_wide_small_silu_pairs(M, K, N):
    """16-, 32- and 64-lane rows of the SiLU pair at 9..16 tokens."""
    note(f"wide SiLU pair {M}x{K} N={N}")
    rng = np.random.default_rng(M * K + N)
    qg, dg = synth.draw_weights(rng, M, K)
    qu, du = synth.draw_weights(rng, M, K)
    x = synth.draw_x(rng, N, K)
    Wg, Wu = upload(qg, dg), upload(qu, du)
    h = host(q8.gemv_pair_silu(Wg, Wu, dev(x)))
    r = oracle.gate_up_silu(qg, dg, qu, du, x, threads())
    bad = np.abs(h - r["h"]) > r["bh"]
    assert not bad.any(), f"{bad.sum()} outputs outside the propagated bound"
    for n in range(N):
        h1 = host(q8.gemv_pair_silu(Wg, Wu, dev(x[n:n + 1])))
        assert np.array_equal(_bits(h1[0]), _bits(h[n])), f"token {n}"
