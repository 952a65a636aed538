"""The GEMV launch in which every wave owns one row group.

For passes of 1 to 4 tokens, when the row groups fit in the resident
waves and a row is a whole number of lane steps, q8_gemv runs a kernel
whose chunk loop is fixed at compile time. Its arithmetic per (row, token)
is the persistent engine's, so its outputs for N = 1..4 must be bitwise
equal to the first tokens of an N = 5 call (which takes the persistent
engine) and within 1e-3 * sum|d*q*x| of the fp64 oracle. Shapes cover 16-, 32- and 64-lane rows, 1 to 16 chunks per
lane, row counts that leave the last row group partly empty, Q4_0, fp32
activations, fp16 outputs, the two-matrix pair, and canary bands.
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


# (M, K): lanes per row and chunks per lane in the comments (Q8_0: C = K/16)
SHAPES = [
    (1001, 768),   # 16 lanes, 3 chunks, 4 rows per wave, last group 1 row
    (333, 1536),   # 32 lanes, 3 chunks, 2 rows per wave, last group 1 row
    (5119, 5120),  # 64 lanes, 5 chunks
    (77, 1024),    # 64 lanes, 1 chunk
    (250, 2048),   # 2 chunks
    (130, 7168),   # 7 chunks
    (64, 8192),    # 8 chunks
    (40, 16384),   # 16 chunks
    (513, 3584),   # 32 lanes, 7 chunks
    (96, 2560),    # 32 lanes, 5 chunks
]


def check(W, q, d, x, what):
    y5 = host(q8.gemv(W, dev(x[:5])))
    for n in (1, 2, 3, 4):
        yn = host(q8.gemv(W, dev(x[:n])))
        assert np.array_equal(yn.view(np.uint32), y5[:n].view(np.uint32)), f"{what}: N={n} vs N=5"
    ref, A = oracle.gemv(q, d, x[:4], threads())
    assert_parity(y5[:4], ref, A, what=what)


@pytest.mark.parametrize("M,K", SHAPES)
def test_q8_shapes_match_engine_and_oracle(M, K):
    note(f"single-group q8 M={M} K={K}")
    c = synth.gemv_case(M, K, 5, seed=M * 7 + K)
    check(upload(c.q, c.d), c.q, c.d, c.x, f"{M}x{K}")


@pytest.mark.parametrize("M,K", [(1001, 5120), (300, 2048), (45, 4096)])
def test_q4_shapes_match_engine_and_oracle(M, K):
    note(f"single-group q4 M={M} K={K}")
    c = synth.q4_0_case(M, K, 5, seed=M + K)
    W = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(c.q, c.d))
    check(W, c.q, c.d, c.x, f"q4 {M}x{K}")


def test_fp32_activations_and_fp16_output():
    note("single-group fp32 x / fp16 y")
    c = synth.gemv_case(333, 1536, 5, seed=5)
    W = upload(c.q, c.d)
    x32 = c.x.astype(np.float32)
    check(W, c.q, c.d, x32, "fp32 x")
    y16 = host(q8.gemv(W, dev(c.x[:1]), out_dtype=torch.float16))
    ref, A = oracle.gemv(c.q, c.d, c.x[:1], threads())
    assert_parity(y16.astype(np.float64), ref, A, out_dtype="f16", what="fp16 y")


def test_pair_rows_of_both_matrices():
    note("single-group pair")
    rng = np.random.default_rng(9)
    qa, da = synth.draw_weights(rng, 301, 2048)
    qb, db = synth.draw_weights(rng, 77, 2048)
    x = synth.draw_x(rng, 5, 2048)
    Wa, Wb = upload(qa, da), upload(qb, db)
    ya5, yb5 = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x)))
    for n in (1, 3):
        ya, yb = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x[:n])))
        assert np.array_equal(ya.view(np.uint32), ya5[:n].view(np.uint32))
        assert np.array_equal(yb.view(np.uint32), yb5[:n].view(np.uint32))
    for q, d, y in ((qa, da, ya5), (qb, db, yb5)):
        ref, A = oracle.gemv(q, d, x, threads())
        assert_parity(y, ref, A, what="pair")


@pytest.mark.parametrize("M,K", [(1001, 768), (5119, 5120), (333, 1536)])
def test_canary_bands(M, K):
    """Rows past the end are read from the last row and never written."""
    note(f"single-group canary M={M} K={K}")
    c = synth.gemv_case(M, K, 3, seed=3)
    W = upload(c.q, c.d)
    buf = torch.full((3 * M + 4096,), float("nan"), device="cuda")
    y = buf[2048:2048 + 3 * M].view(3, M)
    q8.gemv(W, dev(c.x), out=y)
    b = host(buf)
    assert np.all(np.isnan(b[:2048])) and np.all(np.isnan(b[2048 + 3 * M:]))
    assert not np.any(np.isnan(b[2048:2048 + 3 * M]))


# ---------------------------------------------------------------- streaming launches
# More row groups than resident waves: at 1-2 tokens the one-group kernel is
# launched over every group anyway (the hardware starts workgroups as others
# finish); results must equal the persistent launch's (token 0/1 of N = 5).
def sampled_rows(M, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], rng.choice(M, 600, replace=False)]))


@pytest.mark.parametrize("fmt", ["q8", "q4"])
def test_streaming_dense(fmt):
    note(f"streaming dense {fmt}")
    M, K = 40000, 2048
    if fmt == "q8":
        c = synth.gemv_case(M, K, 5, seed=31)
        W = upload(c.q, c.d)
    else:
        c = synth.q4_0_case(M, K, 5, seed=31)
        W = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(c.q, c.d))
    y5 = host(q8.gemv(W, dev(c.x)))
    for n in (1, 2):
        yn = host(q8.gemv(W, dev(c.x[:n])))
        assert np.array_equal(yn.view(np.uint32), y5[:n].view(np.uint32)), f"N={n}"
    rows = sampled_rows(M, 1)
    ref, A = oracle.gemv_rows(c.q, c.d, c.x[:2], rows, threads())
    assert_parity(y5[:2, rows], ref, A, what=f"streaming {fmt}")


def test_streaming_silu_pair():
    note("streaming SiLU pair")
    M, K = 20000, 2048
    rng = np.random.default_rng(32)
    qg, dg = synth.draw_weights(rng, M, K)
    qu, du = synth.draw_weights(rng, M, K)
    x = synth.draw_x(rng, 5, K)
    Wg, Wu = upload(qg, dg), upload(qu, du)
    h5 = host(q8.gemv_pair_silu(Wg, Wu, dev(x)))
    for n in (1, 2):
        hn = host(q8.gemv_pair_silu(Wg, Wu, dev(x[:n])))
        assert np.array_equal(hn.view(np.uint32), h5[:n].view(np.uint32)), f"N={n}"
    rows = sampled_rows(M, 2)
    r = oracle.gate_up_silu(qg[rows], dg[rows], qu[rows], du[rows], x[:2], threads())
    assert np.all(np.abs(h5[:2, rows] - r["h"]) <= r["bh"])


@pytest.mark.parametrize("M,K,q4,xf32", [(768, 2048, False, False), (1408, 1024, True, False),
                                         (300, 96, False, True), (768, 2048, False, True),
                                         (256, 512, False, True), (512, 1024, True, True)])
def test_silu_pair_resident_3_to_8_tokens(M, K, q4, xf32):
    """The SiLU pair's one-group kernel at 3-8 tokens (taken when every
    group fits the resident waves): each token's h is bitwise its one-token
    result, and all of h is within the oracle's propagated bound."""
    note(f"one-group SiLU pair {M}x{K} q4={q4} xf32={xf32} N=3..8")
    rng = np.random.default_rng(M + K)
    draw = synth.draw_weights_q4_0 if q4 else synth.draw_weights
    qg, dg = draw(rng, M, K)
    qu, du = draw(rng, M, K)
    x = synth.draw_x(rng, 8, K)
    if xf32:
        x = x.astype(np.float32)
    if q4:
        Wg = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(qg, dg))
        Wu = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(qu, du))
    else:
        Wg, Wu = upload(qg, dg), upload(qu, du)
    singles = [host(q8.gemv_pair_silu(Wg, Wu, dev(x[n:n + 1])))[0] for n in range(8)]
    r = oracle.gate_up_silu(qg, dg, qu, du, x, threads())
    for N in range(3, 9):
        h = host(q8.gemv_pair_silu(Wg, Wu, dev(x[:N])))
        for n in range(N):
            assert np.array_equal(h[n].view(np.uint32), singles[n].view(np.uint32)), (N, n)
        assert np.all(np.abs(h - r["h"][:N]) <= r["bh"][:N]), f"N={N}"
