"""Several passes of one call in one launch. Where the 9..16-token kernel
does not apply, every full pass (up to 8 tokens, fewer when the x image of
8 would not fit the LDS) runs as one slice of a single grid: the one-group
kernels of 4 or more tokens take their pass from the workgroup's y index
and shift x and every output by it. Shapes the one-group kernel does not
take fall back to one launch per pass inside the library.

Checked through the C ABI, each token against the oracle bound and bitwise
against the same token run alone: the dense GEMV (fp16 and fp32 x, fp32
and fp16 y, 2-4 slices plus a ragged last pass), the pair (two outputs
shifted per pass; Q8_0 and Q4_0), the SiLU pair, passes of 5 tokens set by
the LDS, a shape that falls back, and the shared expert (h, the gate dots
and the gated add all shifted per pass; Q8_0 with fp16 or fp32 x, Q4_0).
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


@pytest.mark.parametrize("M,K,N,xf32,yf16", [
    (1000, 2048, 24, False, False),   # three slices of 8
    (700, 4096, 19, True, True),      # two slices of 8 + 3, fp32 x, fp16 y
    (256, 16384, 12, False, False),   # the LDS holds 5 tokens: 5 + 5 + 2
    (200, 160, 20, False, False),     # ten chunks a row: no one-group kernel, a launch per pass
])
def test_sliced_gemv(M, K, N, xf32, yf16):
    note(f"sliced gemv {M}x{K} N={N} xf32={xf32} yf16={yf16}")
    rng = np.random.default_rng(M + K + N)
    q, d = synth.draw_weights(rng, M, K)
    x = synth.draw_x(rng, N, K)
    if xf32:
        x = x.astype(np.float32)
    W = upload(q, d)
    kw = {"out_dtype": torch.float16} if yf16 else {}
    y = host(q8.gemv(W, dev(x), **kw))
    ref, A = oracle.gemv(q, d, x, threads())
    assert_parity(y, ref, A, out_dtype="f16" if yf16 else "f32", what=f"sliced N={N}")
    for n in range(N):
        y1 = host(q8.gemv(W, dev(x[n:n + 1]), **kw))
        assert np.array_equal(_bits(y1[0]), _bits(y[n])), f"token {n}"


@pytest.mark.parametrize("q4", [False, True])
def test_sliced_pair(q4):
    note(f"sliced pair 600+400 x 1024 N=16 q4={q4}")
    rng = np.random.default_rng(5)
    draw = synth.draw_weights_q4_0 if q4 else synth.draw_weights
    qa, da = draw(rng, 600, 1024)
    qb, db = draw(rng, 400, 1024)
    x = synth.draw_x(rng, 16, 1024)
    pack = (lambda q, d: q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q, d))) if q4 else upload
    Wa, Wb = pack(qa, da), pack(qb, db)
    ya, yb = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x)))
    for q, d, y in ((qa, da, ya), (qb, db, yb)):
        ref, A = oracle.gemv(q, d, x, threads())
        assert_parity(y, ref, A, what="sliced pair")
    for n in (0, 7, 8, 15):
        a1, b1 = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x[n:n + 1])))
        assert np.array_equal(_bits(a1[0]), _bits(ya[n])), f"a token {n}"
        assert np.array_equal(_bits(b1[0]), _bits(yb[n])), f"b token {n}"


def test_sliced_silu_pair():
    note("sliced SiLU pair 500x2048 N=20")
    rng = np.random.default_rng(6)
    qg, dg = synth.draw_weights(rng, 500, 2048)
    qu, du = synth.draw_weights(rng, 500, 2048)
    x = synth.draw_x(rng, 20, 2048)
    Wg, Wu = upload(qg, dg), upload(qu, du)
    h = host(q8.gemv_pair_silu(Wg, Wu, dev(x)))
    r = oracle.gate_up_silu(qg, dg, qu, du, x, threads())
    bad = np.abs(h - r["h"]) > r["bh"]
    assert not bad.any(), f"{bad.sum()} outputs outside the propagated bound"
    for n in (0, 9, 16, 19):
        h1 = host(q8.gemv_pair_silu(Wg, Wu, dev(x[n:n + 1])))
        assert np.array_equal(_bits(h1[0]), _bits(h[n])), f"token {n}"


@pytest.mark.parametrize("T,xf32,q4", [(24, False, False), (20, True, False), (16, False, True)])
def test_sliced_shared_expert(T, xf32, q4):
    note(f"sliced shared expert T={T} xf32={xf32} q4={q4}")
    F, H = 768, 2048
    rng = np.random.default_rng(T)
    draw = synth.draw_weights_q4_0 if q4 else synth.draw_weights
    qg, dg = draw(rng, F, H)
    qu, du = draw(rng, F, H)
    qd, dd = draw(rng, H, F)
    qs, ds = draw(rng, 1, H)
    x = synth.draw_x(rng, T, H)
    if xf32:
        x = x.astype(np.float32)
    base = rng.standard_normal((T, H)).astype(np.float32)
    pack = (lambda q, d: q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q, d))) if q4 else upload
    mats = tuple(pack(a, b) for a, b in ((qg, dg), (qu, du), (qd, dd), (qs, ds)))
    out = dev(base.copy())
    q8.moe_shared_expert(*mats, dev(x), out)
    got = host(out)
    r = oracle.shared_expert(qg, dg, qu, du, qd, dd, qs, ds, x, base, threads=threads())
    err = np.abs(got.astype(np.float64) - r["out"])
    assert np.all(err <= r["bound"]), f"max excess {np.max(err - r['bound']):.3e}"
    for n in (0, 8, T - 1):
        one = dev(base[n:n + 1].copy())
        q8.moe_shared_expert(*mats, dev(x[n:n + 1].copy()), one)
        assert np.array_equal(host(one).view(np.uint32), got[n:n + 1].view(np.uint32)), f"token {n}"
