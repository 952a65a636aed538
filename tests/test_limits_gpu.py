"""The largest K each entry point takes, and the first one it refuses.

A pass's activations sit in the LDS of one workgroup (160 KiB on MI355X),
which bounds K per entry point: the dense GEMV and the pair at K = 81920
with fp16 x and 40960 with fp32 x (one token per pass, so N = 2 runs as two
passes); the LM head at 81408 (its fused kernel keeps 1 KiB of its own) at
N = 1 and 3; the routed GEMV at 20352 with fp16 x and 10176 with fp32 x;
the routed FFN with F = 10176 (its down projection reads fp32 h). At each
limit every output is checked against the oracle (the LM head's ids are the
planted rows, and the oracle's gate confirms them); 32 past it the call is
refused with Q8_ERR_SHAPE before anything is launched.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import (assert_parity, dev, host, note, require_gpu, threads, upload,
                            upload_bank)

pytestmark = pytest.mark.gpu

SHAPE = -2  # Q8_ERR_SHAPE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()  # gfx950: 160 KiB of LDS per workgroup


def _refused(fn):
    with pytest.raises(q8.Q8Error) as e:
        fn()
    assert e.value.status == SHAPE, str(e.value)


@pytest.mark.parametrize("K,xf32,M", [(81920, False, 700), (40960, True, 500)])
def test_gemv_at_the_largest_k(K, xf32, M):
    note(f"gemv at K={K} xf32={xf32}")
    c = synth.gemv_case(M, K, 2, seed=K)
    x = c.x.astype(np.float32) if xf32 else c.x
    W = upload(c.q, c.d)
    y = host(q8.gemv(W, dev(x)))
    ref, A = oracle.gemv(c.q, c.d, x, threads())
    assert_parity(y, ref, A, what=f"K={K}")
    y1 = host(q8.gemv(W, dev(x[1:2])))
    assert np.array_equal(y1[0].view(np.uint32), y[1].view(np.uint32))
    Wa, Wb = upload(c.q[:300], c.d[:300]), upload(c.q[300:], c.d[300:])
    ya, yb = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x)))
    assert np.array_equal(np.concatenate([ya, yb], 1).view(np.uint32), y.view(np.uint32))
    note(f"gemv at K={K + 32} xf32={xf32}: refused")
    c2 = synth.gemv_case(16, K + 32, 1, seed=1)
    x2 = c2.x.astype(np.float32) if xf32 else c2.x
    W2 = upload(c2.q, c2.d)
    _refused(lambda: q8.gemv(W2, dev(x2)))
    _refused(lambda: q8.gemv_pair(W2, W2, dev(x2)))


@pytest.mark.parametrize("N", [1, 3])
def test_lmhead_at_the_largest_k(N):
    K = 81408
    # 1500 rows: below the size where the head runs as GEMV + argmax
    # launches, so the fused kernel takes the whole LDS
    note(f"lmhead 1500x{K} N={N}")
    c = synth.lmhead_case(1500, K, N, seed=N)
    W = upload(c.q, c.d)
    logits, ids = q8.lmhead_argmax(W, dev(c.x))
    logits, ids = host(logits), host(ids)
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(logits, ref, A, what=f"lmhead K={K}")
    istar, gated, _ = oracle.argmax_gate(ref, A)
    assert gated.all() and np.array_equal(istar, c.planted_rows)
    assert list(ids) == list(c.planted_rows)
    note(f"lmhead at K={K + 32}: refused (the dense GEMV takes this K)")
    c2 = synth.gemv_case(64, K + 32, 1, seed=2)
    W2 = upload(c2.q, c2.d)
    _refused(lambda: q8.lmhead_argmax(W2, dev(c2.x)))
    y = host(q8.gemv(W2, dev(c2.x)))
    ref2, A2 = oracle.gemv(c2.q, c2.d, c2.x, threads())
    assert_parity(y, ref2, A2, what=f"gemv K={K + 32}")


@pytest.mark.parametrize("K,xf32", [(20352, False), (10176, True)])
def test_routed_gemv_at_the_largest_k(K, xf32):
    note(f"routed gemv at K={K} xf32={xf32}")
    E, M, T, topk = 6, 300, 3, 2
    rng = np.random.default_rng(K)
    qb = np.empty((E, M, K), np.int8)
    db = np.empty((E, M, K // 32), np.float16)
    for e in range(E):
        qb[e], db[e] = synth.draw_weights(rng, M, K)
    x = synth.draw_x(rng, T, K)
    if xf32:
        x = x.astype(np.float32)
    ids = np.array([[5, 0], [2, 5], [1, 3]], np.int32)
    bank = upload_bank(qb, db)
    yp = host(q8.moe_gemv(bank, dev(ids), dev(x)))
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            ref, A = oracle.gemv(qb[e], db[e], x[t:t + 1], threads())
            assert_parity(yp[t * topk + j:t * topk + j + 1], ref, A, what=f"pair ({t},{j})")
    note(f"routed gemv at K={K + 32}: refused")
    q2, d2 = synth.draw_weights(rng, 2 * 16, K + 32)
    bank2 = upload_bank(q2.reshape(2, 16, K + 32), d2.reshape(2, 16, -1))
    x2 = synth.draw_x(rng, T, K + 32)
    if xf32:
        x2 = x2.astype(np.float32)
    _refused(lambda: q8.moe_gemv(bank2, dev(np.zeros((T, 1), np.int32)), dev(x2)))


def test_routed_ffn_at_the_largest_f():
    F, H, E, T, topk = 10176, 2048, 3, 2, 2
    note(f"routed ffn F={F} H={H}")
    rng = np.random.default_rng(F)
    planes = {}
    for name, (M, K) in (("gate", (F, H)), ("up", (F, H)), ("down", (H, F))):
        q = np.empty((E, M, K), np.int8)
        d = np.empty((E, M, K // 32), np.float16)
        for e in range(E):
            q[e], d[e] = synth.draw_weights(rng, M, K)
        planes[name] = (q, d)
    x = synth.draw_x(rng, T, H)
    ids = np.array([[2, 0], [1, 2]], np.int32)
    gw = np.array([[0.7, 0.3], [0.4, 0.6]], np.float32)
    c = synth.MoeCase(*planes["gate"], *planes["up"], *planes["down"], x, ids, gw)
    B = [upload_bank(*planes[n]) for n in ("gate", "up", "down")]
    out = host(q8.moe_ffn(*B, dev(ids), dev(gw), dev(x)))
    e2e = oracle.moe_ffn(c, threads())
    assert np.all(np.abs(out - e2e["out"]) <= e2e["bound"])
    note(f"routed ffn F={F + 32}: refused")
    small = {}
    for name, (M, K) in (("gate", (F + 32, 64)), ("up", (F + 32, 64)), ("down", (64, F + 32))):
        q, d = synth.draw_weights(rng, E * M, K)
        small[name] = upload_bank(q.reshape(E, M, K), d.reshape(E, M, -1))
    xs = synth.draw_x(rng, T, 64)
    _refused(lambda: q8.moe_ffn(small["gate"], small["up"], small["down"], dev(ids), dev(gw),
                                dev(xs)))
