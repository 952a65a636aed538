"""Parity of the Q4_0 GEMV (q8_gemv on a Q4_0-format matrix) with the oracle.

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
    y = host(q8.gemv(q8.pack_q4_0(case["blocks"]), dev(case["x"])))
    assert np.array_equal(y.astype(np.float64), case["y"]), case["why"]


SHAPES = [(1024, 1024, 1), (1000, 96, 3), (333, 2048, 4), (517, 768, 8), (64, 32, 2),
          (129, 800, 5), (2050, 5120, 2), (7, 160, 9), (1, 1024, 1), (300, 4096, 16)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_random_parity(M, K, N):
    note(f"q4 random M={M} K={K} N={N}")
    c = synth.q4_0_case(M, K, N, seed=M + K + N)
    y = host(q8.gemv(upload_q4(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y, ref, A, what=f"q4 {M}x{K} N={N}")


def test_full_5120_n1_and_pair_shape():
    note("q4 5120x5120 N=1 and 17408x5120 N=4 (sampled rows)")
    c = synth.q4_0_case(5120, 5120, 1, seed=0)
    y = host(q8.gemv(upload_q4(c.q, c.d), dev(c.x)))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    assert_parity(y, ref, A, what="q4 5120")
    c = synth.q4_0_case(17408, 5120, 4, seed=1)
    y = host(q8.gemv(upload_q4(c.q, c.d), dev(c.x)))
    rows = np.unique(np.concatenate([[0, 17407], np.random.default_rng(0).choice(17408, 1500)]))
    ref, A = oracle.gemv_rows(c.q, c.d, c.x, rows, threads())
    assert_parity(y[:, rows], ref, A, what="q4 17408 N=4")


@pytest.mark.parametrize("M,K", [(513, 1024), (64, 96)])
def test_fp16_output_and_fp32_activations(M, K):
    note(f"q4 fp16 out / fp32 x M={M} K={K}")
    c = synth.q4_0_case(M, K, 3, seed=M)
    W = upload_q4(c.q, c.d)
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    y16 = host(q8.gemv(W, dev(c.x), out_dtype=torch.float16))
    assert_parity(y16.astype(np.float64), ref, A, out_dtype="f16", what="q4 fp16 out")
    x32 = c.x.astype(np.float32)
    y = host(q8.gemv(W, dev(x32)))
    ref32, A32 = oracle.gemv(c.q, c.d, x32, threads())
    assert_parity(y, ref32, A32, what="q4 fp32 x")


@pytest.mark.parametrize("K", [5120, 768, 96])
def test_n_invariance_bitwise(K):
    note(f"q4 N invariance K={K}")
    c = synth.q4_0_case(777, K, 16, seed=K)
    W = upload_q4(c.q, c.d)
    x = dev(c.x)
    solo = np.stack([host(q8.gemv(W, x[n:n + 1]))[0] for n in range(16)])
    for N in (2, 3, 5, 8, 9, 16):
        yN = host(q8.gemv(W, x[:N].contiguous()))
        assert np.array_equal(yN.view(np.uint32), solo[:N].view(np.uint32)), f"N={N}"


def test_extreme_nibbles_and_scales_bitwise():
    """Every weight -8 or 7 with d = 1 and integer activations: exact sums."""
    note("q4 extreme nibbles")
    K, M = 256, 64
    rng = np.random.default_rng(4)
    q = np.where(rng.random((M, K)) < 0.5, -8, 7).astype(np.int8)
    d = np.ones((M, K // 32), np.float16)
    x = rng.integers(-3, 4, size=(2, K)).astype(np.float16)
    y = host(q8.gemv(upload_q4(q, d), dev(x)))
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ q.astype(np.float64).T)


# ---------------------------------------------------------------- the rest of the family
def q4_pair(M, K, N, seed):
    rng = np.random.default_rng(seed)
    qa, da = synth.draw_weights_q4_0(rng, M, K)
    qb, db = synth.draw_weights_q4_0(rng, M, K)
    x = synth.draw_x(rng, N, K)
    return qa, da, qb, db, x


@pytest.mark.parametrize("M,K,N", [(3000, 1024, 1), (517, 2048, 4), (129, 96, 8)])
def test_q4_pair_and_silu_pair(M, K, N):
    note(f"q4 pair/silu M={M} K={K} N={N}")
    qa, da, qb, db, x = q4_pair(M, K, N, seed=M + N)
    Wa, Wb = upload_q4(qa, da), upload_q4(qb, db)
    ya, yb = (host(t) for t in q8.gemv_pair(Wa, Wb, dev(x)))
    for q, d, y in ((qa, da, ya), (qb, db, yb)):
        ref, A = oracle.gemv(q, d, x, threads())
        assert_parity(y, ref, A, what="q4 pair")
    assert np.array_equal(ya.view(np.uint32), host(q8.gemv(Wa, dev(x))).view(np.uint32))
    h = host(q8.gemv_pair_silu(Wa, Wb, dev(x)))
    r = oracle.gate_up_silu(qa, da, qb, db, x, threads())
    assert np.all(np.abs(h - r["h"]) <= r["bh"])


def test_q4_lmhead_and_draft_head():
    note("q4 lm head")
    V, K, N = 20000, 1024, 3
    rng = np.random.default_rng(11)
    q, d = synth.draw_weights_q4_0(rng, V, K)
    x = synth.draw_x(rng, N, K)
    W = upload_q4(q, d)
    logits, ids = q8.lmhead_argmax(W, dev(x))
    logits, ids = host(logits), host(ids)
    ref, A = oracle.gemv(q, d, x, threads())
    assert_parity(logits, ref, A, what="q4 logits")
    istar, gated, cands = oracle.argmax_gate(ref, A)
    for n in range(N):
        assert ids[n] == istar[n] if gated[n] else ids[n] in cands[n]
    assert np.array_equal(ids, oracle.argmax_first(logits))
    rows = rng.choice(V, 3000, replace=False).astype(np.int32)
    Wd = upload_q4(q[rows], d[rows])
    ld, idd = q8.lmhead_argmax(Wd, dev(x), row_ids=dev(rows))
    assert np.array_equal(host(ld).view(np.uint32), logits[:, rows].view(np.uint32))
    want, gated, cands = oracle.argmax_masked(ref[:, rows], A[:, rows], rows)
    for n in range(N):
        assert host(idd)[n] == want[n] if gated[n] else host(idd)[n] in cands[n]


def q4_moe_case(E, F, H, T, topk, seed, down_q8=False):
    rng = np.random.default_rng(seed)
    qg = np.empty((E, F, H), np.int8); dg = np.empty((E, F, H // 32), np.float16)
    qu = np.empty_like(qg); du = np.empty_like(dg)
    qd = np.empty((E, H, F), np.int8); dd = np.empty((E, H, F // 32), np.float16)
    for e in range(E):
        qg[e], dg[e] = synth.draw_weights_q4_0(rng, F, H)
        qu[e], du[e] = synth.draw_weights_q4_0(rng, F, H)
        qd[e], dd[e] = (synth.draw_weights(rng, H, F) if down_q8 else
                        synth.draw_weights_q4_0(rng, H, F))
    x = synth.draw_x(rng, T, H)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    z = np.exp(rng.normal(0, 1, size=(T, topk)))
    gw = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return synth.MoeCase(qg, dg, qu, du, qd, dd, x, ids, gw)


def bank_q4(qb, db):
    return q8.pack_bank_q4_0(np.stack([synth.to_gguf_q4_0_blocks(qb[e], db[e])
                                       for e in range(qb.shape[0])]))


@pytest.mark.parametrize("down_q8", [False, True])
def test_q4_routed_experts(down_q8):
    note(f"q4 moe ffn down_q8={down_q8}")
    c = q4_moe_case(E=16, F=256, H=512, T=8, topk=4, seed=3 + down_q8, down_q8=down_q8)
    g, u = bank_q4(c.q_gate, c.d_gate), bank_q4(c.q_up, c.d_up)
    if down_q8:
        dn = q8.pack_bank(np.stack([synth.to_gguf_blocks(c.q_down[e], c.d_down[e])
                                    for e in range(c.E)]))
    else:
        dn = bank_q4(c.q_down, c.d_down)
    out = host(q8.moe_ffn(g, u, dn, dev(c.expert_ids), dev(c.gate_w), dev(c.x)))
    ref = oracle.moe_ffn(c, threads())
    assert np.all(np.abs(out - ref["out"]) <= ref["bound"])
    # routed GEMV on a Q4_0 bank equals q8_gemv on the chosen expert, bitwise
    yp = host(q8.moe_gemv(g, dev(c.expert_ids), dev(c.x)))
    for t in (0, 5):
        for j in range(c.topk):
            e = int(c.expert_ids[t, j])
            ref1 = host(q8.gemv(g.expert(e), dev(c.x[t:t + 1])))[0]
            assert np.array_equal(yp[t * c.topk + j].view(np.uint32), ref1.view(np.uint32))


def test_q4_router_matrix():
    note("q4 router")
    rng = np.random.default_rng(8)
    q, d = synth.draw_weights_q4_0(rng, 64, 1024)
    x = synth.draw_x(rng, 5, 1024)
    logits, ids, gw = q8.moe_router(upload_q4(q, d), dev(x), 6)
    L = host(logits)
    rid, rw, dl = oracle.topk_softmax(L, 6)
    assert np.array_equal(host(ids), rid)
    assert np.all(np.abs(host(gw).astype(np.float64) - rw) <= oracle.topk_softmax_bound(rw, dl))
    ref, A = oracle.gemv(q, d, x, threads())
    assert_parity(L, ref, A, what="q4 router logits")
