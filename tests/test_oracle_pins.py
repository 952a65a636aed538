"""Pins for the CPU oracle: it is checked against things other than itself.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a wrong sign, a wrong block index, a transposed operand, a flushed subnormal,
a mis-decoded byte) fails at least one test:

* fp16 decoding against numpy's binary16 for every finite bit pattern;
* GGUF block decoding against hand-built blocks with hand-derived results;
* exact rational brute force (fractions.Fraction from the raw block bytes,
  decoded with Python's struct 'e' format, independent of the oracle's own
  decoders) on tiny inputs, random and adversarial;
* closed forms: unit vectors recover single quants, subnormal scales and
  activations, zero blocks contribute exactly zero, power-of-two scaling is
  exact, integer-valued data equals an int64 matmul (numpy) on non-square
  shapes, per-block power-of-two scales equal an int64 block decomposition;
* the floating-point bound: an fp32 emulation stays inside gamma_{K+1}*A.
"""
import math
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from quantized_weight_gemv_q8_amd import synth
from tests.golden_io import load_handbuilt

TWO53 = 2.0 ** -53


# ------------------------------------------------------------- decoders
def test_half_decoder_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 10) & 0x1F) != 0x1F
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    for b in bits[finite]:
        v = oracle.half_to_double(int(b))
        r = ref[b]
        assert v == r and np.signbit(v) == np.signbit(r), hex(int(b))


def test_half_decoder_specials():
    assert oracle.half_to_double(0x7C00) == float("inf")
    assert oracle.half_to_double(0xFC00) == float("-inf")
    assert np.isnan(oracle.half_to_double(0x7E00))
    assert oracle.half_to_double(0x0001) == 2.0 ** -24
    assert oracle.half_to_double(0x0400) == 2.0 ** -14


@pytest.mark.parametrize("case", load_handbuilt(), ids=lambda c: c["name"])
def test_golden_handbuilt(case):
    q, d = oracle.decode_blocks(case["blocks"])
    y, A = oracle.gemv(q, d, case["x"])
    assert np.array_equal(y, case["y"]), (case["why"], y, case["y"])


def test_block_decoder_roundtrip_random():
    c = synth.gemv_case(7, 96, 1, seed=3)
    blocks = synth.to_gguf_blocks(c.q, c.d)
    assert blocks.shape == (7, 3, 34)
    q, d = oracle.decode_blocks(blocks)
    assert np.array_equal(q, c.q)
    assert np.array_equal(d.view(np.uint16), c.d.view(np.uint16))


# ------------------------------------------------------------- brute force
def _exact_from_blocks(blocks, x):
    """Exact y and A as Fractions, decoding the raw bytes with struct."""
    M, nb, _ = blocks.shape
    K = nb * 32
    N = x.shape[0]
    xf = [[Fraction(float(v)) for v in x[n]] for n in range(N)]
    y = [[Fraction(0)] * M for _ in range(N)]
    A = [[Fraction(0)] * M for _ in range(N)]
    for m in range(M):
        for b in range(nb):
            raw = bytes(blocks[m, b])
            (dv,) = struct.unpack("<e", raw[:2])
            qs = struct.unpack("32b", raw[2:])
            for i, qv in enumerate(qs):
                w = Fraction(dv) * qv
                for n in range(N):
                    t = w * xf[n][b * 32 + i]
                    y[n][m] += t
                    A[n][m] += abs(t)
    return y, A


def _adversarial_blocks(rng, M, K):
    nb = K // 32
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    pool = np.array([0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x0000, 0x8000, 0x1234, 0x0200],
                    np.uint16)
    d = pool[rng.integers(0, len(pool), size=(M, nb))].view(np.float16)
    q[rng.random((M, K)) < 0.1] = -128
    return q, d


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("K", [32, 64, 96])
def test_bruteforce_fraction(seed, K):
    rng = np.random.default_rng(100 + seed)
    M = int(rng.integers(1, 5))
    N = int(rng.integers(1, 4))
    if seed % 2:
        q, d = _adversarial_blocks(rng, M, K)
        xb = rng.integers(0, 0x7C00, size=(N, K)).astype(np.uint16)  # finite, incl. subnormals
        xb |= (rng.random((N, K)) < 0.5).astype(np.uint16) << 15
        x = xb.view(np.float16)
    else:
        q, d = synth.draw_weights(rng, M, K)
        x = synth.draw_x(rng, N, K)
    blocks = synth.to_gguf_blocks(q, d)
    qo, do = oracle.decode_blocks(blocks)
    y, A = oracle.gemv(qo, do, x)
    ye, Ae = _exact_from_blocks(blocks, x)
    for n in range(N):
        for m in range(M):
            tol = Fraction(K) * Fraction(TWO53) * Ae[n][m]
            assert abs(Fraction(y[n, m]) - ye[n][m]) <= tol
            assert abs(Fraction(A[n, m]) - Ae[n][m]) <= tol


def test_bruteforce_fraction_fp32_x():
    rng = np.random.default_rng(7)
    q, d = synth.draw_weights(rng, 3, 64)
    x = rng.normal(0, 1, size=(2, 64)).astype(np.float32)
    y, A = oracle.gemv(q, d, x)
    for n in range(2):
        for m in range(3):
            e = sum(Fraction(float(d[m, k // 32])) * int(q[m, k]) * Fraction(float(x[n, k]))
                    for k in range(64))
            a = sum(abs(Fraction(float(d[m, k // 32])) * int(q[m, k]) * Fraction(float(x[n, k])))
                    for k in range(64))
            assert abs(Fraction(y[n, m]) - e) <= 64 * Fraction(TWO53) * a


# ------------------------------------------------------------- closed forms
@pytest.mark.parametrize("j", [0, 1, 15, 16, 31, 32, 63, 95])
def test_unit_vector_recovers_each_int8(j):
    K = 96
    rng = np.random.default_rng(j)
    q = rng.integers(-128, 128, size=(256, K)).astype(np.int8)
    q[:, j] = np.arange(256) - 128  # every int8 value once
    d = np.full((256, K // 32), 1.0, np.float16)
    x = np.zeros((1, K), np.float16)
    x[0, j] = 1.0
    y, _ = oracle.gemv(q, d, x)
    assert np.array_equal(y[0], (np.arange(256) - 128).astype(np.float64))


def test_subnormal_scale_and_activation():
    K = 64
    q = np.zeros((2, K), np.int8)
    q[0, 40] = 127
    q[1, 3] = -128
    d = np.array([[0x3C00, 0x0001], [0x0001, 0x3C00]], np.uint16).view(np.float16)
    x = np.zeros((2, K), np.float16)
    x[0, 40] = 1.0
    x[1, 3] = np.uint16(0x0001).view(np.float16)  # 2^-24
    y, _ = oracle.gemv(q, d, x)
    assert y[0, 0] == 127 * 2.0 ** -24  # subnormal d, unit x
    assert y[1, 1] == -128 * 2.0 ** -24 * 2.0 ** -24  # subnormal d times subnormal x
    assert y[0, 1] == 0 and y[1, 0] == 0


def test_zero_blocks_contribute_exactly_zero():
    c = synth.gemv_case(32, 256, 3, seed=11)
    q, d = c.q.copy(), c.d.copy()
    rng = np.random.default_rng(5)
    zero_d = rng.random(d.shape) < 0.2
    zero_q = (rng.random(d.shape) < 0.2) & ~zero_d
    d[zero_d] = 0.0
    for m, b in zip(*np.nonzero(zero_q)):
        q[m, b * 32:(b + 1) * 32] = 0
    d[5] = 0.0  # an all-zero row
    y, A = oracle.gemv(q, d, c.x)
    assert np.all(y[:, 5] == 0) and np.all(A[:, 5] == 0)
    # removing the zero blocks (row by row) leaves every output unchanged
    for m in range(32):
        keep = ~(zero_d[m] | zero_q[m])
        kk = np.repeat(keep, 32)
        if not keep.any():
            assert np.all(y[:, m] == 0)
            continue
        yr, _ = oracle.gemv(q[m:m + 1, kk], d[m:m + 1, keep], np.ascontiguousarray(c.x[:, kk]))
        assert np.array_equal(yr[:, 0], y[:, m])


@pytest.mark.parametrize("s", [-4, -1, 1, 3, 4])
def test_power_of_two_scaling_is_exact(s):
    rng = np.random.default_rng(20 + s)
    M, K = 16, 160
    q = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    d = (2.0 ** rng.uniform(-9, -3, size=(M, K // 32))).astype(np.float16)  # normal after * 2^s
    x = synth.draw_x(rng, 2, K)
    y, _ = oracle.gemv(q, d, x)
    d2 = (d.astype(np.float64) * 2.0 ** s).astype(np.float16)
    assert np.array_equal(d2.astype(np.float64), d.astype(np.float64) * 2.0 ** s)
    y2, _ = oracle.gemv(q, d2, x)
    assert np.array_equal(y2, y * 2.0 ** s)


@pytest.mark.parametrize("M,K,N", [(24, 640, 3), (640, 96, 2), (5, 5120, 4)])
def test_integer_exact_equals_int64_matmul(M, K, N):
    """x integer in [-8, 8], d = 2^e constant: y = 2^e * (q @ x^T) exactly."""
    rng = np.random.default_rng(M * 7 + K)
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    xi = rng.integers(-8, 9, size=(N, K))
    x = xi.astype(np.float16)
    e = -3
    d = np.full((M, K // 32), 2.0 ** e, np.float16)
    y, _ = oracle.gemv(q, d, x)
    ref = (q.astype(np.int64) @ xi.T.astype(np.int64)).T * 2.0 ** e
    assert np.array_equal(y, ref)


def test_per_block_scales_equal_block_decomposition():
    """d varies per block as 2^e_b: y = sum_b 2^e_b * (int64 block dot), exact."""
    rng = np.random.default_rng(9)
    M, K, N = 12, 320, 3
    nb = K // 32
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    xi = rng.integers(-8, 9, size=(N, K))
    eb = rng.integers(-3, 4, size=(M, nb))
    d = (2.0 ** eb).astype(np.float16)
    y, _ = oracle.gemv(q, d, xi.astype(np.float16))
    blockdot = np.einsum("mbk,nbk->nmb", q.reshape(M, nb, 32).astype(np.int64),
                         xi.reshape(N, nb, 32).astype(np.int64))
    ref8 = (blockdot * (2 ** (eb + 3))[None]).sum(axis=2)  # 8*y as an integer
    assert np.array_equal(y * 8, ref8.astype(np.float64))


def test_matches_float64_matmul_of_dequantized_weights():
    c = synth.gemv_case(200, 1024, 3, seed=1)
    y, A = oracle.gemv(c.q, c.d, c.x)
    w = (c.q.reshape(200, 32, 32).astype(np.float64) * c.d.astype(np.float64)[:, :, None]).reshape(200, 1024)
    ref = c.x.astype(np.float64) @ w.T
    assert np.all(np.abs(y - ref) <= 2 * 1024 * TWO53 * A)
    assert np.allclose(A, np.abs(c.x.astype(np.float64)) @ np.abs(w).T, rtol=1e-12)


def test_fp32_emulation_inside_higham_bound():
    """Any fp32 order of the K products + scales stays within gamma_{K+1} * A."""
    c = synth.gemv_case(64, 5120, 1, seed=2)
    y, A = oracle.gemv(c.q, c.d, c.x)
    q32 = c.q.astype(np.float32).reshape(64, 160, 32)
    x32 = c.x.astype(np.float32).reshape(1, 160, 32)
    blk = np.cumsum(q32 * x32, axis=2, dtype=np.float32)[:, :, -1]  # per-block fp32 sums
    acc = np.cumsum(blk * c.d.astype(np.float32), axis=1, dtype=np.float32)[:, -1]
    u = 2.0 ** -24
    n = 5120 + 1
    gamma = n * u / (1 - n * u)
    assert np.all(np.abs(acc - y[0]) <= gamma * A[0])
    assert gamma < oracle.REL_TOL


def test_threads_and_sampled_rows_agree():
    c = synth.gemv_case(300, 512, 2, seed=4)
    y1, A1 = oracle.gemv(c.q, c.d, c.x, threads=1)
    y3, A3 = oracle.gemv(c.q, c.d, c.x, threads=3)
    assert np.array_equal(y1, y3) and np.array_equal(A1, A3)
    rows = np.array([299, 0, 17, 150, 17])
    ys, As = oracle.gemv_rows(c.q, c.d, c.x, rows, threads=2)
    assert np.array_equal(ys, y1[:, rows]) and np.array_equal(As, A1[:, rows])


# ------------------------------------------------------------- gates
def test_check_close_bound():
    y = np.array([[1.0, -2.0, 0.0]])
    A = np.array([[10.0, 4.0, 0.0]])
    ok, rel, nbad = oracle.check_close(y + np.array([[0.009, -0.003, 0.0]]), y, A)
    assert ok and nbad == 0 and abs(rel - 0.0009) < 1e-12
    ok, _, nbad = oracle.check_close(y + np.array([[0.011, 0, 0]]), y, A)
    assert not ok and nbad == 1
    ok, _, nbad = oracle.check_close(y + np.array([[0, 0, 1e-30]]), y, A)
    assert not ok  # A == 0 demands an exact zero


def test_fp16_ulp():
    assert oracle.fp16_ulp(np.array([1.0]))[0] == 2.0 ** -10
    assert oracle.fp16_ulp(np.array([1.5]))[0] == 2.0 ** -10
    assert oracle.fp16_ulp(np.array([2.0]))[0] == 2.0 ** -9
    assert oracle.fp16_ulp(np.array([1e-6]))[0] == 2.0 ** -24
    assert oracle.fp16_ulp(np.array([0.0]))[0] == 2.0 ** -24


def test_argmax_first_ties_and_signed_zero():
    L = np.array([[0.0, 3.0, 3.0, -1.0], [-0.0, 0.0, -5.0, -0.0], [1.0, 2.0, 0.5, 2.0]])
    assert list(oracle.argmax_first(L)) == [1, 0, 1]


def test_argmax_gate_sets():
    L = np.array([[5.0, 4.0, 1.0], [5.0, 4.999, 1.0]])
    A = np.full_like(L, 100.0)  # b = 0.1
    istar, gated, cands = oracle.argmax_gate(L, A)
    assert list(istar) == [0, 0]
    assert list(gated) == [True, False]
    assert list(cands[0]) == [0] and list(cands[1]) == [0, 1]


# ------------------------------------------------------------- MoE stages
def test_moe_route_handbuilt():
    ids = np.array([[2, 0], [0, 3], [2, 1]], np.int32)  # T=3, topk=2, E=4
    counts, offsets, pairs, active = oracle.moe_route(ids, 4)
    # pairs p = t*2 + j: (0,0)->2 p0, (0,1)->0 p1, (1,0)->0 p2, (1,1)->3 p3, (2,0)->2 p4, (2,1)->1 p5
    assert list(counts) == [2, 1, 2, 1]
    assert list(offsets) == [0, 2, 3, 5, 6]
    assert list(pairs) == [1, 2, 5, 0, 4, 3]
    assert list(active) == [0, 1, 2, 3]
    counts, offsets, pairs, active = oracle.moe_route(np.array([[3]], np.int32), 5)
    assert list(counts) == [0, 0, 0, 1, 0] and list(active) == [3] and list(pairs) == [0]
    with pytest.raises(ValueError):
        oracle.moe_route(np.array([[5]], np.int32), 5)


def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    z = np.array([-3.0, -0.5, 0.25, 2.0, 7.0])
    assert np.allclose(oracle.silu(z) - oracle.silu(-z), z, rtol=0, atol=1e-15)  # silu(z)-silu(-z) = z
    assert abs(oracle.silu(np.array([40.0]))[0] - 40.0) < 1e-15
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16


def test_moe_combine_handbuilt():
    gw = np.array([[0.25, 0.75]], np.float32)
    yp = np.array([[4.0, -8.0], [8.0, 16.0]])  # pairs (0,0), (0,1); H=2
    out, S = oracle.moe_combine(gw, yp)
    assert np.array_equal(out, [[7.0, 10.0]]) and np.array_equal(S, [[7.0, 14.0]])


def _dense(qm, dm):
    R, C = qm.shape
    return (qm.reshape(R, C // 32, 32).astype(np.float64) * dm.astype(np.float64)[:, :, None]).reshape(R, C)


def test_moe_ffn_top1_equals_dense_composition():
    c = synth.moe_case(E=4, F=64, H=96, T=5, topk=1, seed=2)
    c.gate_w[:] = 1.0
    r = oracle.moe_ffn(c)
    for t in range(c.T):
        e = c.expert_ids[t, 0]
        xt = c.x[t].astype(np.float64)
        g = _dense(c.q_gate[e], c.d_gate[e]) @ xt
        u = _dense(c.q_up[e], c.d_up[e]) @ xt
        h = (g / (1 + np.exp(-g)) * u).astype(np.float32).astype(np.float64)
        ref = _dense(c.q_down[e], c.d_down[e]) @ h
        assert np.all(np.abs(r["out"][t] - ref) <= 1e-9 * (np.abs(_dense(c.q_down[e], c.d_down[e])) @ np.abs(h)) + 1e-300)


def test_moe_ffn_identical_experts_is_routing_independent():
    c = synth.moe_case(E=5, F=64, H=64, T=4, topk=3, seed=8)
    for arr in (c.q_gate, c.d_gate, c.q_up, c.d_up, c.q_down, c.d_down):
        arr[:] = arr[0]
    r1 = oracle.moe_ffn(c)
    c.expert_ids[:] = np.array([[4, 1, 0], [2, 3, 1], [0, 2, 4], [1, 0, 3]], np.int32)
    r2 = oracle.moe_ffn(c)
    assert np.allclose(r1["out"], r2["out"], rtol=1e-12, atol=1e-15)
    # and it equals the single dense FFN scaled by sum_j w = 1 (up to fp32 rounding of gate_w)
    xt = c.x.astype(np.float64)
    g = xt @ _dense(c.q_gate[0], c.d_gate[0]).T
    u = xt @ _dense(c.q_up[0], c.d_up[0]).T
    h = (g / (1 + np.exp(-g)) * u).astype(np.float32).astype(np.float64)
    ref = h @ _dense(c.q_down[0], c.d_down[0]).T * c.gate_w.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.allclose(r1["out"], ref, rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------- generator
def test_generator_is_deterministic_and_distributed():
    a = synth.gemv_case(64, 1024, 2, seed=0)
    b = synth.gemv_case(64, 1024, 2, seed=0)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.d.view(np.uint16), b.d.view(np.uint16))
    assert a.q.min() >= -127 and a.q.max() <= 127
    big = synth.gemv_case(2048, 1024, 1, seed=0)
    sub = np.mean(np.abs(big.d.astype(np.float64)) < 2.0 ** -14)
    assert 0.28 < sub < 0.32  # ~30.2% of |N(0,0.02)|/127 scales are fp16 subnormals
    # x of a wider draw starts with the narrower draw (same stream after the weights)
    c = synth.pair_case(8, 64, 1)
    e = synth.pair_case(8, 64, 4)
    assert np.array_equal(c.x[0].view(np.uint16), e.x[0].view(np.uint16))


def test_lmhead_planting_small():
    c = synth.lmhead_case(V=4096, K=1024, N=3, seed=0)
    y, A = oracle.gemv(c.q, c.d, c.x, threads=oracle.default_threads())
    istar, gated, _ = oracle.argmax_gate(y, A)
    assert list(istar) == list(c.planted_rows)
    assert gated.all()
    for n in range(3):
        others = np.delete(y[n], c.planted_rows[n])
        sigma = others.std()
        assert y[n, c.planted_rows[n]] - others.max() >= 3 * sigma


# ---------------------------------------------------------------- router
def test_router_closed_form_weights():
    """Logits ln 1, ln 2, ln 3, ln 6 give softmax weights 1:2:3:6 exactly
    (up to the fp32 rounding of the logits), ordered by descending logit."""
    L = np.log(np.array([[1.0, 2.0, 3.0, 6.0]])).astype(np.float32)
    ids, w, dl = oracle.topk_softmax(L, 4)
    assert list(ids[0]) == [3, 2, 1, 0]
    assert np.allclose(w[0], np.array([6, 3, 2, 1]) / 12.0, rtol=1e-6, atol=0)
    assert np.allclose(dl[0], np.log(6.0 / np.array([6, 3, 2, 1])), rtol=0, atol=1e-6)
    ids2, w2, _ = oracle.topk_softmax(L, 2)  # top 2 of them: 6 and 3 -> 2/3, 1/3
    assert list(ids2[0]) == [3, 2] and np.allclose(w2[0], [2 / 3, 1 / 3], rtol=1e-6)


def test_router_top1_weight_is_one_and_id_is_first_argmax():
    L = synth.router_case(9, 37, seed=3)
    ids, w, _ = oracle.topk_softmax(L, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(ids[:, 0], np.argmax(L, axis=1))  # numpy: first maximum


def test_router_equal_logits_take_lowest_indices_with_equal_weights():
    L = np.full((2, 10), np.float32(0.25))
    L[1, 7] = np.float32(-0.0)
    L[1, 3] = np.float32(0.0)
    L[1, [0, 1, 2, 4, 5, 6, 8, 9]] = -1.0
    ids, w, _ = oracle.topk_softmax(L, 4)
    assert list(ids[0]) == [0, 1, 2, 3] and np.all(w[0] == 0.25)
    assert list(ids[1][:2]) == [3, 7]  # -0 == +0: the lower index first
    assert w[1][0] == w[1][1]


def test_router_matches_renormalised_full_softmax_brute_force():
    """A different formula: softmax over all experts, keep the picked ones,
    renormalise; the picked set is checked against a brute-force ordering."""
    L = synth.router_case(6, 11, seed=4)
    for k in (1, 3, 11):
        ids, w, _ = oracle.topk_softmax(L, k)
        for t in range(L.shape[0]):
            ranked = sorted(range(11), key=lambda e: (-float(L[t, e]), e))
            assert list(ids[t]) == ranked[:k]
            p = np.exp(L[t].astype(np.float64))
            p = p / p.sum()
            ref = p[ranked[:k]] / p[ranked[:k]].sum()
            assert np.allclose(w[t], ref, rtol=1e-12, atol=0)


def test_router_invariances():
    """Adding a constant to every logit of a token changes nothing; permuting
    the experts permutes the ids; each token is routed independently of the
    other tokens of the batch."""
    L = synth.router_case(5, 24, seed=5, ties=False)
    ids, w, _ = oracle.topk_softmax(L, 6)
    ids_s, w_s, _ = oracle.topk_softmax(L + np.float32(0.5), 6)
    # fp32 rounding of the shifted logits moves the weights by ~1e-7 at most
    assert np.array_equal(ids, ids_s) and np.allclose(w, w_s, rtol=1e-6)
    perm = np.random.default_rng(0).permutation(24)
    ids_p, w_p, _ = oracle.topk_softmax(L[:, perm], 6)
    assert np.array_equal(perm[ids_p], ids) and np.allclose(w_p, w, rtol=0, atol=0)
    ids_1, w_1, _ = oracle.topk_softmax(L[2:3], 6)
    assert np.array_equal(ids_1[0], ids[2]) and np.array_equal(w_1[0], w[2])


def test_router_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.topk_softmax(np.zeros((1, 4), np.float32), 5)
    with pytest.raises(ValueError):
        oracle.topk_softmax(np.array([[0.0, np.nan]], np.float32), 1)


# ---------------------------------------------------------------- dense gate/up + SiLU
def test_gate_up_silu_closed_forms():
    """Hand-built rows with d = 1 and unit quants give g and u exactly, so h
    is silu at known points: silu(1) = 1/(1+e^-1), silu(-1) = -e^-1/(1+e^-1),
    silu(0) = 0 whatever u is."""
    K = 32
    qg = np.zeros((3, K), np.int8)
    qu = np.zeros((3, K), np.int8)
    qg[0, 0], qu[0, 0] = 1, 2     # g = 1, u = 2
    qg[1, 0], qu[1, 0] = -1, 3    # g = -1, u = 3
    qg[2, 5], qu[2, 0] = 0, 7     # g = 0, u = 7
    d = np.ones((3, 1), np.float16)
    x = np.zeros((1, K), np.float16)
    x[0, 0] = 1.0
    r = oracle.gate_up_silu(qg, d, qu, d, x)
    e = math.exp(-1.0)
    assert r["g"][0].tolist() == [1.0, -1.0, 0.0] and r["u"][0].tolist() == [2.0, 3.0, 7.0]
    assert math.isclose(r["h"][0, 0], 2.0 / (1.0 + e), rel_tol=1e-15)
    assert math.isclose(r["h"][0, 1], 3.0 * (-e / (1.0 + e)), rel_tol=1e-15)
    assert r["h"][0, 2] == 0.0


def test_gate_up_silu_large_gate_is_identity_times_up():
    """For large positive g, silu(g) -> g: h -> g*u; for large negative g, h -> 0."""
    rng = np.random.default_rng(0)
    K = 64
    qg = np.full((2, K), 127, np.int8)
    qg[1] = -127
    qu = rng.integers(-127, 128, size=(2, K)).astype(np.int8)
    d = np.full((2, 2), 1.0, np.float16)
    x = np.ones((1, K), np.float16)
    r = oracle.gate_up_silu(qg, d, qu, d, x)
    assert math.isclose(r["h"][0, 0], r["g"][0, 0] * r["u"][0, 0], rel_tol=1e-12)
    assert abs(r["h"][0, 1]) < 1e-300 * abs(r["u"][0, 1]) + 1e-300


# ---------------------------------------------------------------- masked LM head
def test_masked_argmax_identity_subset_equals_full():
    c = synth.lmhead_case(600, 256, 3, seed=1)
    L, A = oracle.gemv(c.q, c.d, c.x)
    ids, gated, _ = oracle.argmax_masked(L, A, np.arange(600))
    assert np.array_equal(ids, oracle.argmax_first(L)) and gated.all()


def test_masked_argmax_maps_back_and_keeps_subset_order_for_ties():
    """A subset holding the full argmax row returns that vocabulary id; equal
    logits go to the earlier position in the subset, whatever their ids."""
    c = synth.lmhead_case(600, 256, 2, seed=2)
    L, A = oracle.gemv(c.q, c.d, c.x)
    full = oracle.argmax_first(L)
    rng = np.random.default_rng(0)
    sub = rng.choice(600, 100, replace=False)
    sub[37] = full[0]
    sub[60] = full[1] if full[1] != full[0] else sub[60]
    ids, gated, _ = oracle.argmax_masked(L[:, sub], A[:, sub], sub)
    assert ids[0] == full[0]
    # exact ties: two positions with identical logits, higher id first
    Lt = np.array([[1.0, 3.0, 3.0, 2.0]])
    ids, gated, cands = oracle.argmax_masked(Lt, np.zeros_like(Lt), np.array([5, 90, 7, 1]))
    assert ids[0] == 90 and not gated[0] and set(cands[0]) == {90, 7}


# ---------------------------------------------------------------- Q4_0
@pytest.mark.parametrize("case", load_handbuilt("q4_0_handbuilt.txt", 18), ids=lambda c: c["name"])
def test_q4_0_handbuilt_fixtures(case):
    q, d = oracle.decode_q4_0_blocks(case["blocks"])
    y, _ = oracle.gemv(q, d, case["x"])
    assert np.array_equal(y, case["y"]), case["why"]


def test_q4_0_decode_every_nibble_position():
    """Each nibble lands on its own element: a block whose byte j holds
    (a_j, b_j) in (low, high) nibbles decodes to a_j - 8 at j and b_j - 8 at
    j + 16, for every j and every nibble value."""
    for v in range(16):
        blk = np.full((1, 1, 18), 0x88, np.uint8)
        blk[0, 0, :2] = (0x00, 0x3C)
        for j in range(16):
            blk[0, 0, 2 + j] = ((15 - v) << 4) | v
        q, d = oracle.decode_q4_0_blocks(blk)
        assert d[0, 0] == 1.0
        assert np.all(q[0, :16] == v - 8) and np.all(q[0, 16:] == 7 - v)


def test_q4_0_synth_roundtrip():
    rng = np.random.default_rng(0)
    q, d = synth.draw_weights_q4_0(rng, 7, 96)
    assert q.min() >= -8 and q.max() <= 7
    q2, d2 = oracle.decode_q4_0_blocks(synth.to_gguf_q4_0_blocks(q, d))
    assert np.array_equal(q2, q) and np.array_equal(d2.view(np.uint16), d.view(np.uint16))


# ---------------------------------------------------------------- shared expert
def test_sigmoid_closed_forms():
    """sigma(0) = 1/2, sigma(ln 3) = 3/4, sigma(-ln 3) = 1/4,
    sigma(z) + sigma(-z) = 1, and no overflow far out on either side."""
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    assert math.isclose(oracle.sigmoid(np.array([math.log(3.0)]))[0], 0.75, rel_tol=1e-15)
    assert math.isclose(oracle.sigmoid(np.array([-math.log(3.0)]))[0], 0.25, rel_tol=1e-15)
    z = np.array([-30.0, -2.5, -0.1, 0.7, 4.0, 30.0])
    assert np.allclose(oracle.sigmoid(z) + oracle.sigmoid(-z), 1.0, rtol=0, atol=1e-15)
    far = oracle.sigmoid(np.array([-1000.0, 1000.0]))
    assert far[0] == 0.0 and far[1] == 1.0
    # sigma' = sigma (1 - sigma): a central difference at z = 0.3
    h = 1e-5
    num = (oracle.sigmoid(np.array([0.3 + h]))[0] - oracle.sigmoid(np.array([0.3 - h]))[0]) / (2 * h)
    s3 = oracle.sigmoid(np.array([0.3]))[0]
    assert abs(num - s3 * (1 - s3)) < 1e-9


def _shexp_case(seed, T=3, F=64, H=96, gate_row=None):
    rng = np.random.default_rng(seed)
    qg, dg = synth.draw_weights(rng, F, H)
    qu, du = synth.draw_weights(rng, F, H)
    qd, dd = synth.draw_weights(rng, H, F)
    qsg, dsg = synth.draw_weights(rng, 1, H)
    if gate_row is not None:
        qsg, dsg = gate_row
    x = synth.draw_x(rng, T, H)
    base = rng.normal(0.0, 1.0, size=(T, H)).astype(np.float32)
    return qg, dg, qu, du, qd, dd, qsg, dsg, x, base


def test_shared_expert_equals_dense_composition():
    """Against the same layer written with dequantised fp64 matrices and
    numpy products: x -> silu(Wg x) * (Wu x) -> Wd (.) -> base + sigma(w.x) * (.)."""
    qg, dg, qu, du, qd, dd, qsg, dsg, x, base = _shexp_case(4)
    r = oracle.shared_expert(qg, dg, qu, du, qd, dd, qsg, dsg, x, base)
    xf = x.astype(np.float64)
    g = xf @ _dense(qg, dg).T
    u = xf @ _dense(qu, du).T
    h = (g / (1.0 + np.exp(-g))) * u
    s = h.astype(np.float32).astype(np.float64) @ _dense(qd, dd).T
    gl = xf @ _dense(qsg, dsg).T
    ref = base.astype(np.float64) + s / (1.0 + np.exp(-gl))
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12)
    assert np.all(r["bound"] > 0)


def test_shared_expert_gate_extremes_select_base_or_sum():
    """A gate row whose dot is +-40 (one quant of 1 with d = 40 against
    x[0] = 1): sigma = 1 - 4e-18 or 4e-18, so out is base + s or base, up to
    that margin; a flipped sign or a dropped gate fails one of them."""
    H = 96
    x0 = None
    for sign, expect_s in ((1, True), (-1, False)):
        qsg = np.zeros((1, H), np.int8)
        qsg[0, 0] = sign
        dsg = np.zeros((1, H // 32), np.float16)
        dsg[0, 0] = 40.0
        c = list(_shexp_case(9, gate_row=(qsg, dsg)))
        c[8] = c[8].copy()
        c[8][:, 0] = 1.0
        r = oracle.shared_expert(*c)
        base = c[9].astype(np.float64)
        assert np.allclose(r["gate"], 1.0 if expect_s else 0.0, rtol=0, atol=1e-15)
        want = base + r["s"] if expect_s else base
        assert np.allclose(r["out"], want, rtol=0, atol=1e-12 * (1 + np.abs(r["s"]).max()))
        if x0 is None:
            x0 = r["s"]
    assert np.abs(x0).max() > 1e-3  # the expert's output is not trivially zero


def test_shared_expert_zero_down_returns_base_exactly():
    qg, dg, qu, du, qd, dd, qsg, dsg, x, base = _shexp_case(5)
    r = oracle.shared_expert(qg, dg, qu, du, np.zeros_like(qd), dd, qsg, dsg, x, base)
    assert np.array_equal(r["out"], base.astype(np.float64))
