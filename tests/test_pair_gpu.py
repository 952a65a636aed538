"""Parity of the fused gate+up pair (q8_gemv_pair) with the oracle.

Full-size workload: two [17408][5120] Q8_0 matrices sharing x, N = 1, 2, 4,
8 (speculative-verify widths). The oracle checks every row of both
matrices at N = 1 and 8 (a sample of rows at 2 and 4, and every row of
smaller pairs); the pair must equal two single q8_gemv calls bitwise.
The fused SiLU pair (q8_gemv_pair_silu) is gated against the oracle's
propagated bound on h = silu(g) * u, against silu of the pair's own g and
u within fp32 rounding, for fp16 output, multi-pass N and N-invariance.
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


@pytest.fixture(scope="module")
def full_pair():
    c = synth.pair_case(17408, 5120, 8, seed=0)
    return c, upload(c.qa, c.da), upload(c.qb, c.db)


@pytest.mark.parametrize("N", [1, 2, 4, 8])
def test_full_size_pair(full_pair, N):
    """Every row of both matrices at N = 1 and 8; a sample of rows at 2, 4."""
    note(f"pair 17408x5120 N={N}")
    c, Wa, Wb = full_pair
    x = c.x[:N]
    ya, yb = q8.gemv_pair(Wa, Wb, dev(x))
    ya, yb = host(ya), host(yb)
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([[0, 1, 17407], rng.choice(17408, 1500, replace=False)]))
    for q, d, y, name in ((c.qa, c.da, ya, "gate"), (c.qb, c.db, yb, "up")):
        if N in (1, 8):
            ref, A = oracle.gemv(q, d, x, threads())
            assert_parity(y, ref, A, what=f"{name} N={N} all rows")
        else:
            ref, A = oracle.gemv_rows(q, d, x, rows, threads())
            assert_parity(y[:, rows], ref, A, what=f"{name} N={N}")
    # the pair equals two single GEMVs bitwise
    sa = host(q8.gemv(Wa, dev(x)))
    sb = host(q8.gemv(Wb, dev(x)))
    assert np.array_equal(ya.view(np.uint32), sa.view(np.uint32))
    assert np.array_equal(yb.view(np.uint32), sb.view(np.uint32))


def test_full_size_pair_n_invariance(full_pair):
    note("pair N invariance")
    c, Wa, Wb = full_pair
    x = dev(c.x)
    y8a, y8b = (host(t) for t in q8.gemv_pair(Wa, Wb, x[:8].contiguous()))
    for n in (0, 3, 7):
        y1a, y1b = (host(t) for t in q8.gemv_pair(Wa, Wb, x[n:n + 1].contiguous()))
        assert np.array_equal(y1a[0].view(np.uint32), y8a[n].view(np.uint32))
        assert np.array_equal(y1b[0].view(np.uint32), y8b[n].view(np.uint32))


@pytest.mark.parametrize("Ma,Mb,K,N", [(300, 517, 768, 3), (64, 64, 1024, 1), (1000, 7, 96, 8)])
def test_small_pair_all_rows(Ma, Mb, K, N):
    note(f"pair {Ma}/{Mb}x{K} N={N}")
    rng = np.random.default_rng(Ma + Mb)
    qa, da = synth.draw_weights(rng, Ma, K)
    qb, db = synth.draw_weights(rng, Mb, K)
    x = synth.draw_x(rng, N, K)
    ya, yb = q8.gemv_pair(upload(qa, da), upload(qb, db), dev(x), out_dtype=torch.float32)
    for q, d, y in ((qa, da, host(ya)), (qb, db, host(yb))):
        ref, A = oracle.gemv(q, d, x, threads())
        assert_parity(y, ref, A, what="small pair")


# ---------------------------------------------------------------- gate/up + SiLU
def check_silu(h, r, what):
    err = np.abs(np.asarray(h, np.float64) - r["h"])
    bad = err > r["bh"]
    assert not bad.any(), f"{what}: {bad.sum()} outputs outside the propagated bound"


@pytest.mark.parametrize("N", [1, 4, 8])
def test_full_size_silu(full_pair, N):
    """Every output at N = 1 and 8; a sample of rows at 4."""
    note(f"pair+silu 17408x5120 N={N}")
    c, Wa, Wb = full_pair
    x = c.x[:N]
    h = host(q8.gemv_pair_silu(Wa, Wb, dev(x)))
    if N in (1, 8):
        r = oracle.gate_up_silu(c.qa, c.da, c.qb, c.db, x, threads())
        check_silu(h, r, f"N={N} all rows")
    else:
        rng = np.random.default_rng(100 + N)
        rows = np.unique(np.concatenate([[0, 1, 17407], rng.choice(17408, 1500, replace=False)]))
        r = oracle.gate_up_silu(c.qa[rows], c.da[rows], c.qb[rows], c.db[rows], x, threads())
        check_silu(h[:, rows], r, f"N={N}")
    # h is silu of the pair's own g and u, within fp32 rounding of the epilogue
    ya, yb = (host(t).astype(np.float64) for t in q8.gemv_pair(Wa, Wb, dev(x)))
    ref = oracle.silu(ya) * yb
    assert np.all(np.abs(h - ref) <= 1e-6 * np.abs(ref) + 1e-30)


def test_silu_n_invariance(full_pair):
    note("pair+silu N invariance")
    c, Wa, Wb = full_pair
    x = dev(c.x)
    h8 = host(q8.gemv_pair_silu(Wa, Wb, x[:8].contiguous()))
    for n in (0, 5):
        h1 = host(q8.gemv_pair_silu(Wa, Wb, x[n:n + 1].contiguous()))
        assert np.array_equal(h1[0].view(np.uint32), h8[n].view(np.uint32))


@pytest.mark.parametrize("M,K,N,f16", [(300, 768, 3, False), (7, 96, 8, False), (64, 1024, 1, True),
                                       (517, 2048, 12, False), (129, 160, 16, True)])
def test_small_silu_all_rows(M, K, N, f16):
    note(f"pair+silu {M}x{K} N={N} f16={f16}")
    rng = np.random.default_rng(M + K + N)
    qg, dg = synth.draw_weights(rng, M, K)
    qu, du = synth.draw_weights(rng, M, K)
    x = synth.draw_x(rng, N, K)
    h = q8.gemv_pair_silu(upload(qg, dg), upload(qu, du), dev(x),
                          out_dtype=torch.float16 if f16 else torch.float32)
    r = oracle.gate_up_silu(qg, dg, qu, du, x, threads(), out_dtype="f16" if f16 else "f32")
    check_silu(host(h), r, f"{M}x{K} N={N}")
