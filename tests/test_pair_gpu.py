"""Parity of the fused gate+up pair (q8_gemv_pair) with the oracle.

Full-size workload: two [17408][5120] Q8_0 matrices sharing x, N = 1, 2, 4,
8 (speculative-verify widths). The oracle checks a sample of rows from
both matrices (first, last and 1500 random rows each, plus every row of a
smaller pair); the pair must equal two single q8_gemv calls bitwise.
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
def test_full_size_pair_sampled_rows(full_pair, N):
    note(f"pair 17408x5120 N={N}")
    c, Wa, Wb = full_pair
    x = c.x[:N]
    ya, yb = q8.gemv_pair(Wa, Wb, dev(x))
    ya, yb = host(ya), host(yb)
    rng = np.random.default_rng(N)
    rows = np.unique(np.concatenate([[0, 1, 17407], rng.choice(17408, 1500, replace=False)]))
    for q, d, y, name in ((c.qa, c.da, ya, "gate"), (c.qb, c.db, yb, "up")):
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
