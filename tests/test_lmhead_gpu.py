"""Parity of the LM head GEMV + argmax (q8_lmhead_argmax) with the oracle.

Full-size workload: V = 151936 vocabulary rows, K = 5120, N = 1 and 4, one
planted row per token. The oracle computes every logit (fp64), so the
argmax gate is exact: tokens whose top-2 gap exceeds the bound must return
the oracle's id, others an id from the candidate set; the GPU ids must
also be consistent with the GPU logits (first maximum). Sampled logits are
checked against the bound. Small cases cover ties (lowest index wins),
signed zeros, the logits == NULL path and multi-pass N.
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


def check_lmhead(c, logits, ids, full=True):
    N = c.x.shape[0]
    assert np.array_equal(ids, oracle.argmax_first(logits)), "ids inconsistent with GPU logits"
    if full:
        ref, A = oracle.gemv(c.q, c.d, c.x, threads())
        assert_parity(logits, ref, A, what="logits")
        istar, gated, cands = oracle.argmax_gate(ref, A)
        for n in range(N):
            if gated[n]:
                assert ids[n] == istar[n], f"token {n}: {ids[n]} != {istar[n]}"
            else:
                assert ids[n] in cands[n]
        return gated


@pytest.fixture(scope="module")
def vocab():
    c = synth.lmhead_case(151936, 5120, 4, seed=0)
    return c, upload(c.q, c.d)


@pytest.mark.parametrize("N", [1, 2, 4])
def test_full_vocab(vocab, N):
    note(f"lmhead 151936x5120 N={N}")
    c4, W = vocab
    c = synth.LmHeadCase(c4.q, c4.d, c4.x[:N], c4.planted_rows[:N], c4.planted_target[:N])
    logits, ids = q8.lmhead_argmax(W, dev(c.x))
    logits, ids = host(logits), host(ids)
    gated = check_lmhead(c, logits, ids)
    assert gated.all()
    assert list(ids) == list(c.planted_rows)
    # lean path: no logits written, same ids
    _, ids2 = q8.lmhead_argmax(W, dev(c.x), logits=False)
    assert np.array_equal(host(ids2), ids)


def test_planted_margin_is_at_least_3_sigma(vocab):
    c, W = vocab
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    for n in range(4):
        r = c.planted_rows[n]
        others = np.delete(ref[n], r)
        assert ref[n, r] - others.max() >= 3 * others.std()


def test_full_vocab_planted_at_3_sigma(vocab):
    """The gate near its edge: token 0's planted row is re-planted to lead
    the runner-up by the +3 sigma margin (sigma the population std of the
    other logits), with the smallest fp16 scale that reaches it; the token
    is gated and the GPU returns that row."""
    note("lmhead 151936x5120 planted at +3 sigma")
    c4, _ = vocab
    c = synth.LmHeadCase(c4.q.copy(), c4.d.copy(), c4.x[:2].copy(), c4.planted_rows[:2].copy(),
                         c4.planted_target[:2].copy())
    r = int(c.planted_rows[0])
    L, _ = oracle.gemv(c.q, c.d, c.x[:1], threads())
    others = np.delete(L[0], r)
    sigma = others.std()
    xn = c.x[0].astype(np.float64)
    s_abs = np.abs(xn).sum()
    c.q[r] = (np.sign(xn) * 127).astype(np.int8)
    c.d[r] = synth.fp16_at_least((others.max() + 3 * sigma) / (127.0 * s_abs))
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    margin = ref[0, r] - np.delete(ref[0], r).max()
    step = 127.0 * s_abs * float(np.spacing(c.d[r, 0]))  # one fp16 step of the scale
    assert 3 * sigma <= margin < 3 * sigma + step
    logits, ids = q8.lmhead_argmax(upload(c.q, c.d), dev(c.x))
    gated = check_lmhead(c, host(logits), host(ids))
    assert gated[0] and int(host(ids)[0]) == r


def test_token_outside_gate_set_takes_a_candidate():
    """Two rows whose logits differ by less than the bound: the token is not
    gated, so any id of its candidate set is correct; the GPU must return
    one of them, the first maximum of its own logits. A third token with
    two identical top rows must return the lower index."""
    note("lmhead candidate-set rule")
    c = synth.lmhead_case(8192, 2048, 3, seed=17)
    V = c.q.shape[0]
    for n in range(3):
        r = int(c.planted_rows[n])
        twin = (r + 1) % V if n < 2 else (r + 4096) % V
        c.q[twin] = c.q[r]
        c.d[twin] = c.d[r]
        if n < 2:
            # one quant one step smaller where |x| is smallest: the twin trails
            # by d * |x_k|, far inside the bound
            k = int(np.argmin(np.abs(c.x[n].astype(np.float64)) + (c.q[r] == 0) * 1e9))
            c.q[twin, k] = c.q[r, k] - np.sign(c.q[r, k])
    ref, A = oracle.gemv(c.q, c.d, c.x, threads())
    istar, gated, cands = oracle.argmax_gate(ref, A)
    assert not gated.any()
    logits, ids = q8.lmhead_argmax(upload(c.q, c.d), dev(c.x))
    logits, ids = host(logits), host(ids)
    check_lmhead(c, logits, ids)
    for n in range(3):
        r = int(c.planted_rows[n])
        assert int(ids[n]) in set(cands[n].tolist()) and int(ids[n]) in {r, (r + 1) % V, (r + 4096) % V}
    r2 = int(c.planted_rows[2])
    assert int(ids[2]) == min(r2, (r2 + 4096) % V)  # exact tie: the lower index


@pytest.mark.parametrize("V,K,N", [(4096, 1024, 3), (1000, 768, 8), (333, 96, 11), (1, 32, 1)])
def test_small_vocab_full_oracle(V, K, N):
    note(f"lmhead small V={V} K={K} N={N}")
    c = synth.lmhead_case(V, K, min(N, V), seed=V)
    if N > V:
        c.x = synth.draw_x(np.random.default_rng(1), N, K)
    logits, ids = q8.lmhead_argmax(upload(c.q, c.d), dev(c.x))
    check_lmhead(c, host(logits), host(ids))


def test_ties_go_to_lowest_index():
    note("lmhead ties")
    K, V = 256, 3000
    rng = np.random.default_rng(0)
    q = rng.integers(-20, 21, size=(V, K)).astype(np.int8)
    d = np.full((V, K // 32), 2.0 ** -6, np.float16)
    x = rng.integers(-2, 3, size=(2, K)).astype(np.float16)  # integer data: logits exact
    q[2500] = 60  # a clear winner for token 0 ...
    x[0] = np.abs(x[0])
    q[1777] = q[2500]  # ... duplicated at a lower index
    q[2999] = q[2500]
    logits, ids = q8.lmhead_argmax(upload(q, d), dev(x))
    logits, ids = host(logits), host(ids)
    assert ids[0] == 1777
    assert ids[1] == oracle.argmax_first(logits)[1]


def test_all_zero_logits_pick_row_zero():
    note("lmhead zeros")
    K, V = 64, 5000
    q = np.zeros((V, K), np.int8)
    d = np.full((V, K // 32), 1.0, np.float16)
    d[::2] = -0.0
    x = np.ones((1, K), np.float16)
    q[::3] = -1
    d[::3] = 0.0  # -0 * ... and +0 products mixed: all logits are zero of either sign
    logits, ids = q8.lmhead_argmax(upload(q, d), dev(x))
    assert np.all(host(logits) == 0)
    assert host(ids)[0] == 0


def test_workspace_reused_across_shapes_returns_to_zero():
    """One zero-filled workspace, sized for the largest vocabulary, serves
    calls whose grids differ (vocab size, token count, multi-pass N, with
    and without logits): every call's ids match the oracle, the ids-only
    call (which goes through the workspace's scratch logits at 1-2 tokens)
    returns the same ids, and the whole workspace (argmax slots, counters
    and scratch) reads zero after each call, ready for the next one."""
    shapes = [(4096, 1024, 1), (333, 96, 11), (20000, 512, 4), (1, 32, 1), (9, 64, 2),
              (20000, 512, 2), (4096, 1024, 8), (20000, 512, 1)]
    nws = q8.lmhead_ws_bytes(max(V for V, _, _ in shapes), 1)
    assert nws >= 4608 + 8 * 20000
    ws = torch.zeros((nws,), dtype=torch.uint8, device="cuda")
    for i, (V, K, N) in enumerate(shapes):
        note(f"lmhead ws reuse V={V} K={K} N={N}")
        c = synth.lmhead_case(V, K, min(N, V), seed=100 + i)
        if N > V:
            c.x = synth.draw_x(np.random.default_rng(i), N, K)
        W = upload(c.q, c.d)
        logits, ids = q8.lmhead_argmax(W, dev(c.x), ws=ws)
        check_lmhead(c, host(logits), host(ids))
        assert not host(ws).any(), "workspace not returned to zero"
        _, ids2 = q8.lmhead_argmax(W, dev(c.x), logits=False, ws=ws)
        assert np.array_equal(host(ids2), host(ids)), "ids-only call differs"
        assert not host(ws).any(), "workspace not returned to zero after an ids-only call"


def test_workspace_smaller_than_the_vocabulary_needs_is_refused():
    """The workspace grows with V (scratch logits for two tokens): one sized
    for a smaller vocabulary is refused with Q8_ERR_WORKSPACE, nothing
    launched."""
    c = synth.lmhead_case(4096, 256, 1, seed=7)
    ws = torch.zeros((q8.lmhead_ws_bytes(1024, 1),), dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="-5|WORKSPACE|workspace"):
        q8.lmhead_argmax(upload(c.q, c.d), dev(c.x), logits=False, ws=ws)


# ---------------------------------------------------------------- draft head (vocabulary subset)
def gather(c, rows):
    return synth.LmHeadCase(c.q[rows], c.d[rows], c.x, c.planted_rows, c.planted_target)


@pytest.mark.parametrize("N", [1, 4])
def test_draft_head_subset_of_full_vocab(vocab, N):
    """A 32768-row ranked subset containing the planted rows: ids come back
    as vocabulary ids and match the oracle on the subset; the subset's
    logits are bitwise the full head's logits at those rows."""
    note(f"draft head 32768 of 151936 N={N}")
    c4, W = vocab
    rng = np.random.default_rng(5)
    others = np.setdiff1d(np.arange(151936), c4.planted_rows[:4])
    rows = rng.choice(others, 32768, replace=False).astype(np.int32)
    rows[rng.choice(32768, 4, replace=False)] = c4.planted_rows[:4]
    assert len(np.unique(rows)) == 32768
    sub = gather(c4, rows)
    Ws = upload(sub.q, sub.d)
    x = dev(c4.x[:N])
    logits, ids = q8.lmhead_argmax(Ws, x, row_ids=dev(rows))
    logits, ids = host(logits), host(ids)
    L, A = oracle.gemv(sub.q, sub.d, c4.x[:N], threads())
    assert_parity(logits, L, A, what="draft logits")
    want, gated, cands = oracle.argmax_masked(L, A, rows)
    for n in range(N):
        assert ids[n] == want[n] if gated[n] else ids[n] in cands[n]
    assert list(ids) == list(c4.planted_rows[:N])
    full_logits, _ = q8.lmhead_argmax(W, x)
    assert np.array_equal(host(full_logits)[:, rows].view(np.uint32), logits.view(np.uint32))
    # lean path
    _, ids2 = q8.lmhead_argmax(Ws, x, logits=False, row_ids=dev(rows))
    assert np.array_equal(host(ids2), ids)


def test_draft_head_ties_go_to_earlier_subset_position():
    note("draft head ties")
    K, S = 256, 900
    rng = np.random.default_rng(3)
    q = rng.integers(-20, 21, size=(S, K)).astype(np.int8)
    d = np.full((S, K // 32), 2.0 ** -6, np.float16)
    x = np.abs(rng.integers(-2, 3, size=(1, K))).astype(np.float16)  # integer data: exact logits
    q[500] = 60
    q[120] = q[500]  # the same winning row at an earlier position
    rows = rng.permutation(100000)[:S].astype(np.int32)
    rows[120], rows[500] = 99999, 3  # the earlier position has the larger vocabulary id
    _, ids = q8.lmhead_argmax(upload(q, d), dev(x), row_ids=dev(rows))
    assert host(ids)[0] == 99999


def test_draft_head_identity_subset_equals_plain_head():
    note("draft head identity subset")
    c = synth.lmhead_case(5000, 1024, 3, seed=9)
    W = upload(c.q, c.d)
    x = dev(c.x)
    l1, i1 = q8.lmhead_argmax(W, x)
    l2, i2 = q8.lmhead_argmax(W, x, row_ids=dev(np.arange(5000, dtype=np.int32)))
    assert np.array_equal(host(i1), host(i2))
    assert np.array_equal(host(l1).view(np.uint32), host(l2).view(np.uint32))
