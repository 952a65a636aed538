"""Every hot entry point replays correctly inside a HIP graph.

The decode step is one graph replay per token (memra wiki, feature list:
CUDA-graph decode). Each test captures calls on a side stream, replays the
graph several times with eager work and synchronisations in between (the
outputs are cleared eagerly before each replay), and requires every replay
to equal the eager result bitwise. The LM head's workspace counters must be
back at zero after each replay, or the next replay's ids would be wrong.
"""
import numpy as np
import pytest

import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import dev, host, note, require_gpu, torch, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def capture(step):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def replay_matches(g, outs, eager, clear):
    for r in range(4):
        for t in clear:
            t.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert np.array_equal(host(o).view(np.uint8), e.view(np.uint8)), f"replay {r}"


def test_gemv_pair_silu_q4_in_one_graph():
    note("graph: gemv, pair, silu pair, q4")
    c = synth.pair_case(3000, 1024, 4, seed=2)
    Wa, Wb = upload(c.qa, c.da), upload(c.qb, c.db)
    q4 = synth.q4_0_case(2000, 1024, 4, seed=3)
    W4 = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q4.q, q4.d))
    x = dev(c.x)
    y = torch.empty((4, 3000), device="cuda")
    ya = torch.empty((4, 3000), device="cuda")
    yb = torch.empty((4, 3000), device="cuda")
    h = torch.empty((4, 3000), device="cuda", dtype=torch.float16)
    y4 = torch.empty((4, 2000), device="cuda")
    outs = [y, ya, yb, h, y4]

    def step():
        q8.gemv(Wa, x, out=y)
        q8.gemv_pair(Wa, Wb, x, out_a=ya, out_b=yb)
        q8.gemv_pair_silu(Wa, Wb, x, out=h)
        q8.gemv(W4, x, out=y4)

    step()
    torch.cuda.synchronize()
    eager = [host(o).copy() for o in outs]
    g = capture(step)
    replay_matches(g, outs, eager, outs)


def test_lmhead_and_draft_head_graph_replays_reset_the_workspace():
    note("graph: lm head + draft head")
    c = synth.lmhead_case(20000, 1024, 3, seed=5)
    W = upload(c.q, c.d)
    rows = np.random.default_rng(0).choice(20000, 4096, replace=False).astype(np.int32)
    rows[:3] = c.planted_rows[:3]
    Wd = upload(c.q[rows], c.d[rows])
    rid = dev(rows)
    x = dev(c.x)
    ws1 = torch.zeros((q8.lmhead_ws_bytes(20000, 3),), dtype=torch.uint8, device="cuda")
    ws2 = torch.zeros((q8.lmhead_ws_bytes(4096, 3),), dtype=torch.uint8, device="cuda")
    logits = torch.empty((3, 20000), device="cuda")
    ids = torch.empty((3,), dtype=torch.int32, device="cuda")
    ids2 = torch.empty((3,), dtype=torch.int32, device="cuda")
    # one token with logits: the GEMV + argmax pair of launches
    ws3 = torch.zeros((q8.lmhead_ws_bytes(20000, 1),), dtype=torch.uint8, device="cuda")
    logits1 = torch.empty((1, 20000), device="cuda")
    ids1 = torch.empty((1,), dtype=torch.int32, device="cuda")
    # two tokens, ids only, draft head: GEMV into the workspace's scratch + argmax
    ws4 = torch.zeros((q8.lmhead_ws_bytes(4096, 2),), dtype=torch.uint8, device="cuda")
    ids4 = torch.empty((2,), dtype=torch.int32, device="cuda")

    def step():
        q8.lmhead_argmax(W, x, logits=logits, ids=ids, ws=ws1)
        q8.lmhead_argmax(Wd, x, logits=False, ids=ids2, ws=ws2, row_ids=rid)
        q8.lmhead_argmax(W, x[1:2], logits=logits1, ids=ids1, ws=ws3)
        q8.lmhead_argmax(Wd, x[1:3], logits=False, ids=ids4, ws=ws4, row_ids=rid)

    step()
    torch.cuda.synchronize()
    eager = [host(logits).copy(), host(ids).copy(), host(ids2).copy(), host(logits1).copy(),
             host(ids1).copy(), host(ids4).copy()]
    assert list(eager[1]) == list(c.planted_rows[:3]) and list(eager[2]) == list(c.planted_rows[:3])
    assert eager[4][0] == c.planted_rows[1] and list(eager[5]) == list(c.planted_rows[1:3])
    assert np.array_equal(eager[3][0].view(np.uint32), eager[0][1].view(np.uint32))
    g = capture(step)
    for r in range(4):
        logits.fill_(0)
        logits1.fill_(0)
        ids.fill_(-1)
        ids2.fill_(-1)
        ids1.fill_(-1)
        ids4.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(logits).view(np.uint32), eager[0].view(np.uint32))
        assert np.array_equal(host(logits1).view(np.uint32), eager[3].view(np.uint32))
        assert np.array_equal(host(ids), eager[1]) and np.array_equal(host(ids2), eager[2])
        assert np.array_equal(host(ids1), eager[4]) and np.array_equal(host(ids4), eager[5])
        assert not any(host(w).any() for w in (ws1, ws2, ws3, ws4)), \
            f"replay {r}: workspace not reset"
