"""Parity of the on-device router (q8_moe_topk_softmax, q8_moe_router) with the oracle.

Picked experts are integer results of comparisons of the same fp32 logits
on both sides, so they must equal the oracle's exactly (including the rule
for equal logits and -0 == +0). Gate weights are within the derived fp32
bound of the fp64 softmax (oracle.topk_softmax_bound). Invariance: a
token's experts and weights are bitwise the same whether it is routed alone
or in a batch. End to end: q8_moe_router's logits are q8_gemv's bitwise,
its outputs feed q8_moe_ffn, and the routed layer captured in a graph
replays bitwise equal to eager calls.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import dev, host, note, require_gpu, threads, torch, upload, upload_bank

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check_router(L, ids, gw, topk):
    rid, rw, dl = oracle.topk_softmax(L, topk)
    assert np.array_equal(ids, rid), "picked experts differ from the oracle"
    err = np.abs(gw.astype(np.float64) - rw)
    bound = oracle.topk_softmax_bound(rw, dl)
    assert np.all(err <= bound), f"gate weights off by {np.max(err - bound):.3e} beyond the bound"


@pytest.mark.parametrize("T,E,topk", [(16, 128, 8), (37, 1000, 32), (3, 4096, 64), (5, 1, 1),
                                      (7, 63, 63), (2, 65, 2), (64, 256, 8)])
def test_topk_softmax_matches_oracle(T, E, topk):
    note(f"router T={T} E={E} topk={topk}")
    L = synth.router_case(T, E, seed=E + T)
    ids, gw = q8.moe_topk_softmax(dev(L), topk)
    check_router(L, host(ids), host(gw), topk)


def test_topk_softmax_extreme_logits():
    note("router extreme logits")
    rng = np.random.default_rng(7)
    L = rng.normal(0, 1, size=(6, 200)).astype(np.float32)
    L[0, :] = np.float32(-3e38)
    L[0, 17] = np.float32(3e38)  # weights underflow to exactly 1, 0, 0, ...
    L[1, ::3] = np.float32(1e-42)  # subnormals and zeros
    L[1, 1::3] = np.float32(0.0)
    L[1, 2::3] = np.float32(-0.0)
    L[2, :] = np.float32(-1.0)  # all equal: the lowest experts, equal weights
    L[3, 100:] = np.float32(88.0)  # many ties at the top
    L[4] = np.arange(200, dtype=np.float32)[::-1] * np.float32(1e-3)
    L[5] = -np.abs(L[5])
    for k in (1, 8, 64):
        ids, gw = q8.moe_topk_softmax(dev(L), k)
        check_router(L, host(ids), host(gw), k)


def test_routing_is_independent_of_the_batch():
    note("router batch invariance")
    L = synth.router_case(24, 512, seed=11)
    ids, gw = q8.moe_topk_softmax(dev(L), 16)
    ids, gw = host(ids), host(gw)
    for t in (0, 5, 23):
        i1, g1 = q8.moe_topk_softmax(dev(L[t:t + 1]), 16)
        assert np.array_equal(host(i1)[0], ids[t])
        assert np.array_equal(host(g1)[0].view(np.uint32), gw[t].view(np.uint32))
    # other tokens' logits changed: token 3 unchanged
    L2 = L.copy()
    L2[np.arange(24) != 3] = synth.router_case(23, 512, seed=12)
    i2, g2 = q8.moe_topk_softmax(dev(L2), 16)
    assert np.array_equal(host(i2)[3], ids[3])
    assert np.array_equal(host(g2)[3].view(np.uint32), gw[3].view(np.uint32))


@pytest.fixture(scope="module")
def routed_layer():
    c = synth.moe_case(E=128, F=768, H=2048, T=16, topk=8, seed=0)
    rng = np.random.default_rng(21)
    qr, dr = synth.draw_weights(rng, 128, 2048)
    return c, upload(qr, dr), (qr, dr), (upload_bank(c.q_gate, c.d_gate),
                                         upload_bank(c.q_up, c.d_up),
                                         upload_bank(c.q_down, c.d_down))


def test_router_from_q8_matrix_feeds_the_experts(routed_layer):
    note("router from Q8 matrix -> moe_ffn")
    c, Wr, (qr, dr), (g, u, d) = routed_layer
    x = dev(c.x)
    logits, ids, gw = q8.moe_router(Wr, x, 8)
    ref_logits = q8.gemv(Wr, x)
    assert np.array_equal(host(logits).view(np.uint32), host(ref_logits).view(np.uint32))
    L = host(logits)
    check_router(L, host(ids), host(gw), 8)
    # the logits themselves against the oracle's GEMV bound
    y, A = oracle.gemv(qr, dr, c.x, threads())
    ok, rel, nbad = oracle.check_close(L.astype(np.float64), y, A)
    assert ok, f"router logits: {nbad} outside the bound"
    # the routed experts consume the device routing directly
    ws = torch.zeros((q8.moe_ws_bytes(c.E, 16, 8, c.F, c.H),), dtype=torch.uint8, device="cuda")
    out = host(q8.moe_ffn(g, u, d, ids, gw, x, ws=ws))
    cc = synth.MoeCase(c.q_gate, c.d_gate, c.q_up, c.d_up, c.q_down, c.d_down, c.x,
                       host(ids).astype(np.int32), host(gw))
    ref = oracle.moe_ffn(cc, threads())
    assert np.all(np.abs(out - ref["out"]) <= ref["bound"])


def test_routed_layer_graph_replays_match_eager(routed_layer):
    note("router + moe_ffn in a graph")
    c, Wr, _, (g, u, d) = routed_layer
    x = dev(c.x)
    T, topk = 16, 8
    logits = torch.empty((T, c.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    out = torch.empty((T, c.H), dtype=torch.float32, device="cuda")
    ws = torch.zeros((q8.moe_ws_bytes(c.E, T, topk, c.F, c.H),), dtype=torch.uint8, device="cuda")

    def step():
        q8.moe_router(Wr, x, topk, logits=logits, ids=ids, gate_w=gw)
        q8.moe_ffn(g, u, d, ids, gw, x, out=out, ws=ws)

    step()
    eager = (host(ids).copy(), host(gw).copy(), host(out).copy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    for r in range(3):
        out.fill_(0.0)
        gw.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ids), eager[0]), f"replay {r}: ids"
        assert np.array_equal(host(gw).view(np.uint32), eager[1].view(np.uint32)), f"replay {r}: gate_w"
        assert np.array_equal(host(out).view(np.uint32), eager[2].view(np.uint32)), f"replay {r}: out"


@pytest.mark.parametrize("T,E,K,q4,xf32,topk", [
    (16, 128, 2048, False, False, 8),   # the routed layer's router: two passes in one launch
    (1, 100, 1024, False, False, 6),    # one token (keys in registers)
    (9, 100, 1024, False, False, 6),    # ragged expert count, a pass of 8 and one of 1
    (64, 128, 2048, False, False, 8),   # eight passes in one launch
    (12, 64, 2048, False, False, 4),    # keys in one register per lane
    (13, 200, 512, False, False, 16),   # 32 lanes per row, ragged last group
    (17, 256, 256, False, False, 64),   # 16 lanes per row, topk at its maximum
    (9, 9, 256, False, False, 9),       # topk = E = 9: every expert picked
    (64, 256, 512, False, False, 64),   # 64 tokens, four keys per lane
    (7, 256, 256, False, False, 64),    # one pass of 7
    (65, 128, 2048, False, False, 8),   # eight passes of 8 and one of 1
    (64, 128, 2048, False, True, 8),    # fp32 x
    (16, 256, 4096, False, False, 8),   # 256 experts over K = 4096
    (7, 4096, 512, False, False, 64),   # E and topk at their maximum (keys in LDS)
    (16, 128, 2048, True, False, 8),    # Q4_0 router matrix
    (5, 96, 96, True, True, 4),         # Q4_0, fp32 x, three blocks per row
])
def test_router_equals_gemv_then_topk(T, E, K, q4, xf32, topk):
    """q8_moe_router returns bitwise q8_gemv's logits and bitwise
    q8_moe_topk_softmax's ids and weights over them, with duplicated router
    rows so that equal logits occur; the picks also match the oracle's."""
    note(f"router T={T} E={E} K={K} q4={q4} xf32={xf32} topk={topk}")
    rng = np.random.default_rng(T * 7919 + E)
    if q4:
        q, d = synth.draw_weights_q4_0(rng, E, K)
    else:
        q, d = synth.draw_weights(rng, E, K)
    q[E // 2] = q[E // 3]  # equal rows: equal logits, the lower expert first
    d[E // 2] = d[E // 3]
    W = q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q, d)) if q4 else upload(q, d)
    x = synth.draw_x(rng, T, K)
    xd = dev(x.astype(np.float32) if xf32 else x)
    logits, ids, gw = q8.moe_router(W, xd, topk)
    ref_logits = q8.gemv(W, xd)
    assert np.array_equal(host(logits).view(np.uint32), host(ref_logits).view(np.uint32))
    rid, rgw = q8.moe_topk_softmax(ref_logits, topk)
    assert np.array_equal(host(ids), host(rid))
    assert np.array_equal(host(gw).view(np.uint32), host(rgw).view(np.uint32))
    check_router(host(logits), host(ids), host(gw), topk)
