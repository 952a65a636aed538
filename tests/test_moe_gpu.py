"""Parity of the routed-expert path (q8_moe_gemv, q8_moe_ffn) with the oracle.

Full-size workload: 128 experts, gate/up [768][2048] and down [2048][768]
Q8_0, top-8 routing of 16 tokens (ids drawn without replacement per
token, softmax gate weights). Gated stage by stage, each stage against the
exact inputs it consumed: the device CSR equals the oracle's; h is within
its propagated bound of silu(g)*u; the down GEMV is within 1e-3*sum|dqh| of
the oracle run on the GPU's own h; the combine is within fp32 rounding of
the fp64 combine of the GPU's y_pair; end to end within the propagated
bound of the fp64 chain. Invariances: a token's output is bitwise
unchanged when the other tokens' ids or activations change (the pages'
batch-composition contract), top-1 routing equals plain q8_gemv on the
chosen expert bitwise, and permuting the expert bank (with ids remapped)
changes nothing.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import (assert_parity, dev, host, note, require_gpu, threads, torch, upload,
                            upload_bank)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def banks(c):
    return (upload_bank(c.q_gate, c.d_gate), upload_bank(c.q_up, c.d_up),
            upload_bank(c.q_down, c.d_down))


def run_ffn(c, B, ids=None, x=None, ws=None):
    ids = c.expert_ids if ids is None else ids
    x = c.x if x is None else x
    g, u, d = B
    T, topk = ids.shape
    if ws is None:
        ws = torch.zeros((q8.moe_ws_bytes(c.E, T, topk, c.F, c.H),), dtype=torch.uint8, device="cuda")
    out = q8.moe_ffn(g, u, d, dev(ids.astype(np.int32)), dev(c.gate_w), dev(x), ws=ws)
    return host(out), ws


@pytest.fixture(scope="module")
def full():
    c = synth.moe_case(E=128, F=768, H=2048, T=16, topk=8, seed=0)
    return c, banks(c)


def stagewise(c, B):
    out, ws = run_ffn(c, B)
    T, topk = c.expert_ids.shape
    v = q8.moe_ws_views(ws, c.E, T, topk, c.F, c.H)
    counts, offsets, pairs, active = oracle.moe_route(c.expert_ids, c.E)
    assert np.array_equal(host(v["counts"]), counts)
    assert np.array_equal(host(v["offsets"]), offsets)
    assert np.array_equal(host(v["pairs"]), pairs)
    na = int(host(v["n_active"])[0])
    assert na == len(active) and np.array_equal(host(v["active"])[:na], active)
    s1 = oracle.moe_gate_up(c, threads())
    h = host(v["h"])
    err = np.abs(h - s1["h"])
    assert np.all(err <= s1["bh"]), f"h: {(err > s1['bh']).sum()} outside bound"
    y_pair = host(v["y_pair"])
    yref, Ay = oracle.moe_down(c, h, threads())
    assert_parity(y_pair, yref, Ay, what="down on GPU h")
    comb, S = oracle.moe_combine(c.gate_w, y_pair)
    assert np.all(np.abs(out - comb) <= 1e-6 * S + 1e-30)
    e2e = oracle.moe_ffn(c, threads())
    assert np.all(np.abs(out - e2e["out"]) <= e2e["bound"])
    return out


def test_full_size_stagewise(full):
    note("moe e128 top8 t16 stagewise")
    c, B = full
    stagewise(c, B)


def test_batch_composition_invariance(full):
    note("moe batch composition")
    c, B = full
    base, _ = run_ffn(c, B)
    ids2 = c.expert_ids.copy()
    rng = np.random.default_rng(7)
    for t in range(1, c.T):
        ids2[t] = rng.choice(c.E, c.topk, replace=False)
    x2 = c.x.copy()
    x2[1:] = synth.draw_x(rng, c.T - 1, c.H)
    out2, _ = run_ffn(c, B, ids=ids2, x=x2)
    assert np.array_equal(out2[0].view(np.uint32), base[0].view(np.uint32))
    # a batch of one token gives the same row too
    c1 = synth.MoeCase(c.q_gate, c.d_gate, c.q_up, c.d_up, c.q_down, c.d_down, c.x[:1],
                       c.expert_ids[:1], c.gate_w[:1])
    out1, _ = run_ffn(c1, B)
    assert np.array_equal(out1[0].view(np.uint32), base[0].view(np.uint32))


def test_routed_gemv_equals_plain_gemv(full):
    """Per-pair outputs of q8_moe_gemv equal q8_gemv on the chosen expert, bitwise."""
    note("moe routed gemv vs plain gemv")
    c, (g, u, d) = full
    ids = dev(c.expert_ids.astype(np.int32))
    x = dev(c.x)
    yp = host(q8.moe_gemv(g, ids, x))  # [T*topk][F]
    for t in (0, 5, 15):
        for j in (0, 7):
            e = int(c.expert_ids[t, j])
            ref = host(q8.gemv(g.expert(e), x[t:t + 1].contiguous()))[0]
            assert np.array_equal(yp[t * c.topk + j].view(np.uint32), ref.view(np.uint32))
    # and the combined form
    gw = dev(c.gate_w)
    yc = host(q8.moe_gemv(g, ids, x, gate_w=gw))
    comb, S = oracle.moe_combine(c.gate_w, yp)
    assert np.all(np.abs(yc - comb) <= 1e-6 * S + 1e-30)


@pytest.mark.parametrize("E,F,H,T,topk", [(8, 64, 128, 5, 2), (16, 96, 256, 3, 4), (4, 32, 768, 9, 4),
                                          (3, 160, 96, 12, 3)])
def test_small_configs_stagewise(E, F, H, T, topk):
    note(f"moe small E={E} F={F} H={H} T={T} topk={topk}")
    c = synth.moe_case(E, F, H, T, topk, seed=E + F)
    stagewise(c, banks(c))


def test_full_dims_larger_batch_stagewise():
    """The layer's shapes at 40 tokens (320 pairs, about 2.5 per active
    expert): experts spanning several two-pair slots, every stage against
    the oracle."""
    note("moe e128 top8 t40 stagewise")
    c = synth.moe_case(E=128, F=768, H=2048, T=40, topk=8, seed=40)
    stagewise(c, banks(c))


def test_expert_permutation_invariance():
    note("moe expert permutation")
    c = synth.moe_case(E=12, F=64, H=256, T=6, topk=3, seed=3)
    base, _ = run_ffn(c, banks(c))
    perm = np.random.default_rng(0).permutation(c.E)  # new index of old expert e = inv[e]
    inv = np.argsort(perm)
    cp = synth.MoeCase(c.q_gate[perm], c.d_gate[perm], c.q_up[perm], c.d_up[perm], c.q_down[perm],
                       c.d_down[perm], c.x, inv[c.expert_ids].astype(np.int32), c.gate_w)
    out, _ = run_ffn(cp, banks(cp))
    assert np.array_equal(out.view(np.uint32), base.view(np.uint32))


def test_routed_gemv_fp32_per_pair_inputs():
    note("moe routed gemv fp32 per-pair x")
    c = synth.moe_case(E=6, F=64, H=768, T=4, topk=2, seed=11)
    W = upload_bank(c.q_down, c.d_down)  # [H][F] experts, input dim F
    h = np.random.default_rng(2).normal(0, 1, size=(c.T * c.topk, c.F)).astype(np.float32)
    yp = host(q8.moe_gemv(W, dev(c.expert_ids), dev(h), x_per_pair=True))
    ref, A = oracle.moe_down(c, h)
    assert_parity(yp, ref, A, what="per-pair fp32")


def test_invalid_ids_are_skipped_and_counted():
    """Out-of-range expert ids: the pair is left out (zero row) and the
    workspace error word counts it; a later valid call writes 0 again, also
    when the same workspace is replayed in a graph."""
    note("moe invalid ids")
    c = synth.moe_case(E=5, F=64, H=128, T=3, topk=2, seed=1)
    W = upload_bank(c.q_gate, c.d_gate)
    ws = torch.full((q8.moe_ws_bytes(c.E, 3, 2, 0, 64),), 0x7F, dtype=torch.uint8, device="cuda")
    views = q8.moe_ws_views(ws, c.E, 3, 2, 0, 64)
    ids = c.expert_ids.copy()
    ids[1, 1] = 99
    ids[2, 0] = -3
    yp = host(q8.moe_gemv(W, dev(ids), dev(c.x), ws=ws))
    assert int(host(views["n_bad_ids"])[0]) == 2
    assert np.all(yp[1 * 2 + 1] == 0) and np.all(yp[2 * 2 + 0] == 0)
    e = int(ids[1, 0])
    ref, A = oracle.gemv(c.q_gate[e], c.d_gate[e], c.x[1:2])
    assert_parity(yp[2:3], ref, A, what="valid slot next to invalid one")
    good = dev(c.expert_ids)
    q8.moe_gemv(W, good, dev(c.x), ws=ws)
    assert int(host(views["n_bad_ids"])[0]) == 0
    # under graph replay: the word follows the ids of each replay
    idt = dev(ids)
    xt = dev(c.x)
    out = torch.empty((6, 64), dtype=torch.float32, device="cuda")
    q8.moe_gemv(W, idt, xt, out=out, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.moe_gemv(W, idt, xt, out=out, ws=ws)
    for bad, want in ((ids, 2), (c.expert_ids, 0), (ids, 2)):
        idt.copy_(torch.from_numpy(np.ascontiguousarray(bad)).cuda())
        torch.cuda.synchronize()
        g.replay()
        assert int(host(views["n_bad_ids"])[0]) == want


def test_many_experts_route_in_its_own_launch():
    """With 4096 experts and 4096 pairs the route's LDS does not fit next to
    the activations, so it runs as a separate launch before the routed
    kernels; the results and the workspace must be the same as ever."""
    note("moe E=4096 T=512 separate route launch")
    c = synth.moe_case(E=4096, F=32, H=128, T=512, topk=8, seed=21)
    stagewise(c, banks(c))
    W = upload_bank(c.q_gate, c.d_gate)
    ids = c.expert_ids.copy()
    ids[7, 3] = -1
    ws = torch.zeros((q8.moe_ws_bytes(c.E, c.T, c.topk, 0, c.F),), dtype=torch.uint8, device="cuda")
    yp = host(q8.moe_gemv(W, dev(ids), dev(c.x), ws=ws))
    assert np.all(yp[7 * 8 + 3] == 0)
    assert int(host(q8.moe_ws_views(ws, c.E, c.T, c.topk, 0, c.F)["n_bad_ids"])[0]) == 1
    e = int(ids[7, 2])
    ref, A = oracle.gemv(c.q_gate[e], c.d_gate[e], c.x[7:8])
    assert_parity(yp[7 * 8 + 2:7 * 8 + 3], ref, A, what="valid slot next to invalid one")
