"""The routed FFN without a workspace (q8_moe_ffn_noalloc, for callers that
cannot allocate) against q8_moe_ffn with a caller workspace.

Through the C ABI on the full 128-expert top-8 layer: two no-allocation
calls in a row, the second with fewer tokens, each bitwise equal to the
workspace entry point on the same inputs; then a capture into a HIP graph
replayed with the routing changed between replays; a shape whose
workspace exceeds the scratch array is refused before any launch.
"""
import numpy as np
import pytest

import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import dev, host, note, require_gpu, torch, upload_bank

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer():
    require_gpu()
    c = synth.moe_case(E=128, F=768, H=2048, T=16, topk=8, seed=0)
    B = (upload_bank(c.q_gate, c.d_gate), upload_bank(c.q_up, c.d_up),
         upload_bank(c.q_down, c.d_down))
    return c, B


def _with_ws(c, B, T):
    ws = torch.zeros((q8.moe_ws_bytes(c.E, T, c.topk, c.F, c.H),), dtype=torch.uint8, device="cuda")
    return host(q8.moe_ffn(*B, dev(c.expert_ids[:T]), dev(c.gate_w[:T]), dev(c.x[:T]), ws=ws))


def test_noalloc_equals_workspace_entry_on_two_calls(layer):
    c, B = layer
    note("moe noalloc T=16 then T=4")
    ref16, ref4 = _with_ws(c, B, 16), _with_ws(c, B, 4)
    got16 = host(q8.moe_ffn_noalloc(*B, dev(c.expert_ids), dev(c.gate_w), dev(c.x)))
    got4 = host(q8.moe_ffn_noalloc(*B, dev(c.expert_ids[:4]), dev(c.gate_w[:4]), dev(c.x[:4])))
    assert np.array_equal(got16.view(np.uint32), ref16.view(np.uint32))
    assert np.array_equal(got4.view(np.uint32), ref4.view(np.uint32))


def test_noalloc_graph_replays(layer):
    c, B = layer
    note("moe noalloc graph replay")
    ids = dev(c.expert_ids)
    gw, x = dev(c.gate_w), dev(c.x)
    out = torch.empty((16, c.H), dtype=torch.float32, device="cuda")
    q8.moe_ffn_noalloc(*B, ids, gw, x, out=out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q8.moe_ffn_noalloc(*B, ids, gw, x, out=out)
    rng = np.random.default_rng(3)
    for _ in range(3):
        new_ids = np.stack([rng.choice(c.E, c.topk, replace=False) for _ in range(16)]).astype(np.int32)
        ids.copy_(torch.from_numpy(new_ids).cuda())
        torch.cuda.synchronize()
        g.replay()
        got = host(out)
        cc = synth.MoeCase(c.q_gate, c.d_gate, c.q_up, c.d_up, c.q_down, c.d_down, c.x, new_ids,
                           c.gate_w)
        assert np.array_equal(got.view(np.uint32), _with_ws(cc, B, 16).view(np.uint32))


def test_noalloc_refuses_shapes_beyond_the_scratch(layer):
    c, B = layer
    T = 128  # 1024 pairs: h and y_pair alone need 11.5 MB
    assert q8.moe_ws_bytes(c.E, T, c.topk, c.F, c.H) > q8.noalloc_scratch_bytes()
    rng = np.random.default_rng(5)
    ids = np.stack([rng.choice(c.E, c.topk, replace=False) for _ in range(T)]).astype(np.int32)
    gw = np.full((T, c.topk), 1.0 / c.topk, np.float32)
    x = synth.draw_x(rng, T, c.H)
    with pytest.raises(q8.Q8Error) as e:
        q8.moe_ffn_noalloc(*B, dev(ids), dev(gw), dev(x))
    assert e.value.status == -5
