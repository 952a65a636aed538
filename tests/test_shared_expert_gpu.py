"""Parity of the shared expert (q8_moe_shared_expert) with the oracle.

out[t] += sigmoid(Wsg x_t) * Wd (silu(Wg x_t) * Wu x_t), accumulated into
a routed output: every output within the bound oracle.shared_expert
propagates from the GEMV bounds, at the routed layer's expert shape (F =
768, H = 2048) for 1 and 16 tokens (two passes), on ragged small shapes,
with Q4_0 matrices and fp32 activations. A token's result is bitwise the
same alone or in a batch, the workspace needs no clearing, and the call
replays from a graph bitwise.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import dev, host, note, require_gpu, threads, torch, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _case(T, F, H, seed, q4=False, xf32=False):
    rng = np.random.default_rng(seed)
    draw = synth.draw_weights_q4_0 if q4 else synth.draw_weights
    qg, dg = draw(rng, F, H)
    qu, du = draw(rng, F, H)
    qd, dd = draw(rng, H, F)
    qs, ds = draw(rng, 1, H)
    x = synth.draw_x(rng, T, H)
    if xf32:
        x = x.astype(np.float32)
    base = rng.normal(0.0, 1.0, size=(T, H)).astype(np.float32)
    pack = (lambda q, d: q8.pack_q4_0(synth.to_gguf_q4_0_blocks(q, d))) if q4 else upload
    mats = [pack(qg, dg), pack(qu, du), pack(qd, dd), pack(qs, ds)]
    return (qg, dg, qu, du, qd, dd, qs, ds, x, base), mats


def _run(mats, x, base, ws=None):
    out = dev(base.copy())
    q8.moe_shared_expert(*mats, dev(x), out, ws=ws)
    return host(out)


@pytest.mark.parametrize("T,F,H,q4,xf32", [
    (1, 768, 2048, False, False),   # the routed layer's expert shape, one token
    (16, 768, 2048, False, False),  # two passes of 8
    (5, 96, 256, True, True),       # Q4_0, fp32 x
    (11, 160, 96, False, True),     # ragged, three blocks per row, two passes
    (3, 64, 1024, True, False),
])
def test_shared_expert_matches_oracle(T, F, H, q4, xf32):
    note(f"shared expert T={T} F={F} H={H} q4={q4} xf32={xf32}")
    args, mats = _case(T, F, H, seed=T * 31 + F, q4=q4, xf32=xf32)
    got = _run(mats, args[8], args[9])
    r = oracle.shared_expert(*args, threads=threads())
    err = np.abs(got.astype(np.float64) - r["out"])
    assert np.all(err <= r["bound"]), f"max excess {np.max(err - r['bound']):.3e}"
    assert np.abs(r["out"] - args[9]).max() > 1e-4  # the expert changed the output


def test_shared_expert_is_per_token_and_needs_no_clear():
    """Token 3 alone gives bitwise its result inside a 12-token batch; the
    same (uncleared) workspace serves both calls."""
    note("shared expert batch invariance")
    args, mats = _case(12, 768, 2048, seed=3)
    x, base = args[8], args[9]
    ws = torch.full((q8.moe_shared_ws_bytes(768, 2048, 12),), 0x7f, dtype=torch.uint8,
                    device="cuda")
    full = _run(mats, x, base, ws)
    one = _run(mats, x[3:4].copy(), base[3:4].copy(), ws)
    assert np.array_equal(one.view(np.uint32), full[3:4].view(np.uint32))


def test_shared_expert_graph_replay():
    note("shared expert graph replay")
    args, mats = _case(4, 96, 512, seed=8)
    x = dev(args[8])
    base = dev(args[9])
    out = base.clone()
    ws = torch.empty((q8.moe_shared_ws_bytes(96, 512, 4),), dtype=torch.uint8, device="cuda")

    def step():
        q8.moe_shared_expert(*mats, x, out, ws=ws)

    out.copy_(base)
    step()
    torch.cuda.synchronize()
    eager = host(out).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(3):
        out.copy_(base)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), eager.view(np.uint32)), f"replay {r}"
