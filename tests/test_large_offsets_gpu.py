"""Weights past 4 GiB: every address of a row, a scale, an expert and an
output is computed in 64 bits.

One Q8_0 matrix of 1,099,776 x 4096 (4.5 GB of quants: rows from 524,288
on start past 2^31 bytes, rows from 1,048,576 on past 2^32), drawn with
``synth.draw_weights_tiled`` (quant rows repeat every 4099 rows and scale
rows every 4111, so no row repeats another's pair). For K = 4096 the packer's planes are the
quant matrix and the scale matrix themselves (ld_qs = K, ld_d = K/32, no
padding), which the test asserts before uploading them as they are. Two
tokens, each with its argmax planted at a row past 2^32 bytes.

- q8_gemv at N = 2, every output against the oracle; at N = 1 each token
  bitwise equal to its row of the two-token result;
- q8_lmhead_argmax at N = 2: the planted ids exactly (the argmax gate holds
  for both tokens), logits bitwise those of the GEMV;
- q8_moe_gemv over the same bytes seen as 537 experts of 2048 x 4096
  (expert 512 starts at byte 2^32): each pair's output bitwise equal to the
  dense rows of its expert;
- q8_moe_ffn with gate, up and down banks cut from the same bytes (the up
  and down experts of the largest id start past 2^32 bytes), stage by stage
  against the oracle.
"""
import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth
from tests.gpu_util import assert_parity, dev, host, note, require_gpu, threads, torch

pytestmark = pytest.mark.gpu

K = 4096
ROWS_PER_EXPERT = 2048
N_EXPERTS = 537
V = N_EXPERTS * ROWS_PER_EXPERT  # 1,099,776 rows, 4.5 GB of quants
PAST_4G = (1 << 32) // K          # first row whose quants start past 2^32 bytes


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.fixture(scope="module")
def big():
    note(f"large matrix {V}x{K}: drawing and uploading")
    rng = synth.rng_for(4099)
    q, d = synth.draw_weights_tiled(rng, V, K)
    x = synth.draw_x(rng, 2, K)
    rows = np.array([V - 1, PAST_4G + 12345], np.int64)
    synth.plant_argmax_rows(q, d, x, rows)
    ld_qs, ld_d, _, _ = q8.pack_layout(V, K)
    assert (ld_qs, ld_d) == (K, K // 32), "the packed planes are q and d themselves"
    W = q8.PackedQ8(torch.from_numpy(q).cuda(), torch.from_numpy(d.view(np.int16)).cuda(), V, K)
    assert W.qs.numel() > (1 << 32)
    ref, A = oracle.gemv(q, d, x, threads())
    return dict(q=q, d=d, x=x, rows=rows, W=W, ref=ref, A=A)


@pytest.fixture(scope="module")
def dense(big):
    note("large matrix: q8_gemv N=2")
    return host(q8.gemv(big["W"], dev(big["x"])))


def test_gemv_every_row(big, dense):
    assert_parity(dense, big["ref"], big["A"], what=f"{V}x{K} N=2")
    for n in range(2):
        note(f"large matrix: q8_gemv N=1 token {n}")
        y1 = host(q8.gemv(big["W"], dev(big["x"][n:n + 1])))
        assert np.array_equal(y1[0].view(np.uint32), dense[n].view(np.uint32)), f"token {n}"


def test_lmhead_planted_past_4g(big, dense):
    note("large matrix: q8_lmhead_argmax N=2")
    logits, ids = q8.lmhead_argmax(big["W"], dev(big["x"]))
    logits, ids = host(logits), host(ids)
    istar, gated, _ = oracle.argmax_gate(big["ref"], big["A"])
    assert gated.all() and np.array_equal(istar, big["rows"])
    assert list(ids) == list(big["rows"])
    assert np.array_equal(logits.view(np.uint32), dense.view(np.uint32))


def _bank(W, first, count, M, Kb):
    """Experts first .. first+count-1 of the matrix's bytes seen as [*][M][Kb]."""
    qs = W.qs.view(-1, M, Kb)[first:first + count]
    d = W.d.view(-1, M, Kb // 32)[first:first + count]
    return q8.PackedBank(qs, d, M, Kb, count)


def test_routed_gemv_experts_past_4g(big, dense):
    note("large matrix: q8_moe_gemv over 537 experts")
    bank = _bank(big["W"], 0, N_EXPERTS, ROWS_PER_EXPERT, K)
    ids = np.array([[536, 512, 3, 300], [511, 535, 0, 268]], np.int32)
    yp = host(q8.moe_gemv(bank, dev(ids), dev(big["x"])))
    topk = ids.shape[1]
    for t in range(2):
        for j in range(topk):
            e = int(ids[t, j])
            rows = dense[t, e * ROWS_PER_EXPERT:(e + 1) * ROWS_PER_EXPERT]
            assert np.array_equal(yp[t * topk + j].view(np.uint32), rows.view(np.uint32)), (t, e)


def test_moe_ffn_banks_past_4g(big):
    note("large matrix: q8_moe_ffn, banks cut from the same bytes")
    F, H, E = ROWS_PER_EXPERT, K, 268
    W, q, d = big["W"], big["q"], big["d"]
    gate = _bank(W, 0, E, F, H)
    up = _bank(W, 269, E, F, H)
    down = _bank(W, 269, E, H, F)
    # the same planes on the host, as the oracle reads them
    qA, dA = q.reshape(-1, F, H), d.reshape(-1, F, H // 32)
    qB, dB = q.reshape(-1, H, F), d.reshape(-1, H, F // 32)
    ids = np.array([[267, 266, 0, 100], [1, 267, 265, 200]], np.int32)
    gw = np.array([[0.4, 0.3, 0.2, 0.1], [0.25, 0.25, 0.3, 0.2]], np.float32)
    c = synth.MoeCase(qA[0:E], dA[0:E], qA[269:269 + E], dA[269:269 + E], qB[269:269 + E],
                      dB[269:269 + E], big["x"], ids, gw)
    assert (269 + 267) * F * H >= (1 << 32)  # the largest id's up and down experts
    T, topk = ids.shape
    ws = torch.zeros((q8.moe_ws_bytes(E, T, topk, F, H),), dtype=torch.uint8, device="cuda")
    out = host(q8.moe_ffn(gate, up, down, dev(ids), dev(gw), dev(big["x"]), ws=ws))
    v = q8.moe_ws_views(ws, E, T, topk, F, H)
    s1 = oracle.moe_gate_up(c, threads())
    h = host(v["h"])
    assert np.all(np.abs(h - s1["h"]) <= s1["bh"]), "h outside its bound"
    yref, Ay = oracle.moe_down(c, h, threads())
    assert_parity(host(v["y_pair"]), yref, Ay, what="down on GPU h")
    e2e = oracle.moe_ffn(c, threads())
    assert np.all(np.abs(out - e2e["out"]) <= e2e["bound"])
