"""Host-side tests of the C ABI: no kernel is launched here.

* the library loads and exports every function include/q8gemv.h declares;
* the load-time packer round-trips GGUF Q8_0 blocks byte for byte and
  writes 16-byte-aligned rows with zero padding;
* every synchronous validation error is reachable with bad arguments (the
  pointers are never dereferenced because validation fails first).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "q8gemv.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(q8.LIB_PATH):
        from quantized_weight_gemv_q8_amd import build
        build.build()
    return q8.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q8_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(q8.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
    # and they are real dynamic symbols of the shared object
    nm = os.popen(f"nm -D --defined-only {q8.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", nm), name


def test_status_strings(L):
    for code in range(0, -9, -1):
        s = q8.status_str(code)
        assert s and s != "unknown status"
    assert q8.status_str(5) == "unknown status"


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (17, 1024), (5, 5120), (2, 768)])
def test_pack_roundtrip_and_layout(L, M, K):
    c = synth.gemv_case(M, K, 1, seed=M + K)
    c.q[0, :32] = -128  # extremes
    c.d[0, 0] = np.float16(0.0)
    blocks = synth.to_gguf_blocks(c.q, c.d)
    ld_qs, ld_d, qb, db = q8.pack_layout(M, K)
    assert ld_qs == K and ld_qs % 16 == 0
    assert ld_d >= K // 32 and ld_d % 8 == 0 and ld_d - K // 32 < 8
    assert qb == M * ld_qs and db == 2 * M * ld_d
    qs, d = q8.pack_host(blocks)
    assert np.array_equal(qs[:, :K], c.q)
    assert np.array_equal(d[:, :K // 32], c.d.view(np.uint16))
    assert np.all(d[:, K // 32:] == 0)
    back = q8.unpack_host(qs, d, M, K)
    assert back.tobytes() == blocks.tobytes()


def _mat(qs=0x10000, d=0x20000, M=64, K=256, ld_qs=None, ld_d=None):
    ld_d = (K // 32 + 7) // 8 * 8 if ld_d is None else ld_d
    return q8._Matrix(qs, d, M, K, K if ld_qs is None else ld_qs, ld_d)


def _bank(m, E):
    return q8._Bank(m, m.M * m.ld_qs, m.M * m.ld_d, E)


X, Y, WS = 0x100000, 0x200000, 0x300000


def gemv_rc(L, W=None, x=X, xdt=1, y=Y, ydt=2, N=1):
    W = _mat() if W is None else W
    return L.q8_gemv(ctypes.byref(W), x, xdt, y, ydt, N, None)


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (17, 1024), (5, 5120)])
def test_q4_0_pack_roundtrip_and_layout(L, M, K):
    rng = np.random.default_rng(M + K)
    q, d = synth.draw_weights_q4_0(rng, M, K)
    blocks = synth.to_gguf_q4_0_blocks(q, d)
    ld_qs, ld_d, qb, db = q8.pack_q4_0_layout(M, K)
    assert ld_qs == K // 2 and ld_qs % 16 == 0 and ld_d % 8 == 0 and ld_d >= K // 32
    qs, dd = q8.pack_q4_0_host(blocks)
    assert qs.shape == (M, ld_qs) and dd.shape == (M, ld_d)
    # the nibble plane holds each block's 16 data bytes in GGUF order
    assert np.array_equal(qs[:, :K // 2].reshape(M, K // 32, 16), blocks[:, :, 2:])
    assert np.all(dd[:, K // 32:] == 0)
    assert np.array_equal(q8.unpack_q4_0_host(qs, dd, M, K), blocks)


def test_format_validation(L):
    """The format field selects the row layout check; unknown formats and
    mixed formats in one call are rejected before any device work."""
    def m(fmt, **kw):
        w = _mat(**kw)
        w.format = fmt
        return w
    q4 = m(1, K=256, ld_qs=128)
    assert L.q8_gemv(ctypes.byref(q4), X, 1, Y, 2, 1, None) in (0, -6)  # a valid Q4_0 shape
    assert L.q8_gemv(ctypes.byref(m(1, K=256, ld_qs=112)), X, 1, Y, 2, 1, None) == -2
    assert L.q8_gemv(ctypes.byref(m(0, K=256, ld_qs=128)), X, 1, Y, 2, 1, None) == -2  # Q8 needs K
    assert L.q8_gemv(ctypes.byref(m(1, K=256, ld_qs=136)), X, 1, Y, 2, 1, None) == -3
    assert L.q8_gemv(ctypes.byref(m(2)), X, 1, Y, 2, 1, None) == -4
    assert L.q8_gemv_pair(ctypes.byref(_mat()), ctypes.byref(m(1)), X, 1, Y, Y + 4096, 2, 1,
                          None) == -4
    assert L.q8_gemv_pair_silu(ctypes.byref(_mat()), ctypes.byref(m(1)), X, 1, Y, 2, 1, None) == -4
    assert L.q8_pack_q4_0_layout(4, 48, None, None, None, None) == -2


def test_gemv_validation(L):
    assert L.q8_gemv(None, X, 1, Y, 2, 1, None) == -1
    assert gemv_rc(L, W=_mat(qs=0)) == -1
    assert gemv_rc(L, x=0) == -1
    assert gemv_rc(L, y=0) == -1
    assert gemv_rc(L, W=_mat(M=0)) == -2
    assert gemv_rc(L, W=_mat(K=48, ld_qs=48, ld_d=8)) == -2
    assert gemv_rc(L, W=_mat(K=0)) == -2
    assert gemv_rc(L, W=_mat(ld_qs=128)) == -2
    assert gemv_rc(L, W=_mat(ld_d=2)) == -2
    assert gemv_rc(L, N=0) == -2
    assert gemv_rc(L, W=_mat(ld_qs=264)) == -3
    assert gemv_rc(L, W=_mat(ld_d=9)) == -3
    assert gemv_rc(L, W=_mat(qs=0x10008)) == -3
    assert gemv_rc(L, W=_mat(d=0x20002)) == -3
    assert gemv_rc(L, x=X + 8) == -3
    assert gemv_rc(L, y=Y + 2) == -3
    assert gemv_rc(L, xdt=3) == -4
    assert gemv_rc(L, ydt=0) == -4
    assert gemv_rc(L, y=X + 64) == -8  # y inside x's [N][K] range
    assert L.q8_gemv_pair(ctypes.byref(_mat()), None, X, 1, Y, Y + 4096, 2, 1, None) == -1
    W2 = _mat(K=512, ld_qs=512, ld_d=16)
    assert L.q8_gemv_pair(ctypes.byref(_mat()), ctypes.byref(W2), X, 1, Y, Y + 4096, 2, 1, None) == -2
    assert L.q8_gemv_pair(ctypes.byref(_mat()), ctypes.byref(_mat()), X, 1, Y, Y + 16, 2, 1, None) == -8
    # fused gate/up + SiLU
    sl = L.q8_gemv_pair_silu
    assert sl(ctypes.byref(_mat()), None, X, 1, Y, 2, 1, None) == -1
    assert sl(ctypes.byref(_mat()), ctypes.byref(W2), X, 1, Y, 2, 1, None) == -2
    assert sl(ctypes.byref(_mat()), ctypes.byref(_mat(M=32)), X, 1, Y, 2, 1, None) == -2
    assert sl(ctypes.byref(_mat()), ctypes.byref(_mat()), X, 1, Y, 2, 0, None) == -2
    assert sl(ctypes.byref(_mat()), ctypes.byref(_mat()), X, 1, 0, 2, 1, None) == -1
    assert sl(ctypes.byref(_mat()), ctypes.byref(_mat()), X, 1, Y, 5, 1, None) == -4
    assert sl(ctypes.byref(_mat()), ctypes.byref(_mat()), X, 1, Y + 2, 2, 1, None) == -3
    assert sl(ctypes.byref(_mat()), ctypes.byref(_mat()), X, 1, X + 32, 2, 1, None) == -8


def test_lmhead_validation(L):
    W = _mat()
    n = L.q8_lmhead_ws_bytes(64, 1)
    assert n > 0
    # slots and counters (4608 bytes), then scratch logits for two tokens,
    # rounded up to 256 bytes; independent of N
    assert n == 4608 + 512
    assert L.q8_lmhead_ws_bytes(151936, 1) == 4608 + 151936 * 8
    assert L.q8_lmhead_ws_bytes(151936, 8) == L.q8_lmhead_ws_bytes(151936, 1)
    assert L.q8_lmhead_ws_bytes(1, 1) == 4608 + 256
    ok = dict(x=X, xdt=1, logits=Y, ids=Y + 0x10000, N=1, ws=WS, nws=n)

    def rc(**kw):
        a = dict(ok, **kw)
        return L.q8_lmhead_argmax(ctypes.byref(W), a["x"], a["xdt"], a["logits"], a["ids"], a["N"],
                                  a["ws"], a["nws"], None)
    assert rc(ids=0) == -1
    assert rc(N=0) == -2
    assert rc(xdt=7) == -4
    assert rc(ws=0) == -5
    assert rc(nws=n - 1) == -5
    assert rc(ws=WS + 4) == -5
    assert rc(ids=Y + 2) == -3
    assert rc(ids=Y) == -8  # ids inside logits
    RID = 0x700000

    def rr(rid=RID, **kw):
        a = dict(ok, **kw)
        return L.q8_lmhead_argmax_rows(ctypes.byref(W), rid, a["x"], a["xdt"], a["logits"],
                                       a["ids"], a["N"], a["ws"], a["nws"], None)
    assert rr(rid=0) == -1
    assert rr(rid=RID + 2) == -3
    assert rr(rid=Y + 0x10000 - 8) == -8  # row ids overlap ids
    assert rr(rid=WS) == -8
    assert rr(nws=n - 1) == -5


def test_moe_validation(L):
    E, T, topk, F, H = 8, 4, 2, 64, 128
    g = _bank(_mat(M=F, K=H), E)
    u = _bank(_mat(qs=0x40000, d=0x50000, M=F, K=H), E)
    dn = _bank(_mat(qs=0x60000, d=0x70000, M=H, K=F), E)
    n = L.q8_moe_ws_bytes(E, T, topk, F, H)
    assert n > 0
    off = (ctypes.c_size_t * 7)()
    assert L.q8_moe_ws_layout(E, T, topk, F, H, off) == 0
    assert list(off) == sorted(off) and all(o % 256 == 0 for o in off)
    assert L.q8_moe_ws_layout(E, T, E + 1, F, H, off) == -2
    IDS, GW, XX, OUT = 0x800000, 0x810000, 0x820000, 0x900000

    def rc(gate=g, up=u, down=dn, ids=IDS, gw=GW, x=XX, xdt=1, out=OUT, T_=T, k=topk, ws=WS, nws=n):
        return L.q8_moe_ffn(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), ids, gw, x, xdt,
                            out, T_, k, ws, nws, None)
    assert rc(ids=0) == -1
    assert rc(gw=0) == -1
    assert rc(k=E + 1) == -2
    assert rc(T_=0) == -2
    bad_down = _bank(_mat(qs=0x60000, d=0x70000, M=H, K=2 * F), E)
    assert rc(down=bad_down) == -2
    bad_e = _bank(_mat(qs=0x40000, d=0x50000, M=F, K=H), E - 1)
    assert rc(up=bad_e) == -2
    assert rc(xdt=9) == -4
    assert rc(nws=n - 1) == -5
    assert rc(ids=IDS + 2) == -3
    assert rc(out=XX) == -8
    # routed GEMV
    n1 = L.q8_moe_ws_bytes(E, T, topk, 0, F)
    assert L.q8_moe_gemv(ctypes.byref(g), IDS, None, XX, 1, 0, OUT, T, topk, WS, n1 - 1, None) == -5
    assert L.q8_moe_gemv(ctypes.byref(g), IDS, None, XX, 1, 0, 0, T, topk, WS, n1, None) == -1
    bad_stride = q8._Bank(g.e0, g.stride_qs - 16, g.stride_d, E)
    assert L.q8_moe_gemv(ctypes.byref(bad_stride), IDS, None, XX, 1, 0, OUT, T, topk, WS, n1, None) == -2


def test_router_validation(L):
    LG, IDS, GW, XX = 0x800000, 0x900000, 0xA00000, 0xB00000
    T, E, k = 4, 128, 8

    def rc(lg=LG, T_=T, E_=E, k_=k, ids=IDS, gw=GW):
        return L.q8_moe_topk_softmax(lg, T_, E_, k_, ids, gw, None)
    assert rc(lg=0) == -1 and rc(ids=0) == -1 and rc(gw=0) == -1
    assert rc(T_=0) == -2 and rc(E_=0) == -2 and rc(k_=0) == -2
    assert rc(k_=E + 1) == -2
    assert rc(E_=4097, k_=8) == -2  # more experts than the wave holds
    assert rc(E_=100, k_=65) == -2  # more picks than lanes
    assert rc(lg=LG + 2) == -3 and rc(gw=GW + 1) == -3
    assert rc(ids=LG + 16) == -8  # ids inside the logits
    assert rc(gw=IDS + 4) == -8  # gate_w overlaps ids
    W = _mat(M=E, K=256)
    assert L.q8_moe_router(ctypes.byref(W), 0, 1, T, k, LG, IDS, GW, None) == -1
    assert L.q8_moe_router(ctypes.byref(W), XX, 7, T, k, LG, IDS, GW, None) == -4
    assert L.q8_moe_router(ctypes.byref(W), XX, 1, T, E + 1, LG, IDS, GW, None) == -2
    assert L.q8_moe_router(ctypes.byref(W), XX, 1, T, k, LG, XX, GW, None) == -8


def test_valid_call_without_gfx950_is_refused(L):
    if L.q8_device_check(0) == 0:
        pytest.skip("a gfx950 device is present; this check is for hosts without one")
    assert gemv_rc(L) == -6
    assert L.q8_device_check(0) == -6


def test_shared_expert_validation(L):
    """q8_moe_shared_expert refuses bad arguments before touching the
    device: shapes that do not chain (Wg/Wu [F][H], Wd [H][F], Wsg [1][H]),
    mixed gate/up/gate-row formats, null pointers, a short or misaligned
    workspace and overlapping buffers."""
    F, H, T = 64, 256, 3
    g, u = _mat(M=F, K=H), _mat(M=F, K=H)
    dn, sg = _mat(M=H, K=F), _mat(M=1, K=H)
    n = L.q8_moe_shared_ws_bytes(F, H, T)
    assert n >= 4 * (T * F + T)  # h and the gate dots, fp32
    assert L.q8_moe_shared_ws_bytes(0, H, T) == 0
    ok = dict(g=g, u=u, d=dn, s=sg, x=X, xdt=1, T=T, out=Y, ws=WS, nws=n)

    def rc(**kw):
        a = dict(ok, **kw)
        return L.q8_moe_shared_expert(ctypes.byref(a["g"]), ctypes.byref(a["u"]),
                                      ctypes.byref(a["d"]), ctypes.byref(a["s"]), a["x"],
                                      a["xdt"], a["T"], a["out"], a["ws"], a["nws"], None)
    assert rc(x=0) == -1
    assert rc(out=0) == -1
    assert rc(d=_mat(M=H, K=2 * F)) == -2  # down does not take h
    assert rc(s=_mat(M=2, K=H)) == -2      # the gate is one row
    assert rc(u=_mat(M=F, K=2 * H)) == -2
    assert rc(T=0) == -2
    assert rc(xdt=9) == -4
    q4u = _mat(M=F, K=H)
    q4u.format = q8.Q8_FMT_Q4_0
    assert rc(u=q4u) == -4                 # gate and up in one format
    q4s = _mat(M=1, K=H)
    q4s.format = q8.Q8_FMT_Q4_0
    assert rc(s=q4s) == -4                 # the gate row is the pair's extra row
    assert rc(ws=0) == -5
    assert rc(nws=n - 1) == -5
    assert rc(ws=WS + 8) == -5
    assert rc(x=X + 8) == -3
    assert rc(out=X) == -8                 # out over x
    assert rc(ws=Y) == -8                  # workspace over out


def test_shared_expert_binding_rejects_bad_out():
    """The Python binding refuses an out that is not a contiguous fp32
    [T][H] tensor before calling the library."""
    import torch
    W = q8.PackedQ8(torch.zeros((64, 256), dtype=torch.int8),
                    torch.zeros((64, 8), dtype=torch.int16), 64, 256)
    x = torch.zeros((2, 256), dtype=torch.float16)
    for bad in (torch.zeros((256, 2)).t(), torch.zeros((2, 256), dtype=torch.float16),
                torch.zeros((3, 256))):
        with pytest.raises(ValueError):
            q8.moe_shared_expert(W, W, W, W, x, bad)


def test_bindings_reject_mismatched_buffers():
    """Every binding refuses a caller-provided buffer of the wrong shape,
    dtype or layout before the library is called (a short buffer would
    otherwise be written past its end)."""
    import torch
    W = q8.PackedQ8(torch.zeros((64, 256), dtype=torch.int8),
                    torch.zeros((64, 8), dtype=torch.int16), 64, 256)
    x = torch.zeros((2, 256), dtype=torch.float16)
    for bad in (torch.zeros((2, 63)), torch.zeros((64, 2)).t(), torch.zeros((2, 64), dtype=torch.int32)):
        with pytest.raises(ValueError):
            q8.gemv(W, x, out=bad)
        with pytest.raises(ValueError):
            q8.gemv_pair_silu(W, W, x, out=bad)
        with pytest.raises(ValueError):
            q8.gemv_pair(W, W, x, out_a=bad, out_b=bad)
    with pytest.raises(ValueError):
        q8.lmhead_argmax(W, x, logits=torch.zeros((2, 63)))
    with pytest.raises(ValueError):
        q8.lmhead_argmax(W, x, ids=torch.zeros((2,), dtype=torch.int64))
    with pytest.raises(ValueError):
        q8.lmhead_argmax(W, x, row_ids=torch.zeros((63,), dtype=torch.int32))
    L = torch.zeros((2, 64))
    with pytest.raises(ValueError):
        q8.moe_topk_softmax(L, 8, ids=torch.zeros((2, 7), dtype=torch.int32))
    with pytest.raises(ValueError):
        q8.moe_router(W, x, 8, logits=torch.zeros((2, 63)))


def test_bindings_refuse_host_tensors():
    """A host tensor handed to a kernel would be dereferenced by the GPU:
    the bindings refuse it (checked last, after the shape checks)."""
    import torch
    W = q8.PackedQ8(torch.zeros((64, 256), dtype=torch.int8),
                    torch.zeros((64, 8), dtype=torch.int16), 64, 256)
    x = torch.zeros((2, 256), dtype=torch.float16)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.gemv(W, x)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.gemv_pair_silu(W, W, x)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.moe_topk_softmax(torch.zeros((2, 64)), 8)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.moe_router(W, x, 8)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.lmhead_argmax(W, x)


def test_bindings_check_packed_planes():
    """Packed weights whose planes do not match their shape fields are
    refused before any launch: a short quant plane, a column-sliced scale
    plane, a wrong dtype, a bank with too few experts."""
    import torch
    x = torch.zeros((2, 256), dtype=torch.float16)
    good_q = torch.zeros((64, 256), dtype=torch.int8)
    good_d = torch.zeros((64, 8), dtype=torch.int16)
    bad = [
        q8.PackedQ8(torch.zeros((63, 256), dtype=torch.int8), good_d, 64, 256),  # short qs
        q8.PackedQ8(good_q, torch.zeros((64, 16), dtype=torch.int16)[:, ::2], 64, 256),  # strided d
        q8.PackedQ8(good_q[:, :128], good_d, 64, 256),  # rows shorter than K
        q8.PackedQ8(good_q, torch.zeros((64, 8), dtype=torch.float16), 64, 256),  # d dtype
        q8.PackedQ8(good_q.view(-1), good_d, 64, 256),  # flat qs
        q8.PackedQ8(good_q[:, :128], good_d, 64, 256, q8.Q8_FMT_Q8_0),
    ]
    for W in bad:
        with pytest.raises(ValueError, match="packed matrix plane"):
            q8.gemv(W, x)
    # Q4_0 rows hold K/2 bytes: the same [64][128] plane is valid for it
    ok = q8.PackedQ8(torch.zeros((64, 128), dtype=torch.int8), good_d, 64, 256, q8.Q8_FMT_Q4_0)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.gemv(ok, x)
    bank_q = torch.zeros((4, 64, 256), dtype=torch.int8)
    bank_d = torch.zeros((4, 64, 8), dtype=torch.int16)
    ids = torch.zeros((2, 2), dtype=torch.int32)
    gw = torch.zeros((2, 2), dtype=torch.float32)
    for B in (q8.PackedBank(bank_q[:3], bank_d, 64, 256, 4),
              q8.PackedBank(bank_q, bank_d[:, :, :4], 64, 256, 4),
              q8.PackedBank(bank_q[:, :32], bank_d, 64, 256, 4)):
        with pytest.raises(ValueError, match="packed bank plane"):
            q8.moe_gemv(B, ids, x.view(2, 256), gate_w=gw)
    good = q8.PackedBank(bank_q, bank_d, 64, 256, 4)
    with pytest.raises(ValueError, match="on the GPU"):
        q8.moe_gemv(good, ids, x, gate_w=gw)


def test_moe_noalloc_validation(L):
    """The no-allocation routed FFN validates like q8_moe_ffn and refuses a
    shape whose workspace exceeds the library's scratch array before it
    touches the runtime; a shape that fits gets as far as the device check."""
    assert L.q8_noalloc_scratch_bytes() == 8 << 20
    E, topk = 8, 2
    IDS, GW, XX, OUT = 0x800000, 0x810000, 0x820000, 0x90000000

    def rc(T, F, H):
        g = _bank(_mat(M=F, K=H), E)
        u = _bank(_mat(qs=0x4000000, d=0x5000000, M=F, K=H), E)
        dn = _bank(_mat(qs=0x6000000, d=0x7000000, M=H, K=F), E)
        return L.q8_moe_ffn_noalloc(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), IDS, GW,
                                    XX, 1, OUT, T, topk, None)
    assert L.q8_moe_ws_bytes(E, 1024, topk, 1024, 2048) > L.q8_noalloc_scratch_bytes()
    assert rc(1024, 1024, 2048) == -5
    assert rc(4, 64, 128) == -6  # fits; no gfx950 device on this host
    g = _bank(_mat(M=64, K=128), E)
    assert L.q8_moe_ffn_noalloc(ctypes.byref(g), ctypes.byref(g), ctypes.byref(g), 0, GW, XX, 1,
                                OUT, 4, topk, None) in (-1, -2)
