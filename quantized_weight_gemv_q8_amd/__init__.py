"""MI355X-native Q8_0 weight-only GEMV for LLM decode (HIP, gfx950).

Thin Python binding over the C ABI of ``libq8gemv.so`` (declared in
``include/q8gemv.h``). This module only marshals arguments: every step of
the computation runs in the library's HIP kernels. PyTorch provides device
buffers and the current stream; nothing here computes on the CPU, and
nothing falls back to another implementation: if the library is missing or
the device is not gfx950, calls raise.

Entry points (same names as the C ABI, without the ``q8_`` prefix):
``pack``/``unpack`` (load-time repack of GGUF Q8_0 blocks), ``gemv``,
``gemv_pair``, ``lmhead_argmax``, ``moe_gemv``, ``moe_ffn``,
``device_check``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libq8gemv.so")

Q8_DT_F16 = 1
Q8_DT_F32 = 2

# every function the header declares
EXPORTS = (
    "q8_status_str", "q8_device_check", "q8_pack_layout", "q8_pack_host", "q8_unpack_host",
    "q8_pack_q4_0_layout", "q8_pack_q4_0_host", "q8_unpack_q4_0_host",
    "q8_gemv", "q8_gemv_pair", "q8_gemv_pair_silu", "q8_lmhead_ws_bytes", "q8_lmhead_argmax",
    "q8_lmhead_argmax_rows",
    "q8_moe_ws_bytes", "q8_moe_ws_layout", "q8_moe_gemv", "q8_moe_ffn", "q8_moe_topk_softmax",
    "q8_moe_router", "q8_moe_shared_ws_bytes", "q8_moe_shared_expert",
    "q8_noalloc_scratch_bytes", "q8_moe_ffn_noalloc",
)


class Q8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


Q8_FMT_Q8_0 = 0
Q8_FMT_Q4_0 = 1


class _Matrix(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("d", ctypes.c_void_p), ("M", ctypes.c_int64),
                ("K", ctypes.c_int64), ("ld_qs", ctypes.c_int64), ("ld_d", ctypes.c_int64),
                ("format", ctypes.c_int32)]


class _Bank(ctypes.Structure):
    _fields_ = [("e0", _Matrix), ("stride_qs", ctypes.c_int64), ("stride_d", ctypes.c_int64),
                ("E", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libq8gemv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m quantized_weight_gemv_q8_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        pm, pb = ctypes.POINTER(_Matrix), ctypes.POINTER(_Bank)
        sig = {
            "q8_status_str": ([i32], ctypes.c_char_p),
            "q8_device_check": ([i32], i32),
            "q8_pack_layout": ([i64, i64, vp, vp, vp, vp], i32),
            "q8_pack_host": ([vp, i64, i64, vp, i64, vp, i64], i32),
            "q8_unpack_host": ([vp, i64, vp, i64, i64, i64, vp], i32),
            "q8_pack_q4_0_layout": ([i64, i64, vp, vp, vp, vp], i32),
            "q8_pack_q4_0_host": ([vp, i64, i64, vp, i64, vp, i64], i32),
            "q8_unpack_q4_0_host": ([vp, i64, vp, i64, i64, i64, vp], i32),
            "q8_gemv": ([pm, vp, i32, vp, i32, i32, vp], i32),
            "q8_gemv_pair": ([pm, pm, vp, i32, vp, vp, i32, i32, vp], i32),
            "q8_gemv_pair_silu": ([pm, pm, vp, i32, vp, i32, i32, vp], i32),
            "q8_lmhead_ws_bytes": ([i64, i32], sz),
            "q8_lmhead_argmax": ([pm, vp, i32, vp, vp, i32, vp, sz, vp], i32),
            "q8_lmhead_argmax_rows": ([pm, vp, vp, i32, vp, vp, i32, vp, sz, vp], i32),
            "q8_moe_ws_bytes": ([i32, i32, i32, i64, i64], sz),
            "q8_moe_ws_layout": ([i32, i32, i32, i64, i64, vp], i32),
            "q8_moe_gemv": ([pb, vp, vp, vp, i32, i32, vp, i32, i32, vp, sz, vp], i32),
            "q8_moe_ffn": ([pb, pb, pb, vp, vp, vp, i32, vp, i32, i32, vp, sz, vp], i32),
            "q8_moe_topk_softmax": ([vp, i32, i32, i32, vp, vp, vp], i32),
            "q8_moe_router": ([pm, vp, i32, i32, i32, vp, vp, vp, vp], i32),
            "q8_moe_shared_ws_bytes": ([i64, i64, i32], sz),
            "q8_moe_shared_expert": ([pm, pm, pm, pm, vp, i32, i32, vp, vp, sz, vp], i32),
            "q8_noalloc_scratch_bytes": ([], sz),
            "q8_moe_ffn_noalloc": ([pb, pb, pb, vp, vp, vp, i32, vp, i32, i32, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().q8_status_str(int(status)).decode()


def _check(rc: int, where: str):
    if rc != 0:
        raise Q8Error(rc, where)


def device_check(device: int = 0) -> int:
    return lib().q8_device_check(device)


# ---------------------------------------------------------------- packing
def pack_layout(M: int, K: int):
    ld_qs, ld_d = ctypes.c_int64(), ctypes.c_int64()
    qb, db = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().q8_pack_layout(M, K, ctypes.byref(ld_qs), ctypes.byref(ld_d), ctypes.byref(qb),
                                ctypes.byref(db)), "q8_pack_layout")
    return ld_qs.value, ld_d.value, qb.value, db.value


def pack_host(blocks: np.ndarray):
    """GGUF Q8_0 blocks uint8 [M][K/32][34] -> host planes (qs int8 [M][ld_qs], d uint16 [M][ld_d])."""
    blocks = np.ascontiguousarray(blocks, np.uint8)
    M, nb, bb = blocks.shape
    if bb != 34:
        raise ValueError("Q8_0 blocks are 34 bytes")
    K = nb * 32
    ld_qs, ld_d, _, _ = pack_layout(M, K)
    qs = np.empty((M, ld_qs), np.int8)
    d = np.empty((M, ld_d), np.uint16)
    _check(lib().q8_pack_host(blocks.ctypes.data, M, K, qs.ctypes.data, ld_qs, d.ctypes.data, ld_d),
           "q8_pack_host")
    return qs, d


def unpack_host(qs: np.ndarray, d: np.ndarray, M: int, K: int) -> np.ndarray:
    qs = np.ascontiguousarray(qs, np.int8)
    d = np.ascontiguousarray(d, np.uint16)
    out = np.empty((M, K // 32, 34), np.uint8)
    _check(lib().q8_unpack_host(qs.ctypes.data, qs.shape[1], d.ctypes.data, d.shape[1], M, K,
                                out.ctypes.data), "q8_unpack_host")
    return out


@dataclasses.dataclass
class PackedQ8:
    """One packed matrix on the device (split planes, 16-byte rows): Q8_0
    by default, or Q4_0 (fmt = Q8_FMT_Q4_0, qs holding the nibble plane)."""
    qs: "torch.Tensor"  # int8 [M][ld_qs]
    d: "torch.Tensor"   # int16 (fp16 bit patterns) [M][ld_d]
    M: int
    K: int
    fmt: int = Q8_FMT_Q8_0

    def cmat(self) -> _Matrix:
        return _Matrix(self.qs.data_ptr(), self.d.data_ptr(), self.M, self.K,
                       self.qs.stride(0), self.d.stride(0), self.fmt)

    @property
    def nbytes(self) -> int:
        return self.qs.numel() + 2 * self.d.numel()


@dataclasses.dataclass
class PackedBank:
    """E packed matrices of one shape and format: qs [E][M][ld_qs], d [E][M][ld_d]."""
    qs: "torch.Tensor"
    d: "torch.Tensor"
    M: int
    K: int
    E: int
    fmt: int = Q8_FMT_Q8_0

    def cbank(self) -> _Bank:
        e0 = _Matrix(self.qs.data_ptr(), self.d.data_ptr(), self.M, self.K,
                     self.qs.stride(1), self.d.stride(1), self.fmt)
        return _Bank(e0, self.qs.stride(0), self.d.stride(0), self.E)

    def expert(self, e: int) -> PackedQ8:
        return PackedQ8(self.qs[e], self.d[e], self.M, self.K, self.fmt)


def pack(blocks: np.ndarray, device="cuda") -> PackedQ8:
    """Repack GGUF Q8_0 blocks [M][K/32][34] and upload them."""
    import torch
    qs, d = pack_host(blocks)
    M, K = blocks.shape[0], blocks.shape[1] * 32
    return PackedQ8(torch.from_numpy(qs).to(device), torch.from_numpy(d.view(np.int16)).to(device),
                    M, K)


def pack_bank(blocks: np.ndarray, device="cuda") -> PackedBank:
    """Blocks uint8 [E][M][K/32][34] -> one device bank."""
    import torch
    E, M, nb, _ = blocks.shape
    K = nb * 32
    planes = [pack_host(blocks[e]) for e in range(E)]
    qs = np.stack([p[0] for p in planes])
    d = np.stack([p[1] for p in planes]).view(np.int16)
    return PackedBank(torch.from_numpy(qs).to(device), torch.from_numpy(d).to(device), M, K, E)


def unpack(W: PackedQ8) -> np.ndarray:
    return unpack_host(W.qs.cpu().numpy(), W.d.cpu().numpy().view(np.uint16), W.M, W.K)


# ---------------------------------------------------------------- Q4_0 packing
def pack_q4_0_layout(M: int, K: int):
    ld_qs, ld_d = ctypes.c_int64(), ctypes.c_int64()
    qb, db = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().q8_pack_q4_0_layout(M, K, ctypes.byref(ld_qs), ctypes.byref(ld_d),
                                     ctypes.byref(qb), ctypes.byref(db)), "q8_pack_q4_0_layout")
    return ld_qs.value, ld_d.value, qb.value, db.value


def pack_q4_0_host(blocks: np.ndarray):
    """GGUF Q4_0 blocks uint8 [M][K/32][18] -> host planes (nibbles uint8
    [M][ld_qs], d uint16 [M][ld_d])."""
    blocks = np.ascontiguousarray(blocks, np.uint8)
    M, nb, bb = blocks.shape
    if bb != 18:
        raise ValueError("Q4_0 blocks are 18 bytes")
    K = nb * 32
    ld_qs, ld_d, _, _ = pack_q4_0_layout(M, K)
    qs = np.empty((M, ld_qs), np.uint8)
    d = np.empty((M, ld_d), np.uint16)
    _check(lib().q8_pack_q4_0_host(blocks.ctypes.data, M, K, qs.ctypes.data, ld_qs, d.ctypes.data,
                                   ld_d), "q8_pack_q4_0_host")
    return qs, d


def unpack_q4_0_host(qs: np.ndarray, d: np.ndarray, M: int, K: int) -> np.ndarray:
    qs = np.ascontiguousarray(qs, np.uint8)
    d = np.ascontiguousarray(d, np.uint16)
    out = np.empty((M, K // 32, 18), np.uint8)
    _check(lib().q8_unpack_q4_0_host(qs.ctypes.data, qs.shape[1], d.ctypes.data, d.shape[1], M, K,
                                     out.ctypes.data), "q8_unpack_q4_0_host")
    return out


def pack_q4_0(blocks: np.ndarray, device="cuda") -> PackedQ8:
    """Repack GGUF Q4_0 blocks [M][K/32][18] and upload them (qs holds the
    nibble plane)."""
    import torch
    qs, d = pack_q4_0_host(blocks)
    M, K = blocks.shape[0], blocks.shape[1] * 32
    return PackedQ8(torch.from_numpy(qs.view(np.int8)).to(device),
                    torch.from_numpy(d.view(np.int16)).to(device), M, K, Q8_FMT_Q4_0)


def pack_bank_q4_0(blocks: np.ndarray, device="cuda") -> PackedBank:
    """Q4_0 blocks uint8 [E][M][K/32][18] -> one device bank."""
    import torch
    E, M, nb, _ = blocks.shape
    planes = [pack_q4_0_host(blocks[e]) for e in range(E)]
    qs = np.stack([p[0] for p in planes]).view(np.int8)
    d = np.stack([p[1] for p in planes]).view(np.int16)
    return PackedBank(torch.from_numpy(qs).to(device), torch.from_numpy(d).to(device), M, nb * 32,
                      E, Q8_FMT_Q4_0)


# ---------------------------------------------------------------- hot path
def _dt(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return Q8_DT_F16
    if t.dtype == torch.float32:
        return Q8_DT_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t, shape, dtypes, name):
    """Caller-provided buffers must match what the call writes or reads:
    a contiguous tensor of exactly this shape and one of these dtypes."""
    import torch
    if (not isinstance(t, torch.Tensor) or tuple(t.shape) != tuple(shape) or t.dtype not in dtypes
            or not t.is_contiguous()):
        names = "/".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} must be a contiguous {names} tensor of shape {tuple(shape)}")
    return t


def _check_packed(W):
    """A packed matrix or bank must hold the planes its header fields
    describe: qs int8/uint8 with M rows of at least the row's bytes (K, or
    K/2 for Q4_0) and d int16 with M rows of at least K/32 scales, each
    with unit inner stride ([E][M][...] for a bank). The library reads
    M * ld bytes from each plane, so a short or column-sliced plane would
    be read past its end or at the wrong bytes."""
    import torch
    row_bytes = W.K // 2 if W.fmt == Q8_FMT_Q4_0 else W.K
    lead = (W.E,) if isinstance(W, PackedBank) else ()
    for t, name, dts, width in ((W.qs, "qs", (torch.int8, torch.uint8), row_bytes),
                                (W.d, "d", (torch.int16,), W.K // 32)):
        ok = (isinstance(t, torch.Tensor) and t.dtype in dts and t.dim() == len(lead) + 2
              and tuple(t.shape[:-1]) == lead + (W.M,) and t.shape[-1] >= width
              and t.stride(-1) == 1 and t.stride(-2) >= width)
        if ok and lead:
            ok = W.E == 1 or t.stride(0) >= W.M * t.stride(1)
        if not ok:
            kind = "bank" if lead else "matrix"
            raise ValueError(f"packed {kind} plane {name} must be a {'/'.join(str(d)[6:] for d in dts)} "
                             f"tensor of shape {lead + (W.M,)} x >={width} with unit inner stride "
                             f"(got {tuple(t.shape) if isinstance(t, torch.Tensor) else type(t)})")


def _on_gpu(*args):
    """Every tensor handed to a kernel (packed weights included) must live
    in device memory: a host address would be read or written by the GPU.
    Packed weights are first checked against their own shape fields."""
    for a in args:
        if isinstance(a, (PackedQ8, PackedBank)):
            _check_packed(a)
    for a in args:
        if a is None:
            continue
        ts = (a.qs, a.d) if isinstance(a, (PackedQ8, PackedBank)) else (a,)
        for t in ts:
            if not t.is_cuda:
                raise ValueError("every tensor argument must be on the GPU")


def _f(torch):
    return (torch.float32, torch.float16)


def _as_2d(x, K):
    if x.dim() == 1:
        x = x.view(1, -1)
    if x.dim() != 2 or x.shape[1] != K or not x.is_contiguous():
        raise ValueError(f"x must be a contiguous [N][{K}] tensor")
    return x


def gemv(W: PackedQ8, x, out=None, out_dtype=None, stream=None):
    """y[n][m] = sum_k dequant(W)[m][k] * x[n][k]; x fp16/fp32 [N][K] -> y [N][M]."""
    import torch
    x = _as_2d(x, W.K)
    N = x.shape[0]
    if out is None:
        out = torch.empty((N, W.M), dtype=out_dtype or torch.float32, device=x.device)
    _need(out, (N, W.M), _f(torch), "out")
    _on_gpu(W, x, out)
    _check(lib().q8_gemv(ctypes.byref(W.cmat()), x.data_ptr(), _dt(x), out.data_ptr(), _dt(out), N,
                         _stream(stream)), "q8_gemv")
    return out


def gemv_pair(Wa: PackedQ8, Wb: PackedQ8, x, out_a=None, out_b=None, out_dtype=None, stream=None):
    """(Wa x, Wb x) in one launch sharing the staging of x."""
    import torch
    x = _as_2d(x, Wa.K)
    N = x.shape[0]
    dt = out_dtype or torch.float32
    if out_a is None:
        out_a = torch.empty((N, Wa.M), dtype=dt, device=x.device)
    if out_b is None:
        out_b = torch.empty((N, Wb.M), dtype=dt, device=x.device)
    if out_a.dtype != out_b.dtype:
        raise TypeError("out_a and out_b must share a dtype")
    _need(out_a, (N, Wa.M), _f(torch), "out_a")
    _need(out_b, (N, Wb.M), _f(torch), "out_b")
    _on_gpu(Wa, Wb, x, out_a, out_b)
    _check(lib().q8_gemv_pair(ctypes.byref(Wa.cmat()), ctypes.byref(Wb.cmat()), x.data_ptr(),
                              _dt(x), out_a.data_ptr(), out_b.data_ptr(), _dt(out_a), N,
                              _stream(stream)), "q8_gemv_pair")
    return out_a, out_b


def gemv_pair_silu(Wg: PackedQ8, Wu: PackedQ8, x, out=None, out_dtype=None, stream=None):
    """h = silu(Wg x) * (Wu x), fp32 (or fp16) [N][M]."""
    import torch
    x = _as_2d(x, Wg.K)
    N = x.shape[0]
    if out is None:
        out = torch.empty((N, Wg.M), dtype=out_dtype or torch.float32, device=x.device)
    _need(out, (N, Wg.M), _f(torch), "out")
    _on_gpu(Wg, Wu, x, out)
    _check(lib().q8_gemv_pair_silu(ctypes.byref(Wg.cmat()), ctypes.byref(Wu.cmat()), x.data_ptr(),
                                   _dt(x), out.data_ptr(), _dt(out), N, _stream(stream)),
           "q8_gemv_pair_silu")
    return out


def lmhead_ws_bytes(V: int, N: int) -> int:
    return lib().q8_lmhead_ws_bytes(V, N)


def lmhead_argmax(W: PackedQ8, x, logits=True, ids=None, ws=None, stream=None, row_ids=None):
    """Returns (logits fp32 [N][V] or None, ids int32 [N]). With ``row_ids``
    (int32 [V] on the device) W is a draft head over a vocabulary subset and
    ids are mapped through it."""
    import torch
    x = _as_2d(x, W.K)
    N = x.shape[0]
    if logits is True:
        logits = torch.empty((N, W.M), dtype=torch.float32, device=x.device)
    elif logits is False:
        logits = None
    if ids is None:
        ids = torch.empty((N,), dtype=torch.int32, device=x.device)
    if logits is not None:
        _need(logits, (N, W.M), (torch.float32,), "logits")
    _need(ids, (N,), (torch.int32,), "ids")
    nws = lmhead_ws_bytes(W.M, N)
    if ws is None:
        ws = torch.zeros((nws,), dtype=torch.uint8, device=x.device)
    _need(ws, (ws.numel(),), (torch.uint8,), "ws")
    lp = logits.data_ptr() if logits is not None else None
    nb = ws.numel() * ws.element_size()
    if row_ids is not None:
        _need(row_ids, (W.M,), (torch.int32,), "row_ids (one entry per row of W)")
    _on_gpu(W, x, logits, ids, ws, row_ids)
    if row_ids is None:
        rc = lib().q8_lmhead_argmax(ctypes.byref(W.cmat()), x.data_ptr(), _dt(x), lp, ids.data_ptr(),
                                    N, ws.data_ptr(), nb, _stream(stream))
    else:
        rc = lib().q8_lmhead_argmax_rows(ctypes.byref(W.cmat()), row_ids.data_ptr(), x.data_ptr(),
                                         _dt(x), lp, ids.data_ptr(), N, ws.data_ptr(), nb,
                                         _stream(stream))
    _check(rc, "q8_lmhead_argmax")
    return logits, ids


def moe_ws_bytes(E: int, T: int, topk: int, F: int, M: int) -> int:
    return lib().q8_moe_ws_bytes(E, T, topk, F, M)


def moe_ws_layout(E: int, T: int, topk: int, F: int, M: int):
    off = (ctypes.c_size_t * 7)()
    _check(lib().q8_moe_ws_layout(E, T, topk, F, M, off), "q8_moe_ws_layout")
    return list(off)


def moe_ws_views(ws, E: int, T: int, topk: int, F: int, M: int) -> dict:
    """Named views into a MoE workspace (layout documented in the header)."""
    import torch
    off = moe_ws_layout(E, T, topk, F, M)
    P = T * topk

    def view(i, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[off[i]:off[i] + nbytes].view(dt)

    v = dict(counts=view(0, E, torch.int32), offsets=view(1, E + 1, torch.int32),
             pairs=view(2, P, torch.int32), active=view(3, E, torch.int32),
             n_active=view(4, 1, torch.int32), y_pair=view(6, P * M, torch.float32).view(P, M))
    # the error word: pairs whose expert id was out of range in the last call
    v["n_bad_ids"] = ws[off[4] + 8:off[4] + 12].view(torch.int32)
    if F > 0:
        v["h"] = view(5, P * F, torch.float32).view(P, F)
    return v


def moe_gemv(W: PackedBank, expert_ids, x, gate_w=None, x_per_pair=False, out=None, ws=None,
             stream=None):
    """Routed GEMV; returns y [T*topk][M] (gate_w None) or the combine [T][M]."""
    import torch
    T, topk = expert_ids.shape
    P = T * topk
    _need(expert_ids, (T, topk), (torch.int32,), "expert_ids")
    if gate_w is not None:
        _need(gate_w, (T, topk), (torch.float32,), "gate_w")
    _need(x, (P if x_per_pair else T, W.K), _f(torch), "x")
    if out is None:
        out = torch.empty((T if gate_w is not None else P, W.M), dtype=torch.float32,
                          device=x.device)
    _need(out, (T if gate_w is not None else P, W.M), (torch.float32,), "out")
    nws = moe_ws_bytes(W.E, T, topk, 0, W.M)
    if ws is None:
        ws = torch.empty((nws,), dtype=torch.uint8, device=x.device)
    _need(ws, (ws.numel(),), (torch.uint8,), "ws")
    _on_gpu(W, expert_ids, gate_w, x, out, ws)
    _check(lib().q8_moe_gemv(ctypes.byref(W.cbank()), expert_ids.data_ptr(),
                             gate_w.data_ptr() if gate_w is not None else None, x.data_ptr(),
                             _dt(x), int(bool(x_per_pair)), out.data_ptr(), T, topk, ws.data_ptr(),
                             ws.numel(), _stream(stream)), "q8_moe_gemv")
    return out


def moe_ffn(gate: PackedBank, up: PackedBank, down: PackedBank, expert_ids, gate_w, x, out=None,
            ws=None, stream=None):
    """Routed SiLU-gated expert FFN; returns out fp32 [T][H]."""
    import torch
    T, topk = expert_ids.shape
    H = gate.K
    _need(expert_ids, (T, topk), (torch.int32,), "expert_ids")
    _need(gate_w, (T, topk), (torch.float32,), "gate_w")
    _need(x, (T, H), _f(torch), "x")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(out, (T, H), (torch.float32,), "out")
    nws = moe_ws_bytes(gate.E, T, topk, gate.M, H)
    if ws is None:
        ws = torch.empty((nws,), dtype=torch.uint8, device=x.device)
    _need(ws, (ws.numel(),), (torch.uint8,), "ws")
    _on_gpu(gate, up, down, expert_ids, gate_w, x, out, ws)
    _check(lib().q8_moe_ffn(ctypes.byref(gate.cbank()), ctypes.byref(up.cbank()),
                            ctypes.byref(down.cbank()), expert_ids.data_ptr(), gate_w.data_ptr(),
                            x.data_ptr(), _dt(x), out.data_ptr(), T, topk, ws.data_ptr(),
                            ws.numel(), _stream(stream)), "q8_moe_ffn")
    return out


def noalloc_scratch_bytes() -> int:
    return lib().q8_noalloc_scratch_bytes()


def moe_ffn_noalloc(gate: PackedBank, up: PackedBank, down: PackedBank, expert_ids, gate_w, x,
                    out=None, stream=None):
    """q8_moe_ffn on the library's own scratch array (no workspace; calls on
    one GPU must not overlap). Returns out fp32 [T][H]."""
    import torch
    T, topk = expert_ids.shape
    H = gate.K
    _need(expert_ids, (T, topk), (torch.int32,), "expert_ids")
    _need(gate_w, (T, topk), (torch.float32,), "gate_w")
    _need(x, (T, H), _f(torch), "x")
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=x.device)
    _need(out, (T, H), (torch.float32,), "out")
    _on_gpu(gate, up, down, expert_ids, gate_w, x, out)
    _check(lib().q8_moe_ffn_noalloc(ctypes.byref(gate.cbank()), ctypes.byref(up.cbank()),
                                    ctypes.byref(down.cbank()), expert_ids.data_ptr(),
                                    gate_w.data_ptr(), x.data_ptr(), _dt(x), out.data_ptr(), T,
                                    topk, _stream(stream)), "q8_moe_ffn_noalloc")
    return out


def moe_topk_softmax(logits, topk: int, ids=None, gate_w=None, stream=None):
    """Router on the device: (expert_ids int32 [T][topk], gate_w fp32 [T][topk])
    from router logits fp32 [T][E]."""
    import torch
    if logits.dtype != torch.float32 or logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous fp32 [T][E] tensor")
    T, E = logits.shape
    if ids is None:
        ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    if gate_w is None:
        gate_w = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    _need(ids, (T, topk), (torch.int32,), "ids")
    _need(gate_w, (T, topk), (torch.float32,), "gate_w")
    _on_gpu(logits, ids, gate_w)
    _check(lib().q8_moe_topk_softmax(logits.data_ptr(), T, E, topk, ids.data_ptr(),
                                     gate_w.data_ptr(), _stream(stream)), "q8_moe_topk_softmax")
    return ids, gate_w


def moe_router(Wr: PackedQ8, x, topk: int, logits=None, ids=None, gate_w=None, stream=None):
    """Router from a Q8_0 router matrix [E][K]: returns (logits fp32 [T][E],
    expert_ids int32 [T][topk], gate_w fp32 [T][topk])."""
    import torch
    x = _as_2d(x, Wr.K)
    T = x.shape[0]
    if logits is None:
        logits = torch.empty((T, Wr.M), dtype=torch.float32, device=x.device)
    if ids is None:
        ids = torch.empty((T, topk), dtype=torch.int32, device=x.device)
    if gate_w is None:
        gate_w = torch.empty((T, topk), dtype=torch.float32, device=x.device)
    _need(logits, (T, Wr.M), (torch.float32,), "logits")
    _need(ids, (T, topk), (torch.int32,), "ids")
    _need(gate_w, (T, topk), (torch.float32,), "gate_w")
    _on_gpu(Wr, x, logits, ids, gate_w)
    _check(lib().q8_moe_router(ctypes.byref(Wr.cmat()), x.data_ptr(), _dt(x), T, topk,
                               logits.data_ptr(), ids.data_ptr(), gate_w.data_ptr(),
                               _stream(stream)), "q8_moe_router")
    return logits, ids, gate_w


def moe_shared_ws_bytes(F: int, H: int, T: int) -> int:
    return lib().q8_moe_shared_ws_bytes(F, H, T)


def moe_shared_expert(Wg: PackedQ8, Wu: PackedQ8, Wd: PackedQ8, Wsg: PackedQ8, x, out,
                      ws=None, stream=None):
    """Shared expert added in place to ``out`` (fp32 [T][H], e.g. the routed
    output): out[t] += sigmoid(Wsg x_t) * Wd (silu(Wg x_t) * Wu x_t).
    Returns ``out``."""
    import torch
    x = _as_2d(x, Wg.K)
    T = x.shape[0]
    if out.dtype != torch.float32 or tuple(out.shape) != (T, Wg.K) or not out.is_contiguous():
        raise ValueError("out must be a contiguous fp32 [T][H] tensor")
    nws = moe_shared_ws_bytes(Wg.M, Wg.K, T)
    if ws is None:
        ws = torch.empty((nws,), dtype=torch.uint8, device=x.device)
    _need(ws, (ws.numel(),), (torch.uint8,), "ws")
    _on_gpu(Wg, Wu, Wd, Wsg, x, out, ws)
    _check(lib().q8_moe_shared_expert(ctypes.byref(Wg.cmat()), ctypes.byref(Wu.cmat()),
                                      ctypes.byref(Wd.cmat()), ctypes.byref(Wsg.cmat()),
                                      x.data_ptr(), _dt(x), T, out.data_ptr(), ws.data_ptr(),
                                      ws.numel() * ws.element_size(), _stream(stream)),
           "q8_moe_shared_expert")
    return out
