"""CPU oracle for Q8_0 weight-only GEMV, LM-head argmax and routed-expert FFN.

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this package. It shares no code with
the HIP library (``quantized_weight_gemv_q8_amd``) and imports nothing from
it; both are fed from the seeded generator, which holds no GEMV arithmetic.

Layers:

* ``q8_oracle.c`` (plain C, fp64, sequential in k; built by gcc with
  -ffp-contract=off, no fast-math): the dequant-and-dot itself, its own fp16
  and GGUF block decoders.
* this module: the gates built on it. Each function names the passage it
  follows.

Sources: memra wiki (feature list: Q8_0 decode matvecs, expert-major CSR
MoE batching, CUDA-graph decode returning 4 bytes/token; gate paragraph:
kernel-check of every kernel against a CPU reference, the run-gen argmax
gate) and memra performance (serving exactness arc: a request's tokens must
not depend on its co-arrivals). The numeric contract (per-output error at
most 1e-3 * sum|d*q*x|; argmax identical wherever the top-2 gap exceeds that
bound) is the library's stated acceptance bar; the pages fix the format and
the gates, not a tolerance.
"""

from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

REL_TOL = 1e-3  # per-output bound: |err| <= REL_TOL * sum_k |d*q*x|
QK = 32

_lib = None


def build(force: bool = True) -> str:
    """Compile q8_oracle.c with gcc (plain C, IEEE fp64, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lpthread", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.or_half_to_double.argtypes = [ctypes.c_uint16]
        L.or_half_to_double.restype = ctypes.c_double
        L.or_decode_blocks.argtypes = [vp, i64, i64, vp, vp]
        L.or_decode_blocks.restype = i32
        L.or_gemv_f16x.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i32]
        L.or_gemv_f16x.restype = i32
        L.or_gemv_f32x.argtypes = [vp, vp, i64, i64, vp, i64, vp, vp, i32]
        L.or_gemv_f32x.restype = i32
        L.or_gemv_rows_f16x.argtypes = [vp, vp, i64, i64, vp, i64, vp, i64, vp, vp, i32]
        L.or_gemv_rows_f16x.restype = i32
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ---------------------------------------------------------------- decoding
def half_to_double(bits: int) -> float:
    """IEEE binary16 bit pattern -> exact float (oracle's own decoder)."""
    return _get().or_half_to_double(bits & 0xFFFF)


def decode_blocks(blocks: np.ndarray):
    """GGUF Q8_0 blocks uint8 [M][K/32][34] -> (q int8 [M][K], d fp16 [M][K/32])."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
    M, nb, bb = blocks.shape
    if bb != 2 + QK:
        raise ValueError("Q8_0 blocks are 34 bytes")
    K = nb * QK
    q = np.empty((M, K), np.int8)
    d = np.empty((M, nb), np.uint16)
    rc = _get().or_decode_blocks(_p(blocks), M, K, _p(q), _p(d))
    if rc:
        raise ValueError(f"or_decode_blocks rc={rc}")
    return q, d.view(np.float16)


# ---------------------------------------------------------------- the GEMV
def gemv(q: np.ndarray, d: np.ndarray, x: np.ndarray, threads: int = 1):
    """y[n][m] = sum_k d[m][k/32]*q[m][k]*x[n][k] in fp64; also A = sum|terms|.

    x may be fp16 (decode activations) or fp32 (MoE intermediate h).
    Returns (y, A), both float64 [N][M].
    """
    q = np.ascontiguousarray(q, np.int8)
    d16 = np.ascontiguousarray(d, np.float16).view(np.uint16)
    M, K = q.shape
    if d16.shape != (M, K // QK) or K % QK:
        raise ValueError("shape mismatch between q and d")
    x = np.ascontiguousarray(x)
    if x.ndim != 2 or x.shape[1] != K:
        raise ValueError("x must be [N][K]")
    N = x.shape[0]
    y = np.empty((N, M), np.float64)
    A = np.empty((N, M), np.float64)
    L = _get()
    if x.dtype == np.float16:
        rc = L.or_gemv_f16x(_p(q), _p(d16), M, K, _p(x.view(np.uint16)), N, _p(y), _p(A), threads)
    elif x.dtype == np.float32:
        rc = L.or_gemv_f32x(_p(q), _p(d16), M, K, _p(x), N, _p(y), _p(A), threads)
    else:
        raise TypeError("x must be float16 or float32")
    if rc:
        raise ValueError(f"oracle gemv rc={rc}")
    return y, A


def gemv_rows(q, d, x, rows, threads: int = 1):
    """Oracle on a sample of weight rows: returns (y, A) float64 [N][len(rows)]."""
    q = np.ascontiguousarray(q, np.int8)
    d16 = np.ascontiguousarray(d, np.float16).view(np.uint16)
    x = np.ascontiguousarray(x, np.float16)
    rows = np.ascontiguousarray(rows, np.int64)
    M, K = q.shape
    N = x.shape[0]
    R = rows.shape[0]
    y = np.empty((N, R), np.float64)
    A = np.empty((N, R), np.float64)
    rc = _get().or_gemv_rows_f16x(_p(q), _p(d16), M, K, _p(x.view(np.uint16)), N,
                                  _p(rows), R, _p(y), _p(A), threads)
    if rc:
        raise ValueError(f"oracle gemv_rows rc={rc}")
    return y, A


def bound(A: np.ndarray, y: np.ndarray | None = None, out_dtype: str = "f32") -> np.ndarray:
    """Per-output acceptance bound.

    b = 1e-3 * A. When the output is stored as fp16, add half an fp16 ulp of
    the exact result, which covers the final rounding for fp16-subnormal
    outputs; for normal outputs the fp16 rounding already fits inside b.
    """
    b = REL_TOL * np.asarray(A, np.float64)
    if out_dtype == "f16":
        if y is None:
            raise ValueError("fp16 bound needs y")
        b = b + 0.5 * fp16_ulp(y)
    return b


def fp16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of fp16 values at |v| (2^-24 for subnormals and zero)."""
    a = np.abs(np.asarray(v, np.float64))
    out = np.full(a.shape, 2.0 ** -24)
    nz = a >= 2.0 ** -14
    e = np.floor(np.log2(a[nz]))
    out[nz] = 2.0 ** (e - 10)
    return out


def check_close(y_gpu: np.ndarray, y: np.ndarray, A: np.ndarray, out_dtype: str = "f32"):
    """GEMV gate: pass iff |y_gpu - y| <= bound for every output.

    Returns (ok, max_rel, n_bad) with max_rel = max |y_gpu - y| / A (0 where
    A == 0; there y_gpu must be exactly zero).
    """
    y_gpu = np.asarray(y_gpu, np.float64)
    err = np.abs(y_gpu - y)
    b = bound(A, y, out_dtype)
    bad = ~(err <= b)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(A > 0, err / np.where(A > 0, A, 1.0), np.where(err > 0, np.inf, 0.0))
    return (not bad.any()), float(rel.max(initial=0.0)), int(bad.sum())


# ---------------------------------------------------------------- argmax gate
def argmax_first(L: np.ndarray) -> np.ndarray:
    """Index of the first maximum of each row (ties -> lowest index; -0 == +0)."""
    return np.argmax(np.asarray(L, np.float64), axis=-1)


def argmax_gate(L: np.ndarray, A: np.ndarray):
    """Which tokens have an argmax that the bound cannot flip.

    For each token n: i* = first argmax of the oracle logits L[n];
    b = 1e-3*A[n]. Token n is gated (exact argmax required) iff
    L[n,i*] - b[n,i*] > max_{j != i*} (L[n,j] + b[n,j]); otherwise any id in
    the candidate set {j : L[n,j] + b[n,j] >= L[n,i*] - b[n,i*]} is correct.
    Follows the run-gen argmax gate (memra wiki, gate paragraph: the argmax
    must MATCH before any number counts).

    Returns (istar int64 [N], gated bool [N], candidates list of int arrays).
    """
    L = np.asarray(L, np.float64)
    b = REL_TOL * np.asarray(A, np.float64)
    N = L.shape[0]
    istar = argmax_first(L)
    gated = np.zeros(N, bool)
    cands = []
    for n in range(N):
        i = istar[n]
        lo = L[n, i] - b[n, i]
        hi = L[n] + b[n]
        others = np.delete(hi, i)
        gated[n] = bool(lo > (others.max() if others.size else -np.inf))
        cands.append(np.nonzero(hi >= lo)[0])
    return istar, gated, cands


# ---------------------------------------------------------------- MoE
def moe_route(expert_ids: np.ndarray, E: int):
    """Expert-major CSR of the routed (token, slot) pairs.

    Pair p = t*topk + j. counts[e] = #pairs routed to e; offsets = exclusive
    prefix sum (E+1 entries); pairs lists p grouped by expert in ascending e,
    and inside one expert in ascending p. active = experts with counts > 0,
    ascending. Follows the expert-major CSR batching of routed experts
    (memra wiki, feature list, the MoE item).
    """
    ids = np.asarray(expert_ids)
    T, topk = ids.shape
    counts = np.zeros(E, np.int32)
    buckets = [[] for _ in range(E)]
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if not 0 <= e < E:
                raise ValueError(f"expert id {e} out of range")
            counts[e] += 1
            buckets[e].append(t * topk + j)
    offsets = np.zeros(E + 1, np.int32)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    pairs = np.array([p for e in range(E) for p in buckets[e]], np.int32)
    active = np.array([e for e in range(E) if counts[e] > 0], np.int32)
    return counts, offsets, pairs, active


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)) in fp64, evaluated as z * e^z / (1 + e^z)
    for z < 0 (the same function; exp(-z) would overflow below z = -709)."""
    z = np.asarray(z, np.float64)
    ez = np.exp(np.minimum(z, 0.0))
    return np.where(z >= 0, z / (1.0 + np.exp(-np.maximum(z, 0.0))), z * ez / (1.0 + ez))


# ---------------------------------------------------------------- propagated bounds
# Each step after a GEMV receives inputs that are only known to lie within
# their own bounds; these functions carry those bounds through the step
# (first-order terms with the derivative's maximum, the second-order cross
# term, and a relative allowance for the step's own fp32 rounding taken on
# the magnitudes the device may see). Each is pinned by an adversarial
# construction that reaches it and by an fp32 emulation that stays inside.

def silu_mul_bound(g, u, bg, bu):
    """Bound on h' - silu(g)*u for h' = silu(g')*u' evaluated in fp32, when
    |g' - g| <= bg and |u' - u| <= bu.

    silu(g') u' - silu(g) u = (silu(g') - silu(g)) u + silu(g') (u' - u),
    with |silu'| <= 1.0999 < 1.1 (its maximum, near z = 2.4) and
    |silu(g')| <= |silu(g)| + 1.1 bg, so the exact part is at most
    P = 1.1 bg |u| + |silu(g)| bu + 1.1 bg bu. The fp32 evaluation (exp,
    add, divide, multiply: a few units of 2^-24 each) adds at most
    1e-6 (|h| + P), h = silu(g) u.
    """
    g = np.asarray(g, np.float64)
    u = np.asarray(u, np.float64)
    sg = silu(g)
    P = 1.1 * bg * np.abs(u) + np.abs(sg) * bu + 1.1 * bg * bu
    return P + 1e-6 * (np.abs(sg * u) + P)


def down_bound(qd, dd, A_down, bh):
    """Bound on a GEMV W_down h' whose input h' is within bh of h.

    |W h' - W h| <= |W| bh (|W| the elementwise absolute dequantized
    weights); the GEMV's own error is at most 1e-3 * A(h') and
    A(h') <= A(h) + |W| bh, so the total is
    1e-3 * A(h) + (1 + 1e-3) |W| bh. A_down [N][M] is A(h) from ``gemv``;
    bh is [N][K].
    """
    M = qd.shape[0]
    wabs = (np.abs(np.asarray(qd).astype(np.int32)).astype(np.float64).reshape(M, -1, QK)
            * np.asarray(dd, np.float64)[:, :, None]).reshape(M, -1)
    return REL_TOL * np.asarray(A_down, np.float64) + (1.0 + REL_TOL) * (np.asarray(bh) @ wabs.T)


def combine_bound(gate_w, per_pair, S):
    """Bound on sum_j w_j y'_j (fp32, ascending j) when each y'_j is within
    per_pair[:, j] of y_j: sum_j w_j per_pair_j, plus 1e-6 of the magnitude
    the fp32 sum may see, S + that sum (S = sum_j |w_j y_j|). per_pair is
    [T][topk][M]; S is [T][M]."""
    gw = np.asarray(gate_w, np.float64)
    prop = (np.abs(gw)[:, :, None] * np.asarray(per_pair, np.float64)).sum(axis=1)
    return prop + 1e-6 * (np.asarray(S, np.float64) + prop)


def sigmoid_bound(sg, b_arg):
    """Bound on an fp32 sigmoid(z') when |z' - z| <= b_arg and sg =
    sigmoid(z): |sigma'| <= 1/4 gives L = b_arg / 4; exp, add and
    reciprocal in fp32 add at most 1e-6 (sg + L)."""
    L = 0.25 * np.asarray(b_arg, np.float64)
    return L + 1e-6 * (np.asarray(sg, np.float64) + L)


def gated_add_bound(base, sg, bsg, s, bs):
    """Bound on base + sg' * s' (fp32 fused multiply-add) when |sg' - sg| <=
    bsg and |s' - s| <= bs: the product's error sg bs + bsg |s| + bsg bs,
    plus 1e-6 of the magnitude the fp32 result may see."""
    s = np.asarray(s, np.float64)
    P = sg * bs + bsg * np.abs(s) + bsg * bs
    return P + 1e-6 * (np.abs(np.asarray(base, np.float64)) + sg * np.abs(s) + P)


def moe_gate_up(case, threads: int = 1):
    """Stage 1 of the routed FFN: per pair p=(t,j) with e = ids[t,j]:
    g = W_gate[e] x_t, u = W_up[e] x_t (fp64), their A sums, and
    h = silu(g) * u with a propagated bound.

    Bound on h (fp32 GPU h vs this fp64 h): ``silu_mul_bound`` of the two
    GEMV bounds. Returns dict of [P][F] arrays in pair order p = t*topk + j.
    """
    T, topk = case.expert_ids.shape
    F = case.q_gate.shape[1]
    P = T * topk
    g = np.empty((P, F)); u = np.empty((P, F)); Ag = np.empty((P, F)); Au = np.empty((P, F))
    for e in np.unique(case.expert_ids):
        tj = np.argwhere(case.expert_ids == e)
        xs = case.x[tj[:, 0]]
        ge, age = gemv(case.q_gate[e], case.d_gate[e], xs, threads)
        ue, aue = gemv(case.q_up[e], case.d_up[e], xs, threads)
        p = tj[:, 0] * topk + tj[:, 1]
        g[p], Ag[p], u[p], Au[p] = ge, age, ue, aue
    h = silu(g) * u
    bh = silu_mul_bound(g, u, REL_TOL * Ag, REL_TOL * Au)
    return dict(g=g, u=u, Ag=Ag, Au=Au, h=h, bh=bh)


def moe_down(case, h_pairs: np.ndarray, threads: int = 1):
    """Stage 2: y_pair[p] = W_down[e] h[p] (fp64) for the given fp32 h [P][F].

    Takes the GPU's own h as input so the down GEMV is gated against exactly
    the activations it consumed. Returns (y_pair [P][H], A [P][H]).
    """
    T, topk = case.expert_ids.shape
    H = case.q_down.shape[1]
    P = T * topk
    h_pairs = np.ascontiguousarray(h_pairs, np.float32)
    y = np.empty((P, H)); A = np.empty((P, H))
    for e in np.unique(case.expert_ids):
        tj = np.argwhere(case.expert_ids == e)
        p = tj[:, 0] * topk + tj[:, 1]
        ye, ae = gemv(case.q_down[e], case.d_down[e], h_pairs[p], threads)
        y[p], A[p] = ye, ae
    return y, A


def moe_combine(gate_w: np.ndarray, y_pairs: np.ndarray):
    """Stage 3: out[t] = sum_j gate_w[t,j] * y_pair[t*topk+j] (ascending j), fp64.

    Returns (out [T][H], S [T][H] = sum_j |gate_w * y_pair|).
    """
    gw = np.asarray(gate_w, np.float64)
    T, topk = gw.shape
    yp = np.asarray(y_pairs, np.float64).reshape(T, topk, -1)
    out = np.zeros((T, yp.shape[2]))
    S = np.zeros_like(out)
    for j in range(topk):
        out = out + gw[:, j:j + 1] * yp[:, j]
        S = S + np.abs(gw[:, j:j + 1] * yp[:, j])
    return out, S


def moe_ffn(case, threads: int = 1):
    """End-to-end chain: out[t] = sum_j w_tj * W_down[e] (silu(W_gate[e] x_t) * W_up[e] x_t).

    The down stage consumes h rounded to fp32 (the activation dtype the
    GPU's down GEMV reads); that rounding (<= 2^-24 |h|) is inside the
    1e-6*|h| term of the h bound. Also returns a propagated bound for an
    fp32 GPU result: per pair ``down_bound`` (the down GEMV's own bound plus
    |W_down| applied to the h bound), then ``combine_bound`` over the
    gate-weighted pairs.
    """
    s1 = moe_gate_up(case, threads)
    y, Ay = moe_down(case, s1["h"].astype(np.float32), threads)
    T, topk = case.expert_ids.shape
    H = case.q_down.shape[1]
    per_pair = np.zeros((T * topk, H))
    for e in np.unique(case.expert_ids):
        tj = np.argwhere(case.expert_ids == e)
        p = tj[:, 0] * topk + tj[:, 1]
        per_pair[p] = down_bound(case.q_down[e], case.d_down[e], Ay[p], s1["bh"][p])
    out, S = moe_combine(case.gate_w, y)
    b = combine_bound(case.gate_w, per_pair.reshape(T, topk, H), S)
    return dict(out=out, bound=b, stage1=s1, y_pair=y, A_pair=Ay)


# ---------------------------------------------------------------- router
def topk_softmax(logits: np.ndarray, topk: int):
    """Router of a routed layer: per token, pick the topk experts with the
    largest router logits and weight them by a softmax over the picked logits.

    The pages route on the device with m-invariant router kernels and require
    a token's routing not to depend on its co-arrivals (memra performance,
    serving exactness arc). They do not spell out the router's arithmetic;
    this is the plain reading used by the library: selection compares the
    fp32 logits exactly, in descending order, equal logits going to the
    lower expert index first (-0 equals +0); the weights are
    w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the picked logits, in
    fp64 (l_0 is the largest). Renormalising a softmax over all experts to
    the picked ones gives the same weights.

    Returns (ids int32 [T][topk], w float64 [T][topk], dl float64 [T][topk]
    with dl = l_0 - l_j >= 0).
    """
    L = np.asarray(logits, np.float32)
    T, E = L.shape
    if not 1 <= topk <= E:
        raise ValueError("need 1 <= topk <= E")
    if not np.isfinite(L).all():
        raise ValueError("router logits must be finite")
    ids = np.empty((T, topk), np.int32)
    w = np.empty((T, topk))
    dl = np.empty((T, topk))
    idx = np.arange(E)
    for t in range(T):
        v = L[t].astype(np.float64)
        order = np.lexsort((idx, -v))[:topk]  # primary: larger logit; then lower index
        sel = v[order]
        z = np.exp(sel - sel[0])
        ids[t] = order
        w[t] = z / z.sum()
        dl[t] = sel[0] - sel
    return ids, w, dl


def topk_softmax_bound(w: np.ndarray, dl: np.ndarray) -> np.ndarray:
    """Error bound for fp32 router weights against ``topk_softmax``.

    An fp32 evaluation rounds l_j - l_0 (relative 2^-24, so an absolute
    2^-24*dl_j in the exponent), evaluates exp (a few ulps), sums topk
    positive terms (at most (topk-1)*2^-24 relative) and divides (2^-24):
    |dw_j| <= 2^-23 * (dl_j + 2*topk + 8) * w_j, with margin. Weights
    below fp32's smallest normal number (exp(l_j - l_0) under about
    e^-87) carry no relative precision (subnormal, or flushed to zero by
    the device's exp): they get an absolute allowance of 2^-126.
    """
    topk = w.shape[-1]
    return 2.0 ** -23 * (dl + 2 * topk + 8) * w + 2.0 ** -126


# ---------------------------------------------------------------- dense gate/up
def gate_up_silu(qg, dg, qu, du, x, threads: int = 1, out_dtype: str = "f32"):
    """Dense SiLU-gated pair of an MLP: h = silu(W_gate x) * (W_up x), fp64.

    The MLP step after the fused gate+up pair (memra performance, qwen/silu
    class): silu(z) = z / (1 + exp(-z)). Bound on an fp32 (or fp16) GPU h:
    ``silu_mul_bound`` of the two GEMV bounds (+ half an fp16 ulp of h for
    fp16 output).
    Returns dict(h, bh, g, u) of [N][M] arrays.
    """
    g, Ag = gemv(qg, dg, x, threads)
    u, Au = gemv(qu, du, x, threads)
    h = silu(g) * u
    bh = silu_mul_bound(g, u, REL_TOL * Ag, REL_TOL * Au)
    if out_dtype == "f16":
        bh = bh + 0.5 * fp16_ulp(h)
    return dict(h=h, bh=bh, g=g, u=u)


# ---------------------------------------------------------------- shared expert
def sigmoid(z: np.ndarray) -> np.ndarray:
    """sigma(z) = 1 / (1 + e^-z) in fp64, as e^z / (1 + e^z) for z < 0 (the
    same function, without overflow of e^-z)."""
    z = np.asarray(z, np.float64)
    ez = np.exp(np.minimum(z, 0.0))
    return np.where(z >= 0, 1.0 / (1.0 + np.exp(-np.maximum(z, 0.0))), ez / (1.0 + ez))


def shared_expert(qg, dg, qu, du, qd, dd, qsg, dsg, x, base, threads: int = 1):
    """Shared expert of a routed MoE layer, added to the routed output:
    out[t] = base[t] + sigmoid(w_sg . x_t) * W_down (silu(W_gate x_t) * W_up x_t).

    The pages' MoE models run a dense expert on every token beside the
    routed ones, scaled per token by its own sigmoid gate, and count that
    gate's dot product among the decode kernels they fused (memra wiki,
    board notes on the 35B MoE decode; memra performance, flip history).
    The plain reading: the shared expert is an MLP of the routed experts'
    shape (gate/up [F][H], down [H][F]); the gate is one row [1][H] whose
    dot with x_t goes through a logistic sigmoid; the result is added to
    the routed output.

    fp64 throughout; the down GEMV takes h rounded to fp32 (the GPU's
    activation dtype; the rounding is inside the 1e-6 * |h| term of h's
    bound). Bound on an fp32 GPU result: ``gated_add_bound`` of the gate's
    ``sigmoid_bound`` and the down projection's ``down_bound`` (b_h from
    gate_up_silu). Returns dict(out, bound, s, gate, h) with out [T][H],
    gate [T].
    """
    st = gate_up_silu(qg, dg, qu, du, x, threads)
    s, As = gemv(qd, dd, st["h"].astype(np.float32), threads)
    bs = down_bound(qd, dd, As, st["bh"])
    gl, Agl = gemv(qsg, dsg, x, threads)
    sg = sigmoid(gl[:, 0])
    bsg = sigmoid_bound(sg, REL_TOL * Agl[:, 0])
    base = np.asarray(base, np.float64)
    out = base + sg[:, None] * s
    bound = gated_add_bound(base, sg[:, None], bsg[:, None], s, bs)
    return dict(out=out, bound=bound, s=s, gate=sg, h=st["h"])


# ---------------------------------------------------------------- masked LM head
def argmax_masked(L_sub: np.ndarray, A_sub: np.ndarray, row_ids: np.ndarray):
    """Argmax over a ranked subset of the vocabulary (the pages' draft LM
    head, which reads only the rows of a chosen subset: memra wiki, MTP
    speculative decoding with a vocab-masked draft head).

    L_sub [N][S] are the logits of the subset rows in subset order, A_sub
    their sum|d*q*x|; row_ids [S] the vocabulary id of each subset row. The
    winner is the first maximum in subset order, reported as its vocabulary
    id; gating as ``argmax_gate`` on the subset. Returns (ids int64 [N],
    gated bool [N], candidate vocabulary ids per token).
    """
    row_ids = np.asarray(row_ids, np.int64)
    istar, gated, cands = argmax_gate(L_sub, A_sub)
    return row_ids[istar], gated, [row_ids[c] for c in cands]


# ---------------------------------------------------------------- Q4_0
def decode_q4_0_blocks(blocks: np.ndarray):
    """GGUF Q4_0 blocks [M][K/32][18] -> (q int8 [M][K] in -8..7, d float16 [M][K/32]).

    The pages decode Q4_0 next to Q8_0 (memra wiki, feature list) but print
    no bytes; this is the standard GGUF block: little-endian fp16 d, then 16
    bytes whose low nibbles are elements 0..15 and high nibbles elements
    16..31 of the block, each stored with +8; the weight is d * (nibble - 8).
    The GEMV over the decoded (q, d) is then the same definition as for
    Q8_0 (``gemv``).
    """
    b = np.asarray(blocks, np.uint8)
    M, nb, _ = b.shape
    d = (b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)).view(np.float16)
    qs = b[:, :, 2:].astype(np.int16)
    lo = (qs & 0x0F) - 8
    hi = (qs >> 4) - 8
    q = np.concatenate([lo, hi], axis=2).reshape(M, nb * 32).astype(np.int8)
    return q, d
