"""Seeded synthetic inputs for the Q8_0 decode workloads.

This module draws inputs only: int8 quants, fp16 block scales, fp16
activations, MoE routing ids and gate weights, and the GGUF-style 34-byte
block encoding of a weight matrix. It holds none of the GEMV arithmetic, so
both the CPU oracle (test side) and the HIP path can be fed from it.

Value distributions follow the decode-shaped workloads this library is
measured on (the pages run real Q8_0 GGUF models; these arrays stand in for
them):

* q  : int8, uniform on [-127, 127]
* d  : fp16 = RNE(|N(0, 0.02)| / 127), drawn in fp64 then rounded
* x  : fp16 = RNE(N(0, 1))

Draw order is fixed so that every array is a pure function of the seed:
weights first (one matrix after another, q then d), then x, then any
workload-specific extras (LM-head planting, MoE routing).

The Q8_0 block itself (an fp16 scale ``d`` followed by 32 int8 quants,
weight = d*q) is the GGUF format the memra pages load and decode (memra wiki,
feature list: the NVFP4/Q4_0/Q8_0 decode item and the loaders item;
topairepos memra listing, crate table row memra-gguf).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

QK = 32  # quants per Q8_0 block
BLOCK_BYTES = 2 + QK  # fp16 scale + 32 int8


def rng_for(seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(seed)


def draw_weights(rng: np.random.Generator, M: int, K: int):
    """One Q8_0 matrix [M][K]: returns (q int8 [M][K], d float16 [M][K/32])."""
    if K % QK:
        raise ValueError(f"K={K} is not a multiple of {QK}")
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    d = (np.abs(rng.normal(0.0, 0.02, size=(M, K // QK))) / 127.0).astype(np.float16)
    return q, d


def draw_weights_tiled(rng: np.random.Generator, M: int, K: int, q_period: int = 4099,
                       d_period: int = 4111):
    """A Q8_0 matrix of several GB at a small fraction of the drawing cost:
    the quants of q_period rows and the scales of d_period rows are drawn
    as in ``draw_weights``, and row m takes quant row m % q_period and scale
    row m % d_period. With two distinct primes no (quants, scales) pair
    recurs within q_period * d_period rows, so a row read from a wrong
    offset (a multiple of 2^31 or 2^32 bytes, say) meets other quants,
    other scales or both. Elementwise the distributions are those of
    ``draw_weights``."""
    if K % QK:
        raise ValueError(f"K={K} is not a multiple of {QK}")
    qb = rng.integers(-127, 128, size=(q_period, K), dtype=np.int8)
    db = (np.abs(rng.normal(0.0, 0.02, size=(d_period, K // QK))) / 127.0).astype(np.float16)

    def tile(block, period):
        out = np.empty((M,) + block.shape[1:], block.dtype)
        for m0 in range(0, M, period):
            out[m0:m0 + period] = block[:min(period, M - m0)]
        return out

    return tile(qb, q_period), tile(db, d_period)


def draw_x(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    return rng.normal(0.0, 1.0, size=(N, K)).astype(np.float16)


def to_gguf_blocks(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Encode (q [M][K], d [M][K/32]) as GGUF Q8_0 blocks: uint8 [M][K/32][34].

    Byte layout per block: little-endian fp16 scale (2 bytes) then the 32
    int8 quants in K order.
    """
    M, K = q.shape
    nb = K // QK
    out = np.empty((M, nb, BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = d.astype("<f2").view(np.uint8).reshape(M, nb, 2)
    out[:, :, 2:] = q.view(np.uint8).reshape(M, nb, QK)
    return out


@dataclasses.dataclass
class GemvCase:
    q: np.ndarray  # int8 [M][K]
    d: np.ndarray  # float16 [M][K/32]
    x: np.ndarray  # float16 [N][K]

    @property
    def M(self):
        return self.q.shape[0]

    @property
    def K(self):
        return self.q.shape[1]

    @property
    def N(self):
        return self.x.shape[0]


def gemv_case(M: int, K: int, N: int, seed: int = 0) -> GemvCase:
    """Dense decode GEMV workload (e.g. 1024x1024 or 5120x5120 at N=1)."""
    rng = rng_for(seed)
    q, d = draw_weights(rng, M, K)
    x = draw_x(rng, N, K)
    return GemvCase(q, d, x)


@dataclasses.dataclass
class PairCase:
    qa: np.ndarray
    da: np.ndarray
    qb: np.ndarray
    db: np.ndarray
    x: np.ndarray


def pair_case(M: int, K: int, N: int, seed: int = 0) -> PairCase:
    """Fused gate+up workload: two [M][K] matrices sharing one x (gate drawn first)."""
    rng = rng_for(seed)
    qa, da = draw_weights(rng, M, K)
    qb, db = draw_weights(rng, M, K)
    x = draw_x(rng, N, K)
    return PairCase(qa, da, qb, db, x)


def logit_sigma(K: int) -> float:
    """Analytic std of one logit sum_k d*q*x under the distributions above.

    Var = K * E[d^2] * E[q^2] * E[x^2], with E[d^2] = (0.02/127)^2,
    E[q^2] = 127*128/3 (uniform on -127..127) and E[x^2] = 1.
    """
    e_d2 = (0.02 / 127.0) ** 2
    e_q2 = 127.0 * 128.0 / 3.0
    return math.sqrt(K * e_d2 * e_q2)


def fp16_at_least(v: float) -> np.float16:
    """Smallest fp16 value >= v (v finite, positive)."""
    h = np.float16(v)
    if float(h) < v:
        h = np.nextafter(h, np.float16(np.inf))
    return h


@dataclasses.dataclass
class LmHeadCase:
    q: np.ndarray
    d: np.ndarray
    x: np.ndarray
    planted_rows: np.ndarray  # int64 [N]: the row planted as token n's argmax
    planted_target: np.ndarray  # float64 [N]: the analytic level the planted logit was raised to


def lmhead_case(V: int, K: int, N: int, seed: int = 0, lead_sigmas: float = 8.9) -> LmHeadCase:
    """LM-head workload with one planted argmax row per token.

    After drawing W and x, token n gets a distinct row r_n (drawn with
    ``rng.choice`` without replacement). Its quants become 127*sign(x[n,k])
    and every scale of the row becomes the smallest fp16 D_n with
    D_n * 127 * sum_k |x[n,k]| >= lead_sigmas * sigma, sigma the analytic
    logit std. The default 8.9 sigma sits about 3 sigma above the expected
    maximum of V Gaussian logits plus one sigma of slack, so the planted row
    leads the runner-up by at least 3 sigma; the tests confirm the margin
    with the oracle on the drawn data.
    """
    if N > V:
        raise ValueError("need N <= V distinct planted rows")
    rng = rng_for(seed)
    q, d = draw_weights(rng, V, K)
    x = draw_x(rng, N, K)
    rows = rng.choice(V, size=N, replace=False).astype(np.int64)
    target = plant_argmax_rows(q, d, x, rows, lead_sigmas)
    return LmHeadCase(q, d, x, rows, target)


def plant_argmax_rows(q: np.ndarray, d: np.ndarray, x: np.ndarray, rows, lead_sigmas: float = 8.9):
    """In place: row rows[n] becomes token n's planted argmax (quants
    127*sign(x[n,k]), every scale the smallest fp16 D_n with
    D_n * 127 * sum_k |x[n,k]| >= lead_sigmas * sigma). Returns the analytic
    targets, float64 [N]."""
    N, K = x.shape
    target = np.full(N, lead_sigmas * logit_sigma(K), dtype=np.float64)
    for n in range(N):
        xn = x[n].astype(np.float64)
        r = int(rows[n])
        q[r] = (np.sign(xn) * 127).astype(np.int8)
        s_abs = float(np.abs(xn).sum())
        d[r] = fp16_at_least(target[n] / (127.0 * s_abs))
    return target


@dataclasses.dataclass
class MoeCase:
    q_gate: np.ndarray  # int8 [E][F][H]
    d_gate: np.ndarray  # f16  [E][F][H/32]
    q_up: np.ndarray
    d_up: np.ndarray
    q_down: np.ndarray  # int8 [E][H][F]
    d_down: np.ndarray  # f16  [E][H][F/32]
    x: np.ndarray  # f16 [T][H]
    expert_ids: np.ndarray  # int32 [T][topk], distinct per token
    gate_w: np.ndarray  # f32 [T][topk]

    @property
    def E(self):
        return self.q_gate.shape[0]

    @property
    def F(self):
        return self.q_gate.shape[1]

    @property
    def H(self):
        return self.q_gate.shape[2]

    @property
    def T(self):
        return self.x.shape[0]

    @property
    def topk(self):
        return self.expert_ids.shape[1]


def moe_case(E: int, F: int, H: int, T: int, topk: int, seed: int = 0) -> MoeCase:
    """Routed-expert workload: E experts, each gate/up [F][H] and down [H][F].

    Draw order: for e in 0..E-1: gate (q, d), up (q, d), down (q, d); then
    x [T][H]; then per token ``rng.choice(E, topk, replace=False)``; then
    gate logits N(0,1) [T][topk], turned into per-token softmax weights in
    fp64 and rounded to fp32 (the router output this layer consumes).
    """
    if topk > E:
        raise ValueError("topk > E")
    rng = rng_for(seed)
    qg = np.empty((E, F, H), np.int8)
    dg = np.empty((E, F, H // QK), np.float16)
    qu = np.empty_like(qg)
    du = np.empty_like(dg)
    qd = np.empty((E, H, F), np.int8)
    dd = np.empty((E, H, F // QK), np.float16)
    for e in range(E):
        qg[e], dg[e] = draw_weights(rng, F, H)
        qu[e], du[e] = draw_weights(rng, F, H)
        qd[e], dd[e] = draw_weights(rng, H, F)
    x = draw_x(rng, T, H)
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(T)]).astype(np.int32)
    logits = rng.normal(0.0, 1.0, size=(T, topk))
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    gate_w = (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    return MoeCase(qg, dg, qu, du, qd, dd, x, ids, gate_w)


# Named workloads (sizes of one decode step's layer GEMVs).
WORKLOADS = {
    "gemv_1024": dict(kind="gemv", M=1024, K=1024, N=1),
    "gemv_5120": dict(kind="gemv", M=5120, K=5120, N=1),
    "pair_17408x5120": dict(kind="pair", M=17408, K=5120, Ns=(1, 2, 4, 8)),
    "lmhead_151936x5120": dict(kind="lmhead", V=151936, K=5120, Ns=(1, 4)),
    "moe_e128_top8_t16": dict(kind="moe", E=128, F=768, H=2048, T=16, topk=8),
}


def router_case(T: int, E: int, seed: int = 0, ties: bool = True) -> np.ndarray:
    """Router logits fp32 [T][E] ~ N(0,1). With ``ties``, token 0 gets an
    exact tie at its top (two experts share the largest logit) and token 1
    a block of equal logits, so the ordering rule for equal logits is
    exercised; a -0.0/+0.0 pair is planted where E allows."""
    rng = rng_for(seed)
    L = rng.normal(0.0, 1.0, size=(T, E)).astype(np.float32)
    if ties and E >= 4:
        L[0, E - 1] = L[0].max()
        L[0, 1] = L[0, E - 1]
        if T > 1:
            L[1, : E // 2] = np.float32(0.5)
        if T > 2:
            L[2, :] = np.float32(-3.0)
            L[2, E // 3] = np.float32(-0.0)
            L[2, E // 4] = np.float32(0.0)
    return L


# ---------------------------------------------------------------- Q4_0
def draw_weights_q4_0(rng: np.random.Generator, M: int, K: int):
    """One Q4_0 matrix [M][K]: (q int8 [M][K] uniform in -8..7, d float16
    [M][K/32] = |N(0, 0.02)| / 8, the same weight scale as the Q8_0 draws)."""
    q = rng.integers(-8, 8, size=(M, K), dtype=np.int8)
    d = (np.abs(rng.normal(0.0, 0.02, size=(M, K // QK))) / 8.0).astype(np.float16)
    return q, d


def to_gguf_q4_0_blocks(q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """(q in -8..7 [M][K], d [M][K/32]) -> GGUF Q4_0 blocks uint8 [M][K/32][18]:
    fp16 d little-endian, then byte j = (q[j+16] + 8) << 4 | (q[j] + 8)."""
    M, K = q.shape
    nb = K // QK
    u = (q.astype(np.int16) + 8).astype(np.uint8).reshape(M, nb, 32)
    out = np.empty((M, nb, 18), np.uint8)
    dv = np.ascontiguousarray(d, np.float16).view(np.uint16)
    out[:, :, 0] = (dv & 0xFF).astype(np.uint8)
    out[:, :, 1] = (dv >> 8).astype(np.uint8)
    out[:, :, 2:] = u[:, :, :16] | (u[:, :, 16:] << 4)
    return out


def q4_0_case(M: int, K: int, N: int, seed: int = 0) -> GemvCase:
    """Q4_0 GEMV workload: weights (q in -8..7, d) then x ~ N(0,1) fp16."""
    rng = rng_for(seed)
    q, d = draw_weights_q4_0(rng, M, K)
    x = draw_x(rng, N, K)
    return GemvCase(q, d, x)
