"""Pins for the oracle's tolerance functions (CPU only).

Every bound that gates a GPU result is pinned from two sides, by something
other than itself:

* soundness: an independent fp32 emulation of the device's evaluation order
  (numpy float32 arithmetic; the inputs displaced anywhere inside their own
  bounds, extremes included) stays inside the bound on many cases;
* tightness: an adversarial construction (every input error at its bound,
  signs aligned with the derivative) reaches most of the bound, so a bound
  made several times looser fails; a value displaced by twice the bound on
  a constructed worst case is rejected.

The device orders emulated here are those the library documents: the
router's weights are exp(l_j - l_0) summed by a 64-lane butterfly and
divided (fp32 expf), silu(g) u is g / (1 + expf(-g)) * u, the sigmoid gate
is 1 / (1 + expf(-z)), and the gated add is one fp32 fused multiply-add.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32
TINY = 2.0 ** -126


# ------------------------------------------------------------- fp32 helpers
def _ulp_nudge(v, steps):
    """Move fp32 values by `steps` (array of -1/0/+1) units in the last place."""
    v = np.asarray(v, F32)
    up = np.nextafter(v, F32(np.inf))
    dn = np.nextafter(v, F32(-np.inf))
    return np.where(steps > 0, up, np.where(steps < 0, dn, v)).astype(F32)


def _exp32(z, rng):
    """fp32 exp within one unit in the last place of the exact value (the
    device's expf accuracy), the unit chosen at random."""
    with np.errstate(over="ignore"):
        e = np.exp(np.asarray(z, np.float64)).astype(F32)
    return _ulp_nudge(e, rng.integers(-1, 2, size=np.shape(e)))


def _within(center, radius, sign, rng=None):
    """An fp32 value within `radius` of the exact `center`: at the edge in
    direction `sign` (0: uniformly inside), pulled back inside after the
    rounding to fp32."""
    center = np.asarray(center, np.float64)
    radius = np.asarray(radius, np.float64)
    if rng is not None:
        t = rng.uniform(-1, 1, size=np.broadcast(center, radius).shape)
        target = center + t * radius
    else:
        target = center + sign * radius
    v = target.astype(F32)
    over = np.abs(v.astype(np.float64) - center) > radius
    v = np.where(over, np.nextafter(v, center.astype(F32)), v).astype(F32)
    return v


# ------------------------------------------------------------- router softmax
def _softmax_device_order(sel, rng, flush):
    """Weights of the picked fp32 logits `sel` (descending) as the device
    evaluates them: fp32 differences to the first, expf, a 64-lane xor
    butterfly sum (32, 16, ..., 1), fp32 division."""
    k = len(sel)
    d = (sel - sel[0]).astype(F32)
    z = _exp32(d, rng)
    z[0] = F32(1.0)  # exp(0) is exact
    if flush:
        z = np.where(np.abs(z) < TINY, F32(0), z).astype(F32)
    lanes = np.zeros(64, F32)
    lanes[:k] = z
    s = lanes.copy()
    idx = np.arange(64)
    for delta in (32, 16, 8, 4, 2, 1):
        s = (s + s[idx ^ delta]).astype(F32)
    return (z / s[:k]).astype(F32)


def _router_logits(rng, case):
    E = int(rng.choice([8, 64, 128, 256]))
    k = min(E, int(rng.choice([1, 2, 8, 64])))
    kind = case % 6
    if kind == 0:
        L = rng.normal(0, 1, (1, E))
    elif kind == 1:
        L = rng.normal(0, 30, (1, E))  # weights down to fp32 underflow
    elif kind == 2:
        L = rng.integers(-3, 4, (1, E)).astype(float)  # ties
    elif kind == 3:
        L = rng.normal(0, 1, (1, E)) * 1e-39  # subnormal logits
    elif kind == 4:
        L = rng.normal(0, 10, (1, E)) + 100.0  # large magnitudes, inexact differences
    else:
        L = rng.normal(0, 1, (1, E)) * 1e4  # huge spread
    return L.astype(F32), k


def test_router_bound_contains_fp32_emulation():
    rng = np.random.default_rng(11)
    worst_rel = 0.0
    for case in range(1500):
        L, k = _router_logits(rng, case)
        ids, w, dl = oracle.topk_softmax(L, k)
        b = oracle.topk_softmax_bound(w, dl)[0]
        for flush in (False, True):
            we = _softmax_device_order(L[0, ids[0]], rng, flush)
            err = np.abs(we.astype(np.float64) - w[0])
            assert (err <= b).all(), (case, flush, (err / b).max())
            m = w[0] > 2.0 ** -100
            if m.any():
                worst_rel = max(worst_rel, float((err[m] / b[m]).max()))
    # the bound is not loose: fp32 reaches a sizeable part of it
    assert worst_rel >= 0.15, worst_rel


def test_router_bound_rejects_precision_mistakes():
    rng = np.random.default_rng(12)
    L = rng.normal(0, 2, (64, 128)).astype(F32)
    ids, w, dl = oracle.topk_softmax(L, 8)
    b = oracle.topk_softmax_bound(w, dl)
    # weights rounded through fp16 (a plausible storage mistake)
    w16 = w.astype(np.float16).astype(np.float64)
    assert (np.abs(w16 - w) > b).any()
    # a softmax over all experts, not renormalised to the picked ones
    full = np.exp(L.astype(np.float64) - L.max(axis=1, keepdims=True))
    full /= full.sum(axis=1, keepdims=True)
    wf = np.take_along_axis(full, ids.astype(np.int64), axis=1)
    assert (np.abs(wf - w) > b).all()


def test_router_bound_displaced_worst_case_fails():
    # largest bound: topk = 64 picks spread over a wide range of logits
    L = np.linspace(10, -60, 64).astype(F32)[None, :]
    ids, w, dl = oracle.topk_softmax(L, 64)
    b = oracle.topk_softmax_bound(w, dl)
    assert b.max() > 2.0 ** -23 * (2 * 64 + 8) * w.min()  # the worst case is large
    bad = w + 2 * b
    assert (np.abs(bad - w) > b).all()
    assert not (np.abs(bad - w) <= b).any()


# ------------------------------------------------------------- SiLU * mul
def _silu_mul_fp32(g32, u32, rng):
    """silu(g) * u as the device evaluates it: g / (1 + expf(-g)) * u."""
    e = _exp32(-g32.astype(np.float64), rng)
    den = (F32(1.0) + e).astype(F32)
    sg = (g32 / den).astype(F32)
    return (sg * u32).astype(F32)


_G_EXTREMES = np.array([-120.0, -90.0, -20.0, -5.0, -1.2785, -1e-3, 0.0, 1e-3, 1.0, 2.3994,
                        5.0, 20.0, 90.0, 120.0])


def test_silu_mul_bound_contains_fp32_emulation():
    rng = np.random.default_rng(21)
    n = 4000
    g = np.concatenate([rng.normal(0, 3, n), np.repeat(_G_EXTREMES, 50)])
    u = np.concatenate([rng.normal(0, 3, n), rng.normal(0, 50, 50 * len(_G_EXTREMES))])
    # GEMV bounds from plausible magnitudes: 1e-3 of an |g|-sized sum, some tiny
    bg = 1e-3 * np.abs(rng.normal(0, 3, g.size)) * rng.choice([1.0, 1e-3, 1e-6], g.size)
    bu = 1e-3 * np.abs(rng.normal(0, 3, u.size)) * rng.choice([1.0, 1e-3, 1e-6], u.size)
    h = oracle.silu(g) * u
    b = oracle.silu_mul_bound(g, u, bg, bu)
    for sg_ in (-1, 1):
        for su in (-1, 1):
            hv = _silu_mul_fp32(_within(g, bg, sg_), _within(u, bu, su), rng)
            err = np.abs(hv.astype(np.float64) - h)
            assert (err <= b).all(), (err / b).max()
    hv = _silu_mul_fp32(_within(g, bg, 0, rng), _within(u, bu, 0, rng), rng)
    assert (np.abs(hv.astype(np.float64) - h) <= b).all()


def test_silu_mul_bound_is_reached_near_the_steepest_point():
    # silu' peaks at ~1.0998 near z = 2.3994; errors aligned with it reach the bound
    g, u, bg, bu = np.array([2.3994]), np.array([1.5]), np.array([1e-3]), np.array([1e-3])
    h = oracle.silu(g) * u
    b = oracle.silu_mul_bound(g, u, bg, bu)
    exact = oracle.silu(g + bg) * (u + bu)  # no rounding: the propagation alone
    assert abs(exact[0] - h[0]) <= b[0]
    assert abs(exact[0] - h[0]) >= 0.95 * b[0]
    assert abs((h + 2 * b)[0] - h[0]) > b[0]


# ------------------------------------------------------------- sigmoid gate
def test_sigmoid_bound_contains_fp32_emulation_and_is_reached_at_zero():
    rng = np.random.default_rng(31)
    z = np.concatenate([rng.normal(0, 4, 3000), [-100.0, -30.0, -1.0, 0.0, 1.0, 30.0, 100.0]])
    bz = 1e-3 * np.abs(rng.normal(0, 4, z.size)) + 1e-7
    s = oracle.sigmoid(z)
    b = oracle.sigmoid_bound(s, bz)
    for sgn in (-1, 1, 0):
        zv = _within(z, bz, sgn, rng if sgn == 0 else None)
        e = _exp32(-zv.astype(np.float64), rng)
        sv = (F32(1.0) / (F32(1.0) + e).astype(F32)).astype(F32)
        err = np.abs(sv.astype(np.float64) - s)
        assert (err <= b).all(), (err / b).max()
    # at z = 0 the derivative is 1/4: an argument error of bz moves it by ~bz/4
    b0 = oracle.sigmoid_bound(np.array([0.5]), np.array([1e-3]))[0]
    moved = oracle.sigmoid(np.array([1e-3]))[0] - 0.5
    assert 0.95 * b0 <= moved <= b0


# ------------------------------------------------------------- down projection
def _small_q8(rng, M, K):
    q = rng.integers(-127, 128, (M, K)).astype(np.int8)
    d = (np.abs(rng.normal(0, 0.02, (M, K // 32))) / 127).astype(np.float16)
    return q, d


def _dense(q, d):
    M, K = q.shape
    return (q.astype(np.float64).reshape(M, -1, 32) * d.astype(np.float64)[:, :, None]).reshape(M, K)


def test_down_bound_adversarial_input_reaches_it():
    rng = np.random.default_rng(41)
    q, d = _small_q8(rng, 16, 64)
    W = _dense(q, d)
    h = rng.normal(0, 1, (3, 64)).astype(np.float32)
    bh = 1e-3 * np.abs(rng.normal(0, 1, (3, 64)))
    y, A = oracle.gemv(q, d, h)
    b = oracle.down_bound(q, d, A, bh)
    for n in range(3):
        for m in range(16):
            hp = h[n].astype(np.float64) + np.sign(W[m]) * bh[n]  # every input at its bound
            yp = W[m] @ hp + oracle.REL_TOL * (np.abs(W[m]) @ np.abs(hp))  # and the GEMV's own
            err = abs(yp - y[n, m])
            assert err <= b[n, m] * (1 + 1e-12)
            assert err >= 0.99 * b[n, m]


def test_down_bound_contains_fp32_gemv_of_perturbed_input():
    rng = np.random.default_rng(42)
    q, d = _small_q8(rng, 32, 96)
    W = _dense(q, d)
    h = rng.normal(0, 1, (4, 96)).astype(np.float32)
    bh = 1e-3 * np.abs(rng.normal(0, 1, (4, 96)))
    y, A = oracle.gemv(q, d, h)
    b = oracle.down_bound(q, d, A, bh)
    for trial in range(20):
        hp = _within(h.astype(np.float64), bh, 0, rng)
        # an fp32 GEMV in a shuffled order
        order = rng.permutation(96)
        acc = np.zeros((4, 32), F32)
        Wf = W.astype(F32)
        for k in order:
            acc = (acc + (hp[:, k:k + 1] * Wf[None, :, k]).astype(F32)).astype(F32)
        assert (np.abs(acc.astype(np.float64) - y) <= b).all()


# ------------------------------------------------------------- combine
def test_combine_bound_reached_and_contains_fp32_sum():
    rng = np.random.default_rng(51)
    T, topk, M = 5, 8, 40
    gw = rng.dirichlet(np.ones(topk), T).astype(np.float32)
    y = rng.normal(0, 2, (T, topk, M))
    per = 1e-3 * np.abs(rng.normal(0, 2, (T, topk, M)))
    out, S = oracle.moe_combine(gw, y.reshape(T * topk, M))
    b = oracle.combine_bound(gw, per, S)
    # every pair at its bound in the same direction
    yp = y + per
    outp = (gw.astype(np.float64)[:, :, None] * yp).sum(axis=1)
    err = np.abs(outp - out)
    assert (err <= b).all() and (err >= 0.99 * b).all()
    # fp32 ascending-j sum of fp32 pairs inside their bounds
    for trial in range(10):
        yp32 = _within(y, per, 0, rng)
        acc = np.zeros((T, M), F32)
        for j in range(topk):
            acc = np.fma(gw[:, j:j + 1], yp32[:, j], acc).astype(F32) if hasattr(np, "fma") else \
                (acc + (gw[:, j:j + 1] * yp32[:, j]).astype(F32)).astype(F32)
        assert (np.abs(acc.astype(np.float64) - out) <= b).all()


# ------------------------------------------------------------- gated add
def test_gated_add_bound_reached_and_contains_fp32_fma():
    rng = np.random.default_rng(61)
    n = 2000
    base = rng.normal(0, 5, n)
    s = rng.normal(0, 5, n)
    sg = rng.uniform(0.05, 1, n)
    bsg = 1e-4 * rng.uniform(0.1, 1, n)
    bs = 1e-3 * np.abs(s) * rng.uniform(0.1, 1, n)
    exact = base + sg * s
    b = oracle.gated_add_bound(base, sg, bsg, s, bs)
    adv = base + (sg + bsg) * (s + np.sign(s) * bs)
    err = np.abs(adv - exact)
    assert (err <= b).all()
    # with a small base the product's propagated error is nearly all of it
    small = oracle.gated_add_bound(1e-3 * base, sg, bsg, s, bs)
    assert (err >= 0.95 * small).all()
    for sgn in (-1, 1, 0):
        sgv = _within(sg, bsg, sgn, rng if sgn == 0 else None).astype(np.float64)
        sv = _within(s, bs, -sgn, rng if sgn == 0 else None).astype(np.float64)
        basev = base.astype(F32).astype(np.float64)
        # fp32 fma: one rounding of the exact sgv * sv + basev
        out32 = (sgv * sv + basev).astype(F32).astype(np.float64)
        assert (np.abs(out32 - (basev - base + exact)) <= b).all()


# ------------------------------------------------------------- compositions
def _moe_small(seed):
    from quantized_weight_gemv_q8_amd import synth
    return synth.moe_case(4, 64, 64, 3, 2, seed=seed)


def test_moe_ffn_bound_reached_by_stagewise_worst_case():
    """Each stage's output displaced to the edge of its own bound, signs
    aligned for one output: the end-to-end bound covers it and is nearly
    reached (a bound made looser inside moe_ffn would not be)."""
    c = _moe_small(3)
    r = oracle.moe_ffn(c)
    T, topk = c.expert_ids.shape
    s1 = r["stage1"]
    t, m = 1, 7
    out = 0.0
    for j in range(topk):
        p = t * topk + j
        e = c.expert_ids[t, j]
        W = _dense(c.q_down[e], c.d_down[e])
        hp = s1["h"][p].astype(np.float32).astype(np.float64) + np.sign(W[m]) * s1["bh"][p]
        yp = W[m] @ hp + oracle.REL_TOL * (np.abs(W[m]) @ np.abs(hp))
        out += float(c.gate_w[t, j]) * yp
    err = abs(out - r["out"][t, m])
    assert err <= r["bound"][t, m]
    assert err >= 0.9 * r["bound"][t, m]


def test_shared_expert_bound_reached_by_worst_case():
    rng = np.random.default_rng(71)
    F_, H_, T_ = 64, 32, 2
    qg, dg = _small_q8(rng, F_, H_)
    qu, du = _small_q8(rng, F_, H_)
    qd, dd = _small_q8(rng, H_, F_)
    qs_, ds_ = _small_q8(rng, 1, H_)
    x = rng.normal(0, 1, (T_, H_)).astype(np.float16)
    base = rng.normal(0, 1, (T_, H_))
    r = oracle.shared_expert(qg, dg, qu, du, qd, dd, qs_, ds_, x, base)
    st = oracle.gate_up_silu(qg, dg, qu, du, x)
    s_, As = oracle.gemv(qd, dd, st["h"].astype(np.float32))
    bs = oracle.down_bound(qd, dd, As, st["bh"])
    gl, Agl = oracle.gemv(qs_, ds_, x)
    sg = oracle.sigmoid(gl[:, 0])
    bsg = oracle.sigmoid_bound(sg, oracle.REL_TOL * Agl[:, 0])
    t, m = 0, 5
    sgn = np.sign(s_[t, m]) or 1.0
    adv = base[t, m] + (sg[t] + bsg[t]) * (s_[t, m] + sgn * bs[t, m])
    err = abs(adv - r["out"][t, m])
    assert err <= r["bound"][t, m]
    assert err >= 0.8 * r["bound"][t, m]  # the rest is the fp32 allowance


# ------------------------------------------------------------- fp16 output bound
def test_fp16_output_bound_contains_rounded_fp32_results():
    rng = np.random.default_rng(81)
    K = 5120
    gamma = (K + 1) * 2.0 ** -24 / (1 - (K + 1) * 2.0 ** -24)  # Higham's gamma_{K+1}
    y = np.concatenate([rng.normal(0, 1, 3000), rng.normal(0, 1, 3000) * 1e-6,
                        2.0 ** np.arange(-24, 8) * (1 - 2.0 ** -12), 2.0 ** np.arange(-24, 8)])
    A = np.abs(y) * rng.uniform(1, 50, y.size)
    A[:50] = 0.0
    y[:50] = 0.0
    b = oracle.bound(A, y, "f16")
    for sgn in (-1, 1):
        y32 = (y + sgn * gamma * A).astype(F32)
        y16 = y32.astype(np.float16).astype(np.float64)  # round to nearest even
        assert (np.abs(y16 - y) <= b).all()


def test_fp16_output_bound_half_ulp_is_tight_for_subnormal_outputs():
    # outputs in the fp16 subnormal range with a negligible GEMV error: the
    # correctly rounded value (0.3 units of 2^-24 away) passes; the other
    # neighbour (0.7 units away, the wrong rounding direction) fails
    y = (np.arange(1, 200) * 2.0 ** -24) + 0.3 * 2.0 ** -24
    A = np.abs(y) * 1e-6
    b = oracle.bound(A, y, "f16")
    y16 = y.astype(np.float16).astype(np.float64)
    assert (np.abs(y16 - y) <= b).all()
    off = y16 + 2.0 ** -24
    assert (np.abs(off - y) > b).all()
