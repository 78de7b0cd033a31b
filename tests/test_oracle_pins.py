"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: the checks are hand-worked
values from tests/golden (each with its citation), brute force against
numpy's integer matmul, closed forms (sigmoid, softmax), the dequantisation
error bound, and invariants.  Each is chosen so that a plausible slip in the
oracle -- a dropped term, a wrong sign, a swapped index, a transposed
operand, gate and up exchanged -- fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- quantisation
@pytest.mark.parametrize("case", _gold("quant_pins.json")["cases"])
def test_quant_hand_worked(case):
    q, s = oracle.quantize_rows(np.array(case["x"], np.float32))
    assert s[0] == np.float32(case["s"])
    assert q[0].tolist() == case["q"]


def test_quant_invariants():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((37, 203)).astype(np.float32)
    x[:, 5] *= 40.0
    q, s = oracle.quantize_rows(x)
    # |q| <= 127 and the row's largest magnitude maps to +-127
    assert np.abs(q.astype(np.int32)).max() <= 127
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(37), am].astype(np.int32)) == 127)
    assert np.all(np.sign(q[np.arange(37), am]) == np.sign(x[np.arange(37), am]))
    # sign symmetry
    qn, sn = oracle.quantize_rows(-x)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    # power-of-two scaling: codes unchanged, scale scaled exactly
    for p in (-7, 3, 20):
        qp, sp = oracle.quantize_rows(x * np.float32(2.0 ** p))
        assert np.array_equal(qp, q)
        assert np.array_equal(sp, s * np.float32(2.0 ** p))
    # s is max|x| / 127 (to one fp32 rounding)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    assert np.all(np.abs(s.astype(np.float64) - amax / 127.0) <= amax / 127.0 * 2.0 ** -23)
    # dequantisation error bound of round-to-nearest: |x - q*s| <= s/2 (+ fp32 slack)
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))


def test_quant_is_round_half_even_of_fp32_quotient():
    # the decision is taken on the fp32 quotient x/s: q is its nearest
    # integer, ties going to the even one.
    rng = np.random.default_rng(2)
    x = (rng.integers(-508, 509, size=(8, 64)) / 4.0).astype(np.float32)  # many exact halves
    x[:, 0] = 127.0  # s = 1 exactly, so x/s = x
    q, s = oracle.quantize_rows(x)
    assert np.all(s == 1.0)
    v = x.astype(np.float64)
    fl = np.floor(v)
    frac = v - fl
    expect = np.where(frac < 0.5, fl, np.where(frac > 0.5, fl + 1, np.where(fl % 2 == 0, fl, fl + 1)))
    assert np.array_equal(q.astype(np.float64), np.clip(expect, -128, 127))


# ---------------------------------------------------------------- int GEMM
def test_gemm_hand_worked():
    g = _gold("gemm_pins.json")
    acc = oracle.gemm_i32(np.array(g["a"], np.int8), np.array(g["b_nk"], np.int8))
    assert acc.tolist() == g["acc"]
    out = oracle.dense_w8a8(np.array(g["a"], np.int8), np.array(g["s_a"], np.float32),
                            np.array(g["b_nk"], np.int8), np.array(g["s_b"], np.float32))
    assert out.tolist() == g["out"]
    ex = g["extreme"]
    acc = oracle.gemm_i32(np.array(ex["a"], np.int8), np.array(ex["b_nk"], np.int8))
    assert acc.tolist() == ex["acc"]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 33, 65), (64, 48, 256), (5, 130, 1000)])
def test_gemm_brute_force(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    a = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    a[0, 0] = -128
    b[0, 0] = -128
    ref = a.astype(np.int64) @ b.astype(np.int64).T
    assert np.array_equal(oracle.gemm_i32(a, b).astype(np.int64), ref)


def test_dense_scales_against_fp64():
    rng = np.random.default_rng(5)
    M, N, K = 9, 31, 300
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.001, 0.1, M).astype(np.float32)
    sb = rng.uniform(0.001, 0.01, N).astype(np.float32)
    out = oracle.dense_w8a8(a, sa, b, sb)
    ref = (a.astype(np.int64) @ b.astype(np.int64).T).astype(np.float64) * sa[:, None] * sb[None, :]
    # two fp32 roundings of an exact product, plus the int->float rounding
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 3 * 2.0 ** -24)


# ---------------------------------------------------------------- router
def test_router_hand_and_library():
    x = np.array([[1.0, 2.0]], np.float32)
    wr = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]], np.float32)
    b = np.array([0.5, 0.0, -1.0], np.float32)
    assert oracle.router_logits(x, wr, b).tolist() == [[1.5, 2.0, 2.0]]
    rng = np.random.default_rng(3)
    x = rng.standard_normal((11, 257)).astype(np.float32)
    wr = (rng.standard_normal((6, 257)) * 0.02).astype(np.float32)
    b = rng.standard_normal(6).astype(np.float32)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T + b
    got = oracle.router_logits(x, wr, b)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.router_logits(x, wr, None), ref - b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- top-k
@pytest.mark.parametrize("case", _gold("topk_pins.json")["cases"])
def test_topk_hand_worked(case):
    ids, w = oracle.topk_softmax(np.array([case["logits"]], np.float64), case["k"])
    assert ids[0].tolist() == case["ids"]
    assert np.allclose(w[0], np.array(case["w"], np.float32), rtol=0, atol=1e-7)


def test_topk_closed_forms_and_invariants():
    rng = np.random.default_rng(4)
    T, E = 200, 16
    l = rng.standard_normal((T, E)) * 3
    # k = E: the full softmax, in descending order
    ids, w = oracle.topk_softmax(l, E)
    sm = np.exp(l - l.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    assert np.array_equal(ids, np.argsort(-l, axis=1, kind="stable"))
    assert np.allclose(w, np.take_along_axis(sm, ids, 1), rtol=1e-6, atol=1e-7)
    # k = 2: w0 = sigmoid(l0 - l1)
    ids, w = oracle.topk_softmax(l, 2)
    top = np.take_along_axis(l, ids, 1)
    assert np.allclose(w[:, 0], 1 / (1 + np.exp(-(top[:, 0] - top[:, 1]))), rtol=1e-6)
    # k = 5: sum to one, descending, and the picked set is the top-5 by logit
    ids, w = oracle.topk_softmax(l, 5)
    assert np.allclose(w.sum(1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.array_equal(ids, np.argsort(-l, axis=1, kind="stable")[:, :5])
    # shifting all logits of a token changes nothing
    ids2, w2 = oracle.topk_softmax(l + 123.0, 5)
    assert np.array_equal(ids, ids2) and np.allclose(w, w2, atol=1e-7)


# ---------------------------------------------------------------- permute
def test_permute_against_stable_sort():
    rng = np.random.default_rng(6)
    T, E, k = 300, 12, 3
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    counts, offsets, sa = oracle.permute(ids, E)
    assert np.array_equal(counts, np.bincount(ids.reshape(-1), minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(sa, np.argsort(ids.reshape(-1), kind="stable"))
    for e in range(E):
        seg = sa[offsets[e]:offsets[e + 1]]
        assert np.all(ids.reshape(-1)[seg] == e)
        assert np.all(np.diff(seg // k) > 0)  # ascending token order


def test_permute_empty_experts():
    ids = np.array([[3, 0], [3, 0], [0, 3]], np.int32)
    counts, offsets, sa = oracle.permute(ids, 6)
    assert counts.tolist() == [3, 0, 0, 3, 0, 0]
    assert offsets.tolist() == [0, 3, 3, 3, 6, 6, 6]
    assert sa.tolist() == [1, 3, 4, 0, 2, 5]


# ---------------------------------------------------------------- SiLU
def test_silu_values():
    assert oracle.silu(np.float32(0.0)) == 0.0
    assert oracle.silu(np.float32(1.0)) == np.float32(1.0 / (1.0 + math.exp(-1.0)))
    assert oracle.silu(np.float32(-1.0)) == np.float32(-1.0 / (1.0 + math.exp(1.0)))
    v = oracle.silu(np.float32(-100.0))
    assert v == 0.0 and np.signbit(v)  # exp overflows to inf: -100/inf = -0, no NaN
    assert oracle.silu(np.float32(100.0)) == np.float32(100.0)
    g = np.linspace(-30, 30, 601).astype(np.float32)
    got = oracle.silu(g).astype(np.float64)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64)))
    # three fp32 roundings (exp, add, divide) of the exact value
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 4 * 2.0 ** -24 + 1e-45)


# ---------------------------------------------------------------- expert FFN
def _small_layer(T=12, H=64, E=4, k=2, I=32, seed=7, zero_bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, 3] *= 20
    wr = (rng.standard_normal((E, H)) * 0.05).astype(np.float32)
    b = np.zeros(E, np.float32) if zero_bias else rng.standard_normal(E).astype(np.float32)
    w_gu = rng.integers(-127, 128, size=(E, 2 * I, H)).astype(np.int8)
    w_d = rng.integers(-127, 128, size=(E, H, I)).astype(np.int8)
    s_gu = rng.uniform(1e-4, 1e-3, (E, 2 * I)).astype(np.float32)
    s_d = rng.uniform(1e-4, 1e-3, (E, H)).astype(np.float32)
    return x, wr, b, w_gu, s_gu, w_d, s_d


def _ffn_fp64(xq_row, sx, e, wt, w_gu, s_gu, w_d, s_d, I, h_q=None, s_h=None):
    """fp64 evaluation of one assignment from library matmuls."""
    acc = w_gu[e].astype(np.int64) @ xq_row.astype(np.int64)
    g = acc[:I] * float(sx) * s_gu[e, :I].astype(np.float64)
    u = acc[I:] * float(sx) * s_gu[e, I:].astype(np.float64)
    h = g / (1 + np.exp(-g)) * u
    out = dict(acc=acc, h=h)
    if h_q is not None:
        accd = w_d[e].astype(np.int64) @ h_q.astype(np.int64)
        out["accd"] = accd
        out["o"] = wt * accd * float(s_h) * s_d[e].astype(np.float64)
    return out


def test_expert_ffn_against_library_matmul_fp64():
    x, wr, b, w_gu, s_gu, w_d, s_d = _small_layer()
    k, I = 2, 32
    r = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, k, want_acc=True, want_h=True)
    for a in range(x.shape[0] * k):
        t, j = divmod(a, k)
        e = int(r["ids"][t, j])
        ref = _ffn_fp64(r["x_q"][t], r["s_x"][t], e, float(r["w"][t, j]), w_gu, s_gu, w_d, s_d, I,
                        r["h_q"][a], r["s_h"][a])
        assert np.array_equal(r["acc_gu"][a].astype(np.int64), ref["acc"])
        hmax = np.abs(ref["h"]).max()
        assert np.all(np.abs(r["h"][a] - ref["h"]) <= 1e-5 * hmax)
        assert np.array_equal(r["acc_d"][a].astype(np.int64), ref["accd"])
        assert np.allclose(r["o"][a], ref["o"], rtol=1e-5, atol=1e-6 * np.abs(ref["o"]).max())
        # requantised codes: the rounding of h/s_h, within one code where fp32 noise
        # could move a value across a half-integer
        v = ref["h"] / (np.abs(ref["h"]).max() / 127)
        assert np.all(np.abs(r["h_q"][a].astype(np.int64) - np.rint(v)) <= 1)
        clear = np.abs(np.abs(v - np.floor(v)) - 0.5) > 1e-3
        assert np.array_equal(r["h_q"][a][clear].astype(np.int64), np.rint(v[clear]).astype(np.int64))


def test_gate_and_up_not_exchanged():
    # all gate rows large positive and all up rows +1: h = SiLU(g)*u > 0, with g = up-weighted
    # only through the gate half.  Exchanging the halves gives a different sign pattern.
    T, H, E, k, I = 2, 64, 1, 1, 16
    x = np.ones((T, H), np.float32)
    x[1] = -1.0
    wr = np.zeros((E, H), np.float32)
    w_gu = np.zeros((E, 2 * I, H), np.int8)
    w_gu[0, :I, :] = 1    # gate: g = +H*s for token 0, -H*s for token 1
    w_gu[0, I:, :] = 2    # up:   u = 2x gate
    w_d = np.ones((E, H, I), np.int8)
    s_gu = np.full((E, 2 * I), 1.0 / 64, np.float32)
    s_d = np.ones((E, H), np.float32)
    r = oracle.moe_forward(x, wr, None, w_gu, s_gu, w_d, s_d, k, want_h=True)
    # token 0: g = 1*1*... x_q = 127, s_x = 1/127, acc_g = 127*64, g = 64*(1/127*127)/64 = 1
    g0 = np.float32(1.0)
    u0 = np.float32(2.0)
    assert np.allclose(r["h"][0], oracle.silu(g0) * u0, rtol=1e-6)
    # token 1: g = -1, u = -2  -> h = SiLU(-1) * -2 > 0 (exchanging would give SiLU(-2)*-1)
    assert np.allclose(r["h"][1], oracle.silu(np.float32(-1.0)) * np.float32(-2.0), rtol=1e-6)


# ---------------------------------------------------------------- whole layer
def test_zero_input_zero_output():
    x, wr, b, w_gu, s_gu, w_d, s_d = _small_layer()
    x[:] = 0
    r = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, 2)
    assert np.all(r["s_x"] == 0) and np.all(r["x_q"] == 0)
    assert np.all(r["y"] == 0)


def test_token_permutation_equivariance_and_batch_invariance():
    x, wr, b, w_gu, s_gu, w_d, s_d = _small_layer(T=20)
    full = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, 2)
    perm = np.random.default_rng(9).permutation(20)
    p = oracle.moe_forward(x[perm], wr, b, w_gu, s_gu, w_d, s_d, 2)
    assert np.array_equal(p["y"], full["y"][perm])
    sub = [2, 5, 11, 19]
    alone = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, 2, route_tokens=sub)
    assert np.array_equal(alone["y"], full["y"][sub])
    part = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, 2, tokens=sub)
    assert np.array_equal(part["y"], full["y"][sub])


def test_single_expert_reduces_to_dense_swiglu_ffn():
    T, H, I = 6, 64, 32
    x, wr, b, w_gu, s_gu, w_d, s_d = _small_layer(T=T, H=H, E=1, I=I)
    r = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, 1, want_h=True)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)
    # dense path from the oracle's own single-step routines (quant + dense GEMM) and numpy
    xq, sx = oracle.quantize_rows(x)
    gate = oracle.dense_w8a8(xq, sx, w_gu[0][:I], s_gu[0, :I])
    up = oracle.dense_w8a8(xq, sx, w_gu[0][I:], s_gu[0, I:])
    h = oracle.silu(gate) * up
    assert np.array_equal(h, r["h"])
    hq, sh = oracle.quantize_rows(h)
    y = oracle.dense_w8a8(hq, sh, w_d[0], s_d[0])
    assert np.array_equal(y, r["y"])


def test_all_experts_reduces_to_softmax_mixture():
    T, H, E, I = 5, 64, 4, 32
    x, wr, b, w_gu, s_gu, w_d, s_d = _small_layer(T=T, H=H, E=E, I=I, zero_bias=False)
    r = oracle.moe_forward(x, wr, b, w_gu, s_gu, w_d, s_d, E)
    l = x.astype(np.float64) @ wr.astype(np.float64).T + b
    p = np.exp(l - l.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    for t in range(T):
        y = np.zeros(H)
        for e in range(E):
            a = t * E + list(r["ids"][t]).index(e)
            f = _ffn_fp64(r["x_q"][t], r["s_x"][t], e, p[t, e], w_gu, s_gu, w_d, s_d, I,
                          r["h_q"][a], r["s_h"][a])
            y += f["o"]
        assert np.allclose(r["y"][t], y, rtol=1e-5, atol=1e-5 * np.abs(y).max())


def test_combine_order_and_k1():
    rng = np.random.default_rng(8)
    o = rng.standard_normal((4 * 3, 10)).astype(np.float32)
    y = oracle.combine(o, 4, 3)
    ref = (o[0::3].astype(np.float32) + o[1::3]) + o[2::3]
    assert np.array_equal(y, ref)
    assert np.array_equal(oracle.combine(o, 12, 1), o)


# ---------------------------------------------------------------- FP8 E4M3 codes
def test_e4m3_hand_worked():
    g = _gold("fp8_pins.json")
    for c in g["encode"]:
        assert int(oracle.e4m3_encode(np.float32(c["v"]))) == c["code"], c
    for c in g["quant"]:
        q, s = oracle.quantize_rows_fp8(np.array(c["x"], np.float32))
        assert s[0] == np.float32(c["s"]), c
        assert q[0].tolist() == c["q"], c
    d = g["dense"]
    a = oracle.e4m3_encode(np.array(d["a"], np.float32))
    b = oracle.e4m3_encode(np.array(d["b"], np.float32))
    out = oracle.dense_fp8(a, np.array(d["s_a"], np.float32), b, np.array(d["s_b"], np.float32))
    assert out.tolist() == d["out"]


def test_e4m3_format_closed_forms():
    codes = np.arange(256, dtype=np.uint8)
    v = oracle.e4m3_decode(codes)
    finite = ~np.isnan(v)
    # exactly two NaN codes (S.1111.111), no infinities, largest finite 448
    assert np.count_nonzero(~finite) == 2 and not np.isinf(v[finite]).any()
    assert np.nanmax(v) == 448.0 and np.nanmin(v) == -448.0
    # codes 0x00..0x7E increase strictly; the negative half mirrors them
    assert np.all(np.diff(v[:127]) > 0)
    assert np.array_equal(v[128:255], -v[:127])
    # the value formula: subnormals m*2^-9, normals (1 + m/8) * 2^(e-7)
    for c in range(127):
        e, m = c >> 3, c & 7
        ref = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
        assert v[c] == ref
    # round trip of every finite code (negative zero included)
    back = oracle.e4m3_encode(v[finite].astype(np.float32))
    assert np.array_equal(back, codes[finite])


def test_e4m3_encoder_is_nearest_ties_even_by_brute_force():
    rng = np.random.default_rng(5)
    vals = oracle.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = 0.5 * (vals[:-1] + vals[1:])
    x = np.concatenate([rng.standard_normal(3000) * 40, rng.standard_normal(500) * 0.01,
                        mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1e9))]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    mag = np.abs(x.astype(np.float64))
    for xi, gi, ai in zip(x, got, mag):
        d = np.abs(vals - min(ai, 448.0))
        best = np.flatnonzero(d == d.min())
        want = best[0] if best.size == 1 else best[best % 2 == 0][0]  # tie: even mantissa
        assert (gi & 0x7F) == want, (xi, gi, want)
        assert (gi >> 7) == (1 if np.signbit(xi) else 0)


def test_fp8_quant_invariants():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((23, 301)).astype(np.float32)
    x[:, 7] *= 50.0
    q, s = oracle.quantize_rows_fp8(x)
    v = oracle.e4m3_decode(q)
    # the row maximum maps to +-448 and nothing exceeds it
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(v[np.arange(23), am]) == 448.0)
    assert np.abs(v).max() <= 448.0
    # sign symmetry and power-of-two scaling invariance
    qn, sn = oracle.quantize_rows_fp8(-x)
    assert np.array_equal(qn, q ^ 0x80) and np.array_equal(sn, s)
    qp, sp = oracle.quantize_rows_fp8(x * np.float32(2.0 ** 9))
    assert np.array_equal(qp, q) and np.array_equal(sp, s * np.float32(2.0 ** 9))
    # relative error of round-to-nearest with 3 mantissa bits: |x - v*s| <= 2^-4 |x| for normals
    xs = x.astype(np.float64) / s[:, None]
    norm = np.abs(xs) >= 2.0 ** -6
    err = np.abs(xs - v)
    assert np.all(err[norm] <= np.abs(xs[norm]) * 2.0 ** -4 * (1 + 1e-6))
    assert np.all(err[~norm] <= 2.0 ** -10 * (1 + 1e-6))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (17, 9, 130), (8, 33, 512)])
def test_fp8_gemm_exact_against_numpy(M, N, K):
    rng = np.random.default_rng(M * 100 + N)
    a = rng.integers(0, 256, (M, K), dtype=np.uint8)
    b = rng.integers(0, 256, (N, K), dtype=np.uint8)
    a[(a & 0x7F) == 0x7F] = 0x7E  # no NaN codes
    b[(b & 0x7F) == 0x7F] = 0x7E
    acc = oracle.gemm_fp8(a, b)
    ref = oracle.e4m3_decode(a) @ oracle.e4m3_decode(b).T  # exact: the sum needs < 53 bits
    assert np.array_equal(acc, ref)
    out = oracle.dense_fp8(a, np.full(M, 0.5, np.float32), b, np.full(N, 4.0, np.float32))
    assert np.array_equal(out, (ref.astype(np.float32) * np.float32(0.5)) * np.float32(4.0))


def test_fp8_single_expert_reduces_to_dense_chain():
    """E = 1, k = 1: the FP8 expert FFN equals two dense FP8 GEMMs around the
    SwiGLU and the E4M3 requantisation, written out here step by step."""
    rng = np.random.default_rng(8)
    T, H, I = 5, 64, 32
    x = rng.standard_normal((T, H)).astype(np.float32)
    wgu = (rng.standard_normal((1, 2 * I, H)) * 0.05).astype(np.float32)
    wd = (rng.standard_normal((1, H, I)) * 0.05).astype(np.float32)
    qgu, sgu = oracle.quantize_rows_fp8(wgu[0])
    qd, sd = oracle.quantize_rows_fp8(wd[0])
    xq, sx = oracle.quantize_rows_fp8(x)
    gu = oracle.dense_fp8(xq, sx, qgu, sgu)
    h = oracle.silu(gu[:, :I]) * gu[:, I:]
    hq, sh = oracle.quantize_rows_fp8(h)
    o = oracle.dense_fp8(hq, sh, qd, sd)
    r = oracle.moe_forward(x, np.zeros((1, H), np.float32), None, qgu[None], sgu[None], qd[None],
                           sd[None], 1, code="fp8", want_h=True)
    assert np.array_equal(r["x_q"], xq) and np.array_equal(r["h"], h)
    assert np.array_equal(r["h_q"], hq) and np.array_equal(r["s_h"], sh)
    assert np.array_equal(r["y"], o)


# ------------------------------------------- smoothing vector and static/clipped scales
def _scale_of(expr):
    num, _, den = expr.partition("/")
    return np.float32(num) / np.float32(den) if den else np.float32(num)


def test_scale_options_hand_worked():
    g = _gold("scale_options_pins.json")
    for c in g["cases"]:
        m = None if c["m"] is None else np.array(c["m"], np.float32)
        q, s = oracle.quantize_rows_ex(np.array(c["x"], np.float32), m, c["mode"], c["clip"], c["code"])
        assert s[0] == _scale_of(c["s"]), c
        assert q[0].tolist() == c["q"], c


@pytest.mark.parametrize("code", ["int8", "fp8"])
def test_scale_options_reduce_to_plain_quantisation(code):
    """m = 1 with the dynamic scale, a clip at or above every row maximum, and a
    static scale equal to a single row's maximum all give plain absmax codes."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((9, 300)) * np.exp(rng.standard_normal((9, 1)))).astype(np.float32)
    plain = oracle.quantize_rows if code == "int8" else oracle.quantize_rows_fp8
    q0, s0 = plain(x)
    for kw in (dict(col_mul=np.ones(300, np.float32)),
               dict(mode="clipped", clip=float(np.abs(x).max())),
               dict(mode="clipped", clip=1e30)):
        q, s = oracle.quantize_rows_ex(x, code=code, **kw)
        assert np.array_equal(q, q0) and np.array_equal(s, s0), kw
    amax = np.abs(x[3]).max()
    q, s = oracle.quantize_rows_ex(x[3:4], mode="static", clip=float(amax), code=code)
    assert np.array_equal(q[0], q0[3]) and s[0] == s0[3]


def test_smoothing_is_a_per_column_factor():
    """Smoothing by m equals plain quantisation of x * m (the product taken in
    fp32); a power-of-two factor on one column moves only that column's values
    (exactly) until it takes over the row maximum."""
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    m = np.exp2(rng.integers(-3, 4, 64)).astype(np.float32)
    q, s = oracle.quantize_rows_ex(x, m)
    q0, s0 = oracle.quantize_rows(x * m)
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    # a column's factor that is the row's own maximum ratio: that column becomes +-127
    r = 2
    c = int(np.argmin(np.abs(x[r])))
    m2 = np.ones(64, np.float32)
    m2[c] = np.float32(np.abs(x[r]).max() / abs(x[r, c])) * np.float32(4.0)
    q2, _ = oracle.quantize_rows_ex(x[r:r + 1], m2)
    assert abs(int(q2[0, c])) == 127


def test_clipped_codes_saturate():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((6, 256)) * 10).astype(np.float32)
    clip = 5.0
    q, s = oracle.quantize_rows_ex(x, mode="clipped", clip=clip)
    assert np.all(s == np.float32(clip) / np.float32(127))
    assert np.all(q[x >= clip] == 127) and np.all(q[x <= -clip * 128 / 127] == -128)
    qf, sf = oracle.quantize_rows_ex(x, mode="clipped", clip=clip, code="fp8")
    big = np.abs(x) >= clip
    assert np.all((qf[big] & 0x7F) == 0x7E)  # saturated at 448
    assert np.all((qf[big] >> 7) == (x[big] < 0))


def test_moe_smoothing_equivalence_in_real_arithmetic():
    """SmoothQuant leaves the product unchanged: with activations on the int8
    grid (scale 1), a factor m = 1/2 on every column but the first, and the
    weights' input channels carrying 1/m = 2, the gate-up accumulators equal
    the unsmoothed ones exactly, so the whole layer's output is identical."""
    rng = np.random.default_rng(10)
    T, H, E, k, I = 6, 128, 4, 2, 128
    x = (2 * rng.integers(-63, 64, (T, H))).astype(np.float32)
    x[:, 0] = 127.0  # each row's maximum: scale 1, x is its own code (also after smoothing)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    w_gu = rng.integers(-63, 64, (E, 2 * I, H)).astype(np.int8)
    w_d = rng.integers(-127, 128, (E, H, I)).astype(np.int8)
    s_gu = np.full((E, 2 * I), 1e-4, np.float32)
    s_d = np.full((E, H), 1e-3, np.float32)
    m = np.full(H, 0.5, np.float32)
    m[0] = 1.0
    w_gu_s = w_gu.copy()
    w_gu_s[:, :, 1:] *= 2
    ref = oracle.moe_forward(x, wr, None, w_gu, s_gu, w_d, s_d, k, want_acc=True)
    sm = oracle.moe_forward(x, wr, None, w_gu_s, s_gu, w_d, s_d, k, x_smooth=m, want_acc=True)
    assert np.array_equal(sm["x_q"][:, 1:], ref["x_q"][:, 1:] // 2)
    assert np.array_equal(sm["ids"], ref["ids"])  # the router reads the unsmoothed x
    assert np.array_equal(sm["acc_gu"], ref["acc_gu"])
    assert np.array_equal(sm["y"], ref["y"])
