"""GPU parity: every kernel of the HIP path against the CPU oracle, through the
C ABI (via the thin Python binding), on seeded synthetic inputs.

Bars: int8 codes, int32 accumulators, indices and permutations bit-exact;
top-k ids bit-exact except flagged near ties (see _parity); fp32 outputs
within max relative error 1e-3 (they are in fact expected to agree exactly or
to a few ulp, since both sides apply the same fp32 operations in the same
association).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
from _parity import (Y_TOL, near_tie_tokens, rel_metric, stable_sort_assign, sum_rel_metric, to_np,
                     valid_topk)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w8a8_quantized_moe_amd as w8
    return w8


def _say(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ quantisation
QUANT_SHAPES = [(1, 4, 4), (3, 130, 130), (37, 128, 128), (1000, 4096, 4096), (64, 7168, 7168),
                (5, 8192, 8192), (7, 10000, 10000), (2, 1, 1), (9, 256, 300), (4, 2048, 2051),
                # one wave per row up to 2048 columns (eight float4 per lane)
                (9, 1028, 1028), (70, 1536, 1536), (33, 2048, 2048), (6, 2052, 2052)]


@pytest.mark.parametrize("rows,cols,ld", QUANT_SHAPES)
def test_quantize_rows_bitexact(w8, rows, cols, ld):
    _say(f"quantize rows={rows} cols={cols} ld={ld}")
    rng = np.random.default_rng(rows * 7 + cols)
    full = rng.standard_normal((rows, ld)).astype(np.float32)
    full[:, rng.integers(0, cols, size=max(1, cols // 100))] *= 30
    if rows > 2:
        full[1, :] = 0.0          # all-zero row
        full[2, :cols] = 0.5      # all equal
    x = torch.from_numpy(full).cuda()
    q, s = w8.quantize_rows(x[:, :cols])
    torch.cuda.synchronize()
    qo, so = oracle.quantize_rows(full[:, :cols])
    assert np.array_equal(to_np(s), so)
    assert np.array_equal(to_np(q), qo)


def test_quantize_hand_worked(w8):
    import json
    with open(os.path.join(os.path.dirname(__file__), "golden", "quant_pins.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = torch.tensor([c["x"]], dtype=torch.float32, device="cuda")
        q, s = w8.quantize_rows(x)
        assert to_np(s)[0] == np.float32(c["s"])
        assert to_np(q)[0].tolist() == c["q"]


# ------------------------------------------------------------------ dense GEMM
GEMM_SHAPES = [(1, 128, 128), (5, 256, 384), (128, 128, 128), (300, 384, 256), (129, 128, 1024),
               (513, 640, 2048),
               # 256-wide tiles: a 100-row half tile (all waves on 128 rows, deeper
               # ring), a second m-tile of exactly 128 rows, a 200-row partial tile,
               # and a half tile with a two-stage K loop
               (100, 512, 640), (384, 256, 256), (200, 256, 256), (60, 256, 128),
               # partial tiles of 129-255 rows split evenly over the two rows of
               # waves: 5, 6, 7 and 8 fragment rows each (odd counts put an
               # epilogue pass across the split), and a lower row of waves with
               # one fragment row fewer than the upper (170 rows: 96 + 74)
               (385, 256, 256), (406, 256, 384), (417, 512, 256), (449, 256, 256),
               (481, 256, 128), (511, 256, 256), (170, 256, 256),
               # last tiles of at most 64 rows copy only their 1, 2 or 4 activation
               # blocks into a deeper ring: 16 rows over a long K, 17 and 32
               # rows, 33 and 64 rows, the 128-wide tile's ring, and a second
               # m-tile of 40 rows
               (16, 256, 4096), (17, 256, 512), (32, 128, 2048), (33, 512, 256), (64, 256, 1024),
               (296, 256, 640)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_i32_exact(w8, M, N, K):
    _say(f"gemm_i32 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    a = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    a[:, 0] = -128
    b[:, 0] = -128
    bp = w8.pack_weights(torch.from_numpy(b).cuda())
    acc = w8.gemm_i32(torch.from_numpy(a).cuda(), bp, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(acc), oracle.gemm_i32(a, b))


@pytest.mark.parametrize("M,N,K", [(77, 256, 512), (130, 128, 8192), (193, 256, 512), (405, 512, 256),
                                   (40, 256, 1024), (9, 128, 512)])
def test_gemm_f32_exact(w8, M, N, K):
    _say(f"gemm_f32 M={M} N={N} K={K}")
    rng = np.random.default_rng(M * N)
    a = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    b = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sa = rng.uniform(1e-3, 1e-1, M).astype(np.float32)
    sb = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    bp = w8.pack_weights(torch.from_numpy(b).cuda())
    out = w8.gemm(torch.from_numpy(a).cuda(), torch.from_numpy(sa).cuda(), bp,
                  torch.from_numpy(sb).cuda(), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), oracle.dense_w8a8(a, sa, b, sb))


def test_dense_workload_sampled(w8):
    """The dense W8A8 workload at full size (M=4096, K=8192, N=8192): per-token
    quantisation exact on all rows; the GEMM output exact on sampled rows."""
    _say("dense workload 4096x8192x8192")
    inp = synth.dense_inputs(device="cuda")
    M, K, N = inp["M"], inp["K"], inp["N"]
    a_q, s_a = w8.quantize_rows(inp["a"])
    bp = w8.pack_weights(inp["b"])
    out = w8.gemm(a_q, s_a, bp, inp["s_b"], N, K)
    torch.cuda.synchronize()
    a_h = to_np(inp["a"])
    qo, so = oracle.quantize_rows(a_h)
    assert np.array_equal(to_np(a_q), qo) and np.array_equal(to_np(s_a), so)
    rows = np.unique(np.concatenate([np.random.default_rng(0).choice(M, 40, replace=False),
                                     [0, 127, 128, M - 1]]))
    ref = oracle.dense_w8a8(qo[rows], so[rows], to_np(inp["b"]), to_np(inp["s_b"]))
    assert np.array_equal(to_np(out)[rows], ref)


# ------------------------------------------------------------------ MoE layer
MODES = {"dynamic": 0, "clipped": 1, "static": 2}


def _qkw(w8, qopts):
    """Layer options of the x quantisation for the binding (qopts: oracle names)."""
    if not qopts:
        return {}
    sm = qopts.get("x_smooth")
    return dict(x_smooth=None if sm is None else torch.from_numpy(sm).cuda(),
                x_scale_mode=MODES[qopts.get("x_scale_mode", "dynamic")],
                x_clip=qopts.get("x_clip", 0.0))


def _weights(w8, inp, qopts=None):
    if "w_gu_f32" in inp:
        wts, codes = w8.MoEWeights.from_fp32(inp["wr"], inp["b"], inp["w_gu_f32"], inp["w_d_f32"],
                                             keep_codes=True, **_qkw(w8, qopts))
        return wts, codes
    codes = dict(w_gu=inp["w_gu"], s_gu=inp["s_gu"], w_d=inp["w_d"], s_d=inp["s_d"])
    return w8.MoEWeights.from_int8(inp["wr"], inp["b"], inp["w_gu"], inp["s_gu"], inp["w_d"],
                                   inp["s_d"], **_qkw(w8, qopts)), codes


def _gpu_moe(w8, inp, wts):
    """The layer on the GPU: every intermediate, and (INT8 codes) a function
    returning the gate-up GEMM's raw accumulators of given expert-sorted rows."""
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws = torch.empty((max(lay["total_bytes"], 256),), dtype=torch.uint8, device="cuda")
    y = w8.moe_forward(inp["x"], wts, k, workspace=ws)
    torch.cuda.synchronize()
    g = {n: to_np(v) for n, v in w8.workspace_views(ws, T, H, E, k, I).items()}
    g["y"] = to_np(y)
    if wts.code == w8.CODE_INT8:
        acc = w8.moe_gate_up_acc(T, wts, k, ws)
        torch.cuda.synchronize()
        g["acc_gu_rows"] = lambda rows: to_np(acc[torch.as_tensor(rows, dtype=torch.long, device="cuda")])
    return g


def _oracle_codes(inp, codes, qopts=None):
    """The oracle's own int8 weights: for fp32 weights it quantises them itself
    (and the test checks the GPU's offline quantisation against that; with a
    smoothing vector m the gate-up weights take 1/m on their input channels)."""
    if "w_gu_f32" in inp:
        E, twoI, H = inp["w_gu_f32"].shape
        I = twoI // 2
        sm = (qopts or {}).get("x_smooth")
        if sm is None:
            qg, sg = oracle.quantize_rows(to_np(inp["w_gu_f32"]).reshape(E * twoI, H))
        else:
            qg, sg = oracle.quantize_rows_ex(to_np(inp["w_gu_f32"]).reshape(E * twoI, H),
                                             col_mul=np.float32(1.0) / sm)
        qd, sd = oracle.quantize_rows(to_np(inp["w_d_f32"]).reshape(E * H, I))
        ora = dict(w_gu=qg.reshape(E, twoI, H), s_gu=sg.reshape(E, twoI),
                   w_d=qd.reshape(E, H, I), s_d=sd.reshape(E, H))
        for n in ora:
            assert np.array_equal(to_np(codes[n]), ora[n]), f"offline weight quantisation: {n}"
        return ora
    return {n: to_np(v) for n, v in codes.items()}


def check_moe(w8, inp, tokens=None, report=None, qopts=None, run=None):
    """The layer on the GPU against the oracle.  run(w8, inp, wts, codes)
    replaces the multi-launch layer (_gpu_moe) with another entry point."""
    T, H, E, k, I = inp["T"], inp["H"], inp["E"], inp["k"], inp["I"]
    _say(f"moe T={T} H={H} E={E} k={k} I={I} tokens={'all' if tokens is None else len(tokens)}"
         f"{'' if not qopts else ' x options ' + str(sorted(qopts))}")
    wts, codes = _weights(w8, inp, qopts)
    g = run(w8, inp, wts, codes) if run is not None else _gpu_moe(w8, inp, wts)
    oc = _oracle_codes(inp, codes, qopts)
    x = to_np(inp["x"])
    b = to_np(inp["b"])
    o = oracle.moe_forward(x, to_np(inp["wr"]), b, oc["w_gu"], oc["s_gu"], oc["w_d"], oc["s_d"], k,
                           tokens=tokens, want_h=True, want_acc=True, **(qopts or {}))
    tok = o["tokens"]

    # 1. per-token quantisation: exact
    assert np.array_equal(g["x_q"], o["x_q"]) and np.array_equal(g["x_scale"], o["s_x"])
    # 2. router logits: fp32 on GPU vs fp64 oracle
    cond = np.abs(x).astype(np.float64) @ np.abs(to_np(inp["wr"])).astype(np.float64).T
    dl = np.abs(g["logits"].astype(np.float64) - o["logits"])
    assert np.all(dl <= 1e-6 + 2.0 ** -24 * 8 * np.sqrt(H) * cond), float(dl.max())
    # 3. top-k: GPU ids a valid top-k of the GPU's own logits; exact vs oracle except near ties
    assert valid_topk(g["logits"], g["topk_ids"]).all()
    flag = near_tie_tokens(o["logits"], g["logits"], k)
    same = np.all(g["topk_ids"] == o["ids"], axis=1)
    assert np.all(same | flag), f"top-k mismatch on unflagged tokens {np.where(~(same | flag))[0][:10]}"
    diff_tokens = np.where(~same)[0]
    # weights: a logit error d moves exp(l_j - l_0) by a relative 2d and the
    # renormalising sum by at most d more; allow 4d plus fp32 rounding
    delta = dl.max(axis=1)
    w_rel = np.abs(g["topk_w"] - o["w"]) / np.abs(o["w"])
    w_tol = 4.0 * delta[:, None] + 2e-6
    assert np.all((w_rel <= w_tol)[same]), float((w_rel / w_tol)[same].max())
    assert np.allclose(g["topk_w"].sum(1), 1.0, atol=1e-5)
    # 4. permutation: a stable sort of the GPU's own ids; equal to the oracle's without ties
    assert np.array_equal(g["sorted_assign"], stable_sort_assign(g["topk_ids"]))
    cnt = np.bincount(g["topk_ids"].reshape(-1), minlength=E)
    assert np.array_equal(g["expert_counts"], cnt)
    assert g["expert_offsets"][0] == 0 and np.array_equal(np.diff(g["expert_offsets"]), cnt)
    if diff_tokens.size == 0:
        assert np.array_equal(g["sorted_assign"], o["sorted_assign"])
        assert np.array_equal(g["expert_offsets"], o["offsets"])
    # 5-6. per assignment (keyed by a = t*k + j) on the checked tokens
    inv = np.empty(T * k, np.int64)
    inv[g["sorted_assign"]] = np.arange(T * k)
    a_rows = (tok[:, None] * k + np.arange(k)[None, :]).reshape(-1)
    ok_rows = np.repeat(same[tok], k)
    rows_g = inv[a_rows]
    # 5a. the gate-up GEMM's int32 accumulators: bit-exact on every row routed
    #     like the oracle's (same expert)
    acc_g = g["acc_gu_rows"](rows_g)
    assert np.array_equal(acc_g[ok_rows], o["acc_gu"][ok_rows]), \
        f"gate-up accumulators differ on {int((acc_g != o['acc_gu'])[ok_rows].any(axis=1).sum())} rows"
    h_g = g["h"][rows_g]
    hq_g = g["h_q"][rows_g]
    sh_g = g["h_scale"][rows_g]
    n_checked = int(ok_rows.sum())
    f32 = np.float32
    U = 2.0 ** -24
    ids_a = o["ids"][tok].reshape(-1)
    # 5b. h: both sides evaluate SiLU alike (the exponential correctly rounded
    #     to fp32 -- the kernels' exp_f32_rn equals (float)exp((double)x) on
    #     every fp32 input, checked exhaustively on the host -- then IEEE add,
    #     divide and product), so h is bit-exact on every row
    h_o = o["h"].astype(np.float64)
    h_exact = np.all(h_g == o["h"], axis=1) & ok_rows
    assert h_exact.sum() == n_checked, f"h mismatch on {n_checked - int(h_exact.sum())} of {n_checked} rows"
    hb = 6 * U * np.abs(h_o)
    assert np.all((np.abs(h_g.astype(np.float64) - h_o) <= hb)[ok_rows])
    # 6. h's scale and codes: exact on every row whose h is; elsewhere s_h moves
    #    by at most the row's largest h bound / 127 (plus the division's
    #    rounding) and a code may differ only where the oracle's quotient
    #    v = h / s_h lies within the bound on |v_gpu - v| of a rounding
    #    midpoint, by one step
    sh_o = o["s_h"].astype(np.float64)
    assert np.array_equal(sh_g[h_exact], o["s_h"][h_exact])
    assert np.array_equal(hq_g[h_exact], o["h_q"][h_exact])
    ds = hb.max(axis=1) / 127.0 + 2 * U * sh_o
    assert np.all((np.abs(sh_g - sh_o) <= ds)[ok_rows])
    pos = sh_o > 0
    safe = np.where(pos, sh_o, 1.0)[:, None]
    v_o = np.where(pos[:, None], h_o / safe, 0.0)
    dv = np.where(pos[:, None], (hb + np.abs(h_o) * (ds / safe[:, 0])[:, None]) / safe + 4 * U * np.abs(v_o), 0.0)
    frac = np.abs(v_o) - np.floor(np.abs(v_o))
    near = np.abs(frac - 0.5) <= dv
    dq = hq_g.astype(np.int32) - o["h_q"].astype(np.int32)
    assert ((dq == 0) | near)[ok_rows].all(), "h codes differ away from a rounding midpoint"
    assert np.abs(dq[ok_rows]).max(initial=0) <= 1
    n_moved = int((dq[ok_rows] != 0).sum())
    # 6a. the down GEMM, bit for bit on every checked row: its int32
    #     accumulators over the GPU's h codes are the oracle's plus the integer
    #     correction for the codes that moved, and o must be the epilogue
    #     w * (((float)acc * s_h) * s_d) in fp32 on them, with the GPU's own
    #     routing weight and row scale
    o_g = g["o"][a_rows]
    acc_d = o["acc_d"].astype(np.int64)
    for r in np.where(np.any(dq != 0, axis=1) & ok_rows)[0]:
        acc_d[r] += oc["w_d"][ids_a[r]].astype(np.int64) @ dq[r].astype(np.int64)
    assert np.all(np.abs(acc_d) < 2 ** 31)
    w_ga = g["topk_w"][tok].reshape(-1).astype(f32)
    o_acc = (acc_d.astype(np.int32).astype(f32) * sh_g.astype(f32)[:, None]) * oc["s_d"][ids_a].astype(f32)
    o_acc = w_ga[:, None] * o_acc.astype(f32)
    assert np.array_equal(o_g[ok_rows], o_acc[ok_rows]), \
        f"down epilogue differs on {int((o_g != o_acc)[ok_rows].any(axis=1).sum())} of {n_checked} rows"
    # o against the oracle's: where no code moved, the error is the routing
    # weight's (bounded above from the logit error) and the scale's, plus the
    # rounding of the product
    same_codes = ~np.any(dq != 0, axis=1) & ok_rows
    w_rel_a = w_rel[tok].reshape(-1)
    o_err = np.abs(o_g.astype(np.float64) - o["o"])
    o_tol = (w_rel_a[:, None] + (ds / np.where(pos, sh_o, 1.0))[:, None] + 2.0 ** -22) * np.abs(o["o"]).astype(np.float64)
    assert np.all((o_err <= o_tol)[same_codes]), float((o_err - o_tol)[same_codes].max())
    el, mx = rel_metric(o_g[same_codes], o["o"][same_codes]) if same_codes.any() else (0.0, 0.0)
    assert el <= Y_TOL and mx <= Y_TOL, (el, mx)
    # 7. output
    yt = same[tok]
    terms = np.abs(o["o"]).reshape(len(tok), k, H).sum(axis=1)
    sr, mx = sum_rel_metric(g["y"][tok][yt], o["y"][yt], terms[yt]) if yt.any() else (0.0, 0.0)
    assert sr <= Y_TOL and mx <= Y_TOL, (sr, mx)
    el, _ = rel_metric(g["y"][tok][yt], o["y"][yt]) if yt.any() else (0.0, 0.0)
    if report is not None:
        report.update(flagged=int(flag.sum()), differing_ids=int(diff_tokens.size),
                      h_rows_inexact=int(n_checked - h_exact.sum()), h_codes_moved=n_moved, y_sum_rel=sr, y_max=mx,
                      y_elem_rel=el, y_exact=bool(np.array_equal(g["y"][tok][yt], o["y"][yt])))
    return g, o


def test_moe_tiny_full(w8):
    inp = synth.moe_inputs("tiny", device="cuda")
    rep = {}
    check_moe(w8, inp, report=rep)
    _say(f"tiny report {rep}")


def test_moe_decode_full(w8):
    inp = synth.moe_inputs("decode", device="cuda")
    rep = {}
    check_moe(w8, inp, report=rep)
    _say(f"decode report {rep}")


def test_moe_prefill_sampled(w8):
    inp = synth.moe_inputs("prefill", device="cuda")
    T = inp["T"]
    tokens = np.unique(np.concatenate([np.random.default_rng(1).choice(T, 96, replace=False),
                                       [0, 63, 64, T - 1]]))
    rep = {}
    g, o = check_moe(w8, inp, tokens=tokens, report=rep)
    cnt = g["expert_counts"]
    _say(f"prefill report {rep}; top-12 share {synth.zipf_top12_share(cnt):.3f}; "
         f"experts<=3 tokens {(cnt <= 3).sum()}")


def test_moe_large_sampled(w8):
    inp = synth.moe_inputs("large", device="cuda")
    T = inp["T"]
    tokens = np.unique(np.concatenate([np.random.default_rng(2).choice(T, 24, replace=False),
                                       [0, T - 1]]))
    rep = {}
    check_moe(w8, inp, tokens=tokens, report=rep)
    _say(f"large report {rep}")


EDGE = [
    dict(T=1, H=128, E=8, k=2, I=128),
    dict(T=100, H=256, E=16, k=4, I=256),
    dict(T=70, H=128, E=1, k=1, I=128),
    dict(T=33, H=128, E=8, k=8, I=128),
    dict(T=40, H=128, E=256, k=8, I=128),
    dict(T=300, H=256, E=64, k=2, I=128, bias="zipf"),
    dict(T=129, H=384, E=5, k=3, I=384),
    dict(T=65, H=512, E=3, k=1, I=640, weights="fp32"),
    # few rows per expert (register-fed skinny kernel): skewed routing puts
    # several 16-row blocks on the hot experts; A = 4E exactly; K of 6 steps
    dict(T=120, H=256, E=64, k=2, I=256, bias="zipf"),
    dict(T=128, H=256, E=64, k=2, I=128, bias="zipf"),
    dict(T=20, H=384, E=8, k=1, I=384),
    # the largest hidden and intermediate sizes the ABI accepts: x (16384
    # columns) and h (16384 columns) take the two-pass quantiser, K = 16384
    dict(T=40, H=16384, E=8, k=2, I=128),
    dict(T=30, H=128, E=4, k=2, I=16384),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_moe_edge_cases(w8, case):
    over = dict(n_outlier=2, outlier_scale=20.0, bf16_x=False, bias="zero", weights="int8")
    over.update(case)
    inp = synth.moe_inputs("edge", device="cuda", **over)
    check_moe(w8, inp)


# From 2048 tokens the router weights are split into bf16 planes ahead of the
# router GEMM (expert tiles of 32, 64 or 128 by E); these cover each tile
# width, an expert count padded to a whole tile, a ragged last token tile and
# split sums along H.
ROUTER_PLANES = [
    dict(T=2048, H=256, E=256, k=8, I=128),
    # two expert tiles over 18 token tiles (not a multiple of the 8 XCDs the
    # token tiles are dealt to) with a ragged last tile
    dict(T=2230, H=256, E=256, k=4, I=128),
    dict(T=2100, H=512, E=24, k=2, I=128),
    dict(T=2049, H=1024, E=50, k=4, I=128),
    dict(T=4096, H=384, E=200, k=6, I=128),
    dict(T=2048, H=256, E=100, k=3, I=128, bias="zipf"),
]


@pytest.mark.parametrize("case", ROUTER_PLANES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_moe_router_planes(w8, case):
    over = dict(n_outlier=2, outlier_scale=20.0, bf16_x=False, bias="zero", weights="int8")
    over.update(case)
    inp = synth.moe_inputs("edge", device="cuda", **over)
    check_moe(w8, inp)


@pytest.mark.parametrize("T,E,k", [(9_000_000, 4, 1), (1 << 21, 8, 8)], ids=["T9M-top1", "A2^24-top8"])
def test_moe_max_token_count_sampled(w8, T, E, k):
    """Token counts at the ABI's limits: T = 9,000,000 with top-1 (more
    128-token router tiles than a grid dimension other than x can hold) and
    T*k = 2^24 assignments exactly (top-8 of 8 experts: segments of 2^21
    rows).  Row offsets run past 2^31 bytes.  The layer is token-independent,
    so sampled tokens (both sides of the 65535-tile boundary, the last token)
    are checked against the oracle run on those tokens alone: logits within
    the fp32 bound, ids exact away from near ties, y within the 1e-3 bar."""
    H, I = 128, 128
    _say(f"moe T={T} H={H} E={E} k={k} I={I} (sampled)")
    inp = synth.moe_inputs("edge", device="cuda", T=T, H=H, E=E, k=k, I=I, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="int8")
    wts, codes = _weights(w8, inp)
    lay = w8.moe_workspace_layout(T, H, E, k, I)
    ws = torch.empty((lay["total_bytes"],), dtype=torch.uint8, device="cuda")
    y = w8.moe_forward(inp["x"], wts, k, workspace=ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    edges = [0, T - 1] + ([65535 * 128 - 1, 65535 * 128] if T > 65535 * 128 else [])
    tok = np.unique(np.concatenate([rng.choice(T, 24, replace=False), edges]))
    idx = torch.from_numpy(tok).cuda()
    views = w8.workspace_views(ws, T, H, E, k, I)
    g_logits = to_np(views["logits"][idx])
    g_ids = to_np(views["topk_ids"][idx])
    g_y = to_np(y[idx])
    x_s = to_np(inp["x"][idx])
    wr = to_np(inp["wr"])
    oc = {n: to_np(v) for n, v in codes.items()}
    o = oracle.moe_forward(x_s, wr, to_np(inp["b"]), oc["w_gu"], oc["s_gu"], oc["w_d"], oc["s_d"], k)
    cond = np.abs(x_s).astype(np.float64) @ np.abs(wr).astype(np.float64).T
    dl = np.abs(g_logits.astype(np.float64) - o["logits"])
    assert np.all(dl <= 1e-6 + 2.0 ** -24 * 8 * np.sqrt(H) * cond), float(dl.max())
    flag = near_tie_tokens(o["logits"], g_logits, k)
    same = np.all(g_ids == o["ids"], axis=1)
    assert np.all(same | flag)
    terms = np.abs(o["o"]).reshape(len(tok), k, H).sum(axis=1)
    sr, mx = sum_rel_metric(g_y[same], o["y"][same], terms[same])
    assert sr <= Y_TOL and mx <= Y_TOL, (sr, mx)
    del ws, y, inp


def test_moe_router_wide_dynamic_range(w8):
    """Router operands whose values span 2^-20 .. 2^20: column h of x is scaled
    by 2^s_h and column h of the router matrix by 2^-s_h, so every product
    x*w (and the logits) keeps its size while each operand row crosses forty
    binades.  The bf16 three-term split of the router GEMM must still give
    logits within the fp32 error bound of the fp64 oracle, with exact routing
    away from near ties (all checked in check_moe)."""
    for T in (192, 2048):  # router weights split in the GEMM, then ahead of it
        _wide_range_case(w8, T)


def _wide_range_case(w8, T):
    inp = synth.moe_inputs("edge", device="cuda", T=T, H=512, E=40, k=4, I=128, n_outlier=2,
                           outlier_scale=20.0, bf16_x=False, bias="zero", weights="int8")
    g = torch.Generator(device="cuda").manual_seed(11)
    sh = torch.randint(-20, 21, (inp["H"],), generator=g, device="cuda").float()
    inp["x"] = (inp["x"] * torch.exp2(sh)[None, :]).contiguous()
    inp["wr"] = (inp["wr"] * torch.exp2(-sh)[None, :]).contiguous()
    check_moe(w8, inp)


@pytest.mark.parametrize("T,E,k", [(16, 8, 2), (300, 64, 4), (2100, 200, 8)])
def test_moe_exact_logit_ties_go_to_the_lower_expert(w8, T, E, k):
    """Zero router weights make every logit exactly its bias; a bias drawn
    from four values makes exact ties.  The top-k must order by descending
    logit with ties to the lower expert index (the oracle's reading), for the
    fused single-chunk routing (T = 16), the chunked one (T = 300) and the
    weight-plane router (T = 2100).  Tied tokens are excluded from the
    near-tie-tolerant checks elsewhere, so this pins the tie rule itself."""
    _say(f"exact logit ties: T={T} E={E} k={k}")
    inp = synth.moe_inputs("ties", device="cuda", T=T, H=256, E=E, k=k, I=128, n_outlier=0,
                           outlier_scale=1.0, bf16_x=False, bias="zero", weights="int8")
    inp["wr"].zero_()
    b = np.random.default_rng(7 + E).integers(0, 4, size=E).astype(np.float32)
    inp["b"] = torch.from_numpy(b).cuda()
    wts, codes = _weights(w8, inp)
    g = _gpu_moe(w8, inp, wts)
    assert np.array_equal(g["logits"], np.broadcast_to(b, (T, E)))
    want = np.argsort(-b, kind="stable")[:k]  # descending, ties to the lower index
    assert np.array_equal(g["topk_ids"], np.broadcast_to(want, (T, k)))
    o = oracle.moe_forward(to_np(inp["x"]), to_np(inp["wr"]), b, to_np(codes["w_gu"]), to_np(codes["s_gu"]),
                           to_np(codes["w_d"]), to_np(codes["s_d"]), k)
    assert np.array_equal(o["ids"], g["topk_ids"])
    assert np.abs(g["topk_w"].astype(np.float64) - o["w"]).max() <= 1e-6
    assert max(rel_metric(g["y"], o["y"])) <= Y_TOL


def test_moe_zero_input_gives_zero(w8):
    inp = synth.moe_inputs("edge0", device="cuda", T=50, H=256, E=8, k=2, I=256, n_outlier=0,
                           outlier_scale=1.0, bf16_x=False, bias="zero", weights="int8")
    inp["x"].zero_()
    wts, _ = _weights(w8, inp)
    g = _gpu_moe(w8, inp, wts)
    assert np.all(g["x_scale"] == 0) and np.all(g["x_q"] == 0)
    assert np.all(g["y"] == 0)


def test_moe_empty_batch_is_noop(w8):
    inp = synth.moe_inputs("edge1", device="cuda", T=4, H=128, E=4, k=2, I=128, n_outlier=0,
                           outlier_scale=1.0, bf16_x=False, bias="zero", weights="int8")
    wts, _ = _weights(w8, inp)
    x = torch.empty((0, 128), dtype=torch.float32, device="cuda")
    y = w8.moe_forward(x, wts, 2, workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (0, 128)


def test_moe_deterministic_and_token_independent(w8):
    inp = synth.moe_inputs("decode", device="cuda")
    wts, _ = _weights(w8, inp)
    a = _gpu_moe(w8, inp, wts)
    b = _gpu_moe(w8, inp, wts)
    for n in a:
        if not callable(a[n]):
            assert np.array_equal(a[n], b[n]), n
    assert np.array_equal(a["acc_gu_rows"](np.arange(128)), b["acc_gu_rows"](np.arange(128)))
    # permuting tokens permutes the outputs exactly (same token count, same kernels)
    perm = torch.randperm(inp["T"], generator=torch.Generator().manual_seed(3))
    inp2 = dict(inp)
    inp2["x"] = inp["x"][perm.cuda()].contiguous()
    c = _gpu_moe(w8, inp2, wts)
    assert np.array_equal(c["y"], a["y"][perm.numpy()])


def test_quantize_rows_half_integer_and_tiny_scales(w8):
    """Quotients at and next to half-integers (where a reciprocal-multiply
    shortcut could round differently) and rows of subnormal magnitude."""
    rng = np.random.default_rng(11)
    rows = []
    for amax in (127.0, 254.0, 1.0, 3.0e-38, 1.0e-41):
        s = np.float32(amax) / np.float32(127.0)
        k = rng.integers(-126, 126, size=2048).astype(np.float32)  # |k+0.5| < 127: amax stays
        v = (k + np.float32(0.5)) * s                      # near k + 0.5 after division
        v = np.nextafter(v, rng.choice([-np.inf, np.inf], size=v.shape).astype(np.float32))
        v[::3] = (k[::3] + np.float32(0.5)) * s
        v[0] = np.float32(amax)
        rows.append(v.astype(np.float32))
    x = np.stack(rows)
    for cols in (2048, 1024, 512):
        xs = np.ascontiguousarray(x[:, :cols])
        q, sc = w8.quantize_rows(torch.from_numpy(xs).cuda())
        torch.cuda.synchronize()
        qo, so = oracle.quantize_rows(xs)
        assert np.array_equal(to_np(sc), so)
        assert np.array_equal(to_np(q), qo)


# ------------------------------------------- activation-scale options (smoothing, clip, static)
QEX_SHAPES = [(5, 100), (33, 1024), (7, 1028), (5, 2048), (6, 4096), (3, 8192), (2, 10001), (4, 8200)]


@pytest.mark.parametrize("rows,cols", QEX_SHAPES)
@pytest.mark.parametrize("code", ["int8", "fp8"])
def test_quantize_rows_ex_bitexact(w8, rows, cols, code):
    """Smoothing factor, clipped and static scales: codes and scales equal the
    oracle's bit for bit on every kernel path (register-cached rows, one
    workgroup per row, and the general two-pass path)."""
    _say(f"quantize_rows_ex rows={rows} cols={cols} code={code}")
    rng = np.random.default_rng(rows * 31 + cols)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x[:, :: max(1, cols // 11)] *= 40.0
    m = (np.exp2(rng.integers(-3, 4, cols)) * rng.uniform(0.5, 2.0, cols)).astype(np.float32)
    amax = np.abs(x * m).max(axis=1)
    clip = float(np.median(amax)) * 0.7
    xd = torch.from_numpy(x).cuda()
    md = torch.from_numpy(m).cuda()
    c = w8.CODE_FP8 if code == "fp8" else w8.CODE_INT8
    for mode in ("dynamic", "clipped", "static"):
        for use_m in (False, True):
            q, s = w8.quantize_rows(xd, code=c, col_mul=md if use_m else None, scale_mode=MODES[mode],
                                    clip=clip)
            qo, so = oracle.quantize_rows_ex(x, m if use_m else None, mode, clip, code)
            assert np.array_equal(to_np(s), so), (mode, use_m)
            qg = to_np(q)
            assert np.array_equal(qg.view(qo.dtype), qo), (mode, use_m, int((qg.view(qo.dtype) != qo).sum()))
    # the inverse factor (a smoothed layer's weights): the library takes 1/m
    # itself; the oracle is handed the reciprocal as an IEEE fp32 division
    q, s = w8.quantize_rows(xd, code=c, col_mul=md, col_reciprocal=True)
    qo, so = oracle.quantize_rows_ex(x, np.float32(1.0) / m, "dynamic", 0.0, code)
    assert np.array_equal(to_np(s), so)
    assert np.array_equal(to_np(q).view(qo.dtype), qo)


@pytest.mark.parametrize("case", [
    dict(T=100, H=256, E=16, k=4, I=256, weights="fp32", mode="clipped", smooth=True),
    dict(T=300, H=256, E=8, k=2, I=256, weights="fp32", mode="static", smooth=True),
    dict(T=64, H=512, E=8, k=2, I=128, weights="int8", mode="clipped", smooth=False),
], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_moe_with_scale_options(w8, case):
    """The whole layer with a smoothing vector on x (the gate-up weights
    quantised with its inverse) and a clipped or static x scale, against the
    oracle at the INT8 bar (x codes exact, routing, h, codes, o, y)."""
    case = dict(case)
    mode, smooth = case.pop("mode"), case.pop("smooth")
    over = dict(n_outlier=2, outlier_scale=20.0, bf16_x=False, bias="zero")
    over.update(case)
    inp = synth.moe_inputs("edge", device="cuda", **over)
    H = inp["H"]
    rng = np.random.default_rng(H)
    qopts = dict(x_scale_mode=mode)
    x = to_np(inp["x"])
    if smooth:
        m = (1.0 / np.sqrt(np.abs(x).max(axis=0) + 1e-3)).astype(np.float32)  # flattens outlier columns
        m *= rng.uniform(0.9, 1.1, H).astype(np.float32)
        qopts["x_smooth"] = m
        xs = x * m
    else:
        xs = x
    amax = np.abs(xs).max(axis=1)
    qopts["x_clip"] = float(np.quantile(amax, 0.5))  # half of the tokens are clipped
    check_moe(w8, inp, qopts=qopts)
