"""Pins of the CPU oracle against things other than itself (no GPU).

Each test checks one oracle function against a brute force, a closed form,
a hand-made vector, an independent numpy formulation of a special case, or
an invariant of the method, so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, the wrong
rounding) fails at least one of them.  tests/test_oracle_mutants.py plants
such slips in a copy of the oracle and checks that these pins catch them.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth


# ---------------------------------------------------------------- helpers
def np_decode(wbits, codes, D):
    """Independent numpy decoder of packed rows -> signed int64 [rows][D]."""
    codes = np.asarray(codes, np.uint8)
    if wbits == 8:
        return codes.view(np.int8).astype(np.int64)
    if wbits == 4:
        lo = (codes & 15).astype(np.int64)
        hi = (codes >> 4).astype(np.int64)
        out = np.stack([lo, hi], -1).reshape(codes.shape[0], D)
        return (out ^ 8) - 8
    fields = [((codes >> (2 * i)) & 3).astype(np.int64) for i in range(4)]
    out = np.stack(fields, -1).reshape(codes.shape[0], D)
    return (out ^ 2) - 2


def rand_codes(rng, wbits, rows, D):
    return rng.integers(0, 256, size=(rows, D * wbits // 8), dtype=np.uint8) if wbits != 8 else \
        rng.integers(-127, 128, size=(rows, D), dtype=np.int64).astype(np.int8).view(np.uint8)


def mkshape(E, G, tg, k, H=64, I=64, wbits=4, rsf=2.5, n_shared=1):
    return oracle.Shape(H, I, E, G, tg, k, n_shared, wbits, rsf)


def np_scores(x, W, b):
    z = x.astype(np.float64) @ W.astype(np.float64).T
    s = 1.0 / (1.0 + np.exp(-z))
    return s, s + b.astype(np.float64)


def brute_route(s, c, E, G, tg, k, rsf):
    """Brute force: best group subset over all C(G, tg), then a full sort."""
    m = E // G
    gscore = [sum(sorted(c[g * m:(g + 1) * m], reverse=True)[:2]) for g in range(G)]
    best = None
    for sub in itertools.combinations(range(G), tg):      # lexicographic order
        tot = sum(gscore[g] for g in sub)
        if best is None or tot > best[0]:
            best = (tot, sub)
    cand = [e for g in best[1] for e in range(g * m, (g + 1) * m)]
    sel = sorted(cand, key=lambda e: (-c[e], e))[:k]
    ssum = sum(s[e] for e in sel)
    return np.array(sel), np.array([s[e] / ssum * rsf for e in sel])


# ---------------------------------------------------------------- codes
def test_code_layout_by_hand():
    # int4: element 2m = low nibble of byte m, two's complement
    row = np.array([0x8F, 0x70], np.uint8)
    assert [oracle.code(4, row, j) for j in range(4)] == [-1, -8, 0, 7]
    # int2: element 4m+i at bits 2i..2i+1: 0b11_10_01_00 -> 0, 1, -2, -1
    row = np.array([0xE4], np.uint8)
    assert [oracle.code(2, row, j) for j in range(4)] == [0, 1, -2, -1]
    row = np.array([0x80, 0x7F, 0x00, 0xFF], np.uint8)
    assert [oracle.code(8, row, j) for j in range(4)] == [-128, 127, 0, -1]


# ---------------------------------------------------------------- router
@pytest.mark.parametrize("E,G,tg,k,H", [(16, 4, 2, 4, 256), (32, 8, 3, 5, 64),
                                        (256, 8, 4, 8, 128), (12, 3, 1, 4, 32), (8, 8, 8, 3, 32)])
def test_route_matches_brute_force(E, G, tg, k, H):
    rng = np.random.default_rng(E * 131 + k)
    T = 40
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    b = (0.3 * rng.standard_normal(E)).astype(np.float32)
    sh = mkshape(E, G, tg, k, H=H)
    idx, w = oracle.route(sh, x, W, b)
    s_all, c_all = np_scores(x, W, b)
    for t in range(T):
        sel, wr = brute_route(s_all[t], c_all[t], E, G, tg, k, 2.5)
        assert list(idx[t]) == list(sel)
        np.testing.assert_allclose(w[t], wr, rtol=2e-7)
        assert abs(float(np.sum(w[t].astype(np.float64))) - 2.5) <= 2.5 * 1e-6


def test_route_textbook_special_case():
    # one group, no bias, rsf = 1: plain top-k of sigmoid scores, normalised
    rng = np.random.default_rng(7)
    E, H, k, T = 24, 48, 6, 30
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = rng.standard_normal((E, H)).astype(np.float32)
    sh = mkshape(E, 1, 1, k, H=H, rsf=1.0)
    idx, w = oracle.route(sh, x, W, np.zeros(E, np.float32))
    z = x.astype(np.float64) @ W.astype(np.float64).T
    for t in range(T):
        top = np.argsort(-z[t], kind="stable")[:k]           # sigmoid is monotone
        assert list(idx[t]) == list(top)
        sg = 1 / (1 + np.exp(-z[t][top]))
        np.testing.assert_allclose(w[t], sg / sg.sum(), rtol=2e-7)


def _crafted(c_values, G, tg, k):
    """Router inputs whose biased scores are exactly c_values: W = 0 gives s = 1/2."""
    E = len(c_values)
    sh = mkshape(E, G, tg, k, H=32, rsf=1.0)
    x = np.ones((1, 32), np.float32)
    W = np.zeros((E, 32), np.float32)
    b = np.asarray(c_values, np.float32) - np.float32(0.5)
    return oracle.route(sh, x, W, b, margins=True)


def test_route_group_score_is_top2_sum():
    # group 0: one high score; group 1: two moderate; group 2: four medium; group 3: low
    c = [0.9, 0.0, 0.0, 0.0,  0.6, 0.6, 0.0, 0.0,  0.5, 0.5, 0.5, 0.5,  0.1, 0.1, 0.1, 0.1]
    idx, w, m = _crafted(c, G=4, tg=1, k=2)
    # top-2 sums: 0.9, 1.2, 1.0, 0.2 -> group 1 (max-only would pick 0, sum-all group 2)
    assert list(idx[0]) == [4, 5]


def test_route_excluded_groups_never_selected():
    # expert 12 has the best single score but its group's top-2 sum is the worst
    c = [0.6, 0.6, 0.0, 0.0,  -0.2, -0.3, -0.4, -0.5,  0.5, 0.5, 0.1, 0.1,  0.95, -5.0, -5.0, -5.0]
    idx, w, m = _crafted(c, G=4, tg=2, k=6)
    # kept groups 0 (1.2) and 2 (1.0); k = 6 reaches into negative and zero scores
    # of kept groups before any expert of an excluded group
    assert list(idx[0]) == [0, 1, 8, 9, 10, 11]
    assert 12 not in idx[0]


def test_route_ties_go_to_lower_index():
    c = [0.7] * 8 + [0.7] * 8
    idx, w, m = _crafted(c, G=4, tg=2, k=3)
    assert list(idx[0]) == [0, 1, 2]          # groups 0 and 1 kept, experts in index order
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=1e-7)
    assert m[0][0] == 0.0 and m[0][1] == 0.0


def test_route_weights_use_unbiased_scores():
    rng = np.random.default_rng(3)
    E, H = 16, 64
    x = rng.standard_normal((5, H)).astype(np.float32)
    W = rng.standard_normal((E, H)).astype(np.float32) / 8
    b = rng.standard_normal(E).astype(np.float32)
    sh = mkshape(E, 4, 2, 4, H=H, rsf=2.5)
    idx, w = oracle.route(sh, x, W, b)
    s, _ = np_scores(x, W, b)
    for t in range(5):
        ss = s[t][idx[t]]
        np.testing.assert_allclose(w[t], ss / ss.sum() * 2.5, rtol=2e-7)


# ---------------------------------------------------------------- adaptive expert top-p
def _with_p(sh, p):
    sh.top_p = float(np.float32(p))
    return sh


@pytest.mark.parametrize("p", [0.25, 0.5, 0.7, 0.9])
def test_top_p_keeps_the_shortest_prefix_reaching_p(p):
    rng = np.random.default_rng(int(p * 100))
    E, G, tg, k, H, T = 32, 8, 3, 6, 64, 60
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((E, H)) / math.sqrt(H)).astype(np.float32)
    b = (0.3 * rng.standard_normal(E)).astype(np.float32)
    i0, w0 = oracle.route(mkshape(E, G, tg, k, H=H), x, W, b)
    i1, w1 = oracle.route(_with_p(mkshape(E, G, tg, k, H=H), p), x, W, b)
    counts = []
    for t in range(T):
        n = int((i1[t] >= 0).sum())
        counts.append(n)
        assert 1 <= n <= k
        assert list(i1[t][:n]) == list(i0[t][:n])          # a prefix of the selection, in order
        assert np.all(i1[t][n:] == -1) and np.all(w1[t][n:] == 0)
        assert abs(float(w1[t].astype(np.float64).sum()) - 2.5) <= 2.5e-6   # renormalised
        np.testing.assert_allclose(w1[t][:n] / w1[t][0], w0[t][:n] / w0[t][0], rtol=1e-6)
        share = np.cumsum(w0[t].astype(np.float64)) / float(w0[t].astype(np.float64).sum())
        if n > 1:
            assert share[n - 2] < p + 1e-6                   # one fewer does not reach p
        assert share[n - 1] >= p - 1e-6                      # n does
    assert len(set(counts)) > 1                              # the cut adapts per token


def test_top_p_off_and_single_expert():
    rng = np.random.default_rng(5)
    E, H, T = 16, 64, 20
    x = rng.standard_normal((T, H)).astype(np.float32)
    W = (rng.standard_normal((E, H)) / 8).astype(np.float32)
    b = (0.2 * rng.standard_normal(E)).astype(np.float32)
    i0, w0 = oracle.route(mkshape(E, 4, 2, 4, H=H), x, W, b)
    for p in (0.0, 1.0, 1.5):                                # off: the plain selection
        i1, w1 = oracle.route(_with_p(mkshape(E, 4, 2, 4, H=H), p), x, W, b)
        assert np.array_equal(i1, i0) and np.array_equal(w1, w0)
    i1, w1 = oracle.route(_with_p(mkshape(E, 4, 2, 4, H=H), 1e-7), x, W, b)
    assert np.array_equal(i1[:, 0], i0[:, 0]) and np.all(i1[:, 1:] == -1)
    assert np.all(w1[:, 0] == np.float32(2.5)) and np.all(w1[:, 1:] == 0)


def test_top_p_boundary_is_inclusive():
    # four equal scores in the kept group: every share is exactly 1/4, so
    # p = 1/2 is reached with two experts and p = 3/4 with three
    c = [0.8] * 4 + [0.1] * 4
    for p, n in ((0.5, 2), (0.75, 3), (0.5000001, 3)):
        E = len(c)
        sh = _with_p(mkshape(E, 2, 1, 4, H=32, rsf=1.0), p)
        x = np.ones((1, 32), np.float32)
        W = np.zeros((E, 32), np.float32)
        idx, w = oracle.route(sh, x, W, np.asarray(c, np.float32) - np.float32(0.5))
        assert list(idx[0]) == [0, 1, 2, 3][:n] + [-1] * (4 - n)
        np.testing.assert_allclose(w[0][:n], [1.0 / n] * n, rtol=1e-7)


def test_top_p_follows_selection_order_not_weight():
    # the bias ranks the experts by c as 2, 1, 0 while their weights (from the
    # unbiased s) rank 0, 1, 2; the prefix is taken in selection order
    z = np.array([2.0, 0.0, -2.0, -5.0])
    E, H = 4, 32
    x = np.ones((1, H), np.float32)
    W = np.repeat((z / H)[:, None], H, 1).astype(np.float32)
    b = np.array([0.0, 0.5, 1.0, 0.0], np.float32)
    idx, w = oracle.route(_with_p(mkshape(E, 1, 1, 3, H=H, rsf=1.0), 0.3), x, W, b)
    s = 1 / (1 + np.exp(-z))
    assert list(idx[0]) == [2, 1, -1]                        # shares 0.08, then 0.41 >= 0.3
    np.testing.assert_allclose(w[0][:2], s[[2, 1]] / s[[2, 1]].sum(), rtol=1e-6)


def test_top_p_layer_with_one_expert_per_token():
    # p tiny: each token keeps its first expert at weight rsf, so the layer is
    # rsf * FFN_first(x) + FFN_shared(x)
    wl = synth.workload("tiny")
    L, sh = _tiny_layer(wl)
    sh = _with_p(sh, 1e-7)
    idx, w = oracle.route(sh, L.x, L.gate_w, L.bias)
    assert np.all(idx[:, 1:] == -1)
    y, _, _ = oracle.layer_forward(sh, L.x, L.gate_w, L.bias, oracle.layer_experts(L, idx), L.shared)
    q, d = oracle.quant_act(L.x)
    for t in range(wl.T):
        ref = oracle.expert_ffn(sh, L.shared, q[t:t + 1], d[t:t + 1]).astype(np.float64)[0] + \
            wl.rsf * oracle.expert_ffn(sh, L.expert(idx[t, 0]), q[t:t + 1], d[t:t + 1]).astype(np.float64)[0]
        np.testing.assert_allclose(y[t], ref, rtol=0, atol=1e-5 * np.abs(ref).max())


def test_route_rejects_bad_shapes():
    x = np.zeros((1, 32), np.float32)
    with pytest.raises(ValueError):
        oracle.route(mkshape(16, 5, 2, 4, H=32), x, np.zeros((16, 32), np.float32), np.zeros(16, np.float32))
    with pytest.raises(ValueError):
        oracle.route(mkshape(16, 4, 2, 9, H=32), x, np.zeros((16, 32), np.float32), np.zeros(16, np.float32))


# ---------------------------------------------------------------- quantiser
def test_quant_round_half_even_by_hand():
    # amax = 127 gives d = 1 exactly, so q = rint(x)
    x = np.zeros((1, 32), np.float32)
    x[0, :10] = [127, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5, -126.5, 4.4999995]
    q, d = oracle.quant_act(x)
    assert d[0, 0] == 1.0
    assert list(q[0, :10]) == [127, 2, 4, -2, 0, 2, 0, 126, -126, 4]
    # a true division, not a multiply by 1/d: here x/d = 3.4999998 in fp32
    # (rounds to 3) while x * (1/d) lands on 3.5 (would round to 4)
    x = np.zeros((1, 32), np.uint32)
    x[0, 0], x[0, 1] = 0x3FA3D70A, 0x3D107D23       # amax = 1.28, x = 0.0352756
    q, d = oracle.quant_act(x.view(np.float32))
    assert list(q[0, :2]) == [127, 3]


def test_quant_closed_forms():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 256)) * rng.uniform(0.01, 100, (64, 1))).astype(np.float32)
    x[3, 32:64] = 0.0                                         # zero block
    x[5, 0:32] = np.float32(1e-40) * np.sign(rng.standard_normal(32)).astype(np.float32)
    q, d = oracle.quant_act(x)
    xb = x.reshape(64, 8, 32).astype(np.float64)
    qb = q.reshape(64, 8, 32).astype(np.int64)
    amax = np.abs(xb).max(-1)
    # scale = amax / 127 rounded to fp32 (to within half an fp32 ulp, subnormals excepted)
    big = amax > 1e-30
    np.testing.assert_allclose(d[big], (amax / 127)[big], rtol=2 ** -24)
    assert d[3, 1] == 0 and np.all(q[3, 32:64] == 0)
    assert d[5, 0] > 0                                        # no flush to zero
    # the amax element maps to +-127
    arg = np.abs(xb).argmax(-1)
    top = np.take_along_axis(qb, arg[..., None], -1)[..., 0]
    sgn = np.sign(np.take_along_axis(xb, arg[..., None], -1)[..., 0])
    nz = amax > 0
    assert np.all(top[nz] == 127 * sgn[nz])
    # reconstruction error within half a step
    err = np.abs(xb - d[..., None].astype(np.float64) * qb)
    assert np.all(err <= d[..., None] * 0.5 * (1 + 1e-6) + 1e-45)
    assert q.min() >= -127 and q.max() <= 127


# ---------------------------------------------------------------- integer dots
@pytest.mark.parametrize("wbits", [2, 4, 8])
def test_block_dots_brute_force(wbits):
    rng = np.random.default_rng(wbits)
    rows, D, T = 7, 96, 3
    codes = rand_codes(rng, wbits, rows, D)
    q = rng.integers(-127, 128, (T, D)).astype(np.int8)
    got = oracle.block_dots(wbits, codes, D, q)
    W = np_decode(wbits, codes, D)
    for t in range(T):
        for r in range(rows):
            for b in range(D // 32):
                ref = sum(int(W[r, j]) * int(q[t, j]) for j in range(32 * b, 32 * b + 32))
                assert got[t, r, b] == ref


@pytest.mark.parametrize("wbits,lo,bound", [(8, 0x81, 516128), (4, 0x88, 32512), (2, 0xAA, 8128)])
def test_block_dots_extremes(wbits, lo, bound):
    # most negative codes times q = -127 gives the largest block sum
    D = 32
    codes = np.full((1, D * wbits // 8), lo, np.uint8)
    q = np.full((1, D), -127, np.int8)
    assert oracle.block_dots(wbits, codes, D, q)[0, 0, 0] == bound


@pytest.mark.parametrize("wbits", [2, 4, 8])
def test_matvec_equals_dequantised_matmul(wbits):
    rng = np.random.default_rng(40 + wbits)
    rows, D, T = 33, 256, 4
    codes = rand_codes(rng, wbits, rows, D)
    s_w = rng.uniform(0.5, 1.5, rows).astype(np.float32) / 16
    x = rng.standard_normal((T, D)).astype(np.float32)
    q, d = oracle.quant_act(x)
    y = oracle.matvec(wbits, codes, s_w, D, q, d)
    # numpy: dequantise both operands to fp64, plain matmul
    Wf = np_decode(wbits, codes, D).astype(np.float64) * s_w[:, None].astype(np.float64)
    xf = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    ref = xf @ Wf.T
    np.testing.assert_allclose(y, ref, rtol=2 ** -23, atol=0)
    # the oracle's own cross-check path agrees to fp64 rounding
    y64 = oracle.dequant_matmul(wbits, codes, s_w, D, q, d)
    np.testing.assert_allclose(y64, ref, rtol=1e-12)


# ---------------------------------------------------------------- expert / layer
def _tiny_layer(wl):
    L = synth.HostLayer(wl)
    return L, oracle.shape_of(wl)


def test_single_expert_layer_is_dense_swiglu():
    """E = G = tg = k = 1, rsf = 1, no shared expert: the layer is one dense
    SwiGLU, W_d (silu(W_g x) * W_u x), here on the dequantised tensors with h
    kept in fp64; the only difference allowed is the int8 rounding of h."""
    wl = synth.workload("tiny", n_experts=1, n_group=1, topk_group=1, top_k=1, n_shared=0, rsf=1.0)
    L, sh = _tiny_layer(wl)
    ex = L.expert(0)
    y, idx, w = oracle.layer_forward(sh, L.x, L.gate_w, L.bias, {0: ex}, None)
    assert np.all(idx == 0) and np.all(w == 1.0)
    H, I = wl.hidden, wl.inter
    q, d = oracle.quant_act(L.x)
    xf = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    Wg = np_decode(4, ex.gate, H) * ex.gate_s[:, None].astype(np.float64)
    Wu = np_decode(4, ex.up, H) * ex.up_s[:, None].astype(np.float64)
    Wd = np_decode(4, ex.down, I) * ex.down_s[:, None].astype(np.float64)
    g, u = xf @ Wg.T, xf @ Wu.T
    h = g / (1 + np.exp(-g)) * u
    ref = h @ Wd.T
    # bound: |h - dequant(quant(h))| <= amax_block / 254 (+ fp32 roundings of g, u, h)
    amax = np.abs(h).reshape(wl.T, I // 32, 32).max(-1)
    eh = np.repeat(amax / 254 * (1 + 1e-5), 32, axis=1) + 1e-6 * np.abs(h)
    bound = eh @ np.abs(Wd).T + 1e-6 * np.abs(ref)
    assert np.all(np.abs(y - ref) <= bound)
    # the worst-case bound is a small fraction of the output scale, and the
    # actual error (a sum of independent rounding errors) far smaller still
    assert bound.max() < 0.1 * np.abs(ref).max()
    assert np.sqrt(np.mean((y - ref) ** 2)) < 0.01 * np.sqrt(np.mean(ref ** 2))


def test_layer_linear_in_rsf_and_shared_alone():
    wl = synth.workload("tiny")
    L, sh = _tiny_layer(wl)
    idx, _ = oracle.route(sh, L.x, L.gate_w, L.bias)
    ex = oracle.layer_experts(L, idx)
    y1, i1, _ = oracle.layer_forward(sh, L.x, L.gate_w, L.bias, ex, L.shared)
    y2, i2, _ = oracle.layer_forward(oracle.shape_of(wl, rsf=2 * wl.rsf), L.x, L.gate_w, L.bias, ex, L.shared)
    y0, i0, w0 = oracle.layer_forward(oracle.shape_of(wl, rsf=0.0), L.x, L.gate_w, L.bias, ex, L.shared)
    assert np.array_equal(i1, i2) and np.array_equal(i1, i0) and np.all(w0 == 0)
    q, d = oracle.quant_act(L.x)
    ysh = oracle.expert_ffn(sh, L.shared, q, d)
    assert np.array_equal(y0, ysh)                      # rsf = 0: shared expert alone, exactly
    r1 = y1.astype(np.float64) - ysh
    r2 = y2.astype(np.float64) - ysh
    scale = np.abs(y2).max()
    assert np.abs(r2 - 2 * r1).max() <= 4e-7 * scale * 4


def test_layer_equals_sum_of_experts():
    # out = sum_i w_i * FFN_{idx_i}(x) + FFN_shared(x), each FFN on the same quantised x
    wl = synth.workload("tiny")
    L, sh = _tiny_layer(wl)
    idx, w = oracle.route(sh, L.x, L.gate_w, L.bias)
    y, _, _ = oracle.layer_forward(sh, L.x, L.gate_w, L.bias, oracle.layer_experts(L, idx), L.shared)
    q, d = oracle.quant_act(L.x)
    for t in range(wl.T):
        acc = oracle.expert_ffn(sh, L.shared, q[t:t + 1], d[t:t + 1]).astype(np.float64)[0]
        for i in range(wl.top_k):
            acc += float(w[t, i]) * oracle.expert_ffn(sh, L.expert(idx[t, i]), q[t:t + 1], d[t:t + 1])[0]
        np.testing.assert_allclose(y[t], acc, rtol=0, atol=1e-5 * np.abs(acc).max())


def test_expert_tokens_independent():
    # batching tokens through one expert equals running them one at a time
    wl = synth.workload("tiny")
    L, sh = _tiny_layer(wl)
    q, d = oracle.quant_act(L.x)
    yb = oracle.expert_ffn(sh, L.expert(3), q, d)
    for t in range(wl.T):
        assert np.array_equal(yb[t], oracle.expert_ffn(sh, L.expert(3), q[t:t + 1], d[t:t + 1])[0])


# ---------------------------------------------------------------- rmsnorm, permute
def test_rmsnorm_closed_forms():
    x = np.array([[3.0, 4.0], [2.0, 2.0]], np.float32)
    g = np.array([1.0, 2.0], np.float32)
    out = oracle.rmsnorm(x, g, 1e-6)
    np.testing.assert_allclose(out[0], np.array([3, 8]) / math.sqrt(12.5 + 1e-6), rtol=1e-7)
    np.testing.assert_allclose(out[1], np.array([2, 4]) / math.sqrt(4 + 1e-6), rtol=1e-7)
    # unit mean square in, x / sqrt(1 + eps) out
    rng = np.random.default_rng(0)
    v = rng.standard_normal((1, 6144))
    v = (v / np.sqrt((v ** 2).mean())).astype(np.float32)
    o = oracle.rmsnorm(v, np.ones(6144, np.float32), 1e-6)
    ms = (v.astype(np.float64) ** 2).mean()
    np.testing.assert_allclose(o, v / np.sqrt(ms + 1e-6), rtol=1e-7)


def test_permute_skips_dropped_assignments():
    # top-p leaves a per-token prefix; the dropped slots (-1) get no row
    rng = np.random.default_rng(9)
    T, k, E = 40, 6, 16
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    kept = rng.integers(1, k + 1, T)
    for t in range(T):
        idx[t, kept[t]:] = -1
    perm, off, inv = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    live = [a for a in range(T * k) if flat[a] >= 0]
    R = len(live)
    assert off[E] == R == kept.sum()
    assert list(perm[:R]) == sorted(live, key=lambda a: flat[a])
    assert np.all(inv.reshape(-1)[flat < 0] == -1)
    assert np.array_equal(perm[inv.reshape(-1)[flat >= 0]], np.array(live))


def test_permute_is_stable_sort():
    rng = np.random.default_rng(5)
    T, k, E = 50, 4, 12
    idx = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    perm, off, inv = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    ref = sorted(range(T * k), key=lambda a: flat[a])          # Python's sort is stable
    assert list(perm) == ref
    assert list(off) == [0] + list(np.cumsum(np.bincount(flat, minlength=E)))
    assert np.array_equal(perm[inv.reshape(-1)], np.arange(T * k))
    # empty batch
    perm, off, inv = oracle.permute(np.zeros((0, k), np.int32), E)
    assert perm.size == 0 and np.all(off == 0)
