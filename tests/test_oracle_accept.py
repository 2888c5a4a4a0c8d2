"""Pins of the MTP draft-verification oracle (no GPU).

GeekNews #31297, implemented features: drafts of the multi-token-prediction
head are verified by the main model in one batched forward, and rejection
sampling keeps sampled output lossless; the yodev.dev page: greedy output is
identical to plain greedy decoding.  The checks below hold the oracle to
those two properties, and to the closed form of the acceptance rate, by
integrating the oracle's own decisions over midpoint grids of its uniforms
and over drafts weighted by the draft distribution (brute force on tiny
vocabularies); none of them restates the acceptance rule.
"""
import itertools

import numpy as np

import oracle

TAU = 0.7
P0 = np.array([2.0, 0.5, -1.0, 1.0, 0.0], np.float32)
Q0 = np.array([0.0, 1.5, 0.5, 1.0, -2.0], np.float32)
P1 = np.array([-0.5, 1.0, 0.3, 2.2, -1.5], np.float32)
Q1 = np.array([1.0, -1.0, 0.0, 0.7, 0.9], np.float32)
P2 = np.array([0.2, -0.4, 1.8, 0.1, 0.6], np.float32)


def dist(z, tau=TAU):
    """The distribution a logit row stands for at temperature tau (fp64)."""
    e = np.exp((np.asarray(z, np.float64) - float(np.max(z))) / tau)
    return e / e.sum()


def grid(n, dims):
    m = (np.arange(n) + 0.5) / n
    return np.array(list(itertools.product(m, repeat=dims)), np.float64)


def emitted_first(p_rows, q_rows, n, tau=TAU):
    """Frequency of the first emitted token over drafts x ~ q_0 and an n x n
    grid of (u_0, u_1); D = 1."""
    V = p_rows.shape[1]
    u = grid(n, 2)
    qd = dist(q_rows[0], tau)
    freq = np.zeros(V)
    acc = 0.0
    for x in range(V):
        B = len(u)
        pl = np.broadcast_to(p_rows, (B,) + p_rows.shape)
        ql = np.broadcast_to(q_rows, (B,) + q_rows.shape)
        n_acc, nxt, _ = oracle.mtp_accept(np.full((B, 1), x), pl, ql, tau, u)
        first = np.where(n_acc >= 1, x, nxt)
        freq += qd[x] * np.bincount(first, minlength=V) / B
        acc += qd[x] * np.mean(n_acc >= 1)
    return freq, acc


def test_sampled_first_token_is_lossless():
    """Drafts x ~ q and the rule together emit exactly p (grid error 3/n)."""
    n = 200
    freq, _ = emitted_first(np.stack([P0, P1]), Q0[None], n)
    assert np.abs(freq - dist(P0)).max() < 3.0 / n, (freq, dist(P0))


def test_acceptance_rate_is_one_minus_total_variation():
    """P(keep) = sum_x min(p(x), q(x)) for a draft drawn from q."""
    n = 200
    _, acc = emitted_first(np.stack([P0, P1]), Q0[None], n)
    want = np.minimum(dist(P0), dist(Q0)).sum()
    assert abs(acc - want) < 3.0 / n, (acc, want)


def test_second_and_bonus_tokens_follow_their_rows():
    """With q_0 = p_0 the first draft is always kept; the next emitted token
    then follows p_1 (draft x_1 ~ q_1), and with q_1 = p_1 too the bonus
    token follows p_2: the rows are used in order."""
    n = 120
    V = len(P0)
    u = grid(n, 2)
    B = len(u)
    # second token: u_0 fixed, (u_1, u_2) on the grid
    uu = np.concatenate([np.full((B, 1), 0.5), u], axis=1)
    pl = np.broadcast_to(np.stack([P0, P1, P2]), (B, 3, V))
    freq = np.zeros(V)
    q1 = dist(Q1)
    for x0, x1 in itertools.product(range(V), range(V)):
        ql = np.broadcast_to(np.stack([P0, Q1]), (B, 2, V))
        n_acc, nxt, _ = oracle.mtp_accept(np.tile([x0, x1], (B, 1)), pl, ql, TAU, uu)
        assert (n_acc >= 1).all()
        second = np.where(n_acc >= 2, x1, nxt)
        freq += dist(P0)[x0] * q1[x1] * np.bincount(second, minlength=V) / B
    assert np.abs(freq - dist(P1)).max() < 3.0 / n, (freq, dist(P1))
    # bonus token: both drafts kept, u_2 on a fine grid
    m = 4000
    u2 = (np.arange(m) + 0.5) / m
    uu = np.stack([np.full(m, 0.3), np.full(m, 0.9), u2], axis=1)
    pl = np.broadcast_to(np.stack([P0, P1, P2]), (m, 3, V))
    ql = np.broadcast_to(np.stack([P0, P1]), (m, 2, V))
    n_acc, nxt, _ = oracle.mtp_accept(np.tile([3, 1], (m, 1)), pl, ql, TAU, uu)
    assert (n_acc == 2).all()
    assert np.abs(np.bincount(nxt, minlength=V) / m - dist(P2)).max() < 2.0 / m


def test_no_drafts_is_inverse_cdf_sampling_of_p():
    """D = 0: the emitted token is p's inverse CDF at u: monotone in u, the
    first token at u = 0, the last at u -> 1, frequencies p."""
    m = 5000
    V = len(P0)
    u = ((np.arange(m) + 0.5) / m)[:, None]
    n_acc, nxt, _ = oracle.mtp_accept(np.zeros((m, 0), np.int32), np.broadcast_to(P0, (m, 1, V)),
                                      np.zeros((m, 0, V), np.float32), TAU, u)
    assert (n_acc == 0).all() and (np.diff(nxt) >= 0).all()
    assert np.abs(np.bincount(nxt, minlength=V) / m - dist(P0)).max() < 2.0 / m
    ends = np.array([[0.0], [1.0 - 2.0 ** -53]])
    _, e, _ = oracle.mtp_accept(np.zeros((2, 0), np.int32), np.broadcast_to(P0, (2, 1, V)),
                                np.zeros((2, 0, V), np.float32), TAU, ends)
    assert list(e) == [0, V - 1]


def test_identical_draft_and_target_keep_every_draft():
    rng = np.random.default_rng(3)
    B, D, V = 64, 4, 50
    pl = rng.normal(0, 2, (B, D + 1, V)).astype(np.float32)
    draft = rng.integers(0, V, (B, D))
    u = rng.random((B, D + 1))
    n_acc, _, _ = oracle.mtp_accept(draft, pl, pl[:, :D], 1.3, u)
    assert (n_acc == D).all()


def test_greedy_equals_plain_greedy_decoding():
    """tau = 0: the tokens a step emits (kept drafts, then the next token)
    are the target's argmax chain, whatever the draft logits; ties go to the
    lower index."""
    rng = np.random.default_rng(5)
    B, D, V = 200, 4, 37
    pl = rng.integers(-3, 4, (B, D + 1, V)).astype(np.float32)  # many exact ties
    am = np.argmax(pl, axis=2)                                     # first maximum
    draft = am[:, :D].copy()
    cut = rng.integers(0, D + 1, B)                                # first wrong draft
    for b in range(B):
        if cut[b] < D:
            draft[b, cut[b]] = (am[b, cut[b]] + 1 + rng.integers(0, V - 1)) % V
    ql = rng.normal(0, 1, (B, D, V)).astype(np.float32)
    u = rng.random((B, D + 1))
    n_acc, nxt, _ = oracle.mtp_accept(draft, pl, ql, 0.0, u)
    assert (n_acc == cut).all()
    assert (nxt == am[np.arange(B), cut]).all()


def test_temperature_enters_both_distributions():
    """The same logits at two temperatures give the acceptance rate of the
    two tempered distributions."""
    n = 200
    for tau in (0.35, 1.6):
        _, acc = emitted_first(np.stack([P0, P1]), Q0[None], n, tau)
        want = np.minimum(dist(P0, tau), dist(Q0, tau)).sum()
        assert abs(acc - want) < 3.0 / n, (tau, acc, want)
