"""Pins for the oracle's learned chunk representatives and the router's query projection.

[HLA] Methodology paragraph 2: a completed chunk is cut into pooling windows, self-attention
runs inside each window, the token outputs are mean-pooled and a learned projection gives
one representative per window; the router compares a projected query with them.

The pins are hand-derived closed forms and invariants, chosen so that a dropped 1/sqrt(dk),
a sum instead of a mean, a causal mask, a transposed weight or a window cut at the wrong
token each fail at least one of them.
"""
import math

import numpy as np
import pytest

import oracle


def _rng_w(rng, dk, scale=1.0):
    return scale * rng.standard_normal((dk, dk))


def test_two_token_window_by_hand():
    # dk = 4, tokens x0 = e0, x1 = 0; Wq = I, Wk = 2 ln 3 I, Wv = Wp = I.
    # Scores s_ts = (x_t . 2 ln3 x_s) / sqrt(4): row 0 = (ln 3, 0), row 1 = (0, 0).
    # Softmax rows: (3/4, 1/4) and (1/2, 1/2).  V = X: v0 = e0, v1 = 0, so o0 = 3/4 e0 and
    # o1 = 1/2 e0; their mean is 5/8 e0.  Without the 1/sqrt(dk) row 0 would be (9/10, 1/10)
    # and the mean 7/10 e0.
    dk = 4
    X = np.zeros((2, dk))
    X[0, 0] = 1.0
    I = np.eye(dk)
    rep = oracle.window_rep(X, I, 2 * math.log(3) * I, I, I)
    np.testing.assert_allclose(rep, [5 / 8, 0, 0, 0], rtol=0, atol=1e-15)


def test_value_and_output_projections_orientation():
    # same scores as above; V = X Wv^T makes v0 = Wv[:, 0], and rep = Wp (5/8 v0)
    dk = 4
    rng = np.random.default_rng(3)
    Wv, Wp = rng.standard_normal((dk, dk)), rng.standard_normal((dk, dk))
    X = np.zeros((2, dk))
    X[0, 0] = 1.0
    I = np.eye(dk)
    rep = oracle.window_rep(X, I, 2 * math.log(3) * I, Wv, Wp)
    np.testing.assert_allclose(rep, 5 / 8 * Wp @ Wv[:, 0], rtol=1e-14, atol=1e-15)


def test_query_key_projections_orientation():
    # rank-one Wq = e_a e_b^T and Wk = e_a e_c^T give scores x_t[b] x_s[c] / sqrt(dk); a
    # transposed Wq or Wk moves the product off e_a and the scores vanish.
    dk, a, b, c = 6, 1, 3, 4
    Wq = np.zeros((dk, dk)); Wq[a, b] = 1.0
    Wk = np.zeros((dk, dk)); Wk[a, c] = 1.0
    rng = np.random.default_rng(4)
    X = rng.standard_normal((2, dk))
    Wv, Wp = rng.standard_normal((dk, dk)), rng.standard_normal((dk, dk))
    s = np.outer(X[:, b], X[:, c]) / math.sqrt(dk)
    # two-way softmax = logistic of the score difference
    p1 = 1 / (1 + np.exp(-(s[:, 1] - s[:, 0])))
    V = np.stack([Wv @ X[0], Wv @ X[1]])
    mean_o = np.mean([(1 - p1[t]) * V[0] + p1[t] * V[1] for t in range(2)], axis=0)
    np.testing.assert_allclose(oracle.window_rep(X, Wq, Wk, Wv, Wp), Wp @ mean_o, rtol=1e-13, atol=1e-14)


def test_permutation_invariance_inside_a_window():
    # bidirectional attention followed by a mean: the token order inside a window is irrelevant
    rng = np.random.default_rng(5)
    dk = 8
    X = rng.standard_normal((7, dk))
    W = [_rng_w(rng, dk) for _ in range(4)]
    perm = rng.permutation(7)
    np.testing.assert_allclose(oracle.window_rep(X[perm], *W), oracle.window_rep(X, *W), rtol=1e-12, atol=1e-13)
    # ... but not to replacing a token
    Y = X.copy()
    Y[2] += 0.5
    assert np.abs(oracle.window_rep(Y, *W) - oracle.window_rep(X, *W)).max() > 1e-3


def test_zero_query_weights_pool_uniformly():
    # Wq = 0: every score is 0, attention is uniform, every output is mean(V), so the
    # representative is Wp Wv mean(X)
    rng = np.random.default_rng(6)
    dk = 8
    X = rng.standard_normal((5, dk))
    Wk, Wv, Wp = (_rng_w(rng, dk) for _ in range(3))
    rep = oracle.window_rep(X, np.zeros((dk, dk)), Wk, Wv, Wp)
    np.testing.assert_allclose(rep, Wp @ Wv @ X.mean(axis=0), rtol=1e-12, atol=1e-13)


def test_identical_tokens_and_single_token():
    rng = np.random.default_rng(7)
    dk = 8
    x = rng.standard_normal(dk)
    W = [_rng_w(rng, dk) for _ in range(4)]
    for n in (1, 6):
        rep = oracle.window_rep(np.tile(x, (n, 1)), *W)
        np.testing.assert_allclose(rep, W[3] @ W[2] @ x, rtol=1e-12, atol=1e-13)


def test_window_layout_and_ragged_end():
    # C = 8, window = 4, T = 13: chunk 0 = windows [0,4) [4,8); chunk 1 = [8,12) [12,13);
    # T = 9 leaves chunk 1's second window empty (a zero row)
    rng = np.random.default_rng(8)
    dk = 4
    k = rng.standard_normal((13, dk))
    W = [_rng_w(rng, dk) for _ in range(4)]
    reps = oracle.window_reps(k, 8, 4, *W)
    assert reps.shape == (4, dk)
    for row, (lo, hi) in enumerate([(0, 4), (4, 8), (8, 12), (12, 13)]):
        np.testing.assert_array_equal(reps[row], oracle.window_rep(k[lo:hi], *W))
    reps9 = oracle.window_reps(k[:9], 8, 4, *W)
    np.testing.assert_array_equal(reps9[2], oracle.window_rep(k[8:9], *W))
    np.testing.assert_array_equal(reps9[3], np.zeros(dk))
    # one window per chunk when window == C
    np.testing.assert_array_equal(oracle.window_reps(k, 8, 8, *W)[1], oracle.window_rep(k[8:13], *W))


def test_router_query_projection():
    # the projected query Wr qbar against r equals the raw query against Wr^T r (rows: r Wr)
    rng = np.random.default_rng(9)
    T, dk, C, n_rep = 40, 6, 8, 2
    q = rng.standard_normal((T, dk))
    reps = rng.standard_normal((T // C * n_rep, dk))
    Wr = rng.standard_normal((dk, dk))
    g_proj = oracle.router_gates(q, reps, n_rep, C, 0.0, Wr=Wr)["gates"]
    g_fold = oracle.router_gates(q, reps @ Wr, n_rep, C, 0.0)["gates"]
    np.testing.assert_allclose(g_proj, g_fold, rtol=1e-12, atol=1e-14)
    # identity projection changes nothing; a non-symmetric one does
    np.testing.assert_array_equal(oracle.router_gates(q, reps, n_rep, C, 0.0, Wr=np.eye(dk))["gates"],
                                  oracle.router_gates(q, reps, n_rep, C, 0.0)["gates"])
    assert np.abs(oracle.router_gates(q, reps, n_rep, C, 0.0, Wr=Wr.T)["gates"] - g_proj).max() > 1e-3


def test_decode_query_projection():
    rng = np.random.default_rng(10)
    dk, dv, Nc, n_rep = 6, 5, 3, 2
    q, k = rng.standard_normal(dk), rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    cA, cB = 0.5 * rng.standard_normal((Nc, dk, dk)), rng.standard_normal((Nc, dv, dk))
    reps = rng.standard_normal((Nc, n_rep, dk))
    Wr = rng.standard_normal((dk, dk))
    args = (q, k, v, 0.7, 0.9, rng.standard_normal((dv, dk)), np.eye(dk), cA, cB)
    a = oracle.decode_step(*args, reps, 0.0, Wr=Wr)
    b = oracle.decode_step(*args, reps @ Wr, 0.0)
    np.testing.assert_allclose(a["gates"], b["gates"], rtol=1e-12)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-12)
