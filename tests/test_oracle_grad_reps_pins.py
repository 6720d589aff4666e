"""Pins for the learned-representative gradient oracle (``oracle.grad_reps``) and for the
router gradient with learned representatives (``oracle.router_backward``, n_rep < C), CPU
only.

Both differentiate torch restatements with autograd; they are pinned here against what
they share no code with: central finite differences of the numpy forward oracle
(``oracle.window_reps``, ``oracle.router_gates``) along random directions, and the closed
form of a one-token window.  dk != window and a ragged last chunk (a window cut short and
one with no tokens) make a transposed operand or a layout slip fail.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def _check_dir(f, x, grad, rng, rtol=1e-6, what=""):
    x = np.asarray(x, np.float64)
    for _ in range(2):
        d = rng.standard_normal(np.shape(x))
        fd = (f(x + EPS * d) - f(x - EPS * d)) / (2 * EPS)
        an = float(np.sum(grad * d))
        assert abs(an - fd) <= rtol * max(1.0, abs(fd)), f"{what}: autograd {an} vs finite difference {fd}"


@pytest.mark.parametrize("with_wr", [False, True])
def test_window_reps_backward_matches_finite_differences(with_wr):
    rng = np.random.default_rng(91)
    C, window, dk = 8, 4, 5
    T = 2 * C + 3  # last chunk: a window of 3 tokens and one with none
    k = rng.standard_normal((T, dk))
    W = {n: rng.standard_normal((dk, dk)) / np.sqrt(dk) for n in ("Wq", "Wk", "Wv", "Wp", "Wr")}
    n_rows = -(-T // C) * (C // window)
    dreps = rng.standard_normal((n_rows, dk))
    Wr = W["Wr"] if with_wr else None
    r = oracle.window_reps_backward(k, C, window, W["Wq"], W["Wk"], W["Wv"], W["Wp"], dreps, Wr=Wr)
    args = dict(k=k, Wq=W["Wq"], Wk=W["Wk"], Wv=W["Wv"], Wp=W["Wp"])
    if with_wr:
        args["Wr"] = Wr
    else:
        assert r["dWr"] is None

    def loss(name, y):
        a = dict(args, **{name: y})
        reps = oracle.window_reps(a["k"], C, window, a["Wq"], a["Wk"], a["Wv"], a["Wp"])
        if with_wr:
            reps = reps @ a["Wr"]
        return float(np.sum(dreps * reps))

    for name in args:
        _check_dir(lambda y, n=name: loss(n, y), args[name], r["d" + name], rng, what=name)
    # the empty window passes nothing: its tokens do not exist, and its row's seed is unused
    d2 = dreps.copy()
    d2[-1] = 0.0
    r2 = oracle.window_reps_backward(k, C, window, W["Wq"], W["Wk"], W["Wv"], W["Wp"], d2, Wr=Wr)
    np.testing.assert_array_equal(r2["dk"], r["dk"])


def test_one_token_window_closed_form():
    """n = 1: P = [1], rep = Wp Wv x, so dx = Wv^T Wp^T drep, dWp = drep (Wv x)^T,
    dWv = (Wp^T drep) x^T and the query and key weights receive nothing."""
    rng = np.random.default_rng(92)
    dk = 4
    x = rng.standard_normal((1, dk))
    Wq, Wk, Wv, Wp = (rng.standard_normal((dk, dk)) for _ in range(4))
    drep = rng.standard_normal((1, dk))
    r = oracle.window_reps_backward(x, 1, 1, Wq, Wk, Wv, Wp, drep)
    np.testing.assert_allclose(r["dk"][0], Wv.T @ Wp.T @ drep[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dWp"], np.outer(drep[0], Wv @ x[0]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dWv"], np.outer(Wp.T @ drep[0], x[0]), rtol=1e-12, atol=1e-14)
    assert np.all(r["dWq"] == 0) and np.all(r["dWk"] == 0)


def test_router_backward_with_learned_reps():
    rng = np.random.default_rng(93)
    C, n_rep, dk = 6, 2, 5
    T = 4 * C + 1
    N = -(-T // C)
    q = 3.0 * rng.standard_normal((T, dk))
    reps = rng.standard_normal((N * n_rep, dk))
    dG = rng.standard_normal((N, N))
    r = oracle.router_backward(q, reps, n_rep, C, dG)

    def lr(**kw):
        a = dict(dict(q=q, reps=reps), **kw)
        g = oracle.router_gates(a["q"], a["reps"], n_rep, C, 0.0)["gates"]
        return float(np.sum(np.tril(dG, -1) * g))

    _check_dir(lambda y: lr(q=y), q, r["dq"], rng, what="router q")
    _check_dir(lambda y: lr(reps=y), reps, r["dreps"], rng, what="router reps")
    # the last chunk's representatives are never read
    assert np.all(r["dreps"][(N - 1) * n_rep:] == 0)
