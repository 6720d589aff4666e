"""Pins for the Gated DeltaNet-2 gradient oracle (``oracle.grad_gdn2``), CPU only.

It differentiates a torch restatement of the Gated DeltaNet-2 forward with autograd, and is
pinned here against what it shares no code with:

* central finite differences of the numpy forward oracle (``oracle.gdn2``) along random
  directions, for every input of both per-chunk pieces and of the whole routed prefill;
* the collapse to the Gated DeltaNet gradient oracle (``oracle.grad``, pinned on its own)
  when every gate is one scalar per token: with a_t = alpha_t, b_t = w_t = beta_t on every
  channel the forward is Gated DeltaNet's, so dq, dk, dv, dS0 and dgates agree and the
  scalar gradients are the channel sums (dalpha = sum_c da, dbeta = sum_c db + sum_c dw);
* the closed form of one token from a given state.

Shapes use dk != dv so that a transposed operand fails loudly; gates are drawn per channel
so that a channel mix-up fails too.
"""
import numpy as np
import pytest

import oracle

EPS = 1e-6


def _seq(rng, T, dk, dv):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = np.exp(-np.logaddexp(0, rng.standard_normal((T, dk)) - 2.0))
    b = 1 / (1 + np.exp(-rng.standard_normal((T, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((T, dv))))
    return q, k, v, a, b, w


def _check_dir(f, x, grad, rng, rtol=1e-6, what=""):
    """<grad, d> against the central difference of f along two random directions d."""
    x = np.asarray(x, np.float64)
    for _ in range(2):
        d = rng.standard_normal(np.shape(x))
        fd = (f(x + EPS * d) - f(x - EPS * d)) / (2 * EPS)
        an = float(np.sum(grad * d))
        assert abs(an - fd) <= rtol * max(1.0, abs(fd)), f"{what}: autograd {an} vs finite difference {fd}"


def test_outputs_piece_matches_finite_differences():
    rng = np.random.default_rng(71)
    C, dk, dv = 4, 5, 3
    T = 3 * C + 2
    q, k, v, a, b, w = _seq(rng, T, dk, dv)
    N = -(-T // C)
    S = rng.standard_normal((N, dv, dk))
    dO = rng.standard_normal((T, dv))
    r = oracle.gdn2_chunk_outputs_backward(q, k, v, a, b, w, C, S, dO)
    args = dict(q=q, k=k, v=v, a=a, b=b, w=w, S=S)

    def loss(name, y):
        x = dict(args, **{name: y})
        return float(np.sum(dO * oracle.gdn2_routed_outputs(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], C, x["S"])))

    for name in args:
        key = "dS_routed" if name == "S" else "d" + name
        _check_dir(lambda y, n=name: loss(n, y), args[name], r[key], rng, what=name)


def test_maps_piece_matches_finite_differences():
    rng = np.random.default_rng(72)
    C, dk, dv = 4, 5, 3
    T = 3 * C + 1
    _, k, v, a, b, w = _seq(rng, T, dk, dv)
    A, B = oracle.gdn2_chunk_transitions(k, v, a, b, w, C)
    dA, dB = rng.standard_normal(A.shape), rng.standard_normal(B.shape)
    r = oracle.gdn2_chunk_transitions_backward(k, v, a, b, w, C, dA, dB)
    args = dict(k=k, v=v, a=a, b=b, w=w)

    def loss(name, y):
        x = dict(args, **{name: y})
        A2, B2 = oracle.gdn2_chunk_transitions(x["k"], x["v"], x["a"], x["b"], x["w"], C)
        return float(np.sum(dA * A2) + np.sum(dB * B2))

    for name in args:
        _check_dir(lambda y, n=name: loss(n, y), args[name], r["d" + name], rng, what=name)


def test_prefill_backward_matches_finite_differences():
    rng = np.random.default_rng(73)
    C, dk, dv = 4, 5, 3
    T = 4 * C + 3
    q, k, v, a, b, w = _seq(rng, T, dk, dv)
    q *= 3.0  # spread the gates
    S0 = rng.standard_normal((dv, dk))
    dO = rng.standard_normal((T, dv))
    tau = 1e-3
    ref = oracle.gdn2_hla_prefill_backward(q, k, v, a, b, w, C, tau, dO, S0=S0)
    assert ref["mask"].sum() > 0
    args = dict(q=q, k=k, v=v, a=a, b=b, w=w, S0=S0)

    def loss(name, y):
        x = dict(args, **{name: y})
        o = oracle.gdn2_hla_prefill(x["q"], x["k"], x["v"], x["a"], x["b"], x["w"], C, tau, S0=x["S0"])["o"]
        return float(np.sum(dO * o))

    for name in args:
        _check_dir(lambda y, n=name: loss(n, y), args[name], ref["d" + name], rng, what=name)


def test_caller_gates_match_finite_differences():
    rng = np.random.default_rng(74)
    C, dk, dv = 3, 4, 6
    T = 4 * C
    q, k, v, a, b, w = _seq(rng, T, dk, dv)
    N = T // C
    G = rng.uniform(0.05, 0.95, (N, N))
    tau = 0.4
    G[np.abs(G - tau) < 0.05] += 0.1
    dO = rng.standard_normal((T, dv))
    ref = oracle.gdn2_hla_prefill_backward(q, k, v, a, b, w, C, tau, dO, gates_in=G)

    def loss(Gx):
        return float(np.sum(dO * oracle.gdn2_hla_prefill(q, k, v, a, b, w, C, tau, gates_in=Gx)["o"]))

    for i in range(N):
        for j in range(i):
            E = np.zeros((N, N))
            E[i, j] = 1.0
            fd = (loss(G + EPS * E) - loss(G - EPS * E)) / (2 * EPS)
            assert abs(ref["dgates"][i, j] - fd) <= 1e-6 * max(1.0, abs(fd)), (i, j)
            if G[i, j] < tau:
                assert ref["dgates"][i, j] == 0.0


@pytest.mark.parametrize("with_s0", [False, True])
def test_scalar_gates_collapse_to_gated_deltanet(with_s0):
    rng = np.random.default_rng(75)
    C, dk, dv = 4, 5, 3
    T = 3 * C + 3
    q, k, v, _, _, _ = _seq(rng, T, dk, dv)
    q *= 3.0
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal(T) - 2.0))
    S0 = rng.standard_normal((dv, dk)) if with_s0 else None
    dO = rng.standard_normal((T, dv))
    a = np.repeat(alpha[:, None], dk, 1)
    b = np.repeat(beta[:, None], dk, 1)
    w = np.repeat(beta[:, None], dv, 1)
    g2 = oracle.gdn2_hla_prefill_backward(q, k, v, a, b, w, C, 1e-3, dO, S0=S0)
    g1 = oracle.hla_prefill_backward(q, k, v, beta, alpha, C, 1e-3, dO, S0=S0)
    assert np.array_equal(g1["mask"], g2["mask"])
    for n in ("dq", "dk", "dv", "dS0", "dgates"):
        np.testing.assert_allclose(g2[n], g1[n], rtol=1e-10, atol=1e-12, err_msg=n)
    np.testing.assert_allclose(g2["da"].sum(1), g1["dalpha"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g2["db"].sum(1) + g2["dw"].sum(1), g1["dbeta"], rtol=1e-10, atol=1e-12)


def test_one_token_closed_form():
    """One token from S0: o = Sd q - (Sd k)((b o k) . q) + (w o v)(k . q) with Sd = S0 diag(a),
    so dq = Sd^T dO - (b o k)((Sd k) . dO) + k ((w o v) . dO), dv = w o dO (k . q),
    dw = v o dO (k . q), dS0 = (dO q^T - (dO (b o k) . q) k^T) diag(a)."""
    rng = np.random.default_rng(76)
    dk, dv = 4, 3
    q, k, v, a, b, w = _seq(rng, 1, dk, dv)
    S0 = rng.standard_normal((1, dv, dk))
    dO = rng.standard_normal((1, dv))
    r = oracle.gdn2_chunk_outputs_backward(q, k, v, a, b, w, 1, S0, dO)
    Sd = S0[0] * a[0][None, :]
    bk = b[0] * k[0]
    kq = float(k[0] @ q[0])
    dq = Sd.T @ dO[0] - bk * float((Sd @ k[0]) @ dO[0]) + k[0] * float((w[0] * v[0]) @ dO[0])
    np.testing.assert_allclose(r["dq"][0], dq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dv"][0], w[0] * dO[0] * kq, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r["dw"][0], v[0] * dO[0] * kq, rtol=1e-12, atol=1e-14)
    dS0 = (np.outer(dO[0], q[0]) - float(bk @ q[0]) * np.outer(dO[0], k[0])) * a[0][None, :]
    np.testing.assert_allclose(r["dS_routed"][0], dS0, rtol=1e-12, atol=1e-14)
