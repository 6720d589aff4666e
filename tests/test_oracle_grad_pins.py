"""Pins for the gradient oracle (``oracle.grad``), CPU only.

The gradient oracle differentiates a torch restatement of the forward with autograd.  It is
pinned here against things it does not share code with:

* central finite differences of the numpy forward oracle (``oracle.gdn``), along random
  directions, for every input of every backward piece and of the whole routed prefill;
* closed forms of a one-token chunk and of one gated history pair.

Thresholds are placed in the widest gap between the gates, so the small perturbations never
flip a skip decision.  Shapes use dk != dv so that transposed operands fail loudly.
"""
import math

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
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal(T) - 2.0))
    return q, k, v, beta, alpha


def _fd(f, x, d):
    return (f(x + EPS * d) - f(x - EPS * d)) / (2 * EPS)


def _check_dir(f, x, grad, rng, rtol=1e-6, what=""):
    """<grad, d> against the central difference of f along two random directions d."""
    for _ in range(2):
        d = rng.standard_normal(np.shape(x))
        fd = _fd(f, np.asarray(x, np.float64), d)
        an = float(np.sum(grad * d))
        assert abs(an - fd) <= rtol * max(1.0, abs(fd)), f"{what}: autograd {an} vs finite difference {fd}"


def _gap_tau(g, mask_hist):
    """A threshold in the widest gap between the history gates (none within the gap)."""
    vals = np.sort(g[mask_hist])
    gaps = np.diff(vals)
    i = int(np.argmax(gaps))
    return float(0.5 * (vals[i] + vals[i + 1])), float(gaps[i])


@pytest.mark.parametrize("skip", [False, True])
def test_prefill_backward_matches_finite_differences(skip):
    rng = np.random.default_rng(11)
    C, dk, dv = 4, 5, 3
    T = 4 * C + 3  # five chunks, the last one ragged
    q, k, v, beta, alpha = _seq(rng, T, dk, dv)
    q *= 3.0  # spread the gates
    S0 = rng.standard_normal((dv, dk))
    dO = rng.standard_normal((T, dv))
    N = -(-T // C)
    hist = np.tril(np.ones((N, N), bool), -1)
    g = oracle.router_gates(q, k, C, C, 0.0)["gates"]
    tau, gap = _gap_tau(g, hist) if skip else (1e-3, 1.0)
    assert gap > 1e-3
    ref = oracle.hla_prefill_backward(q, k, v, beta, alpha, C, tau, dO, S0=S0)
    if skip:
        assert 0 < ref["mask"].sum() < hist.sum()

    def loss(**kw):
        args = dict(q=q, k=k, v=v, beta=beta, alpha=alpha, S0=S0)
        args.update(kw)
        o = oracle.hla_prefill(args["q"], args["k"], args["v"], args["beta"], args["alpha"], C, tau, S0=args["S0"])["o"]
        return float(np.sum(dO * o))

    for name, x in (("q", q), ("k", k), ("v", v), ("beta", beta), ("alpha", alpha), ("S0", S0)):
        _check_dir(lambda y, n=name: loss(**{n: y}), x, ref["d" + name], rng, what=name)


def test_gate_gradient_matches_finite_differences():
    """Caller gates: dL/dg_ij for every history pair; zero for the skipped ones."""
    rng = np.random.default_rng(12)
    C, dk, dv = 3, 4, 6
    T = 4 * C
    q, k, v, beta, alpha = _seq(rng, T, dk, dv)
    N = T // C
    G = rng.uniform(0.05, 0.95, (N, N))
    tau = 0.4
    G[np.abs(G - tau) < 0.05] += 0.1
    dO = rng.standard_normal((T, dv))
    ref = oracle.hla_prefill_backward(q, k, v, beta, alpha, C, tau, dO, gates_in=G)

    def loss(Gx):
        return float(np.sum(dO * oracle.hla_prefill(q, k, v, beta, alpha, C, tau, gates_in=Gx)["o"]))

    for i in range(N):
        for j in range(i):
            E = np.zeros((N, N))
            E[i, j] = 1.0
            fd = _fd(loss, G, E)
            assert abs(ref["dgates"][i, j] - fd) <= 1e-6 * max(1.0, abs(fd)), (i, j)
            if G[i, j] < tau:
                assert ref["dgates"][i, j] == 0.0
    assert np.count_nonzero(ref["dgates"]) > 0 and ref["mask"].sum() < N * (N - 1) // 2


def test_pieces_match_finite_differences():
    rng = np.random.default_rng(13)
    C, dk, dv = 4, 5, 3
    T = 3 * C + 2
    q, k, v, beta, alpha = _seq(rng, T, dk, dv)
    N = -(-T // C)
    A, B = oracle.chunk_transitions(k, v, beta, alpha, C)
    dA, dB = rng.standard_normal(A.shape), rng.standard_normal(B.shape)
    r = oracle.chunk_transitions_backward(k, v, beta, alpha, C, dA, dB)

    def lt(**kw):
        a = dict(k=k, v=v, beta=beta, alpha=alpha)
        a.update(kw)
        A2, B2 = oracle.chunk_transitions(a["k"], a["v"], a["beta"], a["alpha"], C)
        return float(np.sum(dA * A2) + np.sum(dB * B2))

    for name, x in (("k", k), ("v", v), ("beta", beta), ("alpha", alpha)):
        _check_dir(lambda y, n=name: lt(**{n: y}), x, r["d" + name], rng, what="transitions " + name)

    Sr = rng.standard_normal((N, dv, dk))
    dO = rng.standard_normal((T, dv))
    r = oracle.chunk_outputs_backward(q, k, v, beta, alpha, C, Sr, dO)

    def lo(**kw):
        a = dict(q=q, k=k, v=v, beta=beta, alpha=alpha, S=Sr)
        a.update(kw)
        return float(np.sum(dO * oracle.routed_outputs(a["q"], a["k"], a["v"], a["beta"], a["alpha"], C, a["S"])))

    for name, x in (("q", q), ("k", k), ("v", v), ("beta", beta), ("alpha", alpha), ("S", Sr)):
        key = "dS_routed" if name == "S" else "d" + name
        _check_dir(lambda y, n=name: lo(**{n: y}), x, r[key], rng, what="outputs " + name)

    G = np.tril(rng.uniform(0.1, 0.9, (N, N)), -1)
    mask = np.tril(rng.uniform(size=(N, N)) < 0.7, -1)
    ghat = np.where(mask, G, 0.0)
    S0 = rng.standard_normal((dv, dk))
    dS = rng.standard_normal((N, dv, dk))
    r = oracle.routed_states_backward(A, B, ghat, mask, dS, S0=S0)

    def lc(**kw):
        a = dict(A=A, B=B, g=ghat, S0=S0)
        a.update(kw)
        return float(np.sum(dS * oracle.routed_states(a["A"], a["B"], a["g"], mask, S0=a["S0"])))

    for name, key, x in (("A", "dA", A), ("B", "dB", B), ("S0", "dS0", S0)):
        _check_dir(lambda y, n=name: lc(**{n: y}), x, r[key], rng, what="compose " + name)
    for i in range(N):
        for j in range(i):
            E = np.zeros((N, N))
            E[i, j] = 1.0
            fd = _fd(lambda y: lc(g=y), ghat, E)
            assert abs(r["dghat"][i, j] - fd) <= 1e-6 * max(1.0, abs(fd))

    dG = rng.standard_normal((N, N))
    r = oracle.router_backward(q, k, C, C, dG)

    def lr(**kw):
        a = dict(q=q, k=k)
        a.update(kw)
        g = oracle.router_gates(a["q"], a["k"], C, C, 0.0)["gates"]
        return float(np.sum(np.tril(dG, -1) * g))

    _check_dir(lambda y: lr(q=y), q, r["dq"], rng, what="router q")
    _check_dir(lambda y: lr(k=y), k, r["dreps"], rng, what="router reps")


def test_pieces_chain_to_the_whole_backward():
    """The decomposition the library uses: outputs -> composition -> chunk maps and router,
    summed, equals the one-graph gradient."""
    rng = np.random.default_rng(14)
    C, dk, dv = 4, 5, 3
    T = 4 * C + 1
    q, k, v, beta, alpha = _seq(rng, T, dk, dv)
    q *= 3.0
    S0 = rng.standard_normal((dv, dk))
    dO = rng.standard_normal((T, dv))
    N = -(-T // C)
    g = oracle.router_gates(q, k, C, C, 0.0)["gates"]
    tau, _ = _gap_tau(g, np.tril(np.ones((N, N), bool), -1))
    whole = oracle.hla_prefill_backward(q, k, v, beta, alpha, C, tau, dO, S0=S0)
    fw = oracle.hla_prefill(q, k, v, beta, alpha, C, tau, S0=S0)
    ro = oracle.chunk_outputs_backward(q, k, v, beta, alpha, C, fw["S_routed"], dO)
    rc = oracle.routed_states_backward(fw["A"], fw["B"], fw["ghat"], fw["mask"], ro["dS_routed"], S0=S0)
    rt = oracle.chunk_transitions_backward(k, v, beta, alpha, C, rc["dA"], rc["dB"])
    rr = oracle.router_backward(q, k, C, C, rc["dghat"])
    np.testing.assert_allclose(ro["dq"] + rr["dq"], whole["dq"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ro["dk"] + rt["dk"] + rr["dreps"], whole["dk"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ro["dv"] + rt["dv"], whole["dv"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ro["dbeta"] + rt["dbeta"], whole["dbeta"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ro["dalpha"] + rt["dalpha"], whole["dalpha"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rc["dS0"], whole["dS0"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(rc["dghat"], whole["dgates"], rtol=1e-10, atol=1e-12)


def test_one_token_closed_form():
    """T = 1: o = S q, S = alpha S0 (I - beta k k^T) + beta v k^T, L = dO . o."""
    rng = np.random.default_rng(15)
    dk, dv = 5, 3
    q, k, v, beta, alpha = _seq(rng, 1, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    dO = rng.standard_normal((1, dv))
    r = oracle.hla_prefill_backward(q, k, v, beta, alpha, 1, 1e-3, dO, S0=S0)
    q1, k1, v1, b, a, d = q[0], k[0], v[0], beta[0], alpha[0], dO[0]
    kq = k1 @ q1
    S = a * S0 @ (np.eye(dk) - b * np.outer(k1, k1)) + b * np.outer(v1, k1)
    np.testing.assert_allclose(r["dv"][0], b * kq * d, rtol=1e-12)
    np.testing.assert_allclose(r["dq"][0], S.T @ d, rtol=1e-12)
    np.testing.assert_allclose(r["dbeta"][0], kq * (d @ v1) - a * kq * (d @ S0 @ k1), rtol=1e-12)
    np.testing.assert_allclose(r["dalpha"][0], d @ S0 @ q1 - b * kq * (d @ S0 @ k1), rtol=1e-12)
    np.testing.assert_allclose(r["dS0"], a * np.outer(d, q1 - b * kq * k1), rtol=1e-12)
    dk_ref = -a * b * (kq * (S0.T @ d) + (d @ S0 @ k1) * q1) + b * (d @ v1) * q1
    np.testing.assert_allclose(r["dk"][0], dk_ref, rtol=1e-12)


def test_one_gated_pair_closed_form():
    """Two one-token chunks with a caller gate g on the pair: the routed state of chunk 1 is
    S~ = g (S0 A_0 + B_0) + (1 - g) S0, so dL/dg = <dS~, S0 A_0 + B_0 - S0> with
    dS~ = alpha_1 dO_1 (q_1 - beta_1 (k_1 . q_1) k_1)^T."""
    rng = np.random.default_rng(16)
    dk, dv = 4, 3
    q, k, v, beta, alpha = _seq(rng, 2, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    dO = np.zeros((2, dv))
    dO[1] = rng.standard_normal(dv)
    G = np.array([[0.0, 0.0], [0.37, 0.0]])
    r = oracle.hla_prefill_backward(q, k, v, beta, alpha, 1, 0.1, dO, S0=S0, gates_in=G)
    A0 = alpha[0] * (np.eye(dk) - beta[0] * np.outer(k[0], k[0]))
    B0 = beta[0] * np.outer(v[0], k[0])
    dS = alpha[1] * np.outer(dO[1], q[1] - beta[1] * (k[1] @ q[1]) * k[1])
    np.testing.assert_allclose(r["dgates"][1, 0], np.sum(dS * (S0 @ A0 + B0 - S0)), rtol=1e-12)
    # and chunk 0's own output gradient is zero, so dS0 is the gated pass-through only
    dS0 = 0.37 * dS @ A0.T + (1 - 0.37) * dS
    np.testing.assert_allclose(r["dS0"], dS0, rtol=1e-12)
    assert math.isfinite(r["dgates"][1, 0])
