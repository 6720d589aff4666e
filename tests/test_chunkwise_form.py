"""CPU check of the chunkwise algebra the HIP kernels implement (not the oracle).

The kernels never run the token loop.  Per chunk of n tokens they form, in the stored
state orientation M = S^T [dk, dv]:

  g_t = sum_{s<=t} log alpha_s,  gamma_t = exp(g_t),  Gamma_ts = exp(g_t - g_s) (s <= t)
  L = strictly_lower(diag(beta) (K K^T) o Gamma),  Tt = (I + L)^-1 diag(beta)
  W = Tt diag(gamma) K,  U = Tt V,  D_s = exp(g_{n-1} - g_s)
  At = gamma_{n-1} I - K^T diag(D) W,   Bc = K^T diag(D) U          (M_end = At M0 + Bc)
  P = (Q K^T) o Gamma (lower, with diagonal)
  Qp = diag(gamma) Q - P W,  O_intra = P U                           (O = O_intra + Qp M0)

This test checks that algebra against the oracle in float64, so a derivation mistake is
caught before any kernel runs.
"""
import numpy as np
import pytest

import oracle


def chunk_form(q, k, v, beta, alpha):
    n = k.shape[0]
    g = np.cumsum(np.log(alpha))
    gam = np.exp(g)
    Gam = np.tril(np.exp(g[:, None] - g[None, :]))
    L = np.tril(beta[:, None] * (k @ k.T) * Gam, -1)
    Tt = np.linalg.solve(np.eye(n) + L, np.diag(beta))
    W = Tt @ (gam[:, None] * k)
    U = Tt @ v
    D = np.exp(g[-1] - g)
    At = gam[-1] * np.eye(k.shape[1]) - k.T @ (D[:, None] * W)
    Bc = k.T @ (D[:, None] * U)
    P = (q @ k.T) * Gam
    Qp = gam[:, None] * q - P @ W
    Oi = P @ U
    return At, Bc, Qp, Oi


@pytest.mark.parametrize("n", [1, 5, 13, 64])
def test_chunk_form_matches_oracle(n):
    rng = np.random.default_rng(n)
    dk, dv = 7, 5
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((n, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal(n)))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal(n) - 3))
    S0 = rng.standard_normal((dv, dk))
    At, Bc, Qp, Oi = chunk_form(q, k, v, beta, alpha)
    A, B = oracle.chunk_transition(k, v, beta, alpha)
    np.testing.assert_allclose(At, A.T, atol=1e-12)
    np.testing.assert_allclose(Bc, B.T, atol=1e-12)
    o, S = oracle.gdn_recurrent(q, k, v, beta, alpha, S0=S0)
    M0 = S0.T
    np.testing.assert_allclose(Oi + Qp @ M0, o, atol=1e-12)
    np.testing.assert_allclose(At @ M0 + Bc, S.T, atol=1e-12)


def test_gated_step_in_stored_orientation():
    # S -> S + g (S A + B - S)  <=>  M -> M + g (At M + Bc - M), with M = S^T, At = A^T, Bc = B^T.
    rng = np.random.default_rng(0)
    S = rng.standard_normal((3, 4))
    A = rng.standard_normal((4, 4))
    B = rng.standard_normal((3, 4))
    g = 0.37
    lhs = (S + g * (S @ A + B - S)).T
    M = S.T
    rhs = M + (A.T - np.eye(4)) @ (g * M) + g * B.T
    np.testing.assert_allclose(lhs, rhs, atol=1e-14)
