"""Pins for the Gated DeltaNet-2 oracle ([GDN2] abstract): its reductions to Gated DeltaNet,
closed forms for decay, erase and write, the order of decay and edit, and the exactness of
its chunk maps.  Shapes use dk != dv so transposed operands fail."""
import numpy as np

import oracle


def _seq(rng, T, dk, dv):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal((T, dk)) - 3))
    b = 1 / (1 + np.exp(-rng.standard_normal((T, dk))))
    w = 1 / (1 + np.exp(-rng.standard_normal((T, dv))))
    return q, k, v, alpha, b, w


def test_collapses_to_gated_deltanet():
    # b = w = beta and a scalar decay: the Gated DeltaNet recurrence (pinned on its own)
    rng = np.random.default_rng(1)
    T, dk, dv = 23, 6, 4
    q, k, v, _, _, _ = _seq(rng, T, dk, dv)
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    alpha = np.exp(-np.logaddexp(0, rng.standard_normal(T)))
    S0 = rng.standard_normal((dv, dk))
    o2, S2 = oracle.gdn2_recurrent(q, k, v, np.repeat(alpha[:, None], dk, 1), np.repeat(beta[:, None], dk, 1),
                                   np.repeat(beta[:, None], dv, 1), S0=S0)
    o1, S1 = oracle.gdn_recurrent(q, k, v, beta, alpha, S0=S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-13)
    A2, B2 = oracle.gdn2_chunk_transitions(k, v, np.repeat(alpha[:, None], dk, 1), np.repeat(beta[:, None], dk, 1),
                                           np.repeat(beta[:, None], dv, 1), 8)
    A1, B1 = oracle.chunk_transitions(k, v, beta, alpha, 8)
    np.testing.assert_allclose(A2, A1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(B2, B1, rtol=1e-12, atol=1e-14)


def test_single_token_from_zero():
    # S = (w o v) k^T, so o = (k . q) (w o v)
    rng = np.random.default_rng(2)
    q, k, v, alpha, b, w = _seq(rng, 1, 5, 3)
    o, S = oracle.gdn2_recurrent(q, k, v, alpha, b, w)
    np.testing.assert_allclose(S, np.outer(w[0] * v[0], k[0]), rtol=1e-14)
    np.testing.assert_allclose(o[0], (k[0] @ q[0]) * w[0] * v[0], rtol=1e-13)


def test_pure_channel_decay():
    # b = w = 0: only the decay acts, S_T = S0 diag(prod_t alpha_t)
    rng = np.random.default_rng(3)
    q, k, v, alpha, _, _ = _seq(rng, 9, 5, 3)
    S0 = rng.standard_normal((3, 5))
    _, S = oracle.gdn2_recurrent(q, k, v, alpha, np.zeros((9, 5)), np.zeros((9, 3)), S0=S0)
    np.testing.assert_allclose(S, S0 * np.prod(alpha, axis=0)[None, :], rtol=1e-13)


def test_erase_is_per_key_channel():
    # S0 = v0 k0^T with a unit k0 and the same key again, no decay and no write:
    # b = 1 erases everything; b = e_c erases key channel c only (S (b o k) k^T would not)
    rng = np.random.default_rng(4)
    dk, dv = 5, 3
    k0 = rng.standard_normal(dk)
    k0 /= np.linalg.norm(k0)
    v0 = rng.standard_normal(dv)
    S0 = np.outer(v0, k0)
    one = np.ones((1, dk))
    _, S = oracle.gdn2_recurrent(None, k0[None], np.zeros((1, dv)), one, one, np.zeros((1, dv)), S0=S0)
    np.testing.assert_allclose(S, 0, atol=1e-15)
    c = 2
    bc = np.zeros((1, dk))
    bc[0, c] = 1
    _, S = oracle.gdn2_recurrent(None, k0[None], np.zeros((1, dv)), one, bc, np.zeros((1, dv)), S0=S0)
    expect = S0.copy()
    expect[:, c] = 0
    np.testing.assert_allclose(S, expect, atol=1e-15)


def test_write_gate_is_per_value_channel():
    rng = np.random.default_rng(5)
    dk, dv, j = 4, 3, 1
    k = rng.standard_normal((1, dk))
    v = rng.standard_normal((1, dv))
    wj = np.zeros((1, dv))
    wj[0, j] = 1
    _, S = oracle.gdn2_recurrent(None, k, v, np.ones((1, dk)), np.zeros((1, dk)), wj)
    expect = np.zeros((dv, dk))
    expect[j] = v[0, j] * k[0]
    np.testing.assert_allclose(S, expect, rtol=1e-15)


def test_decay_acts_before_the_edit():
    # k = (1, 1)/sqrt 2, b = 1, no write: decay first gives S0 diag(a) (I - k k^T); editing
    # first would give S0 (I - k k^T) diag(a), decaying value rows diag(a) S0 (I - k k^T)
    a = np.array([[0.5, 0.25]])
    k = np.array([[1.0, 1.0]]) / np.sqrt(2)
    S0 = np.array([[1.0, 2.0], [3.0, 4.0]])
    _, S = oracle.gdn2_recurrent(None, k, np.zeros((1, 2)), a, np.ones((1, 2)), np.zeros((1, 2)), S0=S0)
    P = np.array([[0.5, -0.5], [-0.5, 0.5]])
    np.testing.assert_allclose(S, S0 @ np.diag(a[0]) @ P, rtol=1e-15, atol=1e-15)
    assert np.abs(S0 @ P @ np.diag(a[0]) - S).max() > 0.1 and np.abs(np.diag(a[0]) @ S0 @ P - S).max() > 0.1


def test_chunk_maps_are_exact():
    # composing the chunk maps from S0 reproduces the token recurrence's final state, and
    # the routed outputs with states from the maps reproduce the token outputs
    rng = np.random.default_rng(6)
    T, dk, dv, C = 29, 6, 4, 8
    q, k, v, alpha, b, w = _seq(rng, T, dk, dv)
    S0 = rng.standard_normal((dv, dk))
    o_ref, S_ref = oracle.gdn2_recurrent(q, k, v, alpha, b, w, S0=S0)
    A, B = oracle.gdn2_chunk_transitions(k, v, alpha, b, w, C)
    S = S0
    starts = []
    for i in range(A.shape[0]):
        starts.append(S)
        S = S @ A[i] + B[i]
    np.testing.assert_allclose(S, S_ref, rtol=1e-11, atol=1e-12)
    o = oracle.gdn2_routed_outputs(q, k, v, alpha, b, w, C, np.stack(starts))
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-12)


def test_routed_prefill_with_all_gates_one_is_the_recurrence():
    # caller gates of one on every history chunk compose every map: the native recurrence
    rng = np.random.default_rng(7)
    T, dk, dv, C = 26, 5, 3, 8
    q, k, v, alpha, b, w = _seq(rng, T, dk, dv)
    N = -(-T // C)
    r = oracle.gdn2_hla_prefill(q, k, v, alpha, b, w, C, 0.5, gates_in=np.ones((N, N)))
    o_ref, _ = oracle.gdn2_recurrent(q, k, v, alpha, b, w)
    np.testing.assert_allclose(r["o"], o_ref, rtol=1e-11, atol=1e-12)


def test_decode_step_collapses_and_follows_the_recurrence():
    rng = np.random.default_rng(8)
    dk, dv, Nc = 6, 4, 3
    q, k, v, alpha, b, w = _seq(rng, 1, dk, dv)
    B0 = rng.standard_normal((dv, dk))
    A0 = np.eye(dk) + 0.1 * rng.standard_normal((dk, dk))
    cA, cB = 0.5 * rng.standard_normal((Nc, dk, dk)), rng.standard_normal((Nc, dv, dk))
    reps = rng.standard_normal((Nc, 2, dk))
    # native: the live state follows the token recurrence
    r = oracle.gdn2_decode_step(q[0], k[0], v[0], alpha[0], b[0], w[0], B0, None, None, None, None, 0.0)
    o_ref, S_ref = oracle.gdn2_recurrent(q, k, v, alpha, b, w, S0=B0)
    np.testing.assert_allclose(r["B_cur"], S_ref, rtol=1e-13)
    np.testing.assert_allclose(r["o"], o_ref[0], rtol=1e-13)
    # collapsed gates: Gated DeltaNet's decode step, routed read included
    be, al = 0.6, 0.8
    r2 = oracle.gdn2_decode_step(q[0], k[0], v[0], np.full(dk, al), np.full(dk, be), np.full(dv, be), B0, A0,
                                 cA, cB, reps, 0.3)
    r1 = oracle.decode_step(q[0], k[0], v[0], be, al, B0, A0, cA, cB, reps, 0.3)
    for key in ("o", "B_cur", "A_cur", "gates"):
        np.testing.assert_allclose(r2[key], r1[key], rtol=1e-12, atol=1e-14)
