"""Oracle for the Gated DeltaNet-2 recurrence (float64 numpy).  Test infrastructure only.

[GDN2] the Gated DeltaNet-2 abstract, reproduced on the thelatestinai.com pages: the state
keeps Gated DeltaNet's adaptive forgetting but decays per key channel (as Kimi Delta
Attention does), and the single scalar of the delta edit is split into a channel-wise erase
gate b_t on the key side and a channel-wise write gate w_t on the value side.  With b_t and
w_t equal to one scalar it is Kimi Delta Attention; when the decay is one scalar too it is
Gated DeltaNet.

Reading taken here (the pages give no formula): with the math state S [dv, dk] and
alpha_t, b_t in (0, 1)^dk, w_t in (0, 1)^dv, token t does
    S' = S diag(alpha_t)                        (channel-wise decay of the key channels)
    S  = S' - (S' k_t) (b_t o k_t)^T + (w_t o v_t) k_t^T,      o_t = S q_t
i.e. the read S' k_t is erased from key channel c in proportion to b_t[c] k_t[c], and the
write is gated per value channel.  Each token is affine in S, so a chunk is one exact
affine map S -> S A + B ([HLA] Methodology paragraph 1), which HLA composes unchanged.
"""
from __future__ import annotations

import numpy as np

from .gdn import chunk_bounds, decode_read, routed_states, router_gates


def gdn2_recurrent(q, k, v, alpha, b, w, S0=None):
    """Token by token.  q, k [T, dk], v [T, dv], alpha, b [T, dk], w [T, dv]; q may be None.
    Returns (o [T, dv] or None, S_final [dv, dk])."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64, copy=True)
    o = None if q is None else np.zeros((T, dv))
    for t in range(T):
        Sd = S * alpha[t][None, :]
        S = Sd - np.outer(Sd @ k[t], b[t] * k[t]) + np.outer(w[t] * v[t], k[t])
        if q is not None:
            o[t] = S @ q[t]
    return o, S


def gdn2_chunk_transition(k, v, alpha, b, w):
    """Exact affine map (A [dk, dk], B [dv, dk]) of one chunk, built token by token:
    A <- A diag(alpha_t) (I - k_t (b_t o k_t)^T), and B is the chunk's state from zero."""
    dk = k.shape[1]
    A = np.eye(dk)
    for t in range(k.shape[0]):
        Ad = A * alpha[t][None, :]
        A = Ad - np.outer(Ad @ k[t], b[t] * k[t])
    _, B = gdn2_recurrent(None, k, v, alpha, b, w)
    return A, B


def gdn2_chunk_transitions(k, v, alpha, b, w, C):
    """(A [N, dk, dk], B [N, dv, dk]) for every chunk of one (batch, head) sequence."""
    A, B = [], []
    for s, e in chunk_bounds(k.shape[0], C):
        a_, b_ = gdn2_chunk_transition(k[s:e], v[s:e], alpha[s:e], b[s:e], w[s:e])
        A.append(a_)
        B.append(b_)
    return np.stack(A), np.stack(B)


def gdn2_routed_outputs(q, k, v, alpha, b, w, C, S_routed):
    """Outputs when chunk i starts from S_routed[i] and runs its own tokens."""
    o = np.zeros((k.shape[0], v.shape[1]))
    for i, (s, e) in enumerate(chunk_bounds(k.shape[0], C)):
        o[s:e], _ = gdn2_recurrent(q[s:e], k[s:e], v[s:e], alpha[s:e], b[s:e], w[s:e], S0=S_routed[i])
    return o


def gdn2_hla_prefill(q, k, v, alpha, b, w, C, tau, reps=None, n_rep=None, gates_in=None, S0=None, Wr=None):
    """Routed prefill for one (batch, head) under the GDN-2 recurrence: the chunk maps are
    GDN-2's, the router and the gated composition are HLA's, unchanged."""
    if reps is None:
        reps, n_rep = k, C
    A, B = gdn2_chunk_transitions(k, v, alpha, b, w, C)
    r = router_gates(q, reps, n_rep, C, tau, gates_in=gates_in, Wr=Wr)
    S = routed_states(A, B, r["ghat"], r["mask"], S0=S0)
    o = gdn2_routed_outputs(q, k, v, alpha, b, w, C, S)
    return dict(A=A, B=B, S_routed=S, o=o, **r)


def gdn2_decode_step(q, k, v, alpha, b, w, B_cur, A_cur, cache_A, cache_B, cache_reps, tau, gates_in=None,
                     commit=False, Wr=None):
    """One decode step under the GDN-2 recurrence: the live chunk takes the token,
    B_cur <- B_cur diag(alpha)(I - k (b o k)^T) + (w o v) k^T and A_cur likewise without the
    write; the routed read over the cached chunks is HLA's (decode_step)."""
    lin = np.diag(alpha) @ (np.eye(k.shape[0]) - np.outer(k, b * k))
    return decode_read(q, B_cur @ lin + np.outer(w * v, k), None if A_cur is None else A_cur @ lin,
                       cache_A, cache_B, cache_reps, tau, gates_in=gates_in, commit=commit, Wr=Wr)
