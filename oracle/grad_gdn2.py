"""Oracle for the backward pass of the Gated DeltaNet-2 routed prefill (float64).  Test
infrastructure only.

What is differentiated is exactly the forward that ``oracle.gdn2`` states, restated here in
float64 PyTorch CPU ops so that reverse-mode automatic differentiation (torch.autograd, a
library routine) can take its gradient.  [GDN2] the Gated DeltaNet-2 abstract: channel-wise
decay a_t, a channel-wise erase gate b_t on the key side and a channel-wise write gate w_t
on the value side.  The reading of ``oracle.gdn2`` (the pages print no formula): with the
math state S [dv, dk], token t does
    S' = S diag(a_t),   S = S' - (S' k_t)(b_t o k_t)^T + (w_t o v_t) k_t^T,   o_t = S q_t;
each chunk's exact affine map S -> S A + B is the same tokens applied to the identity and
to zero ([HLA] Methodology paragraph 1), and the router and the gated composition are
Gated DeltaNet's, unchanged ([HLA] Methodology paragraphs 2-4).

Orientation as in ``oracle.gdn2``: S [dv, dk], A [dk, dk], B [dv, dk], a and b [T, dk],
w [T, dv].  Every function takes and returns float64 numpy arrays.

Pinned by tests/test_oracle_grad_gdn2_pins.py: central finite differences of the numpy
forward oracle (separate code), the collapse to the Gated DeltaNet gradient oracle when
the gates are scalars (a = alpha, b = w = beta on every channel), and the closed form of
one token.
"""
from __future__ import annotations

import numpy as np
import torch

from .gdn import chunk_bounds, router_gates
from .grad import _compose, _grads, _history_gates, _np, _t

_F = torch.float64


def _recurrent(q, k, v, a, b, w, S):
    """Token by token from state S; returns (o [T, dv] or None, S_end)."""
    outs = []
    for t in range(k.shape[0]):
        Sd = S * a[t][None, :]
        S = Sd - torch.outer(Sd @ k[t], b[t] * k[t]) + torch.outer(w[t] * v[t], k[t])
        if q is not None:
            outs.append(S @ q[t])
    return (torch.stack(outs) if q is not None else None), S


def _chunk_map(k, v, a, b, w):
    """(A, B) of one chunk: the tokens applied to the identity (no write) and to zero."""
    dk, dv = k.shape[1], v.shape[1]
    A = torch.eye(dk, dtype=_F)
    for t in range(k.shape[0]):
        Ad = A * a[t][None, :]
        A = Ad - torch.outer(Ad @ k[t], b[t] * k[t])
    _, B = _recurrent(None, k, v, a, b, w, torch.zeros((dv, dk), dtype=_F))
    return A, B


def _chunk_outputs(q, k, v, a, b, w, C, S_routed):
    o = []
    for i, (s, e) in enumerate(chunk_bounds(q.shape[0], C)):
        oi, _ = _recurrent(q[s:e], k[s:e], v[s:e], a[s:e], b[s:e], w[s:e], S_routed[i])
        o.append(oi)
    return torch.cat(o)


_NAMES = ("dq", "dk", "dv", "da", "db", "dw")


def gdn2_chunk_outputs_backward(q, k, v, a, b, w, C, S_routed, dO):
    """Reverse of ``oracle.gdn2.gdn2_routed_outputs``: upstream dO [T, dv] ->
    dict(dq, dk, dv, da, db, dw, dS_routed [N, dv, dk])."""
    xs = (q, k, v, a, b, w, S_routed)
    ts = [_t(x, True) for x in xs]
    o = _chunk_outputs(*ts[:6], C, ts[6])
    g = _grads(o, ts, _t(dO))
    return {n: _np(gi, x) for n, gi, x in zip(_NAMES + ("dS_routed",), g, xs)}


def gdn2_chunk_transitions_backward(k, v, a, b, w, C, dA, dB):
    """Reverse of ``oracle.gdn2.gdn2_chunk_transitions``: upstream dA [N, dk, dk],
    dB [N, dv, dk] -> dict(dk, dv, da, db, dw)."""
    xs = (k, v, a, b, w)
    ts = [_t(x, True) for x in xs]
    As, Bs = [], []
    for s, e in chunk_bounds(k.shape[0], C):
        A_, B_ = _chunk_map(*(t[s:e] for t in ts))
        As.append(A_)
        Bs.append(B_)
    out = torch.cat([torch.stack(As).reshape(-1), torch.stack(Bs).reshape(-1)])
    seed = torch.cat([_t(dA).reshape(-1), _t(dB).reshape(-1)])
    g = _grads(out, ts, seed)
    return {n: _np(gi, x) for n, gi, x in zip(_NAMES[1:], g, xs)}


def gdn2_hla_prefill_backward(q, k, v, a, b, w, C, tau, dO, S0=None, gates_in=None):
    """Gradients of sum(dO * o) for the Gated DeltaNet-2 routed prefill of one (batch,
    head) with raw-key representatives (n_rep = C), through the token recurrence, the chunk
    maps, the gated composition and the router, in one autograd graph.

    Returns dict(dq, dk, dv, da, db, dw, dS0, dgates, mask); the skip mask is the float32
    decision of ``oracle.gdn.router_gates``, held fixed (a skipped pair passes no gradient),
    and with ``gates_in`` the caller's gates receive dgates and the router is not part of
    the graph."""
    T, dk = np.shape(k)
    dv = np.shape(v)[1]
    fw = router_gates(np.asarray(q, np.float64), np.asarray(k, np.float64), C, C, tau, gates_in=gates_in)
    mask = fw["mask"]
    xs = (q, k, v, a, b, w)
    ts = [_t(x, True) for x in xs]
    qt, kt, vt, at, bt, wt = ts
    S0t = _t(np.zeros((dv, dk)) if S0 is None else S0, True)
    if gates_in is None:
        g = _history_gates(qt, kt, C, C)
        if g.requires_grad:  # a single chunk has no history gates
            g.retain_grad()
        leaf_g = g
    else:
        leaf_g = _t(np.tril(np.asarray(gates_in, np.float64), -1), True)
        g = leaf_g
    As, Bs = [], []
    for s, e in chunk_bounds(T, C):
        A_, B_ = _chunk_map(kt[s:e], vt[s:e], at[s:e], bt[s:e], wt[s:e])
        As.append(A_)
        Bs.append(B_)
    S = _compose(As, Bs, g, mask, S0t)
    o = _chunk_outputs(qt, kt, vt, at, bt, wt, C, S)
    (o * _t(dO)).sum().backward()
    out = {n: _np(x.grad, y) for n, x, y in zip(_NAMES, ts, xs)}
    out["dS0"] = _np(S0t.grad, np.zeros((dv, dk)))
    N = len(Bs)
    dg = _np(leaf_g.grad, np.zeros((N, N))) if leaf_g.requires_grad else np.zeros((N, N))
    out["dgates"] = np.where(mask, dg, 0.0)
    out["mask"] = mask
    return out
