"""Oracle for the backward pass of the routed prefill (float64).  Test infrastructure only.

What is differentiated is exactly the forward that ``oracle.gdn`` states, restated here in
float64 PyTorch CPU ops so that reverse-mode automatic differentiation (torch.autograd, a
library routine) can take its gradient:

* the gated delta rule token by token, S <- alpha_t S (I - beta_t k_t k_t^T) +
  beta_t v_t k_t^T and o_t = S q_t ([HLA] Methodology paragraph 1);
* each chunk's exact affine map S -> S A + B built token by token ([HLA] Methodology
  paragraph 1, Key Contributions 2);
* the router: qbar_i = mean of q over chunk i, l_ij = log-mean-exp over chunk j's keys of
  qbar_i . r / sqrt(dk), g_ij = sigmoid(l_ij) for j < i ([HLA] Overview, Methodology
  paragraph 2);
* the gated chronological composition S -> g (S A_j + B_j) + (1 - g) S over the active
  history chunks ([HLA] Methodology paragraphs 3 and 4);
* each chunk's outputs: its own tokens run from its routed state.

The skip decision g < tau is a step function of g.  Its derivative is zero almost
everywhere, so a skipped pair passes no gradient, and an active pair's gate receives the
composition's.  The mask is taken from ``oracle.gdn.router_gates`` (the float32 decision)
and held fixed.

Orientation as in ``oracle.gdn``: S [dv, dk], A [dk, dk], B [dv, dk], all per (batch,
head) sequence.  Every function takes and returns float64 numpy arrays.

Pinned by tests/test_oracle_grad_pins.py: central finite differences of the numpy
forward oracle (separate code) and closed forms of one-token sequences.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .gdn import chunk_bounds, router_gates

_F = torch.float64


def _t(x, grad=False):
    t = torch.tensor(np.asarray(x, np.float64), dtype=_F)
    return t.requires_grad_(grad)


def _np(x, like=None):
    if x is None:
        return np.zeros(like.shape) if like is not None else None
    return x.detach().numpy().copy()


# ----------------------------------------------------------------------------- forward in torch
def _recurrent(q, k, v, beta, alpha, S):
    """Token-by-token gated delta rule from state S; returns (o [T, dv] or None, S_end)."""
    outs = []
    for t in range(k.shape[0]):
        Sk = S @ k[t]
        S = alpha[t] * (S - beta[t] * torch.outer(Sk, k[t])) + beta[t] * torch.outer(v[t], k[t])
        if q is not None:
            outs.append(S @ q[t])
    return (torch.stack(outs) if q is not None else None), S


def _chunk_map(k, v, beta, alpha):
    """(A, B) of one chunk: the product of the per-token linear parts in token order, and
    the chunk's state from zero."""
    dk, dv = k.shape[1], v.shape[1]
    A = torch.eye(dk, dtype=_F)
    for t in range(k.shape[0]):
        A = alpha[t] * (A - beta[t] * torch.outer(A @ k[t], k[t]))
    _, B = _recurrent(None, k, v, beta, alpha, torch.zeros((dv, dk), dtype=_F))
    return A, B


def _history_gates(q, reps, n_rep, C):
    """g [N, N]: sigmoid of the log-mean-exp pooled scores for j < i, zero elsewhere."""
    T, dk = q.shape
    bounds = chunk_bounds(T, C)
    N = len(bounds)
    qbar = [q[s:e].mean(dim=0) for s, e in bounds]
    rows = []
    for i in range(N):
        row = []
        for j in range(N):
            if j < i:
                s = reps[j * n_rep:(j + 1) * n_rep] @ qbar[i] / math.sqrt(dk)
                row.append(torch.sigmoid(torch.logsumexp(s, 0) - math.log(n_rep)))
            else:
                row.append(torch.zeros((), dtype=_F))
        rows.append(torch.stack(row))
    return torch.stack(rows)


def _compose(A, B, ghat, mask, S0):
    """Routed state of every query chunk: active history chunks applied in time order."""
    N = len(B)
    out = []
    for i in range(N):
        S = S0
        for j in range(i):
            if mask[i, j]:
                S = ghat[i, j] * (S @ A[j] + B[j]) + (1.0 - ghat[i, j]) * S
        out.append(S)
    return out


def _chunk_outputs(q, k, v, beta, alpha, C, S_routed):
    o = []
    for i, (s, e) in enumerate(chunk_bounds(q.shape[0], C)):
        oi, _ = _recurrent(q[s:e], k[s:e], v[s:e], beta[s:e], alpha[s:e], S_routed[i])
        o.append(oi)
    return torch.cat(o)


def _grads(out, inputs, seed):
    """Vector-Jacobian product: gradients of sum(seed * out) w.r.t. inputs (None where the
    output does not depend on an input)."""
    return torch.autograd.grad(out, inputs, grad_outputs=seed, allow_unused=True)


# ----------------------------------------------------------------------------- backward pieces
def routed_states_backward(A, B, ghat, mask, dS, S0=None):
    """Reverse of ``oracle.routed_states``: upstream dS [N, dv, dk] (gradient w.r.t. each
    query chunk's routed state) -> dict(dA [N, dk, dk], dB [N, dv, dk], dghat [N, N]
    (zero on skipped and non-history pairs), dS0 [dv, dk])."""
    N, dv, dk = np.shape(B)
    At, Bt, gt = _t(A, True), _t(B, True), _t(ghat, True)
    S0t = _t(np.zeros((dv, dk)) if S0 is None else S0, True)
    out = torch.stack(_compose(At, Bt, gt, np.asarray(mask, bool), S0t))
    g = _grads(out, (At, Bt, gt, S0t), _t(dS))
    return dict(dA=_np(g[0], A), dB=_np(g[1], B), dghat=_np(g[2], ghat), dS0=_np(g[3], np.zeros((dv, dk))))


def chunk_outputs_backward(q, k, v, beta, alpha, C, S_routed, dO):
    """Reverse of ``oracle.routed_outputs`` (each chunk's tokens from its routed state):
    upstream dO [T, dv] -> dict(dq, dk, dv, dbeta, dalpha, dS_routed [N, dv, dk])."""
    ts = [_t(x, True) for x in (q, k, v, beta, alpha, S_routed)]
    o = _chunk_outputs(*ts[:5], C, ts[5])
    g = _grads(o, ts, _t(dO))
    names = ("dq", "dk", "dv", "dbeta", "dalpha", "dS_routed")
    return {n: _np(gi, x) for n, gi, x in zip(names, g, (q, k, v, beta, alpha, S_routed))}


def chunk_transitions_backward(k, v, beta, alpha, C, dA, dB):
    """Reverse of ``oracle.chunk_transitions``: upstream dA [N, dk, dk], dB [N, dv, dk] ->
    dict(dk, dv, dbeta, dalpha)."""
    ts = [_t(x, True) for x in (k, v, beta, alpha)]
    As, Bs = [], []
    for s, e in chunk_bounds(k.shape[0], C):
        a, b = _chunk_map(ts[0][s:e], ts[1][s:e], ts[2][s:e], ts[3][s:e])
        As.append(a)
        Bs.append(b)
    out = torch.cat([torch.stack(As).reshape(-1), torch.stack(Bs).reshape(-1)])
    seed = torch.cat([_t(dA).reshape(-1), _t(dB).reshape(-1)])
    g = _grads(out, ts, seed)
    return {n: _np(gi, x) for n, gi, x in zip(("dk", "dv", "dbeta", "dalpha"), g, (k, v, beta, alpha))}


def router_backward(q, reps, n_rep, C, dgates):
    """Reverse of the history gates of ``oracle.router_gates`` (raw or given
    representatives, no projection): upstream dgates [N, N] (entries j < i are used) ->
    dict(dq [T, dk], dreps (same shape as reps))."""
    qt, rt = _t(q, True), _t(reps, True)
    g = _history_gates(qt, rt, n_rep, C)
    N = g.shape[0]
    seed = torch.tril(_t(dgates)[:N, :N], -1)
    gq, gr = _grads(g, (qt, rt), seed)
    return dict(dq=_np(gq, q), dreps=_np(gr, reps))


# ----------------------------------------------------------------------------- whole prefill
def hla_prefill_backward(q, k, v, beta, alpha, C, tau, dO, S0=None, gates_in=None):
    """Gradients of sum(dO * o) for the routed prefill of one (batch, head) with raw-key
    representatives (n_rep = C), through the UT-free token recurrence, the chunk maps, the
    gated composition and the router, in one autograd graph.

    Returns dict(dq, dk, dv, dbeta, dalpha, dS0, dgates, mask):
      dgates [N, N] is the gradient w.r.t. the history gate g_ij (zero for skipped pairs);
      with ``gates_in`` the gates are the caller's and receive it, and the router is not
      part of the graph.
    """
    T, dk = np.shape(k)
    dv = np.shape(v)[1]
    fw = router_gates(np.asarray(q, np.float64), np.asarray(k, np.float64), C, C, tau, gates_in=gates_in)
    mask = fw["mask"]
    ts = [_t(x, True) for x in (q, k, v, beta, alpha)]
    qt, kt, vt, bt, at = ts
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
        a, b = _chunk_map(kt[s:e], vt[s:e], bt[s:e], at[s:e])
        As.append(a)
        Bs.append(b)
    S = _compose(As, Bs, g, mask, S0t)
    o = _chunk_outputs(qt, kt, vt, bt, at, C, S)
    (o * _t(dO)).sum().backward()
    out = {n: _np(x.grad, y) for n, x, y in zip(("dq", "dk", "dv", "dbeta", "dalpha"), ts, (q, k, v, beta, alpha))}
    out["dS0"] = _np(S0t.grad, np.zeros((dv, dk)))
    N = len(Bs)
    dg = _np(leaf_g.grad, np.zeros((N, N))) if leaf_g.requires_grad else np.zeros((N, N))
    out["dgates"] = np.where(mask, dg, 0.0)
    out["mask"] = mask
    return out
