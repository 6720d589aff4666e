"""Oracle for the backward pass of the learned representatives (float64).  Test
infrastructure only.

What is differentiated is exactly ``oracle.gdn.window_reps``, restated here in float64
PyTorch CPU ops so that reverse-mode automatic differentiation (torch.autograd, a library
routine) can take its gradient.  [HLA] Methodology paragraph 2: each chunk is cut into
pooling windows; inside a window the keys X [n, dk] attend to one another,
    Q = X Wq^T,  K = X Wk^T,  V = X Wv^T,  P = row-softmax(Q K^T / sqrt(dk)),  O = P V,
the n output rows are mean-pooled and projected, rep = Wp mean(O).  With the router's
query projection Wr [dk, dk] folded in (as the library's representatives carry it), a
representative row is rep Wr, so that qbar Wr^T . rep = qbar . (rep Wr); weights are
[out, in] as in ``oracle.gdn``.  A window with no tokens gives a zero row (no gradient).

Pinned by tests/test_oracle_grad_reps_pins.py: central finite differences of the numpy
forward oracle (separate code) for every input, and the one-token window's closed form.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .gdn import chunk_bounds
from .grad import _grads, _np, _t


def _window_rep(X, Wq, Wk, Wv, Wp):
    n, dk = X.shape
    Q, K, V = X @ Wq.T, X @ Wk.T, X @ Wv.T
    P = torch.softmax(Q @ K.T / math.sqrt(dk), dim=1)
    return Wp @ (P @ V).mean(dim=0)


def window_reps_backward(k, C, window, Wq, Wk, Wv, Wp, dreps, Wr=None):
    """Reverse of ``oracle.gdn.window_reps`` (then times Wr when given) for one (batch,
    head) sequence: upstream dreps [N * C / window, dk] -> dict(dk [T, dk], dWq, dWk, dWv,
    dWp, dWr (None without Wr))."""
    T, dk = np.shape(k)
    n_rep = C // window
    xs = [k, Wq, Wk, Wv, Wp] + ([Wr] if Wr is not None else [])
    ts = [_t(x, True) for x in xs]
    kt, Wqt, Wkt, Wvt, Wpt = ts[:5]
    rows = []
    for c, (s, e) in enumerate(chunk_bounds(T, C)):
        for w in range(n_rep):
            lo, hi = s + w * window, min(s + (w + 1) * window, e)
            rows.append(_window_rep(kt[lo:hi], Wqt, Wkt, Wvt, Wpt) if hi > lo else torch.zeros(dk, dtype=kt.dtype))
    reps = torch.stack(rows)
    if Wr is not None:
        reps = reps @ ts[5]
    g = _grads(reps, ts, _t(dreps))
    out = {n: _np(gi, x) for n, gi, x in zip(("dk", "dWq", "dWk", "dWv", "dWp", "dWr"), g, xs)}
    out.setdefault("dWr", None)
    return out
