"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This module only draws and rounds numbers.  It contains none of the gated
delta rule or HLA arithmetic, so both the HIP path and the CPU oracle can take
their inputs from it without sharing any computation.

Recipe (every draw uses numpy's PCG64 through ``default_rng``):

* every tensor is drawn per (tensor, batch row b, head h, 4096-token segment)
  from ``default_rng([seed, stream, tensor_id, b, h, segment])``, so any slice
  can be regenerated on its own (sampled parity checks, suffix replays);
* q, k ~ N(0, 1) drawn in float32, L2-normalised per token in float64; v ~ N(0, 1);
* beta = sigmoid(x), x ~ N(0, 1);
* alpha = exp(-softplus(x + 2)), x ~ N(0, 1) (the "slow" variant uses x - 3,
  median alpha ~ 0.95, which keeps chunk transitions far from zero);
* optional planted signal: v of every token with (t + 1) % period == 0 is
  multiplied by a scale (x8 for the long-context routed workload) before rounding;
* q, k, v are then rounded to the storage dtype: float32, or bfloat16 by
  round-to-nearest-even from the float32 value; beta and alpha are float32.

Storage arrays are what the GPU receives: ``uint16`` bit patterns for bf16 and
``float32`` for fp32.  ``to_f64`` widens them exactly for the oracle.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEGMENT = 4096
_TENSOR_ID = {"q": 1, "k": 2, "v": 3, "beta": 4, "alpha": 5, "gates": 6, "At": 7, "Bc": 8, "S0": 9,
              "Wq": 10, "Wk": 11, "Wv": 12, "Wp": 13, "Wr": 14, "ga": 15, "gb": 16, "gw": 17,
              "dO": 18, "dS": 19, "dreps": 20, "dgates": 21}


# --------------------------------------------------------------------------- rounding
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to the storage dtype ('bf16' -> uint16 bits, 'f32' -> float32)."""
    x32 = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exactly widen a storage array to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def round_values(x: np.ndarray, dtype: str) -> np.ndarray:
    """float64 values exactly representable in ``dtype`` (round-trip through storage)."""
    return to_f64(to_storage(x, dtype), dtype)


# --------------------------------------------------------------------------- draws
def _rng(seed: int, stream: int, tensor: str, *idx: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), _TENSOR_ID[tensor], *[int(i) for i in idx]])


def _normal_rows(seed, stream, tensor, b, h, t0, t1, width):
    """Normals for tokens [t0, t1) of (b, h), width values per token (float32)."""
    out = np.empty((t1 - t0, width) if width else (t1 - t0,), dtype=np.float32)
    s_first, s_last = t0 // SEGMENT, (t1 - 1) // SEGMENT
    pos = 0
    for s in range(s_first, s_last + 1):
        seg_lo = s * SEGMENT
        n_seg = SEGMENT  # a segment is always drawn whole so slices agree with full draws
        shape = (n_seg, width) if width else (n_seg,)
        seg = _rng(seed, stream, tensor, b, h, s).standard_normal(shape, dtype=np.float32)
        lo, hi = max(t0, seg_lo) - seg_lo, min(t1, seg_lo + n_seg) - seg_lo
        out[pos:pos + hi - lo] = seg[lo:hi]
        pos += hi - lo
    return out


def _l2_normalise(x32: np.ndarray) -> np.ndarray:
    x = x32.astype(np.float64)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class TokenInputs:
    """Per-token inputs in storage form, layout [B, T, H, d] and [B, T, H]."""

    dtype: str
    q: np.ndarray | None
    k: np.ndarray
    v: np.ndarray
    beta: np.ndarray
    alpha: np.ndarray
    t0: int = 0
    meta: dict = field(default_factory=dict)

    def f64(self, name: str) -> np.ndarray:
        x = getattr(self, name)
        if name in ("beta", "alpha"):
            return np.asarray(x, dtype=np.float64)
        return to_f64(x, self.dtype)


def gen_tokens(B, T, H, dk, dv, dtype="bf16", seed=0, stream=0, alpha_mode="config",
               beta_mode="config", plant_period=None, plant_scale=8.0, t_range=None,
               with_q=True, threads=None) -> TokenInputs:
    """Draw q, k, v, beta, alpha for tokens ``t_range`` (default [0, T)) of a [B, T, H] batch.

    Tokens are indexed by their absolute position t, so a suffix drawn alone equals the same
    suffix of a full draw.
    """
    t0, t1 = (0, T) if t_range is None else t_range
    assert 0 <= t0 < t1 <= T
    n = t1 - t0
    sd = np.uint16 if dtype == "bf16" else np.float32
    q = np.empty((B, n, H, dk), dtype=sd) if with_q else None
    k = np.empty((B, n, H, dk), dtype=sd)
    v = np.empty((B, n, H, dv), dtype=sd)
    beta = np.empty((B, n, H), dtype=np.float32)
    alpha = np.empty((B, n, H), dtype=np.float32)
    tpos = np.arange(t0, t1)

    def one(bh):
        b, h = bh
        if with_q:
            q[b, :, h] = to_storage(_l2_normalise(_normal_rows(seed, stream, "q", b, h, t0, t1, dk)), dtype)
        k[b, :, h] = to_storage(_l2_normalise(_normal_rows(seed, stream, "k", b, h, t0, t1, dk)), dtype)
        vv = _normal_rows(seed, stream, "v", b, h, t0, t1, dv).astype(np.float64)
        if plant_period:
            vv[(tpos + 1) % plant_period == 0] *= plant_scale
        v[b, :, h] = to_storage(vv, dtype)
        xb = _normal_rows(seed, stream, "beta", b, h, t0, t1, 0).astype(np.float64)
        xa = _normal_rows(seed, stream, "alpha", b, h, t0, t1, 0).astype(np.float64)
        if beta_mode == "config":
            bb = _sigmoid(xb)
        elif beta_mode == "zero":
            bb = np.zeros_like(xb)
        elif beta_mode == "one":
            bb = np.ones_like(xb)
        else:
            raise ValueError(beta_mode)
        if alpha_mode == "config":
            aa = np.exp(-_softplus(xa + 2.0))
        elif alpha_mode == "slow":
            aa = np.exp(-_softplus(xa - 3.0))
        elif alpha_mode == "one":
            aa = np.ones_like(xa)
        else:
            raise ValueError(alpha_mode)
        beta[b, :, h] = bb.astype(np.float32)
        alpha[b, :, h] = aa.astype(np.float32)

    pairs = [(b, h) for b in range(B) for h in range(H)]
    nthreads = threads or min(16, max(1, len(pairs)))
    if nthreads > 1 and len(pairs) > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one, pairs))
    else:
        for p in pairs:
            one(p)
    return TokenInputs(dtype=dtype, q=q, k=k, v=v, beta=beta, alpha=alpha, t0=t0,
                       meta=dict(B=B, T=T, H=H, dk=dk, dv=dv, seed=seed, stream=stream,
                                 alpha_mode=alpha_mode, beta_mode=beta_mode))


def gen_decode_tokens(Bs, H, dk, dv, step, dtype="bf16", seed=0, stream=7, alpha_mode="config"):
    """One token per sequence for decode step ``step``: q, k, v [Bs, H, d], beta, alpha [Bs, H]."""
    rng = np.random.default_rng([seed, stream, 100, int(step)])
    q = _l2_normalise(rng.standard_normal((Bs, H, dk), dtype=np.float32))
    k = _l2_normalise(rng.standard_normal((Bs, H, dk), dtype=np.float32))
    v = rng.standard_normal((Bs, H, dv), dtype=np.float32).astype(np.float64)
    xb = rng.standard_normal((Bs, H), dtype=np.float32).astype(np.float64)
    xa = rng.standard_normal((Bs, H), dtype=np.float32).astype(np.float64)
    shift = 2.0 if alpha_mode == "config" else -3.0
    return dict(q=to_storage(q, dtype), k=to_storage(k, dtype), v=to_storage(v, dtype),
                beta=_sigmoid(xb).astype(np.float32),
                alpha=np.exp(-_softplus(xa + shift)).astype(np.float32))


def gen_gdn2_decode_gates(Bs, H, dk, dv, step, seed=0, stream=7, alpha_mode="config") -> dict:
    """Gated DeltaNet-2 gates of one decode token per sequence: a, b [Bs, H, dk] and
    w [Bs, H, dv], float32, with the distributions of gen_gdn2_gates."""
    rng = np.random.default_rng([seed, stream, 101, int(step)])
    shift = -3.0 if alpha_mode == "slow" else 2.0
    xa = rng.standard_normal((Bs, H, dk), dtype=np.float32).astype(np.float64)
    xb = rng.standard_normal((Bs, H, dk), dtype=np.float32).astype(np.float64)
    xw = rng.standard_normal((Bs, H, dv), dtype=np.float32).astype(np.float64)
    return dict(a=np.exp(-_softplus(xa + shift)).astype(np.float32), b=_sigmoid(xb).astype(np.float32),
                w=_sigmoid(xw).astype(np.float32))


def gen_gates(B, H, N, seed=0, stream=0, mode="skip_heavy") -> np.ndarray:
    """Caller-supplied gates [B, H, N, N] float32 (only entries j < i are read)."""
    rng = _rng(seed, stream, "gates", B, H, N)
    if mode == "skip_heavy":
        g = _sigmoid(rng.normal(-4.0, 3.0, size=(B, H, N, N)))
    elif mode == "uniform":
        g = rng.uniform(0.0, 1.0, size=(B, H, N, N))
    elif mode == "binary":
        g = (rng.uniform(size=(B, H, N, N)) < 0.5).astype(np.float64)
    else:
        raise ValueError(mode)
    return g.astype(np.float32)


def gen_transitions(B, H, N, dk, dv, dtype="bf16", seed=0, stream=0, norm=0.95, b_scale=0.3):
    """Random chunk transitions in state orientation: At [B,H,N,dk,dk] with spectral norm
    ``norm`` and Bc [B,H,N,dk,dv], rounded to ``dtype`` (storage form)."""
    rng = _rng(seed, stream, "At", B, H, N, dk)
    G = rng.standard_normal((B, H, N, dk, dk))
    s = np.linalg.norm(G, ord=2, axis=(-2, -1))
    At = G * (norm / s)[..., None, None]
    rng2 = _rng(seed, stream, "Bc", B, H, N, dv)
    Bc = b_scale * rng2.standard_normal((B, H, N, dk, dv))
    return to_storage(At, dtype), to_storage(Bc, dtype)


def gen_pooler_weights(H, dk, dtype="bf16", seed=0, stream=0, shared=False, qk_scale=1.0, r_scale=None) -> dict:
    """Seeded weights of the chunk-representative pooler and the router query projection,
    each [H, dk, dk] (or [1, dk, dk] when ``shared``) in storage form, layout [out, in].
    Wq, Wk ~ N(0, qk_scale^2), so the window's attention scores are of order one; Wv, Wp
    ~ N(0, 1 / dk), so they roughly preserve vector norms; Wr ~ N(0, r_scale^2) (default
    1 / sqrt(dk)); a large r_scale spreads the router's gates away from one half."""
    nh = 1 if shared else H
    out = {}
    for name in ("Wq", "Wk", "Wv", "Wp", "Wr"):
        rng = _rng(seed, stream, name, nh, dk)
        sd = qk_scale if name in ("Wq", "Wk") else 1.0 / math.sqrt(dk)
        if name == "Wr" and r_scale is not None:
            sd = r_scale
        out[name] = to_storage(sd * rng.standard_normal((nh, dk, dk)), dtype)
    return out


def gen_gdn2_gates(B, T, H, dk, dv, seed=0, stream=0, alpha_mode="config", t_range=None) -> dict:
    """Per-token, per-channel gates of the Gated DeltaNet-2 recurrence, float32:
    a [B, T, H, dk] = exp(-softplus(x + 2)) (the "slow" variant x - 3), b [B, T, H, dk] =
    sigmoid(x) and w [B, T, H, dv] = sigmoid(x), x ~ N(0, 1) drawn per (tensor, b, h,
    4096-token segment) like the token tensors, so any token range regenerates alone."""
    t0, t1 = (0, T) if t_range is None else t_range
    shift = -3.0 if alpha_mode == "slow" else 2.0
    out = {n: np.empty((B, t1 - t0, H, wdt), np.float32) for n, wdt in (("a", dk), ("b", dk), ("w", dv))}
    for b in range(B):
        for h in range(H):
            out["a"][b, :, h] = np.exp(-_softplus(_normal_rows(seed, stream, "ga", b, h, t0, t1, dk).astype(np.float64)
                                                  + shift))
            out["b"][b, :, h] = _sigmoid(_normal_rows(seed, stream, "gb", b, h, t0, t1, dk).astype(np.float64))
            out["w"][b, :, h] = _sigmoid(_normal_rows(seed, stream, "gw", b, h, t0, t1, dv).astype(np.float64))
    return out


def gen_state(B, H, dk, dv, seed=0, stream=0, scale=0.5) -> np.ndarray:
    """A float32 initial state [B, H, dk, dv] (state orientation)."""
    rng = _rng(seed, stream, "S0", B, H, dk, dv)
    return (scale * rng.standard_normal((B, H, dk, dv))).astype(np.float32)


def gen_cotangent(shape, seed=0, stream=0, name="dO", scale=1.0) -> np.ndarray:
    """A seeded upstream gradient (a random direction for a vector-Jacobian product):
    float32 N(0, scale^2) of the given shape."""
    rng = _rng(seed, stream, name, *shape)
    return (scale * rng.standard_normal(tuple(shape))).astype(np.float32)


# --------------------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    C: int
    dtype: str
    tau: float = 1e-3
    plant_period: int | None = None
    replay: int | None = None     # Tail-Replay suffix length
    decode_steps: int | None = None
    n_cache: int | None = None    # cached chunks per sequence (decode)

    @property
    def N(self) -> int:
        return math.ceil(self.T / self.C)


WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=256, H=1, dk=64, dv=64, C=64, dtype="f32"),
    "native_prefill": Workload("native_prefill", B=4, T=4096, H=16, dk=128, dv=128, C=64, dtype="bf16"),
    "routed_prefill": Workload("routed_prefill", B=1, T=32768, H=16, dk=128, dv=128, C=64, dtype="bf16",
                               plant_period=4096),
    "decode": Workload("decode", B=256, T=64 * 64, H=16, dk=128, dv=128, C=64, dtype="bf16",
                       decode_steps=512, n_cache=64),
    "tail_replay": Workload("tail_replay", B=8, T=32768, H=16, dk=128, dv=128, C=64, dtype="bf16",
                            replay=math.ceil(0.1 * 32768)),
}

# distinct seed streams per workload keep their draws independent
STREAM = {"tiny": 0, "native_prefill": 1, "routed_prefill": 2, "decode": 3, "tail_replay": 4}
