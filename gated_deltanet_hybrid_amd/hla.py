"""Thin Python binding of libhla.so (ctypes).

Argument marshalling only: every function checks tensor shapes, dtypes and strides,
then calls the C entry point of the same name with raw device pointers and torch's
current stream.  All arithmetic runs in the HIP kernels; there is no fallback.  Loading
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

# HLA_LIBRARY names another build of the same library (for instance the host-sanitized one)
_LIB_PATH = os.environ.get("HLA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhla.so")
_lib = None

HLA_F32, HLA_BF16 = 0, 1
KERNEL_CHUNK, KERNEL_SCAN, KERNEL_GATES, KERNEL_COMPOSE, KERNEL_DECODE, KERNEL_REPS = 0, 1, 2, 3, 4, 5
KERNEL_BWD_SAVE, KERNEL_BWD_ADJOINT, KERNEL_BWD_REDUCE, KERNEL_BWD_CHUNK, KERNEL_BWD_ROUTER = 6, 7, 8, 9, 10
KERNEL_PREFILL, KERNEL_BWD_REPS = 11, 12
FN_CHUNK_TRANSITIONS, FN_GDN_PREFILL, FN_ROUTE_MIX, FN_WU_HANDOFF, FN_CHUNK_REPS = 0, 1, 2, 3, 4
FN_COMPOSE_BACKWARD, FN_PREFILL_BACKWARD, FN_CHUNK_BACKWARD = 5, 6, 7
FN_COMPOSE_BACKWARD_MIN, FN_PREFILL_BACKWARD_MIN = 8, 9  # smallest workspaces (history segments)
FN_GDN2_CHUNK_BACKWARD, FN_GDN2_PREFILL_BACKWARD, FN_GDN2_PREFILL_BACKWARD_MIN = 10, 11, 12
FN_ROUTER_BACKWARD, FN_CHUNK_REPS_BACKWARD = 13, 14
CHUNK = 64
MAX_CACHE_SLOTS = 1024
REPS_SCRATCH_BYTES = 32 << 20  # fixed device scratch of chunk_reps_noalloc
ERR_SCRATCH_LIMIT = 9


class HlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {library().hla_status_string(status).decode()} (status {status})")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("ld_T", ctypes.c_int64),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("C", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_P = ctypes.c_void_p
_SIGS = {
    "hla_abi_version": (ctypes.c_int32, []),
    "hla_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "hla_workspace_bytes": (ctypes.c_int32, [ctypes.c_int32, ctypes.POINTER(Dims), ctypes.c_int32,
                                             ctypes.POINTER(ctypes.c_size_t)]),
    "hla_chunk_transitions": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P,
                                               ctypes.c_size_t, _P]),
    "hla_gdn_prefill": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                         ctypes.c_size_t, _P]),
    "hla_gdn2_chunk_transitions": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P,
                                                    ctypes.c_size_t, _P]),
    "hla_gdn2_prefill": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "hla_chunk_reps": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                        ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]),
    "hla_chunk_reps_noalloc": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                                ctypes.c_int64, _P, _P]),
    "hla_route_mix": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, ctypes.c_int32, ctypes.c_int64, _P, _P, _P,
                                       _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "hla_compose_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
    "hla_chunk_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                            _P, _P, _P, ctypes.c_size_t, _P]),
    "hla_prefill_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P,
                                              _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "hla_gdn2_chunk_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "hla_gdn2_prefill_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                   ctypes.c_size_t, _P]),
    "hla_router_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, _P, ctypes.c_int32, ctypes.c_int64, _P, _P, _P,
                                             _P, _P, ctypes.c_size_t, _P]),
    "hla_chunk_reps_backward": (ctypes.c_int32, [ctypes.POINTER(Dims), _P, ctypes.c_int32, _P, _P, _P, _P, _P,
                                                 ctypes.c_int64, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                                 _P]),
    "hla_timing_enable": (ctypes.c_int32, [ctypes.c_int32]),
    "hla_timing_read": (ctypes.c_int32, [ctypes.c_int32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "hla_gdn_decode": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32, _P,
                                        ctypes.c_int32, _P, ctypes.c_float, _P, _P, ctypes.c_int32, _P]),
    "hla_gdn2_decode": (ctypes.c_int32, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                         _P, ctypes.c_int32, _P, ctypes.c_float, _P, _P, ctypes.c_int32, _P]),
}


def library(path: str | None = None) -> ctypes.CDLL:
    """Load libhla.so (once).  Raises if it is missing: there is no fallback path."""
    global _lib
    if _lib is None:
        p = path or _LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m gated_deltanet_hybrid_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        raise HlaError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HLA_BF16
    if t.dtype == torch.float32:
        return HLA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _token_view(t: torch.Tensor, name: str):
    """[B, T, H, d] tensor whose rows may be a window of a longer allocation.
    Returns (B, T, H, d, ld_T)."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be [B, T, H, d]")
    B, T, H, d = t.shape
    s = t.stride()
    if s[3] != 1 or s[2] != d or s[1] != H * d or s[0] % (H * d) != 0 or s[0] // (H * d) < T:
        raise ValueError(f"{name} must be row-major within a batch row (a token window of [B, ld_T, H, d])")
    return B, T, H, d, s[0] // (H * d)


def _scalar_view(t: torch.Tensor, B, T, H, ld_T, name):
    if t.dtype != torch.float32 or tuple(t.shape) != (B, T, H):
        raise ValueError(f"{name} must be float32 [B, T, H]")
    s = t.stride()
    if s[2] != 1 or s[1] != H or s[0] != ld_T * H:
        raise ValueError(f"{name} must share the token window layout of k")


def _need(t, shape, dtype, name):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def make_dims(B, T, H, ld_T, dk, dv, dtype_code, C=CHUNK) -> Dims:
    return Dims(B, T, H, ld_T, dk, dv, C, dtype_code)


def workspace_bytes(fn: int, dims: Dims, n_rep: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(library().hla_workspace_bytes(fn, ctypes.byref(dims), n_rep, ctypes.byref(out)), "hla_workspace_bytes")
    return out.value


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device) if nbytes else None


def _inputs(k, v, beta, alpha, q=None, C=CHUNK):
    B, T, H, dk, ld_T = _token_view(k, "k")
    Bv, Tv, Hv, dv, ldv = _token_view(v, "v")
    if (Bv, Tv, Hv, ldv) != (B, T, H, ld_T) or v.dtype != k.dtype:
        raise ValueError("v must match k's batch, tokens, heads, row length and dtype")
    if q is not None:
        Bq, Tq, Hq, dq, ldq = _token_view(q, "q")
        if (Bq, Tq, Hq, dq, ldq) != (B, T, H, dk, ld_T) or q.dtype != k.dtype:
            raise ValueError("q must match k")
    _scalar_view(beta, B, T, H, ld_T, "beta")
    _scalar_view(alpha, B, T, H, ld_T, "alpha")
    return make_dims(B, T, H, ld_T, dk, dv, _dtype_code(k), C)


def wu_buffer(k, v, beta, alpha, C=CHUNK):
    """A buffer for the W | U hand-off from chunk_transitions to gdn_prefill (bf16), else None."""
    n = workspace_bytes(FN_WU_HANDOFF, _inputs(k, v, beta, alpha, C=C))
    return torch.empty(n, dtype=torch.uint8, device=k.device) if n else None


def _check_wu(wu, d):
    """The W | U hand-off buffer has no size argument in the C ABI: it must hold
    hla_workspace_bytes(HLA_FN_WU_HANDOFF) bytes on the inputs' device."""
    if wu is None:
        return
    need = workspace_bytes(FN_WU_HANDOFF, d)
    if need == 0:
        return  # float32 takes no hand-off: the library rejects a buffer (HLA_ERR_UNSUPPORTED)
    if wu.dtype != torch.uint8 or not wu.is_cuda or not wu.is_contiguous() or wu.numel() < need:
        raise ValueError(f"wu must be a contiguous CUDA uint8 tensor of at least {need} bytes (see wu_buffer)")


def chunk_transitions(k, v, beta, alpha, At=None, Bc=None, C=CHUNK, ws=None, wu=None):
    """Exact affine map (At, Bc) of every C-token chunk: M_end = At M_start + Bc.
    wu (from wu_buffer) also receives every piece's W | U for a later gdn_prefill."""
    d = _inputs(k, v, beta, alpha, C=C)
    N = math.ceil(d.T / C)
    At = torch.empty((d.B, d.H, N, d.dk, d.dk), dtype=k.dtype, device=k.device) if At is None else At
    Bc = torch.empty((d.B, d.H, N, d.dk, d.dv), dtype=k.dtype, device=k.device) if Bc is None else Bc
    _need(At, (d.B, d.H, N, d.dk, d.dk), k.dtype, "At")
    _need(Bc, (d.B, d.H, N, d.dk, d.dv), k.dtype, "Bc")
    _check_wu(wu, d)
    if ws is None:
        ws = _workspace(workspace_bytes(FN_CHUNK_TRANSITIONS, d), k.device)
    _check(library().hla_chunk_transitions(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(At),
                                           _ptr(Bc), _ptr(wu), _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(k.device)), "hla_chunk_transitions")
    return At, Bc


def gdn_prefill(q, k, v, beta, alpha, S0=None, chunk_init=None, want_o=True, want_state=True, o=None,
                S_final=None, ws=None, C=CHUNK, wu=None):
    """Chunkwise gated delta rule prefill.  Returns (o [B,T,H,dv] or None, S_final or None).
    C is the chunk size of chunk_init (routed mode); native results do not depend on it.
    wu: a buffer chunk_transitions filled from the same inputs, or None."""
    d = _inputs(k, v, beta, alpha, q if want_o else None, C=C)
    N = math.ceil(d.T / C)
    dev = k.device
    if want_o and o is None:
        o = torch.empty((d.B, d.T, d.H, d.dv), dtype=torch.float32, device=dev)
    if not want_o:
        o = None
    if chunk_init is not None:
        want_state = False
    if want_state and S_final is None:
        S_final = torch.empty((d.B, d.H, d.dk, d.dv), dtype=torch.float32, device=dev)
    if not want_state:
        S_final = None
    _need(o, (d.B, d.T, d.H, d.dv), torch.float32, "o")
    _need(S0, (d.B, d.H, d.dk, d.dv), torch.float32, "S0")
    _need(chunk_init, (d.B, d.H, N, d.dk, d.dv), torch.float32, "chunk_init")
    _need(S_final, (d.B, d.H, d.dk, d.dv), torch.float32, "S_final")
    _check_wu(wu, d)
    if ws is None and (chunk_init is None or C != CHUNK):
        ws = _workspace(workspace_bytes(FN_GDN_PREFILL, d), dev)
    _check(library().hla_gdn_prefill(ctypes.byref(d), _ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(beta),
                                     _ptr(alpha), _ptr(S0), _ptr(chunk_init), _ptr(wu), _ptr(o), _ptr(S_final),
                                     _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)), "hla_gdn_prefill")
    return o, S_final


def _gdn2_gates(d, a_decay, b_erase, w_write):
    B, T, H, dk, dv = d.B, d.T, d.H, d.dk, d.dv
    for t, width, name in ((a_decay, dk, "a_decay"), (b_erase, dk, "b_erase"), (w_write, dv, "w_write")):
        Bx, Tx, Hx, dx, ld = _token_view(t, name)
        if (Bx, Tx, Hx, dx, ld) != (B, T, H, width, d.ld_T) or t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32 [B, T, H, {width}] with k's row layout")


def gdn2_chunk_transitions(k, v, a_decay, b_erase, w_write, At=None, Bc=None, C=CHUNK, ws=None):
    """Exact affine maps of every chunk under the Gated DeltaNet-2 recurrence."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    dv = v.shape[-1]
    d = make_dims(B, T, H, ld_T, dk, dv, _dtype_code(k), C)
    _gdn2_gates(d, a_decay, b_erase, w_write)
    N = math.ceil(T / C)
    At = torch.empty((B, H, N, dk, dk), dtype=k.dtype, device=k.device) if At is None else At
    Bc = torch.empty((B, H, N, dk, dv), dtype=k.dtype, device=k.device) if Bc is None else Bc
    _need(At, (B, H, N, dk, dk), k.dtype, "At")
    _need(Bc, (B, H, N, dk, dv), k.dtype, "Bc")
    if ws is None:
        ws = _workspace(workspace_bytes(FN_CHUNK_TRANSITIONS, d), k.device)
    _check(library().hla_gdn2_chunk_transitions(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(a_decay), _ptr(b_erase),
                                                _ptr(w_write), _ptr(At), _ptr(Bc), _ptr(ws),
                                                0 if ws is None else ws.numel(), _stream(k.device)),
           "hla_gdn2_chunk_transitions")
    return At, Bc


def gdn2_prefill(q, k, v, a_decay, b_erase, w_write, S0=None, chunk_init=None, want_o=True, want_state=True,
                 o=None, S_final=None, ws=None, C=CHUNK):
    """Chunkwise Gated DeltaNet-2 prefill (native or routed), as gdn_prefill."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    dv = v.shape[-1]
    d = make_dims(B, T, H, ld_T, dk, dv, _dtype_code(k), C)
    _gdn2_gates(d, a_decay, b_erase, w_write)
    N = math.ceil(T / C)
    dev = k.device
    if want_o and o is None:
        o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    if not want_o:
        o = None
    if chunk_init is not None:
        want_state = False
    if want_state and S_final is None:
        S_final = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if not want_state:
        S_final = None
    _need(o, (B, T, H, dv), torch.float32, "o")
    _need(S0, (B, H, dk, dv), torch.float32, "S0")
    _need(chunk_init, (B, H, N, dk, dv), torch.float32, "chunk_init")
    _need(S_final, (B, H, dk, dv), torch.float32, "S_final")
    if ws is None and (chunk_init is None or C != CHUNK):
        ws = _workspace(workspace_bytes(FN_GDN_PREFILL, d), dev)
    _check(library().hla_gdn2_prefill(ctypes.byref(d), _ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(a_decay),
                                      _ptr(b_erase), _ptr(w_write), _ptr(S0), _ptr(chunk_init), _ptr(o),
                                      _ptr(S_final), _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "hla_gdn2_prefill")
    return o, S_final


def gdn2_hla_prefill(q, k, v, a_decay, b_erase, w_write, tau=1e-3, gates_in=None, S0=None, C=CHUNK):
    """The routed prefill under the Gated DeltaNet-2 recurrence: GDN-2 chunk maps, the HLA
    router and composition unchanged, GDN-2 chunk outputs from the routed states."""
    At, Bc = gdn2_chunk_transitions(k, v, a_decay, b_erase, w_write, C=C)
    r = route_mix(q, k, At, Bc, n_rep=C, tau=tau, S0=S0, gates_in=gates_in, C=C)
    o, _ = gdn2_prefill(q, k, v, a_decay, b_erase, w_write, chunk_init=r["S_routed"], want_state=False, C=C)
    r.update(At=At, Bc=Bc, o=o)
    return r


def chunk_reps(k, W, window=32, C=CHUNK, out=None, ws=None):
    """Learned representatives of every C-token chunk: [B, N * C/window, H, dk] in k's dtype.

    W: dict of Wq, Wk, Wv, Wp and optionally Wr, each [H, dk, dk] or [1, dk, dk] ([out, in],
    k's dtype); Wr (the router's query projection) is folded into the result."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    d = make_dims(B, T, H, ld_T, dk, dk, _dtype_code(k), C)
    N = math.ceil(T / C)
    n_rep = C // window
    ws_ = [W[n] for n in ("Wq", "Wk", "Wv", "Wp")] + ([W["Wr"]] if W.get("Wr") is not None else [])
    nh = ws_[0].shape[0]
    for t in ws_:
        if t.shape != (nh, dk, dk) or nh not in (1, H) or t.dtype != k.dtype or not t.is_contiguous():
            raise ValueError("weights must be contiguous [H or 1, dk, dk] in k's dtype")
    out = torch.empty((B, N * n_rep, H, dk), dtype=k.dtype, device=k.device) if out is None else out
    _need(out, (B, N * n_rep, H, dk), k.dtype, "out")
    if ws is None:
        ws = _workspace(workspace_bytes(FN_CHUNK_REPS, d, n_rep), k.device)
    _check(library().hla_chunk_reps(ctypes.byref(d), _ptr(k), window, _ptr(W["Wq"]), _ptr(W["Wk"]), _ptr(W["Wv"]),
                                    _ptr(W["Wp"]), _ptr(W.get("Wr")), 0 if nh == 1 else dk * dk, _ptr(out),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(k.device)), "hla_chunk_reps")
    return out


def chunk_reps_noalloc(k, W, window=32, C=CHUNK, out=None):
    """chunk_reps for callers that cannot allocate: the library keeps the window means in a
    fixed device array (REPS_SCRATCH_BYTES per GPU) instead of a workspace.  ``out`` may be
    given so that the call allocates nothing on the Python side either."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    d = make_dims(B, T, H, ld_T, dk, dk, _dtype_code(k), C)
    N = math.ceil(T / C)
    n_rep = C // window
    ws_ = [W[n] for n in ("Wq", "Wk", "Wv", "Wp")] + ([W["Wr"]] if W.get("Wr") is not None else [])
    nh = ws_[0].shape[0]
    for t in ws_:
        if t.shape != (nh, dk, dk) or nh not in (1, H) or t.dtype != k.dtype or not t.is_contiguous():
            raise ValueError("weights must be contiguous [H or 1, dk, dk] in k's dtype")
    out = torch.empty((B, N * n_rep, H, dk), dtype=k.dtype, device=k.device) if out is None else out
    _need(out, (B, N * n_rep, H, dk), k.dtype, "out")
    _check(library().hla_chunk_reps_noalloc(ctypes.byref(d), _ptr(k), window, _ptr(W["Wq"]), _ptr(W["Wk"]),
                                            _ptr(W["Wv"]), _ptr(W["Wp"]), _ptr(W.get("Wr")),
                                            0 if nh == 1 else dk * dk, _ptr(out), _stream(k.device)),
           "hla_chunk_reps_noalloc")
    return out


def chunk_reps_backward(k, W, dreps, window=32, C=CHUNK, ws=None):
    """Reverse of chunk_reps: dreps [B, N * C/window, H, dk] float32 (the gradient of its
    output rows) -> dict(dk [B, T, H, dk], dWq, dWk, dWv, dWp, dWr (None without Wr)),
    float32, the weight gradients shaped like the weights ([H or 1, dk, dk])."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    d = make_dims(B, T, H, ld_T, dk, dk, _dtype_code(k), C)
    N = math.ceil(T / C)
    n_rep = C // window
    names = ("Wq", "Wk", "Wv", "Wp") + (("Wr",) if W.get("Wr") is not None else ())
    nh = W["Wq"].shape[0]
    for n in names:
        t = W[n]
        if t.shape != (nh, dk, dk) or nh not in (1, H) or t.dtype != k.dtype or not t.is_contiguous():
            raise ValueError("weights must be contiguous [H or 1, dk, dk] in k's dtype")
    _need(dreps, (B, N * n_rep, H, dk), torch.float32, "dreps")
    f32 = dict(dtype=torch.float32, device=k.device)
    out = {"dk": torch.empty((B, T, H, dk), **f32)}
    for n in ("Wq", "Wk", "Wv", "Wp", "Wr"):
        out["d" + n] = torch.empty((nh, dk, dk), **f32) if n in names else None
    if ws is None:
        ws = _workspace(workspace_bytes(FN_CHUNK_REPS_BACKWARD, d, 1 if "Wr" in names else 0), k.device)
    _check(library().hla_chunk_reps_backward(ctypes.byref(d), _ptr(k), window, _ptr(W["Wq"]), _ptr(W["Wk"]),
                                             _ptr(W["Wv"]), _ptr(W["Wp"]), _ptr(W.get("Wr")),
                                             0 if nh == 1 else dk * dk, _ptr(dreps), _ptr(out["dk"]),
                                             *(_ptr(out["d" + n]) for n in ("Wq", "Wk", "Wv", "Wp", "Wr")),
                                             _ptr(ws), 0 if ws is None else ws.numel(), _stream(k.device)),
           "hla_chunk_reps_backward")
    return out


def router_backward(q, reps, n_rep, gates, dgates, ws=None):
    """Gradients of the history gates (as route_mix computed them from q and reps) to the
    queries and the representatives: dgates [B, H, N, N] float32 -> dict(dq [B, T, H, dk],
    dreps [B, N * n_rep, H, dk]), float32."""
    B, T, H, dk, ld_T = _token_view(q, "q")
    Br, _, Hr, dr, ld_R = _token_view(reps, "reps")
    if (Br, Hr, dr) != (B, H, dk) or reps.dtype != q.dtype:
        raise ValueError("reps must be [B, R, H, dk] in q's dtype")
    d = make_dims(B, T, H, ld_T, dk, dk, _dtype_code(q), CHUNK)
    N = math.ceil(T / CHUNK)
    _need(gates, (B, H, N, N), torch.float32, "gates")
    _need(dgates, (B, H, N, N), torch.float32, "dgates")
    f32 = dict(dtype=torch.float32, device=q.device)
    out = dict(dq=torch.empty((B, T, H, dk), **f32), dreps=torch.empty((B, N * n_rep, H, dk), **f32))
    if ws is None:
        ws = _workspace(workspace_bytes(FN_ROUTER_BACKWARD, d), q.device)
    _check(library().hla_router_backward(ctypes.byref(d), _ptr(q), _ptr(reps), n_rep, ld_R, _ptr(gates),
                                         _ptr(dgates), _ptr(out["dq"]), _ptr(out["dreps"]), _ptr(ws),
                                         0 if ws is None else ws.numel(), _stream(q.device)), "hla_router_backward")
    return out


def route_mix(q, reps, At, Bc, n_rep=CHUNK, tau=1e-3, S0=None, gates_in=None, T=None, out=None, ws=None,
              C=CHUNK):
    """Router gates, skip mask, active lists, n_eff and the routed per-chunk states.

    q [B, T, H, dk] (token window), reps [B, R, H, dk] (token window, chunk j's
    representatives are rows [j n_rep, (j+1) n_rep)), At/Bc from chunk_transitions.
    Returns a dict of gates, mask, active_idx, active_cnt, n_eff, S_routed.
    """
    B, H, N, dk, _ = At.shape
    dv = Bc.shape[-1]
    dev = At.device
    if q is not None:
        Bq, Tq, Hq, dq, ld_T = _token_view(q, "q")
        if (Bq, Hq, dq) != (B, H, dk) or math.ceil(Tq / C) != N:
            raise ValueError("q does not match the transitions")
        T = Tq
    else:
        ld_T = T = T if T is not None else N * C
    ld_R = 0
    if reps is not None:
        Br, Rr, Hr, dr, ld_R = _token_view(reps, "reps")
        if (Br, Hr, dr) != (B, H, dk) or reps.dtype != At.dtype:
            raise ValueError("reps must be [B, R, H, dk] in the transitions' dtype")
    d = make_dims(B, T, H, ld_T, dk, dv, _dtype_code(At), C)
    _need(At, (B, H, N, dk, dk), At.dtype, "At")
    _need(Bc, (B, H, N, dk, dv), At.dtype, "Bc")
    _need(S0, (B, H, dk, dv), torch.float32, "S0")
    _need(gates_in, (B, H, N, N), torch.float32, "gates_in")
    o = out or {}
    gates = o.get("gates") if o.get("gates") is not None else torch.empty((B, H, N, N), dtype=torch.float32, device=dev)
    mask = o.get("mask") if o.get("mask") is not None else torch.empty((B, H, N, N), dtype=torch.uint8, device=dev)
    aidx = o.get("active_idx") if o.get("active_idx") is not None else torch.empty((B, H, N, N), dtype=torch.int32, device=dev)
    acnt = o.get("active_cnt") if o.get("active_cnt") is not None else torch.empty((B, H, N), dtype=torch.int32, device=dev)
    neff = o.get("n_eff") if o.get("n_eff") is not None else torch.empty((B, H, N), dtype=torch.float32, device=dev)
    Sr = o.get("S_routed") if o.get("S_routed") is not None else torch.empty((B, H, N, dk, dv), dtype=torch.float32, device=dev)
    if ws is None:
        ws = _workspace(workspace_bytes(FN_ROUTE_MIX, d, n_rep), dev)
    _check(library().hla_route_mix(ctypes.byref(d), _ptr(q), _ptr(reps), n_rep, ld_R, _ptr(At), _ptr(Bc), _ptr(S0),
                                   _ptr(gates_in), ctypes.c_float(tau), _ptr(gates), _ptr(mask), _ptr(aidx),
                                   _ptr(acnt), _ptr(neff), _ptr(Sr), _ptr(ws), 0 if ws is None else ws.numel(),
                                   _stream(dev)), "hla_route_mix")
    return dict(gates=gates, mask=mask, active_idx=aidx, active_cnt=acnt, n_eff=neff, S_routed=Sr)


def compose_backward(At, Bc, gates, mask, dS_routed, S0=None, want_dS0=True, want_states=False, T=None, C=CHUNK,
                     ws=None):
    """Reverse of the gated composition.  At/Bc as given to route_mix, gates/mask as it
    wrote them, dS_routed [B, H, N, dk, dv] float32.  Returns dict(dAt, dBc, dgates, dS0
    (or None), S_routed (the recomputed routed states, or None))."""
    B, H, N, dk, _ = At.shape
    dv = Bc.shape[-1]
    dev = At.device
    T = T if T is not None else N * C
    d = make_dims(B, T, H, T, dk, dv, _dtype_code(At), C)
    _need(At, (B, H, N, dk, dk), At.dtype, "At")
    _need(Bc, (B, H, N, dk, dv), At.dtype, "Bc")
    _need(gates, (B, H, N, N), torch.float32, "gates")
    _need(mask, (B, H, N, N), torch.uint8, "mask")
    _need(dS_routed, (B, H, N, dk, dv), torch.float32, "dS_routed")
    _need(S0, (B, H, dk, dv), torch.float32, "S0")
    f32 = dict(dtype=torch.float32, device=dev)
    dAt = torch.empty((B, H, N, dk, dk), **f32)
    dBc = torch.empty((B, H, N, dk, dv), **f32)
    dg = torch.empty((B, H, N, N), **f32)
    dS0 = torch.empty((B, H, dk, dv), **f32) if want_dS0 else None
    Sr = torch.empty((B, H, N, dk, dv), **f32) if want_states else None
    if ws is None:
        ws = _workspace(workspace_bytes(FN_COMPOSE_BACKWARD, d), dev)
    _check(library().hla_compose_backward(ctypes.byref(d), _ptr(At), _ptr(Bc), _ptr(gates), _ptr(mask), _ptr(S0),
                                          _ptr(dS_routed), _ptr(dAt), _ptr(dBc), _ptr(dg), _ptr(dS0), _ptr(Sr),
                                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev)),
           "hla_compose_backward")
    return dict(dAt=dAt, dBc=dBc, dgates=dg, dS0=dS0, S_routed=Sr)


def chunk_backward(q, k, v, beta, alpha, chunk_init=None, dO=None, dAt=None, dBc=None, ws=None):
    """Reverse of the per-chunk work (64-token chunks): the outputs from chunk_init (with
    dO [B, T, H, dv] float32) and / or the chunk maps (with dAt, dBc float32).  Returns
    dict(dq, dk, dv, dbeta, dalpha, dchunk_init (or None)), all float32, [B, T, H, *]."""
    d = _inputs(k, v, beta, alpha, q=q if chunk_init is not None else None)
    B, T, H, ld_T, dk, dv = d.B, d.T, d.H, d.ld_T, d.dk, d.dv
    N = math.ceil(T / CHUNK)
    dev = k.device
    _need(chunk_init, (B, H, N, dk, dv), torch.float32, "chunk_init")
    _need(dO, (B, T, H, dv), torch.float32, "dO")
    _need(dAt, (B, H, N, dk, dk), torch.float32, "dAt")
    _need(dBc, (B, H, N, dk, dv), torch.float32, "dBc")
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, H, dk), **f32), dk=torch.empty((B, T, H, dk), **f32),
               dv=torch.empty((B, T, H, dv), **f32), dbeta=torch.empty((B, T, H), **f32),
               dalpha=torch.empty((B, T, H), **f32),
               dchunk_init=torch.empty((B, H, N, dk, dv), **f32) if chunk_init is not None else None)
    if ws is None:
        ws = _workspace(workspace_bytes(FN_CHUNK_BACKWARD, d), dev)
    _check(library().hla_chunk_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                                        _ptr(chunk_init), _ptr(dO), _ptr(dAt), _ptr(dBc), _ptr(out["dq"]),
                                        _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dalpha"]),
                                        _ptr(out["dchunk_init"]), _ptr(ws), 0 if ws is None else ws.numel(),
                                        _stream(dev)), "hla_chunk_backward")
    return out


def prefill_backward(q, k, v, beta, alpha, dO, tau=1e-3, gates_in=None, S0=None, want_dS0=True, want_dgates=True,
                     ws=None):
    """Gradients of the routed prefill (raw-key representatives, 64-token chunks) for the
    upstream gradient dO [B, T, H, dv] float32.  Returns dict(dq, dk, dv, dbeta, dalpha,
    dS0, dgates), float32 (dS0 / dgates None unless wanted).  `ws` (uint8, device) may be
    smaller than workspace_bytes(FN_PREFILL_BACKWARD) down to FN_PREFILL_BACKWARD_MIN's size:
    the composition backward then runs its history steps in segments replayed from
    checkpoints."""
    d = _inputs(k, v, beta, alpha, q=q)
    B, T, H, dk, dv = d.B, d.T, d.H, d.dk, d.dv
    N = math.ceil(T / CHUNK)
    dev = k.device
    _need(dO, (B, T, H, dv), torch.float32, "dO")
    _need(S0, (B, H, dk, dv), torch.float32, "S0")
    _need(gates_in, (B, H, N, N), torch.float32, "gates_in")
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, H, dk), **f32), dk=torch.empty((B, T, H, dk), **f32),
               dv=torch.empty((B, T, H, dv), **f32), dbeta=torch.empty((B, T, H), **f32),
               dalpha=torch.empty((B, T, H), **f32),
               dS0=torch.empty((B, H, dk, dv), **f32) if want_dS0 else None,
               dgates=torch.empty((B, H, N, N), **f32) if want_dgates else None)
    if ws is None:
        ws = _workspace(workspace_bytes(FN_PREFILL_BACKWARD, d), dev)
    _check(library().hla_prefill_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                                          _ptr(S0), _ptr(gates_in), ctypes.c_float(tau), _ptr(dO), _ptr(out["dq"]),
                                          _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dbeta"]), _ptr(out["dalpha"]),
                                          _ptr(out["dS0"]), _ptr(out["dgates"]), _ptr(ws),
                                          0 if ws is None else ws.numel(), _stream(dev)), "hla_prefill_backward")
    return out


def _gdn2_grads(B, T, H, dk, dv, dev):
    f32 = dict(dtype=torch.float32, device=dev)
    return dict(dq=torch.empty((B, T, H, dk), **f32), dk=torch.empty((B, T, H, dk), **f32),
                dv=torch.empty((B, T, H, dv), **f32), da=torch.empty((B, T, H, dk), **f32),
                db=torch.empty((B, T, H, dk), **f32), dw=torch.empty((B, T, H, dv), **f32))


def gdn2_chunk_backward(q, k, v, a_decay, b_erase, w_write, chunk_init=None, dO=None, dAt=None, dBc=None, ws=None):
    """chunk_backward for the Gated DeltaNet-2 recurrence.  Returns dict(dq, dk, dv, da, db,
    dw, dchunk_init (or None)), all float32."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    dv = v.shape[-1]
    d = make_dims(B, T, H, ld_T, dk, dv, _dtype_code(k), CHUNK)
    _gdn2_gates(d, a_decay, b_erase, w_write)
    N = math.ceil(T / CHUNK)
    dev = k.device
    _need(chunk_init, (B, H, N, dk, dv), torch.float32, "chunk_init")
    _need(dO, (B, T, H, dv), torch.float32, "dO")
    _need(dAt, (B, H, N, dk, dk), torch.float32, "dAt")
    _need(dBc, (B, H, N, dk, dv), torch.float32, "dBc")
    out = _gdn2_grads(B, T, H, dk, dv, dev)
    out["dchunk_init"] = (torch.empty((B, H, N, dk, dv), dtype=torch.float32, device=dev)
                          if chunk_init is not None else None)
    if ws is None:
        ws = _workspace(workspace_bytes(FN_GDN2_CHUNK_BACKWARD, d), dev)
    _check(library().hla_gdn2_chunk_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a_decay),
                                             _ptr(b_erase), _ptr(w_write), _ptr(chunk_init), _ptr(dO), _ptr(dAt),
                                             _ptr(dBc), *(_ptr(out[n]) for n in ("dq", "dk", "dv", "da", "db", "dw")),
                                             _ptr(out["dchunk_init"]), _ptr(ws), 0 if ws is None else ws.numel(),
                                             _stream(dev)), "hla_gdn2_chunk_backward")
    return out


def gdn2_prefill_backward(q, k, v, a_decay, b_erase, w_write, dO, tau=1e-3, gates_in=None, S0=None, want_dS0=True,
                          want_dgates=True, ws=None):
    """prefill_backward for the Gated DeltaNet-2 routed prefill.  Returns dict(dq, dk, dv,
    da, db, dw, dS0, dgates), float32 (dS0 / dgates None unless wanted); `ws` may be as
    small as workspace_bytes(FN_GDN2_PREFILL_BACKWARD_MIN)."""
    B, T, H, dk, ld_T = _token_view(k, "k")
    dv = v.shape[-1]
    d = make_dims(B, T, H, ld_T, dk, dv, _dtype_code(k), CHUNK)
    _gdn2_gates(d, a_decay, b_erase, w_write)
    N = math.ceil(T / CHUNK)
    dev = k.device
    _need(dO, (B, T, H, dv), torch.float32, "dO")
    _need(S0, (B, H, dk, dv), torch.float32, "S0")
    _need(gates_in, (B, H, N, N), torch.float32, "gates_in")
    f32 = dict(dtype=torch.float32, device=dev)
    out = _gdn2_grads(B, T, H, dk, dv, dev)
    out["dS0"] = torch.empty((B, H, dk, dv), **f32) if want_dS0 else None
    out["dgates"] = torch.empty((B, H, N, N), **f32) if want_dgates else None
    if ws is None:
        ws = _workspace(workspace_bytes(FN_GDN2_PREFILL_BACKWARD, d), dev)
    _check(library().hla_gdn2_prefill_backward(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(a_decay),
                                               _ptr(b_erase), _ptr(w_write), _ptr(S0), _ptr(gates_in),
                                               ctypes.c_float(tau), _ptr(dO),
                                               *(_ptr(out[n]) for n in ("dq", "dk", "dv", "da", "db", "dw")),
                                               _ptr(out["dS0"]), _ptr(out["dgates"]), _ptr(ws),
                                               0 if ws is None else ws.numel(), _stream(dev)),
           "hla_gdn2_prefill_backward")
    return out


def hla_prefill(q, k, v, beta, alpha, tau=1e-3, gates_in=None, S0=None, C=CHUNK, handoff=True, pooler=None,
                window=32):
    """The routed prefill as three calls: transitions, routing, outputs from routed states.
    Representatives are each chunk's raw keys (n_rep = C), or with ``pooler`` (weights for
    chunk_reps) the learned window representatives (n_rep = C / window).  handoff passes
    W | U from the first call to the last (bf16)."""
    wu = wu_buffer(k, v, beta, alpha, C=C) if handoff else None
    At, Bc = chunk_transitions(k, v, beta, alpha, C=C, wu=wu)
    if pooler is None:
        reps, n_rep = k, C
    else:
        reps, n_rep = chunk_reps(k, pooler, window=window, C=C), C // window
    r = route_mix(q, reps, At, Bc, n_rep=n_rep, tau=tau, S0=S0, gates_in=gates_in, C=C)
    o, _ = gdn_prefill(q, k, v, beta, alpha, chunk_init=r["S_routed"], want_state=False, C=C, wu=wu)
    r.update(At=At, Bc=Bc, o=o, reps=reps)
    return r


def gdn_decode(q, k, v, beta, alpha, S_cur, At_cur=None, At_cache=None, Bc_cache=None, reps_cache=None,
               n_cache=None, gates_in=None, tau=1e-3, o=None, gates_out=None, commit=False):
    """One decode step.  q, k [Bs, H, dk], v [Bs, H, dv]; S_cur/At_cur are updated in place."""
    Bs, H, dk = k.shape
    _need(beta, (Bs, H), torch.float32, "beta")
    _need(alpha, (Bs, H), torch.float32, "alpha")
    return _decode("hla_gdn_decode", (beta, alpha), q, k, v, S_cur, At_cur, At_cache, Bc_cache, reps_cache, n_cache,
                   gates_in, tau, o, gates_out, commit)


def gdn2_decode(q, k, v, a_decay, b_erase, w_write, S_cur, At_cur=None, At_cache=None, Bc_cache=None,
                reps_cache=None, n_cache=None, gates_in=None, tau=1e-3, o=None, gates_out=None, commit=False):
    """One decode step under the Gated DeltaNet-2 recurrence: a_decay, b_erase [Bs, H, dk]
    and w_write [Bs, H, dv] (float32) replace beta and alpha."""
    Bs, H, dk = k.shape
    dv = v.shape[-1]
    _need(a_decay, (Bs, H, dk), torch.float32, "a_decay")
    _need(b_erase, (Bs, H, dk), torch.float32, "b_erase")
    _need(w_write, (Bs, H, dv), torch.float32, "w_write")
    return _decode("hla_gdn2_decode", (a_decay, b_erase, w_write), q, k, v, S_cur, At_cur, At_cache, Bc_cache,
                   reps_cache, n_cache, gates_in, tau, o, gates_out, commit)


def _decode(fn, gates, q, k, v, S_cur, At_cur, At_cache, Bc_cache, reps_cache, n_cache, gates_in, tau, o, gates_out,
            commit):
    Bs, H, dk = k.shape
    dv = v.shape[-1]
    dt = _dtype_code(k)
    dev = k.device
    _need(q, (Bs, H, dk), k.dtype, "q")
    _need(v, (Bs, H, dv), k.dtype, "v")
    _need(S_cur, (Bs, H, dk, dv), torch.float32, "S_cur")
    n_cap, n_rep = 0, 0
    if At_cur is not None:
        _need(At_cur, (Bs, H, dk, dk), torch.float32, "At_cur")
        n_cap = At_cache.shape[2]
        _need(At_cache, (Bs, H, n_cap, dk, dk), k.dtype, "At_cache")
        _need(Bc_cache, (Bs, H, n_cap, dk, dv), k.dtype, "Bc_cache")
        _need(n_cache, (Bs,), torch.int32, "n_cache")
        if reps_cache is not None:
            n_rep = reps_cache.shape[3]
            _need(reps_cache, (Bs, H, n_cap, n_rep, dk), k.dtype, "reps_cache")
        _need(gates_in, (Bs, H, n_cap), torch.float32, "gates_in")
        _need(gates_out, (Bs, H, n_cap), torch.float32, "gates_out")
    if o is None:
        o = torch.empty((Bs, H, dv), dtype=torch.float32, device=dev)
    _need(o, (Bs, H, dv), torch.float32, "o")
    _check(getattr(library(), fn)(Bs, H, dk, dv, dt, _ptr(q), _ptr(k), _ptr(v), *(_ptr(g) for g in gates),
                                  _ptr(S_cur), _ptr(At_cur), _ptr(At_cache), _ptr(Bc_cache), _ptr(reps_cache), n_rep,
                                  _ptr(n_cache), n_cap, _ptr(gates_in), ctypes.c_float(tau), _ptr(o),
                                  _ptr(gates_out), 1 if commit else 0, _stream(dev)), fn)
    return o


def timing_enable(on: bool = True) -> None:
    """Start (or stop) per-kernel HIP-event timing inside the library; clears records."""
    _check(library().hla_timing_enable(1 if on else 0), "hla_timing_enable")


def timing_read(which: int) -> tuple[float, int]:
    """(summed milliseconds, launches) of one kernel kind since timing_enable()."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(library().hla_timing_read(which, ctypes.byref(ms), ctypes.byref(n)), "hla_timing_read")
    return ms.value, n.value
