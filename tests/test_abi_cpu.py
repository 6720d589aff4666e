"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
entry point include/hla.h declares, sizes its workspaces, and rejects invalid arguments
with the documented status before anything is enqueued."""
import ctypes
import os
import re

import pytest

from gated_deltanet_hybrid_amd import hla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hla.h")

OK, NULL_ARG, BAD_SHAPE, BAD_DTYPE, WORKSPACE, HIP, UNSUPPORTED, ALIGN = 0, 1, 2, 3, 4, 5, 6, 7
P = 0x10000          # a 16-byte aligned placeholder address; never dereferenced
PU = 0x10008         # a misaligned one


@pytest.fixture(scope="module")
def lib():
    return hla.library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hla_status_t|const char\*|int32_t)\s+(hla_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"hla_chunk_transitions", "hla_gdn_prefill", "hla_route_mix", "hla_gdn_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.hla_abi_version() == 7
    for s in range(0, 10):
        assert lib.hla_status_string(s)
    assert lib.hla_status_string(99) == b"unknown status"


def dims(B=1, T=256, H=2, ld_T=None, dk=128, dv=128, C=64, dtype=1):
    return hla.Dims(B, T, H, T if ld_T is None else ld_T, dk, dv, C, dtype)


def test_workspace_sizes(lib):
    d = dims(B=2, T=130, H=3, dk=128, dv=64, dtype=1)  # N = 3 chunks
    BHN = 2 * 3 * 3
    assert hla.workspace_bytes(hla.FN_CHUNK_TRANSITIONS, d) == 0
    ab = BHN * 128 * 128 * 2 + BHN * 128 * 64 * 2
    wu = BHN * 64 * (128 + 64) * 2  # W | U of every piece, bf16
    st = BHN * 128 * 64 * 4
    assert hla.workspace_bytes(hla.FN_GDN_PREFILL, d) == ab + wu + st
    assert hla.workspace_bytes(hla.FN_WU_HANDOFF, d) == wu
    # float32 takes no hand-off
    d32 = dims(B=2, T=130, H=3, dk=128, dv=64, dtype=0)
    assert hla.workspace_bytes(hla.FN_WU_HANDOFF, d32) == 0
    assert hla.workspace_bytes(hla.FN_GDN_PREFILL, d32) == 2 * ab + st
    # float32 query-chunk means, then the reordered bf16 copies of At - I and of Bc
    assert hla.workspace_bytes(hla.FN_ROUTE_MIX, d) == 2 * 3 * 3 * 128 * 4 + BHN * 128 * 128 * 2 + BHN * 128 * 64 * 2
    # float32: the means only
    assert hla.workspace_bytes(hla.FN_ROUTE_MIX, d32) == 2 * 3 * 3 * 128 * 4
    out = ctypes.c_size_t()
    assert lib.hla_workspace_bytes(99, ctypes.byref(d), 0, ctypes.byref(out)) == UNSUPPORTED
    assert lib.hla_workspace_bytes(0, ctypes.byref(d), 0, None) == NULL_ARG


def test_workspace_sizes_larger_chunks(lib):
    # C = 256 over T = 700: 3 chunks of 256 tokens, 11 pieces of 64
    d = dims(B=1, T=700, H=2, dk=128, dv=128, C=256, dtype=1)
    pieces = 1 * 2 * 11
    ab = pieces * 128 * 128 * 2 + pieces * 128 * 128 * 2
    # the transitions of the 64-token pieces are composed four at a time
    assert hla.workspace_bytes(hla.FN_CHUNK_TRANSITIONS, d) == ab
    # the prefill runs on pieces whatever C is
    assert hla.workspace_bytes(hla.FN_GDN_PREFILL, d) == ab + pieces * 64 * 256 * 2 + pieces * 128 * 128 * 4
    assert hla.workspace_bytes(hla.FN_WU_HANDOFF, d) == pieces * 64 * 256 * 2
    assert hla.workspace_bytes(hla.FN_ROUTE_MIX, d) == 2 * 3 * 128 * 4 + 2 * 2 * 3 * 128 * 128 * 2


@pytest.mark.parametrize("kw,code", [
    (dict(dk=96), BAD_SHAPE), (dict(dv=32), BAD_SHAPE), (dict(C=96), BAD_SHAPE), (dict(C=512), BAD_SHAPE),
    (dict(T=0), BAD_SHAPE), (dict(ld_T=100), BAD_SHAPE), (dict(B=0), BAD_SHAPE), (dict(H=0), BAD_SHAPE),
    (dict(dtype=2), BAD_DTYPE), (dict(C=128, dtype=0), UNSUPPORTED),
])
def test_chunk_transitions_rejects_bad_dims(lib, kw, code):
    d = dims(**kw)
    assert lib.hla_chunk_transitions(ctypes.byref(d), P, P, P, P, P, P, None, None, 0, None) == code


def test_larger_chunks_need_workspace(lib):
    d = dims(C=128)
    need = hla.workspace_bytes(hla.FN_CHUNK_TRANSITIONS, d)
    assert need > 0
    assert lib.hla_chunk_transitions(ctypes.byref(d), P, P, P, P, P, P, None, None, 0, None) == WORKSPACE
    assert lib.hla_chunk_transitions(ctypes.byref(d), P, P, P, P, P, P, None, P, need - 1, None) == WORKSPACE
    # routed outputs with C > 64 scan the pieces of every chunk from its routed state
    pre = lib.hla_gdn_prefill
    assert pre(ctypes.byref(d), P, P, P, P, P, None, P, None, P, None, None, 0, None) == WORKSPACE


def test_chunk_transitions_rejects_null_and_misaligned(lib):
    d = dims()
    assert lib.hla_chunk_transitions(None, P, P, P, P, P, P, None, None, 0, None) == NULL_ARG
    for i in range(6):
        args = [P] * 6
        args[i] = None
        assert lib.hla_chunk_transitions(ctypes.byref(d), *args, None, None, 0, None) == NULL_ARG
        # vector-loaded tensors need 16 bytes, the per-token scalars (beta, alpha) 4
        args[i] = P + 2 if i in (2, 3) else PU
        assert lib.hla_chunk_transitions(ctypes.byref(d), *args, None, None, 0, None) == ALIGN


def test_prefill_validation(lib):
    d = dims()
    pre = lib.hla_gdn_prefill
    # neither o nor S_final
    assert pre(ctypes.byref(d), P, P, P, P, P, None, None, None, None, None, P, 1 << 30, None) == NULL_ARG
    # o without q
    assert pre(ctypes.byref(d), None, P, P, P, P, None, None, None, P, None, P, 1 << 30, None) == NULL_ARG
    # routed mode with S0 or S_final
    assert pre(ctypes.byref(d), P, P, P, P, P, P, P, None, P, None, None, 0, None) == UNSUPPORTED
    assert pre(ctypes.byref(d), P, P, P, P, P, None, P, None, P, P, None, 0, None) == UNSUPPORTED
    # native mode without enough workspace
    d32 = dims(dtype=0)
    need = hla.workspace_bytes(hla.FN_GDN_PREFILL, d32)
    assert pre(ctypes.byref(d32), P, P, P, P, P, None, None, None, P, P, P, need - 1, None) == WORKSPACE
    assert pre(ctypes.byref(d32), P, P, P, P, P, None, None, None, P, P, None, 0, None) == WORKSPACE
    assert pre(ctypes.byref(d), P, P, P, P, P, None, None, None, P, P, None, 0, None) == WORKSPACE
    assert pre(ctypes.byref(d), P, P, P, P, P, None, None, None, P, P, PU, 1 << 30, None) == ALIGN
    # the W | U hand-off: 16-byte aligned, bf16 only
    assert pre(ctypes.byref(d), P, P, P, P, P, None, P, PU, P, None, None, 0, None) == ALIGN
    assert pre(ctypes.byref(d32), P, P, P, P, P, None, P, P, P, None, None, 0, None) == UNSUPPORTED
    assert lib.hla_chunk_transitions(ctypes.byref(d32), P, P, P, P, P, P, P, None, 0, None) == UNSUPPORTED
    assert lib.hla_chunk_transitions(ctypes.byref(d), P, P, P, P, P, P, PU, None, 0, None) == ALIGN


def test_route_mix_validation(lib):
    d = dims(T=256)  # N = 4
    rm = lib.hla_route_mix
    outs = [P, P, P, P, P, P]  # gates, mask, active_idx, active_cnt, n_eff, S_routed
    ws = hla.workspace_bytes(hla.FN_ROUTE_MIX, d)
    # computed gates need q and reps
    assert rm(ctypes.byref(d), None, P, 64, 256, P, P, None, None, 1e-3, *outs, P, ws, None) == NULL_ARG
    assert rm(ctypes.byref(d), P, None, 64, 256, P, P, None, None, 1e-3, *outs, P, ws, None) == NULL_ARG
    # reps rows: (N - 1) * n_rep must fit in ld_R
    assert rm(ctypes.byref(d), P, P, 64, 191, P, P, None, None, 1e-3, *outs, P, ws, None) == BAD_SHAPE
    assert rm(ctypes.byref(d), P, P, 0, 256, P, P, None, None, 1e-3, *outs, P, ws, None) == BAD_SHAPE
    assert rm(ctypes.byref(d), P, P, 64, 256, P, P, None, None, float("nan"), *outs, P, ws, None) == BAD_SHAPE
    assert rm(ctypes.byref(d), P, P, 64, 256, P, P, None, None, 1e-3, *outs, P, ws - 1, None) == WORKSPACE
    bad = list(outs)
    bad[5] = None
    assert rm(ctypes.byref(d), P, P, 64, 256, P, P, None, None, 1e-3, *bad, P, ws, None) == NULL_ARG


def test_decode_validation(lib):
    dec = lib.hla_gdn_decode
    base = [P, P, P, P, P, P]  # q, k, v, beta, alpha, S_cur
    # (Bs, H, dk, dv, dtype, q, k, v, beta, alpha, S_cur, At_cur, At_cache, Bc_cache, reps, n_rep, n_cache,
    #  n_cap, gates_in, tau, o, gates_out, commit, stream)
    assert dec(0, 1, 128, 128, 1, *base, None, None, None, None, 0, None, 0, None, 0.0, P, None, 0, None) == BAD_SHAPE
    assert dec(1, 1, 128, 128, 5, *base, None, None, None, None, 0, None, 0, None, 0.0, P, None, 0, None) == BAD_DTYPE
    assert dec(1, 1, 128, 128, 1, *base, None, None, None, None, 0, None, 0, None, 0.0, None, None, 0, None) == NULL_ARG
    # commit needs a live transition
    assert dec(1, 1, 128, 128, 1, *base, None, None, None, None, 0, None, 0, None, 0.0, P, None, 1, None) == UNSUPPORTED
    # routed: cache arrays and n_cache required; n_cap bounded; reps unless caller gates
    assert dec(1, 1, 128, 128, 1, *base, P, None, P, P, 64, P, 4, None, 0.0, P, None, 0, None) == NULL_ARG
    assert dec(1, 1, 128, 128, 1, *base, P, P, P, P, 64, P, 1025, None, 0.0, P, None, 0, None) == BAD_SHAPE
    assert dec(1, 1, 128, 128, 1, *base, P, P, P, None, 64, P, 4, None, 0.0, P, None, 0, None) == NULL_ARG
    assert dec(1, 1, 128, 128, 1, *base, P, P, P, P, 0, P, 4, None, 0.0, P, None, 0, None) == BAD_SHAPE
    assert dec(1, 1, 128, 128, 1, *base, P, P, P, P, 64, P, 4, None, 0.0, P + 2, None, 0, None) == ALIGN
    assert dec(1, 1, 128, 128, 1, P, P, P, P, P, PU, P, P, P, P, 64, P, 4, None, 0.0, P, None, 0, None) == ALIGN


def test_binding_fails_loudly_without_library(tmp_path):
    saved = hla._lib
    try:
        hla._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            hla.library(str(tmp_path / "nope.so"))
    finally:
        hla._lib = saved


def test_chunk_reps_validation(lib):
    d = dims(T=256, C=64)  # N = 4 chunks
    cr = lib.hla_chunk_reps
    need = hla.workspace_bytes(hla.FN_CHUNK_REPS, d, 2)
    assert need == 1 * 2 * 4 * 2 * 128 * 4  # float32 window means [B, H, N * n_rep, dk]
    W = [P, P, P, P]  # Wq, Wk, Wv, Wp
    ok = (ctypes.byref(d), P, 32, *W, None, 0, P, P, need, None)
    # (d, k, window, Wq, Wk, Wv, Wp, Wr, w_hstride, reps, ws, ws_bytes, stream)
    assert cr(ctypes.byref(d), None, 32, *W, None, 0, P, P, need, None) == NULL_ARG
    assert cr(ctypes.byref(d), P, 32, P, P, None, P, None, 0, P, P, need, None) == NULL_ARG
    assert cr(ctypes.byref(d), P, 32, *W, None, 0, None, P, need, None) == NULL_ARG
    for bad_window in (0, 4, 24, 48, 128):
        assert cr(ctypes.byref(d), P, bad_window, *W, None, 0, P, P, need, None) == BAD_SHAPE
    assert cr(ctypes.byref(d), P, 32, *W, None, 100, P, P, need, None) == BAD_SHAPE  # overlapping heads
    assert cr(ctypes.byref(d), P, 32, *W, None, 128 * 128 + 4, P, P, need, None) == ALIGN  # 8-byte head step
    assert cr(ctypes.byref(d), P, 32, *W, PU, 0, P, P, need, None) == ALIGN
    assert cr(ctypes.byref(d), P, 32, *W, None, 0, P, P, need - 1, None) == WORKSPACE
    assert cr(ctypes.byref(d), P, 32, *W, None, 0, P, None, 0, None) == WORKSPACE
    assert lib.hla_workspace_bytes(hla.FN_CHUNK_REPS, ctypes.byref(d), 3, ctypes.byref(ctypes.c_size_t())) == BAD_SHAPE
    assert len(ok) == 13


def test_chunk_reps_noalloc_validation(lib):
    """The no-allocation variant checks what hla_chunk_reps checks, then its fixed scratch
    limit, all before anything reaches the GPU."""
    cr = lib.hla_chunk_reps_noalloc
    W = [P, P, P, P]
    d = dims(T=256, C=64)
    # (d, k, window, Wq, Wk, Wv, Wp, Wr, w_hstride, reps, stream)
    assert cr(ctypes.byref(d), None, 32, *W, None, 0, P, None) == NULL_ARG
    assert cr(ctypes.byref(d), P, 32, *W, None, 0, None, None) == NULL_ARG
    assert cr(ctypes.byref(d), P, 24, *W, None, 0, P, None) == BAD_SHAPE
    assert cr(ctypes.byref(d), P, 32, *W, PU, 0, P, None) == ALIGN
    # window means of B H N (C / window) rows of dk float32: 8 x 16 x 1024 x 128 x 4 bytes
    # = 64 MiB > the 32 MiB array; 4 batch rows fit exactly
    big = dims(B=8, T=32768, H=16, C=64)
    assert cr(ctypes.byref(big), P, 32, *W, None, 0, P, None) == hla.ERR_SCRATCH_LIMIT
    assert hla.workspace_bytes(hla.FN_CHUNK_REPS, dims(B=4, T=32768, H=16, C=64), 2) == hla.REPS_SCRATCH_BYTES
    assert b"scratch" in lib.hla_status_string(hla.ERR_SCRATCH_LIMIT)


def test_gdn2_validation(lib):
    d = dims()
    tr, pre = lib.hla_gdn2_chunk_transitions, lib.hla_gdn2_prefill
    # (d, k, v, a, b, w, At, Bc, ws, ws_bytes, stream)
    for i in range(7):
        args = [P] * 7
        args[i] = None
        assert tr(ctypes.byref(d), *args, None, 0, None) == NULL_ARG
    assert tr(ctypes.byref(d), P, P, P + 2, P, P, P, P, None, 0, None) == ALIGN   # gates need 4 bytes
    assert tr(ctypes.byref(d), P, P, P + 4, P, P, P, P, None, 0, None) != ALIGN
    assert tr(ctypes.byref(d), PU, P, P, P, P, P, P, None, 0, None) == ALIGN
    assert tr(ctypes.byref(dims(C=256)), P, P, P, P, P, P, P, None, 0, None) == WORKSPACE
    assert tr(ctypes.byref(dims(C=128, dtype=0)), P, P, P, P, P, P, P, None, 0, None) == UNSUPPORTED
    # (d, q, k, v, a, b, w, S0, chunk_init, o, S_final, ws, ws_bytes, stream)
    need = hla.workspace_bytes(hla.FN_GDN_PREFILL, d)
    assert pre(ctypes.byref(d), P, P, P, P, P, P, None, None, None, None, P, need, None) == NULL_ARG
    assert pre(ctypes.byref(d), None, P, P, P, P, P, None, None, P, None, P, need, None) == NULL_ARG
    assert pre(ctypes.byref(d), P, P, P, P, P, P, P, P, P, None, None, 0, None) == UNSUPPORTED  # routed with S0
    assert pre(ctypes.byref(d), P, P, P, P, P, P, None, None, P, P, P, need - 1, None) == WORKSPACE
    assert pre(ctypes.byref(d), P, P, P, P, None, P, None, None, P, P, P, need, None) == NULL_ARG


def _r(x):
    return (x + 255) // 256 * 256


def test_backward_workspace_sizes(lib):
    d = dims(B=2, T=130, H=3, dk=128, dv=64, dtype=1)  # N = 3 chunks, 3 pairs per (b, h)
    BH, N, P_ = 6, 3, 3
    # (At - I), its transpose and Bc reordered; per pair M, D and g lambda; gate parts; final lambda
    comp = (2 * _r(BH * N * 128 * 128 * 2) + _r(BH * N * 128 * 64 * 2) + 3 * _r(BH * P_ * 128 * 64 * 2)
            + _r(BH * N * N * 2 * 4) + _r(BH * N * 128 * 64 * 4))
    assert hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD, d) == comp
    BHN, nb_out, nb_all = BH * N, 2, 2 + 6
    chunk = (_r(BHN * nb_all * 64 * 128 * 4) + _r(BHN * nb_out * 64 * 128 * 4) + _r(BHN * nb_all * 64 * 2 * 4)
             + _r(BHN * 2 * 64 * 64 * 4))
    assert hla.workspace_bytes(hla.FN_CHUNK_BACKWARD, d) == chunk
    # the prefill backward holds the composition's per-pair states: it grows as N^2
    pb = hla.workspace_bytes(hla.FN_PREFILL_BACKWARD, d)
    assert pb > comp + chunk
    d4 = dims(B=2, T=130 + 3 * 64, H=3, dk=128, dv=64, dtype=1)  # N = 6: 15 pairs
    assert hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD, d4) - hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD, d) >= \
        3 * BH * 12 * 128 * 64 * 2
    out = ctypes.c_size_t()
    for fn in (hla.FN_CHUNK_BACKWARD, hla.FN_PREFILL_BACKWARD, hla.FN_PREFILL_BACKWARD_MIN):
        assert lib.hla_workspace_bytes(fn, ctypes.byref(dims(C=128)), 0, ctypes.byref(out)) == UNSUPPORTED


def _comp_ws(BH, N, dk, dv, e, K):
    """Composition-backward workspace with history segments of K steps: the reordered maps,
    gate parts and lambdas, float32 checkpoints of every chain i > b K at each boundary b K,
    and the first segment's pair slots (chain i holds min(K, i)) for M, D and g lambda."""
    slots = sum(min(K, i) for i in range(1, N))
    nck = sum(N - 1 - b * K for b in range(1, (N - 1) // K + 1) if b * K < N)
    return (2 * _r(BH * N * dk * dk * e) + _r(BH * N * dk * dv * e) + _r(BH * N * N * (dv // 32) * 4)
            + _r(BH * N * dk * dv * 4) + _r(BH * nck * dk * dv * 4) + 3 * _r(BH * slots * dk * dv * e))


def test_backward_minimum_workspace(lib):
    """The one-pass workspace is one segment (K = N, no checkpoint); the smallest is the
    segment length that needs least; the prefill backward adds the same fixed part to both."""
    for T, N in ((130, 3), (130 + 3 * 64, 6), (64, 1), (40 * 64, 40)):
        d = dims(B=2, T=T, H=3, dk=128, dv=64, dtype=1)
        full, mn = hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD, d), hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD_MIN, d)
        assert full == _comp_ws(6, N, 128, 64, 2, N)
        assert mn == min(_comp_ws(6, N, 128, 64, 2, K) for K in range(1, N + 1))
        pf, pm = hla.workspace_bytes(hla.FN_PREFILL_BACKWARD, d), hla.workspace_bytes(hla.FN_PREFILL_BACKWARD_MIN, d)
        assert pf - pm == full - mn
    # at 40 chunks the segments need far less than every pair's slots
    assert mn < full / 2


def test_compose_backward_validation(lib):
    d = dims()
    f = lib.hla_compose_backward
    need = hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD, d)
    # (d, At, Bc, gates, mask, S0, dS, dAt, dBc, dgates, dS0, S_routed, ws, ws_bytes, stream)
    req = [0, 1, 2, 3, 5, 6, 7, 8]  # positions of required pointers among the 11
    for i in req:
        args = [P] * 11
        args[i] = None
        assert f(ctypes.byref(d), *args, P, need, None) == NULL_ARG, i
    args = [P] * 11
    mn = hla.workspace_bytes(hla.FN_COMPOSE_BACKWARD_MIN, d)
    assert mn < need  # N = 4 chunks: segments of one step
    assert f(ctypes.byref(d), *args, P, mn - 1, None) == WORKSPACE
    assert f(ctypes.byref(d), *args, None, 0, None) == WORKSPACE
    bad = list(args)
    bad[0] = PU
    assert f(ctypes.byref(d), *bad, P, need, None) == ALIGN
    bad = list(args)
    bad[2] = P + 2  # gates need 4 bytes
    assert f(ctypes.byref(d), *bad, P, need, None) == ALIGN
    assert f(ctypes.byref(dims(dtype=2)), *args, P, need, None) == BAD_DTYPE


def test_chunk_backward_validation(lib):
    d = dims()
    f = lib.hla_chunk_backward
    need = hla.workspace_bytes(hla.FN_CHUNK_BACKWARD, d)
    # (d, q, k, v, beta, alpha, chunk_init, dO, dAt, dBc, dq, dk, dv, dbeta, dalpha, dinit, ws, ws_bytes, s)
    full = [P] * 15
    assert f(ctypes.byref(d), *full, None, 0, None) == WORKSPACE
    neither = list(full)
    neither[5:9] = [None] * 4
    assert f(ctypes.byref(d), *neither, P, need, None) == NULL_ARG   # no part asked for
    half = list(full)
    half[6] = None                                                   # chunk_init without dO
    assert f(ctypes.byref(d), *half, P, need, None) == NULL_ARG
    half = list(full)
    half[8] = None                                                   # dAt without dBc
    assert f(ctypes.byref(d), *half, P, need, None) == NULL_ARG
    outs_only_map = list(full)
    outs_only_map[5] = outs_only_map[6] = None
    outs_only_map[0] = None                                          # q unused by the map part
    outs_only_map[14] = None                                         # no dchunk_init without outputs
    assert f(ctypes.byref(d), *outs_only_map, P, need - 1, None) == WORKSPACE
    for i in range(9, 14):
        a = list(full)
        a[i] = None
        assert f(ctypes.byref(d), *a, P, need, None) == NULL_ARG, i
    a = list(full)
    a[3] = P + 2
    assert f(ctypes.byref(d), *a, P, need, None) == ALIGN
    assert f(ctypes.byref(dims(C=128)), *full, P, need, None) == UNSUPPORTED


def test_prefill_backward_validation(lib):
    d = dims()
    f = lib.hla_prefill_backward
    need = hla.workspace_bytes(hla.FN_PREFILL_BACKWARD, d)
    # (d, q, k, v, beta, alpha, S0, gates_in, tau, dO, dq, dk, dv, dbeta, dalpha, dS0, dgates, ws, ws_bytes, s)
    def call(args, tau=1e-3, ws=P, nb=need, dd=d):
        return f(ctypes.byref(dd), *args[:7], ctypes.c_float(tau), *args[7:], ws, nb, None)
    full = [P] * 15  # q .. gates_in (7), then dO .. dgates (8)
    for i in (0, 1, 2, 3, 4, 7, 8, 9, 10, 11, 12):
        a = list(full)
        a[i] = None
        assert call(a) == NULL_ARG, i
    opt = list(full)
    opt[5] = opt[6] = opt[13] = opt[14] = None  # S0, gates_in, dS0, dgates are optional
    mn = hla.workspace_bytes(hla.FN_PREFILL_BACKWARD_MIN, d)
    assert mn < need
    assert call(opt, nb=mn - 1) == WORKSPACE
    assert call(opt, ws=None, nb=need) == WORKSPACE
    assert call(full, tau=float("nan")) == BAD_SHAPE
    assert call(full, dd=dims(C=256)) == UNSUPPORTED
    a = list(full)
    a[0] = PU
    assert call(a) == ALIGN


def test_gdn2_backward_workspace_sizes(lib):
    """Column sums of workgroups of 32 state columns (bf16; 16 for float32): dk, da and db
    over every slot, dq over the outputs' slots, dv and dw per part; the prefill backward
    differs from Gated DeltaNet's by the chunk reverse's region only."""
    d = dims(B=2, T=130, H=3, dk=128, dv=64, dtype=1)  # N = 3
    BHN, nb_out, nb_all = 6 * 3, 64 // 32, 64 // 32 + (128 + 64) // 32
    vec = _r(BHN * nb_all * 64 * 128 * 4)
    g2 = 3 * vec + _r(BHN * nb_out * 64 * 128 * 4) + 2 * _r(BHN * 2 * 64 * 64 * 4)
    assert hla.workspace_bytes(hla.FN_GDN2_CHUNK_BACKWARD, d) == g2
    g1 = hla.workspace_bytes(hla.FN_CHUNK_BACKWARD, d)
    for one, two in ((hla.FN_PREFILL_BACKWARD, hla.FN_GDN2_PREFILL_BACKWARD),
                     (hla.FN_PREFILL_BACKWARD_MIN, hla.FN_GDN2_PREFILL_BACKWARD_MIN)):
        assert hla.workspace_bytes(two, d) - hla.workspace_bytes(one, d) == g2 - g1
    d32 = dims(B=2, T=130, H=3, dk=128, dv=64, dtype=0)
    nb_out, nb_all = 64 // 16, 64 // 16 + (128 + 64) // 16
    assert hla.workspace_bytes(hla.FN_GDN2_CHUNK_BACKWARD, d32) == 3 * _r(BHN * nb_all * 64 * 128 * 4) + \
        _r(BHN * nb_out * 64 * 128 * 4) + 2 * _r(BHN * 2 * 64 * 64 * 4)
    out = ctypes.c_size_t()
    for fn in (hla.FN_GDN2_CHUNK_BACKWARD, hla.FN_GDN2_PREFILL_BACKWARD, hla.FN_GDN2_PREFILL_BACKWARD_MIN):
        assert lib.hla_workspace_bytes(fn, ctypes.byref(dims(C=128)), 0, ctypes.byref(out)) == UNSUPPORTED


def test_gdn2_chunk_backward_validation(lib):
    d = dims()
    f = lib.hla_gdn2_chunk_backward
    need = hla.workspace_bytes(hla.FN_GDN2_CHUNK_BACKWARD, d)
    # (d, q, k, v, a, b, w, chunk_init, dO, dAt, dBc, dq, dk, dv, da, db, dw, dinit, ws, ws_bytes, s)
    full = [P] * 17
    assert f(ctypes.byref(d), *full, None, 0, None) == WORKSPACE
    assert f(ctypes.byref(d), *full, P, need - 1, None) == WORKSPACE
    neither = list(full)
    neither[6:10] = [None] * 4
    assert f(ctypes.byref(d), *neither, P, need, None) == NULL_ARG
    half = list(full)
    half[7] = None                                                   # chunk_init without dO
    assert f(ctypes.byref(d), *half, P, need, None) == NULL_ARG
    for i in (1, 2, 3, 4, 5, 10, 11, 12, 13, 14, 15):
        a = list(full)
        a[i] = None
        assert f(ctypes.byref(d), *a, P, need, None) == NULL_ARG, i
    a = list(full)
    a[4] = P + 2  # the erase gate needs 4 bytes
    assert f(ctypes.byref(d), *a, P, need, None) == ALIGN
    a = list(full)
    a[1] = PU
    assert f(ctypes.byref(d), *a, P, need, None) == ALIGN
    assert f(ctypes.byref(dims(C=128)), *full, P, need, None) == UNSUPPORTED


def test_gdn2_prefill_backward_validation(lib):
    d = dims()
    f = lib.hla_gdn2_prefill_backward
    need = hla.workspace_bytes(hla.FN_GDN2_PREFILL_BACKWARD, d)
    # (d, q, k, v, a, b, w, S0, gates_in, tau, dO, dq, dk, dv, da, db, dw, dS0, dgates, ws, ws_bytes, s)
    def call(args, tau=1e-3, ws=P, nb=need, dd=d):
        return f(ctypes.byref(dd), *args[:8], ctypes.c_float(tau), *args[8:], ws, nb, None)
    full = [P] * 17  # q .. gates_in (8), then dO .. dgates (9)
    for i in (0, 1, 2, 3, 4, 5, 8, 9, 10, 11, 12, 13, 14):
        a = list(full)
        a[i] = None
        assert call(a) == NULL_ARG, i
    opt = list(full)
    opt[6] = opt[7] = opt[15] = opt[16] = None  # S0, gates_in, dS0, dgates are optional
    mn = hla.workspace_bytes(hla.FN_GDN2_PREFILL_BACKWARD_MIN, d)
    assert mn < need
    assert call(opt, nb=mn - 1) == WORKSPACE
    assert call(opt, ws=None, nb=need) == WORKSPACE
    assert call(full, tau=float("nan")) == BAD_SHAPE
    assert call(full, dd=dims(C=256)) == UNSUPPORTED
    a = list(full)
    a[5] = P + 2
    assert call(a) == ALIGN


def test_reps_and_router_backward_workspace_sizes(lib):
    d = dims(B=2, T=130, H=3, dk=128, dv=64, dtype=1)  # 3 tiles of 64 tokens, N = 3
    # the router: query means and their gradients, then one part of the gradients per segment
    # of history chunks (about 1024 workgroups over b, h, 128-chunk query groups, segments;
    # 4 to 32 chunks a segment)
    for B, T, H in ((2, 130, 3), (1, 8192, 16), (1, 32768, 16), (2, 700 * 64, 4)):
        dd = dims(B=B, T=T, H=H, dk=128, dv=64, dtype=1)
        N = -(-T // 64)
        nqg = -(-(-(-N // 32)) // 4)
        seg = min(32, max(4, -(-(N * B * H * nqg) // 1024)))
        means = _r(B * H * N * 128 * 4)
        assert hla.workspace_bytes(hla.FN_ROUTER_BACKWARD, dd) == 2 * means + _r(-(-N // seg) * B * H * N * 128 * 4)
    # the pooler: dWq, dWk, dWv per workgroup of 8 tiles (one group at 3 tiles, 2 at 9), then
    # four vectors per window, sized for windows of 8 (8 per tile), then dWp and dWr per chunk
    # of 256 windows of a (b, h)
    for T, groups in ((130, 1), (9 * 64 - 5, 2), (40 * 64, 5)):
        dd = dims(B=2, T=T, H=3, dk=128, dv=64, dtype=1)
        ntl = -(-T // 64)
        chunks = 2 * 3 * (-(-ntl * 8 // 256))
        want = _r(2 * 3 * groups * 3 * 128 * 128 * 4) + _r(4 * 2 * ntl * 8 * 3 * 128 * 4) + \
            _r(2 * chunks * 128 * 128 * 4)
        for wr in (0, 1):
            assert hla.workspace_bytes(hla.FN_CHUNK_REPS_BACKWARD, dd, wr) == want
    out = ctypes.c_size_t()
    assert lib.hla_workspace_bytes(hla.FN_ROUTER_BACKWARD, ctypes.byref(dims(C=128)), 0, ctypes.byref(out)) == \
        UNSUPPORTED


def test_router_backward_validation(lib):
    d = dims()
    f = lib.hla_router_backward
    need = hla.workspace_bytes(hla.FN_ROUTER_BACKWARD, d)
    N = -(-d.T // 64)
    # (d, q, reps, n_rep, ld_R, gates, dgates, dq, dreps, ws, ws_bytes, s)
    def call(q=P, reps=P, n_rep=2, ld_R=N * 2, gates=P, dg=P, dq=P, dr=P, ws=P, nb=need, dd=d):
        return f(ctypes.byref(dd), q, reps, n_rep, ld_R, gates, dg, dq, dr, ws, nb, None)
    for kw in ({"q": None}, {"reps": None}, {"gates": None}, {"dg": None}, {"dq": None}, {"dr": None}):
        assert call(**kw) == NULL_ARG, kw
    assert call(n_rep=0) == BAD_SHAPE
    assert call(n_rep=65) == BAD_SHAPE
    assert call(ld_R=(N - 1) * 2 - 1) == BAD_SHAPE
    assert call(reps=PU) == ALIGN
    assert call(gates=P + 2) == ALIGN
    assert call(nb=need - 1) == WORKSPACE
    assert call(ws=None, nb=0) == WORKSPACE
    assert call(dd=dims(C=128)) == UNSUPPORTED


def test_chunk_reps_backward_validation(lib):
    d = dims()
    f = lib.hla_chunk_reps_backward
    need = hla.workspace_bytes(hla.FN_CHUNK_REPS_BACKWARD, d, 1)
    # (d, k, window, Wq, Wk, Wv, Wp, Wr, w_hstride, dreps, dk, dWq, dWk, dWv, dWp, dWr, ws, ws_bytes, s)
    def call(ptrs, window=32, hs=0, ws=P, nb=need, dd=d):
        p = list(ptrs)
        return f(ctypes.byref(dd), p[0], window, *p[1:6], hs, *p[6:13], ws, nb, None)
    full = [P] * 13  # k, Wq, Wk, Wv, Wp, Wr, then dreps, dk, dWq, dWk, dWv, dWp, dWr
    for i in (0, 1, 2, 3, 4, 6, 7, 8, 9, 10, 11, 12):
        a = list(full)
        a[i] = None
        assert call(a) == NULL_ARG, i
    no_wr = list(full)
    no_wr[5] = no_wr[12] = None  # dWr is needed exactly when Wr is given
    assert call(no_wr, nb=hla.workspace_bytes(hla.FN_CHUNK_REPS_BACKWARD, d, 0) - 1) == WORKSPACE
    assert call(full, window=24) == BAD_SHAPE
    assert call(full, hs=100) == BAD_SHAPE
    a = list(full)
    a[7] = P + 2
    assert call(a) == ALIGN
    assert call(full, nb=need - 1) == WORKSPACE
