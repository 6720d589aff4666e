"""Bitwise determinism: every entry point called twice on the same input buffers gives
bit-identical outputs.

The library sums in a fixed order everywhere (no atomics, no order that depends on
scheduling), so two launches of the same call must agree to the last bit.  Outputs are
written into buffers that are first filled with a canary pattern (NaN for floats, fixed
bytes for integers), so an output element a kernel forgot to write shows up too.  The cases are sized to run several workgroups per kernel (ragged last
chunk; B H a multiple of 8 for the composition's XCD-ordered dispatch)."""
import math

import pytest
import torch

from gated_deltanet_hybrid_amd import inputs
from gpu_util import dev, f32, note, token_tensors

pytestmark = pytest.mark.gpu
C = 64


def hla():
    from gated_deltanet_hybrid_amd import hla as h
    return h


CANARY_INT = {torch.int32: 0x5A5A5A5A, torch.uint8: 0xA5}


def canary(shape, dtype):
    """A buffer filled with a pattern no output takes (NaN for floats, 0x5A5A5A5A / 0xA5 for
    integers), so an element a kernel left unwritten stands out."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.fill_(float("nan") if t.is_floating_point() else CANARY_INT[dtype])
    return t


def same(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    if a.is_floating_point():
        bits = torch.int16 if a.element_size() == 2 else torch.int32
        ok = torch.equal(a.view(bits), b.view(bits))
    else:
        ok = torch.equal(a, b)
    assert ok, f"{what}: two runs of the same call differ"


def no_canary(t, what):
    if t.is_floating_point():
        assert not torch.isnan(t).any(), f"{what}: an output element was not written"
    elif t.dtype in CANARY_INT:
        assert not (t == CANARY_INT[t.dtype]).any(), f"{what}: an output element was not written"


def twice(fn, what):
    """fn(run) returns a dict of output tensors; compare the two runs bit for bit."""
    note(f"determinism: {what}")
    r1 = fn(0)
    r2 = fn(1)
    torch.cuda.synchronize()
    for name in r1:
        if r1[name] is None:
            continue
        no_canary(r1[name], f"{what} {name}")
        same(r1[name], r2[name], f"{what} {name}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_routed_prefill_twice(dtype):
    B, H, T, d = 1, 8, 24 * C - 19, 128 if dtype == "bf16" else 64
    x = inputs.gen_tokens(B, T, H, d, d, dtype=dtype, seed=61, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    h = hla()
    N = math.ceil(T / C)
    tdt = k.dtype

    def run(_):
        At, Bc = canary((B, H, N, d, d), tdt), canary((B, H, N, d, d), tdt)
        wu = h.wu_buffer(k, v, beta, alpha)
        h.chunk_transitions(k, v, beta, alpha, At=At, Bc=Bc, wu=wu)
        out = dict(gates=canary((B, H, N, N), torch.float32), mask=canary((B, H, N, N), torch.uint8),
                   active_idx=canary((B, H, N, N), torch.int32), active_cnt=canary((B, H, N), torch.int32),
                   n_eff=canary((B, H, N), torch.float32), S_routed=canary((B, H, N, d, d), torch.float32))
        r = h.route_mix(q, k, At, Bc, n_rep=C, tau=1e-3, out=out)
        o = canary((B, T, H, d), torch.float32)
        h.gdn_prefill(q, k, v, beta, alpha, chunk_init=r["S_routed"], want_state=False, o=o, wu=wu)
        return dict(At=At, Bc=Bc, o=o, **{n: r[n] for n in ("gates", "mask", "active_idx", "active_cnt", "n_eff",
                                                          "S_routed")})

    twice(run, f"routed prefill {dtype}")


@pytest.mark.parametrize("dtype,Cw", [("bf16", 64), ("f32", 64), ("bf16", 256)])
def test_native_prefill_twice(dtype, Cw):
    B, H, T, d = 2, 4, 19 * C - 7, 128 if dtype == "bf16" else 64
    x = inputs.gen_tokens(B, T, H, d, d, dtype=dtype, seed=62, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    S0 = f32(inputs.gen_state(B, H, d, d, seed=63))
    h = hla()

    def run(_):
        o, S = canary((B, T, H, d), torch.float32), canary((B, H, d, d), torch.float32)
        h.gdn_prefill(q, k, v, beta, alpha, S0=S0, o=o, S_final=S, C=Cw)
        S2 = canary((B, H, d, d), torch.float32)
        h.gdn_prefill(None, k, v, beta, alpha, S0=S0, want_o=False, S_final=S2, C=Cw)
        return dict(o=o, S_final=S, S_state_only=S2)

    twice(run, f"native prefill {dtype} C={Cw}")


def test_decode_twice():
    Bs, H, d, n_cap = 16, 4, 128, 12
    At_s, Bc_s = inputs.gen_transitions(Bs, H, n_cap, d, d, dtype="bf16", seed=64)
    reps_x = inputs.gen_tokens(Bs, n_cap * C, H, d, d, dtype="bf16", seed=65, with_q=False)
    reps = dev(reps_x.k.reshape(Bs, n_cap, C, H, d).transpose(0, 3, 1, 2, 4).copy(), "bf16")
    tok = inputs.gen_decode_tokens(Bs, H, d, d, step=0, dtype="bf16", seed=66)
    S0 = f32(inputs.gen_state(Bs, H, d, d, seed=67))
    h = hla()

    def run(_):
        S = S0.clone()
        A = torch.eye(d, dtype=torch.float32, device="cuda").repeat(Bs, H, 1, 1).contiguous()
        At_c, Bc_c = dev(At_s, "bf16"), dev(Bc_s, "bf16")
        n_cache = torch.arange(Bs, dtype=torch.int32, device="cuda") % (n_cap + 1)
        o, g = canary((Bs, H, d), torch.float32), canary((Bs, H, n_cap), torch.float32)
        h.gdn_decode(dev(tok["q"], "bf16"), dev(tok["k"], "bf16"), dev(tok["v"], "bf16"), f32(tok["beta"]),
                     f32(tok["alpha"]), S, At_cur=A, At_cache=At_c, Bc_cache=Bc_c, reps_cache=reps, n_cache=n_cache,
                     tau=1e-3, o=o, gates_out=g, commit=True)
        return dict(o=o, gates=g, S=S, A=A, At_cache=At_c, Bc_cache=Bc_c, n_cache=n_cache)

    twice(run, "routed decode with commit")


def test_gdn2_twice():
    B, H, T, d = 1, 8, 9 * C - 3, 128
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=68, alpha_mode="slow")
    q, k, v, _, _ = token_tensors(x)
    g = inputs.gen_gdn2_gates(B, T, H, d, d, seed=69, alpha_mode="slow")
    ga, gb, gw = (f32(g[n]) for n in ("a", "b", "w"))
    h = hla()
    N = math.ceil(T / C)

    def run(_):
        At, Bc = canary((B, H, N, d, d), torch.bfloat16), canary((B, H, N, d, d), torch.bfloat16)
        h.gdn2_chunk_transitions(k, v, ga, gb, gw, At=At, Bc=Bc)
        o, S = canary((B, T, H, d), torch.float32), canary((B, H, d, d), torch.float32)
        h.gdn2_prefill(q, k, v, ga, gb, gw, o=o, S_final=S)
        return dict(At=At, Bc=Bc, o=o, S=S)

    twice(run, "gated deltanet-2 maps and native prefill")


def test_chunk_reps_twice():
    B, H, T, d = 1, 4, 7 * C - 9, 128
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=70)
    _, k, _, _, _ = token_tensors(x)
    Wd = {n: dev(a, "bf16") for n, a in inputs.gen_pooler_weights(H, d, dtype="bf16", seed=71).items()}
    h = hla()
    N = math.ceil(T / C)

    def run(_):
        out = canary((B, N * 2, H, d), torch.bfloat16)
        h.chunk_reps(k, Wd, window=32, out=out)
        return dict(reps=out)

    twice(run, "learned representatives")


def test_backward_twice():
    B, H, T, d = 1, 8, 12 * C - 21, 128
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=72, alpha_mode="slow")
    q, k, v, beta, alpha = token_tensors(x)
    dO = f32(inputs.gen_cotangent((B, T, H, d), seed=73))
    S0 = f32(inputs.gen_state(B, H, d, d, seed=74))
    h = hla()

    def run(_):
        r = h.prefill_backward(q, k, v, beta, alpha, dO, tau=1e-3, S0=S0)
        return dict(r)

    twice(run, "routed prefill backward")

    # the smallest workspace: history segments replayed from checkpoints
    d = h.make_dims(B, T, H, T, d, d, 1, C)
    ws = torch.empty(h.workspace_bytes(h.FN_PREFILL_BACKWARD_MIN, d), dtype=torch.uint8, device="cuda")

    def run_seg(_):
        return dict(h.prefill_backward(q, k, v, beta, alpha, dO, tau=1e-3, S0=S0, ws=ws))

    twice(run_seg, "routed prefill backward in history segments")


def test_gdn2_backward_twice():
    B, H, T, d = 1, 8, 6 * C - 13, 128
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=75, alpha_mode="slow")
    q, k, v, _, _ = token_tensors(x)
    g = inputs.gen_gdn2_gates(B, T, H, d, d, seed=76, alpha_mode="slow")
    ga, gb, gw = (f32(g[n]) for n in ("a", "b", "w"))
    dO = f32(inputs.gen_cotangent((B, T, H, d), seed=77))
    h = hla()

    def run(_):
        return dict(h.gdn2_prefill_backward(q, k, v, ga, gb, gw, dO, tau=1e-3))

    twice(run, "gated deltanet-2 routed prefill backward")


def test_reps_and_router_backward_twice():
    B, H, T, d = 1, 4, 7 * C - 9, 128
    x = inputs.gen_tokens(B, T, H, d, d, dtype="bf16", seed=78)
    q, k, v, beta, alpha = token_tensors(x)
    Wd = {n: dev(a, "bf16") for n, a in inputs.gen_pooler_weights(H, d, dtype="bf16", seed=79).items()}
    h = hla()
    N = math.ceil(T / C)
    reps = h.chunk_reps(k, Wd, window=32)
    At, Bc = h.chunk_transitions(k, v, beta, alpha)
    fw = h.route_mix(q, reps, At, Bc, n_rep=2, tau=1e-3)
    dG = f32(inputs.gen_cotangent((B, H, N, N), seed=80, name="dgates")) * fw["mask"].float()

    def run(_):
        r = h.router_backward(q, reps, 2, fw["gates"], dG)
        p = h.chunk_reps_backward(k, Wd, r["dreps"], window=32)
        return dict(dq=r["dq"], dreps=r["dreps"], **{n: t for n, t in p.items() if t is not None})

    twice(run, "router and learned-representative backward")
