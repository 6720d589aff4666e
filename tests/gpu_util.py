"""Helpers for the GPU parity tests: move generated storage arrays to the device and
compare with oracle values.  No arithmetic of the method lives here."""
import sys

import numpy as np
import torch

from gated_deltanet_hybrid_amd import inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str) -> None:
    """Print and flush, so a failing GPU run names its case."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Storage array (uint16 bf16 bits or float32) -> CUDA tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def token_tensors(x: inputs.TokenInputs):
    q = dev(x.q, x.dtype) if x.q is not None else None
    return q, dev(x.k, x.dtype), dev(x.v, x.dtype), f32(x.beta), f32(x.alpha)


# Values below float32's smallest normal cannot be stored by either output dtype (both
# share float32's exponent range), so errors up to that size are rounding, not mistakes.
# Under the workloads' decay (median alpha ~ 0.12) a 64-token chunk's transition is
# ~1e-61 and rounds to zero.
FLOOR = float(np.finfo(np.float32).tiny)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max|got - ref| / max|ref|, counting only the part of each error above FLOOR."""
    if not ref.size:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    err = float(np.max(np.maximum(np.abs(got - ref) - FLOOR, 0.0)))
    if err == 0.0:
        return 0.0
    return err / scale if scale > 0.0 else float("inf")


def assert_close(got, ref, dtype, what, tol=None):
    tol = TOL[dtype] if tol is None else tol
    e = rel_err(np.asarray(got, np.float64), np.asarray(ref, np.float64))
    assert e <= tol, f"{what}: max|diff|/max|ref| = {e:.3e} > {tol:.1e}"
    return e
