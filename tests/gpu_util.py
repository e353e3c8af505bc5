"""Helpers shared by the GPU parity tests: host<->device copies of seeded
inputs and the parity criteria (relative L2 error <= 2e-3 and max abs
error <= 1e-2 against the fp64 oracle, bit-exact where integers decide)."""

from __future__ import annotations

import sys

import numpy as np

REL_L2 = 2e-3
MAX_ABS = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev())


def to_dev_i32(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def rel_l2(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (n if n > 0 else 1.0))


def assert_parity(x, ref, what, rel=REL_L2, mabs=MAX_ABS):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    assert x.shape == ref.shape, f"{what}: shape {x.shape} vs {ref.shape}"
    assert np.isfinite(x).all(), f"{what}: non-finite values"
    r = rel_l2(x, ref)
    m = float(np.abs(x - ref).max()) if x.size else 0.0
    say(f"    {what}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= rel, f"{what}: rel L2 {r:.3e} > {rel}"
    assert m <= mabs, f"{what}: max abs {m:.3e} > {mabs}"


def assert_exact(x, ref, what):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = np.nonzero(x != ref)
    assert x.shape == ref.shape and bad[0].size == 0, (
        f"{what}: {bad[0].size} entries differ, first at {tuple(int(i[0]) for i in bad) if bad[0].size else None}")
