"""Helpers shared by the GPU parity tests: device transfer of seeded host
inputs, the parity metrics and the tolerance gate."""
import sys

import numpy as np
import pytest
import torch

# Gate for floating-point outputs against the fp64 oracle, applied to o and
# S_final over whole tensors: relative L2 error and maximum absolute error.
REL_L2_TOL = 2e-3
MAX_ABS_TOL = 2e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch.device("cuda:0")


def say(msg: str):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tokens(x: np.ndarray, bf16: bool, device):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if bf16:
        t = t.to(torch.bfloat16)   # exact: the values are bf16 already
    return t.to(device)


def dev_f32(x, device):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(x - ref)
    return float(num / den) if den > 0 else float(num)


def max_abs(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref))) if ref.size else 0.0


def assert_parity(name, x, ref, rel=REL_L2_TOL, mab=MAX_ABS_TOL):
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    r, m = rel_l2(x, ref), max_abs(x, ref)
    say(f"  {name}: rel_l2={r:.3e} max_abs={m:.3e}")
    assert r <= rel, f"{name}: rel-L2 {r:.3e} > {rel:.1e}"
    assert m <= mab, f"{name}: max-abs {m:.3e} > {mab:.1e}"
    return r, m


def to_host(t):
    return t.detach().to("cpu").numpy() if t is not None else None
