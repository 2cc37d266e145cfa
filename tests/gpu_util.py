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


class ErrorSums:
    """rel-L2 and max-abs over a tensor seen in pieces (every decode step's o)."""

    def __init__(self):
        self.num = self.den = self.mab = 0.0
        self.finite = True

    def add(self, x, ref):
        x = np.asarray(x, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        self.finite &= bool(np.all(np.isfinite(x)))
        d = x - ref
        self.num += float(np.sum(d * d))
        self.den += float(np.sum(ref * ref))
        self.mab = max(self.mab, float(np.max(np.abs(d))))

    def check(self, name):
        rel = (self.num / self.den) ** 0.5 if self.den > 0 else self.num ** 0.5
        say(f"  {name}: rel_l2={rel:.3e} max_abs={self.mab:.3e}")
        assert self.finite, f"{name}: non-finite values"
        assert rel <= REL_L2_TOL, f"{name}: rel-L2 {rel:.3e} > {REL_L2_TOL:.1e}"
        assert self.mab <= MAX_ABS_TOL, f"{name}: max-abs {self.mab:.3e} > {MAX_ABS_TOL:.1e}"


def to_host(t):
    return t.detach().to("cpu").numpy() if t is not None else None


# Guard bands around output buffers: each output is a view into a larger
# allocation whose bands on both sides hold a byte pattern that no store of
# the library may touch, and whose inside starts as all-ones bytes (NaN in
# fp32 and bf16), so that an element the kernels never write fails the
# parity check's finiteness test as well.
GUARD_BYTES = 16384
GUARD_PATTERN = 0xA5


class Guarded:
    """An output tensor of `shape` inside a guarded allocation."""

    def __init__(self, shape, dtype, device):
        esz = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // esz
        self.n = int(np.prod(shape)) if len(shape) else 1
        self.buf = torch.empty(self.n + 2 * self.g, dtype=dtype, device=device)
        raw = self.buf.view(torch.uint8)
        raw.fill_(GUARD_PATTERN)
        raw[GUARD_BYTES:GUARD_BYTES + self.n * esz].fill_(0xFF)
        self.t = self.buf[self.g:self.g + self.n].view(tuple(shape))

    def check(self, name="output"):
        raw = self.buf.view(torch.uint8)
        lo = raw[:GUARD_BYTES]
        hi = raw[raw.numel() - GUARD_BYTES:]
        bad_lo = int((lo != GUARD_PATTERN).sum().item())
        bad_hi = int((hi != GUARD_PATTERN).sum().item())
        assert bad_lo == 0 and bad_hi == 0, \
            f"{name}: {bad_lo} bytes before and {bad_hi} bytes after the buffer were written"


def guarded(shape, dtype, device):
    return Guarded(shape, dtype, device)
