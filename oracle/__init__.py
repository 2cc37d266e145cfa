"""fp64 CPU oracle for the RDA gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its
Python binding) never imports, links or executes anything here, and this
package imports nothing from the product path.

The arithmetic lives in ``oracle.c`` (plain C, double precision): the gated
delta rule as the page "Raon-1 nano" (ai.satyajit.si), section "The other
1.5B: a hybrid built to forget", orders its recurrent step -- scale the
state by the decay, take the residual e = v - S'k of the scaled state at the
key, add b e k^T -- and read-out o_t = S_t q_t after the update.  This module only marshals NumPy arrays into that library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_default = None


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile an oracle C source into a shared library with gcc (OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, lib_path: str = _LIB):
        if lib_path == _LIB and not os.path.exists(lib_path):
            build(force=False)
        lib = ctypes.CDLL(lib_path)
        p = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.oracle_rda_prefill.argtypes = [p, p, p, p, p, p, i32, ctypes.c_int64,
                                           i32, i32, i32, p, p, p, i32]
        lib.oracle_rda_prefill.restype = ctypes.c_int
        lib.oracle_rda_decode_step.argtypes = [p, p, p, p, p, i32, i32, i32, i32,
                                               p, p, i32]
        lib.oracle_rda_decode_step.restype = ctypes.c_int
        lib.oracle_output_norm_gate.argtypes = [p, p, p, ctypes.c_double, i32,
                                                ctypes.c_int64, i32, p]
        lib.oracle_output_norm_gate.restype = ctypes.c_int
        lib.oracle_prologue.argtypes = [p, p, p, p, i32, i32, p, p, p, p, ctypes.c_double,
                                        ctypes.c_double, p, i32, ctypes.c_int64, i32, i32,
                                        p, p, p, p, p, p]
        lib.oracle_prologue.restype = ctypes.c_int
        lib.oracle_rda_prefill_diag.argtypes = [p, p, p, p, p, p, i32, ctypes.c_int64,
                                                i32, i32, i32, p, p, p, i32]
        lib.oracle_rda_prefill_diag.restype = ctypes.c_int
        lib.oracle_rda_decode_step_diag.argtypes = [p, p, p, p, p, i32, i32, i32, i32, p, p]
        lib.oracle_rda_decode_step_diag.restype = ctypes.c_int
        lib.oracle_threads.argtypes = [i32]
        lib.oracle_threads.restype = ctypes.c_int
        self.lib = lib

    def threads_used(self, threads: int = 0) -> int:
        return int(self.lib.oracle_threads(int(threads)))

    def prefill(self, q, k, v, a, b, cu_seqlens=None, S0=None, threads: int = 0):
        return _prefill(self.lib, q, k, v, a, b, cu_seqlens, S0, threads)

    def decode_step(self, q, k, v, a, b, S, threads: int = 0):
        return _decode_step(self.lib, q, k, v, a, b, S, threads)

    def decode_tokens(self, q, k, v, a, b, S_in, accept=None, threads: int = 0):
        return _decode_tokens(self.lib, q, k, v, a, b, S_in, accept, threads)

    def decode_tokens_diag(self, q, k, v, alpha, b, S_in, accept=None, threads: int = 0):
        return _decode_tokens(self.lib, q, k, v, alpha, b, S_in, accept, threads,
                              prefill=_prefill_diag)

    def prefill_diag(self, q, k, v, alpha, b, cu_seqlens=None, S0=None, threads: int = 0):
        return _prefill_diag(self.lib, q, k, v, alpha, b, cu_seqlens, S0, threads)

    def decode_step_diag(self, q, k, v, alpha, b, S):
        return _decode_step_diag(self.lib, q, k, v, alpha, b, S)

    def output_norm_gate(self, o, g, w, eps: float = 1e-5, act: str = "sigmoid"):
        return _output_norm_gate(self.lib, o, g, w, eps, act)

    def prologue(self, xq, xk, xv, w, beta_raw, delta, g_log, hist_in=None, cu_seqlens=None,
                 act: str = "silu", floor: float = -5.0, l2_eps: float = 1e-6):
        return _prologue(self.lib, xq, xk, xv, w, beta_raw, delta, g_log, hist_in, cu_seqlens,
                         act, floor, l2_eps)


def default() -> Oracle:
    """The oracle build the module-level functions use: liboracle.so beside
    oracle.c, or the build that RDA_ORACLE_LIB names (the tests use this to
    run the pins on a sanitizer build)."""
    global _default
    if _default is None:
        _default = Oracle(os.environ.get("RDA_ORACLE_LIB", _LIB))
    return _default


def _f32(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def threads_used(threads: int = 0) -> int:
    return default().threads_used(threads)


def prefill(q, k, v, a, b, cu_seqlens=None, S0=None, threads: int = 0):
    """Sequential fp64 prefill with the default oracle build (see _prefill)."""
    return default().prefill(q, k, v, a, b, cu_seqlens, S0, threads)


def decode_step(q, k, v, a, b, S, threads: int = 0):
    """One in-place fp64 decode step with the default build (see _decode_step)."""
    return default().decode_step(q, k, v, a, b, S, threads)


def decode_tokens(q, k, v, a, b, S_in, accept=None, threads: int = 0):
    """Several tokens per sequence with the default build (see _decode_tokens)."""
    return default().decode_tokens(q, k, v, a, b, S_in, accept, threads)


def decode_tokens_diag(q, k, v, alpha, b, S_in, accept=None, threads: int = 0):
    """Several tokens per sequence with a per-key-channel decay alpha
    [B, T, H, dk] (see _decode_tokens and _prefill_diag)."""
    return default().decode_tokens_diag(q, k, v, alpha, b, S_in, accept, threads)


def prefill_diag(q, k, v, alpha, b, cu_seqlens=None, S0=None, threads: int = 0):
    """Per-channel-decay prefill with the default build (see _prefill_diag)."""
    return default().prefill_diag(q, k, v, alpha, b, cu_seqlens, S0, threads)


def decode_step_diag(q, k, v, alpha, b, S):
    """Per-channel-decay decode step with the default build."""
    return default().decode_step_diag(q, k, v, alpha, b, S)


def _prefill_diag(lib, q, k, v, alpha, b, cu_seqlens=None, S0=None, threads: int = 0):
    """Sequential fp64 prefill with a per-key-channel decay (oracle.c,
    oracle_rda_prefill_diag): alpha [T, H, dk] in (0, 1]; the rest as in
    _prefill.  Returns (o [T, H, dv], S_final [N, H, dv, dk]) float64."""
    q, k, v, alpha, b = (_f32(x) for x in (q, k, v, alpha, b))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert alpha.shape == (T, H, dk) and b.shape == (T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu, N = None, 1
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (N, H, dv, dk)
    o = np.zeros((T, H, dv))
    S_final = np.zeros((N, H, dv, dk))
    rc = lib.oracle_rda_prefill_diag(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(cu),
                                     N, T, H, dk, dv, _ptr(S0), _ptr(o), _ptr(S_final),
                                     int(threads))
    if rc != 0:
        raise ValueError(f"oracle_rda_prefill_diag failed with code {rc}")
    return o, S_final


def _decode_step_diag(lib, q, k, v, alpha, b, S):
    """One in-place fp64 decode step with a per-key-channel decay on S
    [B, H, dv, dk] (float64, modified); alpha [B, H, dk].  Returns o."""
    q, k, v, alpha, b = (_f32(x) for x in (q, k, v, alpha, b))
    B, H, dk = q.shape
    dv = v.shape[2]
    assert isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous
    assert S.shape == (B, H, dv, dk) and alpha.shape == (B, H, dk)
    o = np.zeros((B, H, dv))
    rc = lib.oracle_rda_decode_step_diag(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), B, H,
                                         dk, dv, _ptr(S), _ptr(o))
    if rc != 0:
        raise ValueError(f"oracle_rda_decode_step_diag failed with code {rc}")
    return o


def output_norm_gate(o, g, w, eps: float = 1e-5, act: str = "sigmoid"):
    """Output epilogue with the default build (see _output_norm_gate)."""
    return default().output_norm_gate(o, g, w, eps, act)


GATE_ACTS = {"sigmoid": 0, "silu": 1, "none": 2}
CONV_ACTS = {"none": 0, "silu": 1}


def prologue(xq, xk, xv, w, beta_raw, delta, g_log, hist_in=None, cu_seqlens=None,
             act: str = "silu", floor: float = -5.0, l2_eps: float = 1e-6):
    """Prologue with the default build (see _prologue)."""
    return default().prologue(xq, xk, xv, w, beta_raw, delta, g_log, hist_in, cu_seqlens,
                              act, floor, l2_eps)


def _prologue(lib, xq, xk, xv, w, beta_raw, delta, g_log, hist_in=None, cu_seqlens=None,
              act="silu", floor=-5.0, l2_eps=1e-6):
    """The steps between the projections and the recurrence (oracle.c,
    oracle_prologue): causal short convolution with history, activation,
    q / k L2 norm, the write gate on v, b = sigmoid(beta_raw) and the
    floored decay.

    xq, xk, xv: raw [T, H, d]; w: [3, H, d, K] (q, k, v; tap K-1 multiplies
    the current token); beta_raw, g_log: [T, H]; delta: [T, H] or None;
    hist_in: [N, 3, K-1, H, d] or None (zeros); cu_seqlens: [N+1] or None.
    Returns (q, k, v [T, H, d], a, b [T, H], hist_out [N, 3, K-1, H, d]),
    all float64.
    """
    xq, xk, xv, beta_raw, g_log = (_f32(x) for x in (xq, xk, xv, beta_raw, g_log))
    T, H, d = xq.shape
    w = _f32(w)
    K = w.shape[-1]
    assert w.shape == (3, H, d, K)
    delta = None if delta is None else _f32(delta)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu, N = None, 1
    if hist_in is not None:
        hist_in = _f32(hist_in)
        assert hist_in.shape == (N, 3, K - 1, H, d)
    q, k, v = (np.zeros((T, H, d)) for _ in range(3))
    a, b = np.zeros((T, H)), np.zeros((T, H))
    hist_out = np.zeros((N, 3, K - 1, H, d))
    rc = lib.oracle_prologue(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(w), K, CONV_ACTS[act],
                             _ptr(hist_in), _ptr(beta_raw), _ptr(delta), _ptr(g_log),
                             float(floor), float(l2_eps), _ptr(cu), N, T, H, d, _ptr(q),
                             _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(hist_out))
    if rc != 0:
        raise ValueError(f"oracle_prologue failed with code {rc}")
    return q, k, v, a, b, hist_out


def _output_norm_gate(lib, o, g, w, eps=1e-5, act="sigmoid"):
    """Per row of the last axis: RMS norm with eps and weight w, times act(g).

    o, g: [..., dv] (values exactly representable in fp32); w: [dv] or None;
    act: "sigmoid", "silu" or "none" (g may then be None).
    Returns float64 of o's shape.
    """
    o = _f32(o)
    dv = o.shape[-1]
    rows = o.size // dv if dv else 0
    g = None if g is None else _f32(g)
    if g is not None:
        assert g.shape == o.shape
    w = None if w is None else _f32(w)
    if w is not None:
        assert w.shape == (dv,)
    out = np.zeros(o.shape, dtype=np.float64)
    rc = lib.oracle_output_norm_gate(_ptr(o), _ptr(g), _ptr(w), float(eps), GATE_ACTS[act],
                                     rows, dv, _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_output_norm_gate failed with code {rc}")
    return out


def _prefill(lib, q, k, v, a, b, cu_seqlens=None, S0=None, threads: int = 0):
    """Sequential fp64 prefill.

    q, k: [T, H, dk]; v: [T, H, dv]; a, b: [T, H] -- any float dtype that is
    exactly representable in fp32 (fp32 or bf16 values widened to fp32).
    cu_seqlens: int32 [N+1] or None (one sequence); S0: [N, H, dv, dk] or None.
    Returns (o [T, H, dv] float64, S_final [N, H, dv, dk] float64).
    """
    q, k, v, a, b = (_f32(x) for x in (q, k, v, a, b))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and v.shape[:2] == (T, H)
    assert a.shape == (T, H) and b.shape == (T, H)
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
    else:
        cu, N = None, 1
    if S0 is not None:
        S0 = _f64(S0)
        assert S0.shape == (N, H, dv, dk)
    o = np.zeros((T, H, dv), dtype=np.float64)
    S_final = np.zeros((N, H, dv, dk), dtype=np.float64)
    rc = lib.oracle_rda_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                _ptr(cu), N, T, H, dk, dv, _ptr(S0), _ptr(o),
                                _ptr(S_final), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_rda_prefill failed with code {rc}")
    return o, S_final


def _decode_step(lib, q, k, v, a, b, S, threads: int = 0):
    """One in-place fp64 decode step on S [B, H, dv, dk] (float64, modified).

    Returns o [B, H, dv] float64.
    """
    q, k, v, a, b = (_f32(x) for x in (q, k, v, a, b))
    B, H, dk = q.shape
    dv = v.shape[2]
    assert isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous
    assert S.shape == (B, H, dv, dk)
    o = np.zeros((B, H, dv), dtype=np.float64)
    rc = lib.oracle_rda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                    B, H, dk, dv, _ptr(S), _ptr(o), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_rda_decode_step failed with code {rc}")
    return o


def _decode_tokens(lib, q, k, v, a, b, S_in, accept=None, threads: int = 0, prefill=None):
    """Several tokens per sequence: the verify of drafted tokens.

    The "Raon-1-nano-gguf" model card runs the model with multi-token
    prediction proposing two drafts per step; verifying them feeds the
    current token and its drafts through the recurrence in order and keeps
    the state only up to the last accepted token.  So: the T tokens of
    sequence n run through the recurrence from S_in[n]; o holds every
    token's output and S the state after the first accept[n] tokens.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; a, b: [B, T, H]; S_in: [B, H, dv, dk];
    accept: ints [B] in [0, T], or None for T.  `prefill` is the recurrence
    the tokens run through (_prefill, or _prefill_diag with a [B, T, H, dk]).
    Returns (o [B, T, H, dv] float64, S [B, H, dv, dk] float64).
    """
    prefill = _prefill if prefill is None else prefill
    q, k, v, a, b = (_f32(x) for x in (q, k, v, a, b))
    B, T, H, dk = q.shape
    dv = v.shape[3]
    S_in = _f64(S_in)
    assert S_in.shape == (B, H, dv, dk)
    acc = np.full(B, T, dtype=np.int64) if accept is None else np.asarray(accept, np.int64)
    assert acc.shape == (B,) and np.all((acc >= 0) & (acc <= T))

    def packed(x, rows):
        return np.ascontiguousarray(x.reshape((B * T,) + x.shape[2:])[rows])

    every = np.arange(B * T)
    cu = (T * np.arange(B + 1)).astype(np.int32)
    o, _ = prefill(lib, *(packed(x, every) for x in (q, k, v, a, b)), cu_seqlens=cu,
                    S0=S_in, threads=threads)
    kept = np.concatenate([n * T + np.arange(acc[n]) for n in range(B)] + [np.zeros(0, int)])
    cu_kept = np.concatenate([[0], np.cumsum(acc)]).astype(np.int32)
    _, S = prefill(lib, *(packed(x, kept) for x in (q, k, v, a, b)), cu_seqlens=cu_kept,
                    S0=S_in, threads=threads)
    return o.reshape(B, T, H, dv), S
