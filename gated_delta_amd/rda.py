"""Thin Python binding of librda.so (argument marshalling only).

Every function here has the name of the C entry point it calls (see
``include/rda.h``) and does no arithmetic of its own: it checks tensor
dtypes, devices and shapes, allocates outputs and the workspace with
``torch.empty`` on the caller's device, validates ``cu_seqlens`` on a host
copy, and passes raw device pointers plus the current HIP stream.  If the
library is not built, the first call raises -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch  # imported before librda.so so both share one HIP runtime

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librda.so")
_lib = None

RDA_BF16 = 0
RDA_FP32 = 1
RDA_CHUNK = 64
RDA_HEAD_DIM = 128
RDA_DECODE_MAX_TOKENS = 64
RDA_GATE_SIGMOID, RDA_GATE_SILU, RDA_GATE_NONE = 0, 1, 2
RDA_CONV_MAX_WIDTH = 4
RDA_CONV_ACT_NONE, RDA_CONV_ACT_SILU = 0, 1
_CONV_ACTS = {"none": RDA_CONV_ACT_NONE, "silu": RDA_CONV_ACT_SILU}
_GATE_ACTS = {"sigmoid": RDA_GATE_SIGMOID, "silu": RDA_GATE_SILU, "none": RDA_GATE_NONE}
RDA_STAGE_TABLE, RDA_STAGE_PREP, RDA_STAGE_WALK = 0, 1, 2
RDA_NUM_STAGES = 3
STAGES = ("table", "prep", "walk")


class RdaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = int(status)
        super().__init__(f"{where}: status {status} ({rda_status_string(status)})")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is not built; run `python -m gated_delta_amd.build` "
                "(the RDA kernels have no non-HIP fallback)")
        lib = ctypes.CDLL(_LIB_PATH)
        p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        lib.rda_abi_version.argtypes = []
        lib.rda_abi_version.restype = ctypes.c_int
        lib.rda_status_string.argtypes = [ctypes.c_int]
        lib.rda_status_string.restype = ctypes.c_char_p
        lib.rda_max_chunks.argtypes = [i32, i32]
        lib.rda_max_chunks.restype = i32
        lib.rda_prefill_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.rda_prefill_workspace_bytes.restype = sz
        pre = [p, p, p, ctypes.c_int, p, p, p, i32, i32, i32, i32, i32, p, p, p, p, sz, p]
        lib.rda_prefill.argtypes = pre
        lib.rda_prefill.restype = ctypes.c_int
        lib.rda_prefill_profiled.argtypes = pre + [p]
        lib.rda_prefill_profiled.restype = ctypes.c_int
        lib.rda_prefill_noalloc.argtypes = pre[:15] + [p]
        lib.rda_prefill_noalloc.restype = ctypes.c_int
        lib.rda_decode_step.argtypes = [p, p, p, ctypes.c_int, p, p, i32, i32, i32, i32, p, p, p]
        lib.rda_decode_step.restype = ctypes.c_int
        lib.rda_decode_tokens.argtypes = [p, p, p, ctypes.c_int, p, p, i32, i32, i32, i32, i32,
                                          p, p, p, p, p]
        lib.rda_decode_tokens.restype = ctypes.c_int
        lib.rda_decode_tokens_diag.argtypes = lib.rda_decode_tokens.argtypes
        lib.rda_decode_tokens_diag.restype = ctypes.c_int
        lib.rda_output_norm_gate.argtypes = [p, p, ctypes.c_int, p, ctypes.c_float, i32,
                                             ctypes.c_int64, i32, p, ctypes.c_int, p]
        lib.rda_output_norm_gate.restype = ctypes.c_int
        lib.rda_prologue.argtypes = [p, p, p, ctypes.c_int, p, i32, i32, p, p, p, p, p,
                                     ctypes.c_float, ctypes.c_float, p, i32, i32, i32, i32,
                                     p, p, p, p, p, p]
        lib.rda_prologue.restype = ctypes.c_int
        lib.rda_decode_step_prologue.argtypes = [p, p, p, ctypes.c_int, p, i32, i32, p, p, p, p,
                                                 p, ctypes.c_float, ctypes.c_float, i32, i32, i32,
                                                 i32, p, p, p]
        lib.rda_decode_step_prologue.restype = ctypes.c_int
        lib.rda_prefill_diag_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.rda_prefill_diag_workspace_bytes.restype = ctypes.c_size_t
        lib.rda_prefill_diag.argtypes = pre[:18]
        lib.rda_prefill_diag.restype = ctypes.c_int
        lib.rda_decode_step_diag.argtypes = [p, p, p, ctypes.c_int, p, p, i32, i32, i32, i32,
                                             p, p, p]
        lib.rda_decode_step_diag.restype = ctypes.c_int
        lib.rda_prefill_norm_gate_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
        lib.rda_prefill_norm_gate_workspace_bytes.restype = sz
        lib.rda_prefill_norm_gate.argtypes = pre[:13] + [p, ctypes.c_int, p, ctypes.c_float, i32,
                                                         p, ctypes.c_int, p, p, sz, p]
        lib.rda_prefill_norm_gate.restype = ctypes.c_int
        lib.rda_chunk_table.argtypes = [p, i32, i32, p, p, p, p]
        lib.rda_chunk_table.restype = ctypes.c_int
        _lib = lib
    return _lib


def lib():
    """The loaded ctypes library (loads it on first use)."""
    return _load()


# ---------------------------------------------------------------------------
# plain queries
# ---------------------------------------------------------------------------
def rda_abi_version() -> int:
    return int(_load().rda_abi_version())


def rda_status_string(status: int) -> str:
    return _load().rda_status_string(int(status)).decode()


def rda_max_chunks(num_seqs: int, total_tokens: int) -> int:
    return int(_load().rda_max_chunks(int(num_seqs), int(total_tokens)))


def rda_prefill_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int,
                                dk: int = RDA_HEAD_DIM, dv: int = RDA_HEAD_DIM) -> int:
    return int(_load().rda_prefill_workspace_bytes(int(num_seqs), int(total_tokens),
                                                   int(num_heads), int(dk), int(dv)))


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _qkv_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RDA_BF16
    if t.dtype == torch.float32:
        return RDA_FP32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _stream_handle(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_cu_seqlens(cu, total_tokens: int) -> np.ndarray:
    """Host-side validation of packed-sequence offsets; returns int32 array."""
    if isinstance(cu, torch.Tensor):
        cu = cu.detach().to("cpu").numpy()
    cu = np.asarray(cu)
    if cu.ndim != 1 or cu.shape[0] < 2:
        raise ValueError("cu_seqlens must be 1-D with at least 2 entries")
    if not np.issubdtype(cu.dtype, np.integer):
        raise TypeError("cu_seqlens must be integers")
    cu64 = cu.astype(np.int64)
    if cu64[0] != 0:
        raise ValueError("cu_seqlens[0] must be 0")
    if np.any(np.diff(cu64) < 0):
        raise ValueError("cu_seqlens must be non-decreasing")
    if cu64[-1] != total_tokens:
        raise ValueError(f"cu_seqlens[-1] = {cu64[-1]} != total tokens {total_tokens}")
    if cu64[-1] > np.iinfo(np.int32).max:
        raise ValueError("cu_seqlens exceeds int32")
    return cu64.astype(np.int32)


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def rda_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                b: torch.Tensor, cu_seqlens=None, S0: Optional[torch.Tensor] = None, *,
                o: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                want_state: bool = True, workspace: Optional[torch.Tensor] = None,
                stream=None, stage_events: Optional[Sequence] = None):
    """Chunked RDA prefill (C entry point ``rda_prefill``).

    q, k [T, H, 128] and v [T, H, 128] (bf16 or fp32, same dtype), a, b
    [T, H] fp32, cu_seqlens (host or device int offsets, [N+1]) or None,
    S0 [N, H, 128, 128] fp32 or None.  Returns (o [T, H, 128] fp32,
    S_final [N, H, 128, 128] fp32 or None).  ``S_final`` may be passed as
    the same tensor as ``S0`` to resume in place.  ``stage_events``: six
    recorded-once torch.cuda.Event objects (start/stop per stage) to time
    the kernels on the launch stream.
    """
    lib_ = _load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(q)
    _need(q, "q", q.dtype, (T, H, dk), dev)
    _need(k, "k", q.dtype, (T, H, dk), dev)
    _need(v, "v", q.dtype, (T, H, dv), dev)
    _need(a, "a", torch.float32, (T, H), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    if cu_seqlens is not None:
        cu_host = check_cu_seqlens(cu_seqlens, T)
        N = cu_host.shape[0] - 1
        if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device == dev \
                and cu_seqlens.dtype == torch.int32 and cu_seqlens.is_contiguous():
            cu_dev = cu_seqlens
        else:
            cu_dev = torch.from_numpy(cu_host).to(dev)
    else:
        N, cu_dev = 1, None
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dv, dk), dev)
    if o is None:
        o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (T, H, dv), dev)
    if S_final is None and want_state:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _need(S_final, "S_final", torch.float32, (N, H, dv, dk), dev)
    need = rda_prefill_workspace_bytes(N, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    args = [_ptr(q), _ptr(k), _ptr(v), dt, _ptr(a), _ptr(b), _ptr(cu_dev), N, T, H, dk, dv,
            _ptr(S0), _ptr(o), _ptr(S_final), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_handle(stream)]
    if stage_events is not None:
        if len(stage_events) != 2 * RDA_NUM_STAGES:
            raise ValueError("stage_events needs 2 events per stage")
        arr = (ctypes.c_void_p * (2 * RDA_NUM_STAGES))(
            *[None if e is None else ctypes.c_void_p(e.cuda_event) for e in stage_events])
        st = lib_.rda_prefill_profiled(*args, arr)
    else:
        st = lib_.rda_prefill(*args)
    if st != 0:
        raise RdaError(st, "rda_prefill")
    return o, S_final


RDA_NOALLOC_SCRATCH_BYTES = 64 << 20
RDA_ERR_TOO_LARGE = 10


def rda_prefill_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                        b: torch.Tensor, cu_seqlens: Optional[torch.Tensor] = None,
                        S0: Optional[torch.Tensor] = None, *, o: torch.Tensor,
                        S_final: Optional[torch.Tensor] = None, stream=None):
    """rda_prefill without a workspace (C entry point ``rda_prefill_noalloc``):
    the library's fixed per-GPU scratch holds the chunk table and factors, so
    the call allocates nothing.  The caller passes every output (o, and
    S_final or None), and cu_seqlens, when given, as a device int32 tensor
    (no host copy is made).  Raises RdaError with RDA_ERR_TOO_LARGE when the
    sizes need more than RDA_NOALLOC_SCRATCH_BYTES."""
    lib_ = _load()
    dev = q.device
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(q)
    for name, t, shape in (("q", q, (T, H, dk)), ("k", k, (T, H, dk)), ("v", v, (T, H, dv))):
        _need(t, name, q.dtype, shape, dev)
    _need(a, "a", torch.float32, (T, H), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    N = 1
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with at least 2 entries")
        N = cu_seqlens.numel() - 1
        _need(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,), dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dv, dk), dev)
    _need(o, "o", torch.float32, (T, H, dv), dev)
    if S_final is not None:
        _need(S_final, "S_final", torch.float32, (N, H, dv, dk), dev)
    st = lib_.rda_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(a), _ptr(b),
                                  _ptr(cu_seqlens), N, T, H, dk, dv, _ptr(S0), _ptr(o),
                                  _ptr(S_final), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_prefill_noalloc")
    return o, S_final


def rda_decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                    b: torch.Tensor, S: torch.Tensor, *, o: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """One in-place decode step (C entry point ``rda_decode_step``).

    q, k, v [B, H, 128] (bf16 or fp32), a, b [B, H] fp32, S [B, H, 128, 128]
    fp32 (updated in place).  Returns o [B, H, 128] fp32.
    """
    lib_ = _load()
    dev = q.device
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(q)
    _need(q, "q", q.dtype, (B, H, dk), dev)
    _need(k, "k", q.dtype, (B, H, dk), dev)
    _need(v, "v", q.dtype, (B, H, dv), dev)
    _need(a, "a", torch.float32, (B, H), dev)
    _need(b, "b", torch.float32, (B, H), dev)
    _need(S, "S", torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, H, dv), dev)
    st = lib_.rda_decode_step(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(a), _ptr(b), B, H, dk, dv,
                              _ptr(S), _ptr(o), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_decode_step")
    return o


_NO_OUTPUT = object()


def _decode_tokens(name, q, k, v, a, b, S_in, S_out, accept, o, stream, diag):
    lib_ = _load()
    dev = k.device
    if k.dim() != 4:
        raise ValueError(f"k must be [B, T, H, d], got shape {tuple(k.shape)}")
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(k)
    want_o = o is not False
    if want_o:
        if q is None:
            raise ValueError("q is required when outputs are produced")
        _need(q, "q", k.dtype, (B, T, H, dk), dev)
    _need(k, "k", k.dtype, (B, T, H, dk), dev)
    _need(v, "v", k.dtype, (B, T, H, dv), dev)
    if diag:
        _need(a, "alpha", torch.float32, (B, T, H, dk), dev)
    else:
        _need(a, "a", torch.float32, (B, T, H), dev)
    _need(b, "b", torch.float32, (B, T, H), dev)
    _need(S_in, "S_in", torch.float32, (B, H, dv, dk), dev)
    if S_out is not None:
        _need(S_out, "S_out", torch.float32, (B, H, dv, dk), dev)
    if accept is not None:
        _need(accept, "accept", torch.int32, (B,), dev)
    if want_o:
        if o is None:
            o = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
        _need(o, "o", torch.float32, (B, T, H, dv), dev)
    else:
        o = None
    st = getattr(lib_, name)(_ptr(q) if want_o else None, _ptr(k), _ptr(v), dt, _ptr(a),
                             _ptr(b), B, T, H, dk, dv, _ptr(S_in), _ptr(S_out),
                             _ptr(accept), _ptr(o), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, name)
    return o


def rda_decode_tokens(q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor,
                      a: torch.Tensor, b: torch.Tensor, S_in: torch.Tensor, *,
                      S_out: Optional[torch.Tensor] = None,
                      accept: Optional[torch.Tensor] = None, o=None,
                      stream=None) -> Optional[torch.Tensor]:
    """Several tokens per sequence in one pass (C entry point ``rda_decode_tokens``).

    q, k, v [B, T, H, 128] (bf16 or fp32), a, b [B, T, H] fp32, S_in
    [B, H, 128, 128] fp32.  S_out (same shape, may be S_in itself) receives
    the state after the first accept[n] tokens of each sequence (accept
    int32 [B] on the device, None = all T); S_out=None leaves every state
    unchanged.  Returns o [B, T, H, 128] fp32 for every token, or None when
    called with o=False (commit only: q is then not read and may be None).
    """
    return _decode_tokens("rda_decode_tokens", q, k, v, a, b, S_in, S_out, accept, o, stream,
                          False)


def rda_decode_tokens_diag(q: Optional[torch.Tensor], k: torch.Tensor, v: torch.Tensor,
                           alpha: torch.Tensor, b: torch.Tensor, S_in: torch.Tensor, *,
                           S_out: Optional[torch.Tensor] = None,
                           accept: Optional[torch.Tensor] = None, o=None,
                           stream=None) -> Optional[torch.Tensor]:
    """rda_decode_tokens with a per-key-channel decay (C entry point
    ``rda_decode_tokens_diag``): alpha [B, T, H, 128] fp32 in place of a;
    everything else as in rda_decode_tokens."""
    return _decode_tokens("rda_decode_tokens_diag", q, k, v, alpha, b, S_in, S_out, accept, o,
                          stream, True)


def rda_chunk_table(cu_seqlens, num_seqs: int, total_tokens: int, device="cuda",
                    stream=None):
    """The chunk table rda_prefill builds (C entry point ``rda_chunk_table``).

    cu_seqlens: device int32 tensor [N+1] or None.  Returns device tensors
    (rec [max_chunks, 4], seq_offsets [N+1], num_chunks [1]).  The offsets
    are NOT validated here, so malformed tables can be inspected.
    """
    lib_ = _load()
    mc = rda_max_chunks(num_seqs, total_tokens)
    if mc < 0:
        raise ValueError("bad sizes")
    rec = torch.empty((max(mc, 1), 4), dtype=torch.int32, device=device)
    seq_off = torch.empty((num_seqs + 1,), dtype=torch.int32, device=device)
    nch = torch.empty((1,), dtype=torch.int32, device=device)
    st = lib_.rda_chunk_table(_ptr(cu_seqlens), int(num_seqs), int(total_tokens), _ptr(rec),
                              _ptr(seq_off), _ptr(nch), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_chunk_table")
    return rec[:mc], seq_off, nch


def rda_output_norm_gate(o: torch.Tensor, g: Optional[torch.Tensor], *,
                         weight: Optional[torch.Tensor] = None, eps: float = 1e-5,
                         act: str = "sigmoid", out: Optional[torch.Tensor] = None,
                         out_dtype=torch.bfloat16, stream=None) -> torch.Tensor:
    """Output norm and gate (C entry point ``rda_output_norm_gate``).

    o [..., 128] fp32 (rda_prefill's or a decode entry point's output); g the
    gate, same shape, bf16 or fp32 (None with act="none"); weight [128] fp32
    or None; act "sigmoid", "silu" or "none".  Returns out, same shape, in
    out_dtype (bf16 or fp32; an fp32 out may be o itself).
    """
    lib_ = _load()
    dev = o.device
    if o.dtype != torch.float32 or o.dim() < 1:
        raise TypeError("o must be a float32 tensor [..., dv]")
    shape = tuple(o.shape)
    dv = shape[-1]
    rows = o.numel() // dv if dv else 0
    _need(o, "o", torch.float32, shape, dev)
    if act not in _GATE_ACTS:
        raise ValueError(f"act must be one of {sorted(_GATE_ACTS)}")
    g_dt = RDA_BF16
    if act != "none":
        if g is None:
            raise ValueError("g is required unless act='none'")
        g_dt = _qkv_dtype(g)
        _need(g, "g", g.dtype, shape, dev)
    else:
        g = None
    if weight is not None:
        _need(weight, "weight", torch.float32, (dv,), dev)
    o_dt = {torch.bfloat16: RDA_BF16, torch.float32: RDA_FP32}.get(out_dtype)
    if o_dt is None:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if out is None:
        out = torch.empty(shape, dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, shape, dev)
    st = lib_.rda_output_norm_gate(_ptr(o), _ptr(g), g_dt, _ptr(weight), float(eps),
                                   _GATE_ACTS[act], rows, dv, _ptr(out), o_dt,
                                   _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_output_norm_gate")
    return out


def rda_prefill_norm_gate_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int,
                                          dk: int = 128, dv: int = 128) -> int:
    return _load().rda_prefill_norm_gate_workspace_bytes(num_seqs, total_tokens, num_heads, dk,
                                                         dv)


def rda_prefill_norm_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, a: torch.Tensor,
                          b: torch.Tensor, g: Optional[torch.Tensor], cu_seqlens=None,
                          S0: Optional[torch.Tensor] = None, *,
                          weight: Optional[torch.Tensor] = None, eps: float = 1e-5,
                          act: str = "sigmoid", out: Optional[torch.Tensor] = None,
                          out_dtype=torch.bfloat16, S_final: Optional[torch.Tensor] = None,
                          want_state: bool = True, workspace: Optional[torch.Tensor] = None,
                          stream=None):
    """Prefill with the output norm and gate fused (C entry point
    ``rda_prefill_norm_gate``): the arguments of rda_prefill and of
    rda_output_norm_gate (g [T, H, 128] bf16 or fp32, or None with
    act="none").  Returns (out [T, H, 128] in out_dtype, S_final or None);
    no fp32 o is formed."""
    lib_ = _load()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(q)
    _need(q, "q", q.dtype, (T, H, dk), dev)
    _need(k, "k", q.dtype, (T, H, dk), dev)
    _need(v, "v", q.dtype, (T, H, dv), dev)
    _need(a, "a", torch.float32, (T, H), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    if cu_seqlens is not None:
        cu_host = check_cu_seqlens(cu_seqlens, T)
        N = cu_host.shape[0] - 1
        cu_dev = torch.from_numpy(cu_host).to(dev)
    else:
        N, cu_dev = 1, None
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dv, dk), dev)
    if act not in _GATE_ACTS:
        raise ValueError(f"act must be one of {sorted(_GATE_ACTS)}")
    g_dt = RDA_BF16
    if act != "none":
        if g is None:
            raise ValueError("g is required unless act='none'")
        g_dt = _qkv_dtype(g)
        _need(g, "g", g.dtype, (T, H, dv), dev)
    else:
        g = None
    if weight is not None:
        _need(weight, "weight", torch.float32, (dv,), dev)
    o_dt = {torch.bfloat16: RDA_BF16, torch.float32: RDA_FP32}.get(out_dtype)
    if o_dt is None:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if out is None:
        out = torch.empty((T, H, dv), dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (T, H, dv), dev)
    if S_final is None and want_state:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    if S_final is not None:
        _need(S_final, "S_final", torch.float32, (N, H, dv, dk), dev)
    need = rda_prefill_norm_gate_workspace_bytes(N, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib_.rda_prefill_norm_gate(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(a), _ptr(b),
                                    _ptr(cu_dev), N, T, H, dk, dv, _ptr(S0), _ptr(g), g_dt,
                                    _ptr(weight), float(eps), _GATE_ACTS[act], _ptr(out), o_dt,
                                    _ptr(S_final), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_prefill_norm_gate")
    return out, S_final


def rda_prologue(x_q: torch.Tensor, x_k: torch.Tensor, x_v: torch.Tensor,
                 conv_w: torch.Tensor, beta_raw: torch.Tensor, g_log: torch.Tensor, *,
                 delta: Optional[torch.Tensor] = None, hist_in: Optional[torch.Tensor] = None,
                 hist_out: Optional[torch.Tensor] = None, cu_seqlens=None, num_seqs: int = 1,
                 conv_act: str = "silu", decay_floor: float = -5.0, l2_eps: float = 1e-6,
                 stream=None):
    """The block's prologue (C entry point ``rda_prologue``).

    x_q, x_k, x_v [..., H, 128] bf16 raw projections (the leading axes are
    the tokens: [T], or [B] / [B, T] for the decode layouts); conv_w
    [3, H, 128, K] fp32; beta_raw, g_log (and delta) [..., H] fp32; hist_in /
    hist_out [N, 3, K-1, H, 128] bf16 (hist_out may be hist_in when every
    sequence has one token).  cu_seqlens: offsets (host array or tensor,
    checked on the host), or None for num_seqs equal-length sequences.
    Returns q, k, v (bf16, shaped like x_q) and a, b (fp32, shaped like
    beta_raw).
    """
    lib_ = _load()
    dev = x_q.device
    if x_q.dtype != torch.bfloat16:
        raise TypeError("x_q, x_k, x_v must be bfloat16")
    shape = tuple(x_q.shape)
    if len(shape) < 2:
        raise ValueError("x_q must be [..., H, d]")
    H, d = shape[-2], shape[-1]
    lead = shape[:-2]
    T = int(np.prod(lead)) if lead else 1
    for name, t in (("x_q", x_q), ("x_k", x_k), ("x_v", x_v)):
        _need(t, name, torch.bfloat16, shape, dev)
    if conv_w.dim() != 4:
        raise ValueError("conv_w must be [3, H, d, K]")
    K = conv_w.shape[-1]
    _need(conv_w, "conv_w", torch.float32, (3, H, d, K), dev)
    for name, t in (("beta_raw", beta_raw), ("g_log", g_log), ("delta", delta)):
        if t is not None:
            _need(t, name, torch.float32, lead + (H,), dev)
    cu_dev = None
    if cu_seqlens is not None:
        cu_np = check_cu_seqlens(cu_seqlens, T)
        num_seqs = len(cu_np) - 1
        cu_dev = torch.from_numpy(cu_np).to(dev)
    hshape = (num_seqs, 3, max(K - 1, 0), H, d)
    for name, t in (("hist_in", hist_in), ("hist_out", hist_out)):
        if t is not None:
            _need(t, name, torch.bfloat16, hshape, dev)
    if conv_act not in _CONV_ACTS:
        raise ValueError(f"conv_act must be one of {sorted(_CONV_ACTS)}")
    q, k, v = (torch.empty(shape, dtype=torch.bfloat16, device=dev) for _ in range(3))
    a, b = (torch.empty(lead + (H,), dtype=torch.float32, device=dev) for _ in range(2))
    st = lib_.rda_prologue(_ptr(x_q), _ptr(x_k), _ptr(x_v), RDA_BF16, _ptr(conv_w), K,
                           _CONV_ACTS[conv_act], _ptr(hist_in), _ptr(hist_out), _ptr(beta_raw),
                           _ptr(delta), _ptr(g_log), float(decay_floor), float(l2_eps),
                           _ptr(cu_dev), int(num_seqs), T, H, d, _ptr(q), _ptr(k), _ptr(v),
                           _ptr(a), _ptr(b), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_prologue")
    return q, k, v, a, b


def rda_decode_step_prologue(x_q: torch.Tensor, x_k: torch.Tensor, x_v: torch.Tensor,
                             conv_w: torch.Tensor, beta_raw: torch.Tensor, g_log: torch.Tensor,
                             S: torch.Tensor, *, delta: Optional[torch.Tensor] = None,
                             hist_in: Optional[torch.Tensor] = None,
                             hist_out: Optional[torch.Tensor] = None, conv_act: str = "silu",
                             decay_floor: float = -5.0, l2_eps: float = 1e-6,
                             o: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step with the prologue in front (C entry point
    ``rda_decode_step_prologue``): x_q, x_k, x_v [B, H, 128] bf16 raw
    projections, conv_w [3, H, 128, K] fp32, beta_raw, g_log (and delta)
    [B, H] fp32, S [B, H, 128, 128] fp32 updated in place, hist_in / hist_out
    [B, 3, K-1, H, 128] bf16 (hist_out may be hist_in).  Returns o [B, H, 128]."""
    lib_ = _load()
    dev = x_q.device
    if x_q.dtype != torch.bfloat16:
        raise TypeError("x_q, x_k, x_v must be bfloat16")
    if x_q.dim() != 3:
        raise ValueError("x_q must be [B, H, d]")
    B, H, d = x_q.shape
    for name, t in (("x_q", x_q), ("x_k", x_k), ("x_v", x_v)):
        _need(t, name, torch.bfloat16, (B, H, d), dev)
    if conv_w.dim() != 4:
        raise ValueError("conv_w must be [3, H, d, K]")
    K = conv_w.shape[-1]
    _need(conv_w, "conv_w", torch.float32, (3, H, d, K), dev)
    for name, t in (("beta_raw", beta_raw), ("g_log", g_log), ("delta", delta)):
        if t is not None:
            _need(t, name, torch.float32, (B, H), dev)
    for name, t in (("hist_in", hist_in), ("hist_out", hist_out)):
        if t is not None:
            _need(t, name, torch.bfloat16, (B, 3, max(K - 1, 0), H, d), dev)
    _need(S, "S", torch.float32, (B, H, d, d), dev)
    if conv_act not in _CONV_ACTS:
        raise ValueError(f"conv_act must be one of {sorted(_CONV_ACTS)}")
    if o is None:
        o = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, H, d), dev)
    st = lib_.rda_decode_step_prologue(_ptr(x_q), _ptr(x_k), _ptr(x_v), RDA_BF16, _ptr(conv_w),
                                       K, _CONV_ACTS[conv_act], _ptr(hist_in), _ptr(hist_out),
                                       _ptr(beta_raw), _ptr(delta), _ptr(g_log),
                                       float(decay_floor), float(l2_eps), B, H, d, d, _ptr(S),
                                       _ptr(o), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_decode_step_prologue")
    return o


def rda_prefill_diag_workspace_bytes(num_seqs: int, total_tokens: int, num_heads: int,
                                     dk: int = RDA_HEAD_DIM, dv: int = RDA_HEAD_DIM) -> int:
    return int(_load().rda_prefill_diag_workspace_bytes(int(num_seqs), int(total_tokens),
                                                        int(num_heads), int(dk), int(dv)))


def rda_prefill_diag(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                     b: torch.Tensor, *, cu_seqlens=None, S0: Optional[torch.Tensor] = None,
                     o: Optional[torch.Tensor] = None, S_final: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None):
    """Prefill with a per-key-channel decay (C entry point ``rda_prefill_diag``).

    q, k, v [T, H, 128] (bf16 or fp32, same dtype); alpha [T, H, 128] fp32
    in (0, 1]; b [T, H] fp32; the rest as in rda_prefill.  Returns (o, S_final).
    """
    lib_ = _load()
    dev = q.device
    T, H, dk = q.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(q)
    for name, t in (("q", q), ("k", k)):
        _need(t, name, q.dtype, (T, H, dk), dev)
    _need(v, "v", q.dtype, (T, H, dv), dev)
    _need(alpha, "alpha", torch.float32, (T, H, dk), dev)
    _need(b, "b", torch.float32, (T, H), dev)
    cu_dev, N = None, 1
    if cu_seqlens is not None:
        cu_np = check_cu_seqlens(cu_seqlens, T)
        N = len(cu_np) - 1
        cu_dev = torch.from_numpy(cu_np).to(dev)
    if S0 is not None:
        _need(S0, "S0", torch.float32, (N, H, dv, dk), dev)
    if o is None:
        o = torch.empty((T, H, dv), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (T, H, dv), dev)
    if S_final is None:
        S_final = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    _need(S_final, "S_final", torch.float32, (N, H, dv, dk), dev)
    need = rda_prefill_diag_workspace_bytes(N, T, H, dk, dv)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    st = lib_.rda_prefill_diag(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(alpha), _ptr(b),
                               _ptr(cu_dev), N, T, H, dk, dv, _ptr(S0), _ptr(o), _ptr(S_final),
                               _ptr(workspace), workspace.numel(), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_prefill_diag")
    return o, S_final


def rda_decode_step_diag(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor,
                         b: torch.Tensor, S: torch.Tensor, *, o: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """One in-place decode step with a per-key-channel decay (C entry point
    ``rda_decode_step_diag``): alpha [B, H, 128] fp32; the rest as in
    rda_decode_step.  Returns o [B, H, 128] fp32."""
    lib_ = _load()
    dev = q.device
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _qkv_dtype(q)
    _need(q, "q", q.dtype, (B, H, dk), dev)
    _need(k, "k", q.dtype, (B, H, dk), dev)
    _need(v, "v", q.dtype, (B, H, dv), dev)
    _need(alpha, "alpha", torch.float32, (B, H, dk), dev)
    _need(b, "b", torch.float32, (B, H), dev)
    _need(S, "S", torch.float32, (B, H, dv, dk), dev)
    if o is None:
        o = torch.empty((B, H, dv), dtype=torch.float32, device=dev)
    _need(o, "o", torch.float32, (B, H, dv), dev)
    st = lib_.rda_decode_step_diag(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(alpha), _ptr(b), B, H,
                                   dk, dv, _ptr(S), _ptr(o), _stream_handle(stream))
    if st != 0:
        raise RdaError(st, "rda_decode_step_diag")
    return o
