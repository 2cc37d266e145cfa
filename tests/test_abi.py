"""The C-ABI library on the CPU: it loads, exports every entry point the
public header declares, sizes workspaces, and rejects bad arguments with the
documented status before anything reaches a device (no compute calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

import table_ref
from gated_delta_amd import rda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rda.h")

OK, NULL, SHAPE, UNSUP, DTYPE, WS, ALIGN, HIPERR, ALIAS, VALUE, TOO_LARGE = range(11)
P = 1 << 40          # fake, well-aligned device addresses: never dereferenced
GiB = 1 << 30


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rda.library_path()):
        import gated_delta_amd.build as b
        b.build()
    return rda.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rda_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rda_prefill", "rda_decode_step", "rda_decode_tokens", "rda_prefill_diag",
              "rda_decode_step_diag", "rda_decode_tokens_diag", "rda_prologue", "rda_output_norm_gate",
              "rda_prefill_workspace_bytes", "rda_prefill_noalloc", "rda_decode_step_prologue",
              "rda_chunk_table", "rda_abi_version", "rda_status_string", "rda_prefill_norm_gate",
              "rda_prefill_norm_gate_workspace_bytes"):
        assert n in names


def test_binding_constants_match_header():
    text = open(HEADER).read()
    vals = {m[0]: int(m[1]) for m in re.findall(r"\b(RDA_[A-Z0-9_]+)\s*=\s*(\d+)", text)}
    vals.update({m[0]: int(m[1]) for m in
                 re.findall(r"#define\s+(RDA_[A-Z0-9_]+)\s+(\d+)", text)})
    for name in ("RDA_BF16", "RDA_FP32", "RDA_CHUNK", "RDA_HEAD_DIM", "RDA_DECODE_MAX_TOKENS",
                 "RDA_GATE_SIGMOID", "RDA_GATE_SILU", "RDA_GATE_NONE", "RDA_CONV_MAX_WIDTH",
                 "RDA_CONV_ACT_NONE", "RDA_CONV_ACT_SILU",
                 "RDA_STAGE_TABLE",
                 "RDA_STAGE_PREP", "RDA_STAGE_WALK", "RDA_NUM_STAGES"):
        assert getattr(rda, name) == vals[name], name


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"librda.so does not export {name}"


def test_version_and_status_strings(lib):
    assert rda.rda_abi_version() == 1
    for s in range(11):
        assert rda.rda_status_string(s) and rda.rda_status_string(s) != "unknown status"
    assert rda.rda_status_string(99) == "unknown status"


def test_max_chunks_matches_reference(lib):
    for N, T in [(1, 0), (1, 1), (1, 64), (1, 65), (8, 32768), (3, 5), (1000, 123457)]:
        assert rda.rda_max_chunks(N, T) == table_ref.max_chunks(N, T)
    assert rda.rda_max_chunks(0, 5) == -1 and rda.rda_max_chunks(1, -1) == -1


def test_workspace_covers_the_segmented_pass(lib):
    """One sequence with few heads gets room for three [P, H, 128, 128]
    state arrays; with 16 heads, or two sequences, it does not."""
    seg = rda.rda_prefill_workspace_bytes(1, 16384, 2)
    two = rda.rda_prefill_workspace_bytes(2, 16384, 2)
    assert seg - two >= 3 * 8 * 2 * 128 * 128 * 4 - 2 * 2 * 131584
    # short sequences keep the one-pass walk: no room for P >= 4 segments
    short = rda.rda_prefill_workspace_bytes(1, 2048, 2) - rda.rda_prefill_workspace_bytes(2, 2048, 2)
    assert short < 3 * 4 * 2 * 128 * 128 * 4


def test_workspace_covers_the_overlapped_plan(lib):
    """One sequence of 16 heads and at least 32 chunks gets room for one
    [H, 128, 128] state (the state the overlapped plan hands from its middle
    launch to its last); two sequences, or fewer chunks, get none."""
    W = rda.rda_prefill_workspace_bytes
    H, state = 16, 16 * 128 * 128 * 4
    per_chunk = W(2, 16384 + 64, H) - W(2, 16384, H)   # factors of one chunk, all heads
    assert per_chunk > 0
    extra = W(1, 16384, H) - 256 * per_chunk            # table + middle state
    assert state <= extra < state + 64 * 1024
    extra_two = W(2, 16384 - 64, H) - 256 * per_chunk    # 256 chunks, no middle state
    assert 0 < extra_two < 64 * 1024
    short = W(1, 31 * 64, H) - 31 * per_chunk            # 31 chunks: no overlap
    assert 0 < short < 64 * 1024


def test_workspace_bytes(lib):
    w1 = rda.rda_prefill_workspace_bytes(1, 16384, 16)
    w2 = rda.rda_prefill_workspace_bytes(1, 16384, 8)
    assert w1 > w2 > 0 and w1 % 256 == 0
    assert rda.rda_prefill_workspace_bytes(1, 16384, 16, 64, 64) == 0
    assert rda.rda_prefill_workspace_bytes(1, 0, 16) > 0


def _prefill(lib, q=P, k=P + GiB, v=P + 2 * GiB, dt=0, a=P + 3 * GiB, b=P + 4 * GiB,
             cu=None, N=1, T=128, H=2, dk=128, dv=128, S0=None, o=P + 5 * GiB,
             Sf=P + 6 * GiB, ws=P + 7 * GiB, wsb=None):
    if wsb is None:
        wsb = rda.rda_prefill_workspace_bytes(N, T, H, 128, 128) if (dk, dv) == (128, 128) else 1 << 30
    return lib.rda_prefill(q, k, v, dt, a, b, cu, N, T, H, dk, dv, S0, o, Sf, ws, wsb, None)


def test_prefill_rejects_bad_arguments(lib):
    assert _prefill(lib, q=None) == NULL
    assert _prefill(lib, o=None) == NULL
    assert _prefill(lib, dt=7) == DTYPE
    assert _prefill(lib, T=-1) == SHAPE
    assert _prefill(lib, N=0) == SHAPE
    assert _prefill(lib, N=2) == SHAPE           # several sequences need cu_seqlens
    assert _prefill(lib, H=0) == SHAPE
    assert _prefill(lib, dk=64) == UNSUP
    assert _prefill(lib, dk=128, dv=256) == UNSUP
    assert _prefill(lib, ws=None) == WS
    assert _prefill(lib, wsb=1024) == WS
    assert _prefill(lib, q=P + 8) == ALIGN
    assert _prefill(lib, Sf=P + 6 * GiB + 4) == ALIGN
    assert _prefill(lib, cu=P + 9 * GiB + 2, N=2) == ALIGN
    assert _prefill(lib, o=P + 16) == ALIAS             # o overlaps q
    assert _prefill(lib, Sf=P + 2 * GiB) == ALIAS       # S_final overlaps v
    assert _prefill(lib, ws=P + 5 * GiB + 256) == ALIAS  # workspace overlaps o
    # S0 == S_final (in-place resume) is allowed to pass validation; a partial
    # overlap is not
    assert _prefill(lib, S0=P + 6 * GiB + 1024, Sf=P + 6 * GiB) == ALIAS


def test_noalloc_scratch_constants_match_header():
    text = open(HEADER).read()
    m = re.search(r"#define\s+RDA_NOALLOC_SCRATCH_BYTES\s+\(\(size_t\)(\d+)\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == rda.RDA_NOALLOC_SCRATCH_BYTES
    assert re.search(r"RDA_ERR_TOO_LARGE\s*=\s*10", text) and rda.RDA_ERR_TOO_LARGE == 10


def _noalloc(lib, q=P, k=P + GiB, v=P + 2 * GiB, dt=0, a=P + 3 * GiB, b=P + 4 * GiB, cu=None,
             N=1, T=1000, H=4, dk=128, dv=128, S0=None, o=P + 5 * GiB, Sf=P + 6 * GiB):
    return lib.rda_prefill_noalloc(q, k, v, dt, a, b, cu, N, T, H, dk, dv, S0, o, Sf, None)


def test_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """Checked on the host before any device call: sizes whose workspace would
    exceed the fixed scratch, and the other size / dtype errors."""
    cap = rda.RDA_NOALLOC_SCRATCH_BYTES
    assert rda.rda_prefill_workspace_bytes(1, 16384, 16) > cap
    assert _noalloc(lib, T=16384, H=16) == TOO_LARGE
    assert _noalloc(lib, T=1 << 20, H=1) == TOO_LARGE
    # the largest single-sequence prompt of 16 heads that fits, and one more chunk
    T = 64
    while rda.rda_prefill_workspace_bytes(1, T + 64, 16) <= cap:
        T += 64
    assert rda.rda_prefill_workspace_bytes(1, T, 16) <= cap
    assert _noalloc(lib, T=T + 64, H=16) == TOO_LARGE
    assert _noalloc(lib, dt=7) == DTYPE
    assert _noalloc(lib, T=-1) == SHAPE
    assert _noalloc(lib, N=0) == SHAPE
    assert _noalloc(lib, N=2) == SHAPE
    assert _noalloc(lib, H=0) == SHAPE
    assert _noalloc(lib, dk=64) == UNSUP


def _dprol(lib, xq=P, xk=P + GiB, xv=P + 2 * GiB, dt=0, w=P + 3 * GiB, K=4, act=1,
           hin=P + 4 * GiB, hout=P + 4 * GiB, beta=P + 5 * GiB, delta=None, glog=P + 6 * GiB,
           floor=-5.0, eps=1e-6, B=8, H=16, dk=128, dv=128, S=P + 7 * GiB, o=P + 8 * GiB):
    return lib.rda_decode_step_prologue(xq, xk, xv, dt, w, K, act, hin, hout, beta, delta, glog,
                                        floor, eps, B, H, dk, dv, S, o, None)


def test_decode_step_prologue_rejects_bad_arguments(lib):
    assert _dprol(lib, dt=1) == UNSUP
    assert _dprol(lib, dt=5) == DTYPE
    assert _dprol(lib, K=0) == VALUE
    assert _dprol(lib, K=5) == VALUE
    assert _dprol(lib, act=3) == VALUE
    assert _dprol(lib, floor=float("nan")) == VALUE
    assert _dprol(lib, eps=-1.0) == VALUE
    assert _dprol(lib, B=-1) == SHAPE
    assert _dprol(lib, H=0) == SHAPE
    assert _dprol(lib, dk=64) == UNSUP
    assert _dprol(lib, B=0, xq=None) == OK          # nothing to do, nothing read
    assert _dprol(lib, xq=None) == NULL
    assert _dprol(lib, S=None) == NULL
    assert _dprol(lib, o=None) == NULL
    assert _dprol(lib, xk=P + GiB + 8) == ALIGN
    assert _dprol(lib, o=P + 16) == ALIAS                   # o overlaps x_q
    assert _dprol(lib, S=P + 5 * GiB) == ALIAS              # S overlaps beta_raw
    assert _dprol(lib, hout=P + 4 * GiB + 256) == ALIAS     # history out overlaps history in
    assert _dprol(lib, o=P + 7 * GiB + 1024) == ALIAS       # o overlaps S


def test_decode_rejects_bad_arguments(lib):
    def dec(q=P, k=P + GiB, v=P + 2 * GiB, dt=0, a=P + 3 * GiB, b=P + 4 * GiB, B=4, H=2,
            dk=128, dv=128, S=P + 5 * GiB, o=P + 6 * GiB):
        return lib.rda_decode_step(q, k, v, dt, a, b, B, H, dk, dv, S, o, None)
    assert dec(B=0) == OK                      # nothing to do: no launch
    assert dec(S=None) == NULL
    assert dec(dt=3) == DTYPE
    assert dec(B=-1) == SHAPE
    assert dec(B=1 << 26, H=16) == SHAPE       # 2 workgroups per (b, h) must fit the grid
    assert dec(dk=96) == UNSUP
    assert dec(o=P + 4) == ALIGN
    assert dec(o=P + 5 * GiB + 512) == ALIAS      # o inside S
    assert dec(S=P + 2 * GiB) == ALIAS            # S over v


def test_decode_tokens_rejects_bad_arguments(lib):
    def dec(q=P, k=P + GiB, v=P + 2 * GiB, dt=0, a=P + 3 * GiB, b=P + 4 * GiB, B=4, T=3, H=2,
            dk=128, dv=128, Si=P + 5 * GiB, So=P + 5 * GiB, acc=None, o=P + 6 * GiB):
        return lib.rda_decode_tokens(q, k, v, dt, a, b, B, T, H, dk, dv, Si, So, acc, o, None)
    assert dec(B=0) == OK                        # nothing to do: no launch
    assert dec(T=0) == OK                        # in place, no tokens: no launch
    assert dec(T=0, So=None) == OK
    assert dec(Si=None) == NULL
    assert dec(So=None, o=None) == NULL          # nothing would be produced
    assert dec(q=None) == NULL                   # q is read when o is produced
    assert dec(k=None) == NULL
    assert dec(dt=2) == DTYPE
    assert dec(B=-1) == SHAPE
    assert dec(T=-1) == SHAPE
    assert dec(T=65) == SHAPE                    # beyond one chunk: rda_prefill's job
    assert dec(B=1 << 26, H=16) == SHAPE
    assert dec(dv=64) == UNSUP
    assert dec(o=P + 8) == ALIGN
    assert dec(acc=P + 7 * GiB + 2) == ALIGN
    assert dec(o=P + 5 * GiB + 4096) == ALIAS    # o inside the state
    assert dec(So=P + 2 * GiB) == ALIAS          # S_out over v
    assert dec(So=P + 5 * GiB + 1024) == ALIAS   # S_out partly over S_in
    assert dec(acc=P + 6 * GiB + 16) == ALIAS    # accept inside o
    assert dec(So=P + 7 * GiB, acc=P + 7 * GiB + 4096) == ALIAS  # accept inside S_out


def test_decode_tokens_diag_rejects_bad_arguments(lib):
    def dec(q=P, k=P + GiB, v=P + 2 * GiB, dt=0, al=P + 3 * GiB, b=P + 4 * GiB, B=4, T=3, H=2,
            dk=128, dv=128, Si=P + 5 * GiB, So=P + 5 * GiB, acc=None, o=P + 6 * GiB):
        return lib.rda_decode_tokens_diag(q, k, v, dt, al, b, B, T, H, dk, dv, Si, So, acc, o,
                                          None)
    assert dec(B=0) == OK
    assert dec(al=None) == NULL
    assert dec(Si=None) == NULL
    assert dec(dt=3) == DTYPE
    assert dec(T=65) == SHAPE
    assert dec(dk=64) == UNSUP
    assert dec(al=P + 3 * GiB + 4) == ALIGN
    # alpha holds B * T * H * dk floats (12 KiB here), not B * T * H as a does
    assert dec(o=P + 3 * GiB + 8192) == ALIAS
    assert dec(So=P + 3 * GiB + 8192) == ALIAS


def test_output_norm_gate_rejects_bad_arguments(lib):
    import ctypes
    lib.rda_output_norm_gate.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_float, ctypes.c_int32,
                                         ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                         ctypes.c_int, ctypes.c_void_p]

    def ng(o=P, g=P + GiB, gdt=0, w=P + 2 * GiB, eps=1e-5, act=0, rows=1000, dv=128,
           out=P + 3 * GiB, odt=0):
        return lib.rda_output_norm_gate(o, g, gdt, w, eps, act, rows, dv, out, odt, None)
    assert ng(rows=0) == OK                       # nothing to do
    assert ng(o=None) == NULL
    assert ng(g=None) == NULL                     # the gate is read
    assert ng(odt=5) == DTYPE
    assert ng(gdt=7) == DTYPE
    assert ng(act=3) == VALUE
    assert ng(eps=-1.0) == VALUE
    assert ng(eps=float("nan")) == VALUE
    assert ng(eps=float("inf")) == VALUE
    assert ng(rows=-1) == SHAPE
    assert ng(dv=64) == UNSUP
    assert ng(out=P + 3 * GiB + 8) == ALIGN
    assert ng(out=P + GiB + 4096) == ALIAS        # out inside g
    assert ng(out=P + 2 * GiB) == ALIAS           # out over the weight
    assert ng(out=P, odt=0) == ALIAS              # bf16 out over fp32 o
    assert ng(rows=1 << 40) == SHAPE              # grid beyond int32 blocks


def test_prefill_norm_gate_rejects_bad_arguments(lib):
    """Every check of both halves before anything is enqueued (host-side
    pointers that are never dereferenced)."""
    rda.lib()     # the binding sets the argument types

    def png(q=P, k=P + GiB, v=P + 2 * GiB, dt=0, a=P + 3 * GiB, b=P + 4 * GiB, cu=None, N=1,
            T=128, H=2, dk=128, dv=128, S0=None, g=P + 5 * GiB, gdt=0, w=P + 6 * GiB, eps=1e-5,
            act=0, out=P + 7 * GiB, odt=0, Sf=P + 8 * GiB, ws=P + 9 * GiB, wsb=None):
        if wsb is None:
            wsb = rda.rda_prefill_norm_gate_workspace_bytes(N, T, H, 128, 128)
        return lib.rda_prefill_norm_gate(q, k, v, dt, a, b, cu, N, T, H, dk, dv, S0, g, gdt, w,
                                         eps, act, out, odt, Sf, ws, wsb, None)
    base = rda.rda_prefill_workspace_bytes(1, 128, 2)
    assert rda.rda_prefill_norm_gate_workspace_bytes(1, 128, 2) == base + 128 * 2 * 128 * 2
    assert rda.rda_prefill_norm_gate_workspace_bytes(1, 128, 2, 64, 64) == 0
    assert png(q=None) == NULL
    assert png(out=None) == NULL
    assert png(g=None) == NULL                    # the gate is read
    assert png(dt=7) == DTYPE
    assert png(gdt=7) == DTYPE
    assert png(odt=5) == DTYPE
    assert png(act=3) == VALUE
    assert png(eps=-1.0) == VALUE
    assert png(eps=float("nan")) == VALUE
    assert png(T=-1) == SHAPE
    assert png(dk=64) == UNSUP
    assert png(ws=None) == WS
    assert png(wsb=rda.rda_prefill_workspace_bytes(1, 128, 2)) == WS   # no room for the slices
    assert png(out=P + 7 * GiB + 8) == ALIGN
    assert png(g=P + 5 * GiB + 4) == ALIGN
    assert png(out=P + 16) == ALIAS               # out over q
    assert png(out=P + 5 * GiB + 1024) == ALIAS   # out inside g
    assert png(out=P + 9 * GiB + 512) == ALIAS    # out inside the workspace
    assert png(Sf=P + 5 * GiB) == ALIAS           # S_final over g
    assert png(ws=P + 5 * GiB - 256) == ALIAS     # workspace over g


def test_prologue_rejects_bad_arguments(lib):
    rda.lib()     # the binding sets the argument types
    T, H = 100, 2
    tok = T * H * 128 * 2          # bytes of one bf16 token tensor

    def pro(xq=P, xk=P + GiB, xv=P + 2 * GiB, xdt=0, w=P + 3 * GiB, K=4, act=1,
            hin=P + 4 * GiB, hout=P + 5 * GiB, beta=P + 6 * GiB, delta=P + 7 * GiB,
            g=P + 8 * GiB, floor=-5.0, eps=1e-6, cu=None, N=4, T=T, H=H, d=128,
            q=P + 9 * GiB, k=P + 10 * GiB, v=P + 11 * GiB, a=P + 12 * GiB, b=P + 13 * GiB):
        return lib.rda_prologue(xq, xk, xv, xdt, w, K, act, hin, hout, beta, delta, g, floor,
                                eps, cu, N, T, H, d, q, k, v, a, b, None)
    assert pro(T=0, hout=None) == OK             # nothing to write
    assert pro(xdt=1) == UNSUP                   # raw projections in bf16 only
    assert pro(xdt=4) == DTYPE
    assert pro(K=0) == VALUE
    assert pro(K=5) == VALUE
    assert pro(act=2) == VALUE
    assert pro(floor=float("nan")) == VALUE
    assert pro(floor=float("inf")) == VALUE
    assert pro(eps=-1.0) == VALUE
    assert pro(N=0) == SHAPE
    assert pro(T=-1) == SHAPE
    assert pro(N=3) == SHAPE                     # 100 tokens do not split into 3 equal runs
    assert pro(H=16 * 65536) == SHAPE
    assert pro(d=64) == UNSUP
    assert pro(xq=None) == NULL
    assert pro(g=None) == NULL
    assert pro(a=None) == NULL
    assert pro(q=P + 9 * GiB + 4) == ALIGN
    assert pro(cu=P + 14 * GiB + 2) == ALIGN
    assert pro(q=P + 16) == ALIAS                # q over the raw q
    assert pro(v=P + 9 * GiB + tok // 2) == ALIAS   # v over q
    assert pro(hout=P + 4 * GiB) == ALIAS        # history in place with 25 tokens per sequence
    assert pro(hout=P + 4 * GiB + 64) == ALIAS   # partial overlap
    assert pro(a=P + 6 * GiB) == ALIAS           # a over beta_raw
    assert pro(b=P + 12 * GiB + 16) == ALIAS     # b over a


def test_prefill_diag_rejects_bad_arguments(lib):
    rda.lib()

    def pre(q=P, k=P + GiB, v=P + 2 * GiB, dt=0, al=P + 3 * GiB, b=P + 4 * GiB, cu=None, N=1,
            T=100, H=2, dk=128, dv=128, S0=None, o=P + 5 * GiB, Sf=P + 6 * GiB,
            ws=P + 7 * GiB, wsb=1 << 30):
        return lib.rda_prefill_diag(q, k, v, dt, al, b, cu, N, T, H, dk, dv, S0, o, Sf, ws,
                                    wsb, None)
    assert pre(dt=3) == DTYPE
    assert pre(T=-1) == SHAPE
    assert pre(N=2) == SHAPE                     # several sequences need offsets
    assert pre(dk=64) == UNSUP
    assert pre(al=None) == NULL
    assert pre(ws=None) == WS
    assert pre(wsb=1024) == WS
    assert pre(o=P + 5 * GiB + 4) == ALIGN
    assert pre(o=P + 3 * GiB + 4096) == ALIAS    # o inside alpha
    assert pre(Sf=P + 7 * GiB) == ALIAS          # S_final over the workspace
    need = lib.rda_prefill_diag_workspace_bytes(1, 100, 2, 128, 128)
    assert need > lib.rda_prefill_workspace_bytes(1, 100, 2, 128, 128)
    assert lib.rda_prefill_diag_workspace_bytes(1, 100, 2, 64, 128) == 0


def test_decode_diag_rejects_bad_arguments(lib):
    rda.lib()

    def dec(q=P, k=P + GiB, v=P + 2 * GiB, dt=0, al=P + 3 * GiB, b=P + 4 * GiB, B=4, H=2,
            dk=128, dv=128, S=P + 5 * GiB, o=P + 6 * GiB):
        return lib.rda_decode_step_diag(q, k, v, dt, al, b, B, H, dk, dv, S, o, None)
    assert dec(B=0) == OK
    assert dec(al=None) == NULL
    assert dec(dt=3) == DTYPE
    assert dec(B=1 << 26, H=16) == SHAPE
    assert dec(dv=96) == UNSUP
    assert dec(al=P + 3 * GiB + 8) == ALIGN
    assert dec(S=P + 3 * GiB) == ALIAS          # S over alpha
    assert dec(o=P + 5 * GiB + 512) == ALIAS    # o inside S


def test_chunk_table_rejects_bad_arguments(lib):
    assert lib.rda_chunk_table(None, 2, 10, P, P + GiB, P + 2 * GiB, None) == SHAPE
    assert lib.rda_chunk_table(None, 1, -3, P, P + GiB, P + 2 * GiB, None) == SHAPE
    assert lib.rda_chunk_table(None, 1, 10, P, None, P + 2 * GiB, None) == NULL
    assert lib.rda_chunk_table(P + 2, 1, 10, P, P + GiB, P + 2 * GiB, None) == ALIGN


def test_cu_seqlens_host_validation():
    assert list(rda.check_cu_seqlens([0, 3, 3, 10], 10)) == [0, 3, 3, 10]
    for bad, T in [([1, 10], 10), ([0, 5, 4, 10], 10), ([0, 9], 10), ([0], 0),
                   (np.array([0.0, 10.0]), 10)]:
        with pytest.raises((ValueError, TypeError)):
            rda.check_cu_seqlens(bad, T)


def test_table_reference_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(50):
        N = int(rng.integers(1, 9))
        lens = rng.integers(0, 300, size=N)
        cu = np.concatenate([[0], np.cumsum(lens)])
        T = int(cu[-1])
        rec, off, nch = table_ref.chunk_table(cu, N, T)
        assert nch == sum(-(-int(x) // 64) for x in lens) <= table_ref.max_chunks(N, T)
        covered = np.zeros(T, dtype=int)
        for c in range(nch):
            n, s, L, j = rec[c]
            assert 1 <= L <= 64 and cu[n] <= s and s + L <= cu[n + 1] and s == cu[n] + 64 * j
            covered[s:s + L] += 1
        assert np.all(covered == 1)
        assert np.all(rec[nch:, 0] == -1)
