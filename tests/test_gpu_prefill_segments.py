"""GPU parity of the segmented state pass of rda_prefill (one bf16 sequence
without offsets and few heads: the sequence cut into P segments, walked from
zero and from the identity, chained, then walked again with outputs) against
the fp64 oracle and against the one-pass walk (MI355X).

The library picks the segmented pass by itself for one sequence without
offsets when H <= 4 and the sequence holds >= 64 chunks; passing
cu_seqlens = [0, T] runs the one-pass walk on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import assert_parity, dev_f32, dev_tokens, guarded, need_gpu, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def segments(T, H):
    """The segment count the library uses (0: one-pass walk)."""
    nch = (T + 63) // 64
    P = min(256 // (16 * H), nch // 16, 16)
    if P < 4:
        return 0
    cps = -(-nch // P)
    return -(-nch // cps)


def long_memory(p, key):
    """Decays close to 1 (log a ~ U(-4e-3, 0)): a segment of 1024 tokens keeps
    about e^-2 of its starting state, so each segment's map is far from zero.
    (With the default gates a state is forgotten below fp32 resolution within
    two chunks, and both passes give the same bits.)"""
    p.a = np.exp(-np.random.default_rng(key).uniform(0.0, 4e-3, p.a.shape)).astype(np.float32)
    return p


def run(p, dev, one_pass=False, S0=None, S_final=None, want_state=True):
    """o (and S_final unless given) inside guard bands, checked after the
    call."""
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    cu = np.array([0, p.total_tokens], dtype=np.int32) if one_pass else None
    go = guarded((p.total_tokens, p.num_heads, 128), torch.float32, dev)
    gs = None
    if S_final is None and want_state:
        gs = guarded((1, p.num_heads, 128, 128), torch.float32, dev)
        S_final = gs.t
    o, Sf = rda.rda_prefill(q, k, v, a, b, cu_seqlens=cu, S0=S0, o=go.t, S_final=S_final,
                            want_state=want_state)
    torch.cuda.synchronize()
    go.check("o")
    if gs is not None:
        gs.check("S_final")
    return to_host(o), (to_host(Sf) if Sf is not None else None)


@pytest.mark.parametrize("gates", ["long", "default"])
@pytest.mark.parametrize("T,H", [(4096, 4), (8192 + 37, 2), (16384, 1), (16384, 2), (16384, 3)])
def test_against_oracle_and_one_pass(dev, T, H, gates):
    P = segments(T, H)
    assert P >= 4
    p = synth.make_prefill(T, H, s0_std=0.02, key=(700, T, H))
    if gates == "long":
        p = long_memory(p, (700, T, H))
    say(f"[segments] T={T} H={H} P={P} gates={gates}")
    S0 = dev_f32(p.S0, dev)
    o, Sf = run(p, dev, S0=S0)
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
    assert_parity("o", o, ro)
    assert_parity("S_final", Sf, rS)
    o1, S1 = run(p, dev, one_pass=True, S0=S0)
    # the two passes agree far inside the oracle bound; with long memory they
    # differ in their rounding (so the segmented pass is the one that ran)
    for name, x, y in (("o", o, o1), ("S_final", Sf, S1)):
        rel = float(np.linalg.norm(x - y) / np.linalg.norm(y))
        say(f"  segmented vs one pass {name}: rel-L2 {rel:.2e}")
        assert rel < 1e-4
    if gates == "long":
        assert not np.array_equal(o, o1)


def test_zero_start_and_no_state(dev):
    T, H = 8192, 2
    p = synth.make_prefill(T, H, key=(701,))
    p = long_memory(p, 701)
    say("[segments] S0 = None, then S_final not requested")
    o, Sf = run(p, dev)
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b)
    assert_parity("o", o, ro)
    assert_parity("S_final", Sf, rS)
    o2, Sf2 = run(p, dev, want_state=False)
    assert Sf2 is None
    assert np.array_equal(o, o2)


def test_resume_in_place(dev):
    """S_final written over S0: the combine reads each row of S0 before it
    writes that row of S_final."""
    T, H = 8192, 2
    p = synth.make_prefill(T, H, s0_std=0.02, key=(702,))
    p = long_memory(p, 702)
    S = dev_f32(p.S0, dev)
    say("[segments] S_final = S0 in place")
    o, _ = run(p, dev, S0=S, S_final=S)
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
    assert_parity("o", o, ro)
    assert_parity("S_final in place", to_host(S), rS)


def test_two_calls_equal_one(dev):
    """Resume across calls: the first half then the second half from its
    final state equals the whole sequence."""
    T, H = 16384, 2
    p = synth.make_prefill(T, H, s0_std=0.02, key=(703,))
    p = long_memory(p, 703)
    half = T // 2
    say("[segments] two halves")
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    S0 = dev_f32(p.S0, dev)
    o1, S1 = rda.rda_prefill(q[:half].contiguous(), k[:half].contiguous(), v[:half].contiguous(),
                             a[:half].contiguous(), b[:half].contiguous(), S0=S0)
    o2, S2 = rda.rda_prefill(q[half:].contiguous(), k[half:].contiguous(), v[half:].contiguous(),
                             a[half:].contiguous(), b[half:].contiguous(), S0=S1)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
    assert_parity("o", np.concatenate([to_host(o1), to_host(o2)]), ro)
    assert_parity("S_final", to_host(S2), rS)


def test_identity_gates(dev):
    """a = 1, b = 0: every segment's map is the identity and E = 0, so the
    state is S0 exactly and o = S0 q."""
    T, H = 8192, 2
    p = synth.make_prefill(T, H, s0_std=0.02, key=(704,))
    p.a[:] = 1.0
    p.b[:] = 0.0
    say("[segments] a = 1, b = 0")
    o, Sf = run(p, dev, S0=dev_f32(p.S0, dev))
    np.testing.assert_allclose(Sf, p.S0, rtol=0, atol=1e-6)
    ref = np.einsum("thk,hvk->thv", p.q.astype(np.float64), p.S0[0].astype(np.float64))
    assert_parity("o = S0 q", o, ref)


def test_bitwise_deterministic(dev):
    T, H = 8192, 2
    p = synth.make_prefill(T, H, s0_std=0.02, key=(705,))
    p = long_memory(p, 705)
    say("[segments] determinism")
    S0 = dev_f32(p.S0, dev)
    a1, b1 = run(p, dev, S0=S0)
    a2, b2 = run(p, dev, S0=S0)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)


# ---- the per-channel decay (rda_prefill_diag) takes the same segmented pass ----

def diag_run(p, alpha, dev, one_pass=False, S0=None, S_final=None):
    """o (and S_final unless given) inside guard bands, checked after the
    call."""
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    cu = np.array([0, p.total_tokens], dtype=np.int32) if one_pass else None
    go = guarded((p.total_tokens, p.num_heads, 128), torch.float32, dev)
    gs = None
    if S_final is None:
        gs = guarded((1, p.num_heads, 128, 128), torch.float32, dev)
        S_final = gs.t
    o, Sf = rda.rda_prefill_diag(q, k, v, dev_f32(alpha, dev), dev_f32(p.b, dev), cu_seqlens=cu,
                                 S0=S0, o=go.t, S_final=S_final)
    torch.cuda.synchronize()
    go.check("o")
    if gs is not None:
        gs.check("S_final")
    return to_host(o), (to_host(Sf) if Sf is not None else None)


@pytest.mark.parametrize("gates", ["long", "default"])
@pytest.mark.parametrize("T,H", [(4096, 4), (8192 + 37, 2), (16384, 1)])
def test_diag_against_oracle_and_one_pass(dev, T, H, gates):
    P = segments(T, H)
    p = synth.make_prefill(T, H, s0_std=0.02, key=(710, T, H))
    if gates == "long":
        rng = np.random.default_rng((710, T, H))
        alpha = np.exp(-rng.uniform(0.0, 4e-3, (T, H, 128))).astype(np.float32)
    else:
        alpha = synth.diag_alpha(T, H, key=(710, T, H))
    say(f"[segments, per-channel] T={T} H={H} P={P} gates={gates}")
    S0 = dev_f32(p.S0, dev)
    o, Sf = diag_run(p, alpha, dev, S0=S0)
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("o", o, ro)
    assert_parity("S_final", Sf, rS)
    o1, S1 = diag_run(p, alpha, dev, one_pass=True, S0=S0)
    for name, x, y in (("o", o, o1), ("S_final", Sf, S1)):
        rel = float(np.linalg.norm(x - y) / np.linalg.norm(y))
        say(f"  segmented vs one pass {name}: rel-L2 {rel:.2e}")
        assert rel < 1e-4
    if gates == "long":
        assert not np.array_equal(o, o1)


def test_diag_resume_in_place(dev):
    T, H = 8192, 2
    p = synth.make_prefill(T, H, s0_std=0.02, key=(711,))
    alpha = np.exp(-np.random.default_rng(711).uniform(0.0, 4e-3, (T, H, 128))).astype(np.float32)
    S = dev_f32(p.S0, dev)
    say("[segments, per-channel] S_final = S0 in place")
    o, _ = diag_run(p, alpha, dev, S0=S, S_final=S)
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("o", o, ro)
    assert_parity("S_final in place", to_host(S), rS)
