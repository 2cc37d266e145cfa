"""GPU tests of rda_decode_step_prologue, the decode step with the block's
prologue in front (short convolution with the history, q/k norm, write
gate, gates, then the state update), one launch per step (MI355X).

It must equal rda_prologue (one-token layout) followed by rda_decode_step
bit for bit -- same arithmetic, q, k, v rounded to bf16 as the prologue
writes them -- and the fp64 oracle's prologue (rounded to bf16, as the
interface is) followed by its decode step within the parity bar."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import ErrorSums, assert_parity, dev_f32, dev_tokens, need_gpu, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def bf(x, dev):
    return dev_tokens(x, True, dev)


def inputs(B, H, K, key):
    x = synth.prologue_inputs(B, H, K, N=B, key=key)
    S0 = synth.decode_state(B, H, key=key)
    return x, S0


def fused(x, S0, dev, act="silu", hist=True, delta=True, hist_mode="in_place"):
    """One fused step; returns (o, S, history after) on the host."""
    S = dev_f32(S0, dev)
    hin = bf(x.hist, dev) if hist else None
    if hist_mode == "in_place":
        hout = hin if hin is not None else torch.full(x.hist.shape, float("nan"),
                                                      dtype=torch.bfloat16, device=dev)
    elif hist_mode == "separate":
        hout = torch.full(x.hist.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    else:
        hout = None
    o = rda.rda_decode_step_prologue(bf(x.xq, dev), bf(x.xk, dev), bf(x.xv, dev),
                                     dev_f32(x.conv_w, dev), dev_f32(x.beta_raw, dev),
                                     dev_f32(x.g_log, dev), S,
                                     delta=dev_f32(x.delta, dev) if delta else None,
                                     hist_in=hin, hist_out=hout, conv_act=act)
    torch.cuda.synchronize()
    return to_host(o), to_host(S), (to_host(hout.float()) if hout is not None else None)


def separate(x, S0, dev, act="silu", hist=True, delta=True):
    """rda_prologue (one token per sequence) then rda_decode_step."""
    B = x.xq.shape[0]
    S = dev_f32(S0, dev)
    hin = bf(x.hist, dev) if hist else None
    hout = torch.full(x.hist.shape, float("nan"), dtype=torch.bfloat16, device=dev)
    q, k, v, a, b = rda.rda_prologue(bf(x.xq, dev), bf(x.xk, dev), bf(x.xv, dev),
                                     dev_f32(x.conv_w, dev), dev_f32(x.beta_raw, dev),
                                     dev_f32(x.g_log, dev),
                                     delta=dev_f32(x.delta, dev) if delta else None,
                                     hist_in=hin, hist_out=hout, num_seqs=B, conv_act=act)
    o = rda.rda_decode_step(q, k, v, a, b, S)
    torch.cuda.synchronize()
    return to_host(o), to_host(S), to_host(hout.float())


def oracle_step(x, S0, act="silu", hist=True, delta=True):
    """The oracle's prologue (one token per sequence), q, k, v rounded to bf16
    as the interface carries them, then its decode step."""
    B = x.xq.shape[0]
    cu = synth.cu_from_lengths([1] * B)
    rq, rk, rv, ra, rb, rh = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw,
                                             x.delta if delta else None, x.g_log,
                                             hist_in=x.hist if hist else None, cu_seqlens=cu,
                                             act=act)
    rq, rk, rv = (synth.round_bf16(r.astype(np.float32)) for r in (rq, rk, rv))
    Sref = S0.astype(np.float64)
    ro = oracle.decode_step(rq, rk, rv, ra.astype(np.float32), rb.astype(np.float32), Sref)
    return ro, Sref, rh


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("act", ["silu", "none"])
def test_equals_prologue_then_decode_bitwise(dev, K, act):
    x, S0 = inputs(8, 16, K, key=(520, K))
    say(f"[decode_prologue] K={K} act={act}: fused vs two calls")
    fo, fS, fh = fused(x, S0, dev, act=act, hist_mode="separate")
    so, sS, sh = separate(x, S0, dev, act=act)
    assert np.array_equal(fo, so), "o differs from rda_prologue + rda_decode_step"
    assert np.array_equal(fS, sS), "S differs from rda_prologue + rda_decode_step"
    assert np.array_equal(fh, sh), "history differs from rda_prologue"
    ro, rS, rh = oracle_step(x, S0, act=act)
    assert_parity("o", fo, ro)
    assert_parity("S", fS, rS)
    assert np.array_equal(fh, rh.astype(np.float32)), "history differs from the oracle"


@pytest.mark.parametrize("hist,delta,mode", [(False, True, "in_place"), (True, False, "in_place"),
                                             (True, True, "none"), (False, False, "separate")])
def test_options(dev, hist, delta, mode):
    x, S0 = inputs(8, 16, 4, key=(521,))
    say(f"[decode_prologue] history={hist} delta={delta} history out={mode}")
    fo, fS, fh = fused(x, S0, dev, hist=hist, delta=delta, hist_mode=mode)
    so, sS, sh = separate(x, S0, dev, hist=hist, delta=delta)
    assert np.array_equal(fo, so) and np.array_equal(fS, sS)
    if fh is not None:
        assert np.array_equal(fh, sh)


def test_history_in_place_equals_separate(dev):
    x, S0 = inputs(8, 16, 4, key=(522,))
    say("[decode_prologue] history in place vs a separate buffer")
    a = fused(x, S0, dev, hist_mode="in_place")
    b = fused(x, S0, dev, hist_mode="separate")
    for p, q in zip(a, b):
        assert np.array_equal(p, q)


def test_decode_batch_every_state(dev):
    """The decode batch (256 sequences x 16 heads), every state against the
    oracle, and bit for bit against the two calls."""
    x, S0 = inputs(256, 16, 4, key=(523,))
    say("[decode_prologue] 256 x 16, every state")
    fo, fS, fh = fused(x, S0, dev)
    so, sS, sh = separate(x, S0, dev)
    assert np.array_equal(fo, so) and np.array_equal(fS, sS) and np.array_equal(fh, sh)
    ro, rS, rh = oracle_step(x, S0)
    assert_parity("o, all states", fo, ro)
    assert_parity("S, all states", fS, rS)


def test_chain_of_steps_equals_one_sequence(dev):
    """Eight fused steps (history in place) equal the oracle's prologue over
    the eight tokens as one sequence per batch entry, then its prefill."""
    B, H, steps = 4, 16, 8
    x = synth.prologue_inputs(B * steps, H, 4, N=B, key=(524,))
    S0 = synth.decode_state(B, H, key=(524,))
    S = dev_f32(S0, dev)
    h = bf(x.hist, dev)
    w = dev_f32(x.conv_w, dev)
    err = ErrorSums()
    outs = []
    say(f"[decode_prologue] chain B={B} steps={steps}")
    for i in range(steps):
        rows = np.arange(B) * steps + i
        outs.append(rda.rda_decode_step_prologue(
            bf(x.xq[rows], dev), bf(x.xk[rows], dev), bf(x.xv[rows], dev), w,
            dev_f32(x.beta_raw[rows], dev), dev_f32(x.g_log[rows], dev), S,
            delta=dev_f32(x.delta[rows], dev), hist_in=h, hist_out=h))
    torch.cuda.synchronize()
    o_dec = np.stack([to_host(t) for t in outs], axis=1)        # [B, steps, H, d]
    cu = synth.cu_from_lengths([steps] * B)
    ref = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw, x.delta, x.g_log,
                          hist_in=x.hist, cu_seqlens=cu)
    rq, rk, rv = (synth.round_bf16(r.astype(np.float32)) for r in ref[:3])
    ro, rS = oracle.prefill(rq, rk, rv, ref[3].astype(np.float32), ref[4].astype(np.float32),
                            cu_seqlens=cu, S0=S0)
    err.add(o_dec.reshape(B * steps, H, 128), ro)
    err.check("chain o")
    assert_parity("chain S", to_host(S), rS)
    assert np.array_equal(to_host(h.float()), ref[5].astype(np.float32))


def test_zero_batch_and_determinism(dev):
    x, S0 = inputs(0, 16, 4, key=(525,))
    S = torch.zeros((0, 16, 128, 128), device=dev)
    o = rda.rda_decode_step_prologue(bf(x.xq, dev), bf(x.xk, dev), bf(x.xv, dev),
                                     dev_f32(x.conv_w, dev), dev_f32(x.beta_raw, dev),
                                     dev_f32(x.g_log, dev), S)
    torch.cuda.synchronize()
    assert o.shape == (0, 16, 128)
    x, S0 = inputs(16, 16, 4, key=(526,))
    say("[decode_prologue] determinism")
    a = fused(x, S0, dev)
    b = fused(x, S0, dev)
    for p, q in zip(a, b):
        assert np.array_equal(p, q)
