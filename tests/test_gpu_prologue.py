"""GPU parity of rda_prologue (short convolution with history, q/k norm,
write gate, gates) against the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import assert_parity, dev_f32, dev_tokens, need_gpu, say, to_host

pytestmark = pytest.mark.gpu

# q, k, v are written in bf16, a quantisation of fp32 arithmetic: every
# element within one bf16 unit of the fp64 value (2^-8 relative) plus an
# absolute floor for components that the convolution cancels to near zero
# (fp32 rounding of the K products, relative to the row's scale), and at
# least 99 % equal to the fp64 value rounded to nearest even.  a and b are
# fp32 results of the hardware exp and reciprocal: 2e-6 relative.  The
# history is raw bf16 data moved, compared bit for bit.
BF16_REL = 2.0 ** -8
ABS_FLOOR = 1e-5
BF16_EXACT_SHARE = 0.99
GATE_REL = 2e-6


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def bf16_dev(x, dev):
    return dev_tokens(x, True, dev)


def check_bf16(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    if ref.size == 0:
        return
    row_scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    bound = BF16_REL * np.abs(ref) + ABS_FLOOR * row_scale + 1e-30
    err = np.abs(got - ref)
    say(f"  {name}: max err / bound = {float(np.max(err / bound)):.3f}")
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} elements out of bound"
    rne = synth.round_bf16(ref.astype(np.float32)).astype(np.float64)
    share = float(np.mean(got == rne))
    say(f"  {name}: share equal to the rounded fp64 value = {share:.5f}")
    assert share >= BF16_EXACT_SHARE, f"{name}: only {share:.4f} round to nearest"


def check_all(got, ref, hist_got=None):
    q, k, v, a, b = got
    rq, rk, rv, ra, rb, rh = ref
    for name, g_, r_ in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        check_bf16(name, to_host(g_.float()), r_)
    for name, g_, r_ in (("a", a, ra), ("b", b, rb)):
        g_ = to_host(g_).astype(np.float64)
        assert np.all(np.abs(g_ - r_) <= GATE_REL * np.abs(r_)), f"{name} out of bound"
    if hist_got is not None:
        assert np.array_equal(to_host(hist_got.float()), rh.astype(np.float32)), "history"


def run(x, dev, K, act="silu", hist=True, delta=True, cu=None, N=1, hist_out=True):
    hin = bf16_dev(x.hist, dev) if hist else None
    hout = (torch.full(x.hist.shape, float("nan"), dtype=torch.bfloat16, device=dev)
            if hist_out else None)
    res = rda.rda_prologue(bf16_dev(x.xq, dev), bf16_dev(x.xk, dev), bf16_dev(x.xv, dev),
                           dev_f32(x.conv_w, dev), dev_f32(x.beta_raw, dev),
                           dev_f32(x.g_log, dev), delta=dev_f32(x.delta, dev) if delta else None,
                           hist_in=hin, hist_out=hout, cu_seqlens=cu, num_seqs=N, conv_act=act)
    torch.cuda.synchronize()
    cu_ref = cu
    if cu is None and N > 1:           # equal-length sequences, as offsets for the oracle
        cu_ref = synth.cu_from_lengths([x.xq.shape[0] // N] * N)
    ref = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw, x.delta if delta else None,
                          x.g_log, hist_in=x.hist if hist else None, cu_seqlens=cu_ref, act=act)
    return res, ref, hout


@pytest.mark.parametrize("T", [1, 5, 127, 128, 129, 300])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_one_sequence(dev, T, K):
    x = synth.prologue_inputs(T, 16, K, key=(500, T, K))
    say(f"[prologue] T={T} H=16 K={K}")
    res, ref, hout = run(x, dev, K)
    check_all(res, ref, hout if K > 1 else None)


@pytest.mark.parametrize("act", ["none", "silu"])
@pytest.mark.parametrize("hist", [True, False])
@pytest.mark.parametrize("delta", [True, False])
def test_options(dev, act, hist, delta):
    x = synth.prologue_inputs(70, 4, 4, key=(501,))
    say(f"[prologue] act={act} hist={hist} delta={delta}")
    res, ref, hout = run(x, dev, 4, act=act, hist=hist, delta=delta)
    check_all(res, ref, hout)


def test_packed_sequences(dev):
    """Empty, shorter-than-the-window and long sequences in one packed call."""
    lens = [0, 1, 2, 3, 150, 0, 7, 1]
    cu = synth.cu_from_lengths(lens).astype(np.int32)
    x = synth.prologue_inputs(int(cu[-1]), 16, 4, N=len(lens), key=(502,))
    say(f"[prologue] packed lengths {lens}")
    res, ref, hout = run(x, dev, 4, cu=cu, N=len(lens))
    check_all(res, ref, hout)
    assert np.array_equal(to_host(hout.float())[0], x.hist[0])   # empty: history kept


def test_equal_length_layouts(dev):
    """cu_seqlens NULL: B sequences of T tokens (the multi-token decode
    layout), and one token per sequence with the history updated in place."""
    B, T, H = 32, 3, 16
    x = synth.prologue_inputs(B * T, H, 4, N=B, key=(503,))
    cu = synth.cu_from_lengths([T] * B).astype(np.int32)
    say(f"[prologue] {B} x {T} tokens, no offsets")
    res, ref, hout = run(x, dev, 4, N=B)
    ref_cu = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw, x.delta, x.g_log,
                             hist_in=x.hist, cu_seqlens=cu)
    for i in range(6):
        assert np.array_equal(ref[i], ref_cu[i])
    check_all(res, ref, hout)
    B = 64
    x = synth.prologue_inputs(B, H, 4, N=B, key=(504,))
    h = bf16_dev(x.hist, dev)
    say(f"[prologue] {B} x 1 token, history in place")
    res = rda.rda_prologue(bf16_dev(x.xq, dev), bf16_dev(x.xk, dev), bf16_dev(x.xv, dev),
                           dev_f32(x.conv_w, dev), dev_f32(x.beta_raw, dev),
                           dev_f32(x.g_log, dev), delta=dev_f32(x.delta, dev), hist_in=h,
                           hist_out=h, num_seqs=B)
    torch.cuda.synchronize()
    ref = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw, x.delta, x.g_log,
                          hist_in=x.hist, cu_seqlens=synth.cu_from_lengths([1] * B))
    check_all(res, ref, h)


def test_zero_tokens_keeps_history(dev):
    x = synth.prologue_inputs(0, 16, 4, N=3, key=(505,))
    say("[prologue] no tokens")
    hout = torch.zeros(x.hist.shape, dtype=torch.bfloat16, device=dev)
    rda.rda_prologue(bf16_dev(x.xq, dev), bf16_dev(x.xk, dev), bf16_dev(x.xv, dev),
                     dev_f32(x.conv_w, dev), dev_f32(x.beta_raw, dev), dev_f32(x.g_log, dev),
                     hist_in=bf16_dev(x.hist, dev), hist_out=hout, num_seqs=3)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(hout.float()), x.hist)


def test_long_prompt(dev):
    """The long prompt: 16384 tokens x 16 heads, width 4, SiLU."""
    x = synth.prologue_inputs(16384, 16, 4, key=(506,))
    say("[prologue] T=16384 H=16")
    res, ref, hout = run(x, dev, 4)
    check_all(res, ref, hout)


def test_prologue_then_prefill(dev):
    """The prologue feeding the prefill, against the oracle's prologue, its
    q, k, v rounded to bf16 as the path's interface is, feeding the oracle's
    prefill."""
    T, H = 200, 4
    x = synth.prologue_inputs(T, H, 4, key=(507,))
    S0 = synth.decode_state(1, H, key=(507,))
    say("[prologue] then prefill, T=200 H=4")
    (q, k, v, a, b), ref, _ = run(x, dev, 4)
    o, S = rda.rda_prefill(q, k, v, a, b, S0=dev_f32(S0, dev))
    torch.cuda.synchronize()
    rq, rk, rv = (synth.round_bf16(r.astype(np.float32)) for r in ref[:3])
    ro, rS = oracle.prefill(rq, rk, rv, ref[3].astype(np.float32), ref[4].astype(np.float32),
                            S0=S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S", to_host(S), rS)


def test_decode_chain_with_history(dev):
    """Eight decode steps, each a one-token prologue updating the history in
    place then rda_decode_step, equal the oracle's prologue over the eight
    tokens as one sequence followed by its prefill."""
    B, H, steps = 4, 16, 8
    x = synth.prologue_inputs(B * steps, H, 4, N=B, key=(508,))
    # token i of sequence n is row n * steps + i
    S0 = synth.decode_state(B, H, key=(508,))
    S = dev_f32(S0, dev)
    h = bf16_dev(x.hist, dev)
    w = dev_f32(x.conv_w, dev)
    outs = []
    say(f"[prologue] decode chain B={B} steps={steps}")
    for i in range(steps):
        rows = np.arange(B) * steps + i
        q, k, v, a, b = rda.rda_prologue(
            bf16_dev(x.xq[rows], dev), bf16_dev(x.xk[rows], dev), bf16_dev(x.xv[rows], dev), w,
            dev_f32(x.beta_raw[rows], dev), dev_f32(x.g_log[rows], dev),
            delta=dev_f32(x.delta[rows], dev), hist_in=h, hist_out=h, num_seqs=B)
        outs.append(rda.rda_decode_step(q, k, v, a, b, S))
    torch.cuda.synchronize()
    o_dec = np.stack([to_host(t) for t in outs], axis=1)        # [B, steps, H, d]
    cu = synth.cu_from_lengths([steps] * B)
    ref = oracle.prologue(x.xq, x.xk, x.xv, x.conv_w, x.beta_raw, x.delta, x.g_log,
                          hist_in=x.hist, cu_seqlens=cu)
    rq, rk, rv = (synth.round_bf16(r.astype(np.float32)) for r in ref[:3])
    ro, rS = oracle.prefill(rq, rk, rv, ref[3].astype(np.float32), ref[4].astype(np.float32),
                            cu_seqlens=cu, S0=S0)
    assert_parity("decode chain o", o_dec.reshape(B * steps, H, 128), ro)
    assert_parity("decode chain S", to_host(S), rS)
    assert np.array_equal(to_host(h.float()), ref[5].astype(np.float32))


def test_bitwise_deterministic(dev):
    x = synth.prologue_inputs(333, 16, 4, key=(509,))
    say("[prologue] determinism")
    outs = []
    for _ in range(2):
        res, _, hout = run(x, dev, 4)
        outs.append([to_host(t.float()) for t in res] + [to_host(hout.float())])
    for p, q in zip(*outs):
        assert np.array_equal(p, q)
