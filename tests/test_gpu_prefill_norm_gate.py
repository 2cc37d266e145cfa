"""GPU parity of rda_prefill_norm_gate, the prefill with the block's output
norm and gate fused (MI355X): the walk leaves each token-head row in 16 bits
per channel -- each 16-channel slice scaled by a power of two into (-1, 1),
as fp16, the scale's exponent carried in the lowest bit of the slice's first
8 values -- and a pass over that form takes the RMS norm and applies the
weight and the gate.

Bars:
  - fp32 out against the oracle's prefill followed by the oracle's output
    norm and gate: the mixer's rel-L2 <= 2e-3, and its max-abs 2e-2 times
    the largest factor w_c act(g_c) that the norm and gate multiply a
    normalised mixer output by;
  - fp32 out against rda_prefill then rda_output_norm_gate on the GPU, per
    element: fp16's spacing is at most 2^-10 of a normal value, so rounding
    moves a value by at most 2^-11 of itself and replacing its lowest bit
    (the values that carry the exponent) by at most 2^-10 more; the row's
    norm, a mean over such values, moves by no more, so
    |d| <= 2 * 3 * 2^-11 |ref| = 3 * 2^-10 |ref|, plus 1e-6 of the largest
    output for the values fp16 holds as subnormals (below 2^-14 of their
    slice's largest);
  - bf16 out equal, bit for bit, to the fp32 out rounded to nearest even
    (the same kernel; a bf16 output only adds its one rounding);
  - S_final equal, bit for bit, to rda_prefill's (the same walk).
"""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import (assert_parity, dev_f32, dev_tokens, guarded, need_gpu, rel_l2, say,
                      to_host)

pytestmark = pytest.mark.gpu

FORM_REL = 3 * 2.0 ** -10


def check_form(out, two):
    """The fused output against the two calls', element by element."""
    out = np.asarray(out, np.float64)
    two = np.asarray(two, np.float64)
    assert np.all(np.isfinite(out))
    d = np.abs(out - two)
    bound = FORM_REL * np.abs(two) + 1e-6 * float(np.max(np.abs(two)) if two.size else 0.0)
    worst = float(np.max(d / np.maximum(bound, 1e-300))) if two.size else 0.0
    say(f"  fused vs two calls: rel_l2={rel_l2(out, two):.3e} worst/bound={worst:.3f}")
    assert np.all(d <= bound), f"{int(np.sum(d > bound))} values beyond the 16-bit form's bound"


def gain(g, w, act):
    """Largest factor w_c act(g_c) the norm and gate apply (1 without either)."""
    a = np.ones(1)
    if act != "none" and g.size:
        x = g.astype(np.float64)
        sig = 1.0 / (1.0 + np.exp(-x))
        a = np.abs(sig if act == "sigmoid" else x * sig)
    ww = np.abs(w.astype(np.float64)) if w is not None else np.ones(1)
    return float(np.max(a) * np.max(ww))


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def gate_inputs(T, H, bf16_gate, key):
    x = synth.epilogue_inputs(max(T * H, 1), bf16=bf16_gate, key=key)
    return x.g[:T * H].reshape(T, H, 128), x.weight


def run_fused(p, g, w, act, out_dtype, dev, g_bf16=True):
    q, k, v = (dev_tokens(getattr(p, n), p.bf16, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    S0 = dev_f32(p.S0, dev)
    T, H = p.total_tokens, p.num_heads
    gd = dev_tokens(g, g_bf16, dev) if act != "none" else None
    wd = dev_f32(w, dev)
    gout = guarded((T, H, 128), out_dtype, dev)
    out, Sf = rda.rda_prefill_norm_gate(q, k, v, a, b, gd, cu_seqlens=p.cu_seqlens, S0=S0,
                                        weight=wd, act=act, out=gout.t, out_dtype=out_dtype)
    torch.cuda.synchronize()
    gout.check("out")
    return to_host(out.float()), to_host(Sf)


def run_two_calls(p, g, w, act, dev, g_bf16=True):
    q, k, v = (dev_tokens(getattr(p, n), p.bf16, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    o, Sf = rda.rda_prefill(q, k, v, a, b, cu_seqlens=p.cu_seqlens, S0=dev_f32(p.S0, dev))
    gd = dev_tokens(g, g_bf16, dev) if act != "none" else None
    out = rda.rda_output_norm_gate(o, gd, weight=dev_f32(w, dev), act=act,
                                   out_dtype=torch.float32)
    torch.cuda.synchronize()
    return to_host(out), to_host(Sf)


CASES = {
    # name: (prefill inputs, act, gate in bf16, weight given)
    "200x4 sigmoid": (lambda: synth.make_prefill(200, 4, bf16=True, s0_std=0.02, key=(600,)),
                      "sigmoid", True, True),
    "varlen silu": (lambda: synth.make_prefill(H=4, lengths=[130, 0, 1, 64, 300], bf16=True,
                                               s0_std=0.05, key=(601,)), "silu", True, True),
    "fp32 inputs, no gate": (lambda: synth.make_prefill(130, 2, bf16=False, s0_std=0.05,
                                                        key=(602,)), "none", True, True),
    "fp32 gate, no weight": (lambda: synth.make_prefill(300, 3, bf16=True, key=(603,)),
                             "sigmoid", False, False),
    "segmented 4096x2": (lambda: synth.make_prefill(4096, 2, bf16=True, s0_std=0.02,
                                                    key=(604,)), "sigmoid", True, True),
    "overlapped 2048x16": (lambda: synth.make_prefill(2048, 16, bf16=True, s0_std=0.02,
                                                      key=(605,)), "silu", True, True),
    # long enough that the last walk launch is cut in two, each part running
    # the norm of rows already walked beside it
    "overlapped, cut 4100x16": (lambda: synth.make_prefill(4100, 16, bf16=True, s0_std=0.02,
                                                           key=(612,)), "sigmoid", True, True),
    # 8 heads: a short first range (8 chunks) and a cut last range
    "overlapped 3000x8": (lambda: synth.make_prefill(3000, 8, bf16=True, s0_std=0.02,
                                                     key=(613,)), "silu", True, True),
    # outputs far outside fp16's range, and far below its normal range: each
    # slice's power-of-two scale must bring them into (-1, 1) either way
    "values x 2^20": (lambda: scaled(synth.make_prefill(300, 2, bf16=True, key=(608,)), 2.0 ** 20),
                      "sigmoid", True, True),
    "values x 2^-24": (lambda: scaled(synth.make_prefill(300, 2, bf16=True, key=(609,)),
                                      2.0 ** -24), "sigmoid", True, True),
}


def scaled(p, f):
    """The same inputs with v (and so o and S) scaled by the power of two f
    (exact in bf16)."""
    p.v = (p.v * f).astype(np.float32)
    p.meta["v_scale"] = f
    return p


@pytest.mark.parametrize("name", list(CASES))
def test_fused_against_oracle(dev, name):
    make, act, g_bf16, with_w = CASES[name]
    p = make()
    T, H = p.total_tokens, p.num_heads
    g, w = gate_inputs(T, H, g_bf16, key=(610, T, H))
    w = w if with_w else None
    say(f"[prefill_norm_gate] {name}: T={T} H={H} N={p.num_seqs} act={act}")
    out32, Sf = run_fused(p, g, w, act, torch.float32, dev, g_bf16)
    out16, Sf16 = run_fused(p, g, w, act, torch.bfloat16, dev, g_bf16)
    assert np.array_equal(out16, synth.round_bf16(out32.astype(np.float32))), \
        "bf16 out is not the fp32 out rounded to nearest even"
    assert np.array_equal(Sf, Sf16)
    two, Sf2 = run_two_calls(p, g, w, act, dev, g_bf16)
    assert np.array_equal(Sf, Sf2), "S_final differs from rda_prefill's"
    check_form(out32, two)
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, cu_seqlens=p.cu_seqlens, S0=p.S0)
    ref = oracle.output_norm_gate(ro.reshape(-1, 128), g.reshape(-1, 128) if act != "none"
                                  else None, w, 1e-5, act).reshape(T, H, 128)
    amp = gain(g, w, act)
    assert_parity(f"{name} out", out32, ref, mab=2e-2 * max(1.0, amp))
    # the state is linear in v: its max-abs bar scales with the values
    vs = float(p.meta.get("v_scale", 1.0))
    assert_parity(f"{name} S_final", Sf, rS, mab=2e-2 * max(1.0, vs))


def test_zero_tokens(dev):
    p = synth.make_prefill(0, 2, bf16=True, s0_std=0.05, key=(606,))
    say("[prefill_norm_gate] T=0")
    g = np.zeros((0, 2, 128), np.float32)
    out, Sf = run_fused(p, g, None, "sigmoid", torch.bfloat16, dev)
    assert out.shape == (0, 2, 128)
    assert np.array_equal(Sf, p.S0)


def test_long_prompt_against_two_calls(dev):
    """16384 x 16 (the overlapped plan, the size the bench times): the fused
    result against the two calls, whose prefill meets the oracle at this size
    in test_gpu_prefill."""
    p = synth.make_prefill(16384, 16, bf16=True, s0_std=0.02, key=(607,))
    g, w = gate_inputs(16384, 16, True, key=(611,))
    say("[prefill_norm_gate] 16384 x 16 against the two calls")
    out32, Sf = run_fused(p, g, w, "sigmoid", torch.float32, dev)
    two, Sf2 = run_two_calls(p, g, w, "sigmoid", dev)
    assert np.array_equal(Sf, Sf2)
    check_form(out32, two)
