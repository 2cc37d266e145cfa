"""GPU parity of rda_output_norm_gate (the block's output norm and gate)
against the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import assert_parity, dev_f32, dev_tokens, need_gpu, say, to_host

pytestmark = pytest.mark.gpu

# A bf16 output is a quantisation of the fp32 result, so its bar is set by
# bf16 rounding rather than by the mixer's 2e-3 rel-L2: every element within
# one bf16 unit in the last place of the fp64 value (2^-8 relative covers
# it: round to nearest gives half a unit, and the fp32 arithmetic before the
# rounding can move a value across a rounding boundary), at least 99 % of
# the elements equal to the fp64 value rounded to nearest even (a truncating
# conversion would miss about half), rel-L2 within 2^-8 and max-abs within
# one unit at the largest magnitude.
BF16_REL = 2.0 ** -8
BF16_EXACT_SHARE = 0.99
F32_REL = 4e-6   # fp32 arithmetic with the hardware exp, reciprocal and rsqrt


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def check(name, out, ref, bf16):
    out = np.asarray(out, dtype=np.float64)
    assert np.all(np.isfinite(out)), f"{name}: non-finite"
    rel = BF16_REL if bf16 else F32_REL
    err = np.abs(out - ref)
    bound = rel * np.abs(ref) + 1e-30
    worst = float(np.max(err / bound)) if ref.size else 0.0
    say(f"  {name}: max err / bound = {worst:.3f}")
    assert np.all(err <= bound), f"{name}: {int(np.sum(err > bound))} elements out of bound"
    if bf16:
        rne = synth.round_bf16(ref.astype(np.float32)).astype(np.float64)
        share = float(np.mean(out == rne)) if ref.size else 1.0
        say(f"  {name}: share equal to the rounded fp64 value = {share:.5f}")
        assert share >= BF16_EXACT_SHARE, f"{name}: only {share:.4f} round to nearest"
        # absolute: one unit at the largest magnitude
        assert_parity(name, out, ref, rel=BF16_REL,
                      mab=BF16_REL * float(np.max(np.abs(ref))) if ref.size else 0.0)
    else:
        assert_parity(name, out, ref)


@pytest.mark.parametrize("rows", [1, 2, 31, 32, 33, 1000])
@pytest.mark.parametrize("act", ["sigmoid", "silu", "none"])
def test_rows_and_activations(dev, rows, act):
    x = synth.epilogue_inputs(rows, key=(400, rows))
    say(f"[epilogue] rows={rows} act={act}")
    out = rda.rda_output_norm_gate(dev_f32(x.o, dev), dev_tokens(x.g, True, dev),
                                   weight=dev_f32(x.weight, dev), act=act)
    torch.cuda.synchronize()
    ref = oracle.output_norm_gate(x.o, x.g if act != "none" else None, x.weight, 1e-5, act)
    check("bf16 out", to_host(out.float()), ref, True)


@pytest.mark.parametrize("g_bf16", [True, False])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_dtypes_and_no_weight(dev, g_bf16, out_dtype):
    x = synth.epilogue_inputs(517, bf16=g_bf16, key=(401,))
    say(f"[epilogue] g_bf16={g_bf16} out={out_dtype}")
    for w in (x.weight, None):
        out = rda.rda_output_norm_gate(dev_f32(x.o, dev), dev_tokens(x.g, g_bf16, dev),
                                       weight=dev_f32(w, dev), eps=1e-5, out_dtype=out_dtype)
        torch.cuda.synchronize()
        ref = oracle.output_norm_gate(x.o, x.g, w, 1e-5, "sigmoid")
        check(f"weight={w is not None}", to_host(out.float()), ref,
              out_dtype == torch.bfloat16)


def test_in_place_fp32_and_eps(dev):
    x = synth.epilogue_inputs(300, key=(402,))
    x.o[:7] = 0.0                       # zero rows give zero output when eps > 0
    say("[epilogue] fp32 in place, eps 0.25")
    o = dev_f32(x.o, dev)
    res = rda.rda_output_norm_gate(o, dev_tokens(x.g, True, dev), weight=dev_f32(x.weight, dev),
                                   eps=0.25, out=o, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert res.data_ptr() == o.data_ptr()
    ref = oracle.output_norm_gate(x.o, x.g, x.weight, 0.25, "sigmoid")
    check("in place", to_host(o), ref, False)
    assert np.all(to_host(o)[:7] == 0.0)


def test_zero_rows(dev):
    say("[epilogue] rows=0")
    out = rda.rda_output_norm_gate(torch.zeros((0, 16, 128), device=dev),
                                   torch.zeros((0, 16, 128), dtype=torch.bfloat16, device=dev))
    torch.cuda.synchronize()
    assert out.shape == (0, 16, 128)


def test_long_prompt_rows(dev):
    """16384 tokens x 16 heads = 262144 rows, the size the bench times."""
    x = synth.epilogue_inputs(16384 * 16, key=(403,))
    say("[epilogue] 262144 rows")
    out = rda.rda_output_norm_gate(dev_f32(x.o, dev).view(16384, 16, 128),
                                   dev_tokens(x.g, True, dev).view(16384, 16, 128),
                                   weight=dev_f32(x.weight, dev))
    torch.cuda.synchronize()
    ref = oracle.output_norm_gate(x.o, x.g, x.weight, 1e-5, "sigmoid")
    check("262144 rows", to_host(out.float()).reshape(-1, 128), ref, True)


def test_prefill_then_epilogue(dev):
    """The whole path, prefill then the output norm and gate, against the
    oracle's prefill then the oracle's epilogue on the same seeded inputs."""
    p = synth.make_prefill(200, 4, bf16=True, s0_std=0.02, key=(404,))
    x = synth.epilogue_inputs(200 * 4, key=(404,))
    g = x.g.reshape(200, 4, 128)
    say("[epilogue] prefill T=200 H=4 then norm gate")
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    o, _ = rda.rda_prefill(q, k, v, dev_f32(p.a, dev), dev_f32(p.b, dev), S0=dev_f32(p.S0, dev))
    out = rda.rda_output_norm_gate(o, dev_tokens(g, True, dev), weight=dev_f32(x.weight, dev))
    torch.cuda.synchronize()
    ro, _ = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
    ref = oracle.output_norm_gate(ro, g, x.weight, 1e-5, "sigmoid")
    assert_parity("prefill + norm gate", to_host(out.float()), ref)


def test_bitwise_deterministic(dev):
    x = synth.epilogue_inputs(777, key=(405,))
    say("[epilogue] determinism")
    outs = []
    for _ in range(2):
        out = rda.rda_output_norm_gate(dev_f32(x.o, dev), dev_tokens(x.g, True, dev),
                                       weight=dev_f32(x.weight, dev))
        torch.cuda.synchronize()
        outs.append(to_host(out.view(torch.int16)))
    assert np.array_equal(outs[0], outs[1])
