"""GPU parity of the per-channel-decay prefill and decode step
(rda_prefill_diag, rda_decode_step_diag) against the fp64 oracle (MI355X)."""
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


def case(T, H, key, s0=0.02, lengths=None):
    p = synth.make_prefill(T, H, lengths=lengths, bf16=True, s0_std=s0, key=key)
    alpha = synth.diag_alpha(p.total_tokens, H, key=key)
    return p, alpha


def run_gpu(p, alpha, dev):
    """o and S_final inside guard bands, checked after the call."""
    q, k, v = (dev_tokens(getattr(p, n), p.bf16, dev) for n in "qkv")
    go = guarded((p.total_tokens, p.num_heads, 128), torch.float32, dev)
    gs = guarded((p.num_seqs, p.num_heads, 128, 128), torch.float32, dev)
    o, S = rda.rda_prefill_diag(q, k, v, dev_f32(alpha, dev), dev_f32(p.b, dev),
                                cu_seqlens=p.cu_seqlens, S0=dev_f32(p.S0, dev), o=go.t,
                                S_final=gs.t)
    torch.cuda.synchronize()
    go.check("o")
    gs.check("S_final")
    return o, S


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 130, 300])
def test_one_sequence(dev, T):
    p, alpha = case(T, 4, (600, T))
    say(f"[prefill_diag] T={T} H=4")
    o, S = run_gpu(p, alpha, dev)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S_final", to_host(S), rS)


@pytest.mark.parametrize("T", [1, 64, 65, 300])
def test_fp32_inputs(dev, T):
    """fp32 q, k, v (the same ABI as rda_prefill): unrounded values, every
    product at full precision, against the oracle on the same fp32 values."""
    p = synth.make_prefill(T, 4, bf16=False, s0_std=0.05, key=(608, T))
    alpha = synth.diag_alpha(T, 4, key=(608, T))
    say(f"[prefill_diag] fp32 T={T} H=4")
    o, S = run_gpu(p, alpha, dev)
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S_final", to_host(S), rS)


def test_fp32_segmented_and_packed(dev):
    """fp32 inputs through the segmented state pass (one long sequence, 2
    heads) and through packed sequences with an empty one."""
    p = synth.make_prefill(4096, 2, bf16=False, s0_std=0.02, key=(609,))
    alpha = np.exp(-np.random.default_rng(609).uniform(0.0, 4e-3, (4096, 2, 128))).astype(np.float32)
    say("[prefill_diag] fp32 segmented 4096 x 2")
    o, S = run_gpu(p, alpha, dev)
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("segmented o", to_host(o), ro)
    assert_parity("segmented S_final", to_host(S), rS)
    p = synth.make_prefill(H=3, lengths=[70, 0, 129, 1], bf16=False, s0_std=0.05, key=(610,))
    alpha = synth.diag_alpha(p.total_tokens, 3, key=(610,))
    say("[prefill_diag] fp32 packed")
    o, S = run_gpu(p, alpha, dev)
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, cu_seqlens=p.cu_seqlens, S0=p.S0)
    assert_parity("packed o", to_host(o), ro)
    assert_parity("packed S_final", to_host(S), rS)


def test_equal_channels_is_the_scalar_prefill(dev):
    """alpha equal on every key channel: the scalar rda_prefill, on the GPU."""
    p = synth.make_prefill(300, 16, bf16=True, s0_std=0.02, key=(601,))
    alpha = np.repeat(p.a[:, :, None], 128, axis=2)
    say("[prefill_diag] equal channels vs rda_prefill")
    o, S = run_gpu(p, alpha, dev)
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    o2, S2 = rda.rda_prefill(q, k, v, dev_f32(p.a, dev), dev_f32(p.b, dev), S0=dev_f32(p.S0, dev))
    torch.cuda.synchronize()
    assert_parity("o vs scalar prefill", to_host(o), to_host(o2))
    assert_parity("S vs scalar prefill", to_host(S), to_host(S2))
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S", to_host(S), rS)


def test_packed_sequences(dev):
    lens = [70, 0, 64, 1, 129, 33]
    p, alpha = case(0, 16, (602,), lengths=lens)
    say(f"[prefill_diag] packed {lens}")
    o, S = run_gpu(p, alpha, dev)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, cu_seqlens=p.cu_seqlens, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S_final", to_host(S), rS)
    assert np.array_equal(to_host(S)[1], p.S0[1])          # empty sequence: S0 unchanged


def test_packed_sequences_many_items(dev):
    """More (chunk, head) items than prep workgroups: each workgroup takes
    several items, its prefetch crossing sequence ends and partial chunks."""
    lens = [1000, 37, 2050, 0, 513, 64]
    p, alpha = case(0, 16, (607,), lengths=lens)
    say(f"[prefill_diag] packed {lens}")
    o, S = run_gpu(p, alpha, dev)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, cu_seqlens=p.cu_seqlens, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S_final", to_host(S), rS)
    assert np.array_equal(to_host(S)[3], p.S0[3])          # empty sequence: S0 unchanged


@pytest.mark.parametrize("kind", ["fast_channels", "near_one", "mixed_blocks"])
def test_decay_regimes(dev, kind):
    """Decays small enough that a 16-token block decays beyond e^60 on some
    channels (the exact elementwise path), decays near 1 (long memory), and
    chunks where only some diagonal blocks take the exact path."""
    T, H = 192, 4
    p, alpha = case(T, H, (603, ["fast_channels", "near_one", "mixed_blocks"].index(kind)))
    if kind == "fast_channels":
        alpha[:, :, :16] = 1e-3        # log2 spans ~150 per block on 16 channels
    elif kind == "near_one":
        alpha[:] = 0.999
    else:
        alpha[16:32, :, 5] = 1e-4      # one block of the first chunk, one channel
    say(f"[prefill_diag] decay regime {kind}")
    o, S = run_gpu(p, alpha, dev)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S_final", to_host(S), rS)


@pytest.mark.parametrize("T,H,bf16", [(2048, 16, True), (4097, 8, True), (3000, 12, True),
                                      (2100, 16, False), (2048, 20, True)])
def test_overlapped_plan_matches_one_pass(dev, T, H, bf16):
    """One sequence without offsets whose walk leaves CUs idle runs the
    overlapped plan in chunk ranges (the prep of the first range, then the
    walk of each range beside the prep of the next on the idle CUs, the
    state handed on between walk launches; 2048 tokens make 3 ranges, 4097
    make 5; with 20 heads the ranges could not grow by 5/4, so two ranges,
    the first launch prepping all the rest); with cu_seqlens = {0, T} the
    same sizes run prep then one walk.
    Both give the same bits, and the plan meets the oracle."""
    import dataclasses
    p = synth.make_prefill(T, H, bf16=bf16, s0_std=0.02, key=(613, T, H))
    alpha = synth.diag_alpha(T, H, key=(613, T, H))
    say(f"[prefill_diag] overlapped plan vs one pass T={T} H={H} bf16={bf16}")
    o1, S1 = (to_host(x) for x in run_gpu(p, alpha, dev))
    one = dataclasses.replace(p, cu_seqlens=np.array([0, T], np.int32))
    o2, S2 = (to_host(x) for x in run_gpu(one, alpha, dev))
    assert np.array_equal(o1, o2), "o differs from the one-pass walk"
    assert np.array_equal(S1, S2), "S_final differs from the one-pass walk"
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("overlapped o", o1, ro)
    assert_parity("overlapped S_final", S1, rS)


def test_long_prompt(dev):
    """The long prompt with per-channel decay: T = 16384, H = 16."""
    p, alpha = case(16384, 16, (604,))
    say("[prefill_diag] T=16384 H=16")
    o, S = run_gpu(p, alpha, dev)
    torch.cuda.synchronize()
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S_final", to_host(S), rS)


def test_decode_steps_equal_prefill(dev):
    """Per-channel decode steps from S0 reproduce the per-channel prefill."""
    T, H = 40, 16
    p, alpha = case(T, H, (605,))
    say("[decode_diag] 40 steps vs prefill")
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    al, b = dev_f32(alpha, dev), dev_f32(p.b, dev)
    o_pre, S_pre = rda.rda_prefill_diag(q, k, v, al, b, S0=dev_f32(p.S0, dev))
    S = dev_f32(p.S0[0][None], dev).contiguous()
    outs = [rda.rda_decode_step_diag(q[t][None].contiguous(), k[t][None].contiguous(),
                                     v[t][None].contiguous(), al[t][None].contiguous(),
                                     b[t][None].contiguous(), S) for t in range(T)]
    torch.cuda.synchronize()
    o_dec = np.concatenate([to_host(x) for x in outs])
    assert_parity("decode vs prefill o", o_dec, to_host(o_pre))
    assert_parity("decode vs prefill S", to_host(S), to_host(S_pre))
    ro, rS = oracle.prefill_diag(p.q, p.k, p.v, alpha, p.b, S0=p.S0)
    assert_parity("decode o vs oracle", o_dec, ro)


@pytest.mark.parametrize("bf16", [True, False])
def test_decode_batch(dev, bf16):
    B, H = 256, 16
    S0 = synth.decode_state(B, H, key=(606,))
    x = synth.decode_step_inputs(0, B, H, key=(606,))
    alpha = synth.diag_alpha(B, H, key=(606,))
    say(f"[decode_diag] B={B} bf16={bf16}")
    S = dev_f32(S0, dev)
    o = rda.rda_decode_step_diag(dev_tokens(x.q, bf16, dev), dev_tokens(x.k, bf16, dev),
                                 dev_tokens(x.v, bf16, dev), dev_f32(alpha, dev),
                                 dev_f32(x.b, dev), S)
    torch.cuda.synchronize()
    Sref = S0.astype(np.float64)
    ro = oracle.decode_step_diag(x.q, x.k, x.v, alpha, x.b, Sref)
    assert_parity("o", to_host(o), ro)
    assert_parity("S", to_host(S), Sref)


def test_bitwise_deterministic(dev):
    p, alpha = case(200, 16, (607,))
    say("[prefill_diag] determinism")
    outs = []
    for _ in range(2):
        o, S = run_gpu(p, alpha, dev)
        torch.cuda.synchronize()
        outs.append((to_host(o), to_host(S)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
