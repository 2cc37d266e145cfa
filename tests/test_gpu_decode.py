"""GPU parity of rda_decode_step against the fp64 oracle, and decode against
prefill (MI355X)."""
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


def step_dev(x: synth.DecodeStepInputs, dev, bf16=True):
    return ([dev_tokens(getattr(x, n), bf16, dev) for n in "qkv"]
            + [dev_f32(x.a, dev), dev_f32(x.b, dev)])


@pytest.mark.parametrize("bf16", [True, False])
def test_decode_small_batch(dev, bf16):
    B, H, steps = 3, 16, 6
    S0 = synth.decode_state(B, H, key=(200,))
    S = dev_f32(S0, dev)
    Sref = S0.astype(np.float64)
    say(f"[decode] B={B} H={H} steps={steps} bf16={bf16}")
    for t in range(steps):
        x = synth.decode_step_inputs(t, B, H, key=(200,))
        o = rda.rda_decode_step(*step_dev(x, dev, bf16), S)
        ro = oracle.decode_step(x.q, x.k, x.v, x.a, x.b, Sref)
        torch.cuda.synchronize()
        assert_parity(f"step {t} o", to_host(o), ro)
    assert_parity("final S", to_host(S), Sref)


def test_decode_full_workload(dev):
    """B=256, H=16, 128 consecutive steps in place (the workload the bench
    times); the oracle follows every one of the 4096 states through every
    step: o of all steps and the final S, element by element."""
    B, H, steps = 256, 16, 128
    S0 = synth.decode_state(B, H)
    S = dev_f32(S0, dev)
    Sref = S0.astype(np.float64)   # [B, H, dv, dk], updated in place by the oracle
    err = ErrorSums()
    say(f"[decode] full workload B={B} H={H} steps={steps}, every state")
    for t in range(steps):
        x = synth.decode_step_inputs(t, B, H)
        o = rda.rda_decode_step(*step_dev(x, dev), S)
        ro = oracle.decode_step(x.q, x.k, x.v, x.a, x.b, Sref)
        err.add(to_host(o), ro)
    err.check("o, all states, all steps")
    assert_parity("final S, all states", to_host(S), Sref)


def test_decode_identity_gates_keep_state(dev):
    B, H = 4, 16
    S0 = synth.decode_state(B, H, key=(202,))
    x = synth.decode_step_inputs(0, B, H, key=(202,))
    x.a[:] = 1.0
    x.b[:] = 0.0
    S = dev_f32(S0, dev)
    say("[decode] a=1, b=0")
    o = rda.rda_decode_step(*step_dev(x, dev), S)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(S), S0)
    ro = oracle.decode_step(x.q, x.k, x.v, x.a, x.b, S0.astype(np.float64))
    assert_parity("identity o", to_host(o), ro)


def test_decode_steps_equal_prefill(dev):
    """T decode steps from S0 reproduce one T-token prefill (both on GPU)."""
    T, H = 100, 4
    p = synth.make_prefill(T, H, bf16=True, s0_std=0.05, key=(203,))
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    say("[decode] decode x100 vs prefill")
    o_pre, S_pre = rda.rda_prefill(q, k, v, a, b, S0=dev_f32(p.S0, dev))
    S = dev_f32(p.S0[0][None], dev).contiguous()
    outs = []
    for t in range(T):
        outs.append(rda.rda_decode_step(q[t][None].contiguous(), k[t][None].contiguous(),
                                        v[t][None].contiguous(), a[t][None].contiguous(),
                                        b[t][None].contiguous(), S))
    torch.cuda.synchronize()
    o_dec = np.concatenate([to_host(x) for x in outs])
    assert_parity("decode vs prefill o", o_dec, to_host(o_pre))
    assert_parity("decode vs prefill S", to_host(S), to_host(S_pre))


def test_decode_bitwise_deterministic(dev):
    B, H = 8, 16
    S0 = synth.decode_state(B, H, key=(204,))
    x = synth.decode_step_inputs(0, B, H, key=(204,))
    outs = []
    say("[decode] determinism")
    for _ in range(2):
        S = dev_f32(S0, dev)
        o = rda.rda_decode_step(*step_dev(x, dev), S)
        torch.cuda.synchronize()
        outs.append((to_host(o), to_host(S)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
