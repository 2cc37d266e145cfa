"""GPU parity of rda_decode_tokens_diag (several tokens per sequence with a
per-key-channel decay) against the fp64 oracle (MI355X)."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import assert_parity, dev_f32, dev_tokens, need_gpu, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def case(B, T, H, key, bf16=True):
    x = synth.decode_tokens_inputs(B, T, H, bf16=bf16, key=key)
    alpha = synth.diag_alpha(B * T, H, key=key).reshape(B, T, H, 128)
    return x, alpha


def args_dev(x, alpha, dev, bf16=True):
    return ([dev_tokens(getattr(x, n), bf16, dev) for n in "qkv"]
            + [dev_f32(alpha, dev), dev_f32(x.b, dev)])


def accept_dev(acc, dev):
    return torch.from_numpy(np.ascontiguousarray(acc, dtype=np.int32)).to(dev)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("T", [1, 3, 7])
def test_verify_and_commit_one_pass(dev, T, bf16):
    B, H = 6, 16
    x, alpha = case(B, T, H, (320, T), bf16)
    x.accept[:2] = [0, T]
    S0 = synth.decode_state(B, H, key=(320, T))
    S_in, S_out = dev_f32(S0, dev), torch.full_like(dev_f32(S0, dev), float("nan"))
    say(f"[decode_tokens_diag] B={B} T={T} bf16={bf16} accept={x.accept.tolist()}")
    o = rda.rda_decode_tokens_diag(*args_dev(x, alpha, dev, bf16), S_in, S_out=S_out,
                                   accept=accept_dev(x.accept, dev))
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens_diag(x.q, x.k, x.v, alpha, x.b, S0, x.accept)
    assert_parity("o, every token", to_host(o), ro)
    assert_parity("committed S", to_host(S_out), rS)
    assert np.array_equal(to_host(S_in), S0)
    assert np.array_equal(to_host(S_out)[0], S0[0])


def test_verify_then_commit_two_calls(dev):
    B, T, H = 8, 3, 16
    x, alpha = case(B, T, H, (321,))
    S0 = synth.decode_state(B, H, key=(321,))
    args = args_dev(x, alpha, dev)
    S = dev_f32(S0, dev)
    say(f"[decode_tokens_diag] verify then commit accept={x.accept.tolist()}")
    o = rda.rda_decode_tokens_diag(*args, S)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(S), S0)
    assert rda.rda_decode_tokens_diag(None, *args[1:], S, S_out=S,
                                      accept=accept_dev(x.accept, dev), o=False) is None
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens_diag(x.q, x.k, x.v, alpha, x.b, S0, x.accept)
    assert_parity("verify o", to_host(o), ro)
    assert_parity("commit S", to_host(S), rS)


def test_one_token_matches_decode_step_diag(dev):
    B, H = 16, 16
    x, alpha = case(B, 1, H, (322,))
    S0 = synth.decode_state(B, H, key=(322,))
    S_a, S_b = dev_f32(S0, dev), dev_f32(S0, dev)
    args = args_dev(x, alpha, dev)
    say("[decode_tokens_diag] T=1 against rda_decode_step_diag")
    o_a = rda.rda_decode_tokens_diag(*args, S_a, S_out=S_a)
    o_b = rda.rda_decode_step_diag(*(t[:, 0].contiguous() for t in args), S_b)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_host(o_a)[:, 0], to_host(o_b), rtol=0, atol=1e-6)
    np.testing.assert_allclose(to_host(S_a), to_host(S_b), rtol=0, atol=1e-6)


def test_channel_constant_decay_is_scalar(dev):
    """alpha equal on every key channel gives rda_decode_tokens with that a."""
    B, T, H = 8, 3, 16
    x, _ = case(B, T, H, (323,))
    alpha = np.ascontiguousarray(np.repeat(x.a[..., None], 128, axis=3))
    S0 = synth.decode_state(B, H, key=(323,))
    args = args_dev(x, alpha, dev)
    S_d, S_s = dev_f32(S0, dev), dev_f32(S0, dev)
    acc = accept_dev(x.accept, dev)
    say("[decode_tokens_diag] channel-constant decay")
    o_d = rda.rda_decode_tokens_diag(*args, S_d, S_out=S_d, accept=acc)
    o_s = rda.rda_decode_tokens(*args[:3], dev_f32(x.a, dev), args[4], S_s, S_out=S_s,
                                accept=acc)
    torch.cuda.synchronize()
    assert_parity("o vs scalar", to_host(o_d), to_host(o_s))
    assert_parity("S vs scalar", to_host(S_d), to_host(S_s))


def test_zero_tokens_and_clamped_accept(dev):
    B, H = 3, 16
    x, alpha = case(B, 0, H, (324,))
    S0 = synth.decode_state(B, H, key=(324,))
    S_out = torch.full((B, H, 128, 128), float("nan"), device=dev)
    say("[decode_tokens_diag] T=0 copy, accept clamping")
    rda.rda_decode_tokens_diag(*args_dev(x, alpha, dev), dev_f32(S0, dev), S_out=S_out)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(S_out), S0)
    T = 3
    x, alpha = case(4, T, H, (325,))
    S0 = synth.decode_state(4, H, key=(325,))
    args = args_dev(x, alpha, dev)
    outs = []
    for acc in ([-5, 0, T + 4, T], [0, 0, T, T]):
        S_out = torch.empty_like(dev_f32(S0, dev))
        rda.rda_decode_tokens_diag(*args, dev_f32(S0, dev), S_out=S_out,
                                   accept=accept_dev(acc, dev))
        torch.cuda.synchronize()
        outs.append(to_host(S_out))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0][:2], S0[:2])


def test_max_tokens_equals_prefill_diag(dev):
    """64 tokens per sequence against rda_prefill_diag over the same packed
    sequences, and against the oracle."""
    B, T, H = 4, rda.RDA_DECODE_MAX_TOKENS, 16
    x, alpha = case(B, T, H, (326,))
    S0 = synth.decode_state(B, H, key=(326,))
    args = args_dev(x, alpha, dev)
    S = dev_f32(S0, dev)
    say(f"[decode_tokens_diag] T={T} against prefill_diag")
    o = rda.rda_decode_tokens_diag(*args, S, S_out=S)
    flat = [t.reshape((B * T,) + tuple(t.shape[2:])).contiguous() for t in args]
    cu = torch.from_numpy(synth.cu_from_lengths([T] * B).astype(np.int32)).to(dev)
    o_pre, S_pre = rda.rda_prefill_diag(*flat, cu_seqlens=cu, S0=dev_f32(S0, dev))
    torch.cuda.synchronize()
    assert_parity("o vs prefill_diag", to_host(o).reshape(B * T, H, 128), to_host(o_pre))
    assert_parity("S vs prefill_diag", to_host(S), to_host(S_pre))
    ro, rS = oracle.decode_tokens_diag(x.q, x.k, x.v, alpha, x.b, S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S", to_host(S), rS)


def test_full_workload(dev):
    """256 sequences x 16 heads, three tokens, per-sequence accept counts,
    in place (the launch the bench times); every one of the 4096 states is
    checked against the oracle."""
    B, T, H = 256, 3, 16
    x, alpha = case(B, T, H, (327,))
    S0 = synth.decode_state(B, H)
    S = dev_f32(S0, dev)
    say(f"[decode_tokens_diag] full workload B={B} T={T} H={H}, every state")
    o = rda.rda_decode_tokens_diag(*args_dev(x, alpha, dev), S, S_out=S,
                                   accept=accept_dev(x.accept, dev))
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens_diag(x.q, x.k, x.v, alpha, x.b, S0, x.accept)
    assert_parity("o, all states", to_host(o), ro)
    assert_parity("S, all states", to_host(S), rS)


def test_bitwise_deterministic(dev):
    B, T, H = 8, 3, 16
    x, alpha = case(B, T, H, (329,))
    S0 = synth.decode_state(B, H, key=(329,))
    say("[decode_tokens_diag] determinism")
    outs = []
    for _ in range(2):
        S = dev_f32(S0, dev)
        o = rda.rda_decode_tokens_diag(*args_dev(x, alpha, dev), S, S_out=S,
                                       accept=accept_dev(x.accept, dev))
        torch.cuda.synchronize()
        outs.append((to_host(o), to_host(S)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
