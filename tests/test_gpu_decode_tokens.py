"""GPU parity of rda_decode_tokens (several tokens per sequence: the verify
of drafted tokens) against the fp64 oracle (MI355X)."""
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


def tok_dev(x: synth.DecodeTokensInputs, dev, bf16=True):
    return ([dev_tokens(getattr(x, n), bf16, dev) for n in "qkv"]
            + [dev_f32(x.a, dev), dev_f32(x.b, dev)])


def accept_dev(acc, dev):
    return torch.from_numpy(np.ascontiguousarray(acc, dtype=np.int32)).to(dev)


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("T", [1, 2, 3, 7])
def test_verify_and_commit_one_pass(dev, T, bf16):
    """Outputs of every token; S_out = state after each sequence's accepted
    prefix (counts 0..T drawn per sequence); S_in untouched."""
    B, H = 6, 16
    x = synth.decode_tokens_inputs(B, T, H, bf16=bf16, key=(300, T))
    x.accept[:2] = [0, T]
    S0 = synth.decode_state(B, H, key=(300, T))
    S_in, S_out = dev_f32(S0, dev), torch.full_like(dev_f32(S0, dev), float("nan"))
    say(f"[decode_tokens] B={B} T={T} H={H} bf16={bf16} accept={x.accept.tolist()}")
    o = rda.rda_decode_tokens(*tok_dev(x, dev, bf16), S_in, S_out=S_out,
                              accept=accept_dev(x.accept, dev))
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0, x.accept)
    assert_parity("o, every token", to_host(o), ro)
    assert_parity("committed S", to_host(S_out), rS)
    assert np.array_equal(to_host(S_in), S0)
    assert np.array_equal(to_host(S_out)[0], S0[0])      # accept 0 copies S_in


def test_in_place_all_accepted(dev):
    B, T, H = 5, 3, 16
    x = synth.decode_tokens_inputs(B, T, H, key=(301,))
    S0 = synth.decode_state(B, H, key=(301,))
    S = dev_f32(S0, dev)
    say(f"[decode_tokens] in place B={B} T={T}")
    o = rda.rda_decode_tokens(*tok_dev(x, dev), S, S_out=S)
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S", to_host(S), rS)


def test_verify_then_commit_two_calls(dev):
    """A read-only verify (no state written) followed by a commit-only call
    (no outputs, q not passed) gives what one pass with the counts gives."""
    B, T, H = 8, 3, 16
    x = synth.decode_tokens_inputs(B, T, H, key=(302,))
    S0 = synth.decode_state(B, H, key=(302,))
    args = tok_dev(x, dev)
    acc = accept_dev(x.accept, dev)
    S = dev_f32(S0, dev)
    say(f"[decode_tokens] verify then commit B={B} T={T} accept={x.accept.tolist()}")
    o_verify = rda.rda_decode_tokens(*args, S)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(S), S0)                  # verify writes no state
    res = rda.rda_decode_tokens(None, *args[1:], S, S_out=S, accept=acc, o=False)
    torch.cuda.synchronize()
    assert res is None
    S1, S_one = dev_f32(S0, dev), torch.empty_like(S)
    o_one = rda.rda_decode_tokens(*args, S1, S_out=S_one, accept=acc)
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0, x.accept)
    assert_parity("verify o", to_host(o_verify), ro)
    assert_parity("commit S", to_host(S), rS)
    assert np.array_equal(to_host(o_verify), to_host(o_one))
    np.testing.assert_allclose(to_host(S), to_host(S_one), rtol=0, atol=1e-6)


def test_accept_counts_are_clamped(dev):
    B, T, H = 4, 3, 16
    x = synth.decode_tokens_inputs(B, T, H, key=(303,))
    S0 = synth.decode_state(B, H, key=(303,))
    args = tok_dev(x, dev)
    say("[decode_tokens] accept clamping")
    outs = []
    for acc in ([-5, 0, T + 4, T], [0, 0, T, T]):
        S_out = torch.empty_like(dev_f32(S0, dev))
        rda.rda_decode_tokens(*args, dev_f32(S0, dev), S_out=S_out, accept=accept_dev(acc, dev))
        torch.cuda.synchronize()
        outs.append(to_host(S_out))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0][:2], S0[:2])


def test_one_token_matches_decode_step(dev):
    """tokens = 1, in place, all accepted: the decode step."""
    B, H = 16, 16
    x = synth.decode_tokens_inputs(B, 1, H, key=(304,))
    S0 = synth.decode_state(B, H, key=(304,))
    S_a, S_b = dev_f32(S0, dev), dev_f32(S0, dev)
    args = tok_dev(x, dev)
    say("[decode_tokens] T=1 against rda_decode_step")
    o_a = rda.rda_decode_tokens(*args, S_a, S_out=S_a)
    o_b = rda.rda_decode_step(*(t[:, 0].contiguous() for t in args), S_b)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_host(o_a)[:, 0], to_host(o_b), rtol=0, atol=1e-6)
    np.testing.assert_allclose(to_host(S_a), to_host(S_b), rtol=0, atol=1e-6)
    ro, rS = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0)
    assert_parity("o", to_host(o_a), ro)
    assert_parity("S", to_host(S_a), rS)


def test_identity_gates_keep_state(dev):
    B, T, H = 4, 3, 16
    x = synth.decode_tokens_inputs(B, T, H, key=(305,))
    x.a[:] = 1.0
    x.b[:] = 0.0
    S0 = synth.decode_state(B, H, key=(305,))
    S = dev_f32(S0, dev)
    say("[decode_tokens] a=1, b=0")
    o = rda.rda_decode_tokens(*tok_dev(x, dev), S, S_out=S)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(S), S0)
    ro, _ = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0)
    assert_parity("identity o", to_host(o), ro)


def test_zero_tokens_copies_state(dev):
    B, H = 3, 16
    x = synth.decode_tokens_inputs(B, 0, H, key=(306,))
    S0 = synth.decode_state(B, H, key=(306,))
    S_out = torch.full((B, H, 128, 128), float("nan"), device=dev)
    say("[decode_tokens] T=0 copy")
    o = rda.rda_decode_tokens(*tok_dev(x, dev), dev_f32(S0, dev), S_out=S_out)
    torch.cuda.synchronize()
    assert o.shape == (B, 0, H, 128)
    assert np.array_equal(to_host(S_out), S0)


def test_empty_batch(dev):
    x = synth.decode_tokens_inputs(0, 3, 16, key=(307,))
    say("[decode_tokens] B=0")
    S = torch.zeros((0, 16, 128, 128), device=dev)
    o = rda.rda_decode_tokens(*tok_dev(x, dev), S, S_out=S)
    torch.cuda.synchronize()
    assert o.shape == (0, 3, 16, 128)


def test_max_tokens_equals_prefill(dev):
    """64 tokens per sequence (the maximum) against rda_prefill over the
    same packed sequences, both on the GPU, and against the oracle."""
    B, T, H = 4, rda.RDA_DECODE_MAX_TOKENS, 16
    x = synth.decode_tokens_inputs(B, T, H, key=(308,))
    S0 = synth.decode_state(B, H, key=(308,))
    args = tok_dev(x, dev)
    S = dev_f32(S0, dev)
    say(f"[decode_tokens] T={T} against prefill")
    o = rda.rda_decode_tokens(*args, S, S_out=S)
    flat = [t.reshape((B * T,) + tuple(t.shape[2:])).contiguous() for t in args]
    cu = torch.from_numpy(synth.cu_from_lengths([T] * B).astype(np.int32)).to(dev)
    o_pre, S_pre = rda.rda_prefill(*flat, cu_seqlens=cu, S0=dev_f32(S0, dev))
    torch.cuda.synchronize()
    assert_parity("o vs prefill", to_host(o).reshape(B * T, H, 128), to_host(o_pre))
    assert_parity("S vs prefill", to_host(S), to_host(S_pre))
    ro, rS = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0)
    assert_parity("o", to_host(o), ro)
    assert_parity("S", to_host(S), rS)


def test_full_workload(dev):
    """256 sequences x 16 heads, one token plus two drafts, per-sequence
    accept counts, in place (the launch the bench times); the oracle checks
    every one of the 4096 states: o of every token and the committed S."""
    B, T, H = 256, 3, 16
    x = synth.decode_tokens_inputs(B, T, H)
    S0 = synth.decode_state(B, H)
    S = dev_f32(S0, dev)
    say(f"[decode_tokens] full workload B={B} T={T} H={H}, every state")
    o = rda.rda_decode_tokens(*tok_dev(x, dev), S, S_out=S, accept=accept_dev(x.accept, dev))
    torch.cuda.synchronize()
    ro, rS = oracle.decode_tokens(x.q, x.k, x.v, x.a, x.b, S0, x.accept)
    assert_parity("o, all states", to_host(o), ro)
    assert_parity("S, all states", to_host(S), rS)


def test_bitwise_deterministic(dev):
    B, T, H = 8, 3, 16
    x = synth.decode_tokens_inputs(B, T, H, key=(310,))
    S0 = synth.decode_state(B, H, key=(310,))
    say("[decode_tokens] determinism")
    outs = []
    for _ in range(2):
        S = dev_f32(S0, dev)
        o = rda.rda_decode_tokens(*tok_dev(x, dev), S, S_out=S, accept=accept_dev(x.accept, dev))
        torch.cuda.synchronize()
        outs.append((to_host(o), to_host(S)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
