"""GPU test of rda_prefill_noalloc, the prefill entry point that allocates
nothing (its chunk table and factors live in the library's fixed per-GPU
scratch): called through the C ABI, it must give what rda_prefill gives on
the same inputs (the same kernels, so bit for bit) and meet the oracle's
bar, on two calls in a row, the second one smaller -- the scratch keeps the
first call's contents, which the second must not depend on."""
import numpy as np
import pytest
import torch

import oracle
from gated_delta_amd import rda, synth
from gpu_util import (assert_parity, dev_f32, dev_tokens, guarded, need_gpu, say, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def inputs(p, dev):
    q, k, v = (dev_tokens(getattr(p, n), p.bf16, dev) for n in "qkv")
    cu = (torch.from_numpy(np.asarray(p.cu_seqlens, np.int32)).to(dev)
          if p.cu_seqlens is not None else None)
    return q, k, v, dev_f32(p.a, dev), dev_f32(p.b, dev), cu, dev_f32(p.S0, dev)


def run_both(p, dev, name):
    q, k, v, a, b, cu, S0 = inputs(p, dev)
    T, H, N = p.total_tokens, p.num_heads, p.num_seqs
    say(f"[noalloc] {name}: T={T} H={H} N={N} bf16={p.bf16}")
    go = guarded((T, H, 128), torch.float32, dev)
    gs = guarded((N, H, 128, 128), torch.float32, dev)
    o1, S1 = rda.rda_prefill_noalloc(q, k, v, a, b, cu, S0, o=go.t, S_final=gs.t)
    torch.cuda.synchronize()
    go.check("o (noalloc)")
    gs.check("S_final (noalloc)")
    o2, S2 = rda.rda_prefill(q, k, v, a, b, cu_seqlens=p.cu_seqlens, S0=S0)
    torch.cuda.synchronize()
    o1, S1, o2, S2 = (to_host(x) for x in (o1, S1, o2, S2))
    assert np.array_equal(o1, o2), f"{name}: o differs from rda_prefill"
    assert np.array_equal(S1, S2), f"{name}: S_final differs from rda_prefill"
    ro, rS = oracle.prefill(p.q, p.k, p.v, p.a, p.b, cu_seqlens=p.cu_seqlens, S0=p.S0)
    assert_parity(f"{name} o", o1, ro)
    assert_parity(f"{name} S_final", S1, rS)


def largest_fitting_prompt(H):
    """The longest single prompt of H heads (a multiple of 64 tokens) whose
    workspace fits the fixed scratch."""
    T = 64
    while rda.rda_prefill_workspace_bytes(1, T + 64, H) <= rda.RDA_NOALLOC_SCRATCH_BYTES:
        T += 64
    return T


def test_two_calls_second_smaller(dev):
    # first: a long single sequence at the scratch's capacity, minus a ragged
    # tail; second: a smaller packed batch with ragged tails
    T = largest_fitting_prompt(16) - 17
    big = synth.make_prefill(T, 16, bf16=True, s0_std=0.02, key=(950,))
    run_both(big, dev, f"first call, {T} x 16")
    small = synth.make_prefill(H=4, lengths=[130, 0, 1, 64, 300], bf16=True, s0_std=0.05,
                               key=(951,))
    run_both(small, dev, "second call, 5 packed sequences x 4 heads")


def test_fp32_and_segmented_after_a_bigger_call(dev):
    # the fp32 path and the segmented state pass (one sequence, 2 heads),
    # each after a larger call has left its factors in the scratch
    run_both(synth.make_prefill(4096, 16, bf16=True, s0_std=0.02, key=(952,)), dev,
             "4096 x 16")
    run_both(synth.make_prefill(4096, 2, bf16=True, s0_std=0.02, key=(953,)), dev,
             "segmented 4096 x 2")
    run_both(synth.make_prefill(200, 3, bf16=False, s0_std=0.05, key=(954,)), dev,
             "fp32 200 x 3")


def test_rejects_too_large_before_launching(dev):
    p = synth.make_prefill(16384, 16, bf16=True, key=(955,))
    q, k, v, a, b, cu, S0 = inputs(p, dev)
    o = torch.empty((16384, 16, 128), dtype=torch.float32, device=dev)
    with pytest.raises(rda.RdaError) as e:
        rda.rda_prefill_noalloc(q, k, v, a, b, cu, S0, o=o)
    assert e.value.status == rda.RDA_ERR_TOO_LARGE
