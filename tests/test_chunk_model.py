"""The chunked WY/UT algebra (NumPy design model) against the fp64 oracle,
and the predicted error of the kernels' bf16 hi/lo precision plan (CPU)."""
import numpy as np
import pytest

import chunk_model as cm
import oracle
import pins
from gated_delta_amd import synth


@pytest.mark.parametrize("T", [1, 7, 8, 9, 63, 64, 65, 130])
def test_chunk_algebra_matches_oracle(T):
    rng = np.random.default_rng([31, T])
    q, k, v, a, b, S0 = pins.random_case(rng, T, 2, 16, 12)
    o, S = oracle.prefill(q, k, v, a, b, S0=S0)
    for C in (8, 64):
        o2, S2 = cm.chunk_prefill(q, k, v, a, b, S0=S0, C=C)
        assert np.abs(o2 - o).max() < 1e-12 and np.abs(S2 - S).max() < 1e-12


def test_chunk_algebra_varlen_and_empty():
    rng = np.random.default_rng(32)
    lens = [70, 0, 64, 1, 129]
    q, k, v, a, b, _ = pins.random_case(rng, sum(lens), 3, 8, 8)
    S0 = rng.standard_normal((len(lens), 3, 8, 8))
    cu = synth.cu_from_lengths(lens)
    o, S = oracle.prefill(q, k, v, a, b, cu_seqlens=cu, S0=S0)
    o2, S2 = cm.chunk_prefill(q, k, v, a, b, cu_seqlens=cu, S0=S0, C=16)
    assert np.abs(o2 - o).max() < 1e-12 and np.abs(S2 - S).max() < 1e-12


def test_kernel_precision_plan_budget():
    """bf16 inputs, fp32 state, hi/lo splits: predicted error far inside
    the rel-L2 2e-3 / max-abs 2e-2 gate, including a long-memory gate."""
    p = synth.make_prefill(512, 1, 128, 128, bf16=True, s0_std=0.02, key=(90,))
    for a_override in (None, 0.98):
        if a_override is not None:
            p.a[:] = np.float32(a_override)
        o, S = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
        o2, S2 = cm.chunk_prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0, plan=cm.KERNEL_PLAN)
        assert cm.rel_l2(o2, o) < 5e-5 and cm.rel_l2(S2, S) < 5e-5
        assert np.abs(o2 - o).max() < 1e-3


def test_single_bf16_plan_is_outside_margin():
    """Rounding every computed operand to one bf16 costs ~2e-3: the reason
    the kernels split computed operands into hi + lo."""
    p = synth.make_prefill(512, 1, 128, 128, bf16=True, s0_std=0.02, key=(91,))
    o, S = oracle.prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0)
    plan = dict(gram="x1", solve="f32", wu="x1", qo="x1", walk_x="x1", walk_s="x1",
                state="f32")
    o2, S2 = cm.chunk_prefill(p.q, p.k, p.v, p.a, p.b, S0=p.S0, plan=plan)
    assert cm.rel_l2(o2, o) > 1e-3
