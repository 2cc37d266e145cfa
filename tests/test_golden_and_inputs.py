"""Generator determinism and the oracle-written golden fixture (CPU)."""
import os

import numpy as np

import oracle
from gated_delta_amd import synth
from golden.make_golden import OUT, input_digest


def _read_fixture():
    rows = {"o": [], "S": []}
    digest = None
    for line in open(OUT):
        if line.startswith("#") or not line.strip():
            continue
        parts = line.split()
        if parts[0] == "inputs_sha256":
            digest = parts[1]
        else:
            rows[parts[0]].append((tuple(int(x) for x in parts[1:-1]), float(parts[-1])))
    return digest, rows


def test_c1_inputs_and_oracle_match_fixture():
    assert os.path.exists(OUT)
    digest, rows = _read_fixture()
    p = synth.config1()
    assert input_digest(p) == digest
    o, S = oracle.prefill(p.q, p.k, p.v, p.a, p.b)
    for idx, val in rows["o"]:
        assert abs(o[idx] - val) <= 1e-14 * max(1.0, abs(val))
    for idx, val in rows["S"]:
        assert abs(S[idx] - val) <= 1e-14 * max(1.0, abs(val))


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0],
                 dtype=np.float32)
    r = synth.round_bf16(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa is 1.0
    assert list(r) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]


def test_generator_shapes_and_ranges():
    p = synth.config2()
    assert p.q.shape == (2048, 16, 128) and p.a.shape == (2048, 16)
    assert p.S0 is None and p.cu_seqlens is None
    assert np.all(p.a > 0) and np.all(p.a < 1) and np.all(p.b > 0) and np.all(p.b < 1)
    n = np.linalg.norm(p.k.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 4e-3)
    assert np.array_equal(synth.round_bf16(p.v), p.v)


def test_varlen_lengths_recipe():
    L = synth.config4_lengths()
    assert len(L) == 8 and L.sum() == 32768 and L.min() >= 512 and L.max() <= 8192
    assert np.array_equal(L, synth.config4_lengths())


def test_decode_inputs_deterministic():
    a = synth.decode_step_inputs(3, B=4, H=2)
    b = synth.decode_step_inputs(3, B=4, H=2)
    c = synth.decode_step_inputs(4, B=4, H=2)
    assert np.array_equal(a.q, b.q) and not np.array_equal(a.q, c.q)
