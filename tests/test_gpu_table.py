"""The GPU chunk table equals the integer CPU reference bit for bit."""
import numpy as np
import pytest
import torch

import table_ref
from gated_delta_amd import rda, synth
from gpu_util import need_gpu, say, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def check(cu, N, T, dev):
    say(f"[table] N={N} T={T}")
    cud = None if cu is None else torch.from_numpy(np.asarray(cu, np.int32)).to(dev)
    rec, off, nch = rda.rda_chunk_table(cud, N, T, device=dev)
    torch.cuda.synchronize()
    rrec, roff, rn = table_ref.chunk_table(cu, N, T)
    assert int(to_host(nch)[0]) == rn
    assert np.array_equal(to_host(off), roff)
    assert np.array_equal(to_host(rec), rrec)


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 16384])
def test_single_sequence_null_offsets(dev, T):
    check(None, 1, T, dev)


def test_varlen_workload_table(dev):
    L = synth.config4_lengths()
    check(synth.cu_from_lengths(L), len(L), int(L.sum()), dev)


def test_random_varlen_tables(dev):
    rng = np.random.default_rng(300)
    for trial in range(20):
        N = int(rng.integers(1, 3000)) if trial % 5 == 0 else int(rng.integers(1, 40))
        lens = rng.integers(0, 400, size=N) * (rng.random(N) > 0.2)
        cu = synth.cu_from_lengths(lens)
        check(cu, N, int(cu[-1]), dev)


def test_malformed_offsets_stay_in_bounds(dev):
    """Unvalidated, non-monotone offsets: the kernel clamps and caps, so the
    table stays within its bound and every record lies inside [0, T)."""
    T, N = 300, 4
    cu = np.array([0, 290, 10, 300, 300], np.int32)
    say("[table] malformed offsets")
    cud = torch.from_numpy(cu).to(dev)
    rec, off, nch = rda.rda_chunk_table(cud, N, T, device=dev)
    torch.cuda.synchronize()
    rec, n = to_host(rec), int(to_host(nch)[0])
    assert 0 <= n <= table_ref.max_chunks(N, T)
    for r in rec[:n]:
        assert 0 <= r[0] < N and 0 <= r[1] and 1 <= r[2] <= 64 and r[1] + r[2] <= T


def _align256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("T", [1, 63, 64, 65, 1000, 16384])
@pytest.mark.parametrize("bf16", [True, False])
def test_prep_written_table_single_sequence(dev, T, bf16):
    """One sequence without offsets (bf16 or fp32 inputs): the prep kernel
    writes the chunk table itself (no table kernel runs).  Read it back from the workspace
    (library-internal layout: records at 0, then sequence offsets and the
    chunk count at the next 256-byte boundaries) and compare with the integer
    reference; the workspace starts filled with a byte pattern so that a
    missing write shows."""
    H = 2
    say(f"[table] prep-written T={T} bf16={bf16}")
    p = synth.make_prefill(T, H, bf16=bf16, key=(900, T))
    dt = torch.bfloat16 if bf16 else torch.float32
    q, k, v = (torch.from_numpy(getattr(p, n)).to(dev).to(dt) for n in "qkv")
    a, b = (torch.from_numpy(x).to(dev) for x in (p.a, p.b))
    mc = table_ref.max_chunks(1, T)
    ws = torch.full((rda.rda_prefill_workspace_bytes(1, T, H),), 0x5A, dtype=torch.uint8,
                    device=dev)
    rda.rda_prefill(q, k, v, a, b, workspace=ws)
    torch.cuda.synchronize()
    w = to_host(ws)
    so = _align256(mc * 16)
    no = so + _align256(2 * 4)
    rec = w[:mc * 16].view(np.int32).reshape(mc, 4)
    off = w[so:so + 8].view(np.int32)
    n = int(w[no:no + 4].view(np.int32)[0])
    rrec, roff, rn = table_ref.chunk_table(None, 1, T)
    assert n == rn and np.array_equal(off, roff) and np.array_equal(rec, rrec)
