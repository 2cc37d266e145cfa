"""HIP graph capture of the library's calls (MI355X).

Every entry point only enqueues kernels on the caller's stream: no device
allocation, no memset, no host synchronisation (with cu_seqlens None, the
binding reads no offsets back).  So a launch-bound caller -- a decode loop,
a short prefill -- can capture the calls once and replay them.  Each test
captures with torch.cuda.graph, replays several times with eager work and
synchronisations between the replays, and checks every replay bit for bit
against the same calls run eagerly (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

from gated_delta_amd import rda, synth
from gpu_util import dev_f32, dev_tokens, need_gpu, say, to_host

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def warm_then_capture(fn):
    """One eager call on a side stream (as torch asks before a capture), then
    the capture of fn on the graph's stream."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def busy(dev):
    """Unrelated eager work between replays."""
    x = torch.randn(1 << 20, device=dev)
    (x * 2 + 1).sum().item()


def test_decode_steps(dev):
    B, H, steps = 8, 16, 4
    S0 = dev_f32(synth.decode_state(B, H, key=(800,)), dev)
    toks = []
    for i in range(steps):
        x = synth.decode_step_inputs(i, B, H, key=(800,))
        toks.append([dev_tokens(getattr(x, n), True, dev) for n in "qkv"]
                    + [dev_f32(x.a, dev), dev_f32(x.b, dev)])
    say(f"[graph] {steps} decode steps, B={B} H={H}")
    S_e = S0.clone()
    outs_e = [rda.rda_decode_step(*toks[i], S_e) for i in range(steps)]
    torch.cuda.synchronize()
    S_g = S0.clone()
    outs_g = [torch.empty((B, H, 128), device=dev) for _ in range(steps)]

    def calls():
        for i in range(steps):
            rda.rda_decode_step(*toks[i], S_g, o=outs_g[i])
    g = warm_then_capture(calls)
    for r in range(REPLAYS):
        S_g.copy_(S0)
        g.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            assert torch.equal(outs_g[i], outs_e[i]), f"replay {r}, step {i}"
        assert torch.equal(S_g, S_e), f"replay {r}, state"
        busy(dev)


@pytest.mark.parametrize("T,H,bf16", [(64, 1, False), (300, 4, True), (4096, 4, True),
                                      (2048, 16, True)])
def test_prefill(dev, T, H, bf16):
    """A short prefill (launch-bound), a packed-size one, one that takes the
    segmented state pass (4096 tokens x 4 heads) and one that takes the
    overlapped plan (2048 x 16: prep of the first chunks, then their walk
    beside the prep of the rest, then the rest of the walk)."""
    p = synth.make_prefill(T, H, bf16=bf16, s0_std=0.02, key=(801, T, H))
    q, k, v = (dev_tokens(getattr(p, n), bf16, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    S0 = dev_f32(p.S0, dev)
    say(f"[graph] prefill T={T} H={H} bf16={bf16}")
    o_e, S_e = rda.rda_prefill(q, k, v, a, b, S0=S0)
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_e)
    S_g = torch.empty_like(S_e)
    ws = torch.empty(rda.rda_prefill_workspace_bytes(1, T, H), dtype=torch.uint8, device=dev)
    g = warm_then_capture(lambda: rda.rda_prefill(q, k, v, a, b, S0=S0, o=o_g, S_final=S_g,
                                                  workspace=ws))
    for r in range(REPLAYS):
        o_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {r}: o"
        assert torch.equal(S_g, S_e), f"replay {r}: S_final"
        busy(dev)


@pytest.mark.parametrize("T,H", [(300, 4), (4100, 16)])
def test_prefill_norm_gate(dev, T, H):
    """The prefill fused with the output norm and gate; 4100 x 16 takes the
    overlapped plan with its last walk launch cut in two, the norm of walked
    rows running beside the walk."""
    p = synth.make_prefill(T, H, bf16=True, s0_std=0.02, key=(803, T, H))
    x = synth.epilogue_inputs(T * H, key=(803, T))
    q, k, v = (dev_tokens(getattr(p, n), True, dev) for n in "qkv")
    a, b = dev_f32(p.a, dev), dev_f32(p.b, dev)
    S0 = dev_f32(p.S0, dev)
    g = dev_tokens(x.g.reshape(T, H, 128), True, dev)
    w = dev_f32(x.weight, dev)
    say(f"[graph] prefill_norm_gate T={T} H={H}")
    o_e, S_e = rda.rda_prefill_norm_gate(q, k, v, a, b, g, S0=S0, weight=w)
    torch.cuda.synchronize()
    o_g = torch.empty_like(o_e)
    S_g = torch.empty_like(S_e)
    ws = torch.empty(rda.rda_prefill_norm_gate_workspace_bytes(1, T, H), dtype=torch.uint8,
                     device=dev)
    gr = warm_then_capture(lambda: rda.rda_prefill_norm_gate(q, k, v, a, b, g, S0=S0, weight=w,
                                                             out=o_g, S_final=S_g, workspace=ws))
    for r in range(REPLAYS):
        o_g.fill_(float("nan"))
        S_g.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {r}: out"
        assert torch.equal(S_g, S_e), f"replay {r}: S_final"
        busy(dev)


def test_block(dev):
    """The whole block -- prologue, prefill, output norm and gate -- as one
    graph."""
    T, H = 256, 4
    x = synth.prologue_inputs(T, H, 4, key=(802,))
    xq, xk, xv = (dev_tokens(getattr(x, n), True, dev) for n in ("xq", "xk", "xv"))
    w, br, gl, de = (dev_f32(getattr(x, n), dev) for n in ("conv_w", "beta_raw", "g_log", "delta"))
    hist = dev_tokens(x.hist, True, dev)
    gate = dev_tokens(synth.epilogue_inputs(T * H, key=(802,)).g, True, dev).reshape(T, H, 128)
    say(f"[graph] block T={T} H={H}")

    def block(hist_out):
        q, k, v, a, b = rda.rda_prologue(xq, xk, xv, w, br, gl, delta=de, hist_in=hist,
                                         hist_out=hist_out)
        o, S = rda.rda_prefill(q, k, v, a, b)
        return rda.rda_output_norm_gate(o, gate), S

    h_e = torch.empty_like(hist)
    out_e, S_e = block(h_e)
    torch.cuda.synchronize()
    h_g = torch.empty_like(hist)
    res = {}

    def capture():
        res["out"], res["S"] = block(h_g)
    g = warm_then_capture(capture)
    for r in range(REPLAYS):
        res["out"].fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(res["out"], out_e), f"replay {r}: block output"
        assert torch.equal(res["S"], S_e), f"replay {r}: state"
        assert torch.equal(h_g, h_e), f"replay {r}: history"
        busy(dev)
