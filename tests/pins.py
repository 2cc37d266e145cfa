"""Pins for the fp64 oracle: checks against what the mathematics fixes.

Each ``pin_*`` takes an oracle handle (anything with ``prefill`` and
``decode_step`` like ``oracle.Oracle``) and raises AssertionError when the
handle disagrees with a result fixed independently of the oracle's code:

* the unrolled product form of the recurrence (brute force, T <= 4),
* exact rational arithmetic on dyadic inputs (bitwise),
* invariants the recurrence must satisfy (identity gates, read-back with
  orthonormal keys, pure decay, linearity, rotation and permutation
  equivariance, the state-norm bound),
* structural identities (resume = one call, packed varlen = separate calls,
  decode steps = prefill).

The recurrence, per the "Raon-1 nano" teardown (section "The other 1.5B: a
hybrid built to forget"): scale the state by the decay, take the residual
e = v - S'k of the scaled state at the key, add b e k^T; read out
o_t = S_t q_t.  As a product: S_t = S_{t-1} A_t + b_t v_t k_t^T
with A_t = a_t (I - b_t k_t k_t^T).  The module is shared by
``test_oracle_pins.py`` (real oracle) and ``test_oracle_mutants.py``
(builds of the oracle with a planted mistake, which must fail some pin).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

RNG_KEY = 777


def _rng(i):
    return np.random.default_rng([RNG_KEY, i])


def _close(x, y, rtol=1e-12, what=""):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, (what, x.shape, y.shape)
    scale = max(1.0, float(np.max(np.abs(y))) if y.size else 1.0)
    err = float(np.max(np.abs(x - y))) if y.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _d(x):
    return np.asarray(x, dtype=np.float64)


def random_case(rng, T, H, dk, dv, unit_keys=True, s0=True):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    a = rng.uniform(0.05, 1.0, (T, H))
    b = rng.uniform(0.0, 1.0, (T, H))
    S0 = rng.standard_normal((1, H, dv, dk)) if s0 else None
    return [_f32(x) for x in (q, k, v, a, b)] + [S0]


# --------------------------------------------------------------------------
# brute force: unrolled product form
# --------------------------------------------------------------------------
def product_form(q, k, v, a, b, S0):
    """One head: S_t = S0 A_1..A_t + sum_{s<=t} b_s v_s k_s^T A_{s+1}..A_t.

    Inputs are float64 arrays q,k [T,dk], v [T,dv], a,b [T], S0 [dv,dk].
    Returns (o [T,dv], S_T [dv,dk]).
    """
    T, dk = k.shape
    I = np.eye(dk)
    A = [a[t] * (I - b[t] * np.outer(k[t], k[t])) for t in range(T)]

    def chain(i, j):  # A_i ... A_j (1-based, inclusive); identity if empty
        P = np.eye(dk)
        for s in range(i, j + 1):
            P = P @ A[s - 1]
        return P

    o = np.zeros((T, v.shape[1]))
    S = None
    for t in range(1, T + 1):
        S = S0 @ chain(1, t)
        for s in range(1, t + 1):
            S = S + b[s - 1] * np.outer(v[s - 1], k[s - 1]) @ chain(s + 1, t)
        o[t - 1] = S @ q[t - 1]
    return o, S


def pin_bruteforce(orc):
    cases = [(1, 1, 4, 4, True), (2, 2, 6, 4, False), (3, 2, 8, 8, True),
             (4, 3, 5, 7, False), (4, 2, 128, 128, True)]
    for i, (T, H, dk, dv, unit) in enumerate(cases):
        q, k, v, a, b, S0 = random_case(_rng(i), T, H, dk, dv, unit_keys=unit)
        o, Sf = orc.prefill(q, k, v, a, b, S0=S0)
        for h in range(H):
            ro, rS = product_form(*(_d(x[:, h]) for x in (q, k, v, a, b)),
                                  S0[0, h])
            _close(o[:, h], ro, 1e-12, f"brute force o case {i} head {h}")
            _close(Sf[0, h], rS, 1e-12, f"brute force S case {i} head {h}")


# --------------------------------------------------------------------------
# exact rational arithmetic on dyadic inputs
# --------------------------------------------------------------------------
def _frac_matmul(A, B):
    return [[sum(A[i][m] * B[m][j] for m in range(len(B))) for j in range(len(B[0]))]
            for i in range(len(A))]


def exact_product_form(q, k, v, a, b, S0):
    """Product form in Fractions for one head (lists of Fractions)."""
    T, dk = len(k), len(k[0])
    S = [row[:] for row in S0]
    outs = []
    for t in range(T):
        A = [[a[t] * ((1 if i == j else 0) - b[t] * k[t][i] * k[t][j]) for j in range(dk)]
             for i in range(dk)]
        S = _frac_matmul(S, A)
        S = [[S[i][j] + b[t] * v[t][i] * k[t][j] for j in range(dk)] for i in range(len(S))]
        outs.append([sum(S[i][j] * q[t][j] for j in range(dk)) for i in range(len(S))])
    return outs, S


def pin_exact_dyadic(orc):
    """Dyadic inputs with few bits: every intermediate is exact in fp64, so
    the oracle must equal exact rational arithmetic bit for bit."""
    F = Fraction
    q = [[F(1, 2), F(-1, 4)], [F(0), F(1)], [F(3, 4), F(1, 2)]]
    k = [[F(1), F(0)], [F(1, 2), F(1, 2)], [F(-1, 4), F(3, 4)]]
    v = [[F(5), F(6), F(-2)], [F(1, 2), F(-3), F(1)], [F(2), F(1, 4), F(-1, 2)]]
    a = [F(1, 2), F(3, 4), F(1)]
    b = [F(1, 2), F(1, 4), F(1)]
    S0 = [[F(1), F(2)], [F(3), F(4)], [F(-1, 2), F(1, 4)]]
    eo, eS = exact_product_form(q, k, v, a, b, S0)
    tof = lambda m: np.array([[float(x) for x in r] for r in m])
    o, Sf = orc.prefill(tof(q)[:, None], tof(k)[:, None], tof(v)[:, None],
                        np.array([[float(x)] for x in a]), np.array([[float(x)] for x in b]),
                        S0=tof(S0)[None, None])
    assert np.array_equal(o[:, 0], tof(eo)), (o[:, 0], tof(eo))
    assert np.array_equal(Sf[0, 0], tof(eS)), (Sf[0, 0], tof(eS))


def pin_hand_example(orc):
    """Worked by hand: S0 = [[1,2],[3,4]], k = (1,0), q = (0,1), v = (5,6),
    a = b = 1/2.  Decay: [[.5,1],[1.5,2]]; prediction (.5,1.5); error
    (4.5,4.5); write .5*error*k^T: S = [[2.75,1],[3.75,2]]; o = S q = (1,2)."""
    o, Sf = orc.prefill(np.array([[[0.0, 1.0]]]), np.array([[[1.0, 0.0]]]),
                        np.array([[[5.0, 6.0]]]), np.array([[0.5]]), np.array([[0.5]]),
                        S0=np.array([[[[1.0, 2.0], [3.0, 4.0]]]]))
    assert np.array_equal(Sf[0, 0], [[2.75, 1.0], [3.75, 2.0]]), Sf[0, 0]
    assert np.array_equal(o[0, 0], [1.0, 2.0]), o[0, 0]


# --------------------------------------------------------------------------
# invariants and closed forms
# --------------------------------------------------------------------------
def pin_identity_gates(orc):
    """a = 1, b = 0 leaves S unchanged and reads o_t = S0 q_t."""
    q, k, v, a, b, S0 = random_case(_rng(10), 9, 2, 6, 5)
    a[:] = 1.0
    b[:] = 0.0
    o, Sf = orc.prefill(q, k, v, a, b, S0=S0)
    assert np.array_equal(Sf, S0), "S changed under a=1, b=0"
    for h in range(2):
        _close(o[:, h], _d(q[:, h]) @ S0[0, h].T, 1e-13, "o under a=1,b=0")


def pin_readback(orc):
    """a = 1, b = 1 and orthonormal keys: after writing v_s under key k_s the
    state maps k_s to v_s, so querying an earlier key reads its value."""
    rng = _rng(11)
    T, dk, dv = 10, 16, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.copy()                       # orthonormal rows
    v = rng.standard_normal((T, dv))
    src = [t // 2 for t in range(T)]             # query an earlier (or same) key
    q = k[src]
    S0 = rng.standard_normal((1, 1, dv, dk))
    # the oracle consumes fp32 inputs; use the rounded values for the check
    k32, q32, v32 = _f32(k), _f32(q), _f32(v)
    o, Sf = orc.prefill(q32[:, None], k32[:, None], v32[:, None],
                        np.ones((T, 1)), np.ones((T, 1)), S0=S0)
    # fp32-rounded keys are orthonormal to ~1e-7, so the read-back holds to ~1e-6
    _close(o[:, 0], _d(v32)[src], 2e-6, "read-back of written values")
    _close(Sf[0, 0] @ _d(k32).T, _d(v32).T, 2e-6, "S k_s = v_s")


def pin_pure_decay(orc):
    """b = 0: S_t = (prod_{s<=t} a_s) S0 and o_t = (prod a) S0 q_t."""
    q, k, v, a, b, S0 = random_case(_rng(12), 7, 2, 5, 4)
    b[:] = 0.0
    o, Sf = orc.prefill(q, k, v, a, b, S0=S0)
    for h in range(2):
        cum = np.cumprod(_d(a[:, h]))
        _close(Sf[0, h], cum[-1] * S0[0, h], 1e-13, "pure decay S")
        _close(o[:, h], cum[:, None] * (_d(q[:, h]) @ S0[0, h].T), 1e-13, "pure decay o")


def pin_single_step(orc):
    """T = 1 from S0 = 0 with q = k: o = b v (k . k)."""
    rng = _rng(13)
    k = _f32(rng.standard_normal((1, 3, 8)))
    v = _f32(rng.standard_normal((1, 3, 5)))
    a = _f32(rng.uniform(0.1, 1, (1, 3)))
    b = _f32(rng.uniform(0, 1, (1, 3)))
    o, Sf = orc.prefill(k, k, v, a, b)
    kk = np.sum(_d(k) ** 2, axis=-1)
    _close(o[0], _d(b)[0, :, None] * _d(v[0]) * kk[0, :, None], 1e-13,
           "T=1 closed form")


def pin_linearity(orc):
    """(S0, V) -> (O, S_T) is linear for fixed q, k, a, b."""
    rng = _rng(14)
    q, k, v1, a, b, S01 = random_case(rng, 12, 2, 6, 5)
    v2 = _f32(rng.standard_normal(v1.shape))
    S02 = rng.standard_normal(S01.shape)
    al, be = 0.75, -1.25   # exact in fp32, so the combined v is exact too
    v3 = _f32(_d(v1) * al + _d(v2) * be)
    o1, s1 = orc.prefill(q, k, v1, a, b, S0=S01)
    o2, s2 = orc.prefill(q, k, v2, a, b, S0=S02)
    o3, s3 = orc.prefill(q, k, v3, a, b, S0=al * S01 + be * S02)
    # v3 is rounded to fp32: allow that rounding (~6e-8 relative)
    _close(o3, al * o1 + be * o2, 1e-6, "linearity o")
    _close(s3, al * s1 + be * s2, 1e-6, "linearity S")


def pin_rotation(orc):
    """q -> R q, k -> R k, S0 -> S0 R^T gives the same o and S_T -> S_T R^T."""
    rng = _rng(15)
    q, k, v, a, b, S0 = random_case(rng, 11, 2, 8, 6)
    R, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    o1, s1 = orc.prefill(q, k, v, a, b, S0=S0)
    qr = _f32(_d(q) @ R.T)
    kr = _f32(_d(k) @ R.T)
    o2, s2 = orc.prefill(qr, kr, v, a, b, S0=S0 @ R.T)
    # rotated inputs are rounded to fp32, so agreement is to ~1e-6
    _close(o2, o1, 1e-5, "rotation o")
    _close(s2, s1 @ R.T, 1e-5, "rotation S")


def pin_permutation(orc):
    """Permuting value channels permutes rows of S and channels of o."""
    rng = _rng(16)
    q, k, v, a, b, S0 = random_case(rng, 9, 2, 6, 7)
    p = rng.permutation(7)
    o1, s1 = orc.prefill(q, k, v, a, b, S0=S0)
    o2, s2 = orc.prefill(q, k, v[:, :, p], a, b, S0=S0[:, :, p, :])
    assert np.array_equal(o2, o1[:, :, p]) and np.array_equal(s2, s1[:, :, p, :])


def pin_norm_bound(orc):
    """||S_t||_2 <= a_t ||S_{t-1}||_2 + b_t ||v_t|| ||k_t|| for unit keys."""
    q, k, v, a, b, S0 = random_case(_rng(17), 20, 1, 6, 6)
    S = np.ascontiguousarray(S0.copy())
    prev = np.linalg.norm(S[0, 0], 2)
    for t in range(20):
        orc.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], S)
        cur = np.linalg.norm(S[0, 0], 2)
        bound = a[t, 0] * prev + b[t, 0] * np.linalg.norm(v[t, 0]) * np.linalg.norm(k[t, 0])
        assert cur <= bound * (1 + 1e-12) + 1e-12, (t, cur, bound)
        prev = cur


# --------------------------------------------------------------------------
# structural identities
# --------------------------------------------------------------------------
def pin_resume(orc):
    """prefill(x) = prefill(x[t1:], S0 = prefill(x[:t1]).S_final)."""
    q, k, v, a, b, S0 = random_case(_rng(18), 30, 2, 8, 8)
    o, s = orc.prefill(q, k, v, a, b, S0=S0)
    for t1 in (1, 13, 29):
        oa, sa = orc.prefill(q[:t1], k[:t1], v[:t1], a[:t1], b[:t1], S0=S0)
        ob, sb = orc.prefill(q[t1:], k[t1:], v[t1:], a[t1:], b[t1:], S0=sa)
        _close(np.concatenate([oa, ob]), o, 1e-13, f"resume o at {t1}")
        _close(sb, s, 1e-13, f"resume S at {t1}")


def pin_varlen(orc):
    """A packed batch equals separate calls per sequence; an empty sequence
    returns its S0 unchanged."""
    rng = _rng(19)
    lens = [5, 0, 9, 1, 0, 4]
    T = sum(lens)
    q, k, v, a, b, _ = random_case(rng, T, 2, 6, 5)
    S0 = rng.standard_normal((len(lens), 2, 5, 6))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, s = orc.prefill(q, k, v, a, b, cu_seqlens=cu, S0=S0)
    for n, L in enumerate(lens):
        t0, t1 = cu[n], cu[n + 1]
        if L == 0:
            assert np.array_equal(s[n], S0[n])
            continue
        on, sn = orc.prefill(q[t0:t1], k[t0:t1], v[t0:t1], a[t0:t1], b[t0:t1], S0=S0[n:n + 1])
        _close(o[t0:t1], on, 1e-14, f"varlen o seq {n}")
        _close(s[n], sn[0], 1e-14, f"varlen S seq {n}")


def pin_decode_equals_prefill(orc):
    """T single-token decode steps equal one T-token prefill."""
    q, k, v, a, b, S0 = random_case(_rng(20), 12, 3, 6, 5)
    o, s = orc.prefill(q, k, v, a, b, S0=S0)
    S = np.ascontiguousarray(S0[0][None].repeat(1, axis=0))   # [1, H, dv, dk]
    for t in range(12):
        ot = orc.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], S)
        _close(ot[0], o[t], 1e-13, f"decode o step {t}")
    _close(S, s, 1e-13, "decode final state")


def pin_decode_tokens(orc):
    """Several tokens per sequence equal that many single-token decode steps
    per sequence; the committed state is the one after the accepted tokens
    (0 keeps S_in, T is the state after every token)."""
    rng = _rng(21)
    B, T, H, dk, dv = 4, 3, 2, 6, 5
    q, k, v, a, b, _ = random_case(rng, B * T, H, dk, dv)
    q, k, v = (x.reshape(B, T, H, -1) for x in (q, k, v))
    a, b = (x.reshape(B, T, H) for x in (a, b))
    S_in = rng.standard_normal((B, H, dv, dk))
    accept = np.array([0, 3, 1, 2])
    o, S = orc.decode_tokens(q, k, v, a, b, S_in, accept)
    o_all, S_all = orc.decode_tokens(q, k, v, a, b, S_in)
    Sd = np.ascontiguousarray(S_in.copy())
    for t in range(T):
        ot = orc.decode_step(q[:, t], k[:, t], v[:, t], a[:, t], b[:, t], Sd)
        _close(o[:, t], ot, 1e-13, f"decode_tokens o token {t}")
        for n in range(B):
            if accept[n] == t + 1:
                _close(S[n], Sd[n], 1e-13, f"decode_tokens state seq {n}")
    assert np.array_equal(S[0], S_in[0])
    _close(S_all, Sd, 1e-13, "decode_tokens state, all accepted")
    _close(o_all, o, 0, "outputs do not depend on accept")


def pin_norm_gate_library(orc):
    """The output epilogue equals torch's RMS norm (a library routine, in
    float64) times torch's sigmoid / SiLU of the gate."""
    import torch
    rng = _rng(22)
    o = _f32(rng.standard_normal((7, 3, 16)) * 2.0)
    g = _f32(rng.standard_normal((7, 3, 16)))
    w = _f32(rng.uniform(0.5, 1.5, 16))
    ot, gt, wt = (torch.from_numpy(x.astype(np.float64)) for x in (o, g, w))
    for eps in (1e-5, 0.3):
        base = torch.nn.functional.rms_norm(ot, (16,), wt, eps)
        _close(orc.output_norm_gate(o, g, w, eps, "sigmoid"), (base * torch.sigmoid(gt)).numpy(),
               1e-13, f"norm gate sigmoid eps {eps}")
        _close(orc.output_norm_gate(o, g, w, eps, "silu"),
               (base * torch.nn.functional.silu(gt)).numpy(), 1e-13, f"norm gate silu eps {eps}")
        _close(orc.output_norm_gate(o, None, None, eps, "none"),
               torch.nn.functional.rms_norm(ot, (16,), None, eps).numpy(), 1e-13,
               f"norm, no gate, eps {eps}")


def pin_norm_gate_closed_forms(orc):
    """A constant row c gives c / sqrt(c^2 + eps) per channel; the gate at 0
    is 1/2 (sigmoid); scaling o by s and eps by s^2 changes nothing; the
    result's mean square is ms / (ms + eps) without weight and gate."""
    dv = 8
    for c, eps in ((3.0, 1e-5), (-0.5, 0.25), (2.0, 4.0)):
        o = np.full((1, dv), c, dtype=np.float32)
        y = orc.output_norm_gate(o, np.zeros((1, dv), np.float32), None, eps, "sigmoid")
        _close(y, np.full((1, dv), 0.5 * c / np.sqrt(c * c + eps)), 1e-14, f"constant row {c}")
    rng = _rng(23)
    o = _f32(rng.standard_normal((5, dv)))
    g = _f32(rng.standard_normal((5, dv)))
    w = _f32(rng.uniform(-1, 1, dv))
    s = 4.0   # a power of two keeps the scaled inputs exact
    _close(orc.output_norm_gate(s * o, g, w, 1e-3 * s * s, "sigmoid"),
           orc.output_norm_gate(o, g, w, 1e-3, "sigmoid"), 1e-13, "scale invariance")
    eps = 0.7
    y = orc.output_norm_gate(o, None, None, eps, "none")
    ms = np.mean(_d(o) ** 2, axis=1)
    _close(np.mean(y ** 2, axis=1), ms / (ms + eps), 1e-13, "mean square after the norm")


def _prologue_case(rng, T, H, d, K):
    x = [_f32(rng.standard_normal((T, H, d))) for _ in range(3)]
    w = _f32(rng.standard_normal((3, H, d, K)) * 0.5)
    beta = _f32(rng.standard_normal((T, H)))
    delta = _f32(rng.standard_normal((T, H)))
    g = _f32(-rng.exponential(2.0, (T, H)))
    return x, w, beta, delta, g


def pin_prologue_library(orc):
    """With no history the convolution is torch's depthwise conv1d with K-1
    zeros of left padding; q and k are then torch's L2 normalisation (eps 0),
    v the convolution itself when the write gate is 1 (delta = 0); SiLU is
    torch's."""
    import torch
    import torch.nn.functional as F
    T, H, d, K = 9, 2, 6, 4
    x, w, beta, _, g = _prologue_case(_rng(24), T, H, d, K)
    for act in ("none", "silu"):
        q, k, v, _, _, _ = orc.prologue(*x, w, beta, None, g, act=act, l2_eps=0.0)
        for i, got in enumerate((q, k, v)):
            xt = torch.from_numpy(x[i].astype(np.float64)).reshape(T, H * d).T[None]   # [1, C, T]
            wt = torch.from_numpy(w[i].astype(np.float64)).reshape(H * d, 1, K)
            y = F.conv1d(F.pad(xt, (K - 1, 0)), wt, groups=H * d)[0].T.reshape(T, H, d)
            if act == "silu":
                y = F.silu(y)
            if i < 2:
                y = F.normalize(y, dim=-1)
            _close(got, y.numpy(), 1e-13, f"prologue tensor {i} act {act}")


def pin_prologue_gates(orc):
    """b = expit(beta_raw) (scipy); a = exp(max(g_log, floor)); with a
    one-tap unit convolution and no activation v is scaled by the write gate,
    which at beta_raw = 0 is 2 sigmoid(delta)."""
    from scipy.special import expit
    T, H, d = 6, 3, 4
    rng = _rng(25)
    x = [_f32(rng.standard_normal((T, H, d))) for _ in range(3)]
    w = np.ones((3, H, d, 1), np.float32)
    beta = _f32(rng.standard_normal((T, H)))
    beta[0] = 0.0
    delta = _f32(rng.standard_normal((T, H)))
    g = _f32(np.array([-10.0, -5.0, -1.0, -0.25, 0.0, -7.5])[:, None].repeat(H, 1))
    q, k, v, a, b, _ = orc.prologue(*x, w, beta, delta, g, act="none", floor=-5.0)
    _close(b, expit(_d(beta)), 1e-15, "b = sigmoid(beta_raw)")
    _close(a, np.exp(np.maximum(_d(g), -5.0)), 1e-15, "floored decay")
    _close(v[0], _d(x[2][0]) * 2.0 * expit(_d(delta[0]))[:, None], 1e-14, "write gate at beta 0")
    _close(v, _d(x[2]) * (expit(_d(beta) + _d(delta)) / expit(_d(beta)))[:, :, None], 1e-14,
           "write gate")
    _close(q, _d(x[0]) / np.sqrt(np.sum(_d(x[0]) ** 2, axis=-1, keepdims=True) + 1e-6), 1e-14,
           "q norm")
    _, _, v0, _, _, _ = orc.prologue(*x, w, beta, None, g, act="none")
    _close(v0, _d(x[2]), 0, "no delta: v unchanged")


def pin_prologue_history(orc):
    """A sequence run in two calls, the history of the first passed to the
    second, equals one call; the history out holds the last K-1 raw tokens
    (from the history in where the sequence is shorter); a packed batch equals
    separate calls."""
    T, H, d, K = 11, 2, 5, 4
    rng = _rng(26)
    x, w, beta, delta, g = _prologue_case(rng, T, H, d, K)
    h0 = _f32(rng.standard_normal((1, 3, K - 1, H, d)))
    full = orc.prologue(*x, w, beta, delta, g, hist_in=h0)
    for cut in (1, 2, 7):
        p1 = orc.prologue(*(y[:cut] for y in x), w, beta[:cut], delta[:cut], g[:cut], hist_in=h0)
        p2 = orc.prologue(*(y[cut:] for y in x), w, beta[cut:], delta[cut:], g[cut:],
                          hist_in=_f32(p1[5]))
        for i in range(5):
            _close(np.concatenate([p1[i], p2[i]]), full[i], 1e-14, f"split at {cut}, output {i}")
        _close(p2[5], full[5], 0, f"split at {cut}, history")
    for i in range(3):
        _close(full[5][0, i], _d(x[i][T - (K - 1):]), 0, f"history of tensor {i}")
    lens = [4, 1, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hs = _f32(rng.standard_normal((len(lens), 3, K - 1, H, d)))
    packed = orc.prologue(*(y[:cu[-1]] for y in x), w, beta[:cu[-1]], delta[:cu[-1]],
                          g[:cu[-1]], hist_in=hs, cu_seqlens=cu)
    for n, L in enumerate(lens):
        t0, t1 = cu[n], cu[n + 1]
        one = orc.prologue(*(y[t0:t1] for y in x), w, beta[t0:t1], delta[t0:t1], g[t0:t1],
                           hist_in=hs[n:n + 1])
        for i in range(5):
            _close(packed[i][t0:t1], one[i], 0, f"packed seq {n} output {i}")
        _close(packed[5][n], one[5][0], 0, f"packed seq {n} history")
    _close(packed[5][2], hs[2], 0, "empty sequence keeps its history")
    _close(packed[5][1, :, :K - 2], hs[1, :, 1:], 0, "one-token sequence shifts its history")


def _diag_case(rng, T, H, dk, dv):
    q, k, v, a, b, S0 = random_case(rng, T, H, dk, dv)
    alpha = _f32(rng.uniform(0.2, 1.0, (T, H, dk)))
    return q, k, v, alpha, b, S0


def pin_diag_scalar_special_case(orc):
    """A decay equal on every key channel is the scalar rule (the scalar
    oracle is pinned on its own)."""
    rng = _rng(27)
    q, k, v, a, b, S0 = random_case(rng, 13, 3, 6, 5)
    alpha = _f32(np.repeat(a[:, :, None], 6, axis=2))
    o1, s1 = orc.prefill_diag(q, k, v, alpha, b, S0=S0)
    o2, s2 = orc.prefill(q, k, v, a, b, S0=S0)
    _close(o1, o2, 1e-13, "diag = scalar, o")
    _close(s1, s2, 1e-13, "diag = scalar, S")


def pin_diag_product_form(orc):
    """Brute force with matrices: S_t = S_{t-1} diag(alpha_t) (I - b k k^T)
    + b v k^T, o_t = S_t q_t, per head (T = 4, two heads)."""
    rng = _rng(28)
    T, H, dk, dv = 4, 2, 5, 3
    q, k, v, alpha, b, S0 = _diag_case(rng, T, H, dk, dv)
    o, S = orc.prefill_diag(q, k, v, alpha, b, S0=S0)
    for h in range(H):
        St = _d(S0[0, h])
        for t in range(T):
            kt = _d(k[t, h])
            St = St @ np.diag(_d(alpha[t, h])) @ (np.eye(dk) - b[t, h] * np.outer(kt, kt)) \
                + b[t, h] * np.outer(_d(v[t, h]), kt)
            _close(o[t, h], St @ _d(q[t, h]), 1e-13, f"diag product form o t={t} h={h}")
        _close(S[0, h], St, 1e-13, f"diag product form S h={h}")


def pin_diag_channel_separation(orc):
    """Keys and queries on channels 0..2 only: the state's other columns
    just decay, S[:, j] = S0[:, j] prod_t alpha_tj, and never reach o."""
    rng = _rng(29)
    T, H, dk, dv = 9, 2, 7, 4
    q, k, v, alpha, b, S0 = _diag_case(rng, T, H, dk, dv)
    q[:, :, 3:] = 0.0
    k[:, :, 3:] = 0.0
    o, S = orc.prefill_diag(q, k, v, alpha, b, S0=S0)
    prod = np.prod(_d(alpha[:, :, 3:]), axis=0)            # [H, 4]
    _close(S[0, :, :, 3:], _d(S0[0, :, :, 3:]) * prod[:, None, :], 1e-14, "untouched columns")
    S0b = S0.copy()
    S0b[..., 3:] = 0.0
    o2, _ = orc.prefill_diag(q, k, v, alpha, b, S0=S0b)
    _close(o, o2, 1e-14, "untouched columns never reach o")


def pin_diag_decode_and_varlen(orc):
    """Decode steps equal the prefill; a packed batch equals separate calls."""
    rng = _rng(30)
    q, k, v, alpha, b, S0 = _diag_case(rng, 10, 3, 6, 5)
    o, s = orc.prefill_diag(q, k, v, alpha, b, S0=S0)
    S = np.ascontiguousarray(_d(S0))
    for t in range(10):
        ot = orc.decode_step_diag(q[t:t + 1], k[t:t + 1], v[t:t + 1], alpha[t:t + 1],
                                  b[t:t + 1], S)
        _close(ot[0], o[t], 1e-13, f"diag decode step {t}")
    _close(S, s, 1e-13, "diag decode final state")
    lens = [4, 0, 6]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S0s = rng.standard_normal((3, 3, 5, 6))
    o, s = orc.prefill_diag(q, k, v, alpha, b, cu_seqlens=cu, S0=S0s)
    for n, L in enumerate(lens):
        t0, t1 = cu[n], cu[n + 1]
        on, sn = orc.prefill_diag(q[t0:t1], k[t0:t1], v[t0:t1], alpha[t0:t1], b[t0:t1],
                                  S0=S0s[n:n + 1])
        _close(o[t0:t1], on, 1e-14, f"diag varlen seq {n}")
        _close(s[n], sn[0], 1e-14, f"diag varlen S seq {n}")


def pin_diag_decode_tokens(orc):
    """Several tokens per sequence with a per-channel decay equal that many
    per-channel decode steps, the committed state the one after the accepted
    tokens; a decay equal on every channel gives the scalar decode_tokens."""
    rng = _rng(31)
    B, T, H, dk, dv = 4, 3, 2, 6, 5
    q, k, v, alpha, b, _ = _diag_case(rng, B * T, H, dk, dv)
    q, k, v, alpha = (x.reshape(B, T, H, -1) for x in (q, k, v, alpha))
    b = b.reshape(B, T, H)
    S_in = rng.standard_normal((B, H, dv, dk))
    accept = np.array([2, 0, 3, 1])
    o, S = orc.decode_tokens_diag(q, k, v, alpha, b, S_in, accept)
    Sd = np.ascontiguousarray(S_in.copy())
    for t in range(T):
        ot = orc.decode_step_diag(q[:, t], k[:, t], v[:, t], alpha[:, t], b[:, t], Sd)
        _close(o[:, t], ot, 1e-13, f"decode_tokens_diag o token {t}")
        for n in range(B):
            if accept[n] == t + 1:
                _close(S[n], Sd[n], 1e-13, f"decode_tokens_diag state seq {n}")
    assert np.array_equal(S[1], S_in[1])
    a = alpha[..., 0].copy()
    flat = _f32(np.repeat(a[..., None], dk, axis=3))
    o1, S1 = orc.decode_tokens_diag(q, k, v, flat, b, S_in, accept)
    o2, S2 = orc.decode_tokens(q, k, v, a, b, S_in, accept)
    _close(o1, o2, 1e-13, "decode_tokens_diag, channel-constant decay: o")
    _close(S1, S2, 1e-13, "decode_tokens_diag, channel-constant decay: S")


ALL_PINS = [pin_bruteforce, pin_exact_dyadic, pin_hand_example, pin_identity_gates,
            pin_readback, pin_pure_decay, pin_single_step, pin_linearity, pin_rotation,
            pin_permutation, pin_norm_bound, pin_resume, pin_varlen,
            pin_decode_equals_prefill, pin_decode_tokens, pin_norm_gate_library,
            pin_norm_gate_closed_forms, pin_prologue_library, pin_prologue_gates,
            pin_prologue_history, pin_diag_scalar_special_case, pin_diag_product_form,
            pin_diag_channel_separation, pin_diag_decode_and_varlen, pin_diag_decode_tokens]
