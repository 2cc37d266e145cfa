"""Chunked (WY / UT-transform) form of the gated delta rule, in NumPy.

Test-side design model, independent of both the oracle and the HIP code: it
restates the chunk algebra the kernels use so that (a) in float64 it can be
checked against the oracle to ~1e-13, proving the algebra, and (b) with
bfloat16 rounding inserted at the kernels' cast points it predicts the error
budget of a precision plan.

Within a chunk of C tokens entering with state S (rows = value channels):

    g_i   = sum_{s<=i} log a_s,   gamma_i = exp(g_i),   gamma_C = gamma_{C-1}
    L_ij  = b_i (gamma_i / gamma_j) k_i . k_j          (j < i, else 0)
    T     = (I + L)^-1                                  (unit lower triangular)
    W     = T diag(b gamma) K,      U' = T diag(b) V
    U     = U' - W S^T                                  (the written errors b_i e_i)
    A_ij  = (gamma_i / gamma_j) q_i . k_j              (j <= i, else 0)
    O     = diag(gamma) Q S^T + A U = O' + Q' S^T,
            O' = A U',  Q' = diag(gamma) Q - A W
    S_out = gamma_C S + U^T diag(gamma_C / gamma) K

Pad rows of a partial last chunk use log a = 0, b = 0, q = k = v = 0, which
leaves every quantity above unchanged for the valid rows.
"""
from __future__ import annotations

import numpy as np


def _bf16(x):
    """Round float64/float32 values to bfloat16 (RNE) via float32."""
    x32 = np.asarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    r = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _split(x):
    hi = _bf16(x)
    lo = _bf16(_f32(x) - hi)
    return hi, lo


def _mm(A, B, mode):
    """Product as the MFMA plan computes it (fp32 accumulate emulated by fp64
    then rounding the result to fp32 for the non-exact modes).

    mode: 'f64' exact; 'x1' both operands bf16; 'xa' split A (B exact bf16);
    'xb' split B (A exact); 'x2a' split A, B one bf16; 'x2b' A one bf16,
    split B; 'x3' hi*hi + hi*lo + lo*hi; 'f32' both fp32."""
    if mode == "f64":
        return A @ B
    if mode == "f32":
        return _f32(_f32(A) @ _f32(B))
    if mode == "x1":
        return _f32(_bf16(A) @ _bf16(B))
    if mode == "xa":
        h, l = _split(A)
        return _f32(h @ B + l @ B)
    if mode == "xb":
        h, l = _split(B)
        return _f32(A @ h + A @ l)
    if mode == "x2a":   # split A, B rounded to one bf16
        h, l = _split(A)
        Bb = _bf16(B)
        return _f32(h @ Bb + l @ Bb)
    if mode == "x2b":   # A rounded to one bf16, split B
        h, l = _split(B)
        Ab = _bf16(A)
        return _f32(Ab @ h + Ab @ l)
    if mode == "x3":
        ah, al = _split(A)
        bh, bl = _split(B)
        return _f32(ah @ bh + ah @ bl + al @ bh)
    raise ValueError(mode)


EXACT = dict(gram="f64", solve="f64", wu="f64", qo="f64", walk_x="f64", walk_s="f64",
             state="f64")
# Plan used by the HIP kernels: exact-bf16 inputs need no split; every
# computed fp32 operand is fed to MFMA as a bf16 hi + lo pair.
KERNEL_PLAN = dict(gram="x1", solve="f32", wu="xa", qo="x3", walk_x="x3", walk_s="xa",
                   state="f32", form="B", walk_y="xb")
# The same algebra with W, Q', U', O' formed per chunk (the WY form written out).
WY_PLAN = dict(gram="x1", solve="f32", wu="xa", qo="x3", walk_x="x3", walk_s="xa",
               state="f32")


def chunk_prefill(q, k, v, a, b, cu_seqlens=None, S0=None, C=64, plan=None):
    """Chunked prefill with the same contract as the oracle's prefill.

    q, k [T,H,dk], v [T,H,dv], a, b [T,H]; returns (o, S_final) in float64.
    """
    plan = EXACT if plan is None else plan
    q, k, v, a, b = (np.asarray(x, dtype=np.float64) for x in (q, k, v, a, b))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens)
    N = len(cu) - 1
    o = np.zeros((T, H, dv))
    S_final = np.zeros((N, H, dv, dk))
    rnd_state = (lambda x: _f32(x)) if plan["state"] == "f32" else (lambda x: x)
    for n in range(N):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n, h], dtype=np.float64)
            for c0 in range(t0, t1, C):
                L_ = min(C, t1 - c0)
                Kc = np.zeros((C, dk)); Qc = np.zeros((C, dk)); Vc = np.zeros((C, dv))
                la = np.zeros(C); bc = np.zeros(C)
                Kc[:L_] = k[c0:c0 + L_, h]; Qc[:L_] = q[c0:c0 + L_, h]
                Vc[:L_] = v[c0:c0 + L_, h]
                la[:L_] = np.log(a[c0:c0 + L_, h]); bc[:L_] = b[c0:c0 + L_, h]
                g = np.cumsum(la)
                if plan["solve"] == "f32":
                    g = _f32(g)
                gam = np.exp(g)
                diff = g[:, None] - g[None, :]
                Gam = np.where(np.tril(np.ones((C, C))) > 0,
                               np.exp(np.minimum(diff, 0.0)), 0.0)
                KK = _mm(Kc, Kc.T, plan["gram"])
                QK = _mm(Qc, Kc.T, plan["gram"])
                Lm = np.tril(bc[:, None] * KK * Gam, -1)
                Am = QK * Gam
                if plan["solve"] == "f32":
                    Lm, Am = _f32(Lm), _f32(Am)
                Tm = np.linalg.inv(np.eye(C) + Lm)
                if plan["solve"] == "f32":
                    Tm = _f32(Tm)
                W = _mm(Tm * (bc * gam)[None, :], Kc, plan["wu"])
                Up = _mm(Tm * bc[None, :], Vc, plan["wu"])
                Qp = _f32(gam[:, None] * Qc - _mm(Am, W, plan["qo"])) \
                    if plan["qo"] != "f64" else gam[:, None] * Qc - Am @ W
                Op = _mm(Am, Up, plan["qo"])
                if plan.get("form") == "B":
                    # walk on the raw inputs and the small factors T_b, A:
                    # X_W = T_b (Gamma (K S^T)), U' = T_b V, O = Gamma (Q S^T) + A U
                    Tb = Tm * bc[None, :]
                    Y = gam[:, None] * _mm(Kc, S.T, plan["walk_y"])
                    X_w = _mm(Tb, Y, plan["walk_x"])
                    Up = _mm(Tb, Vc, plan["wu"])
                    U = Up - X_w
                    Oc = gam[:, None] * _mm(Qc, S.T, plan["walk_y"]) + _mm(Am, U, plan["qo"])
                    o[c0:c0 + L_, h] = Oc[:L_]
                    scale = gam[-1] / gam
                    S = rnd_state(gam[-1] * S + _mm((U * scale[:, None]).T, Kc, plan["walk_s"]))
                    continue
                X_w = _mm(W, S.T, plan.get("walk_w", plan["walk_x"]))
                X_q = _mm(Qp, S.T, plan.get("walk_q", plan["walk_x"]))
                U = Up - X_w
                Oc = Op + X_q
                o[c0:c0 + L_, h] = Oc[:L_]
                scale = gam[-1] / gam
                S = rnd_state(gam[-1] * S + _mm((U * scale[:, None]).T, Kc, plan["walk_s"]))
            S_final[n, h] = S
    return o, S_final


def rel_l2(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))
