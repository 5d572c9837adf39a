"""Admissible envelope of the layer's results (test infrastructure).

Two steps of the layer quantise values that are themselves float32 GEMM results:
h = silu(G) U (before the down GEMM) and [dG dU] (before the gate/up dgrad).  Any
implementation accumulates those GEMMs in float32 with its own rounding; the
matrix core of the target GPU also drops low-order bits of small products inside
a 32-value block (measured: a product 2^-15 below the block's largest is lost).
Near an e4m3 rounding boundary such a difference moves the value to the
neighbouring code, and both codes are correct results of the layer.

This module computes, from the oracle's own values only, (a) the admissible
range of those quantised values when every accumulated element may differ from
its exact value by up to ``eps * sum_k |a_k b_k|``, and (b) a bound on how far
every downstream output may move inside that range (linear propagation with
absolute values).  A result is correct if each quantised stage output lies in
its range and each float output is within ``tol * RMS + bound`` of the oracle.
Where no value sits near a boundary the bound is zero and the comparison is the
plain tolerance.

``eps`` is a model of the accumulation error; tests check it against the
measured gate/up results (|G_gpu - G| <= eps * S elementwise) on every run.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .layer import BLOCK, _qdq, _sigmoid
from .mxfp8 import quantize_range

EPS_ACC = 2.0 ** -15  # the GPU tests' model: measured G / U errors reach 2^-15.96 * sum|a b| (K = 256)
F32_SLACK = 2.0 ** -18   # relative error of float32 elementwise epilogues (exp, products)


def _dev(nom, lo, hi):
    return np.maximum(hi - nom, nom - lo)


def _token_range(a: np.ndarray, err: np.ndarray):
    """quantize_range along the token axis of one expert's rows (32-row blocks, zero tail)."""
    n = a.shape[0]
    npad = -(-n // BLOCK) * BLOCK
    pa = np.zeros((npad,) + a.shape[1:])
    pe = np.zeros((npad,) + a.shape[1:])
    pa[:n] = a
    pe[:n] = err
    nom, lo, hi = quantize_range(pa, pe, axis=0)
    return nom[:n], _dev(nom, lo, hi)[:n]


@dataclass
class ForwardEnvelope:
    eps: float
    eG: dict      # e -> [n, I] bound on |G_computed - G|
    eU: dict
    H_lo: dict    # e -> [n, I] admissible dequantised H
    H_hi: dict
    dH: dict      # e -> [n, I] max deviation of dequantised H
    BY: np.ndarray  # [RS, d] bound on |Y_computed - Y| beyond the tolerance
    By: np.ndarray  # [T, d]


def expert_forward_envelope(fe, A, W1, W2, eps: float = EPS_ACC):
    """One expert's forward envelope: (bound on |dG|, on |dU|, admissible H lo, hi, max H deviation,
    bound on |dY| rows beyond the tolerance) for rows A (dequantised) and weights W1, W2."""
    I = W1.shape[0] // 2
    aX = np.abs(A)
    g_err = eps * (aX @ np.abs(W1[:I]).T)
    u_err = eps * (aX @ np.abs(W1[I:]).T)
    G, U = fe.G, fe.U
    s = _sigmoid(G)
    silu = G * s
    dsilu = s * (1.0 + G * (1.0 - s))
    # |silu(G+a)(U+b) - silu(G)U| <= (|silu'(G)| + |a|/2)|a| (|U| + |b|) + |silu(G)| |b|   (|silu''| <= 1/2)
    h_err = (np.abs(dsilu) + 0.5 * g_err) * g_err * (np.abs(U) + u_err) + np.abs(silu) * u_err
    h_err = h_err + np.abs(fe.h) * F32_SLACK
    nom, lo, hi = quantize_range(fe.h, h_err, axis=1)
    dev = _dev(nom, lo, hi)
    aW2 = np.abs(W2)
    by = dev @ aW2.T + eps * ((np.abs(fe.H) + dev) @ aW2.T)
    return g_err, u_err, lo, hi, dev, by


def forward_envelope(fw, experts, eps: float = EPS_ACC) -> ForwardEnvelope:
    eG, eU, Hlo, Hhi, dHs = {}, {}, {}, {}, {}
    T, k = fw.w.shape
    R = T * k
    BY = np.zeros_like(fw.Yrows)
    E = fw.L.shape[1]
    for e, fe in fw.experts.items():
        W1, W2 = experts(e)
        g_err, u_err, lo, hi, dev, by = expert_forward_envelope(fe, fw.X[fw.rows_of[e]], W1, W2, eps)
        eG[e], eU[e], Hlo[e], Hhi[e], dHs[e] = g_err, u_err, lo, hi, dev
        if e < E:
            lo_r, hi_r = fw.sched.offsets[e], fw.sched.offsets[e + 1]
        else:
            lo_r, hi_r = R + (e - E) * T, R + (e - E + 1) * T
        BY[lo_r:hi_r] = by
    By = np.zeros((T, BY.shape[1]))
    for j in range(k):
        By += fw.w[:, j:j + 1] * BY[fw.sched.pos[:, j]]
    for sh in range(fw.n_shared):
        By += BY[R + sh * T: R + (sh + 1) * T]
    return ForwardEnvelope(eps, eG, eU, Hlo, Hhi, dHs, BY, By)


@dataclass
class BackwardEnvelope:
    GU_lo: dict   # e -> [n, 2I] admissible dequantised [dG dU]
    GU_hi: dict
    Bdx: np.ndarray
    Bdw_r: np.ndarray
    BdW1: dict
    BdW2: dict


def expert_backward_envelope(fe, be, A, DYrows, wrow, W1, W2, eG, eU, devH, eps: float = EPS_ACC):
    """One expert's backward envelope: admissible [dG dU] lo, hi and bounds on |d dX| rows,
    |d dW1|, |d dW2| beyond the tolerance.  eG, eU, devH come from the forward envelope."""
    W2t = _qdq(W2, 0, True)[2]
    W1t = _qdq(W1, 0, True)[2]
    dH = be.dH
    edH = eps * np.abs(wrow)[:, None] * (np.abs(DYrows) @ np.abs(W2t)) + np.abs(dH) * F32_SLACK
    G, U = fe.G, fe.U
    s = _sigmoid(G)
    f = s * (1.0 + G * (1.0 - s))           # dG = dH U f(G);  |f'| <= 0.6
    silu = G * s
    adH = np.abs(dH) + edH
    e_dG = np.abs(U * f) * edH + adH * np.abs(f) * eU + adH * (np.abs(U) + eU) * 0.6 * eG
    e_dU = np.abs(silu) * edH + adH * (np.abs(f) + 0.5 * eG) * eG  # silu' = f
    eGU = np.concatenate([e_dG, e_dU], axis=1) + np.abs(be.dGU) * F32_SLACK
    nom, lo, hi = quantize_range(be.dGU, eGU, axis=1)
    devGU = _dev(nom, lo, hi)
    aW1t = np.abs(W1t)
    bdx = devGU @ aW1t + eps * ((np.abs(be.DGU) + devGU) @ aW1t)
    # weight gradients: token-axis requantisation of ranged operands
    w32 = wrow.astype(np.float32).astype(np.float64)
    dYw = (w32[:, None] * DYrows).astype(np.float32).astype(np.float64)
    dYw_tok, dev_dYw = _token_range(dYw, np.abs(dYw) * 2.0 ** -20)
    H_tok, dev_H = _token_range(fe.H, devH)
    GU_tok, dev_GUt = _token_range(be.DGU, devGU)
    X_tok, _ = _token_range(A, np.zeros_like(A))
    a_dYw, a_H, a_GU, a_X = np.abs(dYw_tok), np.abs(H_tok), np.abs(GU_tok), np.abs(X_tok)
    bdw2 = a_dYw.T @ dev_H + dev_dYw.T @ (a_H + dev_H) + eps * ((a_dYw + dev_dYw).T @ (a_H + dev_H))
    bdw1 = dev_GUt.T @ a_X + eps * ((a_GU + dev_GUt).T @ a_X)
    return lo, hi, bdx, bdw1, bdw2


def backward_envelope(fw, bw, fenv: ForwardEnvelope, dy, x, w_r, experts, score: str) -> BackwardEnvelope:
    eps = fenv.eps
    dy = np.asarray(dy, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    w_r = np.asarray(w_r, dtype=np.float64)
    T, d = dy.shape
    k = fw.idx.shape[1]
    E = w_r.shape[0]
    R = T * k
    DY = _qdq(dy, 1, True)[2]
    wflat = fw.w.reshape(-1)
    BdXrows = np.zeros_like(fw.Yrows)
    GUlo, GUhi, BdW1, BdW2 = {}, {}, {}, {}
    for e, be in bw.experts.items():
        fe = fw.experts[e]
        W1, W2 = experts(e)
        tokens = fw.rows_of[e]
        if e < E:
            lo_r, hi_r = fw.sched.offsets[e], fw.sched.offsets[e + 1]
            wrow = wflat[fw.sched.perm[lo_r:hi_r]]
        else:
            lo_r, hi_r = R + (e - E) * T, R + (e - E + 1) * T
            wrow = np.ones(hi_r - lo_r)
        lo, hi, bdx, bdw1, bdw2 = expert_backward_envelope(fe, be, fw.X[tokens], DY[tokens], wrow, W1, W2,
                                                            fenv.eG[e], fenv.eU[e], fenv.dH[e], eps)
        GUlo[e], GUhi[e], BdW1[e], BdW2[e] = lo, hi, bdw1, bdw2
        BdXrows[lo_r:hi_r] = bdx
    # router: dw = <dy, Y> moves with Y.  Y_r = H_r W2^T is linear in H_r, so
    # |d dw| <= sum_i dev(H_r)_i |(dy_t W2)_i| + eps sum_n |dy_t,n| ((|H_r| + dev) |W2|^T)_n
    Bdw_rows = np.zeros(fw.Yrows.shape[0])
    for e, fe in fw.experts.items():
        W2 = experts(e)[1]
        if e < E:
            lo_r, hi_r = fw.sched.offsets[e], fw.sched.offsets[e + 1]
        else:
            lo_r, hi_r = R + (e - E) * T, R + (e - E + 1) * T
        dyt = dy[fw.rows_of[e]]
        dev = fenv.dH[e]
        acc_err = eps * ((np.abs(fe.H) + dev) @ np.abs(W2).T)
        Bdw_rows[lo_r:hi_r] = np.sum(dev * np.abs(dyt @ W2), axis=1) + np.sum(np.abs(dyt) * acc_err, axis=1)
    Bdw = np.zeros((T, k))
    for j in range(k):
        Bdw[:, j] = Bdw_rows[fw.sched.pos[:, j]]
    inner = np.sum(fw.w * Bdw, axis=1, keepdims=True)
    if score == "softmax":
        c = fw.w
    else:
        Ls = np.take_along_axis(fw.L, fw.idx.astype(np.int64), axis=1)
        sg = _sigmoid(Ls)
        c = sg * (1.0 - sg) / sg.sum(axis=1, keepdims=True)
    BdL = c * (Bdw + inner)
    BdLfull = np.zeros((T, E))
    np.put_along_axis(BdLfull, fw.idx.astype(np.int64), BdL, axis=1)
    Bdx = BdLfull @ np.abs(w_r)
    for j in range(k):
        Bdx += BdXrows[fw.sched.pos[:, j]]
    for sh in range(fw.n_shared):
        Bdx += BdXrows[R + sh * T: R + (sh + 1) * T]
    Bdw_r = BdLfull.T @ np.abs(x)
    return BackwardEnvelope(GUlo, GUhi, Bdx, Bdw_r, BdW1, BdW2)
