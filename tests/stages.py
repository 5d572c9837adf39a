"""Stage-wise parity of the layer on the GPU against the oracle, fed the GPU's own intermediates.

Two steps of the layer quantise values that are themselves float32 results of the GPU
(h = silu(G) U from the gate/up GEMM, [dG dU] from the dgrad of the down GEMM).  Near an e4m3
rounding boundary a float32 result that differs from the exact value in its last bits lands on
the neighbouring code, and both codes are correct results of the layer.  So every stage is
checked on the inputs the GPU actually used (the reading of the pages' "same layer result"
for MXFP8 stages that quantise accumulated values):

* bit-exact: the quantised weights, the transposed requantised weights W1t / W2t, the
  token-axis operands of the weight gradients, and the quantised h and [dG dU] except where
  the oracle's value, computed from the GPU's own inputs, lies within the float32 slack of a
  rounding boundary (those may take either code; the count is logged and bounded);
* max |err| <= 1e-2 x RMS of the oracle tensor (no envelope): every float result (Y slots, y,
  dX rows, dx, dw, dL, dW_r, dW1, dW2), with the oracle's GEMMs run on the GPU's quantised
  operands.

The slack model: a float32 GEMM result may differ from the exact dot product of its (exact)
operands by EPS * sum_k |a_k b_k|, and the float32 element-wise epilogues by REL_F32 relative.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

import moe_inputs
import oracle
from oracle.layer import _qdq
from helpers import log, rms, to_np

TOL = 1e-2
EPS = 2.0 ** -15       # float32 accumulation of the matrix-core GEMMs (measured up to 2^-15.96 at K = 256)
REL_F32 = 2.0 ** -19   # float32 element-wise epilogue (exp, reciprocal, products)
MAX_AMBIGUOUS_MISMATCH = 1e-2  # bound on the fraction of quantised values that took the other code


@dataclass
class StageStats:
    worst: dict = field(default_factory=dict)      # name -> max |err| / RMS
    mismatch: dict = field(default_factory=dict)   # name -> (mismatching values, ambiguous values, total)

    def err(self, name, got, ref, tol=TOL):
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        r = rms(ref)
        e = float(np.max(np.abs(got - ref))) if got.size else 0.0
        rel = e / r if r > 0 else e
        self.worst[name] = max(self.worst.get(name, 0.0), rel)
        assert (e <= tol * r) if r > 0 else (e <= 1e-6), f"{name}: max|err| / rms = {rel:.3e} > {tol:g}"
        return rel

    def codes(self, name, got_dq, ref_dq, lo, hi):
        """Quantised values: equal to the oracle's except where the oracle's value is ambiguous
        (its admissible range under the slack model holds two codes); the other code must lie
        in that range."""
        diff = got_dq != ref_dq
        amb = lo != hi
        assert np.all(~diff | amb), f"{name}: a code differs where the oracle's code is unique"
        assert np.all((got_dq >= lo) & (got_dq <= hi)), f"{name}: a code outside the admissible range"
        a, b, c = self.mismatch.get(name, (0, 0, 0))
        self.mismatch[name] = (a + int(diff.sum()), b + int(amb.sum()), c + diff.size)

    def report(self, label):
        for n, v in self.worst.items():
            log(f"  {label} {n}: max|err|/rms {v:.2e}")
        for n, (a, b, c) in self.mismatch.items():
            log(f"  {label} {n}: {a} of {c} codes differ ({a / max(c, 1):.1e}); {b} ambiguous ({b / max(c, 1):.1e})")
            assert a <= MAX_AMBIGUOUS_MISMATCH * c, f"{name_frac(n)}"


def name_frac(n):
    return f"{n}: too many codes on the other side of a rounding boundary"


def word_major(st):
    """Scales [n/32, K] of a matrix quantised along its n axis, in the library's word-major
    layout [n/128, K, 4] (word q of row k holds blocks 4q .. 4q + 3)."""
    nb, K = st.shape
    return np.ascontiguousarray(st.reshape(nb // 4, 4, K).transpose(0, 2, 1))


def quantized_weights(w1, w2):
    """Oracle MXFP8 of one expert's float32 weights: (w1q, w1s) along d, (w2q, w2s) along I."""
    w1q, w1s = oracle.quantize(np.asarray(w1, np.float64), axis=1)
    w2q, w2s = oracle.quantize(np.asarray(w2, np.float64), axis=1)
    return w1q, w1s, w2q, w2s


class LayerView:
    """Host copies of what the GPU layer saved, and the oracle pieces for a subset of experts."""

    def __init__(self, cfg, inp, layer):
        self.cfg, self.inp, self.layer = cfg, inp, layer
        self.k, self.S, self.T, self.d, self.I = cfg.k, cfg.n_shared, cfg.T, cfg.d, cfg.inter
        self.R = cfg.T * cfg.k
        self.perm = to_np(layer.saved_tensor("perm"))
        self.pos = to_np(layer.saved_tensor("pos"))
        self.offs = to_np(layer.saved_tensor("offsets"))
        self.counts = to_np(layer.saved_tensor("counts"))
        self.tok_off = to_np(layer.saved_tensor("tok_off"))
        self.w = to_np(layer.saved_tensor("w")).astype(np.float64)      # GPU float32 combine weights
        self.idx = to_np(layer.saved_tensor("idx"))
        self.L = to_np(layer.saved_tensor("logits")).astype(np.float64)
        xq, xs = oracle.quantize(inp.x.astype(np.float64), axis=1)
        assert np.array_equal(to_np(layer.saved_tensor("xq")), xq) and np.array_equal(
            to_np(layer.saved_tensor("xs")), xs), "x quantisation"
        self.X = oracle.dequantize(xq, xs, axis=1)
        self.ld = int(layer.wlayout.tok_stride)
        if inp.dy_bits is not None:
            dyq, dys = oracle.quantize(inp.dy.astype(np.float64), axis=1)
            assert np.array_equal(to_np(layer.workspace_tensor("dyq")), dyq) and np.array_equal(
                to_np(layer.workspace_tensor("dys")), dys), "dy quantisation"
            self.DY = oracle.dequantize(dyq, dys, axis=1)

    def rows(self, e):
        """Permuted rows [lo, hi) of expert e, their tokens, slots (t * (k + S) + j) and weights."""
        cfg = self.cfg
        lo, hi = int(self.offs[e]), int(self.offs[e + 1])
        if e < cfg.E:
            sid = self.perm[lo:hi]
            toks = sid // self.k
            slots = toks * (self.k + self.S) + sid % self.k
            wrow = self.w.reshape(-1)[sid]
        else:
            toks = np.arange(hi - lo)
            slots = toks * (self.k + self.S) + self.k + (e - cfg.E)
            wrow = np.ones(hi - lo)
        return lo, hi, toks, slots, wrow


def check_expert_forward(v: LayerView, e, w1, w2, st: StageStats, sample=None):
    """Quantised weights, W1t / W2t, H codes and Y slot rows of expert e (forward stages).
    sample: optional sorted subset of the expert's rows (rows are independent in the forward)."""
    layer, I, d = v.layer, v.I, v.d
    w1q, w1s, w2q, w2s = quantized_weights(w1, w2)
    assert np.array_equal(to_np(layer.w1q[e]), w1q) and np.array_equal(to_np(layer.w1s[e]), w1s), "W1 quant"
    assert np.array_equal(to_np(layer.w2q[e]), w2q) and np.array_equal(to_np(layer.w2s[e]), w2s), "W2 quant"
    W1 = oracle.dequantize(w1q, w1s, axis=1)
    W2 = oracle.dequantize(w2q, w2s, axis=1)
    lo, hi, toks, slots, wrow = v.rows(e)
    if hi == lo:
        return W1, W2, None
    # transposed requantisation, done by the forward GEMMs: bit-exact
    if layer.layout.w1t != layer.layout.total:
        q1t, s1t = oracle.requantize(w1q, w1s, from_axis=1, to_axis=0)   # [2I, d] blocks along 2I
        q2t, s2t = oracle.requantize(w2q, w2s, from_axis=1, to_axis=0)   # [d, I] blocks along d
        assert np.array_equal(to_np(layer.saved_tensor("w1t")[e]), q1t.T), f"W1t codes of expert {e}"
        assert np.array_equal(to_np(layer.saved_tensor("w1ts")[e]), word_major(s1t)), f"W1t scales of expert {e}"
        assert np.array_equal(to_np(layer.saved_tensor("w2t")[e]), q2t.T), f"W2t codes of expert {e}"
        assert np.array_equal(to_np(layer.saved_tensor("w2ts")[e]), word_major(s2t)), f"W2t scales of expert {e}"
    r = np.arange(lo, hi) if sample is None else np.asarray(sample)
    rl = r - lo
    G = to_np(layer.saved_tensor("g")[r]).astype(np.float64)
    U = to_np(layer.saved_tensor("u")[r]).astype(np.float64)
    # G and U themselves: the GEMM of the quantised rows with the quantised weights
    A = v.X[toks[rl]]
    st.err("G", G, A @ W1[:I].T)
    st.err("U", U, A @ W1[I:].T)
    # H from the GPU's own G and U: bit-exact outside the float32 slack of the epilogue
    h = oracle.layer._f32(oracle.swiglu(G, U))
    nom, hlo, hhi = oracle.quantize_range(h, REL_F32 * np.abs(h), axis=1)
    Hg = oracle.dequantize(to_np(layer.saved_tensor("hq")[r]), to_np(layer.saved_tensor("hs")[r]), axis=1)
    st.codes("H", Hg, nom, hlo, hhi)
    # Y rows from the GPU's own H
    ys = to_np(layer.saved_tensor("yslot").view(-1, d)[slots[rl]])
    st.err("Y slots", ys, Hg @ W2.T)
    return W1, W2, Hg


def check_expert_backward(v: LayerView, e, W1, W2, st: StageStats):
    """[dG dU] codes, dX slot rows, token-axis operands, dW1 and dW2 of expert e, every stage on
    the GPU's own inputs.  Returns the oracle's dX rows (from the GPU's [dG dU])."""
    layer, I, d, ld = v.layer, v.I, v.d, v.ld
    lo, hi, toks, slots, wrow = v.rows(e)
    NX = v.cfg.E + v.cfg.n_shared
    if hi == lo:
        assert np.all(to_np(layer.dw1[e]) == 0) and np.all(to_np(layer.dw2[e]) == 0), f"dW of empty expert {e}"
        return None
    G = to_np(layer.saved_tensor("g")[lo:hi]).astype(np.float64)
    U = to_np(layer.saved_tensor("u")[lo:hi]).astype(np.float64)
    W2t = _qdq(W2, 0, True)[2]   # [d, I] requantised along d
    W1t = _qdq(W1, 0, True)[2]   # [2I, d] requantised along 2I
    DY = v.DY[toks]
    # dgrad of the down GEMM and the SwiGLU backward, from the GPU's G, U and combine weights
    dH = wrow[:, None] * (DY @ W2t)
    e_dH = EPS * np.abs(wrow)[:, None] * (np.abs(DY) @ np.abs(W2t))
    dG, dU = oracle.swiglu_backward(dH, G, U)
    s = 1.0 / (1.0 + np.exp(-G))
    e_gu = np.concatenate([np.abs(U * s * (1.0 + G * (1.0 - s))) * e_dH + REL_F32 * np.abs(dG),
                           np.abs(G * s) * e_dH + REL_F32 * np.abs(dU)], axis=1)
    dGU = oracle.layer._f32(np.concatenate([dG, dU], axis=1))
    nom, glo, ghi = oracle.quantize_range(dGU, e_gu, axis=1)
    dguq = to_np(layer.workspace_tensor("dguq")[lo:hi])
    dgus = to_np(layer.workspace_tensor("dgus")[lo:hi])
    DGU = oracle.dequantize(dguq, dgus, axis=1)
    st.codes("dGU", DGU, nom, glo, ghi)
    # dgrad of the gate/up GEMM from the GPU's [dG dU]: the dX slot rows
    dX = DGU @ W1t
    st.err("dX slots", to_np(layer.workspace_tensor("dxslot").view(-1, d)[slots]), dX)
    # token-axis operands of the weight gradients (bit-exact) and the weight gradients
    Hg = oracle.dequantize(to_np(layer.saved_tensor("hq")[lo:hi]), to_np(layer.saved_tensor("hs")[lo:hi]), axis=1)
    dYw = oracle.layer._f32(oracle.layer._f32(wrow)[:, None] * DY)
    o = int(v.tok_off[e])
    o2 = int(v.tok_off[e + 1])
    for name, a, src in (("xt", v.X[toks], "X"), ("ht", Hg, "H"), ("dyt", dYw, "w dY"), ("dgut", DGU, "dGU")):
        q, sc = oracle.token_quantize(a)
        npad = q.shape[0]
        gq = to_np(layer.workspace_tensor(name)[:, o:o2])
        gs = to_np(layer.workspace_tensor(name + "s")[:, o // 32:o2 // 32])
        assert np.array_equal(gq[:, :npad], q.T), f"token-axis codes of {src}, expert {e}"
        assert np.array_equal(gs[:, :npad // 32], sc.T), f"token-axis scales of {src}, expert {e}"
        assert not gq[:, npad:].any() and not gs[:, npad // 32:].any(), f"token-axis padding of {src}, expert {e}"
    st.err("dW2", to_np(layer.dw2[e]), oracle.token_requant(dYw).T @ oracle.token_requant(Hg))
    st.err("dW1", to_np(layer.dw1[e]), oracle.token_requant(DGU).T @ oracle.token_requant(v.X[toks]))
    return dX


def check_router_backward(v: LayerView, st: StageStats, tokens=None):
    """dw = <dy, Y slot> on the GPU's Y slots, dL from the GPU's logits and weights, dW_r."""
    layer, k = v.layer, v.k
    t = np.arange(v.T) if tokens is None else np.asarray(tokens)
    dy = v.inp.dy.astype(np.float64)[t]
    ys = to_np(layer.saved_tensor("yslot")[t]).astype(np.float64)[:, :k]
    dw = np.einsum("td,tjd->tj", dy, ys)
    st.err("dw", to_np(layer.workspace_tensor("dw")[t]), dw)
    score = v.cfg.score
    w = v.w[t]
    dL = oracle.router_backward(v.L[t], v.idx[t], w, dw, score)
    st.err("dL", to_np(layer.workspace_tensor("dl")[t]), dL)
    return dL


def full_layer_checks(cfg, inp, ws, layer, label):
    """Every stage of a small layer on every expert, then dx and dW_r whole."""
    st = StageStats()
    v = LayerView(cfg, inp, layer)
    NX = cfg.E + cfg.n_shared
    dXrows = np.zeros((cfg.T * (cfg.k + cfg.n_shared), cfg.d))
    Hrows = {}
    for e in range(NX):
        W1, W2, _ = check_expert_forward(v, e, *ws[e], st)
        dX = check_expert_backward(v, e, W1, W2, st)
        if dX is not None:
            lo, hi, toks, slots, wrow = v.rows(e)
            dXrows[slots] = dX
    # y from the GPU's own Y slots (fixed slot order) and weights
    ys = to_np(layer.saved_tensor("yslot")).astype(np.float64)
    y = np.einsum("tj,tjd->td", v.w, ys[:, :cfg.k]) + ys[:, cfg.k:].sum(axis=1)
    st.err("y", to_np(layer.y32), y)
    dL = check_router_backward(v, st)
    dLfull = np.zeros((cfg.T, cfg.E))
    np.put_along_axis(dLfull, v.idx.astype(np.int64), dL, axis=1)
    st.err("dW_router", to_np(layer.dw_r), dLfull.T @ inp.x.astype(np.float64))
    dx = dXrows.reshape(cfg.T, cfg.k + cfg.n_shared, cfg.d).sum(axis=1) + dLfull @ inp.w_r.astype(np.float64)
    st.err("dx", to_np(layer.dx32), dx)
    st.report(label)
    return st
