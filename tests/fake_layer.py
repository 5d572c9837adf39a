"""A CPU stand-in for the GPU layer's buffers, filled from the oracle (test infrastructure).

It exposes what the stage checker reads from a MoeLayer (saved / workspace views, outputs,
quantised weights) with the oracle's own intermediates stored in the precisions the library
stores them in.  The CPU tests use it to show that the stage checker accepts a correct layer and
rejects planted mistakes, without a GPU.
"""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch

import moe_inputs
import oracle
from oracle.layer import _qdq
from stages import word_major


def _t(a, dtype=None):
    a = np.ascontiguousarray(a)
    if dtype is not None:
        a = a.astype(dtype)
    return torch.from_numpy(a)


class FakeLayer:
    def __init__(self, cfg, inp, ws):
        T, d, E, k, I, S = cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.n_shared
        NX, R = E + S, T * k
        RS = R + S * T
        ex = oracle.oracle_experts([w[0] for w in ws], [w[1] for w in ws])
        fw = oracle.layer_forward(inp.x, inp.w_r, ex, k, cfg.score, inp.bias, S)
        bw = oracle.layer_backward(fw, inp.dy, inp.x, inp.w_r, ex, cfg.score)
        self.fw, self.bw = fw, bw
        sched = fw.sched
        counts = np.concatenate([sched.counts, np.full(S, T)]).astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        c128 = -(-counts.astype(np.int64) // 128) * 128
        tok_off = np.concatenate([[0], np.cumsum(c128)]).astype(np.int64)
        ld = int(-(-(RS + 127 * NX) // 128) * 128)
        f32 = np.float32
        q = [oracle.quantize(np.asarray(w1, np.float64), axis=1) + oracle.quantize(np.asarray(w2, np.float64), axis=1)
             for w1, w2 in ws]
        self.w1q = _t(np.stack([a[0] for a in q]))
        self.w1s = _t(np.stack([a[1] for a in q]))
        self.w2q = _t(np.stack([a[2] for a in q]))
        self.w2s = _t(np.stack([a[3] for a in q]))
        w1t = np.zeros((NX, d, 2 * I), np.uint8)
        w1ts = np.zeros((NX, 2 * I // 128, d, 4), np.uint8)
        w2t = np.zeros((NX, I, d), np.uint8)
        w2ts = np.zeros((NX, d // 128, I, 4), np.uint8)
        g = np.zeros((RS, I), f32)
        u = np.zeros((RS, I), f32)
        hq = np.zeros((RS, I), np.uint8)
        hs = np.zeros((RS, I // 32), np.uint8)
        dguq = np.zeros((RS, 2 * I), np.uint8)
        dgus = np.zeros((RS, 2 * I // 32), np.uint8)
        ops = {n: (np.zeros((c, ld), np.uint8), np.zeros((c, ld // 32), np.uint8))
               for n, c in (("xt", d), ("ht", I), ("dyt", d), ("dgut", 2 * I))}
        dw1 = np.zeros((NX, 2 * I, d), f32)
        dw2 = np.zeros((NX, d, I), f32)
        wflat = fw.w.reshape(-1)
        dyq, dys = oracle.quantize(inp.dy.astype(np.float64), axis=1)
        DY = oracle.dequantize(dyq, dys, axis=1)
        w32 = fw.w.astype(f32).astype(np.float64).reshape(-1)
        for e in range(NX):
            lo, hi = offs[e], offs[e + 1]
            if hi == lo:
                continue
            a = q[e]
            q1t, s1t = oracle.requantize(a[0], a[1], from_axis=1, to_axis=0)
            q2t, s2t = oracle.requantize(a[2], a[3], from_axis=1, to_axis=0)
            w1t[e], w1ts[e], w2t[e], w2ts[e] = q1t.T, word_major(s1t), q2t.T, word_major(s2t)
            fe, be = fw.experts[e], bw.experts[e]
            g[lo:hi], u[lo:hi] = fe.G, fe.U
            hq[lo:hi], hs[lo:hi] = fe.Hq, fe.Hs
            dguq[lo:hi], dgus[lo:hi] = be.dGUq, be.dGUs
            toks = fw.rows_of[e]
            wr = w32[sched.perm[lo:hi]] if e < E else np.ones(hi - lo)
            dYw = (wr[:, None] * DY[toks]).astype(f32).astype(np.float64)
            o = tok_off[e]
            for n, src in (("xt", fw.X[toks]), ("ht", fe.H), ("dyt", dYw), ("dgut", be.DGU)):
                qq, ss = oracle.token_quantize(src)
                ops[n][0][:, o:o + qq.shape[0]] = qq.T
                ops[n][1][:, o // 32:o // 32 + ss.shape[0]] = ss.T
            dw1[e], dw2[e] = bw.dW1[e], bw.dW2[e]
        slots = np.zeros((T, k + S), np.int64)
        slots[:, :k] = sched.pos
        for sh in range(S):
            slots[:, k + sh] = R + sh * T + np.arange(T)
        self._saved = {
            "logits": _t(fw.L, f32), "idx": _t(fw.idx, np.int32), "w": _t(fw.w, f32),
            "counts": _t(counts), "offsets": _t(offs), "tok_off": _t(tok_off),
            "perm": _t(sched.perm, np.int32), "pos": _t(sched.pos, np.int32),
            "xq": _t(fw.xq), "xs": _t(fw.xs), "g": _t(g), "u": _t(u), "hq": _t(hq), "hs": _t(hs),
            "yslot": _t(fw.Yrows[slots], f32),
            "w1t": _t(w1t), "w1ts": _t(w1ts), "w2t": _t(w2t), "w2ts": _t(w2ts),
        }
        self._work = {
            "dyq": _t(dyq), "dys": _t(dys), "dw": _t(bw.dw, f32), "dl": _t(bw.dL, f32),
            "dguq": _t(dguq), "dgus": _t(dgus), "dxslot": _t(bw.dXrows[slots], f32),
        }
        for n, (qq, ss) in ops.items():
            self._work[n], self._work[n + "s"] = _t(qq), _t(ss)
        self.y32 = _t(fw.y, f32)
        self.dx32 = _t(bw.dx, f32)
        self.dw_r = _t(bw.dw_r, f32)
        self.dw1 = _t(dw1)
        self.dw2 = _t(dw2)
        self.layout = SimpleNamespace(w1t=0, total=1)
        self.wlayout = SimpleNamespace(tok_stride=ld)

    def saved_tensor(self, name):
        return self._saved[name]

    def workspace_tensor(self, name):
        return self._work[name]
