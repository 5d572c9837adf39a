"""Device buffers of one MoE layer around the C ABI (torch provides memory and streams only)."""
from __future__ import annotations

import numpy as np
import torch

from . import (MOE_F_DW_BF16, MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX, make_config, moe_bwd, moe_fwd, moe_query,
               moe_quantize_mxfp8)


def _bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class MoeLayer:
    """Caller-side buffers (weights, saved state, workspace, outputs) of one layer shape."""

    def __init__(self, T, d, E, k, inter, score="softmax", n_shared=0, ring_rows=0, chunk_rows=0,
                 producer_wgs=0, flags=0, device="cuda", with_backward=True):
        self.T, self.d, self.E, self.k, self.I, self.S = T, d, E, k, inter, n_shared
        self.NX = E + n_shared
        self.device = torch.device(device)
        score_fn = MOE_SCORE_SOFTMAX if score == "softmax" else MOE_SCORE_SIGMOID
        self.cfg = make_config(T, d, E, k, inter, n_shared, score_fn, ring_rows, chunk_rows, producer_wgs, flags)
        ws, self.layout, self.wlayout = moe_query(self.cfg, with_workspace_layout=True)
        dev = self.device
        self.saved = torch.empty(self.layout.total, dtype=torch.uint8, device=dev)
        self.workspace = torch.zeros(max(ws, 256), dtype=torch.uint8, device=dev)
        NX, I = self.NX, inter
        self.w1q = torch.empty((NX, 2 * I, d), dtype=torch.uint8, device=dev)
        self.w1s = torch.empty((NX, 2 * I, d // 32), dtype=torch.uint8, device=dev)
        self.w2q = torch.empty((NX, d, I), dtype=torch.uint8, device=dev)
        self.w2s = torch.empty((NX, d, I // 32), dtype=torch.uint8, device=dev)
        self.y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
        self.y32 = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.bias = None
        if with_backward:
            self.dx = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
            self.dx32 = torch.empty((T, d), dtype=torch.float32, device=dev)
            self.dw_r = torch.empty((E, d), dtype=torch.float32, device=dev)
            dwt = torch.bfloat16 if flags & MOE_F_DW_BF16 else torch.float32
            self.dw1 = torch.empty((NX, 2 * I, d), dtype=dwt, device=dev)
            self.dw2 = torch.empty((NX, d, I), dtype=dwt, device=dev)

    @classmethod
    def from_config(cls, cfg, **kw):
        """From a moe_inputs.LayerConfig."""
        return cls(cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.score, cfg.n_shared,
                   with_backward=kw.pop("with_backward", cfg.backward), **kw)

    # ------------------------------------------------------------------ inputs

    def set_inputs(self, x_bits, w_r_bits, bias=None, dy_bits=None):
        self.x = _bf16_tensor(x_bits, self.device)
        self.w_r = _bf16_tensor(w_r_bits, self.device)
        self.bias = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(self.device)
        if dy_bits is not None:
            self.dy = _bf16_tensor(dy_bits, self.device)

    def load_expert(self, e, w1: np.ndarray, w2: np.ndarray, stream=None):
        """Quantise one expert's float32 weights on the device (w1 along d, w2 along I)."""
        t1 = torch.from_numpy(np.ascontiguousarray(w1, np.float32)).to(self.device)
        t2 = torch.from_numpy(np.ascontiguousarray(w2, np.float32)).to(self.device)
        moe_quantize_mxfp8(t1, 1, 2 * self.I, self.d, self.w1q[e], self.w1s[e], stream)
        moe_quantize_mxfp8(t2, 1, self.d, self.I, self.w2q[e], self.w2s[e], stream)
        return t1, t2  # keep alive until the stream has consumed them

    def load_experts(self, it):
        keep = []
        for e, w1, w2 in it:
            keep.append(self.load_expert(e, w1, w2))
            if len(keep) > 4:
                torch.cuda.current_stream().synchronize()
                keep.clear()
        torch.cuda.current_stream().synchronize()

    # ------------------------------------------------------------------ passes

    def forward(self, stream=None, f32=True):
        moe_fwd(self.cfg, self.x, self.w_r, self.bias, self.w1q, self.w1s, self.w2q, self.w2s, self.y,
                self.y32 if f32 else None, self.saved, self.workspace, stream)
        return self.y

    def backward(self, stream=None, f32=True):
        moe_bwd(self.cfg, self.dy, self.x, self.w_r, self.saved, self.dx, self.dx32 if f32 else None, self.dw_r,
                self.dw1, self.dw2, self.workspace, stream)
        return self.dx

    # ------------------------------------------------------------------ saved state

    def saved_tensor(self, name: str) -> torch.Tensor:
        """A typed view of one field of the saved buffer (see moe_saved_layout)."""
        T, d, E, k, I, S, NX = self.T, self.d, self.E, self.k, self.I, self.S, self.NX
        R, RS = T * k, T * k + S * T
        spec = {
            "logits": (torch.float32, (T, E)), "idx": (torch.int32, (T, k)), "w": (torch.float32, (T, k)),
            "counts": (torch.int32, (NX,)), "offsets": (torch.int32, (NX + 1,)),
            "poffsets": (torch.int32, (NX + 1,)), "tok_off": (torch.int64, (NX + 1,)),
            "tile_start": (torch.int32, (NX + 1,)), "tile64": (torch.int32, (NX + 1,)),
            "perm": (torch.int32, (R,)), "pos": (torch.int32, (T, k)),
            "xq": (torch.uint8, (T, d)), "xs": (torch.uint8, (T, d // 32)),
            "g": (torch.float32, (RS, I)), "u": (torch.float32, (RS, I)),
            "hq": (torch.uint8, (RS, I)), "hs": (torch.uint8, (RS, I // 32)),
            "yslot": (torch.float32, (T, k + S, d)),
            "w1t": (torch.uint8, (NX, d, 2 * I)), "w1ts": (torch.uint8, (NX, 2 * I // 128, d, 4)),
            "w2t": (torch.uint8, (NX, I, d)), "w2ts": (torch.uint8, (NX, d // 128, I, 4)),
        }
        dt, shape = spec[name]
        off = getattr(self.layout, name)
        n = int(np.prod(shape)) * torch.tensor([], dtype=dt).element_size()
        return self.saved[off:off + n].view(dt).view(shape)

    def workspace_tensor(self, name: str) -> torch.Tensor:
        """A typed view of one field of the workspace (see moe_workspace_layout)."""
        T, d, k, I, S = self.T, self.d, self.k, self.I, self.S
        RS = T * k + S * T
        ld = int(self.wlayout.tok_stride)
        spec = {
            "status": (torch.int32, (1,)),
            "dyq": (torch.uint8, (T, d)), "dys": (torch.uint8, (T, d // 32)),
            "dw": (torch.float32, (T, k)), "dl": (torch.float32, (T, k)),
            "dguq": (torch.uint8, (RS, 2 * I)), "dgus": (torch.uint8, (RS, 2 * I // 32)),
            "dxslot": (torch.float32, (T, k + S, d)),
            "xt": (torch.uint8, (d, ld)), "xts": (torch.uint8, (d, ld // 32)),
            "ht": (torch.uint8, (I, ld)), "hts": (torch.uint8, (I, ld // 32)),
            "dyt": (torch.uint8, (d, ld)), "dyts": (torch.uint8, (d, ld // 32)),
            "dgut": (torch.uint8, (2 * I, ld)), "dguts": (torch.uint8, (2 * I, ld // 32)),
            "xp": (torch.uint8, (RS, d)), "xps": (torch.uint8, (RS, d // 32)), "yrows": (torch.float32, (RS, d)),
        }
        dt, shape = spec[name]
        off = getattr(self.wlayout, name)
        n = int(np.prod(shape)) * torch.tensor([], dtype=dt).element_size()
        return self.workspace[off:off + n].view(dt).view(shape)
