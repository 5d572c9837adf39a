"""Python binding of the MI355X MoE-layer library (libmoe_mi355x.so, C ABI in include/moe.h).

The entry points keep the C names and only marshal arguments: tensors become device pointers,
the stream defaults to torch's current stream.  Every step of the layer runs in the library's
HIP kernels; PyTorch only provides device memory and streams.  If the library is missing the
import of any entry point raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EALIGN, MOE_EWORKSPACE, MOE_ELAUNCH, MOE_EDEVICE = range(7)
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_F_DIRECT_GATHER = 1
MOE_F_RING_DISPATCH = 2
MOE_F_SERIAL_BWD = 4
MOE_F_IDENTITY_EXPERTS = 8
MOE_F_FORWARD_ONLY = 16
MOE_F_UNFUSED = 32
MOE_F_DW_BF16 = 64
MOE_DEV_RING_TIMEOUT, MOE_DEV_NONFINITE_LOGIT = 1, 2

# every symbol include/moe.h declares
EXPORTS = ("moe_query", "moe_quantize_mxfp8", "moe_requant_transpose", "moe_fwd", "moe_fwd_noalloc", "moe_bwd",
           "moe_set_phase_events", "moe_device_status", "moe_strerror", "moe_probe_mfma")
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20

# phases of moe_fwd / moe_bwd (include/moe.h, MOE_PH_*)
PHASES = ("fwd_begin", "quant_x", "router", "topk", "schedule", "gateup", "down", "combine",
          "bwd_begin", "quant_dy", "router_bwd", "router_wgrad", "requant_w", "dgrad_down", "dgrad_gateup",
          "dx_reduce", "token_requant", "wgrad_down", "wgrad_gateup")


class moe_config(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("score_fn", ctypes.c_int32),
                ("ring_rows", ctypes.c_int32), ("chunk_rows", ctypes.c_int32), ("producer_wgs", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class moe_saved_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "logits", "idx", "w", "counts", "offsets", "poffsets", "tok_off", "tile_start", "tile64", "perm", "pos",
        "xq", "xs", "g", "u", "hq", "hs", "yslot", "w1t", "w1ts", "w2t", "w2ts", "total")]


class moe_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "status", "ring", "ring_s", "ring_flags", "blkcnt", "dyq", "dys", "dw", "dl", "dguq", "dgus", "dxslot",
        "xt", "xts", "ht", "hts", "dyt", "dyts", "dgut", "dguts", "xp", "xps", "yrows", "tok_stride",
        "total")]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {moe_strerror(status)} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              f"`python -m mixture_experts_layer_schedule_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.moe_query.argtypes = [ctypes.POINTER(moe_config), ctypes.POINTER(SZ), ctypes.POINTER(moe_saved_layout),
                                ctypes.POINTER(moe_workspace_layout)]
        L.moe_quantize_mxfp8.argtypes = [P, ctypes.c_int, I64, I64, P, P, P]
        L.moe_requant_transpose.argtypes = [P, P, I64, I64, I64, P, P, P]
        L.moe_fwd.argtypes = [ctypes.POINTER(moe_config), P, P, P, P, P, P, P, P, P, P, SZ, P, SZ, P]
        L.moe_fwd_noalloc.argtypes = [ctypes.POINTER(moe_config), P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_bwd.argtypes = [ctypes.POINTER(moe_config), P, P, P, P, SZ, P, P, P, P, P, P, SZ, P]
        L.moe_set_phase_events.argtypes = [P, I32]
        L.moe_probe_mfma.argtypes = [P, ctypes.c_size_t, I32, ctypes.POINTER(ctypes.c_double),
                                     ctypes.POINTER(ctypes.c_size_t), P]
        L.moe_device_status.argtypes = [P, ctypes.POINTER(I32)]
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_strerror.restype = ctypes.c_char_p
        for n in EXPORTS:
            if n != "moe_strerror":
                getattr(L, n).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    """Device pointer of a tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> int | None:
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(status: int, where: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, where)


def make_config(T, d, E, k, inter, n_shared=0, score_fn=MOE_SCORE_SOFTMAX, ring_rows=0, chunk_rows=0,
                producer_wgs=0, flags=0) -> moe_config:
    return moe_config(T, d, E, k, inter, n_shared, score_fn, ring_rows, chunk_rows, producer_wgs, flags)


def moe_strerror(status: int) -> str:
    return lib().moe_strerror(int(status)).decode()


def moe_query(cfg: moe_config, with_workspace_layout: bool = False):
    """(workspace bytes, saved layout) or, with_workspace_layout, (bytes, saved layout, workspace layout)."""
    ws = ctypes.c_size_t(0)
    sl = moe_saved_layout()
    wl = moe_workspace_layout()
    _check(lib().moe_query(ctypes.byref(cfg), ctypes.byref(ws), ctypes.byref(sl), ctypes.byref(wl)), "moe_query")
    return (ws.value, sl, wl) if with_workspace_layout else (ws.value, sl)


def moe_quantize_mxfp8(src, src_is_f32: int, rows: int, cols: int, q, scales, stream=None) -> None:
    _check(lib().moe_quantize_mxfp8(_ptr(src), int(src_is_f32), rows, cols, _ptr(q), _ptr(scales), _stream(stream)),
           "moe_quantize_mxfp8")


def moe_requant_transpose(q, scales, batch: int, rows: int, cols: int, qt, st, stream=None) -> None:
    _check(lib().moe_requant_transpose(_ptr(q), _ptr(scales), batch, rows, cols, _ptr(qt), _ptr(st),
                                       _stream(stream)), "moe_requant_transpose")


def _nbytes(t, n) -> int:
    """Byte size of a buffer: n if given, else the tensor's size."""
    if n is not None:
        return int(n)
    return t.numel() * t.element_size()


def moe_fwd(cfg, x, w_router, router_bias, w1q, w1s, w2q, w2s, y_bf16, y_f32, saved, workspace,
            stream=None, saved_bytes=None, workspace_bytes=None) -> None:
    _check(lib().moe_fwd(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w1q), _ptr(w1s),
                         _ptr(w2q), _ptr(w2s), _ptr(y_bf16), _ptr(y_f32), _ptr(saved), _nbytes(saved, saved_bytes),
                         _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)), "moe_fwd")


def moe_fwd_noalloc(cfg, x, w_router, router_bias, w1q, w1s, w2q, w2s, y_bf16, y_f32, saved, stream=None,
                    saved_bytes=None) -> None:
    _check(lib().moe_fwd_noalloc(ctypes.byref(cfg), _ptr(x), _ptr(w_router), _ptr(router_bias), _ptr(w1q),
                                 _ptr(w1s), _ptr(w2q), _ptr(w2s), _ptr(y_bf16), _ptr(y_f32), _ptr(saved),
                                 _nbytes(saved, saved_bytes), _stream(stream)), "moe_fwd_noalloc")


def moe_bwd(cfg, dy, x, w_router, saved, dx_bf16, dx_f32, dw_router, dw1, dw2, workspace, stream=None,
            saved_bytes=None, workspace_bytes=None) -> None:
    _check(lib().moe_bwd(ctypes.byref(cfg), _ptr(dy), _ptr(x), _ptr(w_router), _ptr(saved),
                         _nbytes(saved, saved_bytes), _ptr(dx_bf16), _ptr(dx_f32), _ptr(dw_router), _ptr(dw1),
                         _ptr(dw2), _ptr(workspace), _nbytes(workspace, workspace_bytes), _stream(stream)), "moe_bwd")


def moe_probe_mfma(sink, iters: int, stream=None, sink_bytes=None) -> float:
    """Enqueue the matrix-core issue-rate probe; returns the launch's flop count (the caller times
    it).  sink=None asks for the sink size instead: returns -(bytes needed)."""
    flop = ctypes.c_double(0.0)
    need = ctypes.c_size_t(0)
    st = lib().moe_probe_mfma(_ptr(sink), 0 if sink is None else _nbytes(sink, sink_bytes), int(iters),
                              ctypes.byref(flop), ctypes.byref(need), _stream(stream))
    if sink is None and st == MOE_EWORKSPACE:
        return -float(need.value)
    _check(st, "moe_probe_mfma")
    return flop.value


def moe_set_phase_events(events, n_events: int) -> None:
    """events: address of a host array of hipEvent_t (or None with n_events = 0)."""
    _check(lib().moe_set_phase_events(events, int(n_events)), "moe_set_phase_events")


def moe_device_status(workspace) -> int:
    code = ctypes.c_int32(0)
    st = lib().moe_device_status(_ptr(workspace), ctypes.byref(code))
    if st not in (MOE_OK, MOE_EDEVICE):
        _check(st, "moe_device_status")
    return code.value


from .layer import MoeLayer  # noqa: E402,F401
