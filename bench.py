#!/usr/bin/env python3
"""Throughput of one DeepSeek-V3-shape MoE layer, forward + backward, on one MI355X.

Workload: T=8192 tokens, d=7168, 256 routed experts, top-8 sigmoid-normalised routing,
SwiGLU inter 2048, MXFP8 (e4m3 + e8m0 1x32 scales) with float32 accumulation, seed 4;
synthetic inputs (moe_inputs).  A step is moe_fwd + moe_bwd over one batch with every input
already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --config dsv3_fwd --forward-only      (a forward workload, moe_fwd alone)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MXFP8_PEAK = 5.0e15       # dense MXFP8 MFMA, FLOP/s (MI355X published)
HBM_PEAK = 8.0e12         # HBM3E, B/s (MI355X published)
METRIC = "MoE layer fwd+bwd TFLOPS & tokens/s at DSV3 shape; % of MXFP8 MFMA peak"
METRIC_FWD = "MoE layer forward TFLOPS & tokens/s; % of MXFP8 MFMA peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- algorithmic work
#
# Bytes and flops each phase must move / compute: weights once per GEMM pass, activations once in
# and once out per stage, dW once, the dense E-times work not counted.  R = T*k routed rows,
# NX experts; weights are MXFP8 (1 byte + 1/32 scale byte per value); activations as stored.

def phase_work(cfg, tok_pad: int, backward: bool = True, dw_bytes: int = 4) -> dict:
    """With ``backward`` the forward GEMMs also write the weights requantised along the other axis
    (W1^T, W2^T: the dgrad GEMMs' operands), once per weight byte.  dw_bytes: bytes per weight
    gradient element (4, or 2 with MOE_F_DW_BF16)."""
    T, d, E, k, I, S = cfg.T, cfg.d, cfg.E, cfg.k, cfg.inter, cfg.n_shared
    NX, R = E + S, T * cfg.k + S * T
    q = 1 + 1 / 32  # MXFP8 bytes per value
    w1 = NX * 2 * I * d * q
    w2 = NX * d * I * q
    wt = 1.0 if backward else 0.0
    return {
        "quant_x": (0.0, T * d * 2 + T * d * q),
        "router": (2.0 * T * d * E, T * d * 2 + E * d * 2 + T * E * 4),
        "gateup": (2.0 * R * d * 2 * I, w1 * (1 + wt) + R * d * q + R * I * (4 + 4 + q)),
        "down": (2.0 * R * I * d, w2 * (1 + wt) + R * I * q + R * d * 4),
        "combine": (0.0, R * d * 4 + T * d * (2 + 4)),
        "quant_dy": (0.0, T * d * 2 + T * d * q),
        "router_bwd": (2.0 * T * k * d, T * k * d * 4 + T * d * 2),
        "requant_w": (0.0, 0.0),  # done inside the forward GEMMs (counted there)
        "dgrad_down": (2.0 * R * d * I, w2 + R * d * q + R * I * 8 + R * 2 * I * q),
        "dgrad_gateup": (2.0 * R * 2 * I * d, w1 + R * 2 * I * q + R * d * 4),
        "dx_reduce": (0.0, R * d * 4 + T * d * 6),
        "token_requant": (0.0, (R * (2 * d + 3 * I) * q) + tok_pad * (2 * d + 3 * I) * q),
        "wgrad_down": (2.0 * R * d * I, NX * d * I * dw_bytes + tok_pad * (d + I) * q),
        "wgrad_gateup": (2.0 * R * 2 * I * d, NX * 2 * I * d * dw_bytes + tok_pad * (2 * I + d) * q),
    }


# ----------------------------------------------------------------------------- HIP events

class PhaseEvents:
    """hipEvent_t array handed to the library for per-phase timing on the launch stream."""

    def __init__(self, n):
        import torch  # noqa: F401  (loads libamdhip64)
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.n = n
        self.arr = (ctypes.c_void_p * n)()
        for i in range(n):
            if self.hip.hipEventCreate(ctypes.byref(self.arr, i * ctypes.sizeof(ctypes.c_void_p))) != 0:
                raise RuntimeError("hipEventCreate failed")
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float(0)
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.arr[a], self.arr[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


# ----------------------------------------------------------------------------- HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dsv3_fwd_bwd_hbm_traffic.txt")
PHASE_DISPATCHES = {  # phase -> kernel dispatches of one step (name#index in launch order)
    "gateup": ["k_gemm_gateup#0"], "down": ["k_gemm_down#0"], "combine": ["k_combine#0"],
    "router_bwd": ["k_router_bwd#0"],
    "dgrad_down": ["k_gemm_dgrad_down#0"], "dgrad_gateup": ["k_gemm_dgrad_gateup#0"],
    "dx_reduce": ["k_dx_reduce#0"], "wgrad_down": ["k_gemm_wgrad<8, 0>#0"],
    "wgrad_gateup": ["k_gemm_wgrad<8, 1>#0"],
}


def kernel_sources_hash() -> str:
    """sha256 (first 16 hex digits) over the HIP sources, to tell whether counters are current."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "mixture_experts_layer_schedule_amd", "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(phase: str, ring: bool):
    """HBM bytes (read + written) of one launch of the phase's kernels, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when it is missing or the kernels changed
    since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read().splitlines()
    except OSError:
        return None
    current = kernel_sources_hash()
    if not any(line.startswith("# kernel sources sha256[:16]:") and line.split(":")[-1].strip() == current
               for line in text):
        return None
    table = {}
    for line in text:
        parts = line.split()
        if len(parts) >= 4 and not line.startswith("#"):  # name (may hold spaces), n, fetch GB, write GB
            table[" ".join(parts[:-3])] = float(parts[-2]) + float(parts[-1])
    keys = PHASE_DISPATCHES.get(phase)
    if keys and ring and phase == "gateup":
        keys = ["k_ring_gateup#0"]
    if not keys or any(k not in table for k in keys):
        return None
    return round(sum(table[k] for k in keys) * 1e9)


# ----------------------------------------------------------------------------- measured peaks

def measured_peaks(moe, torch, stream) -> dict:
    """What this device reaches, next to the published peaks: the scaled MXFP8 matrix-core issue
    rate (the library's register-only probe), an HBM copy (read + write) and an HBM fill (write
    only) of 2 GiB, each the best of three timed runs."""
    def best(fn, n=3):
        t = []
        for _ in range(n + 1):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            t.append(a.elapsed_time(b) * 1e-3)
        return min(t[1:])  # the first is a warmup
    need = int(-moe.moe_probe_mfma(None, 1))
    sink = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    flop = [0.0]

    def mfma():
        flop[0] = moe.moe_probe_mfma(sink, 4000, stream)
    t_mfma = best(mfma)
    n = 1 << 31
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    t_copy = best(lambda: dst.copy_(src))
    t_fill = best(lambda: dst.fill_(0))
    del src, dst, sink
    return {"mfma_mxfp8_tflops": round(flop[0] / t_mfma / 1e12, 1), "hbm_copy_gbps": round(2 * n / t_copy / 1e9, 1),
            "hbm_write_gbps": round(n / t_fill / 1e9, 1),
            "how": "register-only v_mfma_scale_f32_32x32x64_f8f6f4 loop (moe_probe_mfma); 2 GiB device copy "
                   "(read + write bytes); 2 GiB fill; best of 3"}


# ----------------------------------------------------------------------------- CPU baseline

def host_resources() -> dict:
    """Cores this process may run on, the BLAS pool's thread count and the host's RAM."""
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    except Exception:  # pragma: no cover
        blas = 1
    try:
        ram_gb = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES") / 2 ** 30
    except (ValueError, OSError):  # pragma: no cover
        ram_gb = float("nan")
    return {"affinity_cores": affinity, "blas_threads": blas, "ram_gib": round(ram_gb, 1)}


def cpu_baseline(cfg, inp, n_experts: int, backward: bool = True) -> dict:
    """The float64 oracle timed on a bounded sample: full router/top-k/schedule/combine work on all
    tokens, the expert forward (+ backward with the transposed weight requantisation) on
    ``n_experts`` experts, scaled to the whole layer."""
    import numpy as np

    import moe_inputs
    import oracle
    from oracle.layer import _qdq

    res = host_resources()
    # the oracle's float64 matrix products run on the BLAS pool, everything else on one thread
    cores = max(1, min(res["affinity_cores"], res["blas_threads"]))
    x = inp.x.astype(np.float64)
    t0 = time.perf_counter()
    L = oracle.router_logits(x, inp.w_r, inp.bias)
    idx = oracle.select_topk(L, cfg.k)
    w = oracle.routing_weights(L, idx, cfg.score)
    sched = oracle.build_schedule(idx, cfg.E)
    xq, xs = oracle.quantize(x, axis=1)
    X = oracle.dequantize(xq, xs, axis=1)
    if backward:
        dyq, dys = oracle.quantize(inp.dy.astype(np.float64), axis=1)
        DY = oracle.dequantize(dyq, dys, axis=1)
    t_dense = time.perf_counter() - t0
    # expert sample: experts at evenly spaced quantiles of the load (low to high)
    order = np.argsort(sched.counts, kind="stable")
    n_experts = max(1, min(n_experts, len(order)))
    sample = [int(order[(2 * i + 1) * len(order) // (2 * n_experts)]) for i in range(n_experts)]
    t_exp = 0.0
    rows = 0
    for e in sample:
        w1, w2 = moe_inputs.expert_weights(cfg, e)
        W1 = _qdq(w1, 1, True)[2]
        W2 = _qdq(w2, 1, True)[2]       # input preparation (the layer receives quantised weights)
        toks = sched.perm[sched.offsets[e]:sched.offsets[e + 1]] // cfg.k
        wrow = w.reshape(-1)[sched.perm[sched.offsets[e]:sched.offsets[e + 1]]]
        t1 = time.perf_counter()
        fw = oracle.expert_forward(X[toks], W1, W2)
        if backward:
            W2t = _qdq(W2, 0, True)[2]
            W1t = _qdq(W1, 0, True)[2]
            oracle.expert_backward(fw, X[toks], DY[toks], wrow, W1t, W2t)
        t_exp += time.perf_counter() - t1
        rows += len(toks)
    # combine-side work on the sample's rows, scaled like the experts
    t_total = t_dense + t_exp * (cfg.T * cfg.k) / max(rows, 1)
    what = "forward/backward incl. weight requantisation" if backward else "forward"
    return {
        "value": cfg.T / t_total, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
        "sample": (f"float64 NumPy oracle: router, top-k, schedule and activation quantisation on all {cfg.T} "
                   f"tokens ({t_dense:.1f} s) + expert {what} on {len(sample)} "
                   f"experts at evenly spaced load quantiles ({rows} rows, {t_exp:.1f} s), scaled by routed rows "
                   f"{cfg.T * cfg.k}/{rows}; estimated layer time {t_total:.1f} s"),
        **res,
    }


# ----------------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="dsv3_fwd_bwd")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's token count T (a T sweep; the default workload is unchanged)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-experts", type=int, default=8)
    ap.add_argument("--dominant", default="auto", help="phase reported in roofline (default: longest)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (scales HBM byte counters)")
    ap.add_argument("--flags", type=int, default=0, help="moe_config.flags (2 = ring dispatch)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time moe_fwd alone (MOE_F_FORWARD_ONLY: no state saved for a backward pass)")
    ap.add_argument("--unfused", action="store_true",
                    help="the unfused forward baseline (MOE_F_UNFUSED; implies --forward-only)")
    ap.add_argument("--chunk-rows", type=int, default=0,
                    help="rows per GEMM row tile (moe_config.chunk_rows); 0: tuned per workload")
    ap.add_argument("--ring-rows", type=int, default=0,
                    help="ring capacity in rows with --flags 2 (ring dispatch); 0: the workload's own, else 16384")
    ap.add_argument("--producers", type=int, default=0, help="ring producer workgroups (0: 128)")
    ap.add_argument("--dw-bf16", action="store_true",
                    help="weight gradients in bf16 (MOE_F_DW_BF16); the default writes them in float32")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of one step captured into a HIP graph (phases from eager steps)")
    ap.add_argument("--no-tune", action="store_true",
                    help="skip the per-workload tuning (chunk_rows 256, backward branch on a second stream)")
    args = ap.parse_args()
    if args.unfused:
        args.forward_only = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one MI355X: the layer runs with every expert resident on a single GPU; "
              "it has no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import moe_inputs
    import mixture_experts_layer_schedule_amd as moe
    from mixture_experts_layer_schedule_amd import MoeLayer

    fwd_only = args.forward_only
    cfg = moe_inputs.CONFIGS[args.config].with_(backward=not fwd_only)
    if args.tokens:
        cfg = cfg.with_(T=args.tokens, name=f"{cfg.name}_T{args.tokens}")
    flags = (args.flags | (moe.MOE_F_FORWARD_ONLY if fwd_only else 0) | (moe.MOE_F_UNFUSED if args.unfused else 0)
             | (moe.MOE_F_DW_BF16 if args.dw_bf16 else 0))
    t0 = time.time()
    inp = moe_inputs.layer_inputs(cfg, with_dy=not fwd_only)
    ring_kw = {}
    if flags & moe.MOE_F_RING_DISPATCH:
        ring_kw = dict(ring_rows=args.ring_rows or cfg.ring_rows, producer_wgs=args.producers)
    layer = MoeLayer.from_config(cfg, with_backward=not fwd_only, flags=flags, **ring_kw)
    layer.set_inputs(inp.x_bits, inp.w_r_bits, inp.bias, None if fwd_only else inp.dy_bits)
    log(f"[bench] inputs on device; drawing and quantising {cfg.E + cfg.n_shared} experts")
    layer.load_experts(moe_inputs.iter_expert_weights(cfg, threads=min(16, os.cpu_count() or 8)))
    log(f"[bench] setup {time.time() - t0:.1f} s")

    stream = torch.cuda.current_stream()
    # per-workload tuning before anything is timed: every candidate gives the same bits
    tuning = None
    if args.chunk_rows:
        layer.cfg.chunk_rows = args.chunk_rows
    elif not args.no_tune:
        from mixture_experts_layer_schedule_amd import tune as tuner
        t_tune = time.time()
        cands = None
        if ring_kw and args.producers:   # a producer count given on the command line stays
            ring = int(layer.cfg.ring_rows) or 16384
            cands = list(dict.fromkeys(
                tuner.Knobs(kn.chunk_rows, kn.serial_bwd, args.producers, kn.ring_rows)
                for kn in tuner.candidates(layer.T, layer.E, layer.k, layer.S, not fwd_only, ring)))
        res = tuner.tune(layer, backward=not fwd_only, steps=3, warmup=1, stream=stream, cands=cands)
        tuning = {"chosen": res.best.label(), "ms_per_step": res.table(),
                  "how": "each candidate timed for 3 steps after 1 warm-up step on the same inputs; "
                         "the default (first) stays unless beaten by more than 1 %"}
        log(f"[bench] tuned in {time.time() - t_tune:.1f} s: {res.best.label()} "
            f"({', '.join(f'{k} {v:.2f}' for k, v in list(res.table().items())[:4])} ms)")
    knobs = {"chunk_rows": int(layer.cfg.chunk_rows) or 256,
             "serial_bwd": bool(layer.cfg.flags & moe.MOE_F_SERIAL_BWD)}
    if ring_kw:
        knobs["producer_wgs"] = int(layer.cfg.producer_wgs) or 128
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration copy: 1 GiB read + 1 GiB written")
    ev = PhaseEvents(len(moe.PHASES))
    moe.moe_set_phase_events(ctypes.addressof(ev.arr), ev.n)

    def step(st=stream):
        layer.forward(st)
        if not fwd_only:
            layer.backward(st)

    for i in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done")

    graph = None
    if args.graph:
        # one step captured into a HIP graph (no phase marks inside it), after a warm-up step on
        # a side stream as capture expects
        moe.moe_set_phase_events(None, 0)
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        moe.moe_set_phase_events(ctypes.addressof(ev.arr), ev.n)
        log("[bench] one step captured into a graph")

    def timed(n, replay=False):
        """n steps (or n replays of the captured step) bracketed by events; returns (ms per step,
        per-phase ms from the library's marks; zeros for replays)."""
        pms = {p: 0.0 for p in moe.PHASES}
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        total = 0.0
        for i in range(n):
            start.record(stream)
            if replay:
                graph.replay()
            else:
                step()
            stop.record(stream)
            stop.synchronize()
            total += start.elapsed_time(stop)
            if replay:
                continue
            prev = None
            for p, name in enumerate(moe.PHASES):
                if name == "bwd_begin" and fwd_only:
                    break
                if name in ("fwd_begin", "bwd_begin"):
                    prev = p
                    continue
                pms[name] += ev.elapsed(prev, p)
                prev = p
        return total / n, {k: v / n for k, v in pms.items()}

    # the timed region: the library's default schedule (backward branch on a second stream)
    if graph is not None:
        ms, _ = timed(args.steps, replay=True)
        log(f"[bench] {args.steps} graph replays, {ms:.3f} ms/step")
        _, phase_ms_timed = timed(min(args.steps, 3))  # the same schedule eagerly: its phase marks
    else:
        ms, phase_ms_timed = timed(args.steps)
        log(f"[bench] {args.steps} steps, {ms:.3f} ms/step")
    if fwd_only or knobs["serial_bwd"]:  # one stream: the phase marks come from the timed region
        ms_serial, phase_ms = ms, phase_ms_timed
    else:
        # per-phase breakdown: the same step with every kernel in launch order on one stream
        layer.cfg.flags |= moe.MOE_F_SERIAL_BWD
        n_serial = min(args.steps, 3)
        ms_serial, phase_ms = timed(n_serial)
        layer.cfg.flags &= ~moe.MOE_F_SERIAL_BWD
        log(f"[bench] {n_serial} steps in launch order (phase breakdown), {ms_serial:.3f} ms/step")
    torch.cuda.synchronize()
    moe.moe_set_phase_events(None, 0)
    code = moe.moe_device_status(layer.workspace)
    if code != 0:
        log(f"[bench] device status {code}")
        return 1

    tok_off = layer.saved_tensor("tok_off").cpu().numpy()
    work = phase_work(cfg, int(tok_off[-1]), backward=not fwd_only, dw_bytes=2 if flags & moe.MOE_F_DW_BF16 else 4)
    # the grouped GEMMs' work items: row tiles (up to 256 rows of one expert) x column tiles
    counts = layer.saved_tensor("counts").cpu().numpy()
    row_tiles = int(layer.saved_tensor("tile_start").cpu().numpy()[-1])
    col_tiles = {"gateup": cfg.inter // 128, "down": -(-cfg.d // 256), "dgrad_down": -(-cfg.inter // 256),
                 "dgrad_gateup": -(-cfg.d // 256)}
    sched = {"rows_per_expert_mean": round(float(counts.mean()), 1), "rows_per_expert_max": int(counts.max()),
             "empty_experts": int((counts == 0).sum()), "row_tiles": row_tiles,
             "tiles": {g: row_tiles * n for g, n in col_tiles.items()}}
    gemms = ("gateup", "down") if fwd_only else ("gateup", "down", "dgrad_down", "dgrad_gateup", "wgrad_down",
                                                 "wgrad_gateup")
    flops_fwd = sum(work[p][0] for p in ("gateup", "down"))
    flops_gemm = sum(work[p][0] for p in gemms)
    gemm_ms = sum(phase_ms[p] for p in gemms)
    tflops = flops_gemm / (ms * 1e-3) / 1e12
    phases = {}
    for p, t in phase_ms.items():
        if p in work and t > 0:
            f, b = work[p]
            phases[p] = {"ms": round(t, 4), "tflops": round(f / (t * 1e-3) / 1e12, 2),
                         "gbps": round(b / (t * 1e-3) / 1e9, 1),
                         "mfma_frac": round(f / (t * 1e-3) / MXFP8_PEAK, 4),
                         "roofline_frac": round(max(f / MXFP8_PEAK, b / HBM_PEAK) / (t * 1e-3), 4)}
    dom = max((p for p in phases), key=lambda p: phases[p]["ms"]) if args.dominant == "auto" else args.dominant
    f, b = work[dom]
    # phases whose interval in the timed region covers that phase alone (the others overlap the
    # backward's second-stream branch there): take those from the timed region itself
    clean = dom in ("quant_x", "router", "topk", "schedule", "gateup", "down", "combine", "quant_dy",
                    "wgrad_gateup")
    t = (phase_ms_timed[dom] if clean else phase_ms[dom]) * 1e-3
    if f / MXFP8_PEAK >= b / HBM_PEAK:
        roof = {"bound": "mfma", "achieved": round(f / t / 1e12, 2), "peak": MXFP8_PEAK / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(b / t / 1e9, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    # the committed counters were taken on the default workload only
    default_run = args.config == "dsv3_fwd_bwd" and not args.tokens and not fwd_only and not args.dw_bf16
    roof["traffic"] = measured_traffic(dom, ring=bool(args.flags & 2)) if default_run else None
    roof["kernel"] = dom
    roof["timed_in"] = "timed region" if clean else "launch-order pass"

    peaks = measured_peaks(moe, torch, stream)
    log(f"[bench] measured peaks {peaks}")
    roof["measured_peak"] = (peaks["mfma_mxfp8_tflops"] if roof["bound"] == "mfma" else
                             peaks["hbm_copy_gbps"])
    roof["frac_of_measured"] = round(roof["achieved"] / roof["measured_peak"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] CPU baseline: oracle on a sample of {args.cpu_experts} experts")
        cpu = cpu_baseline(cfg, inp, args.cpu_experts, backward=not fwd_only)

    out = {
        "metric": METRIC_FWD if fwd_only else METRIC,
        "value": round(cfg.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8",
        "data": "synthetic",
        "config": {"workload": (f"{cfg.name}: MoE layer {'fwd' if fwd_only else 'fwd+bwd'}, T={cfg.T} d={cfg.d} "
                                f"E={cfg.E}{f'+{cfg.n_shared} shared' if cfg.n_shared else ''} k={cfg.k} "
                                f"I={cfg.inter} {cfg.score}, seed {cfg.seed}"),
                   "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k, "inter": cfg.inter, "score": cfg.score,
                   "n_shared": cfg.n_shared, "seed": cfg.seed, "parallelism": "single GPU",
                   "path": "unfused" if args.unfused else ("ring" if ring_kw else "fused"), **knobs,
                   **({"graph": True} if graph is not None else {}),
                   **({"dw": "bf16"} if args.dw_bf16 else {}),
                   **({"ring_rows": int(layer.cfg.ring_rows) or 16384} if ring_kw else {})},
        "tuning": tuning,
        "tflops": round(tflops, 2),
        "mfma_frac_layer": round(flops_gemm / (ms * 1e-3) / MXFP8_PEAK, 4),
        "mfma_frac_gemms": round(flops_gemm / (gemm_ms * 1e-3) / MXFP8_PEAK, 4),
        "fwd_tflop": round(flops_fwd / 1e12, 3),
        "ms_per_step_launch_order": round(ms_serial, 4),
        "phases": phases,
        "schedule": sched,
        "roofline": roof,
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
