"""Per-workload tuning of the layer's knobs.

The pages tune their megakernel per workload (minibatch, buffer capacity and the number of SMs
given to data movement: article "Cursor 為 Composer 改造 MoE 訓練：MoK 點樣拆走跨 GPU 樽頸",
section "2.37 倍同 1.41 倍係兩份成績").  On one MI355X with direct gather the knobs that act are:

* ``chunk_rows`` -- rows per GEMM row tile (32 .. 256).  Shorter tiles give the grouped GEMMs
  more work items when experts receive few rows, and stream every weight slice once more per
  extra tile;
* the backward schedule -- the token-axis requantisation of X, H, w*dY and the dW2 GEMM on a
  second stream beside the dgrad chain (the default), or every kernel in launch order
  (``MOE_F_SERIAL_BWD``);
* with the ring dispatch (``MOE_F_RING_DISPATCH``), ``producer_wgs`` -- the workgroups that
  gather rows into the ring while the GEMM computes (the pages' SMs given to data movement) --
  and ``ring_rows``, the ring's capacity (the pages' buffer capacity).  The configured capacity
  is the caller's memory budget: the tuner tries it and a half and a quarter of it, never more
  (a smaller ring fits the workspace sized for the budget), and only row-tile heights that
  divide the capacity tried.

Every candidate produces the same bits (the library guarantees it), so the tuner only times
them on the caller's own layer and inputs and keeps the fastest; the first candidate (the
library default) stays unless another beats it by more than a margin, so that timing noise
between near-equal settings does not flip the choice.  It is host logic over the C
ABI: the steps it times are ordinary ``moe_fwd`` / ``moe_bwd`` calls.
"""
from __future__ import annotations

from dataclasses import dataclass, field

from . import MOE_F_RING_DISPATCH, MOE_F_SERIAL_BWD

CHUNK_ROWS = (256, 192, 128, 96, 64, 32)
PRODUCERS = (128, 64, 32, 16, 8)   # the library default first


@dataclass(frozen=True)
class Knobs:
    chunk_rows: int = 256
    serial_bwd: bool = False
    producer_wgs: int = 0   # ring dispatch only (0: not a ring candidate)
    ring_rows: int = 0      # ring dispatch only (0: not a ring candidate)

    def label(self) -> str:
        return (f"chunk_rows={self.chunk_rows}" + (" serial_bwd" if self.serial_bwd else "")
                + (f" producers={self.producer_wgs}" if self.producer_wgs else "")
                + (f" ring_rows={self.ring_rows}" if self.ring_rows else ""))


@dataclass
class TuneResult:
    best: Knobs
    ms: dict = field(default_factory=dict)   # Knobs -> ms per step

    def table(self) -> dict:
        return {k.label(): round(v, 4) for k, v in sorted(self.ms.items(), key=lambda kv: kv[1])}


def candidates(T: int, E: int, k: int, n_shared: int, backward: bool, ring_rows: int = 0) -> list[Knobs]:
    """Knob settings worth timing for a shape.  A tile taller than the largest possible expert
    (T rows for a routed expert, T for the shared one) behaves like that expert's own height,
    so heights above the smallest multiple of 32 holding T rows are dropped.  With a ring of
    ring_rows rows: heights that divide it, every producer count at the first height, the
    default producer count at the others, then half and a quarter of the capacity (when still a
    whole number of the first height's slots) at the first height and default producers."""
    cap = max(32, min(256, -(-T // 32) * 32))
    chunks = [c for c in CHUNK_ROWS if c <= cap] or [cap]
    if cap not in chunks:
        chunks.insert(0, cap)
    serial = (False, True) if backward else (False,)
    if not ring_rows:
        return [Knobs(c, s) for c in chunks for s in serial]
    chunks = [c for c in chunks if ring_rows % c == 0] or [32]
    out = [Knobs(chunks[0], s, p, ring_rows) for p in PRODUCERS for s in serial]
    out += [Knobs(c, s, PRODUCERS[0], ring_rows) for c in chunks[1:] for s in serial]
    for div in (2, 4):
        cap = ring_rows // div
        if ring_rows % div == 0 and cap >= chunks[0] and cap % chunks[0] == 0:
            out += [Knobs(chunks[0], s, PRODUCERS[0], cap) for s in serial]
    return out


def apply(cfg, knobs: Knobs) -> None:
    """Write the knobs into a moe_config (chunk_rows, producer_wgs and ring_rows when set, and
    the MOE_F_SERIAL_BWD bit)."""
    cfg.chunk_rows = knobs.chunk_rows
    if knobs.producer_wgs:
        cfg.producer_wgs = knobs.producer_wgs
    if knobs.ring_rows:
        cfg.ring_rows = knobs.ring_rows
    if knobs.serial_bwd:
        cfg.flags |= MOE_F_SERIAL_BWD
    else:
        cfg.flags &= ~MOE_F_SERIAL_BWD


def tune(layer, backward: bool = True, steps: int = 3, warmup: int = 1, stream=None, timer=None,
         cands: list[Knobs] | None = None, margin: float = 0.01) -> TuneResult:
    """Time every candidate on `layer` (a MoeLayer with inputs and experts loaded) and leave the
    chosen one in layer.cfg: the fastest, if it beats the first candidate by more than `margin`
    (a fraction of its time), else the first.  timer(step_fn, steps) -> ms per step; by default
    device events around `steps` calls on `stream` after `warmup` untimed ones."""
    if cands is None:
        ring = (layer.cfg.ring_rows or 16384) if layer.cfg.flags & MOE_F_RING_DISPATCH else 0
        cands = candidates(layer.T, layer.E, layer.k, layer.S, backward, ring)

    def step():
        layer.forward(stream)
        if backward:
            layer.backward(stream)

    if timer is None:
        timer = _event_timer(stream, warmup)
    res = TuneResult(best=cands[0])
    for kn in cands:
        apply(layer.cfg, kn)
        res.ms[kn] = float(timer(step, steps))
    fastest = min(res.ms, key=lambda kn: (res.ms[kn], cands.index(kn)))
    res.best = fastest if res.ms[fastest] < res.ms[cands[0]] * (1.0 - margin) else cands[0]
    apply(layer.cfg, res.best)
    return res


def _event_timer(stream, warmup):
    import torch

    def run(step, steps):
        st = stream if stream is not None else torch.cuda.current_stream()
        for _ in range(warmup):
            step()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(steps):
            step()
        b.record(st)
        b.synchronize()
        return a.elapsed_time(b) / steps

    return run
