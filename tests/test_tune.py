"""Host logic of the per-workload tuner (mixture_experts_layer_schedule_amd.tune), with a stand-in
layer and timer: no GPU."""
from types import SimpleNamespace

import mixture_experts_layer_schedule_amd as moe
from mixture_experts_layer_schedule_amd import tune


def test_candidates_cover_the_row_tile_heights_and_both_schedules():
    c = tune.candidates(T=8192, E=256, k=8, n_shared=0, backward=True)
    assert {kn.chunk_rows for kn in c} == set(tune.CHUNK_ROWS)
    assert {kn.serial_bwd for kn in c} == {False, True}
    assert c[0] == tune.Knobs(256, False)            # the library default is timed first
    assert len(set(c)) == len(c)


def test_candidates_drop_heights_no_expert_can_fill_and_forward_has_one_schedule():
    c = tune.candidates(T=70, E=8, k=2, n_shared=0, backward=False)
    # an expert has at most T = 70 rows: 96 rows already hold it, taller tiles act the same
    assert [kn.chunk_rows for kn in c] == [96, 64, 32]
    assert all(not kn.serial_bwd for kn in c)
    assert [kn.chunk_rows for kn in tune.candidates(T=1, E=8, k=2, n_shared=1, backward=False)] == [32]


class _Layer:
    def __init__(self):
        self.T, self.E, self.k, self.S = 4096, 64, 4, 0
        self.cfg = moe.make_config(4096, 256, 64, 4, 128, flags=moe.MOE_F_SERIAL_BWD | moe.MOE_F_FORWARD_ONLY)
        self.calls = []

    def forward(self, stream=None):
        self.calls.append(("f", self.cfg.chunk_rows, bool(self.cfg.flags & moe.MOE_F_SERIAL_BWD)))

    def backward(self, stream=None):
        self.calls.append(("b", self.cfg.chunk_rows, bool(self.cfg.flags & moe.MOE_F_SERIAL_BWD)))


def test_tune_times_every_candidate_keeps_the_fastest_and_applies_it():
    layer = _Layer()
    cost = {tune.Knobs(256, False): 5.0, tune.Knobs(128, False): 4.0, tune.Knobs(128, True): 4.0,
            tune.Knobs(64, True): 6.0}
    seen = []

    def timer(step, steps):
        step()
        kn = tune.Knobs(layer.cfg.chunk_rows, bool(layer.cfg.flags & moe.MOE_F_SERIAL_BWD))
        seen.append(kn)
        return cost[kn]

    res = tune.tune(layer, backward=True, timer=timer, cands=list(cost))
    assert seen == list(cost)                                   # each once, in order
    assert res.best == tune.Knobs(128, False)                   # fastest; the earlier of a tie
    assert layer.cfg.chunk_rows == 128 and not layer.cfg.flags & moe.MOE_F_SERIAL_BWD
    assert layer.cfg.flags & moe.MOE_F_FORWARD_ONLY             # other flags untouched
    assert list(res.table()) == ["chunk_rows=128", "chunk_rows=128 serial_bwd", "chunk_rows=256",
                                 "chunk_rows=64 serial_bwd"]
    assert [c[0] for c in layer.calls] == ["f", "b"] * 4        # a step is forward then backward


def test_tune_keeps_the_default_unless_beaten_by_the_margin():
    layer = _Layer()
    cands = [tune.Knobs(256, False), tune.Knobs(128, False), tune.Knobs(64, False)]
    for cost, best in (({256: 10.0, 128: 9.95, 64: 10.5}, 256),   # 0.5 % faster: noise, keep 256
                       ({256: 10.0, 128: 9.8, 64: 9.7}, 64)):     # 3 % faster: switch
        res = tune.tune(layer, backward=False, cands=cands, margin=0.01,
                        timer=lambda step, steps: cost[layer.cfg.chunk_rows])
        assert res.best.chunk_rows == best and layer.cfg.chunk_rows == best


def test_apply_sets_and_clears_the_serial_schedule_bit():
    cfg = moe.make_config(256, 256, 8, 2, 128)
    tune.apply(cfg, tune.Knobs(64, True))
    assert cfg.chunk_rows == 64 and cfg.flags & moe.MOE_F_SERIAL_BWD
    tune.apply(cfg, tune.Knobs(256, False))
    assert cfg.chunk_rows == 256 and not cfg.flags & moe.MOE_F_SERIAL_BWD
    moe.moe_query(cfg)   # a tuned configuration is a valid one


def test_ring_candidates_tune_producers_and_keep_whole_slots():
    c = tune.candidates(T=16384, E=384, k=8, n_shared=1, backward=False, ring_rows=2048)
    assert c[0] == tune.Knobs(256, False, 128, 2048)           # the library default first
    assert {kn.producer_wgs for kn in c} == set(tune.PRODUCERS)
    assert all(kn.ring_rows % kn.chunk_rows == 0 for kn in c)   # whole slots only
    assert {kn.chunk_rows for kn in c} == {256, 128, 64, 32}
    assert {kn.ring_rows for kn in c} == {2048, 1024, 512}      # the budget and below, never above
    assert len(set(c)) == len(c)
    cfg = moe.make_config(16384, 256, 8, 2, 128, ring_rows=2048, flags=moe.MOE_F_RING_DISPATCH)
    ws = moe.moe_query(cfg)[0]
    tune.apply(cfg, tune.Knobs(128, False, 8))
    assert cfg.chunk_rows == 128 and cfg.producer_wgs == 8 and cfg.ring_rows == 2048
    for kn in c:   # every candidate runs in the workspace sized for the budget
        tune.apply(cfg, kn)
        assert moe.moe_query(cfg)[0] <= ws
