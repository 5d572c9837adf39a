"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on the host.

These run without a GPU: only moe_query, moe_strerror and argument validation, which return
before any device call.
"""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_schedule_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(moe.EXPORTS)
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n


def test_query_layout_is_aligned_and_ordered():
    cfg = moe.make_config(256, 256, 8, 2, 128)
    ws, sl = moe.moe_query(cfg)
    offs = [getattr(sl, f) for f, _ in moe.moe_saved_layout._fields_]
    assert all(o % 256 == 0 for o in offs[:-1])
    assert offs == sorted(offs)
    assert sl.yslot + 4 * 256 * 2 * 256 <= sl.total
    assert ws > 0


@pytest.mark.parametrize("kw,status", [
    (dict(d=100), moe.MOE_ESHAPE),       # d not a multiple of 128
    (dict(inter=96), moe.MOE_ESHAPE),
    (dict(k=0), moe.MOE_ESHAPE),
    (dict(k=9, E=8), moe.MOE_ESHAPE),    # k > E
    (dict(E=600), moe.MOE_ESHAPE),
    (dict(n_shared=2), moe.MOE_ESHAPE),
    (dict(score_fn=7), moe.MOE_EINVAL),
    (dict(T=0), moe.MOE_ESHAPE),
    (dict(ring_rows=128), moe.MOE_ESHAPE),   # ring slots hold 256 rows
    (dict(chunk_rows=128), moe.MOE_ESHAPE),
    (dict(producer_wgs=129), moe.MOE_ESHAPE),
    (dict(flags=3), moe.MOE_EINVAL),         # direct gather and ring dispatch together
    (dict(flags=16), moe.MOE_EINVAL),        # unknown flag
])
def test_query_rejects_bad_config(kw, status):
    base = dict(T=256, d=256, E=8, k=2, inter=128)
    base.update(kw)
    score = base.pop("score_fn", 0)
    cfg = moe.make_config(**base, score_fn=score)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_query(cfg)
    assert ei.value.status == status


@pytest.mark.parametrize("flags", [0, 1, 4, 5, 8, 9])
def test_query_accepts_schedule_flags(flags):
    """Direct gather (1) and the launch-order backward (4) are valid alone and together."""
    ws, _ = moe.moe_query(moe.make_config(256, 256, 8, 2, 128, flags=flags))
    assert ws > 0


def test_forward_rejects_null_and_misaligned_pointers_without_launching():
    cfg = moe.make_config(256, 256, 8, 2, 128)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fwd(cfg, 0, 0, None, 0, 0, 0, 0, 0, None, 0, 0, stream=0)
    assert ei.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fwd(cfg, 4096 + 8, 4096, None, 4096, 4096, 4096, 4096, 4096, None, 4096, 4096, stream=0)
    assert ei.value.status == moe.MOE_EALIGN
    bad = moe.make_config(256, 100, 8, 2, 128)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_bwd(bad, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, None, 4096, 4096, 4096, 4096, stream=0)
    assert ei.value.status == moe.MOE_ESHAPE


def test_quantize_rejects_ragged_blocks():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_quantize_mxfp8(4096, 0, 4, 48, 4096, 4096, stream=0)
    assert ei.value.status == moe.MOE_ESHAPE
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_requant_transpose(4096, 4096, 1, 96, 64, 4096, 4096, stream=0)
    assert ei.value.status == moe.MOE_ESHAPE


def test_strerror_covers_every_status():
    for s in range(7):
        assert moe.moe_strerror(s) and moe.moe_strerror(s) != "unknown status"
