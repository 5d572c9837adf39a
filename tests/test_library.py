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


def test_header_structs_match_the_binding():
    """moe_saved_layout / moe_workspace_layout field order in moe.h equals the ctypes mirrors."""
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    for name, cls in (("moe_saved_layout", moe.moe_saved_layout), ("moe_workspace_layout", moe.moe_workspace_layout)):
        body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, flags=re.S).group(1)
        fields = re.findall(r"^\s*size_t\s+(\w+);", body, flags=re.M)
        assert fields == [f for f, _ in cls._fields_], name
    body = re.search(r"typedef struct moe_config \{(.*?)\} moe_config;", text, flags=re.S).group(1)
    fields = re.findall(r"^\s*u?int32_t\s+(\w+);", body, flags=re.M)
    assert fields == [f for f, _ in moe.moe_config._fields_]


@pytest.mark.parametrize("kw", [dict(), dict(ring_rows=256), dict(ring_rows=2048, producer_wgs=8),
                                dict(ring_rows=384, chunk_rows=128, producer_wgs=128)])
def test_ring_dispatch_configurations_are_accepted(kw):
    """The ring dispatch takes any whole number of slots (one chunk of chunk_rows rows each) and
    up to 128 producer workgroups; its buffer lives in the workspace."""
    ws0, _, wl0 = moe.moe_query(moe.make_config(4096, 256, 8, 2, 128), with_workspace_layout=True)
    ws, _, wl = moe.moe_query(moe.make_config(4096, 256, 8, 2, 128, flags=moe.MOE_F_RING_DISPATCH, **kw),
                              with_workspace_layout=True)
    slots = (kw.get("ring_rows") or 16384) // (kw.get("chunk_rows") or 256)
    assert wl.ring_s - wl.ring >= slots * (kw.get("chunk_rows") or 256) * 256 and ws > ws0


def test_ring_workspace_does_not_depend_on_the_row_tile_height():
    """The tuner changes chunk_rows on a layer whose workspace is already allocated: the ring's
    regions are sized by its capacity alone, for every height that divides it."""
    f = moe.MOE_F_RING_DISPATCH
    for ring_rows in (2048, 16384):
        sizes = {moe.moe_query(moe.make_config(4096, 256, 8, 2, 128, ring_rows=ring_rows, chunk_rows=c,
                                               flags=f))[0] for c in (0, 256, 128, 64, 32)}
        assert len(sizes) == 1


@pytest.mark.parametrize("rows", [32, 64, 96, 128, 192, 256])
def test_row_tile_heights_are_accepted_on_the_direct_path(rows):
    """chunk_rows (rows per GEMM row tile) is a tuning knob of every path and leaves the buffer
    layouts unchanged."""
    ws0, sl0 = moe.moe_query(moe.make_config(4096, 256, 8, 2, 128))
    ws, sl = moe.moe_query(moe.make_config(4096, 256, 8, 2, 128, chunk_rows=rows))
    assert ws == ws0 and sl.total == sl0.total


def test_query_layout_is_aligned_and_ordered():
    cfg = moe.make_config(256, 256, 8, 2, 128)
    ws, sl, wl = moe.moe_query(cfg, with_workspace_layout=True)
    for layout in (sl, wl):
        offs = [getattr(layout, f) for f, _ in type(layout)._fields_ if f not in ("tok_stride",)]
        assert all(o % 256 == 0 for o in offs[:-1])
        assert offs == sorted(offs)
    assert sl.yslot + 4 * 256 * 2 * 256 <= sl.w1t
    # transposed weights: NX * 2I * d codes (+ scales) for W1t, half of that for W2t
    assert sl.w1ts - sl.w1t >= 8 * 2 * 128 * 256 and sl.w2ts - sl.w2t >= 8 * 128 * 256
    assert ws == wl.total and ws > 0
    assert wl.tok_stride % 128 == 0 and wl.tok_stride >= 256 * 2 + 127 * 8


def test_forward_only_layout_drops_transposed_weights():
    _, full = moe.moe_query(moe.make_config(256, 256, 8, 2, 128))
    _, fo = moe.moe_query(moe.make_config(256, 256, 8, 2, 128, flags=moe.MOE_F_FORWARD_ONLY))
    assert fo.w1t == fo.w1ts == fo.w2t == fo.w2ts == fo.total
    assert fo.total < full.total


@pytest.mark.parametrize("kw,status", [
    (dict(d=100), moe.MOE_ESHAPE),       # d not a multiple of 128
    (dict(inter=96), moe.MOE_ESHAPE),
    (dict(k=0), moe.MOE_ESHAPE),
    (dict(k=9, E=8), moe.MOE_ESHAPE),    # k > E
    (dict(E=600), moe.MOE_ESHAPE),
    (dict(n_shared=2), moe.MOE_ESHAPE),
    (dict(score_fn=7), moe.MOE_EINVAL),
    (dict(T=0), moe.MOE_ESHAPE),
    (dict(ring_rows=256), moe.MOE_EINVAL),   # ring capacity and producers act on the ring dispatch only
    (dict(producer_wgs=8), moe.MOE_EINVAL),
    (dict(chunk_rows=100), moe.MOE_ESHAPE),  # row tiles: multiples of 32 ...
    (dict(chunk_rows=16), moe.MOE_ESHAPE),
    (dict(chunk_rows=288), moe.MOE_ESHAPE),  # ... up to 256
    (dict(chunk_rows=-32), moe.MOE_ESHAPE),
    (dict(flags=2, ring_rows=300), moe.MOE_ESHAPE),   # ring: whole slots of chunk_rows rows
    (dict(flags=2, ring_rows=128), moe.MOE_ESHAPE),   # ... at least one
    (dict(flags=2, chunk_rows=128, ring_rows=192), moe.MOE_ESHAPE),
    (dict(flags=2, producer_wgs=129), moe.MOE_ESHAPE),
    (dict(flags=3), moe.MOE_EINVAL),         # direct gather and ring dispatch together
    (dict(flags=128), moe.MOE_EINVAL),       # unknown flag
    (dict(flags=32), moe.MOE_EINVAL),        # the unfused forward needs MOE_F_FORWARD_ONLY
    (dict(flags=32 | 16 | 8), moe.MOE_EINVAL),  # ... and real experts
    # the unfused forward's permuted rows: T * (k + S) * d reaches 2^32
    (dict(T=(1 << 32) // (7168 * 2) + 1, d=7168, E=8, k=2, inter=128, flags=48), moe.MOE_ESHAPE),
    # 32-bit operand offsets: T * d reaches 2^32
    (dict(T=(1 << 32) // 7168 + 1, d=7168, E=8, k=1, inter=128), moe.MOE_ESHAPE),
    # one expert's weights 2 * I * d reach 2^32
    (dict(d=65536, inter=32768), moe.MOE_ESHAPE),
    # token-axis operand stride reaches 2^24 (T * k + 127 * E)
    (dict(T=1 << 20, d=128, E=16, k=16, inter=128), moe.MOE_ESHAPE),
    (dict(T=1 << 26, d=128, E=16, k=16, inter=128), moe.MOE_ESHAPE),  # T * k >= 2^30
])
def test_query_rejects_bad_config(kw, status):
    base = dict(T=256, d=256, E=8, k=2, inter=128)
    base.update(kw)
    score = base.pop("score_fn", 0)
    cfg = moe.make_config(**base, score_fn=score)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_query(cfg)
    assert ei.value.status == status


def test_query_accepts_sizes_just_inside_the_limits():
    moe.moe_query(moe.make_config((1 << 32) // 7168, 7168, 8, 1, 128))       # T * d < 2^32
    moe.moe_query(moe.make_config(256, 65536, 8, 2, 32768 - 128))             # 2 I d < 2^32
    moe.moe_query(moe.make_config(1 << 19, 128, 16, 16, 128))                 # stride < 2^24


@pytest.mark.parametrize("flags", [0, 1, 4, 5, 8, 9, 16, 20, 48, 49])
def test_query_accepts_schedule_flags(flags):
    """Direct gather (1), the launch-order backward (4), identity experts (8), forward only (16) and
    the unfused forward (32 with 16)."""
    ws, _ = moe.moe_query(moe.make_config(256, 256, 8, 2, 128, flags=flags))
    assert ws > 0


def test_unfused_layout_holds_the_permuted_rows():
    T, d, E, k, I = 256, 256, 8, 2, 128
    RS = T * k
    _, fo, wfo = moe.moe_query(moe.make_config(T, d, E, k, I, flags=moe.MOE_F_FORWARD_ONLY), with_workspace_layout=True)
    _, uf, wuf = moe.moe_query(moe.make_config(T, d, E, k, I, flags=moe.MOE_F_FORWARD_ONLY | moe.MOE_F_UNFUSED),
                               with_workspace_layout=True)
    assert uf.total == fo.total  # the saved state is the fused forward's
    assert wfo.xp == wfo.xps == wfo.yrows and wfo.yrows <= wfo.total
    assert wuf.xps - wuf.xp >= RS * d and wuf.yrows - wuf.xps >= RS * d // 32
    assert wuf.total - wuf.yrows >= 4 * RS * d


def test_noalloc_forward_rejects_workspace_modes():
    """The ring dispatch and the unfused forward need a workspace: refused before any launch."""
    p, big = 1 << 20, 1 << 40
    for flags in (moe.MOE_F_FORWARD_ONLY | moe.MOE_F_UNFUSED,):
        cfg = moe.make_config(256, 256, 8, 2, 128, flags=flags)
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_fwd_noalloc(cfg, p, p, None, p, p, p, p, p, None, p, stream=0, saved_bytes=big)
        assert ei.value.status == moe.MOE_EINVAL


def test_forward_rejects_null_and_misaligned_pointers_without_launching():
    cfg = moe.make_config(256, 256, 8, 2, 128)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fwd(cfg, 0, 0, None, 0, 0, 0, 0, 0, None, 0, 0, stream=0, saved_bytes=0, workspace_bytes=0)
    assert ei.value.status == moe.MOE_EINVAL
    big = 1 << 40
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fwd(cfg, 4096 + 8, 4096, None, 4096, 4096, 4096, 4096, 4096, None, 4096, 4096, stream=0,
                    saved_bytes=big, workspace_bytes=big)
    assert ei.value.status == moe.MOE_EALIGN
    bad = moe.make_config(256, 100, 8, 2, 128)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_bwd(bad, 4096, 4096, 4096, 4096, 4096, None, 4096, 4096, 4096, 4096, stream=0, saved_bytes=big,
                    workspace_bytes=big)
    assert ei.value.status == moe.MOE_ESHAPE


def test_small_buffers_are_rejected_before_any_launch():
    cfg = moe.make_config(256, 256, 8, 2, 128)
    ws, sl = moe.moe_query(cfg)
    p = 1 << 20  # aligned dummy addresses: the call must return before touching them
    for sb, wb in ((sl.total - 1, ws), (sl.total, ws - 1), (0, 0)):
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_fwd(cfg, p, p, None, p, p, p, p, p, None, p, p, stream=0, saved_bytes=sb, workspace_bytes=wb)
        assert ei.value.status == moe.MOE_EWORKSPACE
        with pytest.raises(moe.MoeError) as ei:
            moe.moe_bwd(cfg, p, p, p, p, p, None, p, p, p, p, stream=0, saved_bytes=sb, workspace_bytes=wb)
        assert ei.value.status == moe.MOE_EWORKSPACE


@pytest.mark.parametrize("flags", [moe.MOE_F_IDENTITY_EXPERTS, moe.MOE_F_FORWARD_ONLY])
def test_backward_rejects_forward_only_modes(flags):
    cfg = moe.make_config(256, 256, 8, 2, 128, flags=flags)
    p, big = 1 << 20, 1 << 40
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_bwd(cfg, p, p, p, p, p, None, p, p, p, p, stream=0, saved_bytes=big, workspace_bytes=big)
    assert ei.value.status == moe.MOE_EINVAL


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
    assert moe.moe_strerror(99) == "unknown status"


def test_mfma_probe_rejects_bad_arguments_without_launching():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_probe_mfma(1 << 20, 0, stream=0, sink_bytes=1 << 30)
    assert ei.value.status == moe.MOE_EINVAL


def test_header_compiles_as_c_and_a_c_program_queries_the_layout(tmp_path):
    """include/moe.h is a C header: a C99 program built with gcc against it links the library
    and gets the same buffer sizes from moe_query as the Python binding, and the same status for a
    rejected configuration."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(moe.LIB_PATH)
    exe = tmp_path / "query_sizes"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I" + os.path.join(root, "include"), os.path.join(root, "tests", "c_abi", "query_sizes.c"),
           "-L" + libdir, "-l:" + os.path.basename(moe.LIB_PATH), "-Wl,-rpath," + libdir, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # warnings from inside the HIP runtime headers are theirs; the program's own must be clean
    if r.returncode != 0 and "query_sizes.c" in r.stderr:
        raise AssertionError(r.stderr[-2000:])
    if r.returncode != 0:
        cmd.remove("-Werror")
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
    for shape in ((8192, 7168, 256, 8, 2048, 0, 0), (16384, 7168, 384, 8, 2048, 1, moe.MOE_F_FORWARD_ONLY),
                  (256, 256, 8, 2, 128, 0, moe.MOE_F_RING_DISPATCH)):
        out = subprocess.run([str(exe), *map(str, shape)], capture_output=True, text=True, check=True).stdout.split()
        T, d, E, k, inter, S, flags = shape
        cfg = moe.make_config(T, d, E, k, inter, S, moe.MOE_SCORE_SIGMOID, flags=flags)
        ws, sl, wl = moe.moe_query(cfg, with_workspace_layout=True)
        assert [int(v) for v in out[:4]] == [moe.MOE_OK, ws, sl.total, wl.total]
        assert int(out[4]) == moe.MOE_ESHAPE and " ".join(out[5:]) == moe.moe_strerror(moe.MOE_ESHAPE)


def test_flag_values_match_the_header():
    """Every MOE_F_* flag the header defines has the same value in the binding, and moe_query
    accepts each one that stands alone on the default path (bf16 weight gradients included)."""
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    flags = {n: int(v) for n, v in re.findall(r"#define (MOE_F_\w+) (\d+)u", text)}
    assert flags and all(getattr(moe, n) == v for n, v in flags.items())
    for f in (moe.MOE_F_DW_BF16, moe.MOE_F_DW_BF16 | moe.MOE_F_RING_DISPATCH | moe.MOE_F_SERIAL_BWD):
        moe.moe_query(moe.make_config(4096, 256, 8, 2, 128, flags=f))

