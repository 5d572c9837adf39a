"""moe_fwd_noalloc (the forward without a workspace, its scratch in a static device array) gives
bit for bit the results of moe_fwd, on two calls in a row, the second with a smaller layer."""
import numpy as np
import pytest

import moe_inputs
from helpers import log

pytestmark = pytest.mark.gpu

BIG = moe_inputs.LayerConfig("noalloc_big", T=600, d=256, E=24, k=4, inter=256, score="sigmoid", seed=41,
                             n_shared=1, zipf_s=1.1, zipf_lam=0.5)
SMALL = moe_inputs.LayerConfig("noalloc_small", T=130, d=128, E=8, k=2, inter=128, score="softmax", seed=42)


def _pair(cfg):
    import torch
    import mixture_experts_layer_schedule_amd as moe
    from helpers import gpu_layer
    inp = moe_inputs.layer_inputs(cfg)
    ref = gpu_layer(cfg, False, inp=inp)                       # moe_fwd with a workspace
    other = gpu_layer(cfg, False, inp=inp)                     # same weights, fresh buffers
    other.saved.fill_(0xA5)
    other.y.fill_(0)
    other.y32.fill_(0)
    moe.moe_fwd_noalloc(other.cfg, other.x, other.w_r, other.bias, other.w1q, other.w1s, other.w2q, other.w2s,
                        other.y, other.y32, other.saved)
    torch.cuda.synchronize()
    return ref, other


def test_noalloc_forward_matches_forward_twice():
    import torch
    for cfg in (BIG, SMALL):  # the second call is smaller than the first
        log(f"no-alloc forward: {cfg.name}")
        ref, got = _pair(cfg)
        assert torch.equal(ref.y, got.y) and torch.equal(ref.y32, got.y32), cfg.name
        for name in ("logits", "idx", "w", "counts", "offsets", "perm", "pos", "xq", "xs", "g", "u", "hq", "hs",
                     "yslot", "w1t", "w1ts", "w2t", "w2ts"):
            a, b = ref.saved_tensor(name), got.saved_tensor(name)
            if name in ("w1t", "w1ts", "w2t", "w2ts"):  # only experts with rows are written
                rows = ref.saved_tensor("counts").cpu().numpy() > 0
                a, b = a[torch.from_numpy(rows).cuda()], b[torch.from_numpy(rows).cuda()]
            assert torch.equal(a, b), (cfg.name, name)


def test_noalloc_rejects_configurations_beyond_its_scratch():
    import mixture_experts_layer_schedule_amd as moe
    cfg = moe.make_config(1 << 19, 128, 512, 1, 128)   # 8192 token blocks x 512 experts x 4 B > 4 MiB
    p = 1 << 20
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_fwd_noalloc(cfg, p, p, None, p, p, p, p, p, None, p, stream=0, saved_bytes=1 << 45)
    assert ei.value.status == moe.MOE_EWORKSPACE
