"""GPU test of moe_layer_forward_noalloc, the allocation-free entry point.

Through the C ABI: two calls in a row (the second with fewer tokens) on a
layer that has no workspace bound, each compared with the existing entry
point moe_layer_forward on a second handle of the same layer (its one-token
calls: bit-identical, since both run the same decode kernels) and with the
fp64 oracle (ids exact unless the selection gap is below 1e-6, outputs within
2e-3 of max|ref| per token).  The second call also checks that nothing of
the first call's state leaks into it, and that NULL ids / weights are
accepted.  Collected last so that a failure here hides no other test.
"""
import sys

import numpy as np
import pytest

from routed_expert_int4_amd import binding as B
from routed_expert_int4_amd import synth
from tests.helpers import MID_A, check_layer

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cfg_name", ["MID_A", "GLM"])
def test_noalloc_forward_matches_forward(cfg_name):
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from routed_expert_int4_amd.layer import DeviceLayer
    cfg = {"MID_A": MID_A, "GLM": synth.GLM}[cfg_name]
    say(f"[gpu] noalloc forward, {cfg_name}")
    weights = synth.gen_layer(cfg, seed=0)
    ref_layer = DeviceLayer(weights, max_T=1)
    # a second handle on the same device tensors with no workspace bound
    bare = B.moe_layer_create(cfg, ref_layer.router_w, ref_layer.bias,
                              [ref_layer.blobs[cfg.n_experts + s] for s in range(cfg.n_shared)])
    B.moe_layer_set_experts(bare, [ref_layer.blobs[e] for e in range(cfg.n_experts)])
    H, k = cfg.hidden, cfg.top_k
    for call, (T, seed) in enumerate([(7, 21), (3, 22)]):
        x_bits = synth.gen_tokens(cfg, T, seed=seed)
        x = DeviceLayer.to_device_bf16(x_bits)
        y = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda:0")
        ids = torch.full((T, k), -7, dtype=torch.int32, device="cuda:0")
        w = torch.full((T, k), float("nan"), dtype=torch.float32, device="cuda:0")
        B.moe_layer_forward_noalloc(bare, x, T, y, ids, w)
        y_ref, ids_ref, w_ref = ref_layer.forward_each(x)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref) and torch.equal(w, w_ref), f"call {call}: routing differs"
        assert torch.equal(y, y_ref), f"call {call}: outputs differ from moe_layer_forward"
        res = check_layer(weights, x_bits, y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy())
        say(f"[gpu] noalloc call {call} (T={T}): bit-identical to moe_layer_forward, oracle rel err "
            f"{res['worst_rel']:.3g}")
        # outputs only, no routing buffers
        y2 = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda:0")
        B.moe_layer_forward_noalloc(bare, x, T, y2)
        torch.cuda.synchronize()
        assert torch.equal(y2, y_ref)
    with pytest.raises(B.MoeError) as err:
        B.moe_layer_forward_noalloc(bare, None, 1, y)
    assert err.value.code == B.MOE_EINVAL
    B.moe_layer_forward_noalloc(bare, x, 0, y)  # T = 0 is a no-op
    B.moe_layer_destroy(bare)
    ref_layer.close()


def test_noalloc_rejects_cached_layer():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from routed_expert_int4_amd.layer import DeviceLayer, ExpertCache
    cfg = MID_A
    weights = synth.gen_layer(cfg, seed=0)
    cache = ExpertCache(cfg, 1, cfg.top_k)
    lay = DeviceLayer(weights, max_T=1, resident=False)
    lay.attach_cache(cache, 0)
    x = DeviceLayer.to_device_bf16(synth.gen_tokens(cfg, 1, seed=23))
    y = torch.empty((1, cfg.hidden), dtype=torch.float32, device="cuda:0")
    with pytest.raises(B.MoeError) as err:
        B.moe_layer_forward_noalloc(lay.handle, x, 1, y)
    assert err.value.code == B.MOE_EINVAL and "cache" in B.last_error()
    lay.close()
    cache.close()
