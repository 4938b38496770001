"""moe_layer_prefill_noalloc against moe_layer_prefill: the allocation-free
entry point (its workspace is the library's fixed device array) gives the
same bits as the entry point with a caller workspace, on two calls in a row,
the second with fewer tokens, and leaves every descriptor as the other one
does."""
import pytest
import torch

from gpu_util import gpu_inputs, say
from routed_expert_ffn_top_amd import binding as B
from routed_expert_ffn_top_amd.inputs import CONFIGS
from routed_expert_ffn_top_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


def _shape(cfg, T):
    return B.make_shape(T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.n_shared, dtype=cfg.dtype, renorm=cfg.renorm)


@pytest.mark.parametrize("name,T1,T2", [("olmoe_t1024", 800, 333), ("dsv2lite_t4096", 512, 97),
                                         ("tiny_fp32", 64, 17)])
def test_noalloc_equals_workspace_entry_point(name, T1, T2):
    cfg = CONFIGS[name].with_(T=T1)
    say(f"noalloc layer vs moe_layer_prefill: {name} T={T1} then T={T2}")
    inp = gpu_inputs(cfg)
    layer = MoELayer(inp)
    for T in (T1, T2):
        s = _shape(cfg, T)
        assert 0 < B.moe_workspace_bytes(s) <= SCRATCH
        X = inp.X[:T]
        A = inp.A[:T]
        r_ref, ws = B.alloc_routes(s), B.alloc_workspace(s)
        Y_ref = A.clone()
        B.moe_layer_prefill(s, X, layer.Wr, layer.bias, None, Y_ref, layer.arena, None, None, r_ref, ws)
        r_na = B.alloc_routes(s)
        for q in r_na.values():
            q.fill_(-7)
        Y = A.clone()
        B.moe_layer_prefill_noalloc(s, X, layer.Wr, layer.bias, None, Y, layer.arena, r_na)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int32), Y_ref.view(torch.int32)), f"T={T}: output differs"
        n = int(r_ref["slot_offset"][-1])
        for key in ("topk_idx", "topk_w", "slot_count", "slot_offset", "route_pos"):
            assert torch.equal(r_na[key], r_ref[key]), f"T={T}: {key} differs"
        for key in ("rec_token", "rec_route"):
            assert torch.equal(r_na[key][:n], r_ref[key][:n]), f"T={T}: {key} differs"
        say(f"  T={T}: same bits ({n} routes)")


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    cfg = CONFIGS["olmoe_t1024"]
    s = _shape(cfg, 1024)
    assert B.moe_workspace_bytes(s) > SCRATCH
    inp = gpu_inputs(cfg.with_(T=16))
    layer = MoELayer(inp)
    Y = torch.zeros((1024, cfg.d), dtype=torch.float32, device="cuda")
    X = torch.zeros((1024, cfg.d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.MoEError) as ei:
        B.moe_layer_prefill_noalloc(s, X, layer.Wr, layer.bias, None, Y, layer.arena, B.alloc_routes(s))
    assert ei.value.status == B.MOE_ERR_WORKSPACE
    assert "64" in str(ei.value) or "67108864" in str(ei.value)
