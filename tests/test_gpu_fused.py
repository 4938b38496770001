"""The fused expert tile (MOE_FFN_FUSED: gate/up, SwiGLU and down in one
kernel per 64-record tile, H kept in LDS; EStream section 3.2, "Fused Expert
Execution with Intra-NPU Pipelining").

It runs the same MFMA instruction over the same k order as the two
projection kernels and rounds H to bf16 the same way, so its output equals
theirs bit for bit; it is also checked against the oracle directly."""
import numpy as np
import pytest
import torch

from gpu_util import check_layer_output, gpu_inputs, say
from routed_expert_ffn_top_amd import binding as B
from routed_expert_ffn_top_amd.inputs import CONFIGS, MoEConfig
from routed_expert_ffn_top_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

# f not a multiple of 128 (so the down projection is never split), several
# 64-record tiles per slot with ragged tails
MID_F = MoEConfig(name="mid_fused", index=71, T=300, d=512, f=448, E=16, k=8)


def _run(layer, inp, fused):
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    B.moe_route_build(s, 0, s.T, L, layer.phi, 0, layer.routes, layer.ws)
    Y = inp.A.clone()
    flags = B.MOE_FFN_EXPERTS | B.MOE_FFN_FINALIZE | (B.MOE_FFN_FUSED if fused else 0)
    B.moe_expert_ffn(s, layer.X, Y, layer.routes, layer.arena, layer.phi, flags, layer.ws)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("cfg", [MID_F, CONFIGS["olmoe_t1024"], CONFIGS["olmoe_t4096"]],
                         ids=["mid", "olmoe_t1024", "olmoe_t4096"])
def test_fused_equals_split_and_oracle(cfg):
    say(f"fused expert tile vs the split kernels and the oracle ({cfg.name})")
    inp = gpu_inputs(cfg)
    layer = MoELayer(inp)
    y_split = _run(layer, inp, False)
    y_fused = _run(layer, inp, True)
    y_again = _run(layer, inp, True)
    assert torch.equal(y_fused.view(torch.int32), y_split.view(torch.int32)), "fused output differs from split"
    assert torch.equal(y_again.view(torch.int32), y_fused.view(torch.int32)), "fused output not reproducible"
    err, ffn, _ = check_layer_output(layer, inp, y_fused)
    say(f"  same bits as the split kernels; rel err {err:.3e}, expert sum {ffn:.3e}")


@pytest.mark.parametrize("kw", [dict(f=1088), dict(dtype="bf16_fp8w"), dict(d=576), dict(f=512, T=64)],
                         ids=["f_too_large", "fp8_weights", "d_not_128", "split_down"])
def test_fused_refuses_uncovered_shapes(kw):
    cfg = MoEConfig(name="fused_refuse", index=72, T=kw.pop("T", 128), d=512, f=448, E=8, k=2).with_(**kw)
    say(f"fused expert tile refuses {cfg.name} {kw}")
    inp = gpu_inputs(cfg)
    layer = MoELayer(inp)
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    B.moe_route_build(s, 0, s.T, L, layer.phi, 0, layer.routes, layer.ws)
    Y = inp.A.clone()
    with pytest.raises(B.MoEError) as ei:
        B.moe_expert_ffn(s, layer.X, Y, layer.routes, layer.arena, layer.phi,
                         B.MOE_FFN_EXPERTS | B.MOE_FFN_FUSED, layer.ws)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
