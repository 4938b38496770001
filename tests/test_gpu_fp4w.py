"""Parity of the MXFP4 weight-only layer (E2M1 expert weight codes with one
E8M0 scale per 32 weights of a row, bf16 activations) with the CPU oracle.

The oracle decodes the same codes and scale bytes from the OCP microscaling
definition into plain weights and runs the layer in fp64. Every decoded
weight is exact in bf16, so the tolerance is that of the bf16 layer:
max|y - y_ref| / max|y_ref| <= 1e-2; routing, descriptors and run-to-run
bits are exact as for every other layer.
"""
import numpy as np
import pytest
import torch

from gpu_util import OracleRun, TOL, check_layer_output, check_y, gpu_inputs, np32, rel_err, say
from routed_expert_ffn_top_amd import binding as B
from routed_expert_ffn_top_amd.inputs import CONFIGS, MoEConfig
from routed_expert_ffn_top_amd.layer import MoELayer
from test_gpu_parity import MID, MID_SHARED, _check_layer, _layer_out

pytestmark = pytest.mark.gpu

MID4 = MID.with_(name="mid_fp4w", dtype="bf16_fp4w")
MID4_SHARED = MID_SHARED.with_(name="mid_shared_fp4w", dtype="bf16_fp4w")


def test_layer_mid_fp4w():
    say("layer mid, MXFP4 weights")
    _check_layer(MID4)


def test_layer_shared_experts_fp4w():
    say("layer with shared experts, MXFP4 weights")
    _check_layer(MID4_SHARED)


def test_layer_ragged_weight_blocks_fp4w():
    say("layer, MXFP4 weights, d = 320 (a 64-row second down block)")
    _check_layer(MoEConfig(name="ragged_fp4w", index=33, T=150, d=320, f=128, E=8, k=2, dtype="bf16_fp4w"))


def test_layer_olmoe_t4096_fp4w():
    say("layer OLMoE T=4096, MXFP4 weights, every token")
    cfg = CONFIGS["olmoe_t4096_fp4w"]
    _check_layer(cfg)


def test_layer_dsv2lite_t4096_fp4w():
    say("layer DSV2-Lite T=4096 (2 shared experts, f = 1408), MXFP4 weights, every token")
    _check_layer(CONFIGS["dsv2lite_t4096_fp4w"])


def test_layer_mixtral_t256_fp4w():
    say("layer Mixtral T=256, MXFP4 weights, split-K down, every token")
    cfg = CONFIGS["mixtral_t256_fp4w"]
    _check_layer(cfg)


def test_fp4w_edge_shapes():
    say("MXFP4 weights: one token and a ragged token count")
    for T in (1, 77):
        _check_layer(MID4.with_(T=T, name=f"mid_fp4w_T{T}"))


def test_fp4w_capacity_split_same_bits():
    say("MXFP4 weights: a capacity split gives the same bits")
    inp = gpu_inputs(MID4)
    y1 = _layer_out(MoELayer(inp), inp)
    split = MoELayer(inp, capacity=(MID4.T * MID4.kp) // 3 + 5)
    assert torch.equal(_layer_out(split, inp), y1)


def test_fp4w_plain_kernel_rejected():
    say("MXFP4 weights: the plain bf16 kernel is refused")
    inp = gpu_inputs(MID4)
    layer = MoELayer(inp)
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    B.moe_route_build(s, 0, s.T, L, layer.phi, 0, layer.routes, layer.ws)
    Y = inp.A.clone()
    with pytest.raises(B.MoEError) as ei:
        B.moe_expert_ffn(s, layer.X, Y, layer.routes, layer.arena, layer.phi,
                         B.MOE_FFN_EXPERTS | B.MOE_FFN_SIMPLE_KERNEL, layer.ws)
    assert ei.value.status == B.MOE_ERR_UNSUPPORTED


def test_paged_equals_resident_fp4w():
    say("paged layer with MXFP4 weights (P=16, G=8) vs resident")
    cfg = CONFIGS["virt_olmoe_t256_fp4w"]
    inp = gpu_inputs(cfg)
    res = MoELayer(inp)
    y_res = _layer_out(res, inp)
    res.close()
    paged = MoELayer(inp, paged=True)
    copy = torch.cuda.Stream()
    for _ in range(2):                   # the arena is reused by the second call
        Y = inp.A.clone()
        paged.forward(Y, copy=copy)
        torch.cuda.synchronize()
        assert torch.equal(Y, y_res), "paging changed the output"
    check_layer_output(paged, inp, Y)


def test_fp4w_quantisation_error_is_bounded():
    say("MXFP4 weights vs the bf16 layer of the same draws")
    i4, ib = gpu_inputs(MID4), gpu_inputs(MID)
    assert torch.equal(i4.A, ib.A) and torch.equal(i4.X, ib.X)
    f4 = np32(_layer_out(MoELayer(i4), i4) - i4.A)      # the FFN part of the output
    fb = np32(_layer_out(MoELayer(ib), ib) - ib.A)
    d = rel_err(f4, fb.astype(np.float64))
    say(f"  rel diff MXFP4 vs bf16 weights: {d:.3e}")
    assert d < 0.5


def _random_scales(inp, seed):
    """Replace the quantiser's block scales (nearly all the same byte for these
    draws) by seeded bytes in [112, 128], about 2 % of them 0 (2^-127), so
    that a scale taken from the wrong row or K block changes the result."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    for name in ("Sg", "Su", "Sd"):
        S = getattr(inp, name)
        R = torch.randint(112, 129, S.shape, generator=gen, device="cuda", dtype=torch.int32)
        Z = torch.rand(S.shape, generator=gen, device="cuda") < 0.02
        setattr(inp, name, torch.where(Z, torch.zeros_like(R), R).to(torch.uint8).contiguous())
    return inp


@pytest.mark.parametrize("cfg", [MID4, MoEConfig(name="ragged_fp4w_scales", index=34, T=120, d=320, f=192, E=6,
                                                   k=2, dtype="bf16_fp4w")], ids=["mid", "ragged"])
def test_fp4w_random_block_scales(cfg):
    say(f"MXFP4 weights with random block scales ({cfg.name})")
    inp = _random_scales(gpu_inputs(cfg), seed=5 + cfg.index)
    assert len(torch.unique(inp.Sd)) > 10
    layer = MoELayer(inp)
    Y = inp.A.clone()
    layer.forward(Y)
    torch.cuda.synchronize()
    err, ffn, _ = check_layer_output(layer, inp, Y)
    say(f"  rel err {err:.3e}, expert sum {ffn:.3e}")
