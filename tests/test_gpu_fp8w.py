"""Parity of the weight-only quantised layer (fp8 e4m3 expert weights with
fp32 row scales, bf16 activations) with the CPU oracle.

The oracle decodes the same e4m3 codes from the format's definition and
applies the same row scales in fp64. Tolerances are those of the bf16 layer:
max|y - y_ref| / max|y_ref| <= 1e-2; routing, descriptors and run-to-run bits
are exact as for every other layer.
"""
import numpy as np
import pytest
import torch

from gpu_util import OracleRun, TOL, check_layer_output, check_y, gpu_inputs, np32, rel_err, say
from routed_expert_ffn_top_amd import binding as B
from routed_expert_ffn_top_amd.inputs import CONFIGS
from routed_expert_ffn_top_amd.layer import MoELayer
from test_gpu_parity import MID, MID_SHARED, _check_layer, _layer_out

pytestmark = pytest.mark.gpu

MID8 = MID.with_(name="mid_fp8w", dtype="bf16_fp8w")
MID8_SHARED = MID_SHARED.with_(name="mid_shared_fp8w", dtype="bf16_fp8w")


def test_layer_mid_fp8w():
    say("layer mid, fp8 weights")
    _check_layer(MID8)


def test_layer_shared_experts_fp8w():
    say("layer with shared experts, fp8 weights")
    _check_layer(MID8_SHARED)


def test_layer_olmoe_t4096_fp8w():
    say("layer OLMoE T=4096, fp8 weights, every token")
    cfg = CONFIGS["olmoe_t4096_fp8w"]
    _check_layer(cfg)


def test_layer_dsv2lite_t4096_fp8w():
    say("layer DSV2-Lite T=4096 (2 shared experts, weights not renormalised), fp8 weights, every token")
    _check_layer(CONFIGS["dsv2lite_t4096_fp8w"])


def test_layer_mixtral_t256_fp8w():
    say("layer Mixtral T=256, fp8 weights, split-K down, every token")
    cfg = CONFIGS["mixtral_t256_fp8w"]
    _check_layer(cfg)


def test_fp8w_step_by_step_and_capacity_split():
    say("fp8 weights: separate calls and a capacity split give the same bits")
    inp = gpu_inputs(MID8)
    layer = MoELayer(inp)
    y1 = _layer_out(layer, inp)
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    B.moe_route_build(s, 0, s.T, L, layer.phi, 0, layer.routes, layer.ws)
    y2 = inp.A.clone()
    B.moe_expert_ffn(s, layer.X, y2, layer.routes, layer.arena, layer.phi,
                     B.MOE_FFN_EXPERTS | B.MOE_FFN_FINALIZE, layer.ws)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    split = MoELayer(inp, capacity=(MID8.T * MID8.kp) // 3 + 5)
    assert torch.equal(_layer_out(split, inp), y1)


def test_fp8w_plain_kernel_rejected():
    say("fp8 weights: the plain bf16 kernel is refused")
    inp = gpu_inputs(MID8)
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


def test_paged_equals_resident_fp8w():
    say("paged layer with fp8 weights (P=16, G=8) vs resident")
    cfg = CONFIGS["virt_olmoe_t256_fp8w"]
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


def test_fp8w_quantisation_error_is_small():
    say("fp8 weights vs the bf16 layer of the same draws")
    i8, ib = gpu_inputs(MID8), gpu_inputs(MID)
    assert torch.equal(i8.A, ib.A) and torch.equal(i8.X, ib.X)
    f8 = np32(_layer_out(MoELayer(i8), i8) - i8.A)      # the FFN part of the output
    fb = np32(_layer_out(MoELayer(ib), ib) - ib.A)
    d = rel_err(f8, fb.astype(np.float64))
    say(f"  rel diff fp8 vs bf16 weights: {d:.3e}")
    assert d < 0.1


def test_fp8w_edge_shapes():
    say("fp8 weights: one token and a ragged token count")
    for T in (1, 77):
        _check_layer(MID8.with_(T=T, name=f"mid_fp8w_T{T}"))


@pytest.mark.parametrize("dtype", ["bf16", "bf16_fp8w", "bf16_fp4w"])
def test_device_pack_equals_host_pack(dtype):
    say(f"gate/up and down packing on the device equal the host packing ({dtype})")
    cfg = MID.with_(dtype=dtype, E=3, k=2, T=4)
    inp = gpu_inputs(cfg)
    s = B.make_shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, P=cfg.E, dtype=dtype)
    arena = B.Arena(s)
    scales = (inp.Sg, inp.Su, inp.Sd) if cfg.quant_weights else None
    for e in range(cfg.E):
        g, u, dn = B.expert_slices(inp.Wg, inp.Wu, inp.Wd, scales, e)
        dev = torch.empty_like(arena.plane_gu[0])
        B.moe_pack_gate_up(s, g, u, dev, 1, 0, 0)
        host = torch.empty_like(dev, device="cpu")
        B.moe_pack_gate_up_host(s, g.cpu(), u.cpu(), host)
        dev_d = torch.empty_like(arena.plane_d[0])
        B.moe_pack_down(s, dn, dev_d, 1, 0, 0)
        host_d = torch.empty_like(dev_d, device="cpu")
        B.moe_pack_down_host(s, dn.cpu(), host_d)
        torch.cuda.synchronize()
        assert torch.equal(dev.cpu().view(torch.uint8), host.view(torch.uint8)), f"gate/up expert {e}"
        assert torch.equal(dev_d.cpu().view(torch.uint8), host_d.view(torch.uint8)), f"down expert {e}"
    arena.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16", "bf16_fp8w", "bf16_fp4w"])
def test_device_pack_many_experts_strided(dtype):
    say(f"packing 3 experts in one call, padded source strides ({dtype})")
    cfg = MID.with_(dtype=dtype, E=3, k=2, T=4)
    inp = gpu_inputs(cfg)
    s = B.make_shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, P=cfg.E, dtype=dtype)
    arena = B.Arena(s)
    scales = (inp.Sg, inp.Su, inp.Sd) if cfg.quant_weights else None
    sl = [B.expert_slices(inp.Wg, inp.Wu, inp.Wd, scales, e) for e in range(cfg.E)]
    pad = 16 if cfg.quant_weights else 64     # keeps every source slice 4-byte aligned

    def stack(parts):
        n = parts[0].numel()
        buf = torch.full((len(parts), n + pad), 7, dtype=parts[0].dtype, device="cuda")
        for e, p in enumerate(parts):
            buf[e, :n] = p.reshape(-1)
        return buf, n + pad

    g, sg = stack([x[0] for x in sl])
    u, _ = stack([x[1] for x in sl])
    dn, sd = stack([x[2] for x in sl])
    B.moe_pack_gate_up(s, g, u, arena.plane_gu, cfg.E, sg, arena.stride_gu)
    B.moe_pack_down(s, dn, arena.plane_d, cfg.E, sd, arena.stride_d)
    torch.cuda.synchronize()
    for e in range(cfg.E):
        host = torch.empty_like(arena.plane_gu[e], device="cpu")
        B.moe_pack_gate_up_host(s, sl[e][0].cpu(), sl[e][1].cpu(), host)
        host_d = torch.empty_like(arena.plane_d[e], device="cpu")
        B.moe_pack_down_host(s, sl[e][2].cpu(), host_d)
        assert torch.equal(arena.plane_gu[e].cpu().view(torch.uint8), host.view(torch.uint8)), f"gate/up {e}"
        assert torch.equal(arena.plane_d[e].cpu().view(torch.uint8), host_d.view(torch.uint8)), f"down {e}"
    arena.close()
