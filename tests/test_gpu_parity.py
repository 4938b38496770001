"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Router logits: within the error bound of the GPU router's fp32 evaluation
order of the oracle's correctly rounded logits (gpu_util.router_bound), and
bitwise run-to-run identical. Bit-exact on shared inputs: top-k ids from the
same logits, slot counts and offsets, records (rec_token, rec_route),
route_pos, n_valid. Whole layers (router on the GPU): ids bit-exact on every
token whose top-k no logit error within the bound can change; near ties
checked for a valid pick. Tolerance: route weights alpha (relative 1e-6 on
shared logits: expf and the softmax sum order differ; plus what the measured
logit difference moves them otherwise), layer output max|y - y_ref| /
max|y_ref| <= 1e-2 for bf16 layers and 1e-5 for the fp32 layer. Inputs are
the seeded synthetic workloads of inputs.py.
"""
import numpy as np
import pytest
import torch

from gpu_util import (OracleRun, TOL, check_descriptors, check_layer_output, check_logits,
                      check_routing_from_gpu_logits, check_y, check_topk, gpu_inputs, gpu_logits, np32, rel_err,
                      sample_tokens, say)
from oracle import oracle as oracle_mod
from routed_expert_ffn_top_amd import binding as B
from routed_expert_ffn_top_amd.inputs import CONFIGS, MoEConfig, make_inputs, make_logits, random_phi
from routed_expert_ffn_top_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

# a mid-size bf16 layer the oracle finishes in about a second: several tiles
# per slot and ragged tails (T*k = 2400 routes over 16 experts)
MID = MoEConfig(name="mid_bf16", index=9, T=300, d=512, f=384, E=16, k=8)
MID_SHARED = MoEConfig(name="mid_shared", index=10, T=200, d=256, f=192, E=12, k=3, n_shared=2,
                       renorm=False)


def _layer_out(layer: MoELayer, inp, logits=None):
    Y = inp.A.clone()
    layer.forward(Y, logits=logits)
    torch.cuda.synchronize()
    return Y


def test_mfma_lane_layout():
    say("mfma layout self-test")
    out = torch.zeros(1024, dtype=torch.float32, device="cuda")
    B.moe_selftest_mfma_layout(out)
    torch.cuda.synchronize()
    i = np.arange(32)[:, None]
    k = np.arange(16)[None, :]
    A = ((3 * i + 5 * k) % 7 - 3).astype(np.float64)
    kk = np.arange(16)[:, None]
    j = np.arange(32)[None, :]
    Bm = ((2 * kk + 7 * j) % 5 - 2).astype(np.float64)
    assert np.array_equal(out.cpu().numpy().reshape(32, 32), A @ Bm)


@pytest.mark.parametrize("name", ["tiny_fp32", "olmoe_t1024", "olmoe_t4096", "virt_olmoe_t256", "mixtral_t256"])
def test_router_logits_within_bound(name):
    """GPU logits within the bound of the oracle's correctly rounded ones, the
    same bits on a second call, and the top-k of the GPU logits equal to the
    oracle's wherever no logit error within the bound can change it."""
    cfg = CONFIGS[name]
    if name == "mixtral_t256":
        cfg = cfg.with_(T=96, f=64)  # router only: keep the expert weights small
    say("router", name)
    inp = gpu_inputs(cfg)
    s = B.make_shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.n_shared, dtype=cfg.dtype, renorm=cfg.renorm)
    L = torch.empty((cfg.T, cfg.E), dtype=torch.float32, device="cuda")
    Wr = inp.Wr.t().contiguous()
    B.moe_router_logits(s, inp.X, Wr, inp.bias, L)
    L2 = torch.empty_like(L)
    B.moe_router_logits(s, inp.X, Wr, inp.bias, L2)
    torch.cuda.synchronize()
    assert torch.equal(L.view(torch.int32), L2.view(torch.int32)), "router not run-to-run identical"
    orun = OracleRun(inp)
    Lg = L.cpu().numpy()
    routes = B.alloc_routes(s)
    ws = B.alloc_workspace(s)
    B.moe_route_build(s, 0, cfg.T, L, list(range(cfg.n_exp)), 0, routes, ws)
    torch.cuda.synchronize()
    check_routing_from_gpu_logits(routes, orun, Lg)


# (T, d, E, dtype, ldx): ragged token counts, d not a multiple of the 64-wide
# slab (fp32 only: bf16 layers need d % 64 == 0), E not a power of two, strided X, and each tokens-per-thread choice
ROUTER_SHAPES = [
    (333, 320, 20, "bf16", 328),
    (1000, 260, 60, "f32", 268),
    (45, 64, 1, "bf16", 72),
    (4100, 256, 64, "bf16", 256),
    (32768, 64, 8, "bf16", 64),
    (20000, 128, 8, "f32", 128),
    (700, 4, 3, "f32", 4),
    (1000, 256, 160, "bf16", 256),
    (130, 128, 256, "bf16", 128),
]


@pytest.mark.parametrize("T,d,E,dtype,ldx", ROUTER_SHAPES)
def test_router_logits_shapes_within_bound(T, d, E, dtype, ldx):
    say("router shape", T, d, E, dtype, ldx)
    cfg = MoEConfig(name="router_shape", index=77, T=T, d=d, f=64, E=E, k=1, dtype=dtype)
    inp = make_inputs(cfg, device="cpu")
    Xp = torch.zeros((T, ldx), dtype=inp.X.dtype)
    Xp[:, :d] = inp.X
    s = B.make_shape(T, d, 64, E, 1, dtype=dtype, ldx=ldx)
    L = torch.empty((T, E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, Xp.cuda(), inp.Wr.t().contiguous().cuda(), inp.bias.cuda() if inp.bias is not None
                        else None, L)
    torch.cuda.synchronize()
    check_logits(L.cpu().numpy(), OracleRun(inp))


ROUTE_CASES = {
    # (T, E, k, n_shared, renorm, P, absent, t0, nt, logit kind)
    "olmoe": (1024, 64, 8, 0, True, 64, 0, 0, 1024, "normal"),
    "dsv2": (4096, 64, 6, 2, False, 66, 0, 0, 4096, "normal"),
    "mixtral": (4096, 8, 2, 0, True, 8, 0, 0, 4096, "normal"),
    "ties": (777, 16, 4, 0, True, 16, 0, 0, 777, "ties"),
    "k_eq_E": (130, 8, 8, 0, True, 8, 0, 0, 130, "normal"),
    "k1": (257, 32, 1, 0, True, 32, 0, 0, 257, "normal"),
    "partial_phi": (1000, 64, 8, 0, True, 16, 48, 0, 1000, "normal"),
    "wide_P": (513, 20, 3, 1, True, 100, 0, 0, 513, "normal"),
    "range": (600, 64, 8, 0, True, 64, 0, 123, 200, "normal"),
    "one_token": (1, 64, 8, 0, True, 64, 0, 0, 1, "normal"),
    "many_blocks": (9000, 64, 8, 0, True, 64, 0, 0, 9000, "normal"),
    "zeros_nan": (300, 40, 5, 0, True, 40, 0, 0, 300, "zeros_nan"),
    "wide_E": (200, 200, 6, 0, False, 200, 0, 0, 200, "ties"),
    "skewed": (2048, 64, 8, 0, True, 64, 0, 0, 2048, "skewed"),
}


@pytest.mark.parametrize("case", list(ROUTE_CASES))
def test_route_build_bitexact(case):
    T, E, k, S, renorm, P, absent, t0, nt, kind = ROUTE_CASES[case]
    say("route build", case)
    L = make_logits(T, E, seed=100 + len(case))
    if kind == "ties":
        L = torch.round(L * 2) / 2      # many exactly equal logits
    if kind == "zeros_nan":
        L = torch.round(L)              # many ties, many exact zeros
        L[L == 0] = torch.where(torch.rand(int((L == 0).sum()), generator=torch.Generator().manual_seed(5)) < 0.5,
                                torch.tensor(-0.0), torch.tensor(0.0))
        L[::7, 3] = float("nan")        # NaN ranks as -infinity
    if kind == "skewed":
        L[:, 5] += 6.0                  # nearly every token picks expert 5
        L[:, 9] -= 30.0                 # expert 9 is never picked
    ne = E + S
    phi = list(range(ne)) if (P == ne and absent == 0) else random_phi(ne, P, seed=3, n_absent=absent).tolist()
    cap = max(1, nt * (k + S))
    s = B.make_shape(T, 64, 64, E, k, S, P=P, capacity=cap, dtype="bf16", renorm=renorm)
    routes = B.alloc_routes(s)
    ws = B.alloc_workspace(s)
    Ld = L.cuda()
    B.moe_route_build(s, t0, nt, Ld, phi, 0, routes, ws)
    torch.cuda.synchronize()
    from oracle import oracle as oracle_mod
    orc = oracle_mod.get()
    idx, alpha = orc.topk(L.numpy(), k, S, renorm)
    kp = k + S
    gi = routes["topk_idx"].cpu().numpy()[t0:t0 + nt]
    assert np.array_equal(gi, idx[t0:t0 + nt])
    gw = routes["topk_w"].cpu().numpy()[t0:t0 + nt].astype(np.float64)
    aref = alpha[t0:t0 + nt]
    assert np.max(np.abs(gw - aref) / np.maximum(aref, 1e-30)) <= 1e-6
    full_idx = routes["topk_idx"].cpu().numpy()
    ref = orc.route_map(full_idx, np.array(phi, dtype=np.int32), P, t0, nt,
                        route_pos=np.full(T * kp, -1, dtype=np.int32))
    check_descriptors(routes, ref)
    assert B.moe_device_errors(s, ws) == 0


def test_route_build_flags_bad_expert_ids():
    say("route build with an out-of-range supplied id")
    T, E, k = 64, 8, 2
    s = B.make_shape(T, 64, 64, E, k, dtype="bf16")
    routes = B.alloc_routes(s)
    ws = B.alloc_workspace(s)
    idx = torch.stack([torch.arange(T) % E, (torch.arange(T) + 1) % E], 1).to(torch.int32)
    idx[5, 1] = 99
    routes["topk_idx"].copy_(idx)
    B.moe_route_build(s, 0, T, None, list(range(E)), B.MOE_ROUTE_RESET, routes, ws)
    torch.cuda.synchronize()
    assert B.moe_device_errors(s, ws) == B.MOE_DEVERR_EXPERT_ID
    assert int(routes["slot_offset"][-1]) == T * k - 1
    assert int(routes["route_pos"][5 * k + 1]) == -1
    assert B.moe_device_errors(s, ws) == 0  # cleared


def _check_layer(cfg, tokens=None, simple=False, repeats=3, **layer_kw):
    """One layer against the oracle. The layer runs `repeats` times back to
    back with no host synchronisation between runs; every run must give the
    same bits (a missing wait inside a kernel shows up as run-to-run
    differences under load), and the output is checked against the oracle."""
    inp = gpu_inputs(cfg)
    layer = MoELayer(inp, **layer_kw)
    outs = []
    for _ in range(repeats):
        Y = inp.A.clone()
        if simple:
            _run_steps(layer, Y, simple=True)
        else:
            layer.forward(Y)
        outs.append(Y)
    torch.cuda.synchronize()
    for r, Yr in enumerate(outs[1:], 1):
        assert torch.equal(Yr.view(torch.int32), Y.view(torch.int32)), f"run {r} differs from the last run"
    err, ffn, _ = check_layer_output(layer, inp, Y, tokens=tokens)
    say(f"  {cfg.name}: rel err {err:.3e}, expert sum {ffn:.3e}")
    return Y, layer, inp


def _run_steps(layer: MoELayer, Y, simple=False):
    """The layer as separate calls: router, route build, expert FFN, combine."""
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    B.moe_route_build(s, 0, s.T, L, layer.phi, 0, layer.routes, layer.ws)
    flags = B.MOE_FFN_EXPERTS | B.MOE_FFN_FINALIZE | (B.MOE_FFN_SIMPLE_KERNEL if simple else 0)
    B.moe_expert_ffn(s, layer.X, Y, layer.routes, layer.arena, layer.phi, flags, layer.ws)


def test_layer_tiny_fp32():
    say("layer tiny fp32")
    _check_layer(CONFIGS["tiny_fp32"])


def test_layer_ragged_weight_blocks():
    """The tiled weight layout's short pieces: bf16 with d = 320 (the down
    slice's second 256-row block has 64 rows) and fp32 with d = 100 (the
    gate/up slice's last K piece is 4 wide, read by the plain kernel)."""
    say("layer, ragged weight blocks")
    _check_layer(MoEConfig(name="ragged_bf16", index=31, T=150, d=320, f=128, E=8, k=2))
    _check_layer(MoEConfig(name="ragged_fp32", index=32, T=50, d=100, f=96, E=6, k=2, dtype="f32"))


def test_layer_mid_bf16():
    say("layer mid bf16")
    _check_layer(MID)


def test_layer_mid_bf16_simple_kernel():
    say("layer mid bf16, plain kernel")
    _check_layer(MID, simple=True)


def test_layer_shared_experts():
    say("layer with shared experts")
    _check_layer(MID_SHARED)


def test_layer_olmoe_t1024():
    say("layer OLMoE T=1024")
    _check_layer(CONFIGS["olmoe_t1024"])


def test_layer_dsv2lite_t4096():
    say("layer DSV2-Lite T=4096, every token")
    cfg = CONFIGS["dsv2lite_t4096"]
    _check_layer(cfg)


def test_layer_olmoe_t4096():
    say("layer OLMoE T=4096, every token")
    cfg = CONFIGS["olmoe_t4096"]
    _check_layer(cfg)


def test_layer_olmoe_large_T():
    """The OLMoE-shaped layer at T = 65536: 524288 routes, so per-route rows sit
    past 2^31 bytes into Yr and every offset into it needs 64 bits. Routing and
    descriptors are checked for every token, outputs on 96 sampled tokens."""
    cfg = CONFIGS["olmoe_t4096"].with_(name="olmoe_t65536", T=65536)
    say("layer OLMoE T=65536 (Yr past 2^31 bytes), routing of every token, 96 sampled outputs")
    inp = gpu_inputs(cfg)
    layer = MoELayer(inp)
    Y = inp.A.clone()
    layer.forward(Y)
    torch.cuda.synchronize()
    err, ffn, _ = check_layer_output(layer, inp, Y, tokens=sample_tokens(cfg.T, 96))
    say(f"  rel err {err:.3e}, expert sum {ffn:.3e}")


def test_layer_mixtral_t4096():
    say("layer Mixtral T=4096 (4 row blocks per expert), every token")
    _check_layer(CONFIGS["mixtral_t4096"], repeats=2)


def test_layer_mixtral_t1024():
    say("layer Mixtral T=1024 (one row block per expert, split-K down), every token")
    _check_layer(CONFIGS["mixtral_t1024"], repeats=2)


def test_layer_mixtral_t256():
    say("layer Mixtral T=256, every token")
    cfg = CONFIGS["mixtral_t256"]
    _check_layer(cfg)


def test_deterministic_and_phi_independent():
    say("determinism, capacity split, phi permutation")
    inp = gpu_inputs(MID)
    base = MoELayer(inp)
    y1 = _layer_out(base, inp)
    y2 = _layer_out(base, inp)
    assert torch.equal(y1, y2), "run-to-run difference"
    kp = MID.kp
    split = MoELayer(inp, capacity=(MID.T * kp) // 3 + 5)
    assert torch.equal(_layer_out(split, inp), y1), "capacity split changed the output"
    perm = random_phi(MID.n_exp, MID.n_exp + 7, seed=11).tolist()
    moved = MoELayer(inp, phi=perm, P=MID.n_exp + 7)
    assert torch.equal(_layer_out(moved, inp), y1), "a different placement changed the output"


def test_two_layers_concurrently_on_two_streams():
    """Two independent layers (each with its own inputs, arena, descriptors
    and workspace) enqueued alternately on two streams, four times each with
    no synchronisation in between, give the bits each gives alone: a call
    keeps no state outside the caller's buffers and its own arena."""
    say("two layers on two streams")
    cfgs = [MID, MID_SHARED]
    layers, inps, ref = [], [], []
    for cfg in cfgs:
        inp = gpu_inputs(cfg)
        layer = MoELayer(inp)
        layers.append(layer)
        inps.append(inp)
        ref.append(_layer_out(layer, inp))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for _ in range(4):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                Y = inps[i].A.clone()
                layers[i].forward(Y, compute=streams[i])
                outs[i].append(Y)
    torch.cuda.synchronize()
    for i in range(2):
        for r, Y in enumerate(outs[i]):
            assert torch.equal(Y.view(torch.int32), ref[i].view(torch.int32)), f"layer {i} run {r} differs"


def test_partial_phi_leaves_out_absent_experts():
    say("partial placement map")
    inp = gpu_inputs(MID)
    layer = MoELayer(inp)
    s = layer.shape
    phi = list(range(MID.n_exp))
    for e in (1, 4, 9):
        phi[e] = -1
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    B.moe_route_build(s, 0, s.T, L, phi, 0, layer.routes, layer.ws)
    Y = inp.A.clone()
    B.moe_expert_ffn(s, layer.X, Y, layer.routes, layer.arena, phi,
                     B.MOE_FFN_EXPERTS | B.MOE_FFN_FINALIZE, layer.ws)
    torch.cuda.synchronize()
    orun = OracleRun(inp)
    same = check_routing_from_gpu_logits(layer.routes, orun, L.cpu().numpy())
    assert same.all(), "near-tie picks: the partial map's records would differ"
    mask = np.isin(orun.idx, [1, 4, 9], invert=True).reshape(-1).astype(np.uint8)
    ref = orun.route_map(phi, s.P)
    check_descriptors(layer.routes, ref)
    check_y(np32(Y), orun.Y(route_mask=mask), np32(inp.A), "bf16")


def test_paged_equals_resident():
    say("paged layer (P=16, G=8) vs resident")
    cfg = CONFIGS["virt_olmoe_t512"]
    inp = gpu_inputs(cfg)
    res = MoELayer(inp)                 # all 64 experts resident
    y_res = _layer_out(res, inp)
    res.close()
    paged = MoELayer(inp, paged=True)   # P = 16 slots, banks of 8
    copy = torch.cuda.Stream()
    Y = inp.A.clone()
    paged.forward(Y, copy=copy)
    torch.cuda.synchronize()
    assert torch.equal(Y, y_res), "paging changed the output"
    y2 = inp.A.clone()
    paged.forward(y2, copy=copy)        # the arena is reused by a second call
    torch.cuda.synchronize()
    assert torch.equal(y2, y_res)
    counts = np.bincount(paged.routes["topk_idx"].cpu().numpy().reshape(-1), minlength=cfg.E)
    say(f"  experts with no routes: {int((counts == 0).sum())}")
    check_layer_output(paged, inp, Y)


def test_edge_shapes():
    say("edge shapes")
    for T in (1, 77):
        _check_layer(MID.with_(T=T, name=f"mid_T{T}"))
    # an empty prompt is a no-op
    cfg = MID.with_(T=0, name="mid_T0")
    inp = make_inputs(MID.with_(T=0), device="cuda")
    layer = MoELayer(inp)
    Y = inp.A.clone()
    layer.forward(Y)
    torch.cuda.synchronize()
    assert Y.shape == (0, MID.d)


# The largest expert table the library takes: 256 routed experts plus 2 shared
# ones (E <= 256, E + shared <= 512), placed at random into 512 physical slots
# (the expert kernels keep at most 512 slot entries on chip), top-8 over a few
# hundred tokens, so that most slots hold one small row block.
MAX_EXP = MoEConfig(name="max_experts", index=81, T=400, d=128, f=128, E=256, k=8, n_shared=2, renorm=False)


@pytest.mark.parametrize("dtype", ["bf16", "bf16_fp8w", "bf16_fp4w"])
def test_layer_max_experts_and_slots(dtype):
    cfg = MAX_EXP.with_(dtype=dtype, name=f"max_experts_{dtype}")
    say(f"largest expert table: {cfg.E} + {cfg.n_shared} experts in 512 slots ({dtype})")
    phi = random_phi(cfg.n_exp, 512, seed=17).tolist()
    _, layer, _ = _check_layer(cfg, phi=phi, P=512)
    counts = layer.routes["slot_count"].cpu().numpy()
    assert counts.shape == (512,) and int((counts > 0).sum()) > 200


@pytest.mark.parametrize("cfg,padx,pady", [(MID, 72, 36), (CONFIGS["tiny_fp32"], 12, 4)], ids=["bf16", "fp32"])
def test_layer_row_strides(cfg, padx, pady):
    """X and Y with row strides wider than d: the same bits as the contiguous
    layer, and Y's padding columns untouched."""
    say(f"layer with row strides ldx = d + {padx}, ldy = d + {pady} ({cfg.name})")
    inp = gpu_inputs(cfg)
    layer = MoELayer(inp)
    y_ref = _layer_out(layer, inp)
    d = cfg.d
    s2 = B.make_shape(cfg.T, d, cfg.f, cfg.E, cfg.k, cfg.n_shared, P=layer.shape.P, dtype=cfg.dtype,
                      renorm=cfg.renorm, ldx=d + padx, ldy=d + pady)
    Xp = torch.full((cfg.T, d + padx), 1000.0, dtype=inp.X.dtype, device="cuda")   # read by mistake: wrong y
    Xp[:, :d] = inp.X
    Yp = torch.full((cfg.T, d + pady), 123.0, dtype=torch.float32, device="cuda")
    Yp[:, :d] = inp.A
    B.moe_layer_prefill(s2, Xp, layer.Wr, layer.bias, None, Yp, layer.arena, None, None,
                        B.alloc_routes(s2), B.alloc_workspace(s2))
    torch.cuda.synchronize()
    assert torch.equal(Yp[:, :d], y_ref), "strided layer differs from the contiguous one"
    assert bool((Yp[:, d:] == 123.0).all()), "padding columns of Y were written"


def test_layer_with_given_logits():
    """moe_layer_prefill with router logits passed in (no W_r): top-k ids,
    route weights and output against the oracle on the same logits."""
    say("layer with given logits")
    inp = gpu_inputs(MID_SHARED)
    layer = MoELayer(inp)
    L = make_logits(MID_SHARED.T, MID_SHARED.E, seed=3, scale=2.0, device="cuda")
    Y = _layer_out(layer, inp, logits=L)
    orun = OracleRun(inp, logits=L.cpu().numpy())
    check_topk(layer.routes, orun)
    err, ffn = check_y(np32(Y), orun.Y(), np32(inp.A), MID_SHARED.dtype)
    say(f"  rel err {err:.3e}, expert sum {ffn:.3e}")
