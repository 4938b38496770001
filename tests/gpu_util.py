"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import oracle as oracle_mod
from routed_expert_ffn_top_amd import binding as B
from routed_expert_ffn_top_amd.inputs import LayerInputs, MoEConfig, make_inputs

TOL = {"bf16": 1e-2, "f32": 1e-5, "bf16_fp8w": 1e-2, "bf16_fp4w": 1e-2}
# The same measure on the FFN part alone, y - A: in the parity inputs the
# residual A ~ N(0,1) dominates max|y|, so the measure on y alone would let a
# large error of the expert sum pass. fp32: twice the accumulation bound
# (d + f + 8) * 2^-24 of the tiny layer.
TOL_FFN = {"bf16": 1e-2, "f32": 5e-5, "bf16_fp8w": 1e-2, "bf16_fp4w": 1e-2}
ALPHA_TOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(y.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def check_y(y: np.ndarray, ref: np.ndarray, A: np.ndarray, dtype: str):
    """Layer output y against the oracle's ref, both holding the residual A:
    max|y - ref| / max|ref| <= TOL and, on the expert sum alone,
    max|(y - A) - (ref - A)| / max|ref - A| <= TOL_FFN. Returns both."""
    y = y.astype(np.float64)
    A = A.astype(np.float64)
    full = rel_err(y, ref)
    ffn = float(np.max(np.abs((y - A) - (ref - A))) / max(np.max(np.abs(ref - A)), 1e-300))
    assert full <= TOL[dtype], f"rel err {full}"
    assert ffn <= TOL_FFN[dtype], f"rel err of the expert sum {ffn}"
    return full, ffn


def gpu_inputs(cfg: MoEConfig, layer=0) -> LayerInputs:
    return make_inputs(cfg, layer=layer, device="cuda")


class OracleRun:
    """Oracle results for one layer's inputs (weights widened to fp32)."""

    def __init__(self, inp: LayerInputs, logits=None):
        self.cfg = cfg = inp.cfg
        self.orc = oracle_mod.get()
        self.X = np32(inp.X)
        self.Wr = np32(inp.Wr)
        self.bias = None if inp.bias is None else np32(inp.bias)
        self.A = np32(inp.A)
        self.L = self.orc.router_logits(self.X, self.Wr, self.bias) if logits is None else logits
        self.idx, self.alpha = self.orc.topk(self.L, cfg.k, cfg.n_shared, cfg.renorm)
        self._w = None
        self._inp = inp

    def weights(self):
        """Weights as the oracle takes them; fp8 codes are decoded by the
        oracle itself and come with their row scales; MXFP4 codes and block
        scales are decoded by the oracle to plain weights."""
        if self._w is None:
            inp = self._inp
            if self.cfg.fp8_weights:
                dec = lambda q: self.orc.fp8e4m3_decode(q.cpu().numpy())
                self._w = (dec(inp.Wg), dec(inp.Wu), dec(inp.Wd))
                self._scales = (np32(inp.Sg), np32(inp.Su), np32(inp.Sd))
            elif self.cfg.fp4_weights:
                dec = lambda q, s: self.orc.mxfp4_decode(q.cpu().numpy(), s.cpu().numpy())
                self._w = (dec(inp.Wg, inp.Sg), dec(inp.Wu, inp.Su), dec(inp.Wd, inp.Sd))
                self._scales = None
            else:
                self._w = (np32(inp.Wg), np32(inp.Wu), np32(inp.Wd))
                self._scales = None
        return self._w

    def route_map(self, phi, P, t0=0, nt=None):
        return self.orc.route_map(self.idx, np.asarray(phi, dtype=np.int32), P, t0, nt)

    def Y(self, tokens=None, route_mask=None):
        Wg, Wu, Wd = self.weights()
        return self.orc.expert_ffn(self.X, self.idx, self.alpha, Wg, Wu, Wd, self.A,
                                   tokens=tokens, route_mask=route_mask, scales=self._scales)


def check_descriptors(routes: dict, ref: dict, n_valid_expected=None):
    cnt = routes["slot_count"].cpu().numpy()
    off = routes["slot_offset"].cpu().numpy()
    assert np.array_equal(cnt, ref["count"]), "slot_count differs"
    assert np.array_equal(off, ref["offset"]), "slot_offset differs"
    n = int(off[-1])
    assert n == ref["n_valid"]
    if n_valid_expected is not None:
        assert n == n_valid_expected
    assert np.array_equal(routes["rec_token"][:n].cpu().numpy(), ref["rec_token"]), "rec_token differs"
    assert np.array_equal(routes["rec_route"][:n].cpu().numpy(), ref["rec_route"]), "rec_route differs"
    assert np.array_equal(routes["route_pos"].cpu().numpy(), ref["route_pos"]), "route_pos differs"


def check_topk(routes: dict, orun: OracleRun):
    """Top-k ids and weights computed from the same logits on both sides
    (logits passed in, not computed by the GPU router): ids bit-exact,
    weights within ALPHA_TOL."""
    idx = routes["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, orun.idx), "top-k ids differ"
    w = routes["topk_w"].cpu().numpy().astype(np.float64)
    rel = np.max(np.abs(w - orun.alpha) / np.maximum(np.abs(orun.alpha), 1e-30))
    assert rel <= ALPHA_TOL, f"alpha rel err {rel}"


# ---------------------------------------------------------------------------
# GPU router logits against the oracle's.
#
# The oracle's logit is the definition: the exact dot product plus the bias,
# rounded once to fp32 (its fp64 sum adds at most (d + 1) 2^-53 sum|x w|).
# The GPU router evaluates the same sum in fp32 in the fixed order its C ABI
# documents: runs of 8 hidden indices, run r feeding partial sum r mod 16,
# each partial sum a chain of m = 8 ceil(d / 128) fused multiply-adds, then 15
# additions of the partial sums and one of the bias. Each of those n = m + 16
# steps rounds once, so (Higham, recursive summation)
#   |L_gpu - exact| <= gamma_n (sum|x w| + |b|),  gamma_n = n u / (1 - n u),
# and |L_gpu - L_oracle| is bounded by that plus the oracle's own rounding.
U32 = 2.0 ** -24


def router_bound(X: np.ndarray, Wr: np.ndarray, bias, L_ref: np.ndarray) -> np.ndarray:
    """Per-logit bound on |L_gpu - L_oracle|. X [T][d], Wr [d][E] (fp32 values)."""
    d = X.shape[1]
    n = 8 * ((d + 127) // 128) + 16
    gamma = n * U32 / (1 - n * U32)
    absdot = np.abs(X.astype(np.float64)) @ np.abs(Wr.astype(np.float64))
    if bias is not None:
        absdot = absdot + np.abs(bias.astype(np.float64))[None, :]
    return gamma * absdot + U32 * np.abs(L_ref.astype(np.float64)) + (d + 1) * 2.0 ** -53 * absdot + 2.0 ** -140


def gpu_logits(layer) -> np.ndarray:
    """The GPU router's logits for a layer's X and W_r (moe_router_logits:
    the same kernel and arguments as the layer's own router step)."""
    s = layer.shape
    L = torch.empty((s.T, s.E), dtype=torch.float32, device="cuda")
    B.moe_router_logits(s, layer.X, layer.Wr, layer.bias, L)
    torch.cuda.synchronize()
    return L.cpu().numpy()


def check_logits(L_gpu: np.ndarray, orun: OracleRun) -> np.ndarray:
    """|L_gpu - L_oracle| within router_bound everywhere; returns the bound."""
    bound = router_bound(orun.X, orun.Wr, orun.bias, orun.L)
    diff = np.abs(L_gpu.astype(np.float64) - orun.L.astype(np.float64))
    assert np.all(np.isfinite(L_gpu)), "non-finite GPU logit"
    assert np.all(diff <= bound), f"logit outside its bound: max diff/bound {np.max(diff / bound):.3g}"
    return bound


def _decided(L: np.ndarray, bound: np.ndarray, k: int) -> np.ndarray:
    """Tokens whose oracle top-k (ids and their order) no logit error within
    the bound can change: each of the first k + 1 values in descending order
    exceeds the next by more than the two values' bounds."""
    T, E = L.shape
    Lk = np.where(np.isnan(L), -np.inf, L).astype(np.float64)
    order = np.lexsort((np.tile(np.arange(E), (T, 1)), -Lk), axis=1)[:, :min(k + 1, E)]
    v = np.take_along_axis(Lk, order, 1)
    b = np.take_along_axis(bound, order, 1)
    gaps = v[:, :-1] - v[:, 1:]
    if gaps.shape[1] == 0:
        return np.ones(T, dtype=bool)
    return np.all(gaps > b[:, :-1] + b[:, 1:], axis=1)


def check_routing_from_gpu_logits(routes: dict, orun: OracleRun, L_gpu: np.ndarray) -> np.ndarray:
    """Top-k of a layer whose router ran on the GPU, against the oracle's
    top-k on the oracle's logits.
      - the GPU logits lie within router_bound of the oracle's;
      - decided tokens (_decided) have bit-exact ids;
      - every other token (a near tie) has a valid choice: each GPU pick e_j
        could be the largest of the experts not yet picked under some logit
        errors within the bound, L[e_j] + b[e_j] >= L[e] - b[e];
      - route weights, where the ids agree, within ALPHA_TOL plus what the
        measured logit difference moves a softmax weight: |d ln alpha| <=
        2 max_e |L_gpu - L_oracle| over the token's logits.
    Returns a mask of the tokens whose ids agree with the oracle's."""
    cfg = orun.cfg
    k = cfg.k
    bound = check_logits(L_gpu, orun)
    idx = routes["topk_idx"].cpu().numpy()
    decided = _decided(orun.L, bound, k)
    same = np.all(idx == orun.idx, axis=1)
    assert np.all(same[decided]), f"{int((~same[decided]).sum())} decided tokens pick other experts"
    Lk = np.where(np.isnan(orun.L), -np.inf, orun.L).astype(np.float64)
    for t in np.nonzero(~decided)[0]:
        left = np.ones(cfg.E, dtype=bool)
        for j in range(k):
            e = idx[t, j]
            assert 0 <= e < cfg.E and left[e], f"token {t}: invalid pick {e}"
            left[e] = False
            if left.any():
                assert Lk[t, e] + bound[t, e] >= np.max(Lk[t, left] - bound[t, left]), f"token {t} rank {j}"
        assert np.array_equal(idx[t, k:], orun.idx[t, k:]), f"token {t}: shared ranks"
    delta = np.max(np.abs(L_gpu.astype(np.float64) - orun.L.astype(np.float64)), axis=1)
    w = routes["topk_w"].cpu().numpy().astype(np.float64)
    rel = np.abs(w - orun.alpha) / np.maximum(np.abs(orun.alpha), 1e-30)
    tol = ALPHA_TOL + 2.0001 * delta[:, None]
    assert np.all(rel[same] <= tol[same]), f"alpha outside tolerance: max rel {np.max(rel[same]):.3g}"
    say(f"  routing: {int((~decided).sum())} near-tie tokens of {len(idx)}, {int((~same).sum())} with "
        f"other picks; max|dL| {np.max(delta):.3g}, max|dL|/bound {np.max(np.abs(L_gpu - orun.L) / bound):.3g}")
    return same


def check_layer_output(layer, inp: LayerInputs, Y: torch.Tensor, tokens=None, orun=None,
                       descriptors=True):
    """A layer run whose router ran on the GPU, against the oracle: routing by
    check_routing_from_gpu_logits, the route map bit-exact (when the build
    covered every route and no token picked other experts), and the output on
    the requested tokens whose picks agree with the oracle's (every token, at
    these seeds) within the dtype's tolerance. Returns (rel err, expert-sum
    rel err, oracle run)."""
    cfg = inp.cfg
    orun = OracleRun(inp) if orun is None else orun
    same = check_routing_from_gpu_logits(layer.routes, orun, gpu_logits(layer))
    if descriptors and same.all() and layer.shape.capacity >= cfg.T * cfg.kp and not layer.paged:
        ref = orun.route_map(layer.phi, layer.shape.P)
        check_descriptors(layer.routes, ref, n_valid_expected=cfg.T * cfg.kp)
    toks = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    toks = toks[same[toks]]
    err, ffn = check_y(np32(Y)[toks], orun.Y(tokens=toks), np32(inp.A)[toks], cfg.dtype)
    return err, ffn, orun


def sample_tokens(T: int, n: int, seed: int = 7) -> np.ndarray:
    if n >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), dtype=np.int64)
