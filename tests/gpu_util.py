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
    idx = routes["topk_idx"].cpu().numpy()
    assert np.array_equal(idx, orun.idx), "top-k ids differ"
    w = routes["topk_w"].cpu().numpy().astype(np.float64)
    rel = np.max(np.abs(w - orun.alpha) / np.maximum(np.abs(orun.alpha), 1e-30))
    assert rel <= ALPHA_TOL, f"alpha rel err {rel}"


def sample_tokens(T: int, n: int, seed: int = 7) -> np.ndarray:
    if n >= T:
        return np.arange(T, dtype=np.int64)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick), dtype=np.int64)
