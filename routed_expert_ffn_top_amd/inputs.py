"""Seeded synthetic inputs for the routed-expert MoE layer workloads.

This module is the only code that both the HIP path and the CPU oracle use.
It draws random tensors and nothing else: no step of the layer's arithmetic
(router, top-k, descriptors, projections, combine) lives here.

Workloads (shapes of the EStream evaluation models; the pages' C4 prompts and
trained checkpoints are replaced by random data of the same shape):

* ``tiny_fp32``      T=64, d=128, E=8, k=2, f=256, fp32, renormalised top-2.
* ``olmoe``          OLMoE-1B-7B-shaped layer: d=2048, E=64, k=8, f=1024, bf16,
                     renormalised top-8 (T=1024 by default, also T=4096).
* ``dsv2lite``       DeepSeek-V2-Lite-shaped layer: d=2048, 64 routed experts,
                     top-6 not renormalised, plus 2 always-on shared experts,
                     f=1408, bf16, T=4096.
* ``mixtral``        Mixtral-8x7B-shaped layer: d=4096, E=8, k=2, f=14336,
                     bf16, renormalised top-2, T in {256, 1024, 4096}.
* ``virt_olmoe``     the OLMoE shape with a Zipf(1.1) popularity bias on the
                     router logits and a P=16 slot arena (expert paging).

Distributions: X ~ N(0,1); W_gate, W_up, W_down, W_router ~ N(0, 0.02^2)
(0.02 is the standard deviation); residual A ~ N(0,1) for parity runs and 0
for timed runs. Values are drawn in fp32 from a seeded torch generator and,
for bf16 workloads, rounded to bf16 (round to nearest even) so that the GPU
and the oracle see exactly the same numbers. The router weight stays fp32.

Weight layout is nn.Linear style ([out, in]): W_gate, W_up [n_exp, f, d],
W_down [n_exp, d, f], with n_exp = E + n_shared (shared experts last).

Weight-only quantised workloads (dtype ``bf16_fp8w``, names ending in
``_fp8w``): the same fp32 weight draws are stored per output row as fp8 e4m3
codes and one fp32 scale, scale = max|row| / 448 (the largest e4m3 value),
codes = row / scale rounded to nearest even by PyTorch's float8_e4m3fn
conversion. The quantised model is then the model under test: both sides get
the codes and the scales.

MXFP4 workloads (dtype ``bf16_fp4w``, names ending in ``_fp4w``): the same
fp32 weight draws in the OCP microscaling format, per row and block of 32
weights along the input dimension: shared exponent
s = floor(log2(max|block|)) - 2 (2 is the exponent of 6, the largest E2M1
value), clamped to [-127, 127] and stored as the byte s + 127; each weight
w / 2^s rounded to the nearest E2M1 value (ties to the even code), values
beyond 6 saturated to 6; an all-zero block gets s = -127. Codes are stored
two per byte, element 2i in the low nibble.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

STD_W = 0.02
ZIPF_S = 1.1


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    d: int
    E: int
    k: int
    f: int
    n_shared: int = 0
    dtype: str = "bf16"          # "bf16", "f32" (X, expert weights, H), "bf16_fp8w"
                                 # (bf16 X and H, fp8 e4m3 weights with row scales)
                                 # or "bf16_fp4w" (bf16 X and H, MXFP4 weights)
    renorm: bool = True          # renormalise the top-k softmax weights
    zipf: bool = False           # Zipf(1.1) popularity bias on the logits
    P: Optional[int] = None      # arena slots (None: one slot per expert)
    G: int = 8                   # slots per bank when paging
    index: int = 0               # workload number used in the seed

    @property
    def n_exp(self) -> int:
        return self.E + self.n_shared

    @property
    def kp(self) -> int:
        """Routes per token: k routed plus the shared experts."""
        return self.k + self.n_shared

    @property
    def slots(self) -> int:
        return self.P if self.P is not None else self.n_exp

    @property
    def torch_dtype(self) -> torch.dtype:
        """Element type of the activations (and of unquantised weights)."""
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def fp8_weights(self) -> bool:
        return self.dtype == "bf16_fp8w"

    @property
    def fp4_weights(self) -> bool:
        return self.dtype == "bf16_fp4w"

    @property
    def quant_weights(self) -> bool:
        """Weights stored as codes plus scales (fp8 rows or MXFP4 blocks)."""
        return self.fp8_weights or self.fp4_weights

    def with_(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)

    def flops(self) -> int:
        """Algorithmic expert FLOPs: 6*d*f per route (gate+up 4df, down 2df)."""
        return 6 * self.T * self.kp * self.d * self.f

    def router_flops(self) -> int:
        return 2 * self.T * self.d * self.E


def _cfg(name, index, **kw) -> MoEConfig:
    return MoEConfig(name=name, index=index, **kw)


CONFIGS = {
    "tiny_fp32": _cfg("tiny_fp32", 1, T=64, d=128, E=8, k=2, f=256, dtype="f32"),
    "olmoe_t1024": _cfg("olmoe_t1024", 2, T=1024, d=2048, E=64, k=8, f=1024),
    "olmoe_t4096": _cfg("olmoe_t4096", 2, T=4096, d=2048, E=64, k=8, f=1024),
    "dsv2lite_t4096": _cfg("dsv2lite_t4096", 3, T=4096, d=2048, E=64, k=6,
                           f=1408, n_shared=2, renorm=False),
    "mixtral_t256": _cfg("mixtral_t256", 4, T=256, d=4096, E=8, k=2, f=14336),
    "mixtral_t1024": _cfg("mixtral_t1024", 4, T=1024, d=4096, E=8, k=2, f=14336),
    "mixtral_t4096": _cfg("mixtral_t4096", 4, T=4096, d=4096, E=8, k=2, f=14336),
}
for _t in (256, 512, 1024, 2048, 4096):
    CONFIGS[f"virt_olmoe_t{_t}"] = _cfg(f"virt_olmoe_t{_t}", 5, T=_t, d=2048,
                                        E=64, k=8, f=1024, zipf=True, P=16, G=8)
# the same workloads with fp8 e4m3 weights (same seeds: same X, router and
# weight draws before quantisation)
for _n in ("olmoe_t1024", "olmoe_t4096", "dsv2lite_t4096", "mixtral_t256", "mixtral_t1024",
           "mixtral_t4096", "virt_olmoe_t256", "virt_olmoe_t1024", "virt_olmoe_t4096"):
    CONFIGS[_n + "_fp8w"] = CONFIGS[_n].with_(name=_n + "_fp8w", dtype="bf16_fp8w")
    CONFIGS[_n + "_fp4w"] = CONFIGS[_n].with_(name=_n + "_fp4w", dtype="bf16_fp4w")


def seed_for(cfg: MoEConfig, layer: int = 0) -> int:
    return 1000 * cfg.index + layer


@dataclasses.dataclass
class LayerInputs:
    cfg: MoEConfig
    X: torch.Tensor               # [T, d]        cfg dtype
    Wr: torch.Tensor              # [d, E]        fp32
    bias: Optional[torch.Tensor]  # [E]           fp32 (Zipf workloads) or None
    Wg: torch.Tensor              # [n_exp, f, d] cfg dtype
    Wu: torch.Tensor              # [n_exp, f, d] cfg dtype
    Wd: torch.Tensor              # [n_exp, d, f] cfg dtype
    A: torch.Tensor               # [T, d]        fp32 residual
    # fp8 weights: Wg, Wu, Wd hold e4m3 codes (uint8) and these the row scales
    # MXFP4: Wg, Wu [n_exp, f, d/2], Wd [n_exp, d, f/2] hold packed E2M1 codes
    # (uint8) and these the E8M0 block scale bytes (uint8 [..., rows, K/32])
    Sg: Optional[torch.Tensor] = None   # [n_exp, f] fp32
    Su: Optional[torch.Tensor] = None   # [n_exp, f] fp32
    Sd: Optional[torch.Tensor] = None   # [n_exp, d] fp32

    def to(self, device) -> "LayerInputs":
        mv = lambda t: None if t is None else t.to(device)
        return LayerInputs(self.cfg, mv(self.X), mv(self.Wr), mv(self.bias),
                           mv(self.Wg), mv(self.Wu), mv(self.Wd), mv(self.A),
                           mv(self.Sg), mv(self.Su), mv(self.Sd))


E4M3_MAX = 448.0


def quantize_rows_e4m3(W: torch.Tensor):
    """Per-row fp8 e4m3 storage of W [..., rows, cols] (fp32): returns
    (codes uint8 [..., rows, cols], scales fp32 [..., rows]) with
    scale = max|row| / 448 (1 for an all-zero row) and codes the e4m3
    encoding of row / scale (round to nearest even)."""
    amax = W.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = (W / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale


# E2M1 magnitudes by code (bit 3 is the sign)
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def quantize_mxfp4(W: torch.Tensor):
    """MXFP4 storage of W [..., rows, K] (fp32, K a multiple of 32): returns
    (codes uint8 [..., rows, K/2], two E2M1 codes per byte with element 2i in
    the low nibble; scales uint8 [..., rows, K/32], E8M0 bytes)."""
    *lead, rows, K = W.shape
    Wb = W.reshape(*lead, rows, K // 32, 32).to(torch.float32)
    amax = Wb.abs().amax(dim=-1)
    # floor(log2 amax) exactly: frexp gives amax = m * 2^e with m in [0.5, 1)
    _, e = torch.frexp(amax)
    s = torch.where(amax > 0, e.to(torch.int32) - 1 - 2, torch.full_like(e, -127, dtype=torch.int32))
    s = s.clamp(-127, 127)
    v = (Wb / torch.ldexp(torch.ones_like(amax), s.to(torch.float32)).unsqueeze(-1)).abs()
    # nearest E2M1 magnitude: bucketize against the midpoints between
    # neighbouring values (a value on a midpoint lands on the lower one), then
    # move midpoint ties from an odd code to the even code above; beyond 6
    # saturates at code 7
    mids = torch.tensor([(a + b) / 2 for a, b in zip(E2M1_VALUES, E2M1_VALUES[1:])],
                        dtype=torch.float32, device=W.device)
    mag = torch.bucketize(v, mids)
    tie = (mag < 7) & (v == mids[mag.clamp(max=6)])
    mag = torch.where(tie & (mag % 2 == 1), mag + 1, mag)
    sign = (Wb < 0) & (mag > 0)
    code = (mag + 8 * sign.to(mag.dtype)).to(torch.uint8).reshape(*lead, rows, K)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return packed.contiguous(), (s + 127).to(torch.uint8).contiguous()


def _normal(gen, shape, std, device):
    t = torch.empty(shape, dtype=torch.float32, device=device)
    t.normal_(0.0, std, generator=gen)
    return t


def zipf_bias(cfg: MoEConfig, gen: torch.Generator, device) -> torch.Tensor:
    """Log-popularity bias: p_e proportional to rank_e^(-1.1), rank = 1 + a
    seeded permutation of the expert ids; returns ln p_e as fp32."""
    perm = torch.randperm(cfg.E, generator=gen, device=device)
    rank = (perm + 1).to(torch.float64)
    w = rank.pow(-ZIPF_S)
    return torch.log(w / w.sum()).to(torch.float32)


def make_inputs(cfg: MoEConfig, layer: int = 0, device="cpu",
                residual: bool = True, seed: Optional[int] = None) -> LayerInputs:
    """Draw one layer's inputs. Same (cfg, layer, device) -> same values."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_for(cfg, layer) if seed is None else seed)
    dt = cfg.torch_dtype
    X = _normal(gen, (cfg.T, cfg.d), 1.0, device).to(dt)
    Wr = _normal(gen, (cfg.d, cfg.E), STD_W, device)
    ne = cfg.n_exp
    Wg = _normal(gen, (ne, cfg.f, cfg.d), STD_W, device)
    Wu = _normal(gen, (ne, cfg.f, cfg.d), STD_W, device)
    Wd = _normal(gen, (ne, cfg.d, cfg.f), STD_W, device)
    Sg = Su = Sd = None
    if cfg.fp8_weights:
        (Wg, Sg), (Wu, Su), (Wd, Sd) = (quantize_rows_e4m3(w) for w in (Wg, Wu, Wd))
    elif cfg.fp4_weights:
        (Wg, Sg), (Wu, Su), (Wd, Sd) = (quantize_mxfp4(w) for w in (Wg, Wu, Wd))
    else:
        Wg, Wu, Wd = Wg.to(dt), Wu.to(dt), Wd.to(dt)
    if residual:
        A = _normal(gen, (cfg.T, cfg.d), 1.0, device)
    else:
        A = torch.zeros((cfg.T, cfg.d), dtype=torch.float32, device=device)
    bias = zipf_bias(cfg, gen, device) if cfg.zipf else None
    return LayerInputs(cfg, X, Wr, bias, Wg, Wu, Wd, A, Sg, Su, Sd)


def make_logits(T: int, E: int, seed: int, scale: float = 1.0,
                device="cpu") -> torch.Tensor:
    """Random fp32 router logits for tests that pass logits in directly."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return _normal(gen, (T, E), scale, torch.device(device))


def identity_phi(n_exp: int) -> torch.Tensor:
    return torch.arange(n_exp, dtype=torch.int32)


def random_phi(n_exp: int, P: int, seed: int, n_absent: int = 0) -> torch.Tensor:
    """A random injective placement map: n_exp - n_absent experts get distinct
    slots in [0, P); the rest are absent (-1)."""
    gen = torch.Generator().manual_seed(seed)
    assert n_exp - n_absent <= P
    experts = torch.randperm(n_exp, generator=gen)
    slots = torch.randperm(P, generator=gen)
    phi = torch.full((n_exp,), -1, dtype=torch.int32)
    for j in range(n_exp - n_absent):
        phi[experts[j]] = slots[j].to(torch.int32)
    return phi


def rows_per_slot_stats(counts) -> dict:
    c = [int(x) for x in counts]
    nz = [x for x in c if x > 0]
    return {"slots": len(c), "active": len(nz), "max": max(c) if c else 0,
            "min_active": min(nz) if nz else 0,
            "mean": (sum(c) / len(c)) if c else 0.0}


__all__ = ["MoEConfig", "CONFIGS", "LayerInputs", "make_inputs", "make_logits", "quantize_rows_e4m3",
           "quantize_mxfp4", "E2M1_VALUES",
           "seed_for", "identity_phi", "random_phi", "zipf_bias", "STD_W",
           "rows_per_slot_stats"]
