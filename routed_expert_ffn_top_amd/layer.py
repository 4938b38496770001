"""One MoE layer set up on the GPU through the C ABI.

Allocation (torch) and argument marshalling only: routing, descriptors, the
expert projections and the combine all run in the HIP library.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import binding as B
from .inputs import LayerInputs


class MoELayer:
    """Holds the device buffers of one layer: X, router weight, the slot
    arena with the experts, route descriptors and the workspace.

    phi      placement map for a resident layer (default: identity, P = E+S)
    paged    keep experts in pinned host memory, page them through an arena
             of cfg.P slots in banks of cfg.G (moe_layer_prefill's paged path)
    capacity route capacity C (default T*K': no split)
    """

    def __init__(self, inp: LayerInputs, phi: Optional[Sequence[int]] = None,
                 P: Optional[int] = None, capacity: Optional[int] = None,
                 paged: bool = False, device="cuda", stream=None):
        cfg = inp.cfg
        self.cfg = cfg
        self.device = torch.device(device)
        ne = cfg.n_exp
        if paged:
            P = cfg.slots if P is None else P
        elif phi is not None:
            P = (max(phi) + 1) if P is None else P
        else:
            P = ne if P is None else P
        self.shape = B.make_shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.n_shared, P=P,
                                  capacity=capacity, dtype=cfg.dtype, renorm=cfg.renorm)
        self.X = inp.X.to(self.device).contiguous()
        # router weight as [E][d] (one row per expert), the layout the C ABI takes
        self.Wr = inp.Wr.to(self.device).t().contiguous()
        self.bias = None if inp.bias is None else inp.bias.to(self.device).contiguous()
        self.routes = B.alloc_routes(self.shape, self.device)
        self.ws = B.alloc_workspace(self.shape, self.device)
        self.paged = paged
        self.arena = B.Arena(self.shape, G=(cfg.G if paged else None), device=self.device)
        Wg = inp.Wg.to(self.device)
        Wu = inp.Wu.to(self.device)
        Wd = inp.Wd.to(self.device)
        scales = None
        if cfg.quant_weights:
            scales = tuple(t.to(self.device) for t in (inp.Sg, inp.Su, inp.Sd))
        if paged:
            # prepacked experts in two pinned host planes, expert after expert,
            # so that consecutive experts load with one transfer per plane
            gu_shape = tuple(self.arena.plane_gu.shape[1:])
            d_shape = tuple(self.arena.plane_d.shape[1:])
            self.host_gu_plane = torch.empty((ne,) + gu_shape, dtype=self.arena.plane_gu.dtype, pin_memory=True)
            self.host_d_plane = torch.empty((ne,) + d_shape, dtype=self.arena.plane_d.dtype, pin_memory=True)
            tmp = torch.empty(gu_shape, dtype=self.arena.plane_gu.dtype, device=self.device)
            tmp_d = torch.empty(d_shape, dtype=self.arena.plane_d.dtype, device=self.device)
            for e in range(ne):
                g, u, dn = B.expert_slices(Wg, Wu, Wd, scales, e)
                B.moe_pack_gate_up(self.shape, g, u, tmp, 1, 0, 0, stream)
                B.moe_pack_down(self.shape, dn, tmp_d, 1, 0, 0, stream)
                self.host_gu_plane[e].copy_(tmp)
                self.host_d_plane[e].copy_(tmp_d)
            self.host_gu = [self.host_gu_plane[e] for e in range(ne)]
            self.host_d = [self.host_d_plane[e] for e in range(ne)]
            self.phi = None
        else:
            self.phi = list(range(ne)) if phi is None else [int(x) for x in phi]
            self.arena.load_resident(Wg, Wu, Wd, self.phi, stream, scales=scales)
            self.host_gu = self.host_d = None
        torch.cuda.synchronize(self.device)

    def forward(self, Y: torch.Tensor, logits: Optional[torch.Tensor] = None,
                compute=None, copy=None) -> torch.Tensor:
        """Y holds the residual A on entry and the layer output on return
        (enqueued on `compute`; not synchronized)."""
        Wr = None if logits is not None else self.Wr
        bias = None if logits is not None else self.bias
        B.moe_layer_prefill(self.shape, self.X, Wr, bias, logits, Y, self.arena,
                            self.host_gu, self.host_d, self.routes, self.ws, compute, copy)
        return Y

    def close(self):
        self.arena.close()
