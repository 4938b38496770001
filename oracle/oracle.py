"""Python face of the CPU oracle (oracle.c) for one routed-expert MoE layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module; the GPU product path never does.

Everything here is argument marshalling around the C functions, plus a
convenience ``layer`` that chains them in the order the method runs:
router logits -> top-k -> route map (Algorithm 1) -> expert FFN and combine
(Eq. 1-2 of "EStream: Fast and Memory-Efficient MoE Prefill through Expert
Virtualization on Mobile NPUs", section 3.2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
          "-fno-fast-math", "-std=c11"]


def build(src: str = SRC, out: str = LIB, extra: Optional[list] = None) -> str:
    """Compile the oracle with gcc (no -ffast-math, no FP contraction)."""
    cmd = ["gcc", *CFLAGS, *(extra or []), src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes binding of one build of oracle.c (the default one, or a variant
    compiled by a test)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        elif path == LIB and os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()   # the default build is older than its source
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_router_logits.argtypes = [_i64, _i64, _i64, _ptr, _i64, _ptr, _ptr, _ptr]
        lib.oracle_router_logits.restype = None
        lib.oracle_topk.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _ptr, _ptr, _ptr]
        lib.oracle_topk.restype = None
        lib.oracle_route_map.argtypes = [_i64, _i64, _i64, _ptr, _i64, _ptr, _i64,
                                         _ptr, _ptr, _ptr, _ptr, _ptr]
        lib.oracle_route_map.restype = _i64
        lib.oracle_expert_ffn.argtypes = [_i64, _i64, _i64, _i64, _ptr, _ptr, _i64, _ptr,
                                          _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr,
                                          _ptr, _ptr]
        lib.oracle_expert_ffn.restype = None
        lib.oracle_fp8e4m3_decode.argtypes = [_i64, _ptr, _ptr]
        lib.oracle_fp8e4m3_decode.restype = None
        lib.oracle_mxfp4_decode.argtypes = [_i64, _i64, _ptr, _ptr, _ptr]
        lib.oracle_mxfp4_decode.restype = None
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        self.lib = lib

    # -- threads -----------------------------------------------------------
    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    # -- steps -------------------------------------------------------------
    def router_logits(self, X: np.ndarray, Wr: np.ndarray,
                      bias: Optional[np.ndarray] = None) -> np.ndarray:
        X = np.ascontiguousarray(X, dtype=np.float32)
        Wr = np.ascontiguousarray(Wr, dtype=np.float32)
        T, d = X.shape
        d2, E = Wr.shape
        assert d == d2
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        L = np.empty((T, E), dtype=np.float32)
        self.lib.oracle_router_logits(T, d, E, _p(X), d, _p(Wr), _p(b), _p(L))
        return L

    def topk(self, L: np.ndarray, k: int, n_shared: int = 0, renorm: bool = True):
        L = np.ascontiguousarray(L, dtype=np.float32)
        T, E = L.shape
        kp = k + n_shared
        idx = np.empty((T, kp), dtype=np.int32)
        alpha = np.empty((T, kp), dtype=np.float64)
        self.lib.oracle_topk(T, E, k, n_shared, int(bool(renorm)), _p(L), _p(idx), _p(alpha))
        return idx, alpha

    def route_map(self, idx: np.ndarray, phi: np.ndarray, P: int, t0: int = 0,
                  nt: Optional[int] = None, route_pos: Optional[np.ndarray] = None):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, kp = idx.shape
        nt = T - t0 if nt is None else nt
        phi = np.ascontiguousarray(phi, dtype=np.int32)
        count = np.zeros(P, dtype=np.int32)
        offset = np.zeros(P + 1, dtype=np.int32)
        cap = max(nt * kp, 1)
        rec_token = np.full(cap, -1, dtype=np.int32)
        rec_route = np.full(cap, -1, dtype=np.int32)
        if route_pos is None:
            route_pos = np.full(T * kp, -1, dtype=np.int32)
        n_valid = self.lib.oracle_route_map(kp, t0, nt, _p(idx), len(phi), _p(phi), P,
                                            _p(count), _p(offset), _p(rec_token),
                                            _p(rec_route), _p(route_pos))
        if n_valid < 0:
            raise ValueError("route map: expert id or slot out of range")
        return dict(count=count, offset=offset, rec_token=rec_token[:n_valid],
                    rec_route=rec_route[:n_valid], route_pos=route_pos,
                    n_valid=int(n_valid))

    def mxfp4_decode(self, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
        """fp32 weights [..., N, K] of MXFP4 codes [..., N, K/2] (two per byte,
        low nibble first) and E8M0 block scales [..., N, K/32]."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        scales = np.ascontiguousarray(scales, dtype=np.uint8)
        K = codes.shape[-1] * 2
        assert scales.shape[-1] * 32 == K and scales.shape[:-1] == codes.shape[:-1]
        N = int(np.prod(codes.shape[:-1]))
        out = np.empty(codes.shape[:-1] + (K,), dtype=np.float32)
        self.lib.oracle_mxfp4_decode(N, K, _p(codes), _p(scales), _p(out))
        return out

    def fp8e4m3_decode(self, q: np.ndarray) -> np.ndarray:
        """Values (fp32) of fp8 e4m3 codes (uint8 array of any shape)."""
        q = np.ascontiguousarray(q, dtype=np.uint8)
        out = np.empty(q.shape, dtype=np.float32)
        self.lib.oracle_fp8e4m3_decode(q.size, _p(q), _p(out))
        return out

    def expert_ffn(self, X: np.ndarray, idx: np.ndarray, alpha: np.ndarray,
                   Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray,
                   A: Optional[np.ndarray] = None, tokens=None,
                   route_mask: Optional[np.ndarray] = None,
                   scales: Optional[tuple] = None) -> np.ndarray:
        """scales: None, or (Sg [ne][f], Su [ne][f], Sd [ne][d]) row scales;
        each weight is then its given value times its row's scale."""
        X = np.ascontiguousarray(X, dtype=np.float32)
        T, d = X.shape
        ne, f, d2 = Wg.shape
        assert d2 == d and Wu.shape == Wg.shape and Wd.shape == (ne, d, f)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        kp = idx.shape[1]
        alpha = np.ascontiguousarray(alpha, dtype=np.float64)
        Wg = np.ascontiguousarray(Wg, dtype=np.float32)
        Wu = np.ascontiguousarray(Wu, dtype=np.float32)
        Wd = np.ascontiguousarray(Wd, dtype=np.float32)
        A = None if A is None else np.ascontiguousarray(A, dtype=np.float32)
        if tokens is None:
            tokens = np.arange(T, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        mask = None
        if route_mask is not None:
            mask = np.ascontiguousarray(route_mask, dtype=np.uint8).reshape(-1)
            assert mask.size == T * kp
        Sg = Su = Sd = None
        if scales is not None:
            Sg, Su, Sd = (np.ascontiguousarray(v, dtype=np.float32) for v in scales)
            assert Sg.shape == (ne, f) and Su.shape == (ne, f) and Sd.shape == (ne, d)
        Y = np.empty((len(tokens), d), dtype=np.float64)
        self.lib.oracle_expert_ffn(d, f, kp, len(tokens), _p(tokens), _p(X), d, _p(idx),
                                   _p(alpha), _p(mask), _p(Wg), _p(Wu), _p(Wd), _p(Sg), _p(Su),
                                   _p(Sd), _p(A), _p(Y))
        return Y

    # -- whole layer -------------------------------------------------------
    def layer(self, X, Wr, bias, Wg, Wu, Wd, A, k, n_shared, renorm,
              phi=None, P=None, tokens=None, logits=None, scales=None):
        """Router (unless logits are given) -> top-k -> route map -> FFN."""
        L = self.router_logits(X, Wr, bias) if logits is None else logits
        idx, alpha = self.topk(L, k, n_shared, renorm)
        ne = Wg.shape[0]
        if phi is None:
            phi = np.arange(ne, dtype=np.int32)
            P = ne
        rm = self.route_map(idx, phi, P)
        Y = self.expert_ffn(X, idx, alpha, Wg, Wu, Wd, A, tokens=tokens, scales=scales)
        return dict(logits=L, idx=idx, alpha=alpha, Y=Y, **rm)


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
