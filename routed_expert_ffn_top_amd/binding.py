"""ctypes binding of the C ABI in include/moe.h (same names, argument
marshalling only: every step runs in the HIP library).

Tensors are torch tensors on the GPU (device pointers are taken with
``data_ptr()``); streams default to torch's current stream. A non-zero status
raises ``MoEError`` carrying the library's message.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_gfx950.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_CAPACITY = -2
MOE_ERR_SLOT_STATE = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5
MOE_ERR_UNSUPPORTED = -6
MOE_DT_F32 = 0
MOE_DT_BF16 = 1
MOE_DT_BF16_FP8W = 2   # bf16 activations, fp8 e4m3 weights with fp32 row scales
MOE_DT_BF16_FP4W = 3   # bf16 activations, MXFP4 weights (E2M1 codes, E8M0 scale per 32)
_DTYPE_CODE = {"f32": MOE_DT_F32, "bf16": MOE_DT_BF16, "bf16_fp8w": MOE_DT_BF16_FP8W,
               "bf16_fp4w": MOE_DT_BF16_FP4W, MOE_DT_F32: MOE_DT_F32, MOE_DT_BF16: MOE_DT_BF16,
               MOE_DT_BF16_FP8W: MOE_DT_BF16_FP8W, MOE_DT_BF16_FP4W: MOE_DT_BF16_FP4W}


def fp4_slice_bytes(N: int, K: int) -> int:
    """Bytes of a packed MXFP4 slice [N][K]: per 256-row block and 32-wide K
    piece, 16 code bytes a row plus the rows' scale bytes padded to 16."""
    piece = lambda rows: rows * 16 + (rows + 15) // 16 * 16
    full, rem = divmod(N, 256)
    return (K // 32) * (full * piece(256) + (piece(rem) if rem else 0))
MOE_DEVERR_EXPERT_ID = 1
MOE_ROUTE_RESET = 1
MOE_FFN_EXPERTS = 1
MOE_FFN_FINALIZE = 2
MOE_FFN_SIMPLE_KERNEL = 4
MOE_FFN_FUSED = 8
MOE_SLOT_AVAILABLE, MOE_SLOT_FILLING, MOE_SLOT_READY, MOE_SLOT_IN_USE = 0, 1, 2, 3
MOE_MAX_EXPERTS = 512


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("P", ctypes.c_int32), ("capacity", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("renorm", ctypes.c_int32), ("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64)]


class moe_routes(ctypes.Structure):
    _fields_ = [("topk_idx", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("slot_count", ctypes.c_void_p), ("slot_offset", ctypes.c_void_p),
                ("rec_token", ctypes.c_void_p), ("rec_route", ctypes.c_void_p),
                ("route_pos", ctypes.c_void_p)]


_lib = None

_VP, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "moe_version": ([], ctypes.c_char_p),
    "moe_last_error": ([ctypes.c_char_p, _SZ], _I32),
    "moe_workspace_bytes": ([_VP], _SZ),
    "moe_workspace_init": ([_VP, _VP, _SZ, _VP], _I32),
    "moe_device_errors": ([_VP, _VP, _SZ, _VP, _VP], _I32),
    "moe_router_logits": ([_VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "moe_route_build": ([_VP, _I32, _I32, _VP, _VP, _I32, _VP, _VP, _SZ, _VP], _I32),
    "moe_expert_ffn": ([_VP, _VP, _VP, _VP, _VP, _VP, _I32, _VP, _SZ, _VP], _I32),
    "moe_layer_prefill": ([_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP, _VP], _I32),
    "moe_layer_prefill_noalloc": ([_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP], _I32),
    "moe_pack_gate_up": ([_VP, _VP, _VP, _VP, _I32, _I64, _I64, _VP], _I32),
    "moe_pack_gate_up_host": ([_VP, _VP, _VP, _VP], _I32),
    "moe_pack_down": ([_VP, _VP, _VP, _I32, _I64, _I64, _VP], _I32),
    "moe_pack_down_host": ([_VP, _VP, _VP], _I32),
    "moe_arena_create": ([_VP, _VP, _VP, _VP, _I64, _I64, _I32], _I32),
    "moe_arena_destroy": ([_VP], None),
    "arena_bind_slot": ([_VP, _I32, _I32, _VP, _VP, _VP], _I32),
    "arena_reserve_slot": ([_VP, _I32, _I32], _I32),
    "arena_publish_slot": ([_VP, _I32, _I32, _VP], _I32),
    "arena_release_slot": ([_VP, _I32], _I32),
    "arena_phi": ([_VP, _VP, _I32], _I32),
    "arena_slot_info": ([_VP, _I32, _VP, _VP], _I32),
    "moe_selftest_mfma_layout": ([_VP, _VP], _I32),
    "moe_profile_begin": ([_I32, _I32], _I32),
    "moe_profile_end": ([_I32, _VP, _I32, _VP], _I32),
}

MOE_KERNEL = {"router": 1, "topk": 2, "route_count": 3, "route_place": 4, "gate_up": 5, "down": 6,
              "combine": 7, "h2d": 8, "fused": 9}


def lib_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load the HIP library, building it first only if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library missing: {LIB_PATH} (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != MOE_OK:
        buf = ctypes.create_string_buffer(512)
        load().moe_last_error(buf, 512)
        raise MoEError(status, buf.value.decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def make_shape(T, d, f, E, k, n_shared=0, P=None, capacity=None, dtype="bf16", renorm=True,
               ldx=None, ldy=None) -> moe_shape:
    kp = k + n_shared
    return moe_shape(T=T, d=d, f=f, E=E, k=k, n_shared=n_shared,
                     P=(E + n_shared) if P is None else P,
                     capacity=max(1, T * kp) if capacity is None else capacity,
                     dtype=_DTYPE_CODE[dtype],
                     renorm=int(bool(renorm)), ldx=d if ldx is None else ldx,
                     ldy=d if ldy is None else ldy)


def routes_struct(r: dict) -> moe_routes:
    return moe_routes(*[_ptr(r[k]) for k in ("topk_idx", "topk_w", "slot_count", "slot_offset",
                                              "rec_token", "rec_route", "route_pos")])


# ----------------------------------------------------------------- calls --
def moe_version() -> str:
    return load().moe_version().decode()


def moe_last_error():
    buf = ctypes.create_string_buffer(512)
    st = load().moe_last_error(buf, 512)
    return st, buf.value.decode()


def moe_workspace_bytes(shape: moe_shape) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(shape)))


def moe_workspace_init(shape, ws, stream=None):
    _check(load().moe_workspace_init(ctypes.byref(shape), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def moe_device_errors(shape, ws, stream=None) -> int:
    v = ctypes.c_int32(0)
    st = load().moe_device_errors(ctypes.byref(shape), _ptr(ws), ws.numel() * ws.element_size(),
                                  ctypes.byref(v), _stream(stream))
    if st not in (MOE_OK, MOE_ERR_INVALID_ARG):
        _check(st)
    return int(v.value)


def moe_router_logits(shape, X, W_r, bias, logits, stream=None):
    _check(load().moe_router_logits(ctypes.byref(shape), _ptr(X), _ptr(W_r), _ptr(bias),
                                    _ptr(logits), _stream(stream)))


def _phi_arr(phi):
    if phi is None:
        return None
    vals = [int(x) for x in phi]
    return (ctypes.c_int32 * len(vals))(*vals)


def moe_route_build(shape, t0, nt, logits, phi, flags, routes: dict, ws, stream=None):
    rs = routes_struct(routes)
    _check(load().moe_route_build(ctypes.byref(shape), t0, nt, _ptr(logits), _phi_arr(phi), flags,
                                  ctypes.byref(rs), _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream)))


def moe_expert_ffn(shape, X, Y, routes: dict, arena, phi, flags, ws, stream=None):
    rs = routes_struct(routes)
    _check(load().moe_expert_ffn(ctypes.byref(shape), _ptr(X), _ptr(Y), ctypes.byref(rs),
                                 arena.handle if arena is not None else None, _phi_arr(phi), flags,
                                 _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_prefill(shape, X, W_r, bias, logits, Y, arena, host_gu, host_d, routes: dict, ws,
                      compute=None, copy=None):
    rs = routes_struct(routes)
    gu = d = None
    if host_gu is not None:
        n = len(host_gu)
        gu = (ctypes.c_void_p * n)(*[_ptr(t) for t in host_gu])
        d = (ctypes.c_void_p * n)(*[_ptr(t) for t in host_d])
    _check(load().moe_layer_prefill(ctypes.byref(shape), _ptr(X), _ptr(W_r), _ptr(bias), _ptr(logits),
                                    _ptr(Y), arena.handle, gu, d, ctypes.byref(rs), _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(compute),
                                    _stream(copy) if copy is not None else None))


def moe_layer_prefill_noalloc(shape, X, W_r, bias, logits, Y, arena, routes: dict, stream=None):
    rs = routes_struct(routes)
    _check(load().moe_layer_prefill_noalloc(ctypes.byref(shape), _ptr(X), _ptr(W_r), _ptr(bias), _ptr(logits),
                                            _ptr(Y), arena.handle, ctypes.byref(rs), _stream(stream)))


def moe_pack_gate_up(shape, Wg, Wu, dst, n, src_stride, dst_stride, stream=None):
    _check(load().moe_pack_gate_up(ctypes.byref(shape), _ptr(Wg), _ptr(Wu), _ptr(dst), n,
                                   src_stride, dst_stride, _stream(stream)))


def moe_pack_gate_up_host(shape, Wg, Wu, dst):
    _check(load().moe_pack_gate_up_host(ctypes.byref(shape), _ptr(Wg), _ptr(Wu), _ptr(dst)))


def moe_pack_down(shape, Wd, dst, n, src_stride, dst_stride, stream=None):
    _check(load().moe_pack_down(ctypes.byref(shape), _ptr(Wd), _ptr(dst), n, src_stride, dst_stride,
                                _stream(stream)))


def moe_pack_down_host(shape, Wd, dst):
    _check(load().moe_pack_down_host(ctypes.byref(shape), _ptr(Wd), _ptr(dst)))


def moe_arena_create(shape, plane_gu, plane_d, stride_gu, stride_d, G) -> int:
    h = ctypes.c_void_p(0)
    _check(load().moe_arena_create(ctypes.byref(h), ctypes.byref(shape), _ptr(plane_gu), _ptr(plane_d),
                                   stride_gu, stride_d, G))
    return h.value


def moe_arena_destroy(handle) -> None:
    load().moe_arena_destroy(handle)


def arena_bind_slot(arena, slot, expert, src_gu, src_d, copy_stream=None):
    _check(load().arena_bind_slot(arena.handle, slot, expert, _ptr(src_gu), _ptr(src_d),
                                  _stream(copy_stream)))


def arena_reserve_slot(arena, slot, expert):
    _check(load().arena_reserve_slot(arena.handle, slot, expert))


def arena_publish_slot(arena, slot, expert, stream=None):
    _check(load().arena_publish_slot(arena.handle, slot, expert, _stream(stream)))


def arena_release_slot(arena, slot):
    _check(load().arena_release_slot(arena.handle, slot))


def arena_phi(arena, n) -> list:
    buf = (ctypes.c_int32 * n)()
    _check(load().arena_phi(arena.handle, buf, n))
    return list(buf)


def arena_slot_info(arena, slot):
    st, ex = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load().arena_slot_info(arena.handle, slot, ctypes.byref(st), ctypes.byref(ex)))
    return int(st.value), int(ex.value)


def moe_selftest_mfma_layout(out, stream=None):
    _check(load().moe_selftest_mfma_layout(_ptr(out), _stream(stream)))


# ------------------------------------------------------- buffer helpers --
def alloc_routes(shape: moe_shape, device="cuda") -> dict:
    kp = shape.k + shape.n_shared
    i32 = dict(dtype=torch.int32, device=device)
    return dict(topk_idx=torch.zeros((shape.T, kp), **i32),
                topk_w=torch.zeros((shape.T, kp), dtype=torch.float32, device=device),
                slot_count=torch.zeros(shape.P, **i32),
                slot_offset=torch.zeros(shape.P + 1, **i32),
                rec_token=torch.full((shape.capacity,), -1, **i32),
                rec_route=torch.full((shape.capacity,), -1, **i32),
                route_pos=torch.full((shape.T * kp,), -1, **i32))


def alloc_workspace(shape: moe_shape, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(shape)
    if n == 0:
        _check(MOE_ERR_INVALID_ARG)
    buf = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    ws = buf[off:off + n]
    moe_workspace_init(shape, ws)
    return ws


class Arena:
    """Device planes of P slots (Eq. 3) plus the library's residency table."""

    def __init__(self, shape: moe_shape, G: Optional[int] = None, device="cuda"):
        self.shape = shape
        if shape.dtype in (MOE_DT_BF16_FP8W, MOE_DT_BF16_FP4W):
            # a slice is its codes then its scales; strides in bytes
            if shape.dtype == MOE_DT_BF16_FP8W:
                self.stride_gu = 2 * shape.f * shape.d + 8 * shape.f
                self.stride_d = shape.d * shape.f + 4 * shape.d
            else:
                self.stride_gu = fp4_slice_bytes(2 * shape.f, shape.d)
                self.stride_d = fp4_slice_bytes(shape.d, shape.f)
            self.plane_gu = torch.empty((shape.P, self.stride_gu), dtype=torch.uint8, device=device)
            self.plane_d = torch.empty((shape.P, self.stride_d), dtype=torch.uint8, device=device)
        else:
            dt = torch.bfloat16 if shape.dtype == MOE_DT_BF16 else torch.float32
            self.stride_gu = 2 * shape.f * shape.d
            self.stride_d = shape.d * shape.f
            self.plane_gu = torch.empty((shape.P, 2 * shape.f, shape.d), dtype=dt, device=device)
            self.plane_d = torch.empty((shape.P, shape.d, shape.f), dtype=dt, device=device)
        self.G = shape.P if G is None else G
        self.handle = moe_arena_create(shape, self.plane_gu, self.plane_d, self.stride_gu,
                                       self.stride_d, self.G)

    def close(self):
        if self.handle:
            moe_arena_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_resident(self, Wg, Wu, Wd, phi: Sequence[int], stream=None, scales=None):
        """Pack and publish every expert e with phi[e] >= 0 into slot phi[e].
        scales: (Sg, Su, Sd) row scales (fp8 codes) or block scales (MXFP4)."""
        for e, s in enumerate(phi):
            if s < 0:
                continue
            g, u, dn = expert_slices(Wg, Wu, Wd, scales, e)
            moe_pack_gate_up(self.shape, g, u, self.plane_gu[s], 1, 0, 0, stream)
            moe_pack_down(self.shape, dn, self.plane_d[s], 1, 0, 0, stream)
            arena_publish_slot(self, s, e, stream)


def expert_slices(Wg, Wu, Wd, scales, e):
    """Expert e's gate, up and down slices in the layout the C ABI takes:
    the weight rows, then (fp8 codes) the rows' fp32 scales as bytes or
    (MXFP4: packed code bytes [N][K/2]) the E8M0 scale bytes [N][K/32]."""
    if scales is None:
        return Wg[e], Wu[e], Wd[e]
    Sg, Su, Sd = scales
    cat = lambda q, sc: torch.cat([q[e].reshape(-1), sc[e].contiguous().view(torch.uint8).reshape(-1)])
    return cat(Wg, Sg), cat(Wu, Su), cat(Wd, Sd)


def moe_profile_begin(kernel: str, max_launches: int):
    _check(load().moe_profile_begin(MOE_KERNEL[kernel], max_launches))


def moe_profile_end(kernel: str, n: int) -> list:
    buf = (ctypes.c_float * n)()
    rec = ctypes.c_int32(0)
    _check(load().moe_profile_end(MOE_KERNEL[kernel], buf, n, ctypes.byref(rec)))
    return [float(buf[i]) for i in range(min(n, rec.value))]
