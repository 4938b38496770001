"""Checks that pin the CPU oracle to facts other than itself.

Each ``check_*`` takes an ``Oracle`` (any build of oracle.c) and raises
AssertionError when the oracle disagrees with:

* hand-worked closed forms (tests/golden/*.json);
* exact integer arithmetic (router on inputs whose sums are exact);
* exact rational arithmetic (router logits are the correctly rounded sums)
  and math.fsum at the OLMoE hidden size;
* a numpy/scipy brute force of a *different* formulation: top-k by lexsort,
  softmax by scipy, the route map by a stable argsort and bincount, and the
  layer as a dense masked sum over every expert on every token;
* special cases (k=1 argmax, k=E full order, k=2 logistic weights, E=1 dense
  SwiGLU, W_up = 0, W_down scaled by 2, expert relabelling, hidden-unit
  permutation, masked routes).

The mutation test runs all of them against oracle builds with planted
mistakes and requires every mistake to be caught.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy.special import softmax, expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _bf16_values(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and widen back to fp32."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _layer_weights(rng, ne, d, f, std=0.02, bf16=True):
    Wg = rng.standard_normal((ne, f, d), dtype=np.float32) * np.float32(std)
    Wu = rng.standard_normal((ne, f, d), dtype=np.float32) * np.float32(std)
    Wd = rng.standard_normal((ne, d, f), dtype=np.float32) * np.float32(std)
    if bf16:
        Wg, Wu, Wd = _bf16_values(Wg), _bf16_values(Wu), _bf16_values(Wd)
    return Wg, Wu, Wd


def _random_routes(rng, T, E, k, n_shared=0):
    """Distinct random experts per token and random positive weights."""
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if n_shared:
        sh = np.tile(np.arange(E, E + n_shared, dtype=np.int32), (T, 1))
        idx = np.concatenate([idx, sh], axis=1)
    alpha = rng.uniform(0.05, 1.0, size=idx.shape)
    return idx, alpha


def dense_brute_force(X, idx, alpha, Wg, Wu, Wd, A=None, route_mask=None):
    """Every expert on every token in fp64 (matrix form), masked by routing."""
    X = X.astype(np.float64)
    T, d = X.shape
    ne = Wg.shape[0]
    M = np.zeros((T, ne))
    kp = idx.shape[1]
    for t in range(T):
        for j in range(kp):
            if route_mask is None or route_mask[t * kp + j]:
                M[t, idx[t, j]] += alpha[t, j]
    Y = np.zeros((T, d)) if A is None else A.astype(np.float64).copy()
    for e in range(ne):
        G = X @ Wg[e].astype(np.float64).T
        U = X @ Wu[e].astype(np.float64).T
        H = G * expit(G) * U
        O = H @ Wd[e].astype(np.float64).T
        Y += M[:, e:e + 1] * O
    return Y


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------- router --
def check_router_golden(orc):
    for case in _load("router_dot.json")["cases"]:
        hx = lambda v: float.fromhex(v)
        x = np.array([[hx(v) for v in case["x"]]], dtype=np.float32)
        w = np.array([hx(v) for v in case["w"]], dtype=np.float32)[:, None]
        b = np.array([hx(case["bias"])], dtype=np.float32)
        L = orc.router_logits(x, w, b)
        assert L[0, 0] == np.float32(hx(case["expect"])), (case["why"], float(L[0, 0]).hex())


def check_router_exact_integers(orc):
    """Small integers scaled by 2^-4: every partial sum is exact, so the
    logits equal the exact integer matrix product."""
    rng = _rng(11)
    T, d, E = 17, 64, 8
    Xi = rng.integers(-8, 9, size=(T, d))
    Wi = rng.integers(-8, 9, size=(d, E))
    bi = rng.integers(-8, 9, size=E)
    X = Xi.astype(np.float32)
    Wr = (Wi.astype(np.float32) / 16).astype(np.float32)
    b = (bi.astype(np.float32) / 16).astype(np.float32)
    L = orc.router_logits(X, Wr, b)
    exact = (Xi @ Wi + bi[None, :]) / 16.0
    assert np.array_equal(L.astype(np.float64), exact)
    L0 = orc.router_logits(X, Wr, None)
    assert np.array_equal(L0.astype(np.float64), (Xi @ Wi) / 16.0)


def _round_f32(q):
    """The fp32 value nearest to the exact rational q, ties to the even
    significand (q within the finite fp32 range)."""
    from fractions import Fraction
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - q), int(np.array(c).view(np.uint32)) & 1))


def check_router_correct_rounding(orc):
    """Logits against exact rational arithmetic: every logit is the fp32
    value nearest to the exact sum of the products and the bias (ties to
    even), except where the exact value lies within the fp64 summation error
    (d + 1) 2^-53 sum|x w| of an fp32 rounding boundary (none at these seeds)."""
    from fractions import Fraction
    rng = _rng(12)
    T, d, E = 6, 96, 8
    X = _bf16_values(rng.standard_normal((T, d), dtype=np.float32))
    Wr = rng.standard_normal((d, E), dtype=np.float32) * np.float32(0.02)
    b = rng.standard_normal(E, dtype=np.float32) * np.float32(0.5)
    L = orc.router_logits(X, Wr, b)
    near = 0
    for t in range(T):
        for e in range(E):
            q = sum(Fraction(float(X[t, i])) * Fraction(float(Wr[i, e])) for i in range(d)) + Fraction(float(b[e]))
            r = _round_f32(q)
            if L[t, e] != r:
                slack = (d + 1) * 2.0 ** -53 * float(np.abs(X[t].astype(np.float64)) @ np.abs(Wr[:, e].astype(np.float64)))
                mid = (Fraction(float(L[t, e])) + Fraction(float(r))) / 2
                assert abs(q - mid) <= Fraction(slack), (t, e, float(L[t, e]), float(r))
                near += 1
    assert near == 0


def check_router_error_bound(orc):
    """At the OLMoE hidden size: |L - s| <= half an fp32 unit of s plus
    (d + 1) 2^-53 sum|x w|, where s is math.fsum of the exact fp64 products
    and the bias (the correctly rounded fp64 sum)."""
    import math
    rng = _rng(13)
    for T, d, E in ((4, 2048, 64), (5, 320, 8)):
        X = _bf16_values(rng.standard_normal((T, d), dtype=np.float32))
        Wr = rng.standard_normal((d, E), dtype=np.float32) * np.float32(0.02)
        b = rng.standard_normal(E, dtype=np.float32) * np.float32(0.1)
        L = orc.router_logits(X, Wr, b).astype(np.float64)
        Xd, Wd = X.astype(np.float64), Wr.astype(np.float64)
        for t in range(T):
            for e in range(E):
                s = math.fsum(list(Xd[t] * Wd[:, e]) + [float(b[e])])
                half_ulp = float(np.spacing(np.float32(abs(s)))) / 2
                slack = (d + 1) * 2.0 ** -53 * float(np.abs(Xd[t]) @ np.abs(Wd[:, e]))
                assert abs(L[t, e] - s) <= half_ulp + slack, (t, e, L[t, e], s)


# ----------------------------------------------------------------- top-k --
def _lexsort_topk(L, k):
    T, E = L.shape
    out = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -L[t].astype(np.float64)))
        out[t] = order[:k]
    return out


def check_topk_bruteforce(orc):
    rng = _rng(21)
    for (T, E, k) in [(50, 64, 8), (40, 8, 2), (30, 64, 6), (20, 5, 5), (25, 7, 1)]:
        L = rng.standard_normal((T, E), dtype=np.float32)
        idx, _ = orc.topk(L, k, 0, True)
        assert np.array_equal(idx, _lexsort_topk(L, k)), (T, E, k)
        # heavy ties: logits drawn from 3 values
        Lt = rng.integers(0, 3, size=(T, E)).astype(np.float32)
        idx, _ = orc.topk(Lt, k, 0, True)
        assert np.array_equal(idx, _lexsort_topk(Lt, k)), ("ties", T, E, k)


def check_topk_special(orc):
    rng = _rng(22)
    L = rng.standard_normal((33, 16), dtype=np.float32)
    idx, _ = orc.topk(L, 1, 0, True)
    assert np.array_equal(idx[:, 0], np.argmax(L, axis=1))
    idx, _ = orc.topk(L, 16, 0, True)
    for t in range(33):
        assert np.array_equal(idx[t], np.argsort(-L[t].astype(np.float64), kind="stable"))
    # hand example with ties: [1, 3, 3, 2, 3] -> 1, 2, 4, then 3
    h = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], dtype=np.float32)
    idx, al = orc.topk(h, 4, 0, False)
    assert idx.tolist() == [[1, 2, 4, 3]]
    z = math.exp(1) + 3 * math.exp(3) + math.exp(2)
    assert abs(al[0, 0] - math.exp(3) / z) < 1e-15
    assert abs(al[0, 3] - math.exp(2) / z) < 1e-15


def check_topk_nan_and_signed_zero(orc):
    """Reading of the routing step for values the pages leave open: a NaN
    logit ranks as -infinity with weight 0; -0 and +0 are equal logits (tie
    to the lower id); a row with no finite logit picks ids in order with
    weight 0."""
    nan, inf = float("nan"), float("inf")
    h = np.array([[nan, 1.0, 0.5, nan, -0.0, 0.0],
                  [nan, nan, nan, nan, nan, nan],
                  [0.0, -0.0, nan, -inf, -0.0, 0.0]], dtype=np.float32)
    idx, al = orc.topk(h, 3, 0, True)
    assert idx.tolist()[0] == [1, 2, 4]                 # -0 at id 4 before +0 at id 5
    z = math.exp(1.0) + math.exp(0.5) + 2 * math.exp(0.0)
    p = [math.exp(1.0) / z, math.exp(0.5) / z, 1.0 / z]
    assert max(abs(al[0, j] - p[j] / sum(p)) for j in range(3)) < 1e-15
    assert idx.tolist()[1] == [0, 1, 2] and np.all(al[1] == 0.0)
    assert idx.tolist()[2] == [0, 1, 4]                 # four equal zeros: the lowest ids
    assert max(abs(al[2, j] - 1.0 / 3.0) for j in range(3)) < 1e-15
    idx, al = orc.topk(h, 3, 0, False)
    assert max(abs(al[0, j] - p[j]) for j in range(3)) < 1e-15
    assert max(abs(al[2, j] - 0.25) for j in range(3)) < 1e-15   # 4 zeros share the mass


def check_alpha(orc):
    rng = _rng(23)
    T, E = 40, 64
    L = rng.standard_normal((T, E), dtype=np.float32)
    sm = softmax(L.astype(np.float64), axis=1)
    for k in (1, 6, 8):
        idx, al = orc.topk(L, k, 0, False)
        ref = np.take_along_axis(sm, idx.astype(np.int64), axis=1)
        assert np.max(np.abs(al - ref)) < 1e-14
        idx, al = orc.topk(L, k, 0, True)
        assert np.max(np.abs(al.sum(axis=1) - 1.0)) < 1e-14
        # renormalised ratios equal the exponentiated logit differences
        r = al[:, 0:1] / al
        lsel = np.take_along_axis(L.astype(np.float64), idx.astype(np.int64), axis=1)
        assert np.max(np.abs(r - np.exp(lsel[:, 0:1] - lsel)) / r) < 1e-13
    # k = E renormalised is the full softmax in rank order
    idx, al = orc.topk(L, E, 0, True)
    assert np.max(np.abs(al - np.take_along_axis(sm, idx.astype(np.int64), 1))) < 1e-14
    # top-2 renormalised: weight of the first choice = logistic(L1 - L2)
    L8 = rng.standard_normal((T, 8), dtype=np.float32)
    idx, al = orc.topk(L8, 2, 0, True)
    l = np.take_along_axis(L8.astype(np.float64), idx.astype(np.int64), axis=1)
    assert np.max(np.abs(al[:, 0] - expit(l[:, 0] - l[:, 1]))) < 1e-14


def check_shared(orc):
    rng = _rng(24)
    L = rng.standard_normal((12, 64), dtype=np.float32)
    idx, al = orc.topk(L, 6, 2, False)
    assert idx.shape == (12, 8)
    assert np.all(idx[:, 6] == 64) and np.all(idx[:, 7] == 65)
    assert np.all(al[:, 6:] == 1.0)
    i2, a2 = orc.topk(L, 6, 0, False)
    assert np.array_equal(idx[:, :6], i2) and np.array_equal(al[:, :6], a2)


# ------------------------------------------------------------- route map --
def _route_map_brute(idx, phi, P, t0, nt):
    T, kp = idx.shape
    routes = np.arange(t0 * kp, (t0 + nt) * kp)
    psi = phi[idx.reshape(-1)[routes]]
    valid = routes[psi >= 0]
    pv = psi[psi >= 0]
    order = np.argsort(pv, kind="stable")
    rec_route = valid[order]
    count = np.bincount(pv, minlength=P)
    offset = np.concatenate([[0], np.cumsum(count)])
    pos = np.full(T * kp, -7, dtype=np.int64)
    pos[routes] = -1
    pos[rec_route] = np.arange(len(rec_route))
    return dict(count=count, offset=offset, rec_route=rec_route,
                rec_token=rec_route // kp, route_pos=pos, n_valid=len(rec_route))


def check_route_map_golden(orc):
    g = _load("route_map_hand.json")
    ex = g["expect"]
    r = orc.route_map(np.array(g["idx"]), np.array(g["phi"]), g["P"])
    for key in ("count", "offset", "rec_token", "rec_route", "route_pos"):
        assert r[key].tolist() == ex[key], key
    assert r["n_valid"] == ex["n_valid"]


def check_route_map_bruteforce(orc):
    rng = _rng(31)
    for (T, E, k, P, absent, t0, nt) in [(100, 64, 8, 64, 0, 0, 100),
                                         (64, 8, 2, 8, 0, 0, 64),
                                         (77, 66, 8, 40, 26, 0, 77),
                                         (50, 64, 8, 16, 48, 10, 25),
                                         (1, 8, 2, 8, 0, 0, 1)]:
        idx, _ = _random_routes(rng, T, E, k)
        perm = rng.permutation(E)
        phi = np.full(E, -1, dtype=np.int32)
        slots = rng.permutation(P)
        for j in range(E - absent):
            phi[perm[j]] = slots[j]
        pos0 = np.full(T * k, -7, dtype=np.int32)
        r = orc.route_map(idx, phi, P, t0, nt, route_pos=pos0)
        b = _route_map_brute(idx, phi, P, t0, nt)
        assert np.array_equal(r["count"], b["count"])
        assert np.array_equal(r["offset"], b["offset"])
        assert np.array_equal(r["rec_route"], b["rec_route"])
        assert np.array_equal(r["rec_token"], b["rec_token"])
        assert np.array_equal(r["route_pos"], b["route_pos"])
        assert r["n_valid"] == b["n_valid"]
        # invariants: counts sum to the placed routes; offsets monotone;
        # every placed (token, rank) appears once; ascending inside a slot
        assert r["count"].sum() == r["n_valid"] == r["offset"][-1]
        assert np.all(np.diff(r["offset"]) >= 0) and r["offset"][0] == 0
        assert len(set(r["rec_route"].tolist())) == r["n_valid"]
        for s in range(P):
            seg = r["rec_route"][r["offset"][s]:r["offset"][s + 1]]
            assert np.all(np.diff(seg) > 0)
            assert np.all(phi[idx.reshape(-1)[seg]] == s)
    # full identity map: every route placed, counts sum to T*k
    idx, _ = _random_routes(rng, 64, 64, 8)
    r = orc.route_map(idx, np.arange(64, dtype=np.int32), 64)
    assert r["n_valid"] == 64 * 8


def check_route_map_errors(orc):
    idx = np.array([[0, 9]], dtype=np.int32)
    try:
        orc.route_map(idx, np.arange(4, dtype=np.int32), 4)
    except ValueError:
        pass
    else:
        raise AssertionError("expert id out of range accepted")
    try:
        orc.route_map(np.array([[0, 1]], dtype=np.int32),
                      np.array([0, 5], dtype=np.int32), 4)
    except ValueError:
        pass
    else:
        raise AssertionError("slot out of range accepted")


# ------------------------------------------------------------------- FFN --
def check_ffn_dense_bruteforce(orc):
    rng = _rng(41)
    for (T, d, f, E, k, S) in [(24, 64, 96, 8, 2, 0), (16, 128, 64, 6, 3, 2)]:
        X = _bf16_values(rng.standard_normal((T, d), dtype=np.float32))
        A = rng.standard_normal((T, d), dtype=np.float32)
        Wg, Wu, Wd = _layer_weights(rng, E + S, d, f, std=0.1)
        idx, alpha = _random_routes(rng, T, E, k, S)
        Y = orc.expert_ffn(X, idx, alpha, Wg, Wu, Wd, A)
        ref = dense_brute_force(X, idx, alpha, Wg, Wu, Wd, A)
        assert _rel(Y, ref) < 1e-12, _rel(Y, ref)
        # a token subset returns the same rows
        sub = np.array([5, 0, T - 1])
        Ys = orc.expert_ffn(X, idx, alpha, Wg, Wu, Wd, A, tokens=sub)
        assert np.array_equal(Ys, Y[sub])
        # masked routes are left out of the sum
        mask = rng.integers(0, 2, size=T * (k + S)).astype(np.uint8)
        Ym = orc.expert_ffn(X, idx, alpha, Wg, Wu, Wd, A, route_mask=mask)
        refm = dense_brute_force(X, idx, alpha, Wg, Wu, Wd, A, route_mask=mask)
        assert _rel(Ym, refm) < 1e-12


def check_ffn_special(orc):
    rng = _rng(42)
    T, d, f = 10, 32, 48
    X = rng.standard_normal((T, d), dtype=np.float32)
    A = rng.standard_normal((T, d), dtype=np.float32)
    Wg, Wu, Wd = _layer_weights(rng, 1, d, f, std=0.2, bf16=False)
    # E = 1, k = 1: the textbook dense SwiGLU FFN, y = A + W2 (silu(W1 x) * (W3 x))
    idx = np.zeros((T, 1), dtype=np.int32)
    alpha = np.ones((T, 1))
    Y = orc.expert_ffn(X, idx, alpha, Wg, Wu, Wd, A)
    x = X.astype(np.float64)
    g = x @ Wg[0].T.astype(np.float64)
    ref = A + ((g / (1 + np.exp(-g))) * (x @ Wu[0].T.astype(np.float64))) @ Wd[0].T.astype(np.float64)
    assert _rel(Y, ref) < 1e-12
    # W_up = 0 leaves the residual untouched, bit for bit
    Y0 = orc.expert_ffn(X, idx, alpha, Wg, np.zeros_like(Wu), Wd, A)
    assert np.array_equal(Y0, A.astype(np.float64))
    # W_down doubled doubles the output exactly (zero residual)
    E, k = 6, 2
    Wg, Wu, Wd = _layer_weights(rng, E, d, f, std=0.2)
    idx, alpha = _random_routes(rng, T, E, k)
    Y1 = orc.expert_ffn(X, idx, alpha, Wg, Wu, Wd, None)
    Y2 = orc.expert_ffn(X, idx, alpha, Wg, Wu, 2 * Wd, None)
    assert np.array_equal(Y2, 2 * Y1)
    # relabelling the experts consistently changes nothing, bit for bit
    perm = rng.permutation(E)
    inv = np.argsort(perm)
    Yp = orc.expert_ffn(X, inv[idx].astype(np.int32), alpha, Wg[perm], Wu[perm], Wd[perm], A)
    Y = orc.expert_ffn(X, idx, alpha, Wg, Wu, Wd, A)
    assert np.array_equal(Yp, Y)
    # permuting the hidden units of every expert leaves y unchanged (up to rounding)
    pf = rng.permutation(f)
    Yf = orc.expert_ffn(X, idx, alpha, Wg[:, pf], Wu[:, pf], Wd[:, :, pf], A)
    assert _rel(Yf, Y) < 1e-13


# ------------------------------------------ fp8 weights (weight-only) --
def check_fp8_decode(orc):
    """Every e4m3 code against PyTorch's own float8_e4m3fn conversion (an
    independent implementation of the same OCP format), plus closed-form
    anchors of the format."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = orc.fp8e4m3_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
               0x3C: 1.5, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in anchors.items():
        assert got[c] == v, (hex(c), got[c], v)
    assert np.signbit(got[0x80]) and got[0x80] == 0.0 and not np.signbit(got[0x00])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.all(np.diff(got[:0x7F].astype(np.float64)) > 0)          # positive codes ascend
    assert np.array_equal(got[0x80:0xFF], -got[:0x7F])                  # sign bit negates


def check_mxfp4_decode(orc):
    """MXFP4: every E2M1 code against the OCP table (golden fixture), every
    E8M0 scale against PyTorch's float8_e8m0fnu conversion (an independent
    implementation), the nibble order and the 32-wide scale blocks on a
    hand-made row."""
    import torch
    table = np.array(_load("mxfp4_e2m1.json")["e2m1"], dtype=np.float32)
    # all 16 codes as the low and as the high nibble, scale 2^0
    codes = np.array([[c | (c << 4) for c in range(16)]], dtype=np.uint8)   # K = 32
    got = orc.mxfp4_decode(codes, np.array([[127]], dtype=np.uint8))[0]
    assert np.array_equal(got[0::2].view(np.uint32), table.view(np.uint32))
    assert np.array_equal(got[1::2].view(np.uint32), table.view(np.uint32))
    # nibble order: byte 0x21 holds element 0 = code 1 (0.5) and element 1 = code 2 (1.0)
    row = np.zeros((1, 16), dtype=np.uint8)
    row[0, 0] = 0x21
    v = orc.mxfp4_decode(row, np.array([[127]], dtype=np.uint8))[0]
    assert v[0] == 0.5 and v[1] == 1.0 and np.all(v[2:] == 0.0)
    # scales: code 2 (1.0) times every E8M0 value; block k // 32 takes scale k // 32
    sc = np.arange(256, dtype=np.uint8)
    ones = np.full((256, 16), 0x22, dtype=np.uint8)                         # K = 32, all 1.0
    got = orc.mxfp4_decode(ones, sc[:, None])[:, 0]
    ref = torch.from_numpy(sc.copy()).view(torch.float8_e8m0fnu).float().numpy()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~fin)
    assert np.array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    two = np.full((1, 32), 0x22, dtype=np.uint8)                            # K = 64: two blocks
    v = orc.mxfp4_decode(two, np.array([[127, 130]], dtype=np.uint8))[0]
    assert np.all(v[:32] == 1.0) and np.all(v[32:] == 8.0)


def check_ffn_row_scales(orc):
    """Weights given as fp8 code values with per-row scales equal the dense
    fp64 brute force on value * scale; unit scales change nothing."""
    rng = _rng(43)
    T, d, f, E, k = 12, 64, 96, 5, 2
    X = _bf16_values(rng.standard_normal((T, d), dtype=np.float32))
    A = rng.standard_normal((T, d), dtype=np.float32)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    qg, qu = (orc.fp8e4m3_decode(rng.choice(finite, size=(E, f, d))) for _ in range(2))
    qd = orc.fp8e4m3_decode(rng.choice(finite, size=(E, d, f)))
    Sg, Su = (np.exp(rng.uniform(-9, -5, size=(E, f))).astype(np.float32) for _ in range(2))
    Sd = np.exp(rng.uniform(-9, -5, size=(E, d))).astype(np.float32)
    idx, alpha = _random_routes(rng, T, E, k)
    Y = orc.expert_ffn(X, idx, alpha, qg, qu, qd, A, scales=(Sg, Su, Sd))
    ref = dense_brute_force(X, idx, alpha, qg.astype(np.float64) * Sg[:, :, None].astype(np.float64),
                            qu.astype(np.float64) * Su[:, :, None].astype(np.float64),
                            qd.astype(np.float64) * Sd[:, :, None].astype(np.float64), A)
    assert _rel(Y, ref) < 1e-12, _rel(Y, ref)
    ones = (np.ones((E, f), np.float32), np.ones((E, f), np.float32), np.ones((E, d), np.float32))
    assert np.array_equal(orc.expert_ffn(X, idx, alpha, qg, qu, qd, A, scales=ones),
                          orc.expert_ffn(X, idx, alpha, qg, qu, qd, A))


def check_layer_chain(orc):
    """The whole chain on a tiny layer equals the brute-force chain."""
    rng = _rng(51)
    T, d, f, E, k = 20, 64, 64, 8, 2
    X = rng.standard_normal((T, d), dtype=np.float32)
    Wr = rng.standard_normal((d, E), dtype=np.float32) * np.float32(0.3)
    Wg, Wu, Wd = _layer_weights(rng, E, d, f, std=0.2)
    A = rng.standard_normal((T, d), dtype=np.float32)
    out = orc.layer(X, Wr, None, Wg, Wu, Wd, A, k, 0, True)
    L = out["logits"]
    idx_b = _lexsort_topk(L, k)
    assert np.array_equal(out["idx"], idx_b)
    sm = softmax(L.astype(np.float64), axis=1)
    a = np.take_along_axis(sm, idx_b.astype(np.int64), 1)
    a = a / a.sum(axis=1, keepdims=True)
    ref = dense_brute_force(X, idx_b, a, Wg, Wu, Wd, A)
    assert _rel(out["Y"], ref) < 1e-12
    assert out["n_valid"] == T * k


ALL_CHECKS = [check_router_golden, check_router_exact_integers, check_router_correct_rounding,
              check_router_error_bound,
              check_topk_bruteforce, check_topk_special, check_topk_nan_and_signed_zero, check_alpha,
              check_shared,
              check_route_map_golden, check_route_map_bruteforce, check_route_map_errors,
              check_ffn_dense_bruteforce, check_ffn_special, check_fp8_decode, check_mxfp4_decode,
              check_ffn_row_scales,
              check_layer_chain]
