// Router logits and top-k routing (EStream, section 2.2: a router assigns
// each token to the top-k of E experts; the per-route weight alpha scales the
// expert output in Eq. 2).
//
// Router: L[t][e] = fp32 fused multiply-add chain over the hidden index in
// ascending order, then + bias[e]. The chain is not split or reassociated:
// the top-k decision is taken on these bits, so they must be reproducible.
// Each thread owns one expert column for NTOK tokens; a workgroup stages a
// 64-wide slab of X (as fp32) and of W_r in LDS and sweeps it.
//
// Top-k: one wave64 per token; each lane owns experts lane, lane+64, ...
// An expert's rank is the number of experts with a larger logit plus the
// number of lower-id experts with an equal logit, so ranks are unique and
// ties go to the lower id; the experts of rank < k are the selection, in
// rank order. Softmax max/sum use fixed xor-butterfly reductions.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(((uint32_t)h) << 16);
}

template <typename TX>
__device__ __forceinline__ float load_x(const TX *p);
template <>
__device__ __forceinline__ float load_x<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

constexpr int kRouterKC = 64;   // hidden-index slab per LDS pass
constexpr int kXS = kRouterKC + 4;   // padded row stride (floats) of both slabs

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// blockDim = 256. EPAD = E rounded up to a power of two (<= 64 here; larger
// E uses several lanes' worth of rows); thread (g, e) owns expert e of NTOK
// tokens g, g + groups, ... with groups = 256 / EPAD. Per 64-wide hidden slab
// the workgroup stages X (as fp32, row per token) and W_r transposed (row per
// expert) in LDS, double-buffered, with the next slab's global loads in
// flight while the current one is used. Each thread reads 4 consecutive
// hidden indices of its expert row and of each token row as 16-byte LDS
// reads and applies the 4 fused multiply-adds in ascending order, so every
// logit is exactly the sequential fp32 chain.
template <typename TX, int NTOK>
__global__ __launch_bounds__(256) void k_router_logits(const TX *__restrict__ X, int64_t ldx,
                                                       const float *__restrict__ Wr,
                                                       const float *__restrict__ bias,
                                                       float *__restrict__ L, int T, int d, int E,
                                                       int epad_log2)
{
    const int epad = 1 << epad_log2;
    const int groups = 256 / epad;
    const int tid = threadIdx.x;
    const int e = tid & (epad - 1);
    const int g = tid >> epad_log2;
    const int tpw = groups * NTOK;           // tokens per workgroup
    const int tbase = blockIdx.x * tpw;

    extern __shared__ float smem[];
    // [2][tpw][kXS] token slabs, then [2][E][kXS] transposed weight slabs
    float *xs = smem;
    float *ws = smem + 2 * tpw * kXS;

    float acc[NTOK];
#pragma unroll
    for (int n = 0; n < NTOK; ++n) acc[n] = 0.0f;

    const int nfull = d / kRouterKC;
    // global -> register staging: each thread moves up to 4 X values and up
    // to 16 W values per slab (tpw*64 <= 2048 and 64*E <= 4096 elements).
    constexpr int XR = 8, WR = 16;
    float xr[XR], wr[WR];
    auto gload = [&](int c) {
        const int i0 = c * kRouterKC;
#pragma unroll
        for (int q = 0; q < XR; ++q) {
            const int id = q * 256 + tid;
            const int r = id / kRouterKC, col = id % kRouterKC, t = tbase + r;
            xr[q] = (r < tpw && t < T) ? load_x<TX>(X + (int64_t)t * ldx + i0 + col) : 0.0f;
        }
#pragma unroll
        for (int q = 0; q < WR; ++q) {
            const int id = q * 256 + tid;
            const int r = id / E, col = id % E;
            wr[q] = (r < kRouterKC) ? Wr[(int64_t)(i0 + r) * E + col] : 0.0f;
        }
    };
    auto sstore = [&](int buf) {
        float *xb = xs + buf * tpw * kXS;
        float *wb = ws + buf * E * kXS;
#pragma unroll
        for (int q = 0; q < XR; ++q) {
            const int id = q * 256 + tid;
            const int r = id / kRouterKC, col = id % kRouterKC;
            if (r < tpw) xb[r * kXS + col] = xr[q];
        }
#pragma unroll
        for (int q = 0; q < WR; ++q) {
            const int id = q * 256 + tid;
            const int r = id / E, col = id % E;
            if (r < kRouterKC) wb[col * kXS + r] = wr[q];
        }
    };

    if (nfull > 0) {
        gload(0);
        sstore(0);
    }
    __syncthreads();
    for (int c = 0; c < nfull; ++c) {
        const int buf = c & 1;
        if (c + 1 < nfull) gload(c + 1);
        if (e < E) {
            const float *wrow = ws + buf * E * kXS + e * kXS;
            const float *xb = xs + buf * tpw * kXS;
#pragma unroll
            for (int i = 0; i < kRouterKC; i += 4) {
                const f32x4_t w4 = *(const f32x4_t *)(wrow + i);
#pragma unroll
                for (int n = 0; n < NTOK; ++n) {
                    const f32x4_t x4 = *(const f32x4_t *)(xb + (g + n * groups) * kXS + i);
                    acc[n] = __builtin_fmaf(x4.x, w4.x, acc[n]);
                    acc[n] = __builtin_fmaf(x4.y, w4.y, acc[n]);
                    acc[n] = __builtin_fmaf(x4.z, w4.z, acc[n]);
                    acc[n] = __builtin_fmaf(x4.w, w4.w, acc[n]);
                }
            }
        }
        if (c + 1 < nfull) sstore(buf ^ 1);
        __syncthreads();
    }
    // tail (d not a multiple of 64): straight from global memory, in order
    if (e < E) {
        for (int i = nfull * kRouterKC; i < d; ++i) {
            const float w = Wr[(int64_t)i * E + e];
#pragma unroll
            for (int n = 0; n < NTOK; ++n) {
                const int t = tbase + g + n * groups;
                if (t < T) acc[n] = __builtin_fmaf(load_x<TX>(X + (int64_t)t * ldx + i), w, acc[n]);
            }
        }
        const float b = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int n = 0; n < NTOK; ++n) {
            const int t = tbase + g + n * groups;
            if (t < T) L[(int64_t)t * E + e] = bias ? acc[n] + b : acc[n];
        }
    }
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

constexpr int kTopkMaxPerLane = 4;   // E <= 256

// blockDim = 256: 4 waves, one token each. Writes ranks 0..k-1 (routed) and
// k..K'-1 (shared) of idx/w for the tokens in [t0, t0 + nt).
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ L, int E, int k,
                                              int n_shared, int renorm, int t0, int nt,
                                              int32_t *__restrict__ idx, float *__restrict__ w,
                                              int32_t *__restrict__ done)
{
    __shared__ float vals[4][256];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tl = blockIdx.x * 4 + wave;
    const bool active = tl < nt;
    const int t = t0 + (active ? tl : 0);
    const int kp = k + n_shared;
    const float NEG_INF = -__builtin_huge_valf();

    float v[kTopkMaxPerLane];
#pragma unroll
    for (int c = 0; c < kTopkMaxPerLane; ++c) {
        const int e = lane + 64 * c;
        float x = NEG_INF;
        if (e < E) {
            x = L[(int64_t)t * E + e];
            if (x != x) x = NEG_INF;  // NaN counts as -infinity
            vals[wave][e] = x;
        }
        v[c] = x;
    }
    __syncthreads();
    if (!active) return;

    int rank[kTopkMaxPerLane];
#pragma unroll
    for (int c = 0; c < kTopkMaxPerLane; ++c) rank[c] = 0;
    for (int e2 = 0; e2 < E; ++e2) {
        const float x2 = vals[wave][e2];
#pragma unroll
        for (int c = 0; c < kTopkMaxPerLane; ++c) {
            const int e = lane + 64 * c;
            rank[c] += (x2 > v[c]) || (x2 == v[c] && e2 < e);
        }
    }

    float m = NEG_INF;
#pragma unroll
    for (int c = 0; c < kTopkMaxPerLane; ++c) m = fmaxf(m, v[c]);
    m = wave_max(m);
    if (m == NEG_INF) m = 0.0f;
    float z[kTopkMaxPerLane];
    float s = 0.0f, ssel = 0.0f;
#pragma unroll
    for (int c = 0; c < kTopkMaxPerLane; ++c) {
        const int e = lane + 64 * c;
        z[c] = (e < E) ? expf(v[c] - m) : 0.0f;
        s += z[c];
        if (e < E && rank[c] < k) ssel += z[c];
    }
    s = wave_sum(s);
    ssel = wave_sum(ssel);
    const float den = renorm ? ssel : s;
#pragma unroll
    for (int c = 0; c < kTopkMaxPerLane; ++c) {
        const int e = lane + 64 * c;
        if (e < E && rank[c] < k) {
            idx[(int64_t)t * kp + rank[c]] = e;
            w[(int64_t)t * kp + rank[c]] = den > 0.0f ? z[c] / den : 0.0f;
        }
    }
    if (lane < n_shared) {
        idx[(int64_t)t * kp + k + lane] = E + lane;
        w[(int64_t)t * kp + k + lane] = 1.0f;
    }
    if (done && lane < kp) done[(int64_t)t * kp + lane] = 0;
}

}  // namespace

hipError_t launch_router_logits(const moe_shape &s, const void *X, const float *Wr,
                                const float *bias, float *L, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    int lg = 3;  // at least 8 expert lanes: at most 32 token groups per workgroup
    while ((1 << lg) < s.E) ++lg;
    if (lg > 6) return hipErrorInvalidValue;  // E <= 64 (checked by the caller)
    const int groups = 256 >> lg;
    const bool many = s.E >= 32;
    const int ntok = many ? 2 : 1;
    const int tpw = groups * ntok;            // <= 256 / EPAD * 2 <= 32 tokens
    const dim3 grid((s.T + tpw - 1) / tpw);
    const size_t shmem = (size_t)2 * (tpw + s.E) * kXS * sizeof(float);
    if (s.dtype == MOE_DT_BF16) {
        if (many)
            hipLaunchKernelGGL((k_router_logits<uint16_t, 2>), grid, dim3(256), shmem, st,
                               (const uint16_t *)X, s.ldx, Wr, bias, L, s.T, s.d, s.E, lg);
        else
            hipLaunchKernelGGL((k_router_logits<uint16_t, 1>), grid, dim3(256), shmem, st,
                               (const uint16_t *)X, s.ldx, Wr, bias, L, s.T, s.d, s.E, lg);
    } else {
        if (many)
            hipLaunchKernelGGL((k_router_logits<float, 2>), grid, dim3(256), shmem, st,
                               (const float *)X, s.ldx, Wr, bias, L, s.T, s.d, s.E, lg);
        else
            hipLaunchKernelGGL((k_router_logits<float, 1>), grid, dim3(256), shmem, st,
                               (const float *)X, s.ldx, Wr, bias, L, s.T, s.d, s.E, lg);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const moe_shape &s, int t0, int nt, const float *L, int32_t *idx,
                       float *w, int32_t *done, hipStream_t st)
{
    if (nt == 0) return hipSuccess;
    const dim3 grid((nt + 3) / 4);
    hipLaunchKernelGGL(k_topk, grid, dim3(256), 0, st, L, s.E, s.k, s.n_shared, s.renorm, t0,
                       nt, idx, w, done);
    return hipGetLastError();
}

}  // namespace moe
