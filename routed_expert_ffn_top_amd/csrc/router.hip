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

// blockDim = 256. EPAD = E rounded up to a power of two (<= 256);
// groups = 256 / EPAD token groups, each thread does NTOK tokens.
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
    const int tok_per_wg = groups * NTOK;
    const int tbase = blockIdx.x * tok_per_wg;

    // X slab: [tok_per_wg][KC + 1] (odd stride: different token rows sit in
    // different banks); W slab: [KC][E].
    extern __shared__ float smem[];
    float *xs = smem;
    float *ws = smem + tok_per_wg * (kRouterKC + 1);

    float acc[NTOK];
#pragma unroll
    for (int n = 0; n < NTOK; ++n) acc[n] = 0.0f;

    for (int i0 = 0; i0 < d; i0 += kRouterKC) {
        const int kc = min(kRouterKC, d - i0);
        for (int q = tid; q < tok_per_wg * kRouterKC; q += 256) {
            const int r = q / kRouterKC, c = q % kRouterKC;
            const int t = tbase + r;
            xs[r * (kRouterKC + 1) + c] =
                (t < T && c < kc) ? load_x<TX>(X + (int64_t)t * ldx + i0 + c) : 0.0f;
        }
        for (int q = tid; q < kRouterKC * E; q += 256) {
            const int r = q / E, c = q % E;
            ws[q] = (r < kc) ? Wr[(int64_t)(i0 + r) * E + c] : 0.0f;
        }
        __syncthreads();
        if (e < E) {
            for (int i = 0; i < kc; ++i) {
                const float w = ws[i * E + e];
#pragma unroll
                for (int n = 0; n < NTOK; ++n)
                    acc[n] = __builtin_fmaf(xs[(g + n * groups) * (kRouterKC + 1) + i], w, acc[n]);
            }
        }
        __syncthreads();
    }
    if (e < E) {
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
    int lg = 0;
    while ((1 << lg) < s.E) ++lg;
    const int groups = 256 >> lg;
    const bool many = s.E >= 32;
    const int ntok = many ? 4 : 1;
    const int tok_per_wg = groups * ntok;
    const dim3 grid((s.T + tok_per_wg - 1) / tok_per_wg);
    const size_t shmem = (size_t)(tok_per_wg * (kRouterKC + 1) + kRouterKC * s.E) * sizeof(float);
    if (s.dtype == MOE_DT_BF16) {
        if (many)
            hipLaunchKernelGGL((k_router_logits<uint16_t, 4>), grid, dim3(256), shmem, st,
                               (const uint16_t *)X, s.ldx, Wr, bias, L, s.T, s.d, s.E, lg);
        else
            hipLaunchKernelGGL((k_router_logits<uint16_t, 1>), grid, dim3(256), shmem, st,
                               (const uint16_t *)X, s.ldx, Wr, bias, L, s.T, s.d, s.E, lg);
    } else {
        if (many)
            hipLaunchKernelGGL((k_router_logits<float, 4>), grid, dim3(256), shmem, st,
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
