// Router logits and top-k routing (EStream, section 2.2: a router assigns
// each token to the top-k of E experts; the per-route weight alpha scales the
// expert output in Eq. 2).
//
// Router: L[t][e] = sum over the hidden index of x * w in fp32, each term one
// fused multiply-add, in a fixed order: runs of 8 consecutive hidden indices,
// run r feeding partial sum r mod 16, each partial sum ascending in the index
// from 0, the 16 partial sums added in ascending order, then + bias[e]. The
// top-k decision is taken on these bits, so the order is part of the result.
//
// Top-k: one wave64 per token; each lane owns experts lane, lane+64, ...
// An expert's rank is the number of experts with a larger logit plus the
// number of lower-id experts with an equal logit, so ranks are unique and
// ties go to the lower id; the experts of rank < k are the selection, in
// rank order. Softmax max/sum use fixed xor-butterfly reductions.
#include "common.h"

namespace moe {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Workgroup barrier that publishes this wave's LDS writes (lgkmcnt(0)) but
// leaves its global loads in flight; __syncthreads would also drain those.
// gfx9 s_waitcnt encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] at bits 15:14.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    __builtin_amdgcn_s_barrier();
}

// Router logits on the fp32 matrix cores. v_mfma_f32_4x4x1_16b performs 16
// independent 4 x 4 outer-product updates D_b += A_b B_b^T: lane l supplies
// A_b[l % 4] and B_b[l % 4] of block b = l / 4 and holds D_b[r][l % 4] in its
// register r. Each update is one fused multiply-add per element, so every
// accumulator element is an fmaf chain (checked bit for bit against fmaf,
// signed zeros and denormals included).
//
// Block b is partial sum b of the logit. At step s (0..7) of hidden group g
// (128 indices), lane l works on hidden index (16 g + b) * 8 + s: run 16 g + b
// of 8 consecutive indices, which feeds partial sum (16 g + b) mod 16 = b, and
// within a run the indices ascend. Rows of a block are 4 tokens, columns 4
// experts.
//
// A wave owns TQ token quads x 4 expert quads (4 TQ tokens x 16 experts, 4 TQ
// independent accumulators, so consecutive instructions do not wait on each
// other); the 4 waves of a workgroup take 4 consecutive token blocks of the
// same 16 experts (grid: ceil(T / (16 TQ)) x ceil(E / 16)).
//   x: each lane loads its run of each of its token rows (8 values) into a
//      register ring PF groups deep; the 16 lanes that share a row read 16
//      adjacent runs, so every load reads whole contiguous row segments.
//   W_r: the 16 expert rows of a group (8 KB) are shared by the 4 waves
//      through a ring of NB LDS buffers. Each wave fetches a quarter of group
//      g + 2 into registers and writes its quarter of group g + 1 into LDS
//      while it multiplies group g; one barrier per group publishes the
//      writes and frees the buffer the next writes take.
// The loads of a group are spread between the multiplies of the previous one
// so that the matrix pipe keeps busy while they queue.
//
// Hidden indices at or past d are taken as x = -0 and w = +0: the product is
// -0, and a + (-0) = a for every a, +0 and -0 included, so padded steps leave
// the chains unchanged. Token and expert rows past T and E are clamped to the
// last row and their results dropped. At the end the 16 partial sums of each
// (token, expert) pass through LDS and are added in ascending order, then the
// bias.
template <typename TX, int TQ, bool FULL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_router_logits(
    const TX *__restrict__ X, int64_t ldx, const float *__restrict__ Wr, const float *__restrict__ bias,
    float *__restrict__ L, int T, int d, int E)
{
    constexpr int XV = sizeof(TX) == 2 ? 1 : 2;   // 16-byte pieces per run of 8 x values
    constexpr int XE = 16 / sizeof(TX);            // x values per piece
#ifdef MOE_ROUTER_PF
    constexpr int PF = MOE_ROUTER_PF;
#else
    constexpr int PF = TQ == 1 ? 4 : 3;            // x ring depth in groups (measured best)
#endif
    constexpr int NB = 3;                          // W_r ring depth in groups (LDS)
    constexpr int U = PF * 2;                      // main-loop unroll: a multiple of PF and of 2
    constexpr int RS = 64 * TQ + 4;                // LDS stride of one partial sum (bank spread)
    constexpr uint32_t XPAD = sizeof(TX) == 2 ? 0x80008000u : 0x80000000u;   // -0 in every x slot
    __shared__ u32x4_t wbuf[NB][512];              // 16 expert rows x 16 runs x 2 halves of 16 bytes
    __shared__ float red[4][16 * RS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int b = lane >> 2, q = lane & 3;
    const int t0 = (blockIdx.x * 4 + wave) * (4 * TQ);
    const int e0 = blockIdx.y * 16;
    const int ng = (d + 127) >> 7;

    // LDS slot of (expert row r, run b, half h) of a group: row-major, the 32
    // pieces of a row rotated by rot(r % 4) = 8 (r & 1) + (r & 2) / 2, so that
    // the 16 lanes of a read (runs b0..b0+3 of rows 4v..4v+3, one half) hit 16
    // distinct 16-byte bank groups.
    auto rot = [](int r) { return 8 * (r & 1) + ((r >> 1) & 1); };
    int rslot[4][2];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int h = 0; h < 2; ++h) rslot[v][h] = (4 * v + q) * 32 + ((2 * b + h + rot(q)) & 31);
    // this lane's two pieces of every group: slot S = (2 wave + k) * 64 + lane
    // holds 4 weights of expert row r at hidden index g * 128 + wcol[k]
    const float *wrow_s[2];
    int wslot[2], wcol[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int S = (2 * wave + k) * 64 + lane, r = S >> 5;
        const int p = ((S & 31) - rot(r)) & 31;   // 2 * run + half
        wslot[k] = S;
        wrow_s[k] = Wr + (int64_t)min(e0 + r, E - 1) * d;
        wcol[k] = (p >> 1) * 8 + (p & 1) * 4;
    }

    const TX *xrow[TQ];
#pragma unroll
    for (int u = 0; u < TQ; ++u) xrow[u] = X + (int64_t)min(t0 + 4 * u + q, T - 1) * ldx;

    // Loads of group g are clamped to the last group (a re-read whose values
    // are not used). With FULL (d % 128 == 0) every run is inside the row;
    // else a piece at or past d is read from the row start (x: replaced by
    // the pad here; w: masked where it is read), so no load depends on a
    // branch.
    auto load_x = [&](int g, int j, u32x4_t (&xv)[TQ][XV]) {
        const int u = j / XV, h = j % XV;
        const int i = min(g, ng - 1) * 128 + b * 8 + h * XE;
        if (FULL) {
            xv[u][h] = *(const u32x4_t *)(xrow[u] + i);
        } else {
            const bool in = i < d;
            const u32x4_t v = *(const u32x4_t *)(xrow[u] + (in ? i : 0));
#pragma unroll
            for (int c = 0; c < 4; ++c) xv[u][h][c] = in ? v[c] : XPAD;
        }
    };
    auto load_w = [&](int g, int k, u32x4_t (&wt)[2]) {
        const int i = min(g, ng - 1) * 128 + wcol[k];   // d % 4 == 0: a piece is inside the row or past it
        wt[k] = *(const u32x4_t *)(wrow_s[k] + (FULL || i < d ? i : 0));
    };
    auto read_w = [&](int g, u32x4_t (&wv)[4][2]) {
        const u32x4_t *buf = wbuf[g % NB];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                wv[v][h] = buf[rslot[v][h]];
                if (!FULL && g * 128 + b * 8 + h * 4 >= d) wv[v][h] = u32x4_t{0, 0, 0, 0};
            }
    };

    f32x4_t acc[TQ][4];
#pragma unroll
    for (int u = 0; u < TQ; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // One group: 8 hidden steps x 4 TQ blocks x 4 expert quads of multiplies.
    // Spread between them: the x loads of group g + PF - 1 into the x slot
    // that group g - 1 released, the W_r loads of group g + 2 into wn, and the
    // LDS writes of group g + 1 from wp. LOADS = false: none of these.
    constexpr int NX = TQ * XV;
    auto group = [&](int g, const u32x4_t (&xv)[TQ][XV], u32x4_t (&xn)[TQ][XV], u32x4_t (&wn)[2],
                     const u32x4_t (&wp)[2], bool loads) {
        lds_barrier();   // group g's rows are in LDS; the buffer of group g + 1 - NB is free
        u32x4_t wv[4][2];
        read_w(g, wv);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            float a[TQ];
#pragma unroll
            for (int u = 0; u < TQ; ++u) {
                if (sizeof(TX) == 2) {
                    const uint32_t w2 = xv[u][0][s >> 1];
                    a[u] = __uint_as_float((s & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
                } else {
                    a[u] = __uint_as_float(xv[u][s >> 2][s & 3]);
                }
            }
#pragma unroll
            for (int u = 0; u < TQ; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[u][v] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[u], __uint_as_float(wv[v][s >> 2][s & 3]),
                                                                  acc[u][v], 0, 0, 0);
            if (loads) {
#pragma unroll
                for (int j = s * NX / 8; j < (s + 1) * NX / 8; ++j) load_x(g + PF - 1, j, xn);
                if (s == 1 || s == 5) load_w(g + 2, s >> 2, wn);
                if (s == 3 || s == 7) wbuf[(g + 1) % NB][wslot[s >> 2]] = wp[s >> 2];
            }
            __builtin_amdgcn_sched_barrier(0);   // keep this step's loads between its multiplies and the next step's
        }
    };

    // prologue: x groups 0 .. PF-2 into x slots; W_r group 0 into LDS, group 1 into registers
    u32x4_t xr[PF][TQ][XV], wt[2][2];
#pragma unroll
    for (int u = 0; u < PF - 1; ++u)
#pragma unroll
        for (int j = 0; j < NX; ++j) load_x(u, j, xr[u]);
#pragma unroll
    for (int k = 0; k < 2; ++k) load_w(0, k, wt[0]);
#pragma unroll
    for (int k = 0; k < 2; ++k) load_w(1, k, wt[1]);
#pragma unroll
    for (int k = 0; k < 2; ++k) wbuf[0][wslot[k]] = wt[0][k];

    // x slot g % PF holds group g; W_r registers wt[g % 2] hold group g + 1
    // (written to LDS during group g) and then take group g + 2.
    int g0 = 0;
    for (; g0 + U <= ng; g0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            group(g0 + u, xr[u % PF], xr[(u + PF - 1) % PF], wt[u % 2], wt[(u + 1) % 2], true);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
        if (g0 + u < ng) group(g0 + u, xr[u % PF], xr[(u + PF - 1) % PF], wt[u % 2], wt[(u + 1) % 2], true);

    // partial sum b of (token 4u + r, expert 4v + q) -> red[b][(4u + r) * 16 + 4v + q]
    float *rw = red[wave];
#pragma unroll
    for (int u = 0; u < TQ; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int r = 0; r < 4; ++r) rw[b * RS + (4 * u + r) * 16 + 4 * v + q] = acc[u][v][r];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TQ; ++j) {
        const int o = lane + 64 * j;
        const int t = t0 + (o >> 4), e = e0 + (o & 15);
        float s = rw[o];
#pragma unroll
        for (int c = 1; c < 16; ++c) s = s + rw[c * RS + o];
        if (t < T && e < E) L[(int64_t)t * E + e] = bias ? s + bias[e] : s;
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

// Order-preserving 64-bit key of (logit, expert): a larger key means a larger
// logit, or an equal logit and a lower expert id. NaN is taken as -infinity
// and -0 as +0, so equal logits give equal high words.
__device__ __forceinline__ uint64_t topk_key(float x, int e)
{
    if (x != x) x = -__builtin_huge_valf();
    if (x == 0.0f) x = 0.0f;
    const uint32_t u = __float_as_uint(x);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)e;
}

// Top-k for one token per wave; lane l holds experts l, l+64, ... (C per
// lane, C = ceil(E/64)). An expert's rank is the number of experts with a
// larger key: ranks are unique, ties go to the lower id, and the experts of
// rank < k are the selection in rank order. Softmax max and sums use fixed
// xor-butterfly reductions.
template <int C>
__global__ __launch_bounds__(256) void k_topk(const float *__restrict__ L, int E, int k,
                                              int n_shared, int renorm, int t0, int nt,
                                              int32_t *__restrict__ idx, float *__restrict__ w,
                                              int32_t *__restrict__ done)
{
    __shared__ uint64_t keys[4][64 * C + 2];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int tl = blockIdx.x * 4 + wave;
    const bool active = tl < nt;
    const int t = t0 + (active ? tl : 0);
    const int kp = k + n_shared;
    const float NEG_INF = -__builtin_huge_valf();

    float v[C];
    uint64_t key[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = lane + 64 * c;
        float x = NEG_INF;
        if (e < E) {
            x = L[(int64_t)t * E + e];
            if (x != x) x = NEG_INF;
        }
        v[c] = x;
        key[c] = topk_key(x, e);
        keys[wave][e] = e < E ? key[c] : 0ull;   // padding keys rank below every expert
    }
    if (lane < 2) keys[wave][64 * C + lane] = 0ull;
    __syncthreads();
    if (!active) return;

    int rank[C];
#pragma unroll
    for (int c = 0; c < C; ++c) rank[c] = 0;
    const int E2 = (E + 1) & ~1;
    for (int e2 = 0; e2 < E2; e2 += 2) {
        const uint64_t k0 = keys[wave][e2], k1 = keys[wave][e2 + 1];
#pragma unroll
        for (int c = 0; c < C; ++c) rank[c] += (int)(k0 > key[c]) + (int)(k1 > key[c]);
    }

    float m = NEG_INF;
#pragma unroll
    for (int c = 0; c < C; ++c) m = fmaxf(m, v[c]);
    m = wave_max(m);
    if (m == NEG_INF) m = 0.0f;
    float z[C];
    float s = 0.0f, ssel = 0.0f;
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int e = lane + 64 * c;
        z[c] = (e < E) ? expf(v[c] - m) : 0.0f;
        s += z[c];
        if (e < E && rank[c] < k) ssel += z[c];
    }
    s = wave_sum(s);
    ssel = wave_sum(ssel);
    const float den = renorm ? ssel : s;
#pragma unroll
    for (int c = 0; c < C; ++c) {
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

template <typename TX, int TQ>
hipError_t launch_router_t(const moe_shape &s, const void *X, const float *Wr, const float *bias, float *L,
                           hipStream_t st)
{
    const dim3 grid((s.T + 16 * TQ - 1) / (16 * TQ), (s.E + 15) / 16);
    if (s.d % 128 == 0)
        hipLaunchKernelGGL((k_router_logits<TX, TQ, true>), grid, dim3(256), 0, st, (const TX *)X, s.ldx, Wr, bias,
                           L, s.T, s.d, s.E);
    else
        hipLaunchKernelGGL((k_router_logits<TX, TQ, false>), grid, dim3(256), 0, st, (const TX *)X, s.ldx, Wr, bias,
                           L, s.T, s.d, s.E);
    return hipGetLastError();
}

hipError_t launch_router_logits(const moe_shape &s, const void *X, const float *Wr,
                                const float *bias, float *L, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    // token quads per wave: 4 (16 accumulators) while that still gives every
    // SIMD a wave, else fewer accumulators and more waves
    const int64_t eb = (s.E + 15) / 16;
    int tq = ((s.T + 15) / 16) * eb >= 1024 ? 4 : (((s.T + 7) / 8) * eb >= 1024 ? 2 : 1);
#ifdef MOE_ROUTER_TQ
    tq = MOE_ROUTER_TQ;
#endif
    if (act_bf16(s)) {
        if (tq == 4) return launch_router_t<uint16_t, 4>(s, X, Wr, bias, L, st);
        if (tq == 2) return launch_router_t<uint16_t, 2>(s, X, Wr, bias, L, st);
        return launch_router_t<uint16_t, 1>(s, X, Wr, bias, L, st);
    }
    if (tq == 4) return launch_router_t<float, 4>(s, X, Wr, bias, L, st);
    if (tq == 2) return launch_router_t<float, 2>(s, X, Wr, bias, L, st);
    return launch_router_t<float, 1>(s, X, Wr, bias, L, st);
}

hipError_t launch_topk(const moe_shape &s, int t0, int nt, const float *L, int32_t *idx,
                       float *w, int32_t *done, hipStream_t st)
{
    if (nt == 0) return hipSuccess;
    const dim3 grid((nt + 3) / 4);
    if (s.E <= 64)
        hipLaunchKernelGGL(k_topk<1>, grid, dim3(256), 0, st, L, s.E, s.k, s.n_shared, s.renorm, t0, nt, idx, w,
                           done);
    else if (s.E <= 128)
        hipLaunchKernelGGL(k_topk<2>, grid, dim3(256), 0, st, L, s.E, s.k, s.n_shared, s.renorm, t0, nt, idx, w,
                           done);
    else
        hipLaunchKernelGGL(k_topk<4>, grid, dim3(256), 0, st, L, s.E, s.k, s.n_shared, s.renorm, t0, nt, idx, w,
                           done);
    return hipGetLastError();
}

}  // namespace moe
