// Route map per physical slot (EStream, section 3.2, Algorithm 1 and the
// compressed-sparse-row route representation): psi_i = Phi(e_i); per-slot
// counts; prefix-sum offsets; records (t_i, i) stored contiguously by slot in
// ascending route order.
//
// The sequential cursor pass is made parallel as a stable counting sort:
//   count  - routes are cut into blocks of 256 consecutive route ids. Inside
//            a block each route gets its stable rank among the block's routes
//            of the same slot: within a wave64 from a ballot match of the
//            slot key (popcount of the same-key lanes below it), across the
//            block's 4 waves from per-wave counts in LDS. The block's
//            per-slot counts go to blk[b][s].
//   place  - each block first forms its absolute bases from the whole blk
//            matrix: base[b][s] = offset[s] + sum_{b' < b} blk[b'][s], with
//            offset the exclusive prefix over slots of the column sums (block
//            0 also writes count[s], offset[s] and offset[P]); then
//            p = base[b][psi_i] + rank_i gives exactly the position the
//            sequential cursor pass would give, since both order records of a
//            slot by ascending route id.
// All arithmetic is integer, so the descriptors are bit-exact and
// independent of scheduling.
#include <algorithm>

#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint64_t lanemask_lt(int lane)
{
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// blockDim = 256 = kRouteBlock.
__global__ __launch_bounds__(256) void k_route_count(const int32_t *__restrict__ idx, int64_t i0,
                                                     int64_t n, int n_exp, int P, PhiArg phi,
                                                     int32_t *__restrict__ blk,
                                                     int32_t *__restrict__ rank,
                                                     int32_t *__restrict__ err,
                                                     int32_t *__restrict__ done, int reset)
{
    __shared__ int32_t wcnt[4][kMaxExp];
    __shared__ int32_t sphi[kMaxExp];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    for (int q = tid; q < 4 * kMaxExp; q += 256) (&wcnt[0][0])[q] = 0;
    for (int q = tid; q < n_exp; q += 256) sphi[q] = phi.v[q];
    __syncthreads();

    const int64_t r = (int64_t)blockIdx.x * kRouteBlock + tid;  // route offset in the build
    const bool in_range = r < n;
    int psi = -1;
    if (in_range) {
        const int64_t i = i0 + r;
        const int e = idx[i];
        if (e >= 0 && e < n_exp) {
            psi = sphi[e];
        } else {
            atomicOr(err, MOE_DEVERR_EXPERT_ID);
        }
        if (reset) done[i] = 0;
    }
    // key in [0, P]; 0 = not placed
    const int key = psi + 1;
    int nbits = 0;
    while ((1 << nbits) <= P) ++nbits;
    uint64_t same = ~0ull;
    for (int b = 0; b < nbits; ++b) {
        const int bit = (key >> b) & 1;
        const uint64_t bal = __ballot(bit);
        same &= bit ? bal : ~bal;
    }
    const int wrank = __popcll(same & lanemask_lt(lane));
    if (psi >= 0 && wrank == 0) wcnt[wave][psi] = __popcll(same);
    __syncthreads();
    if (psi >= 0) {
        int before = wrank;
        for (int w = 0; w < wave; ++w) before += wcnt[w][psi];
        rank[r] = before;
    }
    for (int s = tid; s < P; s += 256)
        blk[(int64_t)blockIdx.x * P + s] = wcnt[0][s] + wcnt[1][s] + wcnt[2][s] + wcnt[3][s];
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// blockDim = 256 = kRouteBlock. blk holds the per-block slot counts of the
// count pass (nblk x P, unscanned).
__global__ __launch_bounds__(256) void k_route_place(const int32_t *__restrict__ idx, int64_t i0,
                                                     int64_t n, int kp, int n_exp, int P, int nblk,
                                                     PhiArg phi, const int32_t *__restrict__ blk,
                                                     const int32_t *__restrict__ rank,
                                                     int32_t *__restrict__ rec_token,
                                                     int32_t *__restrict__ rec_route,
                                                     int32_t *__restrict__ route_pos,
                                                     int32_t *__restrict__ count,
                                                     int32_t *__restrict__ offset)
{
    __shared__ int32_t sphi[kMaxExp];
    __shared__ int32_t part_before[4][64], part_tot[4][64];
    __shared__ int32_t sbase[kMaxExp], stot[kMaxExp];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x;
    for (int q = tid; q < n_exp; q += 256) sphi[q] = phi.v[q];
    // column sums of blk: all blocks (total) and blocks before this one;
    // 64 slots at a time, each wave summing every 4th block
    for (int s0 = 0; s0 < P; s0 += 64) {
        const int s = s0 + lane;
        int before = 0, tot = 0;
        if (s < P) {
#pragma unroll 8
            for (int b2 = wave; b2 < nblk; b2 += 4) {
                const int v = blk[(int64_t)b2 * P + s];
                tot += v;
                before += b2 < b ? v : 0;
            }
        }
        part_before[wave][lane] = before;
        part_tot[wave][lane] = tot;
        __syncthreads();
        if (wave == 0 && s < P) {
            sbase[s] = part_before[0][lane] + part_before[1][lane] + part_before[2][lane] + part_before[3][lane];
            stot[s] = part_tot[0][lane] + part_tot[1][lane] + part_tot[2][lane] + part_tot[3][lane];
        }
        __syncthreads();
    }
    // exclusive prefix over slots, added to the bases
    if (wave == 0) {
        int run = 0;
        for (int s0 = 0; s0 < P; s0 += 64) {
            const int s = s0 + lane;
            const int v = s < P ? stot[s] : 0;
            const int inc = wave_incl_scan(v, lane);
            if (s < P) {
                sbase[s] += run + inc - v;
                if (b == 0) {
                    count[s] = v;
                    offset[s] = run + inc - v;
                }
            }
            run += __shfl(inc, 63, 64);
        }
        if (b == 0 && lane == 0) offset[P] = run;
    }
    __syncthreads();
    const int64_t r = (int64_t)b * kRouteBlock + tid;
    if (r >= n) return;
    const int64_t i = i0 + r;
    const int e = idx[i];
    const int psi = (e >= 0 && e < n_exp) ? sphi[e] : -1;
    if (psi < 0) {
        route_pos[i] = -1;
        return;
    }
    const int p = sbase[psi] + rank[r];
    rec_token[p] = (int32_t)(i / kp);
    rec_route[p] = (int32_t)i;
    route_pos[i] = p;
}

// Routes per logical expert over n routes (integer atomics: order-free).
__global__ __launch_bounds__(256) void k_expert_hist(const int32_t *__restrict__ idx, int64_t n,
                                                     int n_exp, int32_t *__restrict__ count)
{
    __shared__ int32_t h[kMaxExp];
    for (int q = threadIdx.x; q < n_exp; q += 256) h[q] = 0;
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int e = idx[i];
        if (e >= 0 && e < n_exp) atomicAdd(&h[e], 1);
    }
    __syncthreads();
    for (int q = threadIdx.x; q < n_exp; q += 256)
        if (h[q]) atomicAdd(&count[q], h[q]);
}

__global__ void k_fill_i32(int32_t *p, int32_t v, int64_t n)
{
    const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (q < n) p[q] = v;
}

}  // namespace

hipError_t launch_route_count(const moe_shape &s, int64_t i0, int64_t n, const int32_t *idx,
                              const PhiArg &phi, int32_t *blk, int32_t *rank, int32_t *err,
                              int32_t *done, int reset, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const dim3 grid((unsigned)((n + kRouteBlock - 1) / kRouteBlock));
    hipLaunchKernelGGL(k_route_count, grid, dim3(kRouteBlock), 0, st, idx, i0, n,
                       s.E + s.n_shared, s.P, phi, blk, rank, err, done, reset);
    return hipGetLastError();
}

hipError_t launch_route_place(const moe_shape &s, int64_t i0, int64_t n, const int32_t *idx,
                              const PhiArg &phi, const int32_t *blk, const int32_t *rank,
                              int32_t *rec_token, int32_t *rec_route, int32_t *route_pos,
                              int32_t *count, int32_t *offset, hipStream_t st)
{
    // at least one block: block 0 writes count and offset even for n == 0
    const int nblk = (int)((n + kRouteBlock - 1) / kRouteBlock);
    hipLaunchKernelGGL(k_route_place, dim3(nblk > 0 ? nblk : 1), dim3(kRouteBlock), 0, st, idx, i0, n,
                       s.k + s.n_shared, s.E + s.n_shared, s.P, nblk, phi, blk, rank, rec_token, rec_route,
                       route_pos, count, offset);
    return hipGetLastError();
}

hipError_t launch_expert_hist(const moe_shape &s, const int32_t *idx, int64_t n, int32_t *count,
                              hipStream_t st)
{
    const int ne = s.E + s.n_shared;
    hipError_t e = launch_fill_i32(count, 0, ne, st);
    if (e != hipSuccess || n == 0) return e;
    const unsigned g = (unsigned)std::min<int64_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(k_expert_hist, dim3(g), dim3(256), 0, st, idx, n, ne, count);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int32_t v, int64_t n, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

}  // namespace moe
