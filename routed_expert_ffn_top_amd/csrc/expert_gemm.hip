// Grouped expert projections over the route map (EStream, section 3.2,
// "Fused Expert Execution": gather routed rows, gate/up projections as pairs,
// SwiGLU, down projection, weighted scatter; Eq. 1 F_e(x) = W_d (SiLU(W_g x)
// * (W_u x))).
//
// Work is a list of tiles (slot s, BM consecutive records of s, BN columns of
// the slot's weight slice). Each workgroup finds its tile from the per-slot
// record offsets, so the grid is launched for an upper bound and surplus
// workgroups leave at once; nothing is read back to the host.
//
//  gate/up: A = X rows gathered by rec_token (K = d), B = the slot's packed
//           [2f][d] gate/up slice, whose rows alternate 32 gate / 32 up, so a
//           wave's 32-column MFMA tiles come in (gate, up) pairs for the same
//           hidden units; the epilogue writes H[p] = SiLU(g) * u.
//  down:    A = H rows (consecutive records, K = f), B = the slot's [d][f]
//           down slice; the epilogue writes Yr[rec_route[p]] = alpha * out,
//           a private row per route (no atomics), and marks the route done.
//
// Tile order: inside a slot, tiles of one column block are consecutive (they
// share the weight tile), and a slot's tiles are consecutive (they share the
// gathered rows). Workgroup ids are dealt round-robin to the 8 XCDs, so the
// logical tile index is remapped to give each XCD one contiguous range of
// tiles: the sharing happens in that XCD's own L2.
#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct TileInfo {
    int slot, row0, rows, n0;
};

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

constexpr int kXcd = 8;

// bid in [0, total) -> logical tile; XCD x = bid % 8 gets the contiguous
// logical range [x*q + min(x, r), ...) with q = total / 8, r = total % 8.
__device__ __forceinline__ int xcd_remap(int bid, int total)
{
    const int q = total / kXcd, r = total % kXcd;
    const int x = bid % kXcd, pos = bid / kXcd;
    return x * q + min(x, r) + pos;
}

// Wave 0 finds this workgroup's tile; returns false for surplus workgroups.
template <int BM, int BN>
__device__ bool find_tile(const GemmArgs &a, TileInfo *ti)
{
    const int ntn = (a.N + BN - 1) / BN;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int total = 0;
        for (int s0 = 0; s0 < a.P; s0 += 64) {
            const int s = s0 + lane;
            const int cnt = s < a.P ? a.slot_offset[s + 1] - a.slot_offset[s] : 0;
            const int w = (cnt + BM - 1) / BM * ntn;
            total += __shfl(wave_incl_scan(w, lane), 63, 64);
        }
        const int bid = blockIdx.x;
        if (lane == 0) ti->slot = -1;
        if (bid < total) {
            const int L = xcd_remap(bid, total);
            int run = 0;
            for (int s0 = 0; s0 < a.P; s0 += 64) {
                const int s = s0 + lane;
                const int cnt = s < a.P ? a.slot_offset[s + 1] - a.slot_offset[s] : 0;
                const int mt = (cnt + BM - 1) / BM;
                const int w = mt * ntn;
                const int inc = wave_incl_scan(w, lane);
                const int ex = run + inc - w;
                if (s < a.P && w > 0 && L >= ex && L < ex + w) {
                    const int local = L - ex;
                    const int nt = local / mt, ml = local % mt;
                    ti->slot = s;
                    ti->row0 = a.slot_offset[s] + ml * BM;
                    ti->rows = min(BM, cnt - ml * BM);
                    ti->n0 = nt * BN;
                }
                run += __shfl(inc, 63, 64);
            }
        }
    }
    __syncthreads();
    return ti->slot >= 0;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

template <typename TE>
__device__ __forceinline__ float ld_f32(const TE *p);
template <>
__device__ __forceinline__ float ld_f32<float>(const float *p) { return *p; }
template <>
__device__ __forceinline__ float ld_f32<uint16_t>(const uint16_t *p) { return bf16_to_f32(*p); }

template <typename TE>
__device__ __forceinline__ void st_from_f32(TE *p, float v);
template <>
__device__ __forceinline__ void st_from_f32<float>(float *p, float v) { *p = v; }
template <>
__device__ __forceinline__ void st_from_f32<uint16_t>(uint16_t *p, float v) { *p = f32_to_bf16(v); }

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// ---------------------------------------------------------------------------
// bf16 MFMA kernel. WM x WN waves; each wave computes a (BM/WM) x (BN/WN)
// block as 32x32 MFMA tiles (v_mfma_f32_32x32x16_bf16), K step 64,
// double-buffered LDS with a 16-byte pad per row (conflict-free 16-byte
// fragment reads: 8 lanes reading 8 rows touch all 32 banks once).
// MFMA operand layout (32x32x16): lane l supplies row (l % 32) and the 8
// consecutive k values 8*(l / 32) .. +7 of A (and of B^T); result register r
// of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
template <int BM, int BN, int WM, int WN, bool GATEUP>
__global__ __launch_bounds__(WM *WN * 64) void k_gemm_mfma(GemmArgs a)
{
    constexpr int NT = WM * WN * 64;
    constexpr int BK = 64, LDK = BK + 8;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 32, NI = TN / 32;
    constexpr int CA = BM * BK / 8 / NT, CB = BN * BK / 8 / NT;
    static_assert(CA >= 1 && CB >= 1 && MI >= 1 && NI >= 1, "tile shape");
    static_assert(!GATEUP || (TN % 64) == 0, "gate/up pairs need 64-column wave tiles");

    __shared__ TileInfo ti;
    __shared__ __attribute__((aligned(16))) uint16_t lds[2][(BM + BN) * LDK];
    __shared__ int32_t s_route[GATEUP ? 1 : BM];
    __shared__ float s_alpha[GATEUP ? 1 : BM];

    if (!find_tile<BM, BN>(a, &ti)) return;
    const int slot = ti.slot, row0 = ti.row0, rows = ti.rows, n0 = ti.n0;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    const int K = a.K, N = a.N;

    const uint16_t *aptr[CA];
    const uint16_t *bptr[CB];
    int alds[CA], blds[CB];
#pragma unroll
    for (int c = 0; c < CA; ++c) {
        const int id = c * NT + tid, r = id >> 3, kc = (id & 7) * 8;
        const int rr = min(r, rows - 1);
        if (GATEUP)
            aptr[c] = (const uint16_t *)a.A + (int64_t)a.rec_token[row0 + rr] * a.lda + kc;
        else
            aptr[c] = (const uint16_t *)a.A + (int64_t)(row0 + rr) * a.lda + kc;
        alds[c] = r * LDK + kc;
    }
    const uint16_t *Bslot = (const uint16_t *)a.B + (int64_t)slot * a.slot_stride;
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int id = c * NT + tid, r = id >> 3, kc = (id & 7) * 8;
        const int n = min(n0 + r, N - 1);
        bptr[c] = Bslot + (int64_t)n * K + kc;
        blds[c] = (BM + r) * LDK + kc;
    }
    if (!GATEUP) {
        for (int m = tid; m < BM; m += NT) {
            const int rt = a.rec_route[row0 + min(m, rows - 1)];
            s_route[m] = rt;
            s_alpha[m] = a.topk_w[rt];
        }
    }

    u32x4_t ra[CA], rb[CB];
    f32x16_t acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = K / BK;
#pragma unroll
    for (int c = 0; c < CA; ++c) ra[c] = *(const u32x4_t *)(aptr[c]);
#pragma unroll
    for (int c = 0; c < CB; ++c) rb[c] = *(const u32x4_t *)(bptr[c]);
#pragma unroll
    for (int c = 0; c < CA; ++c) *(u32x4_t *)(&lds[0][alds[c]]) = ra[c];
#pragma unroll
    for (int c = 0; c < CB; ++c) *(u32x4_t *)(&lds[0][blds[c]]) = rb[c];
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int k0 = (kt + 1) * BK;
#pragma unroll
            for (int c = 0; c < CA; ++c) ra[c] = *(const u32x4_t *)(aptr[c] + k0);
#pragma unroll
            for (int c = 0; c < CB; ++c) rb[c] = *(const u32x4_t *)(bptr[c] + k0);
        }
        const uint16_t *As = &lds[cur][0];
        const uint16_t *Bs = &lds[cur][BM * LDK];
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            bf16x8_t af[MI], bfr[NI];
            const int koff = ks * 16 + (lane >> 5) * 8;
#pragma unroll
            for (int i = 0; i < MI; ++i)
                af[i] = *(const bf16x8_t *)(As + (wm * TM + i * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
            for (int j = 0; j < NI; ++j)
                bfr[j] = *(const bf16x8_t *)(Bs + (wn * TN + j * 32 + (lane & 31)) * LDK + koff);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                if (wm * TM + i * 32 < rows) {
#pragma unroll
                    for (int j = 0; j < NI; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j],
                                                                            0, 0, 0);
                }
            }
        }
        if (kt + 1 < nk) {
#pragma unroll
            for (int c = 0; c < CA; ++c) *(u32x4_t *)(&lds[cur ^ 1][alds[c]]) = ra[c];
#pragma unroll
            for (int c = 0; c < CB; ++c) *(u32x4_t *)(&lds[cur ^ 1][blds[c]]) = rb[c];
        }
        __syncthreads();
    }

    if (GATEUP) {
        uint16_t *H = (uint16_t *)a.C;
        const int fN = N / 2;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int q = 0; q < NI / 2; ++q) {
                const int fcol = ((n0 + wn * TN) / 64 + q) * 32 + (lane & 31);
                if (fcol >= fN) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m < rows)
                        H[(int64_t)(row0 + m) * a.ldc + fcol] =
                            f32_to_bf16(silu_mul(acc[i][2 * q][r], acc[i][2 * q + 1][r]));
                }
            }
        }
    } else {
        float *Yr = (float *)a.C;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                const int n = n0 + wn * TN + j * 32 + (lane & 31);
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = wm * TM + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (m < rows) Yr[(int64_t)s_route[m] * a.ldc + n] = s_alpha[m] * acc[i][j][r];
                }
            }
        }
        if (n0 == 0)
            for (int m = tid; m < rows; m += NT) a.done[s_route[m]] = 1;
    }
}

// ---------------------------------------------------------------------------
// Plain LDS-tiled kernel (fp32 FMA on the vector ALUs) for fp32 layers; also
// runs bf16 inputs as an independent second path. 64x64 tiles, K step 16,
// 256 threads with 4x4 outputs each. For gate/up a thread owns columns
// {2tx, 2tx+1} (gate) and {32+2tx, 32+2tx+1} (up) of its 64-column block, so
// both halves of each SwiGLU pair are in one thread.
template <typename TE, bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_simple(GemmArgs a)
{
    constexpr int BM = 64, BN = 64, BK = 16;
    __shared__ TileInfo ti;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    __shared__ int32_t s_route[BM];
    __shared__ float s_alpha[BM];
    if (!find_tile<BM, BN>(a, &ti)) return;
    const int slot = ti.slot, row0 = ti.row0, rows = ti.rows, n0 = ti.n0;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int K = a.K, N = a.N;

    int col[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) col[j] = GATEUP ? ((j < 2) ? 2 * tx + j : 32 + 2 * tx + (j - 2)) : tx * 4 + j;

    const int lr = tid >> 2, lk = (tid & 3) * 4;
    const int rr = min(lr, rows - 1);
    const TE *ap = GATEUP ? (const TE *)a.A + (int64_t)a.rec_token[row0 + rr] * a.lda
                          : (const TE *)a.A + (int64_t)(row0 + rr) * a.lda;
    const TE *bp = (const TE *)a.B + (int64_t)slot * a.slot_stride + (int64_t)min(n0 + lr, N - 1) * K;
    if (!GATEUP && tid < BM) {
        const int rt = a.rec_route[row0 + min(tid, rows - 1)];
        s_route[tid] = rt;
        s_alpha[tid] = a.topk_w[rt];
    }

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int kk = k0 + lk + q;
            As[lk + q][lr] = kk < K ? ld_f32<TE>(ap + kk) : 0.0f;
            Bs[lk + q][lr] = kk < K ? ld_f32<TE>(bp + kk) : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][col[j]];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = ty * 4 + i;
        if (m >= rows) continue;
        if (GATEUP) {
            TE *H = (TE *)a.C;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int fcol = n0 / 2 + 2 * tx + j;
                if (n0 + 2 * tx + j < N)
                    st_from_f32<TE>(H + (int64_t)(row0 + m) * a.ldc + fcol, silu_mul(acc[i][j], acc[i][j + 2]));
            }
        } else {
            float *Yr = (float *)a.C;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + col[j];
                if (n < N) Yr[(int64_t)s_route[m] * a.ldc + n] = s_alpha[m] * acc[i][j];
            }
        }
    }
    if (!GATEUP && n0 == 0 && tid < rows) a.done[s_route[tid]] = 1;
}

// Upper bound of tiles: sum over slots of ceil(c_s / BM) <= ceil(R / BM) + P.
inline unsigned grid_bound(const GemmArgs &a, int max_rows, int BM, int BN)
{
    const int64_t mt = (max_rows + BM - 1) / BM + a.P;
    const int64_t ntn = (a.N + BN - 1) / BN;
    return (unsigned)(mt * ntn);
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
hipError_t launch_mfma(const GemmArgs &a, int max_rows, hipStream_t st)
{
    const unsigned g = grid_bound(a, max_rows, BM, BN);
    if (g == 0) return hipSuccess;
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WM, WN, GATEUP>), dim3(g), dim3(WM * WN * 64), 0, st, a);
    return hipGetLastError();
}

template <typename TE, bool GATEUP>
hipError_t launch_simple(const GemmArgs &a, int max_rows, hipStream_t st)
{
    const unsigned g = grid_bound(a, max_rows, 64, 64);
    if (g == 0) return hipSuccess;
    hipLaunchKernelGGL((k_gemm_simple<TE, GATEUP>), dim3(g), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up(const moe_shape &s, const GemmArgs &a, int max_rows, bool simple,
                          hipStream_t st)
{
    if (max_rows == 0) return hipSuccess;
    if (s.dtype == MOE_DT_F32) return launch_simple<float, true>(a, max_rows, st);
    if (simple) return launch_simple<uint16_t, true>(a, max_rows, st);
    return launch_mfma<128, 128, 2, 2, true>(a, max_rows, st);
}

hipError_t launch_down(const moe_shape &s, const GemmArgs &a, int max_rows, bool simple,
                       hipStream_t st)
{
    if (max_rows == 0) return hipSuccess;
    if (s.dtype == MOE_DT_F32) return launch_simple<float, false>(a, max_rows, st);
    if (simple) return launch_simple<uint16_t, false>(a, max_rows, st);
    return launch_mfma<128, 128, 2, 2, false>(a, max_rows, st);
}

}  // namespace moe
