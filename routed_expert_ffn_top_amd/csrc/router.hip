// Router logits and top-k routing (EStream, section 2.2: a router assigns
// each token to the top-k of E experts; the per-route weight alpha scales the
// expert output in Eq. 2).
//
// Router: L[t][e] = fp32 fused multiply-add chain over the hidden index in
// ascending order, then + bias[e]. The chain is not split or reassociated:
// the top-k decision is taken on these bits, so they must be reproducible.
// A lane owns one token and a few experts; W_r comes through scalar loads.
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

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// For each expert j < NE: acc[j] += bcast(w[j], q) * x[q] for q = 0..15 in
// ascending order, where bcast(w, q) is the value that lane q of each 16-lane
// row holds (DPP row_newbcast:q): the 16 lanes of a row hold 16 consecutive
// weights of one expert. The NE chains are interleaved (q outer, j inner) so
// that consecutive multiply-adds are independent. One s_nop 1 covers the two
// wait states a DPP source needs after a vector ALU write.
template <int NE>
__device__ __forceinline__ void fmac16_bcast(float *acc, const float *w, const float *x);

template <>
__device__ __forceinline__ void fmac16_bcast<1>(float *acc, const float *w, const float *x)
{
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %1, %2 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %3 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %4 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %5 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %6 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %7 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %8 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %9 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %10 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %11 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %12 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %13 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %14 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %15 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %16 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %1, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0])
        : "v"(w[0]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]));
}

template <>
__device__ __forceinline__ void fmac16_bcast<2>(float *acc, const float *w, const float *x)
{
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %2, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %4 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %5 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %6 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %7 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %8 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %9 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %10 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %11 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %12 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %13 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %14 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %15 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %16 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %18 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %2, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %3, %19 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1])
        : "v"(w[0]), "v"(w[1]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]));
}

template <>
__device__ __forceinline__ void fmac16_bcast<4>(float *acc, const float *w, const float *x)
{
    asm volatile(
        "s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %4, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %8 row_newbcast:0 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %9 row_newbcast:1 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %10 row_newbcast:2 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %11 row_newbcast:3 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %12 row_newbcast:4 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %13 row_newbcast:5 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %14 row_newbcast:6 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %15 row_newbcast:7 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %16 row_newbcast:8 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %18 row_newbcast:10 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %19 row_newbcast:11 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %20 row_newbcast:12 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %21 row_newbcast:13 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %22 row_newbcast:14 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %0, %4, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %5, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %6, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %7, %23 row_newbcast:15 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
        : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(x[4]), "v"(x[5]), "v"(x[6]), "v"(x[7]), "v"(x[8]), "v"(x[9]), "v"(x[10]), "v"(x[11]), "v"(x[12]), "v"(x[13]), "v"(x[14]), "v"(x[15]));
}

// Router logits. A wave owns 64 tokens (one per lane) and NE consecutive
// experts; the 4 waves of a workgroup take 4 expert blocks of the same 64
// tokens (grid: T/64 x ceil(E / (4 NE))). W_r is [E][d]. The hidden index is
// walked in 16-wide blocks: lane l loads weight (l % 16) of the block for each
// of its experts (one coalesced 64-byte read per expert) and its own token's
// 16 x values; a lane converts each x value once and uses it for NE chains,
// with the weight broadcast across the row inside the multiply-add (see
// fmac16_bcast). Loads run PF blocks ahead of the arithmetic.
template <typename TX, int NE>
__global__ __launch_bounds__(256) void k_router_logits(const TX *__restrict__ X, int64_t ldx,
                                                       const float *__restrict__ Wr,
                                                       const float *__restrict__ bias,
                                                       float *__restrict__ L, int T, int d, int E)
{
    constexpr int PF = sizeof(TX) == 2 ? 8 : 4;
    constexpr int XV = sizeof(TX) == 2 ? 2 : 4;   // 16-byte loads per 16 x values
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int eb = (blockIdx.y * 4 + wave) * NE;   // first expert of this wave
    if (eb >= E) return;                           // no barriers below
    const int t = blockIdx.x * 64 + lane;
    const TX *xrow = X + (int64_t)min(t, T - 1) * ldx;
    const float *wsrc[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) wsrc[j] = Wr + (int64_t)min(eb + j, E - 1) * d + (lane & 15);

    float acc[NE];
#pragma unroll
    for (int j = 0; j < NE; ++j) acc[j] = 0.0f;

    const int nb = d >> 4;   // whole 16-wide blocks
    auto load = [&](int b, u32x4_t *xv, float *wv) {
        const int i0 = min(b, nb - 1) * 16;   // past the end: re-read the last block
#pragma unroll
        for (int h = 0; h < XV; ++h) xv[h] = *(const u32x4_t *)((const char *)(xrow + i0) + 16 * h);
#pragma unroll
        for (int j = 0; j < NE; ++j) wv[j] = wsrc[j][i0];
    };
    auto compute = [&](const u32x4_t *xv, const float *wv) {
        float x[16];
        if (sizeof(TX) == 2) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const uint32_t v = xv[q / 4][q % 4];
                x[2 * q] = __uint_as_float(v << 16);
                x[2 * q + 1] = __uint_as_float(v & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) x[q] = __uint_as_float(xv[q / 4][q % 4]);
        }
        fmac16_bcast<NE>(acc, wv, x);
    };
    if (nb > 0) {
        u32x4_t xr[PF][XV];
        float wr[PF][NE];
#pragma unroll
        for (int u = 0; u < PF; ++u) load(u, xr[u], wr[u]);
        int b0 = 0;
        for (; b0 + PF <= nb; b0 += PF) {
#pragma unroll
            for (int u = 0; u < PF; ++u) {
                u32x4_t xc[XV];
                float wc[NE];
#pragma unroll
                for (int h = 0; h < XV; ++h) xc[h] = xr[u][h];
#pragma unroll
                for (int j = 0; j < NE; ++j) wc[j] = wr[u][j];
                load(b0 + u + PF, xr[u], wr[u]);
                compute(xc, wc);
            }
        }
        // the last nb - b0 < PF blocks are in the ring, block b0 + u in slot u
#pragma unroll
        for (int u = 0; u < PF - 1; ++u)
            if (b0 + u < nb) compute(xr[u], wr[u]);
    }
    // hidden indices past the last whole block, in order
    for (int i = nb * 16; i < d; ++i) {
        const float xv = load_x<TX>(xrow + i);
#pragma unroll
        for (int j = 0; j < NE; ++j)
            acc[j] = __builtin_fmaf(xv, Wr[(int64_t)min(eb + j, E - 1) * d + i], acc[j]);
    }
    if (t < T) {
#pragma unroll
        for (int j = 0; j < NE; ++j)
            if (eb + j < E) L[(int64_t)t * E + eb + j] = bias ? acc[j] + bias[eb + j] : acc[j];
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

template <typename TX, int NE>
hipError_t launch_router_t(const moe_shape &s, const void *X, const float *Wr, const float *bias, float *L,
                           hipStream_t st)
{
    const dim3 grid((s.T + 63) / 64, (s.E + 4 * NE - 1) / (4 * NE));
    hipLaunchKernelGGL((k_router_logits<TX, NE>), grid, dim3(256), 0, st, (const TX *)X, s.ldx, Wr, bias, L,
                       s.T, s.d, s.E);
    return hipGetLastError();
}

hipError_t launch_router_logits(const moe_shape &s, const void *X, const float *Wr,
                                const float *bias, float *L, hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    // experts per wave: 4 while that still gives every SIMD a wave, else fewer
    const int64_t tg = (s.T + 63) / 64;
    int ne = tg * ((s.E + 15) / 16) >= 256 ? 4 : (tg * ((s.E + 7) / 8) >= 256 ? 2 : 1);
#ifdef MOE_ROUTER_NE
    ne = MOE_ROUTER_NE;
#endif
    if (act_bf16(s)) {
        if (ne == 4) return launch_router_t<uint16_t, 4>(s, X, Wr, bias, L, st);
        if (ne == 2) return launch_router_t<uint16_t, 2>(s, X, Wr, bias, L, st);
        return launch_router_t<uint16_t, 1>(s, X, Wr, bias, L, st);
    }
    if (ne == 4) return launch_router_t<float, 4>(s, X, Wr, bias, L, st);
    if (ne == 2) return launch_router_t<float, 2>(s, X, Wr, bias, L, st);
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
