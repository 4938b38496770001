// Weighted combine into the token accumulator (EStream Eq. 2:
// Y_t = A_t + sum over the token's routes of alpha F_e(X_t)), gate/up
// packing (section 3.3, offline layout for the consuming kernel), and an
// MFMA lane-layout self-test.
//
// Combine: Y holds A_t on entry. Each thread owns 4 consecutive columns of
// one token row and adds the token's computed route rows Yr[t*K' + j] in
// ascending j (each route's S partial rows, when the down projection splits
// its K, in ascending split order), so the fp32 sum order is fixed: no
// atomics, bitwise reproducible, and independent of how routes were spread
// over slots, workgroups or invocations.
#include "common.h"

namespace moe {
namespace {

// Route rows are read once: non-temporal loads (measured 11 % faster on the
// OLMoE-shaped layer than ordinary ones). KP > 0: the token has exactly KP
// routes and the down projection does not split its K; every route row is
// requested before the first add (rows of routes not computed are in
// bounds, read and left out), so a thread has KP loads in flight and none
// waits on a flag. KP == 0: any kp and split count.
__device__ __forceinline__ float4 load_nt4(const float *p)
{
    return make_float4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1),
                       __builtin_nontemporal_load(p + 2), __builtin_nontemporal_load(p + 3));
}

template <int KP>
__global__ __launch_bounds__(256) void k_combine(float *__restrict__ Y, int64_t ldy,
                                                 const float *__restrict__ Yr,
                                                 const int32_t *__restrict__ done, int d, int kp,
                                                 int splits, int64_t split_stride, int cblocks)
{
    // one-dimensional grid: block b covers token b / cblocks, columns
    // (b % cblocks) * 1024 .. +1023 (the x dimension holds any T this
    // library accepts; the y dimension would cap it at 65535)
    const int t = (int)(blockIdx.x / (unsigned)cblocks);
    const int c = ((int)(blockIdx.x % (unsigned)cblocks) * 256 + threadIdx.x) * 4;
    if (c >= d) return;
    float4 y = *(const float4 *)(Y + (int64_t)t * ldy + c);
    if constexpr (KP > 0) {
        bool ok[KP];
        float4 v[KP];
#pragma unroll
        for (int j = 0; j < KP; ++j) ok[j] = done[(int64_t)t * KP + j] != 0;
#pragma unroll
        for (int j = 0; j < KP; ++j) v[j] = load_nt4(Yr + ((int64_t)t * KP + j) * d + c);
#pragma unroll
        for (int j = 0; j < KP; ++j) {   // ascending j; a route left out adds nothing
            if (ok[j]) {
                y.x += v[j].x;
                y.y += v[j].y;
                y.z += v[j].z;
                y.w += v[j].w;
            }
        }
    } else {
        for (int j = 0; j < kp; ++j) {
            const int64_t i = (int64_t)t * kp + j;
            if (done[i]) {
                for (int q = 0; q < splits; ++q) {   // route j's partial rows, in order
                    const float4 v = load_nt4(Yr + q * split_stride + i * d + c);
                    y.x += v.x;
                    y.y += v.y;
                    y.z += v.z;
                    y.w += v.w;
                }
            }
        }
    }
    *(float4 *)(Y + (int64_t)t * ldy + c) = y;
}

// Packed gate/up row r of expert e: q = r / 64, w = r % 64; gate row 32q + w
// for w < 32, up row 32q + w - 32 otherwise, written in the tiled layout
// (wtile_off over the [2f][d] slice). One workgroup copies one row as 32-bit
// words (epw elements each; a word never straddles a K piece). With row
// scales (fp8 weights: src_scale_w > 0), the row's fp32 scale moves with it:
// from word src_scale_w + source row of the source slice to word
// dst_scale_w + r of the packed slice (scales stay in row order).
__global__ __launch_bounds__(256) void k_pack_gate_up(const uint32_t *__restrict__ Wg,
                                                      const uint32_t *__restrict__ Wu,
                                                      uint32_t *__restrict__ dst, int64_t row_words,
                                                      int64_t src_stride_w, int64_t dst_stride_w,
                                                      int64_t src_scale_w, int64_t dst_scale_w, int N, int K,
                                                      int epw)
{
    const int r = blockIdx.x;
    const int e = blockIdx.y;
    const int q = r >> 6, w = r & 63;
    const int sr = w < 32 ? 32 * q + w : 32 * q + w - 32;
    const uint32_t *slice = (w < 32 ? Wg : Wu) + (int64_t)e * src_stride_w;
    const uint32_t *src = slice + (int64_t)sr * row_words;
    uint32_t *out = dst + (int64_t)e * dst_stride_w;
    for (int64_t c = threadIdx.x; c < row_words; c += 256) out[wtile_off(r, c * epw, N, K) / epw] = src[c];
    if (src_scale_w > 0 && threadIdx.x == 0)
        dst[(int64_t)e * dst_stride_w + dst_scale_w + r] = slice[src_scale_w + sr];
}

// Down row m of expert e ([d][f] slice, row m = output column m) into the
// tiled layout; fp8 row scales (src_scale_w > 0) are copied in row order.
__global__ __launch_bounds__(256) void k_pack_down(const uint32_t *__restrict__ Wd, uint32_t *__restrict__ dst,
                                                   int64_t row_words, int64_t src_stride_w, int64_t dst_stride_w,
                                                   int64_t scale_w, int N, int K, int epw)
{
    const int m = blockIdx.x;
    const int e = blockIdx.y;
    const uint32_t *slice = Wd + (int64_t)e * src_stride_w;
    const uint32_t *src = slice + (int64_t)m * row_words;
    uint32_t *out = dst + (int64_t)e * dst_stride_w;
    for (int64_t c = threadIdx.x; c < row_words; c += 256) out[wtile_off(m, c * epw, N, K) / epw] = src[c];
    if (scale_w > 0 && threadIdx.x == 0) out[scale_w + m] = slice[scale_w + m];
}

// MXFP4 packing: source row sr of expert e's source slice (codes
// [Nsrc][K/2], then scales [Nsrc][K/32]) to row r of the packed [N][K] slice:
// in each K piece of its 256-row block, its 16 code bytes at row r % 256 and
// its scale byte after the block's codes; the last row of a block zeroes the
// piece's padding. gateup: r is a packed gate/up row (interleaved from Wg
// and Wu), else a down row of Wg. Sources and destinations 4-byte aligned.
__global__ __launch_bounds__(64) void k_pack_fp4(const uint8_t *__restrict__ Wg, const uint8_t *__restrict__ Wu,
                                                 uint8_t *__restrict__ dst, int64_t src_stride, int64_t dst_stride,
                                                 int Nsrc, int N, int K, int gateup)
{
    const int r = blockIdx.x, e = blockIdx.y;
    int sr = r;
    const uint8_t *slice = Wg + (int64_t)e * src_stride;
    if (gateup) {
        const int q = r >> 6, w = r & 63;
        sr = w < 32 ? 32 * q + w : 32 * q + w - 32;
        slice = (w < 32 ? Wg : Wu) + (int64_t)e * src_stride;
    }
    const int b = r / kWRows, rb = r % kWRows, rows = min(kWRows, N - b * kWRows);
    uint8_t *base = dst + (int64_t)e * dst_stride + (int64_t)b * (K / kWK) * fp4_piece_bytes(kWRows);
    const uint8_t *codes = slice + (int64_t)sr * (K / 2);
    const uint8_t *sc = slice + (int64_t)Nsrc * (K / 2) + (int64_t)sr * (K / kWK);
    for (int p = threadIdx.x; p < K / kWK; p += 64) {
        uint8_t *piece = base + (int64_t)p * fp4_piece_bytes(rows);
        const uint32_t *cs = (const uint32_t *)(codes + p * 16);
        uint32_t *cd = (uint32_t *)(piece + rb * 16);
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) cd[w4] = cs[w4];
        piece[rows * 16 + rb] = sc[p];
        if (rb == rows - 1)
            for (int64_t z = (int64_t)rows * 17; z < fp4_piece_bytes(rows); ++z) piece[z] = 0;
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// One wave. A[i][k] and B[k][j] (32x16 and 16x32) with small integer values
// are placed in the operand registers under the assumed layout (lane l: row
// or column l % 32, k = 8*(l/32) .. +7); the result registers are written to
// out[32][32] under the assumed output layout (register r of lane l -> row
// 8*(r/4) + 4*(l/32) + r%4, column l % 32). The host checks out == A*B, which
// holds only if the assumed layouts are the hardware's.
__global__ void k_selftest_mfma(float *out)
{
    const int l = threadIdx.x;
    bf16x8_t av, bv;
    for (int q = 0; q < 8; ++q) {
        const int k = 8 * (l >> 5) + q;
        const int i = l & 31;
        const float aval = (float)((i * 3 + k * 5) % 7 - 3);        // A[i][k]
        const float bval = (float)((k * 2 + (l & 31) * 7) % 5 - 2);  // B[k][j], j = l % 32
        av[q] = (__bf16)aval;
        bv[q] = (__bf16)bval;
    }
    f32x16_t acc;
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        out[row * 32 + (l & 31)] = acc[r];
    }
}

}  // namespace

hipError_t launch_combine(const moe_shape &s, float *Y, const float *Yr, const int32_t *done,
                          hipStream_t st)
{
    if (s.T == 0) return hipSuccess;
    const int cblocks = (s.d / 4 + 255) / 256;
    const dim3 grid((unsigned)((int64_t)s.T * cblocks));
    const int kp = s.k + s.n_shared, splits = down_splits(s);
    const int64_t sstride = (int64_t)s.T * kp * s.d;
    auto go = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, Y, s.ldy, Yr, done, s.d, kp, splits, sstride, cblocks);
    };
    if (splits == 1 && kp == 8)
        go(k_combine<8>);
    else if (splits == 1 && kp == 2)
        go(k_combine<2>);
    else if (splits == 1 && kp == 6)
        go(k_combine<6>);
    else
        go(k_combine<0>);
    return hipGetLastError();
}

hipError_t launch_pack_gate_up(const moe_shape &s, const void *Wg, const void *Wu, void *dst,
                               int n, int64_t src_stride, int64_t dst_stride, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    if (w_fp4(s)) {
        hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)(2 * s.f), (unsigned)n), dim3(64), 0, st, (const uint8_t *)Wg,
                           (const uint8_t *)Wu, (uint8_t *)dst, src_stride, dst_stride, s.f, 2 * s.f, s.d, 1);
        return hipGetLastError();
    }
    const int esz = w_esz(s);
    const int64_t row_words = (int64_t)s.d * esz / 4;
    const int64_t ssw = src_stride * esz / 4, dsw = dst_stride * esz / 4;
    // fp8: the row scales follow the codes ([f] after [f][d], [2f] after [2f][d])
    const int64_t sscale = w_fp8(s) ? (int64_t)s.f * row_words : 0;
    const int64_t dscale = w_fp8(s) ? (int64_t)2 * s.f * row_words : 0;
    hipLaunchKernelGGL(k_pack_gate_up, dim3((unsigned)(2 * s.f), (unsigned)n), dim3(256), 0, st,
                       (const uint32_t *)Wg, (const uint32_t *)Wu, (uint32_t *)dst, row_words, ssw,
                       dsw, sscale, dscale, 2 * s.f, s.d, 4 / esz);
    return hipGetLastError();
}

hipError_t launch_pack_down(const moe_shape &s, const void *Wd, void *dst, int n, int64_t src_stride,
                            int64_t dst_stride, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    if (w_fp4(s)) {
        hipLaunchKernelGGL(k_pack_fp4, dim3((unsigned)s.d, (unsigned)n), dim3(64), 0, st, (const uint8_t *)Wd,
                           (const uint8_t *)nullptr, (uint8_t *)dst, src_stride, dst_stride, s.d, s.d, s.f, 0);
        return hipGetLastError();
    }
    const int esz = w_esz(s);
    const int64_t row_words = (int64_t)s.f * esz / 4;
    const int64_t ssw = src_stride * esz / 4, dsw = dst_stride * esz / 4;
    const int64_t scale = w_fp8(s) ? (int64_t)s.d * row_words : 0;   // [d] scales after the [d][f] codes
    hipLaunchKernelGGL(k_pack_down, dim3((unsigned)s.d, (unsigned)n), dim3(256), 0, st, (const uint32_t *)Wd,
                       (uint32_t *)dst, row_words, ssw, dsw, scale, s.d, s.f, 4 / esz);
    return hipGetLastError();
}

hipError_t launch_selftest_mfma(float *out, hipStream_t st)
{
    hipLaunchKernelGGL(k_selftest_mfma, dim3(1), dim3(64), 0, st, out);
    return hipGetLastError();
}

}  // namespace moe
