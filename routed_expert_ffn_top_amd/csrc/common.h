// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kRouteBlock = 256;      // routes per counting block
constexpr int kMaxExp = MOE_MAX_EXPERTS;

// Placement map passed by value in the kernel arguments (2 KB).
struct PhiArg {
    int32_t v[kMaxExp];
};

// Byte offsets of the workspace regions for one shape.
struct WsLayout {
    size_t err;      // int32[64]: [0] device error word
    size_t ecount;   // int32[kMaxExp]: routes per logical expert (paging)
    size_t blk;      // int32[nblk][P]: per-block slot counts, then bases
    size_t rank;     // int32[C]: in-block stable rank of each route of a build
    size_t done;     // int32[T*K']: 1 once route i's Yr row is computed
    size_t logits;   // float[T][E]
    size_t H;        // dtype[C][f]
    size_t Yr;       // float[S][T*K'][d], S = down_splits (partial sums over f)
    size_t total;
    int nblk;        // ceil(C / kRouteBlock)
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Element formats. MOE_DT_BF16_FP8W: bf16 activations, fp8 e4m3 expert
// weights with one fp32 scale per weight row (a slot slice holds the codes,
// then the scales). MOE_DT_BF16_FP4W: bf16 activations, MXFP4 expert
// weights (E2M1 codes, one E8M0 scale per 32 weights of a row). With
// quantised weights, slice sizes and strides are in bytes (w_esz == 1).
inline bool act_bf16(const moe_shape &s)
{
    return s.dtype == MOE_DT_BF16 || s.dtype == MOE_DT_BF16_FP8W || s.dtype == MOE_DT_BF16_FP4W;
}
inline bool w_fp8(const moe_shape &s) { return s.dtype == MOE_DT_BF16_FP8W; }
inline bool w_fp4(const moe_shape &s) { return s.dtype == MOE_DT_BF16_FP4W; }
inline int w_esz(const moe_shape &s) { return s.dtype == MOE_DT_F32 ? 4 : (s.dtype == MOE_DT_BF16 ? 2 : 1); }

// Tiled layout of an expert weight slice [N][K] in the arena (section 3.3:
// weights are stored offline in the order the kernels consume them). Rows
// form blocks of kWRows; within a block, K is cut into pieces of kWK
// elements (the last piece narrower when K % kWK != 0) stored piece-major,
// each piece holding the block's rows one after another, so that one K step
// of a 256-row weight tile is one contiguous run (16 KB for bf16). Element
// (n, k) sits at element offset
//   kWRows*nb*K + (k / kWK)*rows_nb*kWK + (n % kWRows)*w + k % kWK,
// nb = n / kWRows, rows_nb = min(kWRows, N - kWRows*nb), w = min(kWK, K -
// kWK*(k / kWK)) the width of k's piece. The slice keeps its size.
constexpr int kWRows = 256, kWK = 32;
__host__ __device__ inline int64_t wtile_off(int64_t n, int64_t k, int64_t N, int64_t K)
{
    const int64_t nb = n / kWRows, kp = k / kWK;
    const int64_t rows = N - nb * kWRows < kWRows ? N - nb * kWRows : kWRows;
    const int64_t w = K - kp * kWK < kWK ? K - kp * kWK : kWK;
    return nb * kWRows * K + kp * rows * kWK + (n % kWRows) * w + k % kWK;
}

// Packed MXFP4 slice [N][K]: for each 256-row block and each 32-wide K piece,
// the block's rows' 16 code bytes one row after another, then the rows'
// scale bytes padded with zeros to a multiple of 16. One K step of a weight
// tile is again one contiguous run (rows*16 + align16(rows) bytes).
__host__ __device__ inline int64_t fp4_piece_bytes(int64_t rows) { return rows * 16 + (rows + 15) / 16 * 16; }
inline int64_t fp4_slice_bytes(int64_t N, int64_t K)
{
    const int64_t full = N / kWRows, rem = N % kWRows;
    return (K / kWK) * (full * fp4_piece_bytes(kWRows) + (rem ? fp4_piece_bytes(rem) : 0));
}
// bytes of one expert's packed gate/up slice and down slice (codes + scales
// for the quantised formats)
inline size_t gu_slice_bytes(const moe_shape &s)
{
    if (w_fp4(s)) return (size_t)fp4_slice_bytes(2 * (int64_t)s.f, s.d);
    return (size_t)2 * s.f * s.d * w_esz(s) + (w_fp8(s) ? (size_t)2 * s.f * 4 : 0);
}
inline size_t d_slice_bytes(const moe_shape &s)
{
    if (w_fp4(s)) return (size_t)fp4_slice_bytes(s.d, s.f);
    return (size_t)s.d * s.f * w_esz(s) + (w_fp8(s) ? (size_t)s.d * 4 : 0);
}
// bytes of one unpacked source slice [N][K] handed to the packing calls
inline size_t src_slice_bytes(const moe_shape &s, int64_t N, int64_t K)
{
    if (w_fp4(s)) return (size_t)(N * K / 2 + N * K / 32);
    return (size_t)(N * K * w_esz(s)) + (w_fp8(s) ? (size_t)N * 4 : 0);
}

// Splits of the down projection's K = f: when the down tiles (about
// experts x row blocks x d/256) would not fill the GPU, each tile's K range
// is cut in S pieces whose partial products go to S separate per-route rows,
// summed in fixed order by the combine. S doubles while the tile count stays
// <= 512 and f splits into multiples of 64; at most 4.
inline int down_splits(const moe_shape &s)
{
    if (!act_bf16(s)) return 1;
    const int64_t ne = s.E + s.n_shared;
    const int64_t per = ((int64_t)s.T * (s.k + s.n_shared) + ne - 1) / ne;
    const int64_t tiles = ne * ((per + 255) / 256) * ((s.d + 255) / 256);
    int S = 1;
    while (S < 4 && tiles * S * 2 <= 512 && (s.f % (64 * S * 2)) == 0) S *= 2;
    return S;
}

inline WsLayout ws_layout(const moe_shape &s)
{
    WsLayout w{};
    const size_t kp = (size_t)(s.k + s.n_shared);
    const size_t esz = act_bf16(s) ? 2 : 4;   // H holds activations
    w.nblk = (s.capacity + kRouteBlock - 1) / kRouteBlock;
    size_t o = 0;
    w.err = o;    o = align_up(o + 64 * 4, 256);
    w.ecount = o; o = align_up(o + kMaxExp * 4, 256);
    w.blk = o;    o = align_up(o + (size_t)w.nblk * s.P * 4, 256);
    w.rank = o;   o = align_up(o + (size_t)s.capacity * 4, 256);
    w.done = o;   o = align_up(o + (size_t)s.T * kp * 4, 256);
    w.logits = o; o = align_up(o + (size_t)s.T * s.E * 4, 256);
    w.H = o;      o = align_up(o + (size_t)s.capacity * s.f * esz, 256);
    w.Yr = o;     o = align_up(o + (size_t)down_splits(s) * s.T * kp * s.d * 4, 256);
    w.total = o;
    return w;
}

// Arguments of the grouped expert GEMMs (gate/up + SwiGLU, and down).
// Per slot s the weight slice is B + s * slot_stride, an [N][K] row-major
// matrix; rows of A are gathered X rows (gate/up) or consecutive H rows
// (down) in record order.
struct GemmArgs {
    const int32_t *slot_offset;  // [P+1]
    int P;
    const int32_t *rec_token;    // [C]
    const int32_t *rec_route;    // [C]
    const void *A;               // X (gate/up) or H (down)
    int64_t lda;                 // ldx or f
    const void *B;               // plane base
    int64_t slot_stride;         // elements (bytes for fp8 weights)
    int bfp8;                    // B: fp8 e4m3 codes with fp32 row scales
    int bfp4;                    // B: packed MXFP4 slice (codes and block scales per K piece)
    int64_t scale_off;           // fp8: bytes from a slot slice's start to its row scales
    int N, K;
    void *C;                     // H (gate/up) or Yr (down)
    int64_t ldc;                 // f or d
    int splits;                  // K split in this many equal ranges (down)
    int64_t split_stride;        // elements between the partial outputs
    const float *topk_w;         // down: weight of route i
    int32_t *done;               // down: computed marks
};

// ---- launchers (return hipError_t of the launch) ----
hipError_t launch_router_logits(const moe_shape &s, const void *X, const float *Wr,
                                const float *bias, float *L, hipStream_t st);
hipError_t launch_topk(const moe_shape &s, int t0, int nt, const float *L, int32_t *idx,
                       float *w, int32_t *done, hipStream_t st);
hipError_t launch_route_count(const moe_shape &s, int64_t i0, int64_t n, const int32_t *idx,
                              const PhiArg &phi, int32_t *blk, int32_t *rank, int32_t *err,
                              int32_t *done, int reset, hipStream_t st);
hipError_t launch_route_place(const moe_shape &s, int64_t i0, int64_t n, const int32_t *idx,
                              const PhiArg &phi, const int32_t *blk, const int32_t *rank,
                              int32_t *rec_token, int32_t *rec_route, int32_t *route_pos,
                              int32_t *count, int32_t *offset, hipStream_t st);
hipError_t launch_gate_up(const moe_shape &s, const GemmArgs &a, int max_rows, bool simple,
                          hipStream_t st);
hipError_t launch_down(const moe_shape &s, const GemmArgs &a, int max_rows, bool simple,
                       hipStream_t st);
// Fused expert tile (gate/up, SwiGLU and down in one kernel, H kept in LDS):
// bf16 layers with f <= 1024, d % 128 == 0 and an unsplit down projection.
bool fused_expert_supported(const moe_shape &s);
hipError_t launch_fused_expert(const moe_shape &s, const GemmArgs &gu, const GemmArgs &dn, int max_rows,
                               hipStream_t st);
hipError_t launch_combine(const moe_shape &s, float *Y, const float *Yr, const int32_t *done,
                          hipStream_t st);   // sums the down_splits(s) partial rows of each route
hipError_t launch_pack_gate_up(const moe_shape &s, const void *Wg, const void *Wu, void *dst,
                               int n, int64_t src_stride, int64_t dst_stride, hipStream_t st);
hipError_t launch_pack_down(const moe_shape &s, const void *Wd, void *dst, int n, int64_t src_stride,
                            int64_t dst_stride, hipStream_t st);
hipError_t launch_selftest_mfma(float *out, hipStream_t st);

// Stores a message in the library's error channel (moe_last_error) and
// returns st.
moe_status report_error(moe_status st, const char *msg);
// The resident layer of moe_layer_prefill on a given workspace (all argument
// checks included); with clear_err the workspace's device error word is
// cleared by a kernel first. No host or device memory is allocated.
moe_status layer_prefill_resident(const moe_shape *shape, const void *X, const float *W_r, const float *bias,
                                  const float *logits, float *Y, moe_arena *arena, const moe_routes *routes,
                                  void *ws, size_t ws_bytes, hipStream_t cs, bool clear_err);
hipError_t launch_fill_i32(int32_t *p, int32_t v, int64_t n, hipStream_t st);
hipError_t launch_expert_hist(const moe_shape &s, const int32_t *idx, int64_t n, int32_t *count,
                              hipStream_t st);

}  // namespace moe
