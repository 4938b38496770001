// Grouped expert projections over the route map (EStream, section 3.2,
// "Fused Expert Execution": gather routed rows, gate/up projections as pairs,
// SwiGLU, down projection, weighted scatter; Eq. 1 F_e(x) = W_d (SiLU(W_g x)
// * (W_u x))).
//
// Work is a list of tiles (slot s, BM consecutive records of s, BN columns of
// the slot's weight slice), decoded on the device from the per-slot record
// offsets, so nothing is read back to the host. The ring kernel is persistent
// (as many workgroups as fit on the GPU at once, each walking its tiles); the
// plain kernel is launched for an upper bound on the tile count and surplus
// workgroups leave at once.
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
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));

// Eight fp8 e4m3 codes (bytes 0..7 of w) to eight bf16 values, in order; exact
// (scale 1), two codes per v_cvt_scalef32_pk_bf16_fp8.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(u32x2_t w)
{
    const bf16x2v_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, false);
    const bf16x2v_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.x, 1.0f, true);
    const bf16x2v_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, false);
    const bf16x2v_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w.y, 1.0f, true);
    return bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

struct TileInfo {
    int slot, row0, rows, n0, ks;   // ks: which of the a.splits K ranges
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
            const int w = (cnt + BM - 1) / BM * ntn * a.splits;
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
                const int w = mt * ntn * a.splits;
                const int inc = wave_incl_scan(w, lane);
                const int ex = run + inc - w;
                if (s < a.P && w > 0 && L >= ex && L < ex + w) {
                    const int local = L - ex;
                    const int ml = local % mt, rest = local / mt;
                    ti->slot = s;
                    ti->row0 = a.slot_offset[s] + ml * BM;
                    ti->rows = min(BM, cnt - ml * BM);
                    ti->ks = rest % a.splits;
                    ti->n0 = (rest / a.splits) * BN;
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

// SiLU(g) * u with the hardware exp2 and reciprocal (about 1 ulp each); used
// where the result is rounded to bf16.
__device__ __forceinline__ float silu_mul_fast(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel with direct global->LDS loads and a ring of NS stages.
//
// Tile BM x BN, K step 32 (one stage = BM + BN rows of 64 bytes), WM x WN
// waves, each wave BM/WM x BN/WN as 32x32x16 MFMA tiles
// (v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32 and the 8
// consecutive k values 8*(l / 32) .. +7 of A and of B^T). Operand tiles
// are copied straight from global memory into LDS by global_load_lds_dwordx4
// (16 bytes per lane; one instruction fills 1 KB = 16 rows of one stage), so
// no registers hold staged data and NS-1 stages are in flight while one is
// consumed. Rows are stored XOR-swizzled: the 16-byte chunk c of row r sits
// at chunk position c ^ ((r >> 2) & 3). LDS serves a 16-byte-per-lane read
// for 16 lanes per cycle across 64 banks; 16 consecutive rows at the same
// chunk then land in 16 distinct 16-byte bank groups, so the MFMA fragment
// reads are conflict-free (the DMA writes fill 1 KB contiguously). One
// barrier per stage: after it, every wave's copies into
// this stage have landed (each wave first waits on its own copies) and every
// wave has finished reading the stage that the next copy overwrites.
#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Waits until at most n * STEP vector memory operations of this wave are
// outstanding, for a run-time n in [0, MAXN].
template <int STEP, int MAXN>
__device__ __forceinline__ void wait_vmcnt_stages(int n)
{
    if constexpr (MAXN > 0) {
        if (n >= MAXN) {
            wait_vmcnt<MAXN * STEP>();
            return;
        }
        wait_vmcnt_stages<STEP, MAXN - 1>(n);
    } else {
        wait_vmcnt<0>();
    }
}

// Two floats rounded to bf16 (nearest even) and packed, lo in bits 15:0
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// BF8: the weights (B) are fp8 e4m3 codes with one fp32 scale per weight row
// (the slot slice holds the codes, then the row scales, a.scale_off bytes in).
// B rows then take 32 bytes per stage; each wave's fragments are converted to
// bf16 (exactly: every e4m3 value is a bf16 value) just before its MFMAs, and
// the row scales multiply the fp32 accumulators in the epilogue.
// BF4: the weights (B) are a packed MXFP4 slice. A stage of B holds the tile's
// 256 rows x 16 code bytes (one K piece of 32 weights per row) and the rows'
// 256 E8M0 scale bytes; waves 0-3 copy 1 KB of codes each, waves 4-7 64 B
// of scales each, so every wave issues the same number of copies. A wave
// reads 8 codes (4 bytes) and the row's scale per fragment and decodes them
// with v_cvt_scalef32_pk_bf16_fp4 (code value x power-of-two scale: exact in
// bf16) just before its MFMAs; the epilogue applies no scale.
__device__ __forceinline__ bf16x8_t fp4x8_to_bf16(uint32_t w, float scale)
{
    typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));
    const u32x4v_t u = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3))};
    return __builtin_bit_cast(bf16x8_t, u);
}
// E8M0 scale byte -> fp32: 2^(s-127); s = 0 is the subnormal 2^-127, s = 255 NaN
__device__ __forceinline__ float e8m0_to_f32(uint32_t sb)
{
    return __uint_as_float(sb == 0 ? 0x00400000u : (sb == 255 ? 0x7fc00000u : sb << 23));
}

#ifndef MOE_GEMM_MAX_SLOTS
#define MOE_GEMM_MAX_SLOTS kMaxExp
#endif
constexpr int kGemmMaxSlots = MOE_GEMM_MAX_SLOTS;

template <int BM, int BN, int NS, int WM, int WN, bool GATEUP, bool BF8, bool BF4 = false>
__global__ __launch_bounds__(WM *WN * 64) void k_gemm_mfma_lds(GemmArgs a)
{
    constexpr int NW = WM * WN, NT = NW * 64;
    constexpr int BK = 32, ROWB = 64;                   // bytes per LDS row of A (32 bf16)
    constexpr int BROW = BF8 ? 32 : (BF4 ? 16 : 64);    // bytes per LDS row of B (32 codes or 32 bf16)
    constexpr int BESZ = (BF8 || BF4) ? 1 : 2;          // bytes per B element (B strides in bytes when 1)
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int MI = TM / 32, NI = TN / 32;
    constexpr int STAGE = BM * ROWB + BN * BROW + (BF4 ? BN : 0);   // bytes per stage (BF4: + scales)
    constexpr int AI = BM / 16 / NW, BI = BF4 ? 1 : BN * BROW / 1024 / NW; // copies per wave per stage
    constexpr int LOADS = AI + BI;
    static_assert(BM % (16 * NW) == 0 && (BF4 || (BN * BROW) % (1024 * NW) == 0) && MI >= 1 && NI >= 1, "tile");
    static_assert(!BF4 || (NW == 8 && BN == 256), "MXFP4 copies: 4 waves of codes, 4 of scales");
    static_assert(!(BF8 && BF4), "one weight format");
    static_assert(!GATEUP || (TN % 64) == 0, "gate/up pairs need 64-column wave tiles");
    static_assert(NS >= 3, "the ring needs at least 3 stages");
    static_assert(BK == kWK && kWRows % BN == 0, "a B stage is one K piece of one row block of the tiled layout");

    __shared__ __attribute__((aligned(1024))) char lds[NS * STAGE];
    __shared__ int32_t s_route[2][GATEUP ? 1 : BM];   // by tile parity
    __shared__ float s_alpha[2][GATEUP ? 1 : BM];
    __shared__ float s_scale[2][BF8 ? BN : 1];          // row scales of the tile's B rows, by parity
    __shared__ int32_t s_tpref[kGemmMaxSlots + 1];     // first logical tile of each slot
    __shared__ int32_t s_off[kGemmMaxSlots + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int K = a.K, N = a.N;
    const int Kc = K / a.splits;   // each tile's K range: [ks * Kc, (ks + 1) * Kc)
    const int P = a.P;
    const int ntn = (N + BN - 1) / BN;

    // Tiles of slot s: ceil(count_s / BM) row blocks x ntn column blocks,
    // numbered slot by slot, column block major, row block minor.
    if (tid < 64) {
        int run = 0;
        for (int s0 = 0; s0 < P; s0 += 64) {
            const int s = s0 + lane;
            const int off = s < P ? a.slot_offset[s] : 0;
            const int cnt = s < P ? a.slot_offset[s + 1] - off : 0;
            const int w = (cnt + BM - 1) / BM * ntn * a.splits;
            const int inc = wave_incl_scan(w, lane);
            if (s < P) {
                s_tpref[s] = run + inc - w;
                s_off[s] = off;
            }
            run += __shfl(inc, 63, 64);
        }
        if (lane == 0) {
            s_tpref[P] = run;
            s_off[P] = a.slot_offset[P];
        }
    }
    __syncthreads();
    const int total = s_tpref[P];
    // The workgroups on XCD x = blockIdx % 8 walk one contiguous range of
    // logical tiles together, one tile each per round, so neighbouring tiles
    // (same weight tile, or same gathered rows) run at the same time there.
    const int xcd = blockIdx.x % kXcd, li = blockIdx.x / kXcd;
    const int nwg = ((int)gridDim.x - xcd + kXcd - 1) / kXcd;
    const int qx = total / kXcd, rx = total % kXcd;
    const int cnt_x = qx + (xcd < rx ? 1 : 0), start_x = xcd * qx + min(xcd, rx);
    if (li >= cnt_x) return;

    auto decode = [&](int L) -> TileInfo {
        int lo = 0, hi = P - 1;  // last slot whose first tile is <= L (skips empty slots)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tpref[mid] <= L) lo = mid; else hi = mid - 1;
        }
        const int cnt_s = s_off[lo + 1] - s_off[lo];
        const int mt = (cnt_s + BM - 1) / BM;
        const int local = L - s_tpref[lo];
        const int ml = local % mt;
        TileInfo t;
        t.slot = lo;
        t.row0 = s_off[lo] + ml * BM;
        t.rows = __builtin_amdgcn_readfirstlane(min(BM, cnt_s - ml * BM));
        t.ks = (local / mt) % a.splits;
        t.n0 = (local / mt / a.splits) * BN;
        return t;
    };

    // copy sources: instruction j of this wave covers rows 16*(wave*AI + j)
    // .. +15 of A (and likewise of B); lane -> row + l/4, chunk position l%4
    const char *asrc[AI];
    const char *bsrc[BI];
    int bstep = 0;       // bytes from one stage of B to the next (tiled layout)
    int astep = BK * 2;  // likewise for A (gathered X rows: 64 bytes; H: the block's piece)
    const int lr = lane >> 2, lp = lane & 3;
    // A row of each of this lane's copies (gathered token rows for gate/up)
    auto fetch_rows = [&](const TileInfo &t, int32_t *rows) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int rr = min((wave * AI + j) * 16 + lr, t.rows - 1);
            rows[j] = GATEUP ? a.rec_token[t.row0 + rr] : t.row0 + rr;
        }
    };
    auto set_sources = [&](const TileInfo &t, const int32_t *rows) {
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int r = (wave * AI + j) * 16 + lr;
            const int c = lp ^ ((r >> 2) & 3);
            if (GATEUP) {
                asrc[j] = (const char *)a.A + ((int64_t)rows[j] * a.lda + (int64_t)t.ks * Kc) * 2 + c * 16;
            } else {
                // H rows of this tile's row block, stored block-tiled (see the
                // gate/up epilogue): K pieces of 32 one after another
                const int rr = rows[j] - t.row0;
                asrc[j] = (const char *)a.A +
                          ((int64_t)t.row0 * a.lda + (int64_t)(t.ks * Kc / BK) * t.rows * BK + (int64_t)rr * BK) * 2 +
                          c * 16;
            }
        }
        astep = GATEUP ? BK * 2 : t.rows * BK * 2;
        // The slice is in the tiled layout (wtile_off): the tile's columns lie in
        // one 256-row block whose K pieces of 32 are stored piece after piece,
        // so each stage of B is one contiguous run of rows_nb * 32 elements
        // and the next stage starts bstep bytes further on.
        const char *Bslot = (const char *)a.B + (int64_t)t.slot * a.slot_stride * BESZ;
        const int nb = t.n0 / kWRows;
        const int rows_nb = min(kWRows, N - nb * kWRows);
        if constexpr (BF4) {
            // MXFP4 pieces: rows_nb * 16 code bytes, then the padded scale bytes
            const int64_t piece = fp4_piece_bytes(rows_nb);
            bstep = (int)piece;
            const char *Bblk = Bslot + (int64_t)nb * (K / BK) * fp4_piece_bytes(kWRows) + (int64_t)(t.ks * Kc / BK) * piece;
            if (wave < 4) {
                const int n = min(t.n0 + wave * 64 + lane, N - 1);
                bsrc[0] = Bblk + (int64_t)(n - nb * kWRows) * 16;
            } else {
                const int off = (wave - 4) * 64 + lane * 16;   // lanes 0-3 copy
                bsrc[0] = Bblk + (int64_t)rows_nb * 16 + (off + 16 <= (int)(piece - rows_nb * 16) ? off : 0);
            }
            return;
        }
        bstep = rows_nb * BK * BESZ;
        const char *Bblk = Bslot + ((int64_t)nb * kWRows * K + (int64_t)(t.ks * Kc / BK) * rows_nb * BK) * BESZ;
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            if constexpr (BF8) {
                // 32 rows of 32 bytes per instruction: lane -> row l/2, and the
                // 16-byte half (l%2) ^ ((row >> 3) & 1) of it
                const int r = (wave * BI + j) * 32 + (lane >> 1);
                const int c = (lane & 1) ^ ((r >> 3) & 1);
                const int n = min(t.n0 + r, N - 1);
                bsrc[j] = Bblk + (int64_t)(n - nb * kWRows) * BK + c * 16;
            } else {
                const int r = (wave * BI + j) * 16 + lr;
                const int c = lp ^ ((r >> 2) & 3);
                const int n = min(t.n0 + r, N - 1);
                bsrc[j] = Bblk + (int64_t)(n - nb * kWRows) * BK * 2 + c * 16;
            }
        }
    };
    // down: route id and alpha of tile row tid (threads tid < BM), staged in
    // registers and then stored to the LDS copy of the given parity
    static_assert(NT >= BM, "one route per thread");
    int32_t pre_rt = 0;
    float pre_al = 0.0f;
    auto fetch_route = [&](const TileInfo &t) {
        if (!GATEUP && tid < BM) pre_rt = a.rec_route[t.row0 + min(tid, t.rows - 1)];
    };
    auto fetch_alpha = [&]() {
        if (!GATEUP && tid < BM) pre_al = a.topk_w[pre_rt];
    };
    // fp8 weights: the scale of B row n0 + tid (threads tid < BN)
    float pre_sc = 0.0f;
    auto fetch_scale = [&](const TileInfo &t) {
        if (BF8 && tid < BN) {
            const char *Bslot = (const char *)a.B + (int64_t)t.slot * a.slot_stride;
            pre_sc = *(const float *)(Bslot + a.scale_off + (int64_t)min(t.n0 + tid, N - 1) * 4);
        }
    };
    auto store_routes = [&](int par) {
        if (!GATEUP && tid < BM) {
            s_route[par][tid] = pre_rt;
            s_alpha[par][tid] = pre_al;
        }
        if (BF8 && tid < BN) s_scale[par][tid] = pre_sc;
    };
    auto issue = [&](int kt) {
        char *st = lds + (kt % NS) * STAGE;
        const int64_t kb = (int64_t)kt * astep;
#pragma unroll
        for (int j = 0; j < AI; ++j)
            __builtin_amdgcn_global_load_lds((const GLOBAL_AS void *)(asrc[j] + kb),
                                             (LDS_AS void *)(st + (wave * AI + j) * 1024), 16, 0, 0);
        if constexpr (BF4) {
            // waves 0-3: 64 rows of 16 code bytes; waves 4-7: lanes 0-3 copy 64 scale bytes
            if (wave < 4 || lane < 4)
                __builtin_amdgcn_global_load_lds(
                    (const GLOBAL_AS void *)(bsrc[0] + (int64_t)kt * bstep),
                    (LDS_AS void *)(st + BM * ROWB + (wave < 4 ? wave * 1024 : BN * 16 + (wave - 4) * 64)), 16, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < BI; ++j)
                __builtin_amdgcn_global_load_lds((const GLOBAL_AS void *)(bsrc[j] + (int64_t)kt * bstep),
                                                 (LDS_AS void *)(st + BM * ROWB + (wave * BI + j) * 1024), 16, 0,
                                                 0);
        }
    };

    // fragment addressing: row (lane & 31) of each 32-row tile, logical chunk
    // 2*ks + (lane >> 5), stored at chunk ^ (((lane & 31) >> 2) & 3)
    const int sw = ((lane & 31) >> 2) & 3;
    const int foff[2] = {(lane & 31) * ROWB + ((0 + (lane >> 5)) ^ sw) * 16,
                         (lane & 31) * ROWB + ((2 + (lane >> 5)) ^ sw) * 16};
    f32x16_t acc[MI][NI];
    bf16x8_t af[2][MI], bfr[2][NI];
    u32x2_t braw[2][NI];   // fp8 weights: 8 codes per fragment, converted in mfmas
    // MXFP4: 8 codes per fragment; the row's block scale (one per stage, so
    // read with the step-0 fragments and carried over to step 1)
    uint32_t b4raw[2][NI];
    float b4sc[2][NI];
    const int c4[2] = {(0 + (lane >> 5)) * 4, (2 + (lane >> 5)) * 4};   // code bytes of chunk 2*ks + (lane >> 5)
    // fp8 fragment of B row (lane & 31): 8-byte piece c = 2*ks + (lane >> 5) of
    // the 32-byte row, stored in 16-byte half (c >> 1) ^ ((row >> 3) & 1)
    const int br8 = lane & 31;
    const int boff8[2] = {br8 * 32 + (((0 + (lane >> 5)) >> 1 ^ ((br8 >> 3) & 1)) << 4) + (((0 + (lane >> 5)) & 1) << 3),
                          br8 * 32 + (((2 + (lane >> 5)) >> 1 ^ ((br8 >> 3) & 1)) << 4) + (((2 + (lane >> 5)) & 1) << 3)};
    auto read_frags = [&](int stage, int ks, int set) {
        const char *As = lds + stage * STAGE + wm * TM * ROWB + foff[ks];
#pragma unroll
        for (int i = 0; i < MI; ++i) af[set][i] = *(const bf16x8_t *)(As + i * 32 * ROWB);
        if constexpr (BF8) {
            const char *Bs = lds + stage * STAGE + BM * ROWB + wn * TN * BROW + boff8[ks];
#pragma unroll
            for (int j = 0; j < NI; ++j) braw[set][j] = *(const u32x2_t *)(Bs + j * 32 * BROW);
        } else if constexpr (BF4) {
            const char *Bs = lds + stage * STAGE + BM * ROWB;
            const int r0 = wn * TN + (lane & 31);
#pragma unroll
            for (int j = 0; j < NI; ++j) {
                b4raw[set][j] = *(const uint32_t *)(Bs + (r0 + j * 32) * 16 + c4[ks]);
                if (ks == 0)
                    b4sc[set][j] = e8m0_to_f32(*(const uint8_t *)(Bs + BN * 16 + r0 + j * 32));
                else   // step 1 of the stage whose step-0 fragments are in set 0
                    b4sc[set][j] = b4sc[0][j];
            }
        } else {
            const char *Bs = lds + stage * STAGE + BM * ROWB + wn * TN * ROWB + foff[ks];
#pragma unroll
            for (int j = 0; j < NI; ++j) bfr[set][j] = *(const bf16x8_t *)(Bs + j * 32 * ROWB);
        }
    };
    auto mfmas = [&](int set) {
        if constexpr (BF8) {
#pragma unroll
            for (int j = 0; j < NI; ++j) bfr[set][j] = fp8x8_to_bf16(braw[set][j]);
        }
        if constexpr (BF4) {
#pragma unroll
            for (int j = 0; j < NI; ++j) bfr[set][j] = fp4x8_to_bf16(b4raw[set][j], b4sc[set][j]);
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[set][i], bfr[set][j], acc[i][j], 0, 0, 0);
    };
    // interleave: the (MI + NI) fragment reads of the next step are spread
    // over the MI * NI MFMAs of this step
    constexpr int NRD = MI + NI;   // LDS reads per step (BF4: the scale reads of step 0 ride along)
    auto interleave = [&]() {
#pragma unroll
        for (int q = 0; q < (NRD < MI * NI ? NRD : MI * NI); ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        if constexpr (MI * NI > NRD) __builtin_amdgcn_sched_group_barrier(0x008, MI * NI - NRD, 0);
        if constexpr (NRD > MI * NI) __builtin_amdgcn_sched_group_barrier(0x100, NRD - MI * NI, 0);
    };

    const int nk = Kc / BK;
    int tl = li, par = 0;
    TileInfo cur = decode(start_x + tl);
    int32_t rows[AI];
    fetch_rows(cur, rows);
    set_sources(cur, rows);
    fetch_route(cur);
    fetch_scale(cur);
    fetch_alpha();
    store_routes(0);
#pragma unroll
    for (int p = 0; p < NS - 1; ++p)
        if (p < nk) issue(p);

    for (;;) {
        const bool wave_active = wm * TM < cur.rows;
        // The next tile of this workgroup (nwg further on in the XCD's range):
        // its row indices, route ids and alphas are requested during the first
        // two steps of this tile, so that the switch at the end of the tile
        // waits on nothing.
        const int tn = tl + nwg;
        const bool has_next = tn < cnt_x;
        const TileInfo nxt = has_next ? decode(start_x + tn) : cur;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // Stage 0 of this tile is complete and visible. Loads return in
        // order, and min(NS-2, nk-1) stages were requested after stage 0, so
        // stage 0 is complete once no more than their copies are outstanding
        // (operations issued later, such as the previous tile's output
        // stores, only make the wait stricter). The barrier also drains the
        // previous tile's stores: left outstanding, they make the compiler
        // guard the k loop's fragment reads with a full vmcnt(0) every step.
        wait_vmcnt_stages<LOADS, NS - 2>(min(NS - 2, nk - 1));
        __syncthreads();
        if (wave_active) read_frags(0, 0, 0);

        // Invariant at the top of step kt: stage kt is complete and visible
        // to every wave, and this wave holds stage kt's step-0 fragments in
        // set 0. During step kt, stage kt+1 is made visible (own copies
        // waited for, then a barrier), so that its step-0 fragments can be
        // read while stage kt's last MFMAs run, and stage kt+NS-1 is
        // requested into the slot of stage kt-1, which every wave finished
        // before that barrier.
        for (int kt = 0; kt < nk; ++kt) {
            const int stage = kt % NS;
            const bool more = kt + 1 < nk;
            if (more) {
                // stage kt+1 complete: the stages requested after it are
                // kt+2 .. min(kt+NS-2, nk-1)
                wait_vmcnt_stages<LOADS, NS - 3>(min(NS - 3, nk - 2 - kt));
                // A bare barrier: the stage's data is visible once every wave
                // has waited on its own copies, and the slot refilled below was
                // last read by fragment loads whose results fed MFMAs issued
                // before this point, so no LDS counter needs draining here.
                __builtin_amdgcn_s_barrier();
            }
            if (has_next && kt == 0) {
                fetch_rows(nxt, rows);
                fetch_route(nxt);
                fetch_scale(nxt);
            }
            if (has_next && kt == 1) fetch_alpha();
            if (more && kt + NS - 1 < nk) issue(kt + NS - 1);
            if (wave_active) {
                read_frags(stage, 1, 1);
                mfmas(0);
                interleave();
                // next stage's step-0 fragments (on the last step this re-reads
                // a resident stage; the values are not used)
                read_frags((kt + 1) % NS, 0, 0);
                mfmas(1);
                interleave();
            }
        }

        // Start the next tile's copies before this tile's epilogue, which
        // works from registers: once every wave is past this barrier nothing
        // reads the ring any more.
        if (has_next) {
            if (nk < 2) fetch_alpha();
            __syncthreads();
            set_sources(nxt, rows);
#pragma unroll
            for (int p = 0; p < NS - 1; ++p)
                if (p < nk) issue(p);
            store_routes(par ^ 1);  // the other parity: last read two tiles ago
        }

        // Result layout: register r of lane l holds row 8*(r/4) + 4*(l/32) +
        // r%4 and column l%32 of its 32x32 block. Gate/up: registers r and r+1
        // (r even) are rows R and R+1; adjacent lanes swap one of the two
        // values (a DPP lane swap), so that the even lane holds columns
        // (c, c+1) of row R and the odd lane the same columns of row R+1, and
        // each store instruction writes four whole 64-byte row segments of H.
        // A full tile stores without per-element checks.
        const bool even = (lane & 1) == 0;
        const int cpair = (lane & 31) & ~1;
        const bool full = cur.rows == BM && cur.n0 + BN <= N;
        // fp8 weights: the row scale of each of this lane's accumulator columns
        float sc[NI];
#pragma unroll
        for (int j = 0; j < NI; ++j) sc[j] = BF8 ? s_scale[par][wn * TN + j * 32 + (lane & 31)] : 1.0f;
        auto epilogue = [&](auto checked_t) {
            constexpr bool checked = decltype(checked_t)::value;
            if constexpr (GATEUP) {
                uint16_t *H = (uint16_t *)a.C;
                const int fN = N / 2;
                const int fc0 = ((cur.n0 + wn * TN) / 64) * 32 + cpair;   // first H column pair
                // H is stored block-tiled: the records of this tile's row block
                // (row0 .. row0+rows-1) occupy the same span as row-major, with
                // their columns cut into pieces of 32 stored piece after piece,
                // so that each K step of the down tile reads one contiguous run.
                uint16_t *hbase = H + (int64_t)cur.row0 * a.ldc + (int64_t)(fc0 / BK) * cur.rows * BK + (fc0 % BK);
                const int qstep = cur.rows * BK;
#pragma unroll
                for (int i = 0; i < MI; ++i) {
#pragma unroll
                    for (int r = 0; r < 16; r += 2) {
                        const int m = wm * TM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3) + (even ? 0 : 1);
                        const int mm = checked ? min(m, cur.rows - 1) : m;
#pragma unroll
                        for (int q = 0; q < NI / 2; ++q) {
                            const float s0 = BF8 ? silu_mul_fast(acc[i][2 * q][r] * sc[2 * q], acc[i][2 * q + 1][r] * sc[2 * q + 1])
                                                 : silu_mul_fast(acc[i][2 * q][r], acc[i][2 * q + 1][r]);
                            const float s1 = BF8 ? silu_mul_fast(acc[i][2 * q][r + 1] * sc[2 * q], acc[i][2 * q + 1][r + 1] * sc[2 * q + 1])
                                                 : silu_mul_fast(acc[i][2 * q][r + 1], acc[i][2 * q + 1][r + 1]);
                            const float y = __int_as_float(
                                __builtin_amdgcn_mov_dpp(__float_as_int(even ? s1 : s0), 0xB1, 0xF, 0xF, false));
                            const uint32_t packed = even ? pack_bf16x2(s0, y) : pack_bf16x2(y, s1);
                            if (!checked || (m < cur.rows && fc0 + q * 32 < fN))
                                *(uint32_t *)(hbase + q * qstep + mm * BK) = packed;
                        }
                    }
                }
            } else {
                // Down: each accumulator register is stored as it stands, lanes
                // 0-31 writing 32 consecutive columns (128 bytes) of row R and
                // lanes 32-63 the same columns of row R+4: plain 4-byte stores
                // drain faster per CU than paired 8-byte ones and need no swap.
                float *Yr = (float *)a.C + cur.ks * a.split_stride;
                const int ncol = cur.n0 + wn * TN + (lane & 31);
#pragma unroll
                for (int i = 0; i < MI; ++i) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int m = wm * TM + i * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
                        const int mc = checked ? min(m, cur.rows - 1) : m;
                        float *yrow = Yr + (int64_t)s_route[par][mc] * a.ldc + ncol;
                        const float al = s_alpha[par][mc];
#pragma unroll
                        for (int j = 0; j < NI; ++j)
                            if (!checked || (m < cur.rows && ncol + j * 32 < N))
                                yrow[j * 32] = BF8 ? al * (acc[i][j][r] * sc[j]) : al * acc[i][j][r];
                    }
                }
            }
        };
        if (full)
            epilogue(std::integral_constant<bool, false>());
        else
            epilogue(std::integral_constant<bool, true>());
        if constexpr (!GATEUP) {
            if (cur.n0 == 0 && cur.ks == 0)
                for (int m = tid; m < cur.rows; m += NT) a.done[s_route[par][m]] = 1;
        }
        if (!has_next) break;
        cur = nxt;
        tl = tn;
        par ^= 1;
    }
}

// ---------------------------------------------------------------------------
// Plain LDS-tiled kernel (fp32 FMA on the vector ALUs, whose fp32 peak on
// this GPU equals the matrix cores' fp32 peak) for fp32 layers; also runs bf16
// inputs as an independent second path (its H is row-major [C][f]; the ring
// kernels' H is block-tiled, and a call always runs both projections with the
// same kernel). 64x64 tiles, K step 64 (each thread has its 16 + 16 loads of a
// step in flight at once: the layers this kernel serves are small and
// latency-bound), 256 threads with 4x4 outputs each; every output is one fmaf
// chain in ascending k. For gate/up a thread owns columns
// {2tx, 2tx+1} (gate) and {32+2tx, 32+2tx+1} (up) of its 64-column block, so
// both halves of each SwiGLU pair are in one thread.
template <typename TE, bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_simple(GemmArgs a)
{
    constexpr int BM = 64, BN = 64, BK = 64;
    __shared__ TileInfo ti;
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BN + 4];
    __shared__ int32_t s_route[BM];
    __shared__ float s_alpha[BM];
    if (!find_tile<BM, BN>(a, &ti)) return;
    const int slot = ti.slot, row0 = ti.row0, rows = ti.rows, n0 = ti.n0;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int K = a.K / a.splits, N = a.N;   // this tile's K range: [kb, kb + K)
    const int64_t kb = (int64_t)ti.ks * K;

    int col[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) col[j] = GATEUP ? ((j < 2) ? 2 * tx + j : 32 + 2 * tx + (j - 2)) : tx * 4 + j;

    const int lr = tid >> 2, lk = (tid & 3) * (BK / 4);
    const int rr = min(lr, rows - 1);
    const TE *ap = (GATEUP ? (const TE *)a.A + (int64_t)a.rec_token[row0 + rr] * a.lda
                           : (const TE *)a.A + (int64_t)(row0 + rr) * a.lda) + kb;
    // B row n of the slice, in the tiled layout (wtile_off)
    const TE *bslice = (const TE *)a.B + (int64_t)slot * a.slot_stride;
    const int64_t bn = min(n0 + lr, N - 1);
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
        for (int q = 0; q < BK / 4; ++q) {
            const int kk = k0 + lk + q;
            As[lk + q][lr] = kk < K ? ld_f32<TE>(ap + kk) : 0.0f;
            Bs[lk + q][lr] = kk < K ? ld_f32<TE>(bslice + wtile_off(bn, kb + kk, N, a.K)) : 0.0f;
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
            float *Yr = (float *)a.C + ti.ks * a.split_stride;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = n0 + col[j];
                if (n < N) Yr[(int64_t)s_route[m] * a.ldc + n] = s_alpha[m] * acc[i][j];
            }
        }
    }
    if (!GATEUP && n0 == 0 && ti.ks == 0 && tid < rows) a.done[s_route[tid]] = 1;
}

// Upper bound of tiles: sum over slots of ceil(c_s / BM) <= ceil(R / BM) + P,
// times the column blocks and the K splits.
inline unsigned grid_bound(const GemmArgs &a, int max_rows, int BM, int BN)
{
    const int64_t mt = (max_rows + BM - 1) / BM + a.P;
    const int64_t ntn = (a.N + BN - 1) / BN;
    return (unsigned)(mt * ntn * a.splits);
}

inline int device_cus()
{
    static int cus = 0;
    if (cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return cus;
}

// fp8 B stages are half the size, so a deeper ring would fit; 5 and 6 stages
// measured no faster than the bf16 kernel's 4 (OLMoE T=4096, Mixtral T=256).
#ifdef MOE_FP8_STAGES
#define MOE_FP8_STAGES_OF(NS) MOE_FP8_STAGES
#else
#define MOE_FP8_STAGES_OF(NS) NS
#endif

template <int BM, int BN, int NS, int WM, int WN, bool GATEUP>
hipError_t launch_mfma_lds(const GemmArgs &a, int max_rows, hipStream_t st)
{
    // persistent workgroups, as many as fit on the GPU at once (one per
    // compute unit when the LDS ring fills it), never more than there can be
    // tiles
    if (a.P > kGemmMaxSlots) return hipErrorInvalidValue;   // the slot tables live in LDS
    auto kern = a.bfp8   ? (const void *)k_gemm_mfma_lds<BM, BN, MOE_FP8_STAGES_OF(NS), WM, WN, GATEUP, true>
                : a.bfp4 ? (const void *)k_gemm_mfma_lds<BM, BN, NS, WM, WN, GATEUP, false, true>
                         : (const void *)k_gemm_mfma_lds<BM, BN, NS, WM, WN, GATEUP, false>;
    int per_cu = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WM * WN * 64, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const unsigned g = std::min<unsigned>(grid_bound(a, max_rows, BM, BN), (unsigned)per_cu * (unsigned)device_cus());
    if (g == 0) return hipSuccess;
    if (a.bfp8)
        hipLaunchKernelGGL((k_gemm_mfma_lds<BM, BN, MOE_FP8_STAGES_OF(NS), WM, WN, GATEUP, true>), dim3(g),
                           dim3(WM * WN * 64), 0, st, a);
    else if (a.bfp4)
        hipLaunchKernelGGL((k_gemm_mfma_lds<BM, BN, NS, WM, WN, GATEUP, false, true>), dim3(g),
                           dim3(WM * WN * 64), 0, st, a);
    else
        hipLaunchKernelGGL((k_gemm_mfma_lds<BM, BN, NS, WM, WN, GATEUP, false>), dim3(g), dim3(WM * WN * 64), 0,
                           st, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused expert tile (section 3.2, "Fused Expert Execution with Intra-NPU
// Pipelining": the SwiGLU output stays on chip until the down projection
// consumes it). One workgroup takes FBM = 64 records of one slot through both
// projections:
//   phase 1: H = SiLU(X W_g^T) * (X W_u^T) for all f hidden units, 128 packed
//            gate/up columns (64 hidden units) per pass over K = d, written
//            to LDS as bf16 (64 x f x 2 bytes, at most 128 KB);
//   phase 2: out = H W_d^T, 128 output columns per pass over K = f, with H
//            read from LDS; alpha * out goes to the route's row of Yr, as the
//            split down kernel writes it.
// Both phases run the split kernels' MFMA instruction over the same k order
// with the same fragments, and H is rounded to bf16 the same way, so the
// results equal theirs bit for bit; H just never goes to HBM. Operands
// stream through a 2-stage LDS ring (12 KB per stage: 64 gathered X rows and
// 128 weight rows of one 32-wide K piece in phase 1, 128 weight rows in phase
// 2); 4 waves, each 32 rows x 64 columns. H in LDS is stored like a ring
// stage per K piece of 32 hidden units (64 rows of 64 bytes, 16-byte chunks
// XOR-swizzled by row), so phase 2 reads its A fragments the way the ring
// kernels read a stage. Tiles are numbered slot by slot and dealt to the
// XCDs in contiguous ranges, as in the split kernels.
constexpr int FBM = 64, FNT = 256, FMAXF = 1024;

__global__ __launch_bounds__(FNT, 1) void k_fused_expert(GemmArgs g, GemmArgs dn, int max_tiles)
{
    constexpr int BK = 32, ROWB = 64, STAGE = FBM * ROWB + 128 * ROWB;   // 12 KB
    constexpr int HPIECE = FBM * ROWB;                                     // 4 KB per 32 hidden units
    __shared__ __attribute__((aligned(1024))) char hs[FMAXF / BK * HPIECE];
    __shared__ __attribute__((aligned(1024))) char ring[2 * STAGE];
    __shared__ int32_t s_route[FBM];
    __shared__ float s_alpha[FBM];
    __shared__ int32_t s_tpref[kGemmMaxSlots + 1];
    __shared__ int32_t s_off[kGemmMaxSlots + 1];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rh = wave >> 1, ch = wave & 1;    // 32-row half, 64-column half
    const int P = g.P, d = g.K, f = dn.K;
    if (tid < 64) {
        int run = 0;
        for (int s0 = 0; s0 < P; s0 += 64) {
            const int s = s0 + lane;
            const int off = s < P ? g.slot_offset[s] : 0;
            const int cnt = s < P ? g.slot_offset[s + 1] - off : 0;
            const int w = (cnt + FBM - 1) / FBM;
            const int inc = wave_incl_scan(w, lane);
            if (s < P) {
                s_tpref[s] = run + inc - w;
                s_off[s] = off;
            }
            run += __shfl(inc, 63, 64);
        }
        if (lane == 0) {
            s_tpref[P] = run;
            s_off[P] = g.slot_offset[P];
        }
    }
    __syncthreads();
    const int total = min(s_tpref[P], max_tiles);
    const int xcd = blockIdx.x % kXcd, li = blockIdx.x / kXcd;
    const int nwg = ((int)gridDim.x - xcd + kXcd - 1) / kXcd;
    const int qx = total / kXcd, rx = total % kXcd;
    const int cnt_x = qx + (xcd < rx ? 1 : 0), start_x = xcd * qx + min(xcd, rx);

    const int lr = lane >> 2, lp = lane & 3;
    const int sw = ((lane & 31) >> 2) & 3;
    const int foff[2] = {(lane & 31) * ROWB + ((0 + (lane >> 5)) ^ sw) * 16,
                         (lane & 31) * ROWB + ((2 + (lane >> 5)) ^ sw) * 16};
    const int nk1 = d / BK, nk2 = f / BK;
    const int n1 = (2 * f / 128) * nk1, n2 = (d / 128) * nk2;

    for (int tl = li; tl < cnt_x; tl += nwg) {
        const int L = start_x + tl;
        int lo = 0, hi = P - 1;   // last slot whose first tile is <= L
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_tpref[mid] <= L) lo = mid; else hi = mid - 1;
        }
        const int slot = lo;
        const int row0 = s_off[slot] + (L - s_tpref[slot]) * FBM;
        const int rows = __builtin_amdgcn_readfirstlane(min(FBM, s_off[slot + 1] - row0));
        __syncthreads();   // every wave is done with the previous tile's route entries
        if (tid < FBM) {
            const int rt = dn.rec_route[row0 + min(tid, rows - 1)];
            s_route[tid] = rt;
            s_alpha[tid] = dn.topk_w[rt];
        }
        // this lane's gathered X row (A rows 16 wave + lane / 4) and its chunk
        const int ar = wave * 16 + lr;
        const char *xrow = (const char *)g.A + (int64_t)g.rec_token[row0 + min(ar, rows - 1)] * g.lda * 2 +
                           (lp ^ ((ar >> 2) & 3)) * 16;
        const char *gslot = (const char *)g.B + (int64_t)slot * g.slot_stride * 2;
        const char *dslot = (const char *)dn.B + (int64_t)slot * dn.slot_stride * 2;
        // B copies: rows 32 wave + 16 j + lane / 4 of a 128-row weight stage
        auto bsrc = [&](const char *sl, int N, int K, int n0, int kt, int j) {
            const int r = wave * 32 + j * 16 + lr;
            const int nb = n0 / kWRows, rows_nb = min(kWRows, N - nb * kWRows);
            return sl + ((int64_t)nb * kWRows * K + (int64_t)kt * rows_nb * BK + (int64_t)(n0 % kWRows + r) * BK) * 2 +
                   (lp ^ ((r >> 2) & 3)) * 16;
        };
        auto issue1 = [&](int st) {
            const int cb = st / nk1, kt = st % nk1;
            char *stg = ring + (st & 1) * STAGE;
            __builtin_amdgcn_global_load_lds((const GLOBAL_AS void *)(xrow + (int64_t)kt * BK * 2),
                                             (LDS_AS void *)(stg + wave * 1024), 16, 0, 0);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_global_load_lds((const GLOBAL_AS void *)bsrc(gslot, g.N, d, cb * 128, kt, j),
                                                 (LDS_AS void *)(stg + FBM * ROWB + (wave * 2 + j) * 1024), 16, 0,
                                                 0);
        };
        auto issue2 = [&](int st) {
            const int nb2 = st / nk2, kt = st % nk2;
            char *stg = ring + (st & 1) * STAGE;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                __builtin_amdgcn_global_load_lds((const GLOBAL_AS void *)bsrc(dslot, dn.N, f, nb2 * 128, kt, j),
                                                 (LDS_AS void *)(stg + (wave * 2 + j) * 1024), 16, 0, 0);
        };

        f32x16_t acc[2];
        // phase 1: gate/up pairs and SwiGLU into LDS
        __syncthreads();   // the previous tile is done with the ring and the route entries are in
        issue1(0);
        for (int st = 0; st < n1; ++st) {
            const int cb = st / nk1, kt = st % nk1;
            wait_vmcnt<0>();
            __syncthreads();
            if (st + 1 < n1) issue1(st + 1);
            if (kt == 0)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
            const char *stg = ring + (st & 1) * STAGE;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t a = *(const bf16x8_t *)(stg + rh * 32 * ROWB + foff[ks]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bf16x8_t b = *(const bf16x8_t *)(stg + FBM * ROWB + (ch * 64 + j * 32) * ROWB + foff[ks]);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
                }
            }
            if (kt == nk1 - 1) {
                // hidden units cb * 64 + ch * 32 + (lane & 31): K piece 2 cb + ch of H
                char *hp = hs + (2 * cb + ch) * HPIECE;
                const int c = lane & 31;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int R = rh * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
                    const uint32_t h2 = pack_bf16x2(silu_mul_fast(acc[0][r], acc[1][r]), 0.0f);
                    *(uint16_t *)(hp + R * ROWB + (((c >> 3) ^ ((R >> 2) & 3)) << 4) + (c & 7) * 2) = (uint16_t)h2;
                }
            }
        }
        // phase 2: down projection from H in LDS, alpha * out into the route rows
        wait_vmcnt<0>();
        __syncthreads();   // H complete; the ring is free
        issue2(0);
        for (int st = 0; st < n2; ++st) {
            const int nb2 = st / nk2, kt = st % nk2;
            wait_vmcnt<0>();
            __syncthreads();
            if (st + 1 < n2) issue2(st + 1);
            if (kt == 0)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
            const char *stg = ring + (st & 1) * STAGE;
            const char *hpc = hs + kt * HPIECE;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t a = *(const bf16x8_t *)(hpc + rh * 32 * ROWB + foff[ks]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const bf16x8_t b = *(const bf16x8_t *)(stg + (ch * 64 + j * 32) * ROWB + foff[ks]);
                    acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
                }
            }
            if (kt == nk2 - 1) {
                float *Yr = (float *)dn.C;
                const int ncol = nb2 * 128 + ch * 64 + (lane & 31);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = rh * 32 + 8 * (r / 4) + 4 * (lane >> 5) + (r & 3);
                    if (m < rows) {
                        float *yrow = Yr + (int64_t)s_route[m] * dn.ldc + ncol;
                        const float al = s_alpha[m];
#pragma unroll
                        for (int j = 0; j < 2; ++j) yrow[j * 32] = al * acc[j][r];
                    }
                }
            }
        }
        for (int m = tid; m < rows; m += FNT) dn.done[s_route[m]] = 1;
    }
}

template <typename TE, bool GATEUP>
hipError_t launch_simple(const GemmArgs &a, int max_rows, hipStream_t st)
{
    const unsigned g = grid_bound(a, max_rows, 64, 64);
    if (g == 0) return hipSuccess;
    hipLaunchKernelGGL((k_gemm_simple<TE, GATEUP>), dim3(g), dim3(256), 0, st, a);
    return hipGetLastError();
}

inline hipError_t launch_fused_impl(const GemmArgs &gu, const GemmArgs &dn, int max_rows, hipStream_t st)
{
    if (gu.P > kGemmMaxSlots) return hipErrorInvalidValue;
    const int64_t tiles = (max_rows + FBM - 1) / FBM + gu.P;
    const unsigned grid = (unsigned)std::min<int64_t>(tiles, device_cus());
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL(k_fused_expert, dim3(grid), dim3(FNT), 0, st, gu, dn, (int)tiles);
    return hipGetLastError();
}

}  // namespace

bool fused_expert_supported(const moe_shape &s)
{
    return s.dtype == MOE_DT_BF16 && s.f <= FMAXF && (s.d % 128) == 0 && (s.f % 64) == 0 && down_splits(s) == 1;
}

hipError_t launch_fused_expert(const moe_shape &s, const GemmArgs &gu, const GemmArgs &dn, int max_rows,
                               hipStream_t st)
{
    if (max_rows == 0) return hipSuccess;
    if (!fused_expert_supported(s)) return hipErrorInvalidValue;
    return launch_fused_impl(gu, dn, max_rows, st);
}

// Tile shape of the ring kernel: tile rows, tile columns, stages, wave rows,
// wave columns. (128- and 64-row tiles were measured slower than 256-row
// tiles with idle rows, down to 64 routes per expert.)
#ifndef MOE_RING_TILE
#define MOE_RING_TILE 256, 256, 4, 4, 2
#endif

// MXFP4 weights: 2 wave rows x 4 wave columns, so that each weight fragment
// is decoded by 2 waves instead of 4 (bf16 and fp8 measured slower so).
#ifndef MOE_FP4_TILE
#define MOE_FP4_TILE 256, 256, 4, 2, 4
#endif

hipError_t launch_gate_up(const moe_shape &s, const GemmArgs &a, int max_rows, bool simple,
                          hipStream_t st)
{
    if (max_rows == 0) return hipSuccess;
    if (s.dtype == MOE_DT_F32) return launch_simple<float, true>(a, max_rows, st);
    if (simple) {
        if (a.bfp8 || a.bfp4) return hipErrorInvalidValue;   // the plain kernel reads bf16 weights only
        return launch_simple<uint16_t, true>(a, max_rows, st);
    }
    if (a.bfp4) return launch_mfma_lds<MOE_FP4_TILE, true>(a, max_rows, st);
    return launch_mfma_lds<MOE_RING_TILE, true>(a, max_rows, st);
}

hipError_t launch_down(const moe_shape &s, const GemmArgs &a, int max_rows, bool simple,
                       hipStream_t st)
{
    if (max_rows == 0) return hipSuccess;
    if (s.dtype == MOE_DT_F32) return launch_simple<float, false>(a, max_rows, st);
    if (simple) {
        if (a.bfp8 || a.bfp4) return hipErrorInvalidValue;
        return launch_simple<uint16_t, false>(a, max_rows, st);
    }
    if (a.bfp4) return launch_mfma_lds<MOE_FP4_TILE, false>(a, max_rows, st);
    return launch_mfma_lds<MOE_RING_TILE, false>(a, max_rows, st);
}

}  // namespace moe
