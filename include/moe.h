/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer library.
 *
 * One sparse MoE layer's routed expert FFN over a whole prompt, as in
 * "EStream: Fast and Memory-Efficient MoE Prefill through Expert
 * Virtualization on Mobile NPUs" (arXiv 2609.06551):
 *   router logits -> top-k routing (section 2.2) -> route map per physical
 *   slot (section 3.2, Algorithm 1: slot resolve, count, prefix sum, stable
 *   placement) -> gathered SwiGLU gate/up/down projections (Eq. 1) ->
 *   route-weighted combine into the residual accumulator (Eq. 2),
 * with experts held in a fixed-address slot arena (Eq. 3) that can be paged
 * from pinned host memory (section 3.3, Eq. 4; section 3.4).
 *
 * Conventions
 *  - Every pointer named "device" is GPU memory owned by the caller; the
 *    library never frees it and never allocates device memory in a call.
 *    "host" pointers are CPU memory owned by the caller.
 *  - Streams are hipStream_t values passed as moe_stream (NULL = the null
 *    stream). Every call that takes a stream only enqueues work on it and
 *    returns without waiting for the GPU, unless stated otherwise.
 *  - Calls return MOE_OK (0) or a negative moe_status. Arguments are checked
 *    on the host before anything is enqueued; on error nothing is enqueued
 *    and moe_last_error() describes the problem. Problems only the GPU can
 *    see (an expert id outside [0, E + n_shared) in a caller-supplied top-k)
 *    set a bit in the device error word held in the workspace; such routes
 *    are left out, and moe_device_errors() reports and clears the word.
 *  - Index tensors are int32, route weights and logits fp32, the output
 *    accumulator fp32. X, the expert weights and the intermediate H use
 *    moe_shape.dtype (bf16 or fp32); with MOE_DT_BF16_FP8W and
 *    MOE_DT_BF16_FP4W, X and H are bf16 and the expert weights are stored
 *    quantised (formats below).
 *  - Route numbering: route i = t * K' + j sends token t to its rank-j
 *    expert, K' = k + n_shared. Ranks 0..k-1 are the routed top-k in
 *    descending logit order; ranks k..K'-1 are the shared experts
 *    E..E+n_shared-1 with weight 1.
 *  - Concurrency: calls with their own workspace and descriptors may be in
 *    flight on different streams at once. A workspace or a descriptor set
 *    used by two calls on different streams must be ordered by the caller
 *    (same stream, or events). An arena may be used from several streams
 *    and host threads: its residency table is updated under a lock and
 *    orders loads into a slot after the slot's last use with events.
 *    moe_last_error() reports the calling host thread's last error.
 */
#ifndef ROUTED_EXPERT_FFN_MOE_H
#define ROUTED_EXPERT_FFN_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
typedef void *moe_stream; /* a hipStream_t */

#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad map       */
#define MOE_ERR_CAPACITY (-2)    /* more routes than the descriptors hold  */
#define MOE_ERR_SLOT_STATE (-3)  /* residency protocol violated            */
#define MOE_ERR_WORKSPACE (-4)   /* workspace missing or too small         */
#define MOE_ERR_HIP (-5)         /* a HIP runtime call failed              */
#define MOE_ERR_UNSUPPORTED (-6) /* shape outside what the kernels cover   */

#define MOE_DT_F32 0
#define MOE_DT_BF16 1
/* bf16 activations; expert weights stored as fp8 e4m3 codes (OCP 8-bit
 * float: sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities,
 * S.1111.111 is NaN) with one fp32 scale per weight row, a weight being code
 * times its row's scale: the weight-only quantised experts of the pages'
 * quantised-weight path. A weight slice handed to the packing calls holds
 * its codes row-major followed by its rows' fp32 scales; a packed slice in
 * the arena ([2f][d] gate/up or [d][f] down) holds its codes in the tiled
 * layout of the packing calls followed by its rows' scales ([2f] or [d]) in
 * packed row order; slot strides are then in bytes. The expert kernels
 * decode the codes to bf16 operands exactly and scale the fp32
 * accumulators. */
#define MOE_DT_BF16_FP8W 2
/* bf16 activations; expert weights in OCP MXFP4: 4-bit E2M1 codes (sign, 2
 * exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2,
 * 3, 4, 6) and one E8M0 scale byte (2^(s-127)) per row and block of 32
 * weights along K; a weight is code value times its block's scale, which is
 * exact in bf16. A source slice [N][K] for the packing calls holds the codes
 * row-major, two per byte (element 2i in the low nibble of byte i), then the
 * scales [N][K/32]; its size is N*K/2 + N*K/32 bytes. The packed slice in the
 * arena holds, for each block of 256 rows and each K piece of 32, the rows'
 * 16 code bytes one row after another, then their scale bytes padded with
 * zeros to a multiple of 16 (so one K step of a weight tile is one
 * contiguous run). Strides and slice sizes are in bytes. K (d for gate/up, f
 * for down) must be a multiple of 32. The expert kernels decode the codes
 * with their block scales to bf16 operands (exact). */
#define MOE_DT_BF16_FP4W 3

/* Device error word bits (moe_device_errors). */
#define MOE_DEVERR_EXPERT_ID 1 /* a top-k id outside [0, E + n_shared) */

/* moe_route_build flags */
#define MOE_ROUTE_RESET 1 /* forget which routes of the token range have been
                             computed (implied when logits are given) */

/* moe_expert_ffn flags */
#define MOE_FFN_EXPERTS 1  /* run gate/up + SwiGLU and down for the routes */
#define MOE_FFN_FINALIZE 2 /* combine: Y[t] += sum_j Yr[t*K' + j], fixed j order */
#define MOE_FFN_SIMPLE_KERNEL 4 /* bf16: run the projections with the plain
                                   LDS-tiled vector-ALU kernel instead of the
                                   MFMA kernel (an independent second path);
                                   MOE_ERR_UNSUPPORTED with fp8 or MXFP4
                                   weights */
#define MOE_FFN_FUSED 8 /* bf16 weights: one fused kernel per 64-record tile
                           runs gate/up, SwiGLU and down with H kept on chip
                           (section 3.2, fused expert execution); the same
                           bits as the two projection kernels. Needs f <= 1024,
                           d % 128 == 0 and an unsplit down projection (see
                           moe_expert_ffn), MOE_ERR_UNSUPPORTED otherwise. */

/* Residency states (section 3.3, "Bounded Parameter Arena and Safe Slot Reuse") */
#define MOE_SLOT_AVAILABLE 0
#define MOE_SLOT_FILLING 1
#define MOE_SLOT_READY 2
#define MOE_SLOT_IN_USE 3

#define MOE_MAX_EXPERTS 512 /* E + n_shared and P are at most this */

/*
 * Layer shape. T tokens of hidden size d, E routed experts of inner size f,
 * top-k routing plus n_shared always-on experts, P arena slots, and a route
 * capacity C (section 3.2: descriptors reserve capacity for at most C
 * routes; a build may place at most C routes, larger route sets are split
 * across invocations by token range).
 * Limits: 1 <= k <= E <= 256, k + n_shared <= 64, E + n_shared <= 512,
 * 1 <= P <= 512, T >= 0, T * (k + n_shared) <= 2^30 - 1 routes,
 * T * ceil(d / 1024) < 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 * bf16 and bf16 with fp8 weights: d % 64 == 0, f % 64 == 0.
 * fp32: d % 4 == 0, f % 32 == 0.
 */
typedef struct moe_shape {
    int32_t T;
    int32_t d;
    int32_t f;
    int32_t E;
    int32_t k;
    int32_t n_shared;
    int32_t P;
    int32_t capacity; /* C, >= 1 */
    int32_t dtype;    /* MOE_DT_BF16, MOE_DT_BF16_FP8W, MOE_DT_BF16_FP4W or MOE_DT_F32 */
    int32_t renorm;   /* 1: top-k weights renormalised over the k selected */
    int64_t ldx;      /* row stride of X in elements, >= d */
    int64_t ldy;      /* row stride of Y in elements, >= d, multiple of 4 */
} moe_shape;

/*
 * Route descriptors (section 3.2, "Composed Sparse Route and Parameter
 * Binding"; the compressed-sparse-row route map). All device, caller-owned.
 *   topk_idx    [T][K'] int32  expert ids by rank (written from logits, or
 *                              supplied by the caller)
 *   topk_w      [T][K'] fp32   route weights alpha
 *   slot_count  [P]     int32  routes placed in each slot by the last build
 *   slot_offset [P+1]   int32  exclusive prefix sum of slot_count;
 *                              slot_offset[P] = n_valid
 *   rec_token   [C]     int32  token of record p (records of slot s occupy
 *                              [slot_offset[s], slot_offset[s+1]), in
 *                              ascending route order)
 *   rec_route   [C]     int32  route index i of record p
 *   route_pos   [T*K']  int32  record position of route i in the last build
 *                              that covered it, -1 if it was left out
 */
typedef struct moe_routes {
    int32_t *topk_idx;
    float *topk_w;
    int32_t *slot_count;
    int32_t *slot_offset;
    int32_t *rec_token;
    int32_t *rec_route;
    int32_t *route_pos;
} moe_routes;

/* Opaque host handle of the slot arena and its residency table. */
typedef struct moe_arena moe_arena;

/* Library version string. */
const char *moe_version(void);

/* Copy the calling thread's last error message into buf (NUL-terminated,
 * truncated to n bytes) and return the status of that error (MOE_OK if none). */
moe_status moe_last_error(char *buf, size_t n);

/*
 * Bytes of device workspace the calls need for this shape. The workspace
 * holds the device error word, per-block route counts and ranks, the router
 * logits, the SwiGLU intermediate H [C][f] and the per-route fp32 output rows
 * Yr [S][T*K'][d] (S partial sums over f, see moe_expert_ffn), plus the
 * per-route "computed" marks. One workspace belongs to
 * one layer invocation at a time; it must persist from moe_route_build to
 * the finalizing moe_expert_ffn. Returns 0 for an invalid shape.
 */
size_t moe_workspace_bytes(const moe_shape *shape);

/*
 * Prepare a freshly allocated workspace: clears the device error word (no
 * other region needs initial contents). Call once after allocating `ws`;
 * enqueued on `stream`.
 */
moe_status moe_workspace_init(const moe_shape *shape, void *ws, size_t ws_bytes,
                              moe_stream stream);

/*
 * Synchronize `stream`, read the device error word of `ws`, store it in
 * *errors (may be NULL) and clear it. Returns MOE_OK, or MOE_ERR_INVALID_ARG
 * if bits were set.
 */
moe_status moe_device_errors(const moe_shape *shape, void *ws, size_t ws_bytes,
                             int32_t *errors, moe_stream stream);

/*
 * Router logits, the input of top-k routing (section 2.2).
 *   X      device [T][ldx] dtype
 *   W_r    device [E][d] fp32 (row e holds expert e's weights over the
 *          hidden index: the layout of a linear layer's weight d -> E)
 *   bias   device [E] fp32 or NULL (added after the product)
 *   logits device [T][E] fp32, output
 * Requires X and W_r 16-byte aligned, and for fp32 X ldx % 4 == 0 (bf16 X
 * already needs ldx % 8 == 0; d % 4 == 0 holds for every shape).
 * logits[t][e] = s + bias[e], where s is the fp32 dot product of X[t] and
 * W_r[e] with each term one fused multiply-add, in this order: the hidden
 * index is cut into runs of 8 consecutive values, run r = i / 8 feeds partial
 * sum r % 16, each partial sum is a chain in ascending i starting from 0, and
 * s = ((p0 + p1) + p2) + ... + p15. The pages fix no evaluation order; this
 * one fixes the bits of every logit, so the logits and the top-k decision
 * taken on them are run-to-run reproducible. Each logit is within
 * gamma_n * (sum_i |X[t][i] W_r[e][i]| + |bias[e]|) of the exact value,
 * n = 8 * ceil(d / 128) + 16 roundings, gamma_n = n u / (1 - n u),
 * u = 2^-24 (recursive summation with fused products).
 */
moe_status moe_router_logits(const moe_shape *shape, const void *X,
                             const float *W_r, const float *bias,
                             float *logits, moe_stream stream);

/*
 * Route build for the tokens t0 .. t0+nt-1 (section 3.2, Algorithm 1).
 *   logits  device [T][E] fp32 or NULL. When given, top-k routing runs first
 *           for the token range: ranks by descending logit, equal logits to
 *           the lower expert id (NaN is taken as -infinity); alpha is the
 *           softmax over all E of the selected logits, renormalised over the
 *           k when shape->renorm; shared ranks appended. Results go to
 *           routes->topk_idx / topk_w. When NULL, those arrays must already
 *           hold the routing (written by the caller or an earlier build).
 *   phi     host [E + n_shared] int32, the placement map: phi[e] = slot of
 *           expert e in [0, P), or -1 if not resident; no two experts may
 *           share a slot. Routes of absent experts are left out.
 *   flags   MOE_ROUTE_RESET or 0.
 *   routes  descriptors, see moe_routes. slot_count, slot_offset, rec_* are
 *           rewritten for this build; route_pos is written for the range.
 *   ws      device workspace of at least moe_workspace_bytes(shape) bytes.
 * Requires nt * K' <= capacity (MOE_ERR_CAPACITY otherwise) and
 * 0 <= t0 <= t0 + nt <= T. Records are stable: within a slot they are in
 * ascending route order. Everything is bit-exact and run-to-run identical.
 */
moe_status moe_route_build(const moe_shape *shape, int32_t t0, int32_t nt,
                           const float *logits, const int32_t *phi,
                           int32_t flags, const moe_routes *routes, void *ws,
                           size_t ws_bytes, moe_stream stream);

/*
 * Expert FFN over the routes of the last build, then (optionally) the
 * combine (Eq. 1-2; section 3.2 "Fused Expert Execution").
 *   X      device [T][ldx] dtype, the source activations (gathered by
 *          rec_token)
 *   Y      device [T][ldy] fp32; holds the residual A on entry and
 *          A + sum_j alpha_tj F_e(X_t) after a MOE_FFN_FINALIZE call
 *   arena  slot arena holding the experts named by phi
 *   phi    host [E + n_shared], the same map given to the build. Every slot
 *          it names must hold that expert and be Ready or In-use in the arena
 *          (MOE_ERR_SLOT_STATE otherwise); the stream waits for each such
 *          slot's load, and each slot's release is recorded after the work.
 *   flags  MOE_FFN_EXPERTS and/or MOE_FFN_FINALIZE (and optionally
 *          MOE_FFN_SIMPLE_KERNEL or MOE_FFN_FUSED).
 * MOE_FFN_EXPERTS: for each record p of slot s, H[p] = SiLU(g) * u with
 * (g, u) = X[rec_token[p]] times slot s's gate/up slice, then
 * Yr[rec_route[p]] = alpha * (H[p] times slot s's down slice); the route is
 * marked computed. When the down tiles alone would leave the GPU idle (few
 * routes per expert), the down projection's K = f is split into S equal
 * ranges and each route gets S partial rows (S depends only on the shape).
 * MOE_FFN_FINALIZE: for every token, Y[t] += Yr[t*K'+j] for j = 0..K'-1 in
 * ascending order over the computed routes (each route's partial rows in
 * ascending order). The sum order is fixed, so Y is bitwise run-to-run
 * identical and independent of phi and P.
 * arena and phi may be NULL when only MOE_FFN_FINALIZE is set.
 */
moe_status moe_expert_ffn(const moe_shape *shape, const void *X, float *Y,
                          const moe_routes *routes, moe_arena *arena,
                          const int32_t *phi, int32_t flags, void *ws,
                          size_t ws_bytes, moe_stream stream);

/*
 * Whole layer: router (when W_r is given; else logits must be given),
 * route build, expert FFN and combine.
 *   X, W_r, bias, logits, Y, routes, ws: as above (W_r/bias or logits).
 *   host_gu, host_d: NULL for a resident layer -- every expert must then be
 *     Ready in the arena. Otherwise arrays of E + n_shared host pointers to
 *     each expert's packed gate/up and down slices (as moe_pack_gate_up and
 *     moe_pack_down write them) in pinned memory: the
 *     experts are paged through the arena's banks of G slots on the copy
 *     stream, group by group, overlapped with compute (section 3.4), and
 *     groups with no routes are skipped. Paging synchronizes the compute
 *     stream once, after routing, to read the per-expert route counts.
 * Token ranges are split so that each build fits the capacity.
 */
moe_status moe_layer_prefill(const moe_shape *shape, const void *X,
                             const float *W_r, const float *bias,
                             const float *logits, float *Y, moe_arena *arena,
                             const void *const *host_gu,
                             const void *const *host_d,
                             const moe_routes *routes, void *ws,
                             size_t ws_bytes, moe_stream compute,
                             moe_stream copy);

/*
 * moe_layer_prefill_noalloc -- for callers that cannot allocate memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The resident layer of moe_layer_prefill (host_gu = host_d =
 * NULL, no copy stream), with the same arguments, checks, kernels and
 * results (bit for bit), except that its workspace is a fixed device array
 * inside this library instead of a caller buffer, and it calls no
 * allocating routine (no hipMalloc or hipFree; the arena must already have
 * been loaded, so no event is created either).
 *   Limit: shapes whose moe_workspace_bytes exceeds 64 MiB (67108864 bytes)
 *   are refused with MOE_ERR_WORKSPACE before any GPU work: T <= 815 tokens
 *   for the OLMoE-shaped layer (d = 2048, f = 1024, top-8), T <= 759 for the
 *   DeepSeek-V2-Lite-shaped one, T <= 356 for the Mixtral-shaped one.
 *   Each GPU the library runs on holds its own 64 MiB array until the
 *   process ends. Every call on a GPU uses that GPU's array and finds the
 *   previous call's contents; the device error word is cleared at the start
 *   of each call. Calls that overlap on one GPU (other streams or threads)
 *   race on the array and must be serialized by the caller. Device errors
 *   cannot arise here (routing is computed by the call itself).
 */
moe_status moe_layer_prefill_noalloc(const moe_shape *shape, const void *X,
                                     const float *W_r, const float *bias,
                                     const float *logits, float *Y,
                                     moe_arena *arena,
                                     const moe_routes *routes,
                                     moe_stream stream);

/*
 * Weight packing (section 3.3, "Offline NPU-Consumable Weight Layout":
 * experts are stored in the layout the kernels consume).
 *
 * Tiled slice layout. A slice [N][K] (gate/up: N = 2f, K = d; down: N = d,
 * K = f) is stored in blocks of 256 rows (the last block may be shorter);
 * within a block, K is cut into pieces of 32 elements (the last piece is
 * narrower when K % 32 != 0), stored piece after piece, each piece holding
 * the block's rows one after another. Element (n, k) is at element offset
 *   256*b*K + (k/32)*rows_b*32 + (n%256)*w + k%32,
 * b = n/256, rows_b = min(256, N - 256*b), w = min(32, K - 32*(k/32)).
 * The slice has exactly N*K elements. One K step of a 256-row weight tile is
 * thus one contiguous run (16 KB for bf16), which streams from HBM about 1.5
 * times faster than the same bytes read as 64-byte pieces of 256 rows.
 *
 * Gate/up: expert gate W_g [f][d] and up W_u [f][d] become one [2f][d]
 * slice whose rows alternate in blocks of 32: rows 64q..64q+31 are gate rows
 * 32q..32q+31 and rows 64q+32..64q+63 are up rows 32q..32q+31; that slice is
 * stored tiled. Down: W_d [d][f] stored tiled.
 * moe_pack_gate_up / moe_pack_down: device, n experts (0 <= n <= 65535), source expert stride
 * src_stride and destination stride dst_stride (elements; bytes for
 * MOE_DT_BF16_FP8W, whose source slices are row-major codes followed by one
 * fp32 scale per row, and whose packed slices keep their row scales after
 * the codes, in the packed row order and untiled; bytes for MOE_DT_BF16_FP4W,
 * whose slices are described with that dtype). Sources, destination and
 * strides must be 4-byte aligned (the kernels move 32-bit words); otherwise
 * MOE_ERR_INVALID_ARG.
 * moe_pack_gate_up_host / moe_pack_down_host: the same on host memory, one
 * expert, synchronous.
 */
moe_status moe_pack_gate_up(const moe_shape *shape, const void *W_g,
                            const void *W_u, void *dst, int32_t n,
                            int64_t src_stride, int64_t dst_stride,
                            moe_stream stream);
moe_status moe_pack_gate_up_host(const moe_shape *shape, const void *W_g,
                                 const void *W_u, void *dst);
moe_status moe_pack_down(const moe_shape *shape, const void *W_d, void *dst,
                         int32_t n, int64_t src_stride, int64_t dst_stride,
                         moe_stream stream);
moe_status moe_pack_down_host(const moe_shape *shape, const void *W_d,
                              void *dst);

/*
 * Slot arena (Eq. 3: the slice j of slot s starts at plane_j + s * S_j).
 *   plane_gu  device, P slots of packed gate/up slices (2f*d elements,
 *             tiled layout above), slot stride stride_gu
 *   plane_d   device, P slots of packed down slices (d*f elements, tiled),
 *             slot stride stride_d
 *   (MOE_DT_BF16_FP8W: each slice is its codes then its row scales, and the
 *   strides are in bytes: stride_gu >= 2f*d + 8f, stride_d >= d*f + 4d)
 *   G         slots per bank (1 <= G <= P, P % G == 0); banks are used when
 *             paging (Eq. 4: phi(e) = b*G + r(e))
 * Creates the residency table with every slot Available.
 */
moe_status moe_arena_create(moe_arena **out, const moe_shape *shape,
                            void *plane_gu, void *plane_d, int64_t stride_gu,
                            int64_t stride_d, int32_t G);
void moe_arena_destroy(moe_arena *arena);

/*
 * Load expert `expert` into `slot`: Available/Ready/In-use -> Filling ->
 * Ready. src_gu and src_d (packed slices, as moe_pack_gate_up and
 * moe_pack_down write them) are host (pinned) or device pointers; the copies run on copy_stream after the slot's previous
 * release (if any), and the slot's ready event is recorded after them. The
 * slot's previous mapping is withdrawn first. MOE_ERR_SLOT_STATE if the
 * expert is mapped to another slot or the slot is Filling.
 */
moe_status arena_bind_slot(moe_arena *arena, int32_t slot, int32_t expert,
                           const void *src_gu, const void *src_d,
                           moe_stream copy_stream);

/*
 * Two-phase load for slices the caller writes by other means (e.g.
 * moe_pack_gate_up into the plane), section 3.3: a binding is published only
 * after the slot's gate, up and down slices are populated.
 * arena_reserve_slot: Available/Ready/In-use -> Filling for `expert` (the
 * slot's previous mapping is withdrawn; MOE_ERR_SLOT_STATE if the slot is
 * already Filling or the expert occupies another slot). While Filling, the
 * slot is in no placement map, a moe_expert_ffn whose phi names it fails
 * with MOE_ERR_SLOT_STATE, and arena_bind_slot into it fails likewise. The
 * caller must order its writes after the slot's last release itself (the
 * library's own loads wait for it; writes issued by the caller do not).
 * arena_publish_slot: Filling (reserved for `expert`) -> Ready; the ready
 * event is recorded on `stream` after the caller's writes enqueued there. A
 * slot that was not reserved is reserved and published in one step.
 */
moe_status arena_reserve_slot(moe_arena *arena, int32_t slot, int32_t expert);
moe_status arena_publish_slot(moe_arena *arena, int32_t slot, int32_t expert,
                              moe_stream stream);

/* Withdraw a slot's mapping (Ready or In-use -> Available). A later bind of
 * the slot still waits for its last release. */
moe_status arena_release_slot(moe_arena *arena, int32_t slot);

/* The current placement map over Ready and In-use slots: phi[e] = slot or
 * -1, for e < n (n >= E + n_shared). */
moe_status arena_phi(const moe_arena *arena, int32_t *phi, int32_t n);

/* State (MOE_SLOT_*) and owner expert (-1 if none) of one slot. */
moe_status arena_slot_info(const moe_arena *arena, int32_t slot,
                           int32_t *state, int32_t *expert);

/*
 * Diagnostics: run one v_mfma_f32_32x32x16_bf16 on integer-valued operands
 * laid out as the expert kernels assume and write the 32x32 product, row
 * major, to out (device, 1024 floats). The product equals A*B (A[i][k] =
 * (3i + 5k) % 7 - 3, B[k][j] = (2k + 7j) % 5 - 2) exactly iff the kernels'
 * lane layout is the hardware's.
 */
moe_status moe_selftest_mfma_layout(float *out, moe_stream stream);

/*
 * Per-kernel timing. Kernel ids of the layer's launches: */
#define MOE_KERNEL_ROUTER 1
#define MOE_KERNEL_TOPK 2
#define MOE_KERNEL_ROUTE_COUNT 3
#define MOE_KERNEL_ROUTE_PLACE 4
#define MOE_KERNEL_GATE_UP 5
#define MOE_KERNEL_DOWN 6
#define MOE_KERNEL_COMBINE 7
#define MOE_KERNEL_H2D 8        /* the two host-to-device copies of one bind */
#define MOE_KERNEL_FUSED 9      /* the fused expert kernel (MOE_FFN_FUSED) */
#define MOE_KERNEL_COUNT 10
/* moe_profile_begin arms timing of one kernel id for the next max_launches
 * launches (process-wide): each such launch is bracketed by a pair of HIP
 * events recorded on the launch's stream. moe_profile_end waits for those
 * events, writes up to n per-launch durations in milliseconds to ms (host),
 * stores the number of timed launches in *recorded and disarms. */
moe_status moe_profile_begin(int32_t kernel, int32_t max_launches);
moe_status moe_profile_end(int32_t kernel, float *ms, int32_t n,
                           int32_t *recorded);

#ifdef __cplusplus
}
#endif
#endif /* ROUTED_EXPERT_FFN_MOE_H */
