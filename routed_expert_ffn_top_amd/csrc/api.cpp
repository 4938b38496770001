// C ABI of the routed-expert MoE layer library: argument checks, the slot
// arena with its residency table, and the order of kernel launches.
//
// Residency table (EStream, section 3.3, "Bounded Parameter Arena and Safe
// Slot Reuse"): residency.h holds the states and the stream-ordered events
// that carry the protocol; here it runs on HIP streams and events. "ready" is
// recorded on the copy stream after a slot's slices are copied, and every
// invocation that reads the slot waits for it; "release" is recorded on the
// compute stream after the last invocation that reads the slot, and a later
// load into the slot waits for it. So no invocation sees a partly loaded
// expert, and no load overwrites a slot that queued work still reads,
// without any host wait.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <vector>

#include "common.h"
#include "residency.h"

using namespace moe;

namespace {

thread_local moe_status g_status = MOE_OK;
thread_local char g_msg[512] = {0};

moe_status fail(moe_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_msg, sizeof g_msg, fmt, ap);
    va_end(ap);
    g_status = st;
    return st;
}

moe_status hip_fail(hipError_t e, const char *what)
{
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                        \
    do {                                           \
        hipError_t _e = (expr);                    \
        if (_e != hipSuccess) return hip_fail(_e, what); \
    } while (0)

#define MOE_TRY(expr)                  \
    do {                               \
        moe_status _s = (expr);        \
        if (_s != MOE_OK) return _s;   \
    } while (0)

inline hipStream_t S(moe_stream s) { return (hipStream_t)s; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_shape(const moe_shape *s)
{
    if (!s) return fail(MOE_ERR_INVALID_ARG, "shape is NULL");
    if (s->T < 0 || s->d <= 0 || s->f <= 0)
        return fail(MOE_ERR_INVALID_ARG, "bad sizes T=%d d=%d f=%d", s->T, s->d, s->f);
    if (s->E < 1 || s->E > 256 || s->k < 1 || s->k > s->E)
        return fail(MOE_ERR_INVALID_ARG, "need 1 <= k <= E <= 256 (E=%d k=%d)", s->E, s->k);
    if (s->n_shared < 0 || s->E + s->n_shared > kMaxExp)
        return fail(MOE_ERR_INVALID_ARG, "E + n_shared must be <= %d", kMaxExp);
    if (s->k + s->n_shared > 64) return fail(MOE_ERR_UNSUPPORTED, "k + n_shared must be <= 64");
    if (s->P < 1 || s->P > kMaxExp) return fail(MOE_ERR_INVALID_ARG, "need 1 <= P <= %d", kMaxExp);
    if (s->capacity < 1) return fail(MOE_ERR_INVALID_ARG, "capacity must be >= 1");
    if (s->dtype != MOE_DT_BF16 && s->dtype != MOE_DT_F32 && s->dtype != MOE_DT_BF16_FP8W &&
        s->dtype != MOE_DT_BF16_FP4W)
        return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_DT_BF16, MOE_DT_BF16_FP8W, MOE_DT_BF16_FP4W or MOE_DT_F32");
    if (s->ldx < s->d || s->ldy < s->d || (s->ldy % 4) != 0)
        return fail(MOE_ERR_INVALID_ARG, "need ldx >= d, ldy >= d, ldy %% 4 == 0");
    if ((s->d % 4) != 0) return fail(MOE_ERR_UNSUPPORTED, "d must be a multiple of 4");
    if (act_bf16(*s)) {
        if ((s->d % 64) != 0 || (s->f % 64) != 0)
            return fail(MOE_ERR_UNSUPPORTED, "bf16 layers need d %% 64 == 0 and f %% 64 == 0");
        if ((s->ldx % 8) != 0) return fail(MOE_ERR_UNSUPPORTED, "bf16 X needs ldx %% 8 == 0");
    } else if ((s->f % 32) != 0) {
        return fail(MOE_ERR_UNSUPPORTED, "fp32 layers need f %% 32 == 0");
    }
    const int64_t routes = (int64_t)s->T * (s->k + s->n_shared);
    if (routes > INT32_MAX / 2 || (int64_t)s->capacity * s->f > (int64_t)1 << 40)
        return fail(MOE_ERR_UNSUPPORTED, "too many routes");
    // the combine launches one workgroup per token and 1024 columns, on the
    // grid's x dimension (at most 2^31 - 1 workgroups)
    if ((int64_t)s->T * ((s->d / 4 + 255) / 256) > INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "T * ceil(d / 1024) must be below 2^31");
    return MOE_OK;
}

moe_status check_ws(const moe_shape *s, void *ws, size_t ws_bytes, WsLayout *w)
{
    *w = ws_layout(*s);
    if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
    if (!aligned(ws, 256)) return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < w->total)
        return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, w->total);
    return MOE_OK;
}

moe_status check_routes(const moe_routes *r)
{
    if (!r || !r->topk_idx || !r->topk_w || !r->slot_count || !r->slot_offset || !r->rec_token ||
        !r->rec_route || !r->route_pos)
        return fail(MOE_ERR_INVALID_ARG, "route descriptor pointer is NULL");
    return MOE_OK;
}

moe_status check_phi(const moe_shape *s, const int32_t *phi, PhiArg *out)
{
    if (!phi) return fail(MOE_ERR_INVALID_ARG, "phi is NULL");
    const int ne = s->E + s->n_shared;
    int used[kMaxExp];   // on the stack: the allocation-free entry point runs this too
    for (int q = 0; q < s->P; ++q) used[q] = -1;
    for (int e = 0; e < ne; ++e) {
        const int v = phi[e];
        if (v < -1 || v >= s->P) return fail(MOE_ERR_INVALID_ARG, "phi[%d] = %d outside [-1, P)", e, v);
        if (v >= 0) {
            if (used[v] >= 0)
                return fail(MOE_ERR_INVALID_ARG, "phi maps experts %d and %d to slot %d", used[v], e, v);
            used[v] = e;
        }
        out->v[e] = v;
    }
    for (int e = ne; e < kMaxExp; ++e) out->v[e] = -1;
    return MOE_OK;
}

template <typename T>
T *ws_at(void *ws, size_t off) { return (T *)((char *)ws + off); }

// The router reads X and W_r rows in 16-byte pieces.
moe_status check_router_args(const moe_shape *s, const void *X, const float *W_r)
{
    if (!aligned(X, 16) || !aligned(W_r, 16))
        return fail(MOE_ERR_INVALID_ARG, "router: X and W_r must be 16-byte aligned");
    if (s->dtype == MOE_DT_F32 && (s->ldx % 4) != 0)
        return fail(MOE_ERR_UNSUPPORTED, "router: fp32 X needs ldx %% 4 == 0");
    return MOE_OK;
}

// Per-kernel launch timing (moe_profile_begin / moe_profile_end).
struct KernelTimer {
    std::vector<hipEvent_t> start, stop;
    int armed = 0, next = 0;
};
std::mutex g_prof_mu;
KernelTimer g_prof[MOE_KERNEL_COUNT];

// Records the start event of the next timed launch of `kid`; returns the
// slot index or -1. Cheap when nothing is armed.
int prof_begin(int kid, hipStream_t st)
{
    KernelTimer &k = g_prof[kid];
    if (!k.armed) return -1;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (k.next >= (int)k.start.size()) return -1;
    const int i = k.next++;
    (void)hipEventRecord(k.start[i], st);
    return i;
}

void prof_end(int kid, int i, hipStream_t st)
{
    if (i >= 0) (void)hipEventRecord(g_prof[kid].stop[i], st);
}

#define TIMED(kid, st, expr)                 \
    ([&]() {                                 \
        const int _pi = prof_begin(kid, st); \
        hipError_t _r = (expr);              \
        prof_end(kid, _pi, st);              \
        return _r;                           \
    }())

}  // namespace

// ---------------------------------------------------------------------------
// arena

namespace {

// Streams and events of the residency table: HIP's.
struct HipBackend {
    using Stream = hipStream_t;
    using Event = hipEvent_t;
    hipError_t last = hipSuccess;
    int create(Event *e) { return (last = hipEventCreateWithFlags(e, hipEventDisableTiming)) != hipSuccess; }
    void destroy(Event e) { (void)hipEventDestroy(e); }
    int record(Event e, Stream s) { return (last = hipEventRecord(e, s)) != hipSuccess; }
    int wait(Stream s, Event e) { return (last = hipStreamWaitEvent(s, e, 0)) != hipSuccess; }
    int sync(Event e) { return (last = hipEventSynchronize(e)) != hipSuccess; }
};

}  // namespace

struct moe_arena {
    mutable std::mutex mu;   // guards the residency table
    moe_shape shape;
    char *plane_gu;
    char *plane_d;
    int64_t stride_gu, stride_d;  // elements (bytes for quantised weights)
    int G;
    int esz;
    HipBackend bk;
    ResidencyTable<HipBackend> res;
    moe_arena(const moe_shape &s) : shape(s), res(bk, s.P, s.E + s.n_shared) {}
};

namespace {

// Reports an error of the residency table through the library's error
// channel (errors raised by the caller's own code have already been).
moe_status R(moe_arena *a, moe_status st)
{
    if (st != MOE_OK && a->res.msg()[0]) {
        if (st == MOE_ERR_HIP)
            fail(st, "%s: %s", a->res.msg(), hipGetErrorString(a->bk.last));
        else
            fail(st, "%s", a->res.msg());
        a->res.clear_msg();
    }
    return st;
}

// Binds expert ex[i] to slot sl[i] for i < n, with loads on `st` (see
// ResidencyTable::load). Neighbouring entries whose slots are consecutive
// and whose prepacked host slices follow each other in memory are copied
// with one transfer per plane. With `timed`, the copies (not the waits) are
// bracketed for moe_profile_begin(MOE_KERNEL_H2D). Caller holds the lock.
moe_status arena_bind_many_locked(moe_arena *a, const int *sl, const int *ex, int n, const void *const *src_gu,
                                  const void *const *src_d, hipStream_t st, bool timed)
{
    const moe_shape &s = a->shape;
    const size_t gu_bytes = gu_slice_bytes(s), d_bytes = d_slice_bytes(s);
    // one transfer may cover several slots only where the plane holds the
    // slices back to back
    const bool packed_planes = (size_t)a->stride_gu * a->esz == gu_bytes && (size_t)a->stride_d * a->esz == d_bytes;
    for (int i = 0; i < n; ++i)
        if (!src_gu[i] || !src_d[i]) return fail(MOE_ERR_INVALID_ARG, "bind source is NULL");
    auto write = [&](hipStream_t cs) -> moe_status {
        const int pi = timed ? prof_begin(MOE_KERNEL_H2D, cs) : -1;
        hipError_t e = hipSuccess;
        for (int i = 0; i < n && e == hipSuccess;) {
            int j = i + 1;   // extend while slots are consecutive and host slices contiguous
            while (packed_planes && j < n && sl[j] == sl[j - 1] + 1 &&
                   (const char *)src_gu[j] == (const char *)src_gu[j - 1] + gu_bytes &&
                   (const char *)src_d[j] == (const char *)src_d[j - 1] + d_bytes)
                ++j;
            e = hipMemcpyAsync(a->plane_gu + (size_t)sl[i] * a->stride_gu * a->esz, src_gu[i],
                               gu_bytes * (size_t)(j - i), hipMemcpyDefault, cs);
            if (e == hipSuccess)
                e = hipMemcpyAsync(a->plane_d + (size_t)sl[i] * a->stride_d * a->esz, src_d[i],
                                   d_bytes * (size_t)(j - i), hipMemcpyDefault, cs);
            i = j;
        }
        if (pi >= 0) prof_end(MOE_KERNEL_H2D, pi, cs);
        return e == hipSuccess ? MOE_OK : hip_fail(e, "arena bind copy");
    };
    return R(a, a->res.load(sl, ex, n, st, write));
}

moe_status arena_bind_locked(moe_arena *a, int slot, int expert, const void *src_gu, const void *src_d,
                             hipStream_t st)
{
    return arena_bind_many_locked(a, &slot, &expert, 1, &src_gu, &src_d, st, true);
}

// Checks phi against the arena, makes `st` wait for each named slot's load.
moe_status arena_acquire(moe_arena *a, const int32_t *phi, hipStream_t st)
{
    return R(a, a->res.acquire(phi, st));
}

moe_status arena_release_after(moe_arena *a, const int32_t *phi, hipStream_t st)
{
    return R(a, a->res.release_after(phi, st));
}

// ---------------------------------------------------------------------------
// internal steps (arguments already checked)

moe_status route_build_impl(const moe_shape &s, const WsLayout &w, int t0, int nt, const float *logits,
                            const PhiArg &phi, int flags, const moe_routes &r, void *ws, hipStream_t st)
{
    const int kp = s.k + s.n_shared;
    int32_t *done = ws_at<int32_t>(ws, w.done);
    int reset = (flags & MOE_ROUTE_RESET) ? 1 : 0;
    if (logits) {
        HIP_TRY(TIMED(MOE_KERNEL_TOPK, st, launch_topk(s, t0, nt, logits, r.topk_idx, r.topk_w, done, st)),
                "top-k launch");
        reset = 0;  // top-k cleared the marks of the range
    }
    const int64_t i0 = (int64_t)t0 * kp, n = (int64_t)nt * kp;
    int32_t *blk = ws_at<int32_t>(ws, w.blk);
    int32_t *rank = ws_at<int32_t>(ws, w.rank);
    int32_t *err = ws_at<int32_t>(ws, w.err);
    HIP_TRY(TIMED(MOE_KERNEL_ROUTE_COUNT, st,
                  launch_route_count(s, i0, n, r.topk_idx, phi, blk, rank, err, done, reset, st)),
            "route count launch");
    HIP_TRY(TIMED(MOE_KERNEL_ROUTE_PLACE, st,
                  launch_route_place(s, i0, n, r.topk_idx, phi, blk, rank, r.rec_token, r.rec_route,
                                     r.route_pos, r.slot_count, r.slot_offset, st)),
            "route place launch");
    return MOE_OK;
}

GemmArgs gemm_args(const moe_shape &s, const moe_routes &r, const moe_arena *a)
{
    GemmArgs g{};
    g.slot_offset = r.slot_offset;
    g.P = s.P;
    g.rec_token = r.rec_token;
    g.rec_route = r.rec_route;
    g.topk_w = r.topk_w;
    g.splits = 1;
    (void)a;
    return g;
}

moe_status experts_impl(const moe_shape &s, const WsLayout &w, const void *X, const moe_routes &r,
                        moe_arena *a, int max_rows, bool simple, void *ws, hipStream_t st, bool fused = false)
{
    if (simple && (w_fp8(s) || w_fp4(s)))
        return fail(MOE_ERR_UNSUPPORTED, "the plain kernel reads bf16 or fp32 weights only");
    if (fused && (simple || !fused_expert_supported(s)))
        return fail(MOE_ERR_UNSUPPORTED, "the fused expert kernel needs bf16 weights, f <= 1024, d %% 128 == 0 "
                                         "and an unsplit down projection");
    GemmArgs g = gemm_args(s, r, a);
    g.A = X;
    g.lda = s.ldx;
    g.B = a->plane_gu;
    g.slot_stride = a->stride_gu;
    g.bfp8 = w_fp8(s);
    g.bfp4 = w_fp4(s);
    g.scale_off = (int64_t)2 * s.f * s.d;   // fp8: the row scales follow the codes
    g.N = 2 * s.f;
    g.K = s.d;
    g.C = ws_at<char>(ws, w.H);
    g.ldc = s.f;
    if (!fused) HIP_TRY(TIMED(MOE_KERNEL_GATE_UP, st, launch_gate_up(s, g, max_rows, simple, st)), "gate/up launch");
    GemmArgs h = gemm_args(s, r, a);
    h.A = ws_at<char>(ws, w.H);
    h.lda = s.f;
    h.B = a->plane_d;
    h.slot_stride = a->stride_d;
    h.bfp8 = w_fp8(s);
    h.bfp4 = w_fp4(s);
    h.scale_off = (int64_t)s.d * s.f;
    h.N = s.d;
    h.K = s.f;
    h.C = ws_at<float>(ws, w.Yr);
    h.ldc = s.d;
    h.done = ws_at<int32_t>(ws, w.done);
    h.splits = down_splits(s);
    h.split_stride = (int64_t)s.T * (s.k + s.n_shared) * s.d;
    if (fused) {
        HIP_TRY(TIMED(MOE_KERNEL_FUSED, st, launch_fused_expert(s, g, h, max_rows, st)), "fused expert launch");
        return MOE_OK;
    }
    HIP_TRY(TIMED(MOE_KERNEL_DOWN, st, launch_down(s, h, max_rows, simple, st)), "down launch");
    return MOE_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI

extern "C" {

const char *moe_version(void) { return "routed-expert-ffn-gfx950 0.1"; }

moe_status moe_last_error(char *buf, size_t n)
{
    if (buf && n) {
        strncpy(buf, g_msg, n - 1);
        buf[n - 1] = 0;
    }
    return g_status;
}

size_t moe_workspace_bytes(const moe_shape *shape)
{
    if (check_shape(shape) != MOE_OK) return 0;
    return ws_layout(*shape).total;
}

moe_status moe_workspace_init(const moe_shape *shape, void *ws, size_t ws_bytes, moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    WsLayout w;
    MOE_TRY(check_ws(shape, ws, ws_bytes, &w));
    HIP_TRY(launch_fill_i32(ws_at<int32_t>(ws, w.err), 0, 64, S(stream)), "fill launch");
    return MOE_OK;
}

moe_status moe_device_errors(const moe_shape *shape, void *ws, size_t ws_bytes, int32_t *errors,
                             moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    WsLayout w;
    MOE_TRY(check_ws(shape, ws, ws_bytes, &w));
    int32_t v = 0;
    HIP_TRY(hipStreamSynchronize(S(stream)), "hipStreamSynchronize");
    HIP_TRY(hipMemcpy(&v, ws_at<int32_t>(ws, w.err), 4, hipMemcpyDeviceToHost), "hipMemcpy");
    if (v) HIP_TRY(hipMemset(ws_at<int32_t>(ws, w.err), 0, 4), "hipMemset");
    if (errors) *errors = v;
    if (v) return fail(MOE_ERR_INVALID_ARG, "device error word 0x%x (bit 0: expert id out of range)", v);
    return MOE_OK;
}

moe_status moe_router_logits(const moe_shape *shape, const void *X, const float *W_r, const float *bias,
                             float *logits, moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    if (!X || !W_r || !logits) return fail(MOE_ERR_INVALID_ARG, "router: NULL pointer");
    MOE_TRY(check_router_args(shape, X, W_r));
    HIP_TRY(TIMED(MOE_KERNEL_ROUTER, S(stream), launch_router_logits(*shape, X, W_r, bias, logits, S(stream))),
            "router launch");
    return MOE_OK;
}

moe_status moe_route_build(const moe_shape *shape, int32_t t0, int32_t nt, const float *logits,
                           const int32_t *phi, int32_t flags, const moe_routes *routes, void *ws,
                           size_t ws_bytes, moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    if (shape->T == 0) return MOE_OK;  // an empty prompt: nothing to do
    MOE_TRY(check_routes(routes));
    WsLayout w;
    MOE_TRY(check_ws(shape, ws, ws_bytes, &w));
    if (t0 < 0 || nt < 0 || (int64_t)t0 + nt > shape->T)
        return fail(MOE_ERR_INVALID_ARG, "token range [%d, %d) outside [0, %d)", t0, t0 + nt, shape->T);
    const int64_t kp = shape->k + shape->n_shared;
    if ((int64_t)nt * kp > shape->capacity)
        return fail(MOE_ERR_CAPACITY, "%lld routes exceed capacity %d", (long long)nt * kp, shape->capacity);
    PhiArg pa;
    MOE_TRY(check_phi(shape, phi, &pa));
    return route_build_impl(*shape, w, t0, nt, logits, pa, flags, *routes, ws, S(stream));
}

moe_status moe_expert_ffn(const moe_shape *shape, const void *X, float *Y, const moe_routes *routes,
                          moe_arena *arena, const int32_t *phi, int32_t flags, void *ws, size_t ws_bytes,
                          moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    if (shape->T == 0) return MOE_OK;  // an empty prompt: nothing to do
    MOE_TRY(check_routes(routes));
    WsLayout w;
    MOE_TRY(check_ws(shape, ws, ws_bytes, &w));
    if (flags & MOE_FFN_EXPERTS) {
        if (!X || !arena || !phi) return fail(MOE_ERR_INVALID_ARG, "expert FFN: X, arena and phi are required");
        if (arena->shape.d != shape->d || arena->shape.f != shape->f || arena->shape.P != shape->P ||
            arena->shape.dtype != shape->dtype || arena->shape.E != shape->E ||
            arena->shape.n_shared != shape->n_shared)
            return fail(MOE_ERR_INVALID_ARG, "arena was made for another shape");
        if (act_bf16(*shape) && !aligned(X, 16))
            return fail(MOE_ERR_INVALID_ARG, "X must be 16-byte aligned");
        PhiArg pa;
        MOE_TRY(check_phi(shape, phi, &pa));
        std::lock_guard<std::mutex> lk(arena->mu);
        MOE_TRY(arena_acquire(arena, phi, S(stream)));
        const int max_rows = std::min<int64_t>(shape->capacity, (int64_t)shape->T * (shape->k + shape->n_shared));
        MOE_TRY(experts_impl(*shape, w, X, *routes, arena, max_rows, (flags & MOE_FFN_SIMPLE_KERNEL) != 0, ws,
                             S(stream), (flags & MOE_FFN_FUSED) != 0));
        MOE_TRY(arena_release_after(arena, phi, S(stream)));
    }
    if (flags & MOE_FFN_FINALIZE) {
        if (!Y || !aligned(Y, 16)) return fail(MOE_ERR_INVALID_ARG, "Y must be non-NULL and 16-byte aligned");
        HIP_TRY(TIMED(MOE_KERNEL_COMBINE, S(stream),
                      launch_combine(*shape, Y, ws_at<float>(ws, w.Yr), ws_at<int32_t>(ws, w.done), S(stream))),
                "combine launch");
    }
    return MOE_OK;
}

moe_status moe_pack_gate_up(const moe_shape *shape, const void *W_g, const void *W_u, void *dst, int32_t n,
                            int64_t src_stride, int64_t dst_stride, moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    if (!W_g || !W_u || !dst || n < 0 || n > 65535) return fail(MOE_ERR_INVALID_ARG, "pack: bad arguments");
    const int esz = w_esz(*shape);
    const size_t src_bytes = src_slice_bytes(*shape, shape->f, shape->d);
    if (n > 1 && ((size_t)src_stride * esz < src_bytes || (size_t)dst_stride * esz < gu_slice_bytes(*shape)))
        return fail(MOE_ERR_INVALID_ARG, "pack: strides smaller than a slice");
    if (((src_stride * esz) % 4) != 0 || ((dst_stride * esz) % 4) != 0)
        return fail(MOE_ERR_INVALID_ARG, "pack: strides must be whole 32-bit words");
    if (!aligned(W_g, 4) || !aligned(W_u, 4) || !aligned(dst, 4))
        return fail(MOE_ERR_INVALID_ARG, "pack: sources and destination must be 4-byte aligned");
    HIP_TRY(launch_pack_gate_up(*shape, W_g, W_u, dst, n, src_stride, dst_stride, S(stream)), "pack launch");
    return MOE_OK;
}

// MXFP4: source row sr of a source slice with Nsrc rows (codes [Nsrc][K/2],
// then scales [Nsrc][K/32]) into row r of the packed [N][K] slice at dst.
static void fp4_pack_row_host(const uint8_t *src, int64_t Nsrc, int64_t sr, uint8_t *dst, int64_t N, int64_t K,
                              int64_t r)
{
    const int64_t b = r / kWRows, rb = r % kWRows, rows = std::min<int64_t>(kWRows, N - b * kWRows);
    uint8_t *base = dst + b * (K / kWK) * fp4_piece_bytes(kWRows);
    const uint8_t *codes = src + sr * (K / 2), *sc = src + Nsrc * (K / 2) + sr * (K / kWK);
    for (int64_t p = 0; p < K / kWK; ++p) {
        uint8_t *piece = base + p * fp4_piece_bytes(rows);
        memcpy(piece + rb * 16, codes + p * 16, 16);
        piece[rows * 16 + rb] = sc[p];
        if (rb == rows - 1) memset(piece + rows * 17, 0, (size_t)(fp4_piece_bytes(rows) - rows * 17));
    }
}

moe_status moe_pack_gate_up_host(const moe_shape *shape, const void *W_g, const void *W_u, void *dst)
{
    MOE_TRY(check_shape(shape));
    if (!W_g || !W_u || !dst) return fail(MOE_ERR_INVALID_ARG, "pack: NULL pointer");
    if (w_fp4(*shape)) {
        const int f = shape->f;
        for (int r = 0; r < 2 * f; ++r) {
            const int q = r / 64, w = r % 64;
            const int sr = w < 32 ? 32 * q + w : 32 * q + w - 32;
            fp4_pack_row_host((const uint8_t *)(w < 32 ? W_g : W_u), f, sr, (uint8_t *)dst, 2 * f, shape->d, r);
        }
        return MOE_OK;
    }
    const size_t esz = (size_t)w_esz(*shape);
    const size_t row = (size_t)shape->d * esz;
    const int f = shape->f, d = shape->d;
    for (int r = 0; r < 2 * f; ++r) {
        const int q = r / 64, w = r % 64;
        const int sr = w < 32 ? 32 * q + w : 32 * q + w - 32;   // source row of gate (w < 32) or up
        const char *src = (const char *)(w < 32 ? W_g : W_u) + (size_t)sr * row;
        for (int k = 0; k < d; ++k)   // element (r, k) of the tiled [2f][d] slice
            memcpy((char *)dst + (size_t)wtile_off(r, k, 2 * f, d) * esz, src + (size_t)k * esz, esz);
        if (w_fp8(*shape))   // row scales follow the codes, in the packed row order
            memcpy((char *)dst + (size_t)2 * f * row + (size_t)r * 4,
                   (const char *)(w < 32 ? W_g : W_u) + (size_t)f * row + (size_t)sr * 4, 4);
    }
    return MOE_OK;
}

moe_status moe_pack_down(const moe_shape *shape, const void *W_d, void *dst, int32_t n, int64_t src_stride,
                         int64_t dst_stride, moe_stream stream)
{
    MOE_TRY(check_shape(shape));
    if (!W_d || !dst || n < 0 || n > 65535) return fail(MOE_ERR_INVALID_ARG, "pack: bad arguments");
    const int esz = w_esz(*shape);
    if (n > 1 && ((size_t)src_stride * esz < src_slice_bytes(*shape, shape->d, shape->f) ||
                  (size_t)dst_stride * esz < d_slice_bytes(*shape)))
        return fail(MOE_ERR_INVALID_ARG, "pack: strides smaller than a slice");
    if (((src_stride * esz) % 4) != 0 || ((dst_stride * esz) % 4) != 0)
        return fail(MOE_ERR_INVALID_ARG, "pack: strides must be whole 32-bit words");
    if (!aligned(W_d, 4) || !aligned(dst, 4))
        return fail(MOE_ERR_INVALID_ARG, "pack: sources and destination must be 4-byte aligned");
    HIP_TRY(launch_pack_down(*shape, W_d, dst, n, src_stride, dst_stride, S(stream)), "pack launch");
    return MOE_OK;
}

moe_status moe_pack_down_host(const moe_shape *shape, const void *W_d, void *dst)
{
    MOE_TRY(check_shape(shape));
    if (!W_d || !dst) return fail(MOE_ERR_INVALID_ARG, "pack: NULL pointer");
    if (w_fp4(*shape)) {
        for (int m = 0; m < shape->d; ++m)
            fp4_pack_row_host((const uint8_t *)W_d, shape->d, m, (uint8_t *)dst, shape->d, shape->f, m);
        return MOE_OK;
    }
    const size_t esz = (size_t)w_esz(*shape);
    const int d = shape->d, f = shape->f;
    for (int m = 0; m < d; ++m)
        for (int k = 0; k < f; ++k)   // element (m, k) of the tiled [d][f] slice
            memcpy((char *)dst + (size_t)wtile_off(m, k, d, f) * esz,
                   (const char *)W_d + ((size_t)m * f + k) * esz, esz);
    if (w_fp8(*shape))   // the [d] row scales follow the codes unchanged
        memcpy((char *)dst + (size_t)d * f, (const char *)W_d + (size_t)d * f, (size_t)d * 4);
    return MOE_OK;
}

moe_status moe_arena_create(moe_arena **out, const moe_shape *shape, void *plane_gu, void *plane_d,
                            int64_t stride_gu, int64_t stride_d, int32_t G)
{
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    MOE_TRY(check_shape(shape));
    if (!plane_gu || !plane_d) return fail(MOE_ERR_INVALID_ARG, "plane is NULL");
    const int esz = w_esz(*shape);
    if ((size_t)stride_gu * esz < gu_slice_bytes(*shape) || (size_t)stride_d * esz < d_slice_bytes(*shape))
        return fail(MOE_ERR_INVALID_ARG, "slot strides smaller than the slices");
    if (G < 1 || G > shape->P || shape->P % G != 0)
        return fail(MOE_ERR_INVALID_ARG, "need 1 <= G <= P and P %% G == 0");
    if (!aligned(plane_gu, 16) || !aligned(plane_d, 16) || (stride_gu * esz) % 16 || (stride_d * esz) % 16)
        return fail(MOE_ERR_INVALID_ARG, "planes and slot strides must be 16-byte aligned");
    moe_arena *a = new moe_arena(*shape);
    a->plane_gu = (char *)plane_gu;
    a->plane_d = (char *)plane_d;
    a->stride_gu = stride_gu;
    a->stride_d = stride_d;
    a->G = G;
    a->esz = esz;
    *out = a;
    return MOE_OK;
}

void moe_arena_destroy(moe_arena *a)
{
    delete a;   // the residency table destroys its events
}

moe_status arena_bind_slot(moe_arena *a, int32_t slot, int32_t expert, const void *src_gu, const void *src_d,
                           moe_stream copy_stream)
{
    if (!a) return fail(MOE_ERR_INVALID_ARG, "arena is NULL");
    std::lock_guard<std::mutex> lk(a->mu);
    return arena_bind_locked(a, slot, expert, src_gu, src_d, S(copy_stream));
}

moe_status arena_reserve_slot(moe_arena *a, int32_t slot, int32_t expert)
{
    if (!a) return fail(MOE_ERR_INVALID_ARG, "arena is NULL");
    std::lock_guard<std::mutex> lk(a->mu);
    return R(a, a->res.reserve(slot, expert));
}

moe_status arena_publish_slot(moe_arena *a, int32_t slot, int32_t expert, moe_stream stream)
{
    if (!a) return fail(MOE_ERR_INVALID_ARG, "arena is NULL");
    std::lock_guard<std::mutex> lk(a->mu);
    return R(a, a->res.publish(slot, expert, S(stream)));
}

moe_status arena_release_slot(moe_arena *a, int32_t slot)
{
    if (!a) return fail(MOE_ERR_INVALID_ARG, "arena is NULL");
    std::lock_guard<std::mutex> lk(a->mu);
    return R(a, a->res.release(slot));
}

moe_status arena_phi(const moe_arena *a, int32_t *phi, int32_t n)
{
    if (!a || !phi) return fail(MOE_ERR_INVALID_ARG, "NULL argument");
    const int ne = a->shape.E + a->shape.n_shared;
    if (n < ne) return fail(MOE_ERR_INVALID_ARG, "phi needs %d entries", ne);
    std::lock_guard<std::mutex> lk(a->mu);
    a->res.placement(phi, n);
    return MOE_OK;
}

moe_status arena_slot_info(const moe_arena *a, int32_t slot, int32_t *state, int32_t *expert)
{
    if (!a) return fail(MOE_ERR_INVALID_ARG, "arena is NULL");
    if (slot < 0 || slot >= a->shape.P) return fail(MOE_ERR_INVALID_ARG, "slot %d outside [0, P)", slot);
    std::lock_guard<std::mutex> lk(a->mu);
    if (state) *state = a->res.state(slot);
    if (expert) *expert = a->res.owner(slot);
    return MOE_OK;
}

moe_status moe_profile_begin(int32_t kernel, int32_t max_launches)
{
    if (kernel <= 0 || kernel >= MOE_KERNEL_COUNT || max_launches < 1 || max_launches > 100000)
        return fail(MOE_ERR_INVALID_ARG, "profile: bad kernel id or count");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    KernelTimer &k = g_prof[kernel];
    while ((int)k.start.size() < max_launches) {
        hipEvent_t a, b;
        HIP_TRY(hipEventCreate(&a), "hipEventCreate");
        HIP_TRY(hipEventCreate(&b), "hipEventCreate");
        k.start.push_back(a);
        k.stop.push_back(b);
    }
    k.next = 0;
    k.armed = 1;
    return MOE_OK;
}

moe_status moe_profile_end(int32_t kernel, float *ms, int32_t n, int32_t *recorded)
{
    if (kernel <= 0 || kernel >= MOE_KERNEL_COUNT) return fail(MOE_ERR_INVALID_ARG, "profile: bad kernel id");
    std::lock_guard<std::mutex> lk(g_prof_mu);
    KernelTimer &k = g_prof[kernel];
    k.armed = 0;
    if (recorded) *recorded = k.next;
    for (int i = 0; i < k.next && i < n && ms; ++i) {
        HIP_TRY(hipEventSynchronize(k.stop[i]), "hipEventSynchronize");
        HIP_TRY(hipEventElapsedTime(&ms[i], k.start[i], k.stop[i]), "hipEventElapsedTime");
    }
    k.next = 0;
    return MOE_OK;
}

moe_status moe_selftest_mfma_layout(float *out, moe_stream stream)
{
    if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
    HIP_TRY(launch_selftest_mfma(out, S(stream)), "self-test launch");
    return MOE_OK;
}

}  // extern "C"

namespace moe {

moe_status report_error(moe_status st, const char *msg) { return fail(st, "%s", msg); }

// Checks shared by the layer calls; on success *w is the workspace layout.
static moe_status layer_checks(const moe_shape *shape, const void *X, const float *W_r, const float *logits,
                               float *Y, moe_arena *arena, const moe_routes *routes, void *ws, size_t ws_bytes,
                               WsLayout *w)
{
    MOE_TRY(check_routes(routes));
    MOE_TRY(check_ws(shape, ws, ws_bytes, w));
    if (!X || !Y || !arena) return fail(MOE_ERR_INVALID_ARG, "layer: X, Y and arena are required");
    if (!W_r && !logits) return fail(MOE_ERR_INVALID_ARG, "layer: give W_r or logits");
    if (W_r) MOE_TRY(check_router_args(shape, X, W_r));
    if (!aligned(Y, 16) || (act_bf16(*shape) && !aligned(X, 16)))
        return fail(MOE_ERR_INVALID_ARG, "layer: X and Y must be 16-byte aligned");
    if (arena->shape.d != shape->d || arena->shape.f != shape->f || arena->shape.P != shape->P ||
        arena->shape.dtype != shape->dtype || arena->shape.E != shape->E || arena->shape.n_shared != shape->n_shared)
        return fail(MOE_ERR_INVALID_ARG, "arena was made for another shape");
    return MOE_OK;
}

// The resident layer (every expert Ready in the arena): router, then per
// capacity-sized token range a route build and the expert FFN, then the
// combine. Host state lives on the stack. With clear_err, the workspace's
// device error word is cleared first (by a kernel).
moe_status layer_prefill_resident(const moe_shape *shape, const void *X, const float *W_r, const float *bias,
                                  const float *logits, float *Y, moe_arena *arena, const moe_routes *routes,
                                  void *ws, size_t ws_bytes, hipStream_t cs, bool clear_err)
{
    MOE_TRY(check_shape(shape));
    if (shape->T == 0) return MOE_OK;  // an empty prompt: nothing to do
    WsLayout w;
    MOE_TRY(layer_checks(shape, X, W_r, logits, Y, arena, routes, ws, ws_bytes, &w));
    const moe_shape &s = *shape;
    const int kp = s.k + s.n_shared, ne = s.E + s.n_shared;
    const float *L = logits;
    int32_t phi[kMaxExp];
    PhiArg pa;
    if (clear_err) HIP_TRY(launch_fill_i32(ws_at<int32_t>(ws, w.err), 0, 64, cs), "fill launch");
    if (W_r) {
        L = ws_at<float>(ws, w.logits);
        HIP_TRY(TIMED(MOE_KERNEL_ROUTER, cs, launch_router_logits(s, X, W_r, bias, ws_at<float>(ws, w.logits), cs)),
                "router launch");
    }
    const int tc = (int)std::min<int64_t>(s.T, s.capacity / kp);
    if (s.T > 0 && tc < 1) return fail(MOE_ERR_CAPACITY, "capacity %d below one token's %d routes", s.capacity, kp);
    // every expert must be Ready in the arena; the placement is read and
    // used under the arena's lock
    std::lock_guard<std::mutex> lk(arena->mu);
    arena->res.placement(phi, ne);
    for (int e = 0; e < ne; ++e)
        if (phi[e] < 0) return fail(MOE_ERR_SLOT_STATE, "expert %d is not resident", e);
    MOE_TRY(check_phi(shape, phi, &pa));
    MOE_TRY(arena_acquire(arena, phi, cs));
    for (int t0 = 0; t0 < s.T; t0 += tc) {
        const int nt = std::min(tc, s.T - t0);
        MOE_TRY(route_build_impl(s, w, t0, nt, L, pa, MOE_ROUTE_RESET, *routes, ws, cs));
        MOE_TRY(experts_impl(s, w, X, *routes, arena, nt * kp, false, ws, cs));
    }
    MOE_TRY(arena_release_after(arena, phi, cs));
    HIP_TRY(TIMED(MOE_KERNEL_COMBINE, cs, launch_combine(s, Y, ws_at<float>(ws, w.Yr), ws_at<int32_t>(ws, w.done), cs)),
            "combine launch");
    return MOE_OK;
}

}  // namespace moe

extern "C" {

moe_status moe_layer_prefill(const moe_shape *shape, const void *X, const float *W_r, const float *bias,
                             const float *logits, float *Y, moe_arena *arena, const void *const *host_gu,
                             const void *const *host_d, const moe_routes *routes, void *ws, size_t ws_bytes,
                             moe_stream compute, moe_stream copy)
{
    if ((host_gu == nullptr) != (host_d == nullptr))
        return fail(MOE_ERR_INVALID_ARG, "layer: give both host_gu and host_d, or neither");
    if (!host_gu)
        return layer_prefill_resident(shape, X, W_r, bias, logits, Y, arena, routes, ws, ws_bytes, S(compute), false);
    MOE_TRY(check_shape(shape));
    if (shape->T == 0) return MOE_OK;  // an empty prompt: nothing to do
    WsLayout w;
    MOE_TRY(layer_checks(shape, X, W_r, logits, Y, arena, routes, ws, ws_bytes, &w));
    const moe_shape &s = *shape;
    const int kp = s.k + s.n_shared, ne = s.E + s.n_shared;
    hipStream_t cs = S(compute), ps = copy ? S(copy) : cs;
    const float *L = logits;
    std::vector<int32_t> phi(kMaxExp, -1);
    PhiArg pa;

    // Paged layer (sections 3.3-3.4). Group g holds experts g*G .. g*G+G-1
    // (expert e is member r(e) = e mod G; the permutation pi is the
    // identity), and a group loaded into bank b occupies slots b*G + r(e)
    // (Eq. 4). The first B groups are loaded in group order before routing is
    // known, while the router and top-k run; then the per-expert route counts
    // are read back (the one host synchronisation), groups with no routes are
    // skipped (a prefetched one just frees its bank), and each later group
    // with routes is loaded into the bank released longest ago, only its
    // experts with routes. Loads run on the copy stream, each after its
    // bank's previous release; each group's route build and expert FFN run on
    // the compute stream after its load.
    if ((int64_t)s.T * kp > s.capacity)
        return fail(MOE_ERR_CAPACITY, "paging needs capacity >= T*K' (%lld)", (long long)s.T * kp);
    for (int e = 0; e < ne; ++e)
        if (!host_gu[e] || !host_d[e]) return fail(MOE_ERR_INVALID_ARG, "host expert %d pointer is NULL", e);
    const int G = arena->G, B = s.P / G;
    const int ngroups = (ne + G - 1) / G;
    const int npre = std::min(B, ngroups);
    std::lock_guard<std::mutex> lk(arena->mu);
    arena->res.forget_mapping();   // the previous layer's experts are gone
    std::vector<int> bsl, bex;
    std::vector<const void *> bgu, bd;
    auto bind_group = [&](int g, int bank, const int32_t *counts) -> moe_status {
        bsl.clear(); bex.clear(); bgu.clear(); bd.clear();
        for (int e = g * G; e < std::min(ne, (g + 1) * G); ++e) {
            if (counts && counts[e] == 0) continue;
            bsl.push_back(bank * G + (e % G));
            bex.push_back(e);
            bgu.push_back(host_gu[e]);
            bd.push_back(host_d[e]);
        }
        return arena_bind_many_locked(arena, bsl.data(), bex.data(), (int)bsl.size(), bgu.data(), bd.data(), ps,
                                      true);
    };
    if (ps != cs) {  // prefetch needs its own copy stream to overlap routing
        for (int g = 0; g < npre; ++g) MOE_TRY(bind_group(g, g, nullptr));
    }
    if (W_r) {
        L = ws_at<float>(ws, w.logits);
        HIP_TRY(TIMED(MOE_KERNEL_ROUTER, cs, launch_router_logits(s, X, W_r, bias, ws_at<float>(ws, w.logits), cs)),
                "router launch");
    }
    HIP_TRY(TIMED(MOE_KERNEL_TOPK, cs,
                  launch_topk(s, 0, s.T, L, routes->topk_idx, routes->topk_w, ws_at<int32_t>(ws, w.done), cs)),
            "top-k launch");
    HIP_TRY(TIMED(MOE_KERNEL_ROUTE_COUNT, cs,
                  launch_expert_hist(s, routes->topk_idx, (int64_t)s.T * kp, ws_at<int32_t>(ws, w.ecount), cs)),
            "histogram launch");
    std::vector<int32_t> ecount(ne, 0);
    HIP_TRY(hipMemcpyAsync(ecount.data(), ws_at<int32_t>(ws, w.ecount), ne * 4, hipMemcpyDeviceToHost, cs),
            "hipMemcpyAsync");
    HIP_TRY(hipStreamSynchronize(cs), "hipStreamSynchronize");
    const bool prefetched = ps != cs;
    std::deque<int> banks;  // free or released banks, least recently used first
    if (!prefetched)
        for (int b = 0; b < B; ++b) banks.push_back(b);
    for (int g = 0; g < ngroups; ++g) {
        int routed = 0;
        for (int e = g * G; e < std::min(ne, (g + 1) * G); ++e) routed += ecount[e];
        const bool pre = prefetched && g < npre;
        if (routed == 0) {  // never loaded, or loaded for nothing: its bank is free now
            if (pre) banks.push_front(g);
            continue;
        }
        int bank;
        if (pre) {
            bank = g;
        } else {
            bank = banks.front();
            banks.pop_front();
            MOE_TRY(bind_group(g, bank, ecount.data()));
        }
        std::fill(phi.begin(), phi.end(), -1);
        for (int e = g * G; e < std::min(ne, (g + 1) * G); ++e)
            if (ecount[e] > 0) phi[e] = bank * G + (e % G);
        MOE_TRY(check_phi(shape, phi.data(), &pa));
        MOE_TRY(arena_acquire(arena, phi.data(), cs));
        MOE_TRY(route_build_impl(s, w, 0, s.T, nullptr, pa, 0, *routes, ws, cs));
        MOE_TRY(experts_impl(s, w, X, *routes, arena, s.T * kp, false, ws, cs));
        MOE_TRY(arena_release_after(arena, phi.data(), cs));
        banks.push_back(bank);
    }
    HIP_TRY(TIMED(MOE_KERNEL_COMBINE, cs, launch_combine(s, Y, ws_at<float>(ws, w.Yr), ws_at<int32_t>(ws, w.done), cs)),
                "combine launch");
    return MOE_OK;
}

}  // extern "C"
