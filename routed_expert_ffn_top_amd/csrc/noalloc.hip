// moe_layer_prefill_noalloc: the resident layer of moe_layer_prefill with
// its workspace taken from a fixed device array of this library instead of
// a caller-allocated buffer, for callers that cannot allocate (code under
// HIP graph capture, tight serving loops, harnesses that forbid it).
//
// The array `scratch` lives in the code object: every GPU the library runs
// on holds its own copy, of kScratchBytes, until the process ends. Its
// device address is looked up once per device (with that device current)
// and kept; the kernels receive that address, exactly as they receive the
// caller's workspace in moe_layer_prefill. In host code the array's name is
// not a device address and is never passed anywhere.
//
// Every call on a device shares that device's array and finds the previous
// call's contents: the only region that must start cleared, the device
// error word, is cleared by a kernel at the start of each call (every other
// region is written before it is read). Calls that overlap on one device
// (other streams, other threads) race on the array.
#include <mutex>

#include "common.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on device d, or null

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_layer_prefill_noalloc(const moe_shape *shape, const void *X, const float *W_r,
                                                const float *bias, const float *logits, float *Y,
                                                moe_arena *arena, const moe_routes *routes,
                                                moe_stream stream)
{
    const size_t need = moe_workspace_bytes(shape);
    if (need == 0) {   // an invalid shape: keep the shape check's status and message
        char msg[512];
        const moe_status st = moe_last_error(msg, sizeof msg);
        return report_error(st != MOE_OK ? st : MOE_ERR_INVALID_ARG, msg);
    }
    if (need > kScratchBytes) {
        char msg[200];
        snprintf(msg, sizeof msg,
                 "noalloc layer: this shape needs %zu bytes of workspace; the fixed device scratch holds %zu "
                 "(use moe_layer_prefill with a workspace)",
                 need, kScratchBytes);
        return report_error(MOE_ERR_WORKSPACE, msg);
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return report_error(MOE_ERR_HIP, "noalloc layer: no usable current device");
    void *ptr = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void *p = nullptr;
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) {
                char msg[200];
                snprintf(msg, sizeof msg, "noalloc layer: hipGetSymbolAddress of the scratch array: %s",
                         hipGetErrorString(e));
                return report_error(MOE_ERR_HIP, msg);
            }
            g_scratch_ptr[dev] = p;
        }
        ptr = g_scratch_ptr[dev];
    }
    return layer_prefill_resident(shape, X, W_r, bias, logits, Y, arena, routes, ptr, kScratchBytes,
                                  (hipStream_t)stream, true);
}
