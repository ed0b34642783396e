// fused_add_norm_qkv_noalloc: fused_add_norm_qkv for callers that cannot
// allocate device memory (work recorded under HIP graph capture, tight
// serving loops, harnesses that forbid allocation) and so cannot bring a
// workspace either.  The row statistics, split-K partial sums and arrival
// counters of the call live in one file-scope device array, `scratch`, of
// FP_NOALLOC_SCRATCH_BYTES; each GPU the library runs on holds its own copy
// until the process ends.
//
// In host code the array's name is only a host-side stand-in, not a device
// address: the address of a device's copy comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// ever passed to kernels.  Every call on one GPU shares its array: calls
// that overlap on one GPU (two streams, two threads) race.  The kernels need
// nothing of the array's previous contents: the statistics kernel that every
// split launch starts with clears the arrival counters, and every other
// region is written before it is read.
#include "fp_internal.h"

#include <cstdio>
#include <mutex>

namespace {

static __device__ __align__(256) unsigned char scratch[FP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices] = {};   // device address of `scratch` on each device, once known

fp_status static_scratch(size_t need, void **ws, size_t *ws_bytes, char *msg, size_t cap) {
    if (need > (size_t)FP_NOALLOC_SCRATCH_BYTES) {
        snprintf(msg, cap, "the call needs %zu bytes of scratch; the static scratch holds %zu (FP_NOALLOC_SCRATCH_BYTES)",
                 need, (size_t)FP_NOALLOC_SCRATCH_BYTES);
        return FP_E_WORKSPACE;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        snprintf(msg, cap, "hipGetDevice: %s", hipGetErrorString(e));
        return FP_E_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) {
        snprintf(msg, cap, "device %d is beyond the %d devices the static scratch tracks", dev, kMaxDevices);
        return FP_E_HIP;
    }
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));   // the current device's copy
        if (e != hipSuccess || !ptr) {
            snprintf(msg, cap, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
            return FP_E_HIP;
        }
        g_scratch[dev] = ptr;
    }
    *ws = g_scratch[dev];
    *ws_bytes = (size_t)FP_NOALLOC_SCRATCH_BYTES;
    return FP_OK;
}

}  // namespace

extern "C" fp_status fused_add_norm_qkv_noalloc(
    const void *x, const void *residual, void *h_out, const void *gamma, const void *beta, fp_norm norm,
    float eps, const void *w_qkv, const void *w_scale, const void *bias, void *q, void *k, void *v, int64_t M,
    int64_t hidden, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, fp_dtype act_dtype,
    fp_dtype w_dtype, fp_dtype out_dtype, void *hip_stream) {
    return fp::add_norm_qkv_with_source(x, residual, h_out, gamma, beta, norm, eps, w_qkv, w_scale, bias, q, k, v,
                                        M, hidden, n_heads, n_kv_heads, head_dim, act_dtype, w_dtype, out_dtype,
                                        hip_stream, static_scratch);
}
