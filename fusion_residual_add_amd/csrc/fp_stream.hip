// Dispatch and naming of the weight-streaming (decode) and 128 x 512 (prefill)
// projection kernels (fp_stream.hpp / fp_prefill.hpp, instantiated per dtype
// in fp_stream_*.hip / fp_prefill_*.hip).
#include "fp_device.hpp"

#include <cstdio>

namespace fp {

void launch_stream_bf16(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
void launch_stream_f16(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
void launch_stream_i8(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
void launch_stream_i4(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);

// wq: 0 weights in the activation dtype, 1 int8, 2 int4
hipError_t launch_stream(int act, int wq, const StreamCfg &c, const ProjArgs &a, int grid_wgs, hipStream_t s) {
    if (grid_wgs <= 0 || a.tiles_n <= 0) return hipSuccess;
    if (a.epi == EPI_SWIGLU && c.nr % 2 != 0) return hipErrorInvalidValue;
    // the instantiated row counts (see launch_stream_mf)
    if (c.nr != 2 && !(c.nr == 1 && wq == 0 && c.mf <= 2) && !(c.nr == 4 && wq != 0)) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)grid_wgs;
    if (wq == 1) launch_stream_i8(c, a, grid, s);
    else if (wq == 2) launch_stream_i4(c, a, grid, s);
    else if (act == ACT_F16) launch_stream_f16(c, a, grid, s);
    else launch_stream_bf16(c, a, grid, s);
    return hipGetLastError();
}

void launch_prefill_bf16(const ProjArgs &a, unsigned grid, hipStream_t s);
void launch_prefill_f16(const ProjArgs &a, unsigned grid, hipStream_t s);
void launch_prefill_i8(const ProjArgs &a, unsigned grid, hipStream_t s);
void launch_prefill_i4(const ProjArgs &a, unsigned grid, hipStream_t s);

// wq: 0 weights in the activation dtype, 1 int8, 2 int4
hipError_t launch_prefill(int act, int wq, const ProjArgs &a, hipStream_t s) {
    const int64_t g = (int64_t)a.tiles_m * a.tiles_n * a.splits;
    if (g <= 0) return hipSuccess;
    const unsigned grid = (unsigned)g;
    if (wq == 1) launch_prefill_i8(a, grid, s);
    else if (wq == 2) launch_prefill_i4(a, grid, s);
    else if (act == ACT_F16) launch_prefill_f16(a, grid, s);
    else launch_prefill_bf16(a, grid, s);
    return hipGetLastError();
}

const char *prefill_kernel_name(int act, int wq, int epi) {
    static const char *acts[5] = {"f32", "f16", "bf16", "bf16-i8w", "bf16-i4w"};
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    thread_local char buf[64];
    snprintf(buf, sizeof buf, "prefill_kernel<%s,128x512,%s>", acts[wq ? 2 + wq : act], epis[epi]);
    return buf;
}

const char *stream_kernel_name(int act, int wq, const StreamCfg &c, int epi) {
    static const char *acts[5] = {"f32", "f16", "bf16", "bf16-i8w", "bf16-i4w"};
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    thread_local char buf[64];
    snprintf(buf, sizeof buf, "stream_kernel<%s,m%d,n%d,k%d,%s>", acts[wq ? 2 + wq : act], 16 * c.mf,
             64 * c.nr, 32 * c.u, epis[epi]);
    return buf;
}

}  // namespace fp
