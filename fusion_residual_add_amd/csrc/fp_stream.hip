// Dispatch and naming of the weight-streaming (decode) and 128 x 512 (prefill)
// projection kernels (fp_stream.hpp / fp_prefill.hpp, instantiated per dtype
// in fp_stream_*.hip / fp_prefill_*.hip).
#include "fp_device.hpp"

#include <cstdio>

namespace fp {

hipError_t launch_stream_bf16(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_stream_f16(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_stream_i8(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_stream_i4(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_stream_mx(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_stream_f8(int act, const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s);

// wq: 0 weights in the activation dtype, 1 int8, 2 int4, 3 MXFP4, 4 E4M3 (with E4M3 activation codes)
hipError_t launch_stream(int act, int wq, const StreamCfg &c, const ProjArgs &a, int grid_wgs, hipStream_t s) {
    if (grid_wgs <= 0 || a.tiles_n <= 0) return hipSuccess;
    if (a.epi == EPI_SWIGLU && c.nr % 2 != 0) return hipErrorInvalidValue;
    // the instantiated row counts (see launch_stream_mf)
    if (c.nr != 2 && !(c.nr == 1 && (wq == 0 || wq == 4) && c.mf <= 2) && !(c.nr == 4 && wq != 0))
        return hipErrorInvalidValue;
    if (c.kh != 1 && !(c.kh == 2 && c.nr == 1 && a.epi != EPI_SWIGLU)) return hipErrorInvalidValue;
    // the kernel's own row pass: M more workgroups (one per token), rows of
    // up to 8192 values
    if (c.rp && (wq == 4 || a.M > 64 || a.rp.K > 8192 || !a.rp_flags)) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)(grid_wgs + (c.rp ? a.M : 0));
    if (wq == 1) return launch_stream_i8(c, a, grid, s);
    if (wq == 2) return launch_stream_i4(c, a, grid, s);
    if (wq == 3) return launch_stream_mx(c, a, grid, s);
    if (wq == 4) return launch_stream_f8(act, c, a, grid, s);
    if (act == ACT_F16) return launch_stream_f16(c, a, grid, s);
    return launch_stream_bf16(c, a, grid, s);
}

hipError_t launch_prefill_bf16(const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_prefill_f16(const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_prefill_i8(const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_prefill_i4(const ProjArgs &a, unsigned grid, hipStream_t s);
hipError_t launch_prefill_mx(const ProjArgs &a, unsigned grid, hipStream_t s);

// wq: 0 weights in the activation dtype, 1 int8, 2 int4, 3 MXFP4
hipError_t launch_prefill(int act, int wq, const ProjArgs &a, hipStream_t s) {
    const int64_t g = (int64_t)a.tiles_m * a.tiles_n * a.splits;
    if (g <= 0) return hipSuccess;
    const unsigned grid = (unsigned)g;
    if (wq == 1) return launch_prefill_i8(a, grid, s);
    if (wq == 2) return launch_prefill_i4(a, grid, s);
    if (wq == 3) return launch_prefill_mx(a, grid, s);
    if (act == ACT_F16) return launch_prefill_f16(a, grid, s);
    return launch_prefill_bf16(a, grid, s);
}

const char *prefill_kernel_name(int act, int wq, int epi) {
    static const char *acts[6] = {"f32", "f16", "bf16", "bf16-i8w", "bf16-i4w", "bf16-mxfp4w"};
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    thread_local char buf[64];
    snprintf(buf, sizeof buf, "prefill_kernel<%s,128x512,%s>", acts[wq ? 2 + wq : act], epis[epi]);
    return buf;
}

const char *stream_kernel_name(int act, int wq, const StreamCfg &c, int epi) {
    static const char *acts[6] = {"f32", "f16", "bf16", "bf16-i8w", "bf16-i4w", "bf16-mxfp4w"};
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    thread_local char buf[64];
    const char *an = wq == 4 ? (act == ACT_F16 ? "f16-e4m3" : "bf16-e4m3") : acts[wq ? 2 + wq : act];
    snprintf(buf, sizeof buf, "stream_kernel<%s,m%d,n%d,k%d,%s%s>", an, 16 * c.mf,
             64 * c.nr / c.kh, 32 * c.u, epis[epi], c.rp ? ",rows" : "");
    return buf;
}

}  // namespace fp
