// Row kernels of libfusedproj: the per-token prologue statistics and the
// stand-alone int8 / int4 weight dequantisation (int4 also stages the weight
// of calls that the weight-streaming kernel does not take).
//
// stats_kernel: h = x + residual in fp32 (exact for 16-bit inputs), the
// residual-stream write h_out = rne(h), and the norm statistics of the token
// row -- mean and 1/sqrt(var + eps) for LayerNorm (two passes over the row),
// 0 and 1/sqrt(mean(h^2) + eps) for RMSNorm -- as in the per-token mean /
// variance / reciprocal-root steps of the LayerNorm + QKV fusion sketch
// ("TensorRT-LLM 深度工程实践…", §2.3).  It also clears the split-K arrival
// counters of the projection that follows on the same stream.
#include "fp_device.hpp"

namespace fp {

// TPR threads per token row (a multiple of 64); 256 / TPR rows per workgroup.
template <int ACT, int TPR>
__global__ __launch_bounds__(256) void stats_kernel(StatsArgs a) {
    using T = Act<ACT>;
    using S = typename T::S;
    constexpr int VE = T::VE;
    constexpr int RPW = 256 / TPR;
    constexpr int WPR = TPR / 64;          // waves per row
    __shared__ float red[4][2];
    const int tid = threadIdx.x;
    for (int i = blockIdx.x * 256 + tid; i < a.n_counters; i += gridDim.x * 256) a.counters[i] = 0u;

    const int lane = tid & 63, wave = tid >> 6;
    const int t = tid % TPR;
    const int64_t m = (int64_t)blockIdx.x * RPW + tid / TPR;
    const bool active = m < a.M;
    const S *xr = (const S *)a.x + (active ? m : 0) * a.K;
    const S *rr = a.res ? (const S *)a.res + (active ? m : 0) * a.K : nullptr;
    S *hr = a.h_out ? (S *)a.h_out + (active ? m : 0) * a.K : nullptr;

    float sum = 0.f, ssq = 0.f;
    if (active) {
#pragma unroll 4
        for (int64_t k = (int64_t)t * VE; k < a.K; k += TPR * VE) {
            float h[VE], r[VE];
            T::unpack(*(const u32x4 *)(xr + k), h);
            if (rr) {
                T::unpack(*(const u32x4 *)(rr + k), r);
#pragma unroll
                for (int e = 0; e < VE; ++e) h[e] += r[e];
            }
            if (hr) *(u32x4 *)(hr + k) = T::pack(h);
#pragma unroll
            for (int e = 0; e < VE; ++e) { sum += h[e]; ssq += h[e] * h[e]; }
        }
    }
    if (a.norm == 0 || a.stats == nullptr) return;   // uniform over the grid

    // row sum / sum of squares over the WPR waves of the row
    auto row_sum = [&](float v, int slot) -> float {
        v = wave_sum(v);
        if constexpr (WPR == 1) {
            return v;
        } else {
            if (lane == 0) red[wave][slot] = v;
            __syncthreads();
            const int w0 = (wave / WPR) * WPR;
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < WPR; ++i) s += red[w0 + i][slot];
            return s;
        }
    };
    const float invK = 1.0f / (float)a.K;
    float mean = 0.f, var;
    if (a.norm == 2) {
        mean = row_sum(sum, 0) * invK;
        float dev = 0.f;
        if (active) {
#pragma unroll 4
            for (int64_t k = (int64_t)t * VE; k < a.K; k += TPR * VE) {
                float h[VE], r[VE];
                T::unpack(*(const u32x4 *)(xr + k), h);
                if (rr) {
                    T::unpack(*(const u32x4 *)(rr + k), r);
#pragma unroll
                    for (int e = 0; e < VE; ++e) h[e] += r[e];
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) { const float d = h[e] - mean; dev += d * d; }
            }
        }
        var = row_sum(dev, 1) * invK;
    } else {
        var = row_sum(ssq, 1) * invK;
    }
    if (active && t == 0) a.stats[m] = make_float2(mean, 1.0f / sqrtf(var + a.eps));
}

// out[j, k] = dequant_i8_bf16(q[j, k], scale[j]) for 16 k per thread.
__global__ __launch_bounds__(256) void dequant_kernel(const int8_t *q, const float *scale,
                                                      unsigned short *out, int64_t N, int64_t K) {
    const int64_t per_row = K / 16;
    const int64_t nv = N * per_row;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / per_row;
        const u32x4 qv = *(const u32x4 *)(q + i * 16);
        u32x4 lo, hi;
        dequant16(qv, scale[row], lo, hi);
        *(u32x4 *)(out + i * 16) = lo;
        *(u32x4 *)(out + i * 16 + 8) = hi;
    }
}

// int4 weights, 32 values (one 16-byte load) per thread: out[j, k] =
// bf16_rne(f32_rne(q[j, k] * scale[j, k / 128])), q packed two per byte.
__global__ __launch_bounds__(256) void dequant_i4_kernel(const uint8_t *q, const float *scale,
                                                         unsigned short *out, int64_t N, int64_t K) {
    const int64_t per_row = K / 32;
    const int64_t nv = N * per_row;
    const int64_t groups = K / 128;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < nv; i += (int64_t)gridDim.x * 256) {
        const int64_t row = i / per_row, k0 = (i % per_row) * 32;
        const u32x4 qv = *(const u32x4 *)(q + i * 16);
        u32x4 o[4];
        dequant32_i4(qv, scale[row * groups + k0 / 128], o);
#pragma unroll
        for (int w = 0; w < 4; ++w) *(u32x4 *)(out + i * 32 + 8 * w) = o[w];
    }
}

static const char *kStatsNames[3] = {"stats_kernel<f32>", "stats_kernel<f16>", "stats_kernel<bf16>"};

const char *stats_kernel_name(int act) { return kStatsNames[act]; }

const char *dequant_kernel_name() { return "dequant_kernel"; }

const char *dequant_i4_kernel_name() { return "dequant_i4_kernel"; }

template <int ACT>
static void launch_stats_t(const StatsArgs &a, hipStream_t s) {
    // few tokens: a whole workgroup per row keeps every load of the row in
    // flight at once; many tokens: one wave per row
    if (a.M <= 1024) {
        const int64_t blocks = a.M > 0 ? a.M : 0;
        const int64_t ctr = (a.n_counters + 255) / 256;
        const unsigned grid = (unsigned)(blocks > ctr ? blocks : ctr);
        if (grid) hipLaunchKernelGGL((stats_kernel<ACT, 256>), dim3(grid), dim3(256), 0, s, a);
    } else {
        const int64_t blocks = (a.M + 3) / 4;
        const int64_t ctr = (a.n_counters + 255) / 256;
        const unsigned grid = (unsigned)(blocks > ctr ? blocks : ctr);
        if (grid) hipLaunchKernelGGL((stats_kernel<ACT, 64>), dim3(grid), dim3(256), 0, s, a);
    }
}

hipError_t launch_stats(int act, const StatsArgs &a, hipStream_t s) {
    switch (act) {
    case ACT_F32: launch_stats_t<ACT_F32>(a, s); break;
    case ACT_F16: launch_stats_t<ACT_F16>(a, s); break;
    default:      launch_stats_t<ACT_BF16>(a, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_dequant_i4(const uint8_t *q, const float *scale, void *out, int64_t N, int64_t K,
                             hipStream_t s) {
    const int64_t nv = N * (K / 32);
    if (nv == 0) return hipSuccess;
    int64_t blocks = (nv + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(dequant_i4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, scale,
                       (unsigned short *)out, N, K);
    return hipGetLastError();
}

hipError_t launch_dequant(const int8_t *q, const float *scale, void *out, int64_t N, int64_t K,
                          hipStream_t s) {
    const int64_t nv = N * (K / 16);
    if (nv == 0) return hipSuccess;
    int64_t blocks = (nv + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, scale,
                       (unsigned short *)out, N, K);
    return hipGetLastError();
}

}  // namespace fp
