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

// Per-token E4M3 quantisation for the W8A8 FP8 projection ("TensorRT-LLM
// 深度工程实践…", §3.3: the full-FP8 configuration, whose activation range
// comes from the data at run time).  Per token row: the residual add (h_out
// written, as stats_kernel does), the row statistics, the normalised row n
// (LayerNorm ((h - mean) * rstd) * gamma + beta, RMSNorm (h * rstd) * gamma,
// none: h), amax = max |n|, the row's scale amax / 448 and the codes
// E4M3_rne(clamp(n * (448 / amax), +-448)); a zero row gets scale 0 and zero
// codes.  Everything that decides a code (statistics, n, amax, the scaled
// value) is computed in double precision without contractions, so the code
// is the correctly rounded E4M3 value of the exactly normalised element up to
// double rounding error (about 1e-16 relative), not of an fp32 approximation
// that can sit on the other side of a rounding midpoint.  The double is
// narrowed to fp32 with round-to-odd (24 bits are more than the 3 + 2 that
// make the following nearest-even E4M3 conversion exact) and converted by the
// hardware.  The row is read from memory once per pass (L2 hits after the
// first); the kernel is bound by memory and latency, not by the fp64 rate.
__device__ __forceinline__ float round_to_odd_f32(double t) {
    const float f = (float)t;   // nearest even
    if ((double)f == t) return f;
    unsigned u = __float_as_uint(f);
    if (fabs((double)f) > fabs(t)) u -= 1u;   // toward zero: the truncated value
    return __uint_as_float(u | 1u);
}

// NV > 0: each thread keeps its NV vectors of 8 elements of h in registers
// after the first pass (rows of at most TPR * 8 * NV elements); NV == 0: every
// pass reads the row again.
template <int ACT, int TPR, int NV>
__global__ __launch_bounds__(256) void quant8_kernel(StatsArgs a) {
    using T = Act<ACT>;
    using S = typename T::S;
    constexpr int VE = T::VE;
    static_assert(VE == 8, "16-bit activations");
    constexpr int RPW = 256 / TPR;
    constexpr int WPR = TPR / 64;
    __shared__ double red[4][3];
    const int tid = threadIdx.x;
    for (int i = blockIdx.x * 256 + tid; i < a.n_counters; i += gridDim.x * 256) a.counters[i] = 0u;

    const int lane = tid & 63, wave = tid >> 6;
    const int t = tid % TPR;
    const int64_t m = (int64_t)blockIdx.x * RPW + tid / TPR;
    const bool active = m < a.M;
    const S *xr = (const S *)a.x + (active ? m : 0) * a.K;
    const S *rr = a.res ? (const S *)a.res + (active ? m : 0) * a.K : nullptr;
    S *hr = a.h_out ? (S *)a.h_out + (active ? m : 0) * a.K : nullptr;
    const S *gr = (const S *)a.gamma, *br = (const S *)a.beta;

    // fn(j, k) for this thread's vectors j (elements k .. k + 7) of the row
    auto each = [&](auto fn) {
        if (!active) return;
        if constexpr (NV > 0) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int64_t k = ((int64_t)j * TPR + t) * VE;
                if (k < a.K) fn(j, k);
            }
        } else {
            for (int64_t k = (int64_t)t * VE; k < a.K; k += TPR * VE) fn(0, k);
        }
    };
    auto load_h = [&](int64_t k, float *h) {   // exact: 16-bit x + 16-bit r fits fp32
        T::unpack(*(const u32x4 *)(xr + k), h);
        if (rr) {
            float r[VE];
            T::unpack(*(const u32x4 *)(rr + k), r);
#pragma unroll
            for (int e = 0; e < VE; ++e) h[e] += r[e];
        }
    };
    float hc[NV > 0 ? NV : 1][VE];
    auto get_h = [&](int j, int64_t k, float *h) {
        if constexpr (NV > 0) {
#pragma unroll
            for (int e = 0; e < VE; ++e) h[e] = hc[j][e];
        } else {
            load_h(k, h);
        }
    };
    // a row-wide reduction over the WPR waves of the row (sum or max)
    auto row_red = [&](double v, int slot, bool is_max) -> double {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const double u = __shfl_xor(v, o, 64);
            v = is_max ? fmax(v, u) : __dadd_rn(v, u);
        }
        if constexpr (WPR == 1) {
            return v;
        } else {
            if (lane == 0) red[wave][slot] = v;
            __syncthreads();
            const int w0 = (wave / WPR) * WPR;
            double s = red[w0][slot];
#pragma unroll
            for (int i = 1; i < WPR; ++i) s = is_max ? fmax(s, red[w0 + i][slot]) : __dadd_rn(s, red[w0 + i][slot]);
            return s;
        }
    };

    double sum = 0.0, ssq = 0.0;
    each([&](int j, int64_t k) {
        float h[VE];
        load_h(k, h);
        if constexpr (NV > 0) {
#pragma unroll
            for (int e = 0; e < VE; ++e) hc[j][e] = h[e];
        }
        if (hr) *(u32x4 *)(hr + k) = T::pack(h);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            const double d = (double)h[e];
            sum = __dadd_rn(sum, d);
            ssq = __dadd_rn(ssq, __dmul_rn(d, d));
        }
    });
    const double K = (double)a.K, eps = (double)a.eps;
    double mean = 0.0, rstd = 1.0;
    if (a.norm == 2) {
        mean = row_red(sum, 0, false) / K;
        double dev = 0.0;
        each([&](int j, int64_t k) {
            float h[VE];
            get_h(j, k, h);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                const double d = __dadd_rn((double)h[e], -mean);
                dev = __dadd_rn(dev, __dmul_rn(d, d));
            }
        });
        rstd = 1.0 / sqrt(__dadd_rn(row_red(dev, 1, false) / K, eps));
    } else if (a.norm == 1) {
        rstd = 1.0 / sqrt(__dadd_rn(row_red(ssq, 1, false) / K, eps));
    }
    auto get_n = [&](int j, int64_t k, double *n) {
        float h[VE];
        get_h(j, k, h);
        if (a.norm == 0) {
#pragma unroll
            for (int e = 0; e < VE; ++e) n[e] = (double)h[e];
            return;
        }
        float g[VE], b[VE];
        T::unpack(*(const u32x4 *)(gr + k), g);
        if (a.norm == 2 && br) T::unpack(*(const u32x4 *)(br + k), b);
#pragma unroll
        for (int e = 0; e < VE; ++e) {
            if (a.norm == 2) {
                n[e] = __dmul_rn(__dmul_rn(__dadd_rn((double)h[e], -mean), rstd), (double)g[e]);
                if (br) n[e] = __dadd_rn(n[e], (double)b[e]);
            } else {
                n[e] = __dmul_rn(__dmul_rn((double)h[e], rstd), (double)g[e]);
            }
        }
    };
    double amax = 0.0;
    each([&](int j, int64_t k) {
        double n[VE];
        get_n(j, k, n);
#pragma unroll
        for (int e = 0; e < VE; ++e) amax = fmax(amax, fabs(n[e]));
    });
    amax = row_red(amax, 2, true);
    const double mult = amax > 0.0 ? 448.0 / amax : 0.0;
    if (active && t == 0) a.qscale[m] = (float)(amax / 448.0);
    unsigned char *cr = a.codes + (active ? m : 0) * a.K;
    each([&](int j, int64_t k) {
        double n[VE];
        get_n(j, k, n);
        unsigned w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                v[e] = round_to_odd_f32(fmin(fmax(__dmul_rn(n[4 * i + e], mult), -448.0), 448.0));
            // two conversions of two values each: bytes 0, 1 then 2, 3
            // (the first operand of each in the lower byte), nearest even
            int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
            w[i] = (unsigned)p;
        }
        *(uint2 *)(cr + k) = make_uint2(w[0], w[1]);
    });
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

template <int ACT, int TPR, int NV>
static void launch_quant8_g(const StatsArgs &a, unsigned grid, hipStream_t s) {
    hipLaunchKernelGGL((quant8_kernel<ACT, TPR, NV>), dim3(grid), dim3(256), 0, s, a);
}

// few tokens: a whole workgroup per row; many tokens: one wave per row.  The
// row stays in registers when each thread's share is at most 16 vectors.
template <int ACT, int TPR>
static void launch_quant8_r(const StatsArgs &a, unsigned grid, hipStream_t s) {
    const int64_t nv = (a.K + TPR * 8 - 1) / (TPR * 8);
    if (nv <= 1) launch_quant8_g<ACT, TPR, 1>(a, grid, s);
    else if (nv <= 2) launch_quant8_g<ACT, TPR, 2>(a, grid, s);
    else if (nv <= 4) launch_quant8_g<ACT, TPR, 4>(a, grid, s);
    else if (nv <= 8) launch_quant8_g<ACT, TPR, 8>(a, grid, s);
    else if (nv <= 16) launch_quant8_g<ACT, TPR, 16>(a, grid, s);
    else launch_quant8_g<ACT, TPR, 0>(a, grid, s);
}

template <int ACT>
static void launch_quant8_t(const StatsArgs &a, hipStream_t s) {
    const int64_t ctr = (a.n_counters + 255) / 256;
    if (a.M <= 1024) {
        const unsigned grid = (unsigned)(a.M > ctr ? a.M : ctr);
        if (grid) launch_quant8_r<ACT, 256>(a, grid, s);
    } else {
        const int64_t blocks = (a.M + 3) / 4;
        const unsigned grid = (unsigned)(blocks > ctr ? blocks : ctr);
        if (grid) launch_quant8_r<ACT, 64>(a, grid, s);
    }
}

hipError_t launch_quant8(int act, const StatsArgs &a, hipStream_t s) {
    if (act == ACT_F16) launch_quant8_t<ACT_F16>(a, s);
    else launch_quant8_t<ACT_BF16>(a, s);
    return hipGetLastError();
}

const char *quant8_kernel_name(int act) {
    return act == ACT_F16 ? "quant8_kernel<f16>" : "quant8_kernel<bf16>";
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
