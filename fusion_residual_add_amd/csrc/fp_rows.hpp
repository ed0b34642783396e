// Row pass of libfusedproj held in registers (rows_fast): h = x + residual,
// h_out, the norm statistics and the normalised row of one token, shared by
// the row kernels (fp_rows.hip) and the weight-streaming kernel, which runs
// it in its first workgroups when it forms the rows itself.
#pragma once

#include "fp_device.hpp"

namespace fp {

// Output of the row pass (rows_fast): the statistics only (stats_kernel),
// the normalised rows in the activation dtype (norm_kernel), or their E4M3
// codes and row scales (quant8_kernel).
enum RowOut { OUT_STATS = 0, OUT_ROWS = 1, OUT_CODES = 2 };

// The row pass for rows held in registers (NV > 0): the same values in the
// same order as the looping form of fp_rows.hip, with the memory accesses
// arranged for throughput.  Each
// wave works on one row; x, the residual, gamma and beta are read and h_out,
// the rows or codes written through buffer resources bounded by the row, so
// every access is unconditional (a vector past the row reads zero and its
// stores are dropped) and all loads of a phase are in flight together.  The
// uniform choices (residual present, norm type, h_out wanted) are taken
// outside the per-vector loops.
// blk: the workgroup's index among the nblk workgroups that run the pass.
// DEV: the split-K counters are cleared and the normalised rows written with
// device-coherent stores (gfx950: the sc1 bit; they complete at the
// device-wide coherence point instead of in the XCD's L2), for readers in the
// same launch on other XCDs; otherwise with ordinary stores, for readers in
// later launches.
template <int ACT, int TPR, int NV, int OUT, bool DEV = false>
__device__ __forceinline__ void rows_fast(const StatsArgs &a, const int blk, const int nblk) {
    constexpr bool Q8 = OUT == OUT_CODES;
    using T = Act<ACT>;
    using S = typename T::S;
    constexpr int VE = T::VE;
    static_assert(VE == 8 && NV > 0, "16-bit activations held in registers");
    constexpr int RPW = 256 / TPR;
    constexpr int WPR = TPR / 64;
    __shared__ double red[4][3];
    const int tid = threadIdx.x;
    for (int i = blk * 256 + tid; i < a.n_counters; i += nblk * 256) {
        if constexpr (DEV) __hip_atomic_store(&a.counters[i], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else a.counters[i] = 0u;
    }

    const int lane = tid & 63, wave = tid >> 6;
    const int t = tid % TPR;
    const int64_t m = (int64_t)blk * RPW + __builtin_amdgcn_readfirstlane(tid / TPR);
    const bool active = m < a.M;
    const int64_t mr = active ? m : 0;
    const uint32_t rowb = active ? (uint32_t)(a.K * 2) : 0u;   // 0: every access of the row dropped
    auto rsrc = [](const void *base, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, bytes, 0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rx = rsrc((const S *)a.x + mr * a.K, rowb);
    const bool has_res = a.res != nullptr;
    const __amdgpu_buffer_rsrc_t rr = rsrc(has_res ? (const S *)a.res + mr * a.K : a.x, has_res ? rowb : 0u);
    const bool has_g = OUT != OUT_STATS && a.norm != 0, has_b = OUT != OUT_STATS && a.norm == 2 && a.beta != nullptr;
    const __amdgpu_buffer_rsrc_t rg = rsrc(has_g ? a.gamma : a.x, has_g ? (uint32_t)(a.K * 2) : 0u);
    const __amdgpu_buffer_rsrc_t rb = rsrc(has_b ? a.beta : a.x, has_b ? (uint32_t)(a.K * 2) : 0u);
    auto ld = [](__amdgpu_buffer_rsrc_t r, uint32_t off) -> u32x4 {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    };
    auto koff = [&](int j) -> uint32_t { return (uint32_t)(((j * TPR + t) * VE) * 2); };

    // every load of the row first: x, the residual, gamma, beta (an absent
    // operand's bounded resource holds no bytes: its loads return zero and
    // cost no memory traffic)
    u32x4 xv[NV], rv[NV], gv[NV], bv[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        xv[j] = ld(rx, koff(j));
        rv[j] = ld(rr, koff(j));
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        gv[j] = ld(rg, koff(j));
        bv[j] = ld(rb, koff(j));
    }
    // h = x + residual (exact), kept in registers; h_out.  An absent
    // residual reads as -0 (its zero words with the sign bits set), and
    // x + (-0) is x for every x, -0 included
    const unsigned rneg = has_res ? 0u : 0x80008000u;
    float hc[NV][VE];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        float r[VE];
        T::unpack(xv[j], hc[j]);
        T::unpack(rv[j] | rneg, r);
#pragma unroll
        for (int e = 0; e < VE; ++e) hc[j][e] += r[e];
    }
    if (a.h_out) {
        const __amdgpu_buffer_rsrc_t rh = rsrc((S *)a.h_out + mr * a.K, rowb);
#pragma unroll
        for (int j = 0; j < NV; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, T::pack(hc[j])), rh, koff(j), 0, 0);
    }
    // elements past the row (zero) must not count: only whole vectors lie past K
    auto in_row = [&](int j) { return (int64_t)(j * TPR + t) * VE < a.K; };

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
    const double K = (double)a.K, eps = (double)a.eps;
    double mean = 0.0, rstd = 1.0;
    if (a.norm == 2) {
        double sum = 0.0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (in_row(j)) {
#pragma unroll
                for (int e = 0; e < VE; ++e) sum = __dadd_rn(sum, (double)hc[j][e]);
            }
        mean = row_red(sum, 0, false) / K;
        double dev = 0.0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (in_row(j)) {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const double d = __dadd_rn((double)hc[j][e], -mean);
                    dev = __dadd_rn(dev, __dmul_rn(d, d));
                }
            }
        rstd = 1.0 / sqrt(__dadd_rn(row_red(dev, 1, false) / K, eps));
    } else if (a.norm == 1) {
        double ssq = 0.0;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (in_row(j)) {
#pragma unroll
                for (int e = 0; e < VE; ++e) {
                    const double d = (double)hc[j][e];
                    ssq = __dadd_rn(ssq, __dmul_rn(d, d));
                }
            }
        rstd = 1.0 / sqrt(__dadd_rn(row_red(ssq, 1, false) / K, eps));
    }
    // n in place of h: fp32, in the order of the projection kernels
    const float mu32 = (float)mean, rs32 = (float)rstd;
    if constexpr (OUT == OUT_STATS) {
        if (active && t == 0 && a.stats && a.norm != 0) a.stats[m] = make_float2(mu32, rs32);
        return;
    }
    if (a.norm == 2) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float g[VE], b[VE];
            T::unpack(gv[j], g);
            if (has_b) T::unpack(bv[j], b);
#pragma unroll
            for (int e = 0; e < VE; ++e) {
                const float u = __fmul_rn(__fsub_rn(hc[j][e], mu32), rs32);
                hc[j][e] = fmaf(u, g[e], has_b ? b[e] : 0.f);
            }
        }
    } else if (a.norm == 1) {
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            float g[VE];
            T::unpack(gv[j], g);
#pragma unroll
            for (int e = 0; e < VE; ++e) hc[j][e] = __fmul_rn(__fmul_rn(hc[j][e], rs32), g[e]);
        }
    }
    if constexpr (!Q8) {
        const __amdgpu_buffer_rsrc_t rn = rsrc((S *)a.rows + mr * a.K, rowb);
#pragma unroll
        for (int j = 0; j < NV; ++j)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, T::pack(hc[j])), rn, koff(j), 0, DEV ? 16 : 0);
    } else {
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < NV; ++j)
            if (in_row(j)) {
#pragma unroll
                for (int e = 0; e < VE; ++e) amax = fmaxf(amax, fabsf(hc[j][e]));
            }
        amax = (float)row_red((double)amax, 2, true);
        const float mult = amax > 0.f ? __fdiv_rn(448.f, amax) : 0.f;
        if (active && t == 0) a.qscale[m] = __fdiv_rn(amax, 448.f);
        const __amdgpu_buffer_rsrc_t rc = rsrc(a.codes + mr * a.K, active ? (uint32_t)a.K : 0u);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            unsigned w[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = fminf(fmaxf(__fmul_rn(hc[j][4 * i + e], mult), -448.f), 448.f);
                // two conversions of two values each: bytes 0, 1 then 2, 3
                // (the first operand of each in the lower byte), nearest even
                int p = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
                p = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], p, true);
                w[i] = (unsigned)p;
            }
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, make_uint2(w[0], w[1])), rc, (uint32_t)((j * TPR + t) * VE), 0, 0);
        }
    }
}

}  // namespace fp
