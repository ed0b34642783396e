// HIP kernels of the fused residual-add + norm + projection path, for gfx950
// (CDNA4: wave64, 16x16 MFMA, 160 KB LDS per CU, 8 XCDs with private L2s).
//
// Three kernels:
//  * stats_kernel   - one wave per token row: h = x + r in fp32, optional
//                     residual-stream write h_out = rne(h), row statistics
//                     (mean, 1/sqrt(var + eps)) for the norm, and clearing of
//                     the split-K arrival counters.
//  * proj_kernel    - the fused projection.  Its A-operand loader reads x and
//                     r, re-forms h, normalises it with the row statistics and
//                     gamma/beta, rounds to the activation dtype and writes the
//                     tile to LDS (the normalised rows never reach memory); its
//                     B-operand loader streams [N, K] weight rows, dequantising
//                     int8 to bf16 on the way; the main loop is MFMA
//                     (16x16x32 bf16/f16, 16x16x4 f32) with fp32 accumulation;
//                     the epilogue adds the bias and applies the GQA split,
//                     SwiGLU, tanh-GELU or nothing, and stores.  Optional
//                     split-K: each split stores partial sums and the last
//                     split to arrive at a tile reduces them in a fixed order
//                     and runs the epilogue (deterministic).
//  * dequant_kernel - the stand-alone int8 -> bf16 dequantisation, using the
//                     same device function as the projection's weight loader.
//
// The method is the cross-operator fusion of the TensorRT-LLM pages
// ("TensorRT-LLM 深度工程实践：从模型到生产级推理服务", §2.3 跨算子融合: the
// LayerNorm + QKV and the SwiGLU fusion sketches; "TRT-LLM deep dive",
// Layer Fusion figure: add / bias / norm / GELU in one kernel).  The CUDA
// sketch there is a per-thread scalar loop; this file is a tiled MFMA design.
#include "fp_internal.h"

#include <cstdio>

namespace fp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// ---------------------------------------------------------------------------
// scalar conversions (round-to-nearest-even for every narrowing)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned to_bf16(float f) {
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)f);
}
__device__ __forceinline__ float f16lo(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
__device__ __forceinline__ unsigned to_f16(float f) {
    return (unsigned)__builtin_bit_cast(unsigned short, (_Float16)f);
}

// int8 weight dequantisation: bf16_rne(f32_rne(q * s)).  The single definition
// used by both the projection's weight loader and dequant_kernel.
__device__ __forceinline__ unsigned dequant_i8_bf16(int q, float s) {
    return to_bf16((float)q * s);
}

// 16 int8 values (one 16-byte load) -> 16 bf16 values (two 16-byte vectors).
__device__ __forceinline__ void dequant16(u32x4 qv, float s, u32x4 &lo, u32x4 &hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned w = qv[i];
        int q0 = (int)(w << 24) >> 24, q1 = (int)(w << 16) >> 24;
        int q2 = (int)(w << 8) >> 24, q3 = (int)w >> 24;
        unsigned p0 = dequant_i8_bf16(q0, s) | (dequant_i8_bf16(q1, s) << 16);
        unsigned p1 = dequant_i8_bf16(q2, s) | (dequant_i8_bf16(q3, s) << 16);
        if (i < 2) { lo[2 * i] = p0; lo[2 * i + 1] = p1; }
        else       { hi[2 * (i - 2)] = p0; hi[2 * (i - 2) + 1] = p1; }
    }
}

// ---------------------------------------------------------------------------
// activation-dtype traits
// ---------------------------------------------------------------------------
template <int ACT> struct Act;

template <> struct Act<ACT_BF16> {
    using S = unsigned short;            // storage element
    using Frag = u32x4;                  // one lane's MFMA operand (8 x bf16)
    static constexpr int VE = 8;         // elements per 16-byte vector
    static constexpr int KM = 32;        // K per MFMA
    __device__ static void unpack(u32x4 v, float *f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf16lo(v[i]); f[2 * i + 1] = bf16hi(v[i]); }
    }
    __device__ static u32x4 pack(const float *f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to_bf16(f[2 * i]) | (to_bf16(f[2 * i + 1]) << 16);
        return v;
    }
    __device__ static float ld(const void *p, int64_t i) {
        return __uint_as_float((unsigned)((const unsigned short *)p)[i] << 16);
    }
    __device__ static void st(void *p, int64_t i, float v) {
        ((unsigned short *)p)[i] = (unsigned short)to_bf16(v);
    }
    __device__ static f32x4 mfma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

template <> struct Act<ACT_F16> {
    using S = unsigned short;
    using Frag = u32x4;
    static constexpr int VE = 8;
    static constexpr int KM = 32;
    __device__ static void unpack(u32x4 v, float *f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = f16lo(v[i]); f[2 * i + 1] = f16hi(v[i]); }
    }
    __device__ static u32x4 pack(const float *f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = to_f16(f[2 * i]) | (to_f16(f[2 * i + 1]) << 16);
        return v;
    }
    __device__ static float ld(const void *p, int64_t i) {
        return (float)__builtin_bit_cast(_Float16, ((const unsigned short *)p)[i]);
    }
    __device__ static void st(void *p, int64_t i, float v) {
        ((unsigned short *)p)[i] = (unsigned short)to_f16(v);
    }
    __device__ static f32x4 mfma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};

template <> struct Act<ACT_F32> {
    using S = float;
    using Frag = float;
    static constexpr int VE = 4;
    static constexpr int KM = 4;
    __device__ static void unpack(u32x4 v, float *f) {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
    }
    __device__ static u32x4 pack(const float *f) {
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
        return v;
    }
    __device__ static float ld(const void *p, int64_t i) { return ((const float *)p)[i]; }
    __device__ static void st(void *p, int64_t i, float v) { ((float *)p)[i] = v; }
    __device__ static f32x4 mfma(Frag a, Frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs (hardware id i runs on
// XCD i % 8).  Give each XCD a contiguous range of logical ids so that tiles
// sharing operands share that XCD's L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int hw, int n) {
    const int q = n >> 3, r = n & 7, x = hw & 7, local = hw >> 3;
    return x * q + (x < r ? x : r) + local;
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// tanh-approximation GELU written through the identity
// 0.5 y (1 + tanh(z)) = y / (1 + exp(-2 z)), z = sqrt(2/pi) (y + 0.044715 y^3).
__device__ __forceinline__ float gelu_tanh(float y) {
    const float c = 0.7978845608028654f;
    float z = c * (y + 0.044715f * y * y * y);
    return y / (1.0f + expf(-2.0f * z));
}

// ---------------------------------------------------------------------------
// row statistics (+ residual stream, + counter clearing)
// ---------------------------------------------------------------------------
template <int ACT>
__global__ __launch_bounds__(256) void stats_kernel(StatsArgs a) {
    using T = Act<ACT>;
    using S = typename T::S;
    constexpr int VE = T::VE;
    const int tid = threadIdx.x;
    for (int i = blockIdx.x * 256 + tid; i < a.n_counters; i += gridDim.x * 256) a.counters[i] = 0u;

    const int lane = tid & 63;
    const int64_t m = (int64_t)blockIdx.x * 4 + (tid >> 6);
    if (m >= a.M) return;
    const S *xr = (const S *)a.x + m * a.K;
    const S *rr = a.res ? (const S *)a.res + m * a.K : nullptr;
    S *hr = a.h_out ? (S *)a.h_out + m * a.K : nullptr;

    float sum = 0.f, ssq = 0.f;
    for (int64_t k = (int64_t)lane * VE; k < a.K; k += 64 * VE) {
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
    if (a.norm == 0 || a.stats == nullptr) return;
    const float invK = 1.0f / (float)a.K;
    float mean = 0.f, var;
    if (a.norm == 2) {
        mean = wave_sum(sum) * invK;
        float dev = 0.f;
        for (int64_t k = (int64_t)lane * VE; k < a.K; k += 64 * VE) {
            float h[VE], r[VE];
            T::unpack(*(const u32x4 *)(xr + k), h);
            if (rr) {
                T::unpack(*(const u32x4 *)(rr + k), r);
#pragma unroll
                for (int e = 0; e < VE; ++e) h[e] += r[e];
            }
#pragma unroll
            for (int e = 0; e < VE; ++e) { float d = h[e] - mean; dev += d * d; }
        }
        var = wave_sum(dev) * invK;
    } else {
        var = wave_sum(ssq) * invK;
    }
    if (lane == 0) a.stats[m] = make_float2(mean, 1.0f / sqrtf(var + a.eps));
}

// ---------------------------------------------------------------------------
// fused projection
// ---------------------------------------------------------------------------
template <int ACT, bool WI8, int BM, int BN, int BK, int WM, int WN, int EPI>
__global__ __launch_bounds__(256) void proj_kernel(ProjArgs p) {
    using T = Act<ACT>;
    using S = typename T::S;
    using Frag = typename T::Frag;
    constexpr int VE = T::VE;
    constexpr int KM = T::KM;
    constexpr int LD = BK + VE;                    // LDS row stride (elements), +16 B pad
    constexpr int KV = BK / VE;                    // act vectors per tile row
    constexpr int A_VPT = (BM * KV + 255) / 256;   // A vectors per thread
    constexpr int A_RSTEP = 256 / KV;              // row step between a thread's vectors
    constexpr int WV = WI8 ? BK / 16 : KV;         // 16-byte weight vectors per tile row
    constexpr int B_VPT = (BN * WV + 255) / 256;
    constexpr int B_RSTEP = 256 / WV;
    constexpr int WTM = BM / WM, WTN = BN / WN;    // wave tile
    constexpr int FM = WTM / 16, FN = WTN / 16;    // 16x16 fragments per wave
    static_assert(WM * WN == 4, "four waves per workgroup");
    static_assert(256 % KV == 0 && 256 % WV == 0, "thread -> vector mapping");
    static_assert(WTM % 16 == 0 && WTN % 32 == 0, "wave tile (gate/up pairs need 32)");
    static_assert(!WI8 || ACT == ACT_BF16, "int8 weights feed bf16 MFMA");

    __shared__ __attribute__((aligned(16))) S lds_a[2][BM * LD];
    __shared__ __attribute__((aligned(16))) S lds_b[2][BN * LD];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // ---- which tile / split this workgroup computes
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    const int tile = logical / p.splits, z = logical % p.splits;
    int tm, tn;
    {
        constexpr int GROUP_M = 8;
        const int group = GROUP_M * p.tiles_n;
        const int gid = tile / group, first = gid * GROUP_M;
        const int gsz = min(p.tiles_m - first, GROUP_M);
        const int in = tile % group;
        tm = first + in % gsz;
        tn = in / gsz;
    }
    const int KT = (int)(p.K / BK);
    const int kt0 = (int)((int64_t)KT * z / p.splits);
    const int kt1 = (int)((int64_t)KT * (z + 1) / p.splits);

    // ---- A-side assignment: fixed k-vector, rows a_r0 + i * A_RSTEP
    const int a_kv = tid % KV, a_r0 = tid / KV;
    const S *xp = (const S *)p.x;
    const S *rp = (const S *)p.res;
    int64_t a_off[A_VPT];
    bool a_in[A_VPT], a_ok[A_VPT];
    float a_mu[A_VPT], a_rs[A_VPT];
#pragma unroll
    for (int i = 0; i < A_VPT; ++i) {
        const int rl = a_r0 + i * A_RSTEP;
        const int64_t m = (int64_t)tm * BM + rl;
        a_in[i] = rl < BM;
        a_ok[i] = a_in[i] && m < p.M;
        a_off[i] = a_ok[i] ? m * p.K : 0;
        a_mu[i] = 0.f;
        a_rs[i] = 1.f;
        if (a_ok[i] && p.norm != 0) {
            const float2 st = p.stats[m];
            a_mu[i] = st.x;
            a_rs[i] = st.y;
        }
    }

    // ---- B-side assignment: fixed k-vector, tile rows b_r0 + i * B_RSTEP
    const int b_kv = tid % WV, b_r0 = tid / WV;
    int64_t b_off[B_VPT];
    bool b_in[B_VPT], b_ok[B_VPT];
    float b_sc[B_VPT];
#pragma unroll
    for (int i = 0; i < B_VPT; ++i) {
        const int br = b_r0 + i * B_RSTEP;
        b_in[i] = br < BN;
        int64_t wrow;
        bool valid;
        if constexpr (EPI == EPI_SWIGLU) {
            // 16-row blocks alternate gate / up for the same 16 output columns
            const int blk = br >> 4;
            const int64_t j = (int64_t)tn * (BN / 2) + (blk >> 1) * 16 + (br & 15);
            valid = j < p.F;
            wrow = (blk & 1) ? p.F + j : j;
        } else {
            wrow = (int64_t)tn * BN + br;
            valid = wrow < p.Nw;
        }
        b_ok[i] = b_in[i] && valid;
        b_off[i] = b_ok[i] ? wrow * p.K : 0;
        b_sc[i] = 0.f;
        if constexpr (WI8) {
            if (b_ok[i]) b_sc[i] = p.w_scale[wrow];
        }
    }

    // ---- register staging for one K-step
    u32x4 xa[A_VPT], ra[A_VPT], gv, bv, wb[B_VPT];
    const bool has_res = rp != nullptr;
    const bool has_beta = p.norm == 2 && p.beta != nullptr;

    auto gload = [&](int kt) {
        const int64_t k0 = (int64_t)kt * BK;
        const int64_t ka = k0 + a_kv * VE;
#pragma unroll
        for (int i = 0; i < A_VPT; ++i) {
            if (a_ok[i]) {
                xa[i] = *(const u32x4 *)(xp + a_off[i] + ka);
                if (has_res) ra[i] = *(const u32x4 *)(rp + a_off[i] + ka);
            }
        }
        if (p.norm != 0) gv = *(const u32x4 *)((const S *)p.gamma + ka);
        if (has_beta) bv = *(const u32x4 *)((const S *)p.beta + ka);
#pragma unroll
        for (int i = 0; i < B_VPT; ++i) {
            if (b_ok[i]) {
                if constexpr (WI8)
                    wb[i] = *(const u32x4 *)((const signed char *)p.w + b_off[i] + k0 + b_kv * 16);
                else
                    wb[i] = *(const u32x4 *)((const S *)p.w + b_off[i] + k0 + b_kv * VE);
            }
        }
    };

    auto lstore = [&](int buf) {
        float g[VE], be[VE];
        if (p.norm != 0) T::unpack(gv, g);
        if (has_beta) T::unpack(bv, be);
#pragma unroll
        for (int i = 0; i < A_VPT; ++i) {
            if (!a_in[i]) continue;
            u32x4 out = {0u, 0u, 0u, 0u};
            if (a_ok[i]) {
                float h[VE], r[VE];
                T::unpack(xa[i], h);
                if (has_res) {
                    T::unpack(ra[i], r);
#pragma unroll
                    for (int e = 0; e < VE; ++e) h[e] += r[e];
                }
                if (p.norm != 0) {
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        float n = (h[e] - a_mu[i]) * a_rs[i];
                        n = n * g[e];
                        if (has_beta) n += be[e];
                        h[e] = n;
                    }
                }
                out = T::pack(h);
            }
            *(u32x4 *)&lds_a[buf][(a_r0 + i * A_RSTEP) * LD + a_kv * VE] = out;
        }
#pragma unroll
        for (int i = 0; i < B_VPT; ++i) {
            if (!b_in[i]) continue;
            const int br = b_r0 + i * B_RSTEP;
            if constexpr (WI8) {
                u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
                if (b_ok[i]) dequant16(wb[i], b_sc[i], lo, hi);
                *(u32x4 *)&lds_b[buf][br * LD + b_kv * 16] = lo;
                *(u32x4 *)&lds_b[buf][br * LD + b_kv * 16 + 8] = hi;
            } else {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (b_ok[i]) v = wb[i];
                *(u32x4 *)&lds_b[buf][br * LD + b_kv * VE] = v;
            }
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf) {
        const S *la = lds_a[buf];
        const S *lb = lds_b[buf];
#pragma unroll
        for (int ks = 0; ks < BK / KM; ++ks) {
            const int koff = ks * KM + (lane >> 4) * (KM / 4);
            Frag af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *(const Frag *)&la[(wm * WTM + i * 16 + (lane & 15)) * LD + koff];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *(const Frag *)&lb[(wn * WTN + j * 16 + (lane & 15)) * LD + koff];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = T::mfma(af[i], bf[j], acc[i][j]);
        }
    };

    if (kt0 < kt1) {
        gload(kt0);
        lstore(0);
        __syncthreads();
        for (int kt = kt0; kt < kt1; ++kt) {
            const int buf = (kt - kt0) & 1;
            if (kt + 1 < kt1) gload(kt + 1);
            compute(buf);
            if (kt + 1 < kt1) lstore(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- split-K: publish partials; the last split to arrive reduces them
    if (p.splits > 1) {
        constexpr int NACC = FM * FN * 4;
        float *mine = p.partials + ((int64_t)tile * p.splits + z) * (int64_t)(BM * BN);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    __hip_atomic_store(&mine[((i * FN + j) * 4 + e) * 256 + tid], acc[i][j][e],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
        __syncthreads();
        if (tid == 0) {
            const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_ACQ_REL,
                                                         __HIP_MEMORY_SCOPE_AGENT);
            s_last = prev == (unsigned)(p.splits - 1);
        }
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        const float *base = p.partials + (int64_t)tile * p.splits * (int64_t)(BM * BN);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int idx = ((i * FN + j) * 4 + e) * 256 + tid;
                    float s = 0.f;
                    for (int zz = 0; zz < p.splits; ++zz)
                        s += __hip_atomic_load(&base[(int64_t)zz * (BM * BN) + idx],
                                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    acc[i][j][e] = s;
                }
        (void)NACC;
    }

    // ---- epilogue: lane holds rows 4*(lane/16)+e, column lane%16 of each fragment
    const int64_t m_base = (int64_t)tm * BM + wm * WTM + (lane >> 4) * 4;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = m_base + i * 16 + e;
            if (m >= p.M) continue;
            if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int j = 0; j < FN; j += 2) {
                    const int64_t c = (int64_t)tn * (BN / 2) + (wn * WTN) / 2 + (j / 2) * 16 + (lane & 15);
                    if (c >= p.F) continue;
                    float g = acc[i][j][e], u = acc[i][j + 1][e];
                    if (p.bias) { g += T::ld(p.bias, c); u += T::ld(p.bias, p.F + c); }
                    const float y = silu(g) * u;
                    if (p.out_f32) ((float *)p.out0)[m * p.F + c] = y;
                    else T::st(p.out0, m * p.F + c, y);
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int64_t c = (int64_t)tn * BN + wn * WTN + j * 16 + (lane & 15);
                    if (c >= p.Nw) continue;
                    float y = acc[i][j][e];
                    if (p.bias) y += T::ld(p.bias, c);
                    void *dst;
                    int64_t idx;
                    if constexpr (EPI == EPI_QKV) {
                        if (c < p.nq)               { dst = p.out0; idx = m * p.nq + c; }
                        else if (c < p.nq + p.nkv)  { dst = p.out1; idx = m * p.nkv + (c - p.nq); }
                        else                        { dst = p.out2; idx = m * p.nkv + (c - p.nq - p.nkv); }
                    } else {
                        if constexpr (EPI == EPI_GELU) y = gelu_tanh(y);
                        dst = p.out0;
                        idx = m * p.F + c;
                    }
                    if (p.out_f32) ((float *)dst)[idx] = y;
                    else T::st(dst, idx, y);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// stand-alone int8 -> bf16 dequantisation
// ---------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
TileShape tile_shape(int cfg) {
    switch (cfg) {
    case TILE_DEC16: return {16, 128, 64};
    case TILE_DEC32: return {32, 128, 64};
    case TILE_DEC64: return {64, 128, 64};
    default:         return {128, 128, 64};
    }
}

static const char *kStatsNames[3] = {"stats_kernel<f32>", "stats_kernel<f16>", "stats_kernel<bf16>"};

const char *stats_kernel_name(int act) { return kStatsNames[act]; }

const char *proj_kernel_name(int act, bool w_i8, int tile, int epi) {
    static const char *acts[4] = {"f32", "f16", "bf16", "bf16-i8w"};
    static const char *tiles[TILE_COUNT] = {"dec16", "dec32", "dec64", "pf128"};
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    static char names[4][TILE_COUNT][4][48];
    static bool init = false;
    if (!init) {
        for (int a = 0; a < 4; ++a)
            for (int t = 0; t < TILE_COUNT; ++t)
                for (int e = 0; e < 4; ++e)
                    snprintf(names[a][t][e], sizeof names[a][t][e], "proj_kernel<%s,%s,%s>", acts[a], tiles[t], epis[e]);
        init = true;
    }
    return names[w_i8 ? 3 : act][tile][epi];
}

const char *dequant_kernel_name() { return "dequant_kernel"; }

hipError_t launch_stats(int act, const StatsArgs &a, hipStream_t s) {
    const int64_t rows_blocks = (a.M + 3) / 4;
    const int64_t ctr_blocks = (a.n_counters + 255) / 256;
    const unsigned grid = (unsigned)(rows_blocks > ctr_blocks ? rows_blocks : ctr_blocks);
    if (grid == 0) return hipSuccess;
    switch (act) {
    case ACT_F32:  hipLaunchKernelGGL(stats_kernel<ACT_F32>, dim3(grid), dim3(256), 0, s, a); break;
    case ACT_F16:  hipLaunchKernelGGL(stats_kernel<ACT_F16>, dim3(grid), dim3(256), 0, s, a); break;
    default:       hipLaunchKernelGGL(stats_kernel<ACT_BF16>, dim3(grid), dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int ACT, bool WI8, int EPI>
static hipError_t launch_proj_e(int tile, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (tile) {
    case TILE_DEC16:
        hipLaunchKernelGGL((proj_kernel<ACT, WI8, 16, 128, 64, 1, 4, EPI>), dim3(grid), dim3(256), 0, s, a);
        break;
    case TILE_DEC32:
        hipLaunchKernelGGL((proj_kernel<ACT, WI8, 32, 128, 64, 1, 4, EPI>), dim3(grid), dim3(256), 0, s, a);
        break;
    case TILE_DEC64:
        hipLaunchKernelGGL((proj_kernel<ACT, WI8, 64, 128, 64, 1, 4, EPI>), dim3(grid), dim3(256), 0, s, a);
        break;
    default:
        hipLaunchKernelGGL((proj_kernel<ACT, WI8, 128, 128, 64, 2, 2, EPI>), dim3(grid), dim3(256), 0, s, a);
        break;
    }
    return hipGetLastError();
}

template <int ACT, bool WI8>
static hipError_t launch_proj_t(int tile, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (a.epi) {
    case EPI_QKV:    return launch_proj_e<ACT, WI8, EPI_QKV>(tile, a, grid, s);
    case EPI_SWIGLU: return launch_proj_e<ACT, WI8, EPI_SWIGLU>(tile, a, grid, s);
    case EPI_GELU:   return launch_proj_e<ACT, WI8, EPI_GELU>(tile, a, grid, s);
    default:         return launch_proj_e<ACT, WI8, EPI_LINEAR>(tile, a, grid, s);
    }
}

hipError_t launch_proj(int act, bool w_i8, int tile, const ProjArgs &a, hipStream_t s) {
    const int64_t g = (int64_t)a.tiles_m * a.tiles_n * a.splits;
    if (g <= 0) return hipSuccess;
    const unsigned grid = (unsigned)g;
    if (w_i8) return launch_proj_t<ACT_BF16, true>(tile, a, grid, s);
    switch (act) {
    case ACT_F32: return launch_proj_t<ACT_F32, false>(tile, a, grid, s);
    case ACT_F16: return launch_proj_t<ACT_F16, false>(tile, a, grid, s);
    default:      return launch_proj_t<ACT_BF16, false>(tile, a, grid, s);
    }
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
