// Weight-streaming projection kernel of libfusedproj (gfx950), for decode
// token counts (M <= 64), where the call is bound by reading the weights from
// HBM once ("TensorRT-LLM 深度工程实践…", §3.1: decode is bandwidth-bound;
// §2.3: the LayerNorm + QKV and SwiGLU fusions matter most at small batch).
//
// Design:
//  * Work is split stream-K style: the (weight tile of NB = 64 * NR rows,
//    K chunk of 32 * U) units are laid out tile by tile and every workgroup
//    takes an equal contiguous range of them, so all CUs stream the same
//    number of bytes whatever the tile count.  A range covers one or more
//    tile segments; a tile covered by several workgroups is finished by the
//    last of them to arrive, which adds the partial sums in a fixed order.
//  * Weights go straight from HBM into registers in the MFMA B-operand layout
//    (lane l: row l % 16, eight consecutive k at group l / 16), a whole chunk
//    per wave in flight (NR * U 16-byte loads per lane), reloaded slice by
//    slice as the MFMAs consume them.  int8 weights are dequantised in
//    registers; one 16-byte load then feeds two MFMAs.  int4 weights likewise,
//    one 16-byte load (32 values of one 128-wide scale group) feeding four
//    MFMAs, the group scales loaded with the chunk.
//  * The activation side of each chunk -- x and the residual for all M token
//    rows -- is read (an L2 hit: every workgroup reads it), re-formed as
//    h = x + r, normalised with the row statistics and gamma / beta, rounded to
//    the activation dtype and written to a double-buffered LDS tile that all
//    four waves read their A fragments from.  Its loads are issued before the
//    next chunk's weight loads, so waiting for them never waits for HBM.
//  * Epilogue: bias, then the GQA split / SwiGLU / tanh-GELU / nothing.
#pragma once

#include "fp_device.hpp"

#include <cstdio>
#include <type_traits>

namespace fp {

// WQ: weight storage -- 0 the activation dtype, 1 int8 (one scale per row),
// 2 int4 (one scale per row and group of 128 k, two values per byte).
template <int ACT, int WQ, int MF, int NR, int U, int EPI>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void stream_kernel(ProjArgs p) {
    using T = Act<ACT>;
    constexpr bool WI8 = WQ == 1, WI4 = WQ == 2;
    static_assert(ACT != ACT_F32, "the stream kernel takes 16-bit activations");
    static_assert(WQ == 0 || ACT == ACT_BF16, "int8 / int4 weights feed bf16 MFMA");
    static_assert(EPI != EPI_SWIGLU || NR % 2 == 0, "gate/up fragments come in pairs");
    static_assert(!WI8 || U % 2 == 0, "one int8 load covers two k slices");
    static_assert(!WI4 || U % 4 == 0, "one int4 load covers four k slices (one scale group)");
    constexpr int BMP = 16 * MF;                 // padded token rows
    constexpr int NB = 64 * NR;                  // weight rows per workgroup
    constexpr int CK = 32 * U;                   // k per chunk
    constexpr int LDA = CK + 8;                  // LDS row stride (elements), +16 B pad
    constexpr int NL = WI8 ? U / 2 : WI4 ? U / 4 : U;   // weight loads per fragment per chunk
    constexpr int KVR = CK / 8;                  // 16-byte activation vectors per row per chunk
    constexpr int AV = (BMP * KVR + 255) / 256;  // activation vectors per thread per chunk
    constexpr int AR = 256 / KVR;                // row step between a thread's vectors
    static_assert(256 % KVR == 0, "thread -> activation vector mapping");
    __shared__ __attribute__((aligned(16))) unsigned short lds_a[2][BMP * LDA];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (int)gridDim.x;
    const int g = xcd_remap(blockIdx.x, G);
    const int nchunks = (int)(p.K / CK);
    const int64_t units = (int64_t)p.tiles_n * nchunks;
    // workgroup holding unit v: the largest h with floor(h * units / G) <= v
    auto owner = [&](int64_t v) { return (int)(((v + 1) * G - 1) / units); };

    // one tile segment: tile tn, chunks [c0, c1)
    auto segment = [&](const int tn, const int c0, const int c1) {
        // ---- this lane's weight rows of tile tn (one per fragment).  Rows past the end are
        // clamped to a valid row: the garbage they produce stays in their own
        // accumulator column, which the epilogue never stores.  Keeping every load
        // unconditional keeps the main loop free of branches, so the compiler can
        // count outstanding loads exactly instead of draining them.
        const char *wrow[NR];
        float wsc[NR];
        const float *wsr[NR];   // int4: the row's group scales
    #pragma unroll
        for (int n = 0; n < NR; ++n) {
            int64_t r;
            if constexpr (EPI == EPI_SWIGLU) {
                // fragment pairs (gate, up) of the same 16 output columns
                int64_t j = (int64_t)tn * (NB / 2) + wave * (NR * 8) + (n / 2) * 16 + (lane & 15);
                j = j < p.F ? j : p.F - 1;
                r = (n & 1) ? p.F + j : j;
            } else {
                r = (int64_t)tn * NB + wave * (NR * 16) + n * 16 + (lane & 15);
                r = r < p.Nw ? r : p.Nw - 1;
            }
            wrow[n] = (const char *)p.w + (WI4 ? r * (p.K / 2) : r * p.K * (WI8 ? 1 : 2));
            wsc[n] = 0.f;
            wsr[n] = nullptr;
            if constexpr (WI8) wsc[n] = p.w_scale[r];
            if constexpr (WI4) wsr[n] = p.w_scale + r * (p.K / 128);
        }
        auto wload = [&](int c, int n, int u) -> u32x4 {
            if constexpr (WI8)
                return *(const u32x4 *)(wrow[n] + (int64_t)c * CK + u * 64 + (lane >> 4) * 16);
            else if constexpr (WI4)   // 128 k (one scale group) per u; lane group g: k 32 g .. 32 g + 31
                return *(const u32x4 *)(wrow[n] + (int64_t)c * (CK / 2) + u * 64 + (lane >> 4) * 16);
            else
                return *(const u32x4 *)(wrow[n] + ((int64_t)c * CK + u * 32 + (lane >> 4) * 8) * 2);
        };

        // ---- activation side: fixed k-vector, token rows a_r0 + i * AR (rows past
        // M read row M - 1; they only feed accumulator rows that are never stored).
        // Optional inputs become arithmetic instead of branches:
        //   h = x + rs * r      (rs = 0 and r -> x when there is no residual)
        //   n = ((h - mu) * rstd) * g' + b',  g' = gamma * gs + g1,  b' = beta * bs
        // with (gs, g1) = (1, 0) when there is a norm and (0, 1) otherwise, and
        // bs = 1 only for LayerNorm with a beta (b' = 0 otherwise).
        const int a_kv = tid % KVR, a_r0 = tid / KVR;
        const unsigned short *xp = (const unsigned short *)p.x;
        const unsigned short *rp = p.res ? (const unsigned short *)p.res : xp;
        const float rs = p.res ? 1.f : 0.f;
        const unsigned short *gp = p.norm != 0 ? (const unsigned short *)p.gamma : xp;
        const float gs = p.norm != 0 ? 1.f : 0.f, g1 = p.norm != 0 ? 0.f : 1.f;
        const bool has_beta = p.norm == 2 && p.beta != nullptr;
        const unsigned short *bp = has_beta ? (const unsigned short *)p.beta : gp;
        const float bs = has_beta ? 1.f : 0.f;
        int64_t a_off[AV];
        int a_row[AV];
    #pragma unroll
        for (int i = 0; i < AV; ++i) {
            int row = a_r0 + i * AR;
            row = row < p.M ? row : (int)p.M - 1;
            a_row[i] = row;
            a_off[i] = (int64_t)row * p.K;
        }
        // row statistics: loaded with the first group of loads (see the prologue);
        // without a norm the loads read x (valid memory) and are ignored
        const float2 *stp = p.norm != 0 ? p.stats : (const float2 *)p.x;
        const float st_on = p.norm != 0 ? 1.f : 0.f;
        float a_mu[AV], a_rs[AV];

        // activation registers of one chunk
        struct ARegs {
            u32x4 x[AV], r[AV], g, b;
        };
        auto aload = [&](int c, ARegs &A) {
            const int64_t k = (int64_t)c * CK + a_kv * 8;
    #pragma unroll
            for (int i = 0; i < AV; ++i) {
                A.x[i] = *(const u32x4 *)(xp + a_off[i] + k);
                A.r[i] = *(const u32x4 *)(rp + a_off[i] + k);
            }
            A.g = *(const u32x4 *)(gp + k);
            A.b = *(const u32x4 *)(bp + k);
        };
        auto astore = [&](int buf, const ARegs &A) {
            float g[8], be[8];
            T::unpack(A.g, g);
            T::unpack(A.b, be);
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
                g[e] = g[e] * gs + g1;
                be[e] = be[e] * bs;
            }
    #pragma unroll
            for (int i = 0; i < AV; ++i) {
                if constexpr (AV * AR > BMP) {
                    if (a_r0 + i * AR >= BMP) continue;
                }
                float h[8], r[8];
                T::unpack(A.x[i], h);
                T::unpack(A.r[i], r);
    #pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float hv = fmaf(rs, r[e], h[e]);
                    const float t = (hv - a_mu[i]) * a_rs[i];
                    h[e] = fmaf(t, g[e], be[e]);
                }
                *(u32x4 *)&lds_a[buf][(a_r0 + i * AR) * LDA + a_kv * 8] = T::pack(h);
            }
        };

        f32x4 acc[MF][NR];
    #pragma unroll
        for (int m = 0; m < MF; ++m)
    #pragma unroll
            for (int n = 0; n < NR; ++n) acc[m][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // weight registers of one chunk (int4: with the group scales of the chunk)
        struct WRegs {
            u32x4 w[NR][NL];
            float s[NR][WI4 ? NL : 1];
        };
        auto wload_all = [&](int c, WRegs &W) {
    #pragma unroll
            for (int u = 0; u < NL; ++u)
    #pragma unroll
                for (int n = 0; n < NR; ++n) W.w[n][u] = wload(c, n, u);
            if constexpr (WI4) {
    #pragma unroll
                for (int n = 0; n < NR; ++n) {
                    if constexpr (NL == 2) {   // groups 2c, 2c + 1: adjacent, 8-byte aligned
                        const float2 sv = *(const float2 *)(wsr[n] + 2 * c);
                        W.s[n][0] = sv.x;
                        W.s[n][1] = sv.y;
                    } else {
                        W.s[n][0] = wsr[n][c];
                    }
                }
            }
        };
        // MFMAs of chunk c on the weights in W; when PF, W is then refilled with
        // chunk c + 2 as one burst of loads (a burst keeps each row's 512 contiguous
        // bytes together in the memory controllers' queues)
        auto chunk = [&](int c, int buf, WRegs &W, auto pf) {
            constexpr bool PF = decltype(pf)::value;
            const unsigned short *la = lds_a[buf];
    #pragma unroll
            for (int u = 0; u < NL; ++u) {
                if constexpr (WI4) {
                    u32x4 b[NR][4];
    #pragma unroll
                    for (int n = 0; n < NR; ++n) dequant32_i4(W.w[n][u], W.s[n][u], b[n]);
                    // a lane's 32 int4 are k = 128u + 32 (lane / 16) + [0, 32): four MFMA k slices
    #pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int koff = u * 128 + (lane >> 4) * 32 + qq * 8;
    #pragma unroll
                        for (int m = 0; m < MF; ++m) {
                            const u32x4 a = *(const u32x4 *)&la[(m * 16 + (lane & 15)) * LDA + koff];
    #pragma unroll
                            for (int n = 0; n < NR; ++n) acc[m][n] = T::mfma(a, b[n][qq], acc[m][n]);
                        }
                    }
                } else if constexpr (WI8) {
                    u32x4 lo[NR], hi[NR];
    #pragma unroll
                    for (int n = 0; n < NR; ++n) dequant16(W.w[n][u], wsc[n], lo[n], hi[n]);
                    // a lane's 16 int8 are k = 64u + 16 (lane / 16) + [0, 16): two MFMA k slices
    #pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int koff = u * 64 + (lane >> 4) * 16 + half * 8;
    #pragma unroll
                        for (int m = 0; m < MF; ++m) {
                            const u32x4 a = *(const u32x4 *)&la[(m * 16 + (lane & 15)) * LDA + koff];
    #pragma unroll
                            for (int n = 0; n < NR; ++n) acc[m][n] = T::mfma(a, half ? hi[n] : lo[n], acc[m][n]);
                        }
                    }
                } else {
                    const int koff = u * 32 + (lane >> 4) * 8;
    #pragma unroll
                    for (int m = 0; m < MF; ++m) {
                        const u32x4 a = *(const u32x4 *)&la[(m * 16 + (lane & 15)) * LDA + koff];
    #pragma unroll
                        for (int n = 0; n < NR; ++n) acc[m][n] = T::mfma(a, W.w[n][u], acc[m][n]);
                    }
                }
            }
            if constexpr (PF) {
                __builtin_amdgcn_sched_barrier(0);
                wload_all(c + 2, W);
            }
        };

        // Software pipeline, up to two chunks of weights in flight per wave.
        // Iteration c:
        //   issue the activation loads of chunk c + 2          (into Aload)
        //   MFMAs of chunk c; then refill its weight registers with chunk c + 2
        //   normalise chunk c + 1 into the other LDS buffer    (from Astore)
        //   workgroup barrier
        // Loads retire in issue order, so every wait is for something issued before
        // the weights still in flight: the activations of chunk c + 1 were issued
        // before the weights of chunk c + 1, and the MFMAs of chunk c need only the
        // weights of chunk c.  The three phases are fenced against the scheduler so
        // it cannot hoist a consumer above the loads it must not wait for.
        // Two register sets each for weights (W0/W1) and activations (A0/A1)
        // alternate, so the loop runs in pairs and the last three chunks are peeled.
        WRegs W0, W1;
        ARegs A0, A1;
        auto iter = [&](int c, int buf, WRegs &W, ARegs &Aload, ARegs &Astore, auto pf, auto st) {
            constexpr bool PF = decltype(pf)::value;
            constexpr bool ST = decltype(st)::value;
            if constexpr (PF) aload(c + 2, Aload);
            __builtin_amdgcn_sched_barrier(0);
            chunk(c, buf, W, pf);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (ST) {
                astore(buf ^ 1, Astore);
                __syncthreads();
            }
        };
        const std::true_type Y{};
        const std::false_type N{};
        const int nc = c1 - c0;
        if (nc > 0) {
            // prologue, in issue order: the row statistics and the activations of
            // chunk c0 (needed first), then the weights of c0, the activations and
            // weights of c0 + 1; the fences keep the scheduler from moving a weight
            // burst in front of the loads that the first normalisation waits for
    #pragma unroll
            for (int i = 0; i < AV; ++i) {
                const float2 st = stp[a_row[i]];
                a_mu[i] = st.x * st_on;
                a_rs[i] = st_on != 0.f ? st.y : 1.f;
            }
            aload(c0, A0);
            __builtin_amdgcn_sched_barrier(0);
            wload_all(c0, W0);
            // unconditional (a branch here would make the compiler drain every load
            // at the join); a one-chunk range just reads its chunk twice
            const int c0n = nc > 1 ? c0 + 1 : c0;
            aload(c0n, A1);
            wload_all(c0n, W1);
            __builtin_amdgcn_sched_barrier(0);
            astore(0, A0);
            __syncthreads();
            int c = c0;
            while (c1 - c >= 4) {           // c, c + 1 both prefetch two ahead
                iter(c, 0, W0, A0, A1, Y, Y);
                iter(c + 1, 1, W1, A1, A0, Y, Y);
                c += 2;
            }
            const int left = c1 - c;        // 1, 2 or 3 chunks, starting on W0 / LDS buffer 0
            if (left == 3) {
                iter(c, 0, W0, A0, A1, Y, Y);
                iter(c + 1, 1, W1, A1, A0, N, Y);
                iter(c + 2, 0, W0, A0, A1, N, N);
            } else if (left == 2) {
                iter(c, 0, W0, A0, A1, N, Y);
                iter(c + 1, 1, W1, A1, A0, N, N);
            } else {
                iter(c, 0, W0, A0, A1, N, N);
            }
        }

        // ---- a tile shared with other workgroups: partial sums, and the last
        // contributor to arrive adds them in contributor order
        const int first = owner((int64_t)tn * nchunks), last = owner((int64_t)tn * nchunks + nchunks - 1);
        if (last > first) {
            float flat[MF * NR * 4];
    #pragma unroll
            for (int m = 0; m < MF; ++m)
    #pragma unroll
                for (int n = 0; n < NR; ++n)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) flat[(m * NR + n) * 4 + e] = acc[m][n][e];
            if (!splitk_reduce(p, tn, g - first, last - first + 1, flat)) return;
    #pragma unroll
            for (int m = 0; m < MF; ++m)
    #pragma unroll
                for (int n = 0; n < NR; ++n)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) acc[m][n][e] = flat[(m * NR + n) * 4 + e];
        }

        // ---- epilogue: lane holds token rows 16 m + 4 (lane / 16) + e of weight row lane % 16
    #pragma unroll
        for (int m = 0; m < MF; ++m) {
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m * 16 + (lane >> 4) * 4 + e;
                if (row >= p.M) continue;
                if constexpr (EPI == EPI_SWIGLU) {
    #pragma unroll
                    for (int n = 0; n < NR; n += 2) {
                        const int64_t j = (int64_t)tn * (NB / 2) + wave * (NR * 8) + (n / 2) * 16 + (lane & 15);
                        if (j < p.F) store_swiglu<ACT>(p, row, j, acc[m][n][e], acc[m][n + 1][e]);
                    }
                } else {
    #pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        const int64_t c = (int64_t)tn * NB + wave * (NR * 16) + n * 16 + (lane & 15);
                        if (c >= p.Nw) continue;
                        float y = acc[m][n][e];
                        if (p.bias) y += T::ld(p.bias, c);
                        store_col<ACT, EPI>(p, row, c, y);
                    }
                }
            }
        }
    };

    int64_t u = units * g / G;
    const int64_t u_end = units * (g + 1) / G;
    while (u < u_end) {
        const int tn = (int)(u / nchunks), c0 = (int)(u % nchunks);
        const int64_t left = u_end - u;
        const int c1 = left < nchunks - c0 ? c0 + (int)left : nchunks;
        segment(tn, c0, c1);
        u += c1 - c0;
    }
}

// ---------------------------------------------------------------------------
// launch helpers (instantiated per activation / weight dtype in fp_stream_*.hip)
// ---------------------------------------------------------------------------
template <int ACT, int WQ, int MF, int NR, int U>
inline void launch_stream_cfg(int epi, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (epi) {
    case EPI_QKV:
        hipLaunchKernelGGL((stream_kernel<ACT, WQ, MF, NR, U, EPI_QKV>), dim3(grid), dim3(256), 0, s, a);
        break;
    case EPI_SWIGLU:
        if constexpr (NR % 2 == 0)
            hipLaunchKernelGGL((stream_kernel<ACT, WQ, MF, NR, U, EPI_SWIGLU>), dim3(grid), dim3(256), 0, s, a);
        break;
    case EPI_GELU:
        hipLaunchKernelGGL((stream_kernel<ACT, WQ, MF, NR, U, EPI_GELU>), dim3(grid), dim3(256), 0, s, a);
        break;
    default:
        hipLaunchKernelGGL((stream_kernel<ACT, WQ, MF, NR, U, EPI_LINEAR>), dim3(grid), dim3(256), 0, s, a);
        break;
    }
}

// 64 token rows: 128-wide K chunks (two activation / weight register sets of
// 256-wide chunks do not fit in the register file next to the accumulators)
// Weight rows per workgroup: 64 (NR = 1) only for 16-bit weights at up to 32
// tokens, 256 (NR = 4) only for int8 / int4 weights; only those combinations
// are instantiated.
template <int ACT, int WQ, int MF>
inline void launch_stream_mf(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    constexpr int U = MF >= 4 ? 4 : 8;
    if (c.nr == 2) {
        launch_stream_cfg<ACT, WQ, MF, 2, U>(a.epi, a, grid, s);
    } else if (c.nr == 1) {
        if constexpr (WQ == 0 && MF <= 2) launch_stream_cfg<ACT, WQ, MF, 1, U>(a.epi, a, grid, s);
    } else {
        if constexpr (WQ != 0) launch_stream_cfg<ACT, WQ, MF, 4, U>(a.epi, a, grid, s);   // 256 rows share one A tile
    }
}

template <int ACT, int WQ>
inline void launch_stream_t(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (c.mf) {
    case 1: launch_stream_mf<ACT, WQ, 1>(c, a, grid, s); break;
    case 2: launch_stream_mf<ACT, WQ, 2>(c, a, grid, s); break;
    default: launch_stream_mf<ACT, WQ, 4>(c, a, grid, s); break;
    }
}

}  // namespace fp
