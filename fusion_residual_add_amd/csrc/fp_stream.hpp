// Weight-streaming projection kernel of libfusedproj (gfx950), for decode
// token counts (M <= 64), where the call is bound by reading the weights from
// HBM once ("TensorRT-LLM 深度工程实践…", §3.1: decode is bandwidth-bound;
// §2.3: the LayerNorm + QKV and SwiGLU fusions matter most at small batch).
//
// Design:
//  * Work is split stream-K style: the (weight tile of NB = 64 * NR rows,
//    or 32 with K halves, K chunk of 32 * U) units are laid out tile by tile
//    and every workgroup takes an equal contiguous range of them, so all CUs
//    stream the same number of bytes whatever the tile count.  A range
//    covers one or more tile segments; a tile covered by several workgroups
//    is finished by the last of them to arrive, which adds the partial sums
//    in a fixed order.
//  * Weights go straight from HBM into registers in the MFMA B-operand layout
//    (lane l: row l % 16, eight consecutive k at group l / 16), a whole chunk
//    per wave in flight (16-bit weights: NR * U / KH 16-byte loads per
//    lane), reloaded slice by slice as the MFMAs consume them.  int8 weights
//    are dequantised in registers; one 16-byte load then feeds two MFMAs.
//    int4 weights likewise, one 16-byte load (32 values of one 128-wide scale
//    group) feeding four MFMAs, the group scales loaded with the chunk.
//  * The activation side of each chunk -- the rows of all M tokens, as the
//    row pass formed them once per call (h = x + r, normalised, rounded to
//    the activation dtype), or the per-token E4M3 codes -- is read (an L2
//    hit: every workgroup reads it) and copied (codes: decoded) into a
//    double-buffered LDS tile that all four waves read their A fragments
//    from.  Its loads are issued before the next chunk's weight loads, so
//    waiting for them never waits for HBM.  (Normalising in every workgroup
//    instead, from x, the residual and the row statistics, repeats the same
//    arithmetic on every CU: measured on MI355X, Llama-3-8B decode, 4.5-4.9 us
//    of each call.)
//  * Epilogue: bias, then the GQA split / SwiGLU / tanh-GELU / nothing.
#pragma once

#include "fp_rows.hpp"

#include <cstdio>
#include <type_traits>

namespace fp {

// WQ: weight storage -- 0 the activation dtype, 1 int8 (one scale per row),
// 2 int4 (one scale per row and group of 128 k, two values per byte),
// 3 MXFP4 (E2M1 codes two per byte, one E8M0 scale per row and 32 k),
// 4 E4M3 with one scale per row, for the FP8 W8A8 call: the A side is then
//   the per-token E4M3 codes of the quantisation pass (x = codes [M, K],
//   a_scale [M]) instead of x + residual and the norm, both operands are
//   decoded exactly to bf16 in registers (the products are those of the FP8
//   matrix cores), and the epilogue scales by a_scale[m] * w_scale[c].
// KH: K parts per chunk.  KH = 2 (16-bit and E4M3 weights, no gate/up
// pairing): the four waves are two row groups x two halves of each chunk's
// K, so a workgroup covers 32 weight rows (NR = 1) with the bytes per chunk
// of a 64-row tile; the two halves' sums meet in LDS at the end.  The host
// gives every such workgroup one whole tile (no partial sums between
// workgroups), so a 6144-row QKV weight is 192 tiles on 192 workgroups.
// RP: 0 -- the A rows come formed (p.x); RP > 0 -- the kernel forms them
// itself (p.rp, hidden up to 2048 * RP): M extra workgroups, the first of the
// launch, each run the row pass for one token and publish the row; every
// other workgroup waits for all M rows after it has requested its first two
// chunks of weights (see rp_wait).  The host takes this form where the extra
// workgroups fit on CUs that the streaming grid leaves idle.
template <int ACT, int WQ, int MF, int NR, int U, int EPI, int KH, int RP = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void stream_kernel(ProjArgs p) {
    constexpr bool WF8 = WQ == 4;
    using T = Act<ACT>;                          // activation dtype: bias, outputs
    using TM = Act<WF8 ? ACT_BF16 : ACT>;        // MFMA operands (decoded E4M3 are bf16)
    constexpr bool WI8 = WQ == 1 || WF8, WMX = WQ == 3, WI4 = WQ == 2 || WMX;   // WI8: one byte per weight; WI4: 4-bit weights of either kind
    static_assert(ACT != ACT_F32, "the stream kernel takes 16-bit activations");
    static_assert(WQ == 0 || WF8 || ACT == ACT_BF16, "int8 / int4 / MXFP4 weights feed bf16 MFMA");
    static_assert(EPI != EPI_SWIGLU || NR % 2 == 0, "gate/up fragments come in pairs");
    static_assert(!WI8 || U % 2 == 0, "one int8 load covers two k slices");
    static_assert(!WI4 || U % 4 == 0, "one int4 load covers four k slices (one scale group)");
    constexpr int BMP = 16 * MF;                 // padded token rows
    static_assert(KH == 1 || (KH == 2 && NR == 1 && EPI != EPI_SWIGLU && (WQ == 0 || WF8)), "K halves");
    constexpr int NWR = 4 / KH;                  // row groups of waves
    constexpr int NB = 16 * NR * NWR;            // weight rows per workgroup
    constexpr int CK = 32 * U;                   // k per chunk
    constexpr int LDA = CK + 8;                  // LDS row stride (elements), +16 B pad
    constexpr int NL = WI8 ? U / 2 : WI4 ? U / 4 : U;   // weight loads per fragment per chunk
    constexpr int NLW = NL / KH;                 // ... of them by one wave
    static_assert(NL % KH == 0, "whole loads per K part");
    constexpr int KVR = CK / 8;                  // 16-byte activation vectors per row per chunk
    constexpr int AV = (BMP * KVR + 255) / 256;  // activation vectors per thread per chunk
    constexpr int AR = 256 / KVR;                // row step between a thread's vectors
    static_assert(256 % KVR == 0, "thread -> activation vector mapping");
    __shared__ __attribute__((aligned(16))) unsigned short lds_a[2][BMP * LDA];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = wave % NWR, kh = wave / NWR;   // the wave's row group and K part
    const int ub = kh * NLW;                      // its first load slice of a chunk
    const int G = (int)gridDim.x - (RP > 0 ? (int)p.M : 0);   // workgroups that stream
    const int g = xcd_remap((int)blockIdx.x - (RP > 0 ? (int)p.M : 0), G);
    const int nchunks = (int)(p.K / CK);
    const int64_t units = (int64_t)p.tiles_n * nchunks;
    // workgroup holding unit v: the largest h with floor(h * units / G) <= v
    auto owner = [&](int64_t v) { return (int)(((v + 1) * G - 1) / units); };

    // ---- the kernel's own row pass (RP > 0).  The launch has M extra
    // workgroups, the first M (dispatched before any that waits for them):
    // workgroup b forms token row b (h_out, the normalised row into
    // p.rp.rows, the split-K counters cleared), waits for its stores to
    // complete and publishes the row by storing this launch's tag into the
    // row's flag.  Rows, counters and flags are written with device-coherent
    // stores (complete at the device-wide coherence point, not in the XCD's
    // L2), so a flag is visible only after the row it publishes is in
    // memory; a waiting workgroup (rp_wait) reads the flags with
    // device-coherent loads and only then issues its first load of the rows,
    // which fills its XCD's L2 from memory: no L2 held the rows' lines when
    // the launch started (the launch boundary writes back and invalidates the
    // XCDs' L2s), and nothing in this launch reads them before their flags.
    // (Fences at device scope instead write back and invalidate a whole L2 at
    // every publication and wait: measured on MI355X, Llama-3-8B decode,
    // 26.6 us against 23.6 us for the separate row pass + kernel on QKV.)
    // Measured on MI355X, decode steps on tile-packed weights (median of 3 x
    // 100 steps, both calls): Llama-3-8B 64.3 -> 63.6 us, Llama-2-70B int8 at
    // 1 token 110.1 -> 108.1 us, at 16 tokens 113.1 -> 112.6 us, MXFP4 at 16
    // 102.7 -> 97.2 us.  The gain is small because the hand-over is itself a
    // chain of memory round trips (the rows' loads, the acknowledged stores,
    // the flag, the poll, the rows' first load); waiting for the rows before
    // requesting any weights measured slower (66.8 us for Llama-3-8B), and
    // delaying the weight requests to let the rows' loads ahead gained nothing.
    const int nprod = RP > 0 ? (int)p.M : 0;
    if constexpr (RP > 0) {
        if ((int)blockIdx.x < nprod) {
            rows_fast<ACT, 256, RP, OUT_ROWS, true>(p.rp, (int)blockIdx.x, nprod);
            __builtin_amdgcn_s_waitcnt(0);   // this thread's stores have completed
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(&p.rp_flags[blockIdx.x], p.rp_tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
    // Wait until all M flags hold this launch's tag (lane m of wave 0 polls
    // row m's flag); the workgroup barrier then releases the other waves.
    // The tag is unique per launch within the process, so a flag left by an
    // earlier launch never reads as ready.  The wait is bounded (p.rp_spin
    // polls, about a second): if it runs out the workgroup carries on and
    // stores NaN, so a fault in the dispatch order shows in the outputs
    // instead of hanging the device.  Returns false when it ran out.
    auto rp_wait = [&]() -> bool {
        bool ok = true;
        if (wave == 0) {
            ok = false;
            for (int spin = 0; spin < p.rp_spin; ++spin) {
                const unsigned long long v =
                    lane < p.M ? __hip_atomic_load(&p.rp_flags[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : p.rp_wait_tag;
                if (__ballot(v != p.rp_wait_tag) == 0) {
                    ok = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        return __syncthreads_or(ok ? 0 : 1) == 0;
    };
    bool rp_ok = true;

    // one tile segment: tile tn, chunks [c0, c1)
    // RPF (std::true_type): the launch's first segment of an RP kernel
    auto segment = [&](const int tn, const int c0, const int c1, auto rpf) {
        constexpr bool RPF = decltype(rpf)::value;
        // ---- this lane's weight rows of tile tn (one per fragment).  Rows past the end are
        // clamped to a valid row: the garbage they produce stays in their own
        // accumulator column, which the epilogue never stores.  Keeping every load
        // unconditional keeps the main loop free of branches, so the compiler can
        // count outstanding loads exactly instead of draining them.
        // row bytes; a chunk's bytes per row; the address step per chunk and per
        // 64-byte load slice (row-major rows, or tile-packed 1 KB block slices)
        constexpr int64_t CKB = WI4 ? CK / 2 : WI8 ? CK : CK * 2;
        const int64_t rbytes = WI4 ? p.K / 2 : WI8 ? p.K : p.K * 2;
        const int64_t cstep = p.w_layout ? NL * 8192 : CKB, ustep = p.w_layout ? 8192 : 64;
        const char *wrow[NR];   // this lane's first byte of its row (its 16-byte group of slice 0)
        float wsc[NR];
        const float *wsr[NR];   // int4: the row's group scales
        const unsigned char *wsm[NR];   // MXFP4: the row's block scales
    #pragma unroll
        for (int n = 0; n < NR; ++n) {
            int64_t r;
            if constexpr (EPI == EPI_SWIGLU) {
                // fragment pairs (gate, up) of the same 16 output columns
                int64_t j = (int64_t)tn * (NB / 2) + wr * (NR * 8) + (n / 2) * 16 + (lane & 15);
                j = j < p.F ? j : p.F - 1;
                r = (n & 1) ? p.F + j : j;
            } else {
                r = (int64_t)tn * NB + wr * (NR * 16) + n * 16 + (lane & 15);
                r = r < p.Nw ? r : p.Nw - 1;
            }
            wrow[n] = (const char *)p.w + weight_off(p.w_layout, r, (lane >> 4) * 16, p.F, rbytes);
            wsc[n] = 0.f;
            wsr[n] = nullptr;
            wsm[n] = nullptr;
            if constexpr (WI8) wsc[n] = p.w_scale[r];   // int8: applied when dequantising; E4M3: in the epilogue
            if constexpr (WQ == 2) wsr[n] = p.w_scale + r * (p.K / 128);
            if constexpr (WMX) wsm[n] = (const unsigned char *)p.w_scale + r * (p.K / 32);
        }
        // load slice u of chunk c: row bytes c * CKB + 64 u + 16 (lane / 16) .. + 15
        // (int8 / E4M3: 16 k; int4 / MXFP4: 32 k, one 128-k scale group per u
        // with lane group g at k 32 g; 16-bit: 8 k)
        auto wload = [&](int c, int n, int u) -> u32x4 {
            return *(const u32x4 *)(wrow[n] + (int64_t)c * cstep + (ub + u) * ustep);
        };

        // ---- activation side: fixed k-vector, token rows a_r0 + i * AR (rows past
        // M read row M - 1; they only feed accumulator rows that are never
        // stored).  The A operand comes formed: the normalised rows of the row
        // pass in the activation dtype (or the call's input as it is), or, for
        // E4M3, the per-token codes; a chunk is copied (codes: decoded) into
        // the LDS tile as it is.
        const int a_kv = tid % KVR, a_r0 = tid / KVR;
        int64_t a_off[AV];
    #pragma unroll
        for (int i = 0; i < AV; ++i) {
            int row = a_r0 + i * AR;
            row = row < p.M ? row : (int)p.M - 1;
            a_off[i] = (int64_t)row * p.K;
        }
        struct ARegs {
            u32x4 x[AV];
        };
        // E4M3: the per-token scales of the epilogue's rows (token rows
        // 16 m + 4 (lane / 16) + e), loaded here so that the epilogue does not
        // wait for them
        float asr[MF][4];
    #pragma unroll
        for (int m = 0; m < MF; ++m)
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                int64_t row = m * 16 + (lane >> 4) * 4 + e;
                row = row < p.M ? row : p.M - 1;
                asr[m][e] = WF8 ? p.a_scale[row] : 1.f;
            }
        auto aload = [&](int c, ARegs &A) {
            const int64_t k = (int64_t)c * CK + a_kv * 8;
            if constexpr (WF8) {   // 8 codes per vector
                const unsigned char *cp = (const unsigned char *)p.x;
    #pragma unroll
                for (int i = 0; i < AV; ++i) {
                    const uint2 v = *(const uint2 *)(cp + a_off[i] + k);
                    A.x[i] = (u32x4){v.x, v.y, 0u, 0u};
                }
            } else {
                const unsigned short *xp = (const unsigned short *)p.x;
    #pragma unroll
                for (int i = 0; i < AV; ++i) A.x[i] = *(const u32x4 *)(xp + a_off[i] + k);
            }
        };
        auto astore = [&](int buf, const ARegs &A) {
    #pragma unroll
            for (int i = 0; i < AV; ++i) {
                if constexpr (AV * AR > BMP) {
                    if (a_r0 + i * AR >= BMP) continue;
                }
                u32x4 v;
                if constexpr (WF8) v = decode8_e4m3(A.x[i][0], A.x[i][1]);
                else v = A.x[i];
                *(u32x4 *)&lds_a[buf][(a_r0 + i * AR) * LDA + a_kv * 8] = v;
            }
        };

        f32x4 acc[MF][NR];
    #pragma unroll
        for (int m = 0; m < MF; ++m)
    #pragma unroll
            for (int n = 0; n < NR; ++n) acc[m][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

        // weight registers of one chunk (int4: with the group scales of the
        // chunk; MXFP4: with the block scale code of each lane's load)
        struct WRegs {
            u32x4 w[NR][NLW];
            float s[NR][WI4 ? NL : 1];
            unsigned sm[NR][WMX ? NL : 1];
        };
        auto wload_all = [&](int c, WRegs &W) {
    #pragma unroll
            for (int u = 0; u < NLW; ++u)
    #pragma unroll
                for (int n = 0; n < NR; ++n) W.w[n][u] = wload(c, n, u);
            if constexpr (WMX) {
                // lane group g of load u covers the 32-k block 4 (c * U / 4 + u) + g
    #pragma unroll
                for (int u = 0; u < NL; ++u)
    #pragma unroll
                    for (int n = 0; n < NR; ++n)
                        W.sm[n][u] = wsm[n][(int64_t)c * (CK / 32) + u * 4 + (lane >> 4)];
            } else if constexpr (WI4) {
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
            for (int u = 0; u < NLW; ++u) {
                const int ug = ub + u;   // the load's slice of the chunk
                if constexpr (WI4) {
                    u32x4 b[NR][4];
    #pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        if constexpr (WMX) dequant32_mxfp4(W.w[n][u], W.sm[n][u], b[n]);
                        else dequant32_i4(W.w[n][u], W.s[n][u], b[n]);
                    }
                    // a lane's 32 int4 are k = 128u + 32 (lane / 16) + [0, 32): four MFMA k slices
    #pragma unroll
                    for (int qq = 0; qq < 4; ++qq) {
                        const int koff = ug * 128 + (lane >> 4) * 32 + qq * 8;
    #pragma unroll
                        for (int m = 0; m < MF; ++m) {
                            const u32x4 a = *(const u32x4 *)&la[(m * 16 + (lane & 15)) * LDA + koff];
    #pragma unroll
                            for (int n = 0; n < NR; ++n) acc[m][n] = TM::mfma(a, b[n][qq], acc[m][n]);
                        }
                    }
                } else if constexpr (WI8) {
                    u32x4 lo[NR], hi[NR];
    #pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        if constexpr (WF8) {
                            lo[n] = decode8_e4m3(W.w[n][u][0], W.w[n][u][1]);
                            hi[n] = decode8_e4m3(W.w[n][u][2], W.w[n][u][3]);
                        } else {
                            dequant16(W.w[n][u], wsc[n], lo[n], hi[n]);
                        }
                    }
                    // a lane's 16 int8 are k = 64u + 16 (lane / 16) + [0, 16): two MFMA k slices
    #pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int koff = ug * 64 + (lane >> 4) * 16 + half * 8;
    #pragma unroll
                        for (int m = 0; m < MF; ++m) {
                            const u32x4 a = *(const u32x4 *)&la[(m * 16 + (lane & 15)) * LDA + koff];
    #pragma unroll
                            for (int n = 0; n < NR; ++n) acc[m][n] = TM::mfma(a, half ? hi[n] : lo[n], acc[m][n]);
                        }
                    }
                } else {
                    const int koff = ug * 32 + (lane >> 4) * 8;
    #pragma unroll
                    for (int m = 0; m < MF; ++m) {
                        const u32x4 a = *(const u32x4 *)&la[(m * 16 + (lane & 15)) * LDA + koff];
    #pragma unroll
                        for (int n = 0; n < NR; ++n) acc[m][n] = TM::mfma(a, W.w[n][u], acc[m][n]);
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
            // unconditional (a branch here would make the compiler drain every load
            // at the join); a one-chunk range just reads its chunk twice
            const int c0n = nc > 1 ? c0 + 1 : c0;
            if constexpr (RPF) {
                // the weights of c0 and c0 + 1 first, then the wait for the
                // rows, then their activations
                wload_all(c0, W0);
                wload_all(c0n, W1);
                __builtin_amdgcn_sched_barrier(0);
                rp_ok = rp_wait();
                __builtin_amdgcn_sched_barrier(0);
                aload(c0, A0);
                aload(c0n, A1);
            } else {
                // prologue, in issue order: the activations of chunk c0 (needed
                // first), then the weights of c0, the activations and weights of
                // c0 + 1; the fences keep the scheduler from moving a weight burst
                // in front of the loads that the first LDS copy waits for
                aload(c0, A0);
                __builtin_amdgcn_sched_barrier(0);
                wload_all(c0, W0);
                aload(c0n, A1);
                wload_all(c0n, W1);
            }
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

        // a workgroup whose wait for the rows ran out stores NaN (its partial
        // sums, if it shares the tile, carry them to the tile's last arriver)
        if constexpr (RP > 0) {
            if (!rp_ok) {
    #pragma unroll
                for (int m = 0; m < MF; ++m)
    #pragma unroll
                    for (int n = 0; n < NR; ++n) acc[m][n] = (f32x4){__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
            }
        }

        // ---- K halves: the second half's waves hand their sums to the first
        // half's waves of the same row group through LDS (then hold zeros, so
        // that a shared tile's partial sums below stay whole-workgroup)
        if constexpr (KH == 2) {
            __shared__ float red[NWR][MF * 4][64];
            if (kh) {
    #pragma unroll
                for (int m = 0; m < MF; ++m)
    #pragma unroll
                    for (int e = 0; e < 4; ++e) red[wr][m * 4 + e][lane] = acc[m][0][e];
            }
            __syncthreads();
    #pragma unroll
            for (int m = 0; m < MF; ++m)
    #pragma unroll
                for (int e = 0; e < 4; ++e) acc[m][0][e] = kh ? 0.f : acc[m][0][e] + red[wr][m * 4 + e][lane];
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
        if (kh) return;
    #pragma unroll
        for (int m = 0; m < MF; ++m) {
    #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t row = m * 16 + (lane >> 4) * 4 + e;
                if (row >= p.M) continue;
                // E4M3: the products' sum times the token's and the weight row's scales
                const float as = asr[m][e];
                auto scaled = [&](int n) { return WF8 ? acc[m][n][e] * as * wsc[n] : acc[m][n][e]; };
                if constexpr (EPI == EPI_SWIGLU) {
    #pragma unroll
                    for (int n = 0; n < NR; n += 2) {
                        const int64_t j = (int64_t)tn * (NB / 2) + wr * (NR * 8) + (n / 2) * 16 + (lane & 15);
                        if (j < p.F) store_swiglu<ACT>(p, row, j, scaled(n), scaled(n + 1));
                    }
                } else {
    #pragma unroll
                    for (int n = 0; n < NR; ++n) {
                        const int64_t c = (int64_t)tn * NB + wr * (NR * 16) + n * 16 + (lane & 15);
                        if (c >= p.Nw) continue;
                        float y = scaled(n);
                        if (p.bias) y += T::ld(p.bias, c);
                        store_col<ACT, EPI>(p, row, c, y);
                    }
                }
            }
        }
    };

    int64_t u = units * g / G;
    const int64_t u_end = units * (g + 1) / G;
    bool first_segment = true;
    while (u < u_end) {
        const int tn = (int)(u / nchunks), c0 = (int)(u % nchunks);
        const int64_t left = u_end - u;
        const int c1 = left < nchunks - c0 ? c0 + (int)left : nchunks;
        // a segment that no other workgroup shares ends without a barrier, its
        // last chunk possibly read from LDS buffer 0: every wave must be done
        // with it before the next segment's prologue normalises into buffer 0
        if (!first_segment) __syncthreads();
        if constexpr (RP > 0) {
            if (first_segment) segment(tn, c0, c1, std::true_type{});
            else segment(tn, c0, c1, std::false_type{});
        } else {
            segment(tn, c0, c1, std::false_type{});
        }
        first_segment = false;
        u += c1 - c0;
    }
}

// ---------------------------------------------------------------------------
// launch helpers (instantiated per activation / weight dtype in fp_stream_*.hip)
// ---------------------------------------------------------------------------
template <int ACT, int WQ, int MF, int NR, int U, int KH, int RP>
inline hipError_t launch_stream_epi(int epi, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (epi) {
    case EPI_QKV:
        return launch_k(stream_kernel<ACT, WQ, MF, NR, U, EPI_QKV, KH, RP>, grid, s, a);
    case EPI_SWIGLU:
        if constexpr (NR % 2 == 0 && KH == 1)
            return launch_k(stream_kernel<ACT, WQ, MF, NR, U, EPI_SWIGLU, KH, RP>, grid, s, a);
        return hipErrorInvalidValue;
    case EPI_GELU:
        return launch_k(stream_kernel<ACT, WQ, MF, NR, U, EPI_GELU, KH, RP>, grid, s, a);
    default:
        return launch_k(stream_kernel<ACT, WQ, MF, NR, U, EPI_LINEAR, KH, RP>, grid, s, a);
    }
}

// c.rp: the kernel's own row pass, for rows of up to 8192 values (four
// 16-byte vectors per thread); not for the E4M3 path, whose A side is the
// quantisation pass's codes
template <int ACT, int WQ, int MF, int NR, int U, int KH = 1>
inline hipError_t launch_stream_cfg(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    if (c.rp) {
        if constexpr (WQ != 4) return launch_stream_epi<ACT, WQ, MF, NR, U, KH, 4>(a.epi, a, grid, s);
        return hipErrorInvalidValue;
    }
    return launch_stream_epi<ACT, WQ, MF, NR, U, KH, 0>(a.epi, a, grid, s);
}

// 64 token rows: 128-wide K chunks (two activation / weight register sets of
// 256-wide chunks do not fit in the register file next to the accumulators)
// Weight rows per workgroup: 64 (NR = 1) only for 16-bit and E4M3 weights at
// up to 32 tokens, 256 (NR = 4) only for quantised weights; 32 (NR = 1 with
// K halves, chunks twice as wide so that a wave's loads per chunk stay the
// same) for 16-bit and E4M3 weights at up to 32 tokens; only those
// combinations are instantiated.
template <int ACT, int WQ, int MF>
inline hipError_t launch_stream_mf(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    constexpr int U = MF >= 4 ? 4 : 8;
    if (c.kh == 2) {
        if constexpr ((WQ == 0 || WQ == 4) && MF <= 2)
            if (c.nr == 1) return launch_stream_cfg<ACT, WQ, MF, 1, 2 * U, 2>(c, a, grid, s);
        return hipErrorInvalidValue;
    }
    if (c.nr == 2) return launch_stream_cfg<ACT, WQ, MF, 2, U>(c, a, grid, s);
    if (c.nr == 1) {
        if constexpr ((WQ == 0 || WQ == 4) && MF <= 2) return launch_stream_cfg<ACT, WQ, MF, 1, U>(c, a, grid, s);
        return hipErrorInvalidValue;
    }
    if constexpr (WQ != 0) return launch_stream_cfg<ACT, WQ, MF, 4, U>(c, a, grid, s);   // 256 rows share one A tile
    return hipErrorInvalidValue;
}

template <int ACT, int WQ>
inline hipError_t launch_stream_t(const StreamCfg &c, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (c.mf) {
    case 1: return launch_stream_mf<ACT, WQ, 1>(c, a, grid, s);
    case 2: return launch_stream_mf<ACT, WQ, 2>(c, a, grid, s);
    default: return launch_stream_mf<ACT, WQ, 4>(c, a, grid, s);
    }
}

}  // namespace fp
