// Tiled projection kernel of libfusedproj (gfx950): prefill-sized token
// counts, and every fp32 call.
//
// One workgroup computes a BM x BN tile of the projection.  Its A-operand
// loader reads x and the residual, re-forms h = x + r, normalises it with the
// row statistics and gamma / beta, rounds to the activation dtype and writes
// the tile to LDS -- the normalised rows never reach memory, which is the
// point of the LayerNorm + QKV fusion ("TensorRT-LLM 深度工程实践…", §2.3).
// Its B-operand loader streams [N, K] weight rows (int8 dequantised to bf16
// on the way).  The main loop is 16x16 MFMA (x32 bf16/f16, x4 f32) with fp32
// accumulation; the epilogue applies the bias and the GQA split, SwiGLU,
// tanh-GELU or nothing.  Optional split-K with a deterministic last-arriver
// reduction.
#include "fp_device.hpp"

#include <cstdio>

namespace fp {

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
                    // fp32(fp32(h - mu) * rstd), then gamma and beta with one
                    // rounding: the order every kernel of the library uses
#pragma unroll
                    for (int e = 0; e < VE; ++e) {
                        const float t = (h[e] - a_mu[i]) * a_rs[i];
                        h[e] = fmaf(t, g[e], has_beta ? be[e] : 0.f);
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

    // ---- split-K: the last split to arrive reduces the partials
    if (p.splits > 1) {
        float flat[FM * FN * 4];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) flat[(i * FN + j) * 4 + e] = acc[i][j][e];
        if (!splitk_reduce(p, tile, z, p.splits, flat)) return;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] = flat[(i * FN + j) * 4 + e];
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
                    if (c < p.F) store_swiglu<ACT>(p, m, c, acc[i][j][e], acc[i][j + 1][e]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int64_t c = (int64_t)tn * BN + wn * WTN + j * 16 + (lane & 15);
                    if (c >= p.Nw) continue;
                    float y = acc[i][j][e];
                    if (p.bias) y += T::ld(p.bias, c);
                    store_col<ACT, EPI>(p, m, c, y);
                }
            }
        }
    }
}

TileShape tile_shape(int cfg) {
    switch (cfg) {
    case TILE_DEC16: return {16, 128, 64};
    case TILE_DEC32: return {32, 128, 64};
    case TILE_DEC64: return {64, 128, 64};
    default:         return {128, 128, 64};
    }
}

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

template <int ACT, bool WI8, int EPI>
static hipError_t launch_proj_e(int tile, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (tile) {
    case TILE_DEC16:
        return launch_k(proj_kernel<ACT, WI8, 16, 128, 64, 1, 4, EPI>, grid, s, a);
    case TILE_DEC32:
        return launch_k(proj_kernel<ACT, WI8, 32, 128, 64, 1, 4, EPI>, grid, s, a);
    case TILE_DEC64:
        return launch_k(proj_kernel<ACT, WI8, 64, 128, 64, 1, 4, EPI>, grid, s, a);
    default:
        return launch_k(proj_kernel<ACT, WI8, 128, 128, 64, 2, 2, EPI>, grid, s, a);
    }
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

hipError_t launch_tiled(int act, bool w_i8, int tile, const ProjArgs &a, hipStream_t s) {
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

}  // namespace fp
