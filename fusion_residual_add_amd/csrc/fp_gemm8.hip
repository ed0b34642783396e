// FP8 (W8A8, E4M3) projection kernel of libfusedproj (gfx950): the product of
// the per-token quantised activation rows (quant8_kernel) with E4M3 weights on
// the double-rate v_mfma_f32_32x32x64_f8f6f4, then the same epilogues as the
// 16-bit kernels ("TensorRT-LLM 深度工程实践…", §3.3: the full-FP8 configuration
// with activation ranges taken online; §2.3 for the epilogues).
//
//   y[m, c] = (sum_k e4m3(a[m, k]) e4m3(w[c, k])) * a_scale[m] * w_scale[c]
//             (+ bias[c]), then the GQA split / SwiGLU / tanh-GELU / residual.
//
// One workgroup computes a (32 FM WGM) tokens x (32 FN WGN) weight rows tile
// with 4 waves in a WGM x WGN layout (WGN = 4 / WGM), each wave FM x FN
// fragments of 32 x 32 with fp32 accumulators: 128 x 128 (2 x 2 waves of
// 2 x 2 fragments; two workgroups per CU, for token counts whose large tiles
// would not fill the chip), 256 x 256 (2 x 2 waves of 4 x 4 fragments; the 256
// accumulators per lane live in AGPRs, one workgroup per CU, half the LDS
// bytes read per MFMA), and for decode token counts 32 x 256 or 64 x 256 (1 x 4
// waves sharing the token rows, so no MFMA work goes to padding rows and most
// of each stage is weights).  For SwiGLU the weight rows of a tile are BN / 2 gate
// rows and the BN / 2 matching up rows, and each wave holds gate and up
// fragments of the same columns, so SiLU(g) * u is formed in registers.  K
// advances 128 codes (128 bytes) per step through two LDS stages of A and B,
// both loaded straight from HBM / L2 into LDS (buffer_load ... lds, 16 bytes
// per lane, 16-byte chunks XOR-swizzled by row).
// The quantised activations are read as 1-byte codes: the per-token scale
// needs the whole normalised row (its amax) before any element is coded, so
// the quantisation runs in the kernel before this one and writes the codes
// once (half the bytes of the 16-bit rows the other kernels re-read per
// column tile).
#include "fp_device.hpp"

#include <cstdio>

namespace fp {

namespace g8 {
constexpr int BK = 128;
// swizzled byte offset of 16-byte chunk c (0..7) of tile row r
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char *lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
#else
    (void)r, (void)lds, (void)voff, (void)soff;
#endif
}
typedef __attribute__((ext_vector_type(8))) int i32x8;
}  // namespace g8

// PK: tile-packed weights.  The B tile of a stage is its 16-row blocks'
// two 64-byte K slices, 1 KB each and contiguous in the weight: one wave
// load copies one as it is, and the tile keeps the packed order in LDS
// (block, slice, 16-byte group, row), where a fragment read of 16 rows of
// one 16-byte group covers 256 contiguous bytes.
template <int ACT, int EPI, int FM, int FN, int WGM, bool PK>
__global__ __launch_bounds__(256, FM * FN >= 16 ? 1 : 2) void gemm8_kernel(ProjArgs p) {
    using T = Act<ACT>;
    using namespace g8;
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr int WGN = 4 / WGM;
    constexpr int BM = 32 * FM * WGM, BN = 32 * FN * WGN;
    constexpr int TILEA = BM * BK, TILEB = BN * BK;
    constexpr int IA = BM / 32, IB = BN / 32;   // load instructions per wave and stage
    static_assert(BM % 32 == 0 && BN % 32 == 0, "whole load instructions per wave");
    static_assert(!SW || FN % 2 == 0, "gate and up fragments in pairs");
    __shared__ __attribute__((aligned(16))) unsigned char lA0[TILEA];
    __shared__ __attribute__((aligned(16))) unsigned char lA1[TILEA];
    __shared__ __attribute__((aligned(16))) unsigned char lB0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char lB1[TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WGM, wn = wave / WGM;

    // ---- tile: XCD-aware remap, then grouped raster (8 row tiles per group)
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

    // ---- loads: wave w fills tile rows [BM/4 w, BM/4 (w + 1)) of A and
    // [BN/4 w, BN/4 (w + 1)) of B with 1 KB instructions (8 rows); lane l of
    // instruction i covers row BM/4 w + 8 i + l / 8 at LDS chunk position
    // l % 8, which holds the row's global chunk (l % 8) ^ (row % 8).  Rows past
    // the operand are clamped to its last row (they only feed outputs that are
    // not stored), so every offset stays inside the operand and below 2^32
    // (checked by the host).
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, (short)0,
                                                                        (uint32_t)(p.M * p.K), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)p.w, (short)0,
                                                                        (uint32_t)(p.Nw * p.K), 0x00020000);
    uint32_t a_off[IA], b_off[IB];
#pragma unroll
    for (int i = 0; i < IA; ++i) {
        const int r = (BM / 4) * wave + 8 * i + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        int64_t ma = (int64_t)tm * BM + r;
        ma = ma < p.M ? ma : p.M - 1;
        a_off[i] = (uint32_t)(ma * p.K) + c * 16;
    }
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        int64_t wr;
        if constexpr (PK) {
            // block slice q = IB w + i of the stage: block q / 2 of the tile,
            // slice q % 2 (a block past the weight reads its last block)
            const int q = IB * wave + i, br = 16 * (q >> 1);
            if constexpr (SW) wr = br < BN / 2 ? (int64_t)tn * (BN / 2) + br : p.F + (int64_t)tn * (BN / 2) + (br - BN / 2);
            else wr = (int64_t)tn * BN + br;
            wr = wr < p.Nw ? wr : p.Nw - 16;
            b_off[i] = (uint32_t)(packed_row_off(wr, p.F, p.K, p.w_layout) + (q & 1) * 8192) + lane * 16;
        } else {
            const int r = (BN / 4) * wave + 8 * i + (lane >> 3);
            const int c = (lane & 7) ^ (r & 7);
            if constexpr (SW) wr = r < BN / 2 ? (int64_t)tn * (BN / 2) + r : p.F + (int64_t)tn * (BN / 2) + (r - BN / 2);
            else wr = (int64_t)tn * BN + r;
            wr = wr < p.Nw ? wr : p.Nw - 1;
            b_off[i] = (uint32_t)weight_off(p.w_layout, wr, c * 16, p.F, p.K);
        }
    }
    // stage kt: row bytes kt * BK, the scalar offset (tile-packed weights:
    // that byte's packed offset, additive since BK is a multiple of 64)
    auto issue = [&](int kt, unsigned char *la, unsigned char *lb) {
        const uint32_t soff = (uint32_t)kt * BK;
        const uint32_t wsoff = PK || p.w_layout ? (uint32_t)packed_col_off(soff) : soff;
#pragma unroll
        for (int i = 0; i < IA; ++i) load_lds16(ra, la + (IA * wave + i) * 1024, a_off[i], soff);
#pragma unroll
        for (int i = 0; i < IB; ++i) load_lds16(rw, lb + (IB * wave + i) * 1024, b_off[i], wsoff);
    };

    // ---- fragments: A rows 32 (FM wm + f) + l % 32; B tile rows: SwiGLU the
    // gate blocks 32 (FN/2 wn + f) for f < FN/2 and the matching up blocks
    // BN/2 + 32 (FN/2 wn + f - FN/2), otherwise 32 (FN wn + f).  Lane l
    // supplies k [64 kb + 32 (l / 32), +32) of K sub-step kb as two 16-byte
    // chunks (A and B alike, so the k order inside the operand is the same on
    // both sides).
    const int fr = lane & 31, kh = lane >> 5;
    int arow[FM], brow[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) arow[f] = 32 * (FM * wm + f) + fr;
#pragma unroll
    for (int f = 0; f < FN; ++f)
        brow[f] = SW ? (f < FN / 2 ? 32 * (FN / 2 * wn + f) : BN / 2 + 32 * (FN / 2 * wn + f - FN / 2)) + fr
                     : 32 * (FN * wn + f) + fr;
    auto frag = [&](const unsigned char *l, int row, int kb) -> i32x8 {
        const int c = 4 * kb + 2 * kh;
        const u32x4 lo = *(const u32x4 *)(l + swz(row, c));
        const u32x4 hi = *(const u32x4 *)(l + swz(row, c + 1));
        return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    // packed B tile: chunks c (even) and c + 1 of tile row `row` sit in slice
    // c / 4 of its block, 16-byte groups c % 4 and c % 4 + 1
    auto frag_pk = [&](const unsigned char *l, int row, int kb) -> i32x8 {
        const int c = 4 * kb + 2 * kh;
        const unsigned char *b = l + ((((row >> 4) * 2 + (c >> 2)) << 10) + ((c & 3) << 8) + ((row & 15) << 4));
        const u32x4 lo = *(const u32x4 *)b;
        const u32x4 hi = *(const u32x4 *)(b + 256);
        return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    auto compute = [&](const unsigned char *la, const unsigned char *lb) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            i32x8 af[FM], bf[FN];
#pragma unroll
            for (int f = 0; f < FM; ++f) af[f] = frag(la, arow[f], kb);
#pragma unroll
            for (int f = 0; f < FN; ++f) bf[f] = PK ? frag_pk(lb, brow[f], kb) : frag(lb, brow[f], kb);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)   // formats: 0 = E4M3 for both operands
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0,
                                                                               0, 0, 0, 0);
        }
    };
    // wait for this wave's loads (the current stage) and LDS reads (the
    // previous step's fragments), then a workgroup barrier: the stage has
    // landed for every wave and every wave is done with the other stage.
    // The empty asm statements keep the compiler from moving memory accesses
    // across the barrier.
    auto step_sync = [&]() {
        __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (0 << 8));
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
    };

    // Stage identity alternates; both pointers of a pair come from one
    // condition, so alias analysis still tells the stages apart and the
    // fragment reads of one stage do not wait for the loads into the other.
    // Each step first loads the next stage (past the end: a harmless reload
    // of the last one, never read), then computes on the current one.
    if (kt0 < kt1) {
        issue(kt0, lA0, lB0);
        for (int kt = kt0; kt < kt1; ++kt) {
            const bool odd = ((kt - kt0) & 1) != 0;
            const unsigned char *ca = odd ? lA1 : lA0, *cb = odd ? lB1 : lB0;
            unsigned char *na = odd ? lA0 : lA1, *nb = odd ? lB0 : lB1;
            step_sync();
            issue(kt + 1 < kt1 ? kt + 1 : kt1 - 1, na, nb);
            compute(ca, cb);
        }
        step_sync();   // the last reload has landed before the epilogue reuses the LDS
    }

    // ---- split K (128 x 128 tiles only): the last contributor of a tile
    // sums the partials in order
    if (FM * FN < 16 && p.splits > 1) {
        static_assert(FM * FN * 16 * 256 == BM * BN || FM * FN >= 16, "one accumulator slot per tile element");
        constexpr int NACC = FM * FN * 16;
        float flat[NACC];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) flat[(i * FN + j) * 16 + e] = acc[i][j][e];
        if (!splitk_reduce<NACC>(p, tile, z, p.splits, flat)) return;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = flat[(i * FN + j) * 16 + e];
    }

    // ---- epilogue: scales, bias, activation; staged per wave through LDS in
    // [row][col] order (rows padded by 32 bytes), then stored as runs of 8
    // columns (16 bytes of 16-bit outputs)
    constexpr int OUTC = SW ? 16 * FN : 32 * FN;   // output columns per wave
    constexpr int NJ = SW ? FN / 2 : FN;            // output fragments per wave
    constexpr int SROW = OUTC * 4 + 32;             // staging row pitch, bytes
    // each wave stages in its own half of a B tile buffer, or, where half of
    // one is too small, in a whole tile buffer of its own
    constexpr bool STG_B = 2 * 32 * SROW <= TILEB;
    static_assert(STG_B || (32 * SROW <= TILEA && 32 * SROW <= TILEB), "staging fits");
    unsigned char *stg = STG_B ? (wave < 2 ? lB0 : lB1) + (wave & 1) * (TILEB / 2)
                               : wave == 0 ? lA0 : wave == 1 ? lA1 : wave == 2 ? lB0 : lB1;
    const int64_t col0 = SW ? (int64_t)tn * (BN / 2) + OUTC * wn : (int64_t)tn * BN + OUTC * wn;
    const int64_t ncols = SW ? p.F : p.Nw;
    // per-column weight scale and bias of this lane (SwiGLU: gate, then up)
    float cs[FN], cb[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int jo = SW ? j % (FN / 2) : j;
        int64_t c = col0 + 32 * jo + fr;
        c = c < ncols ? c : ncols - 1;
        const int64_t cw = SW && j >= FN / 2 ? c + p.F : c;
        cs[j] = p.w_scale[cw];
        cb[j] = p.bias ? T::ld(p.bias, cw) : 0.f;
    }
    const bool of32 = p.out_f32 != 0;
    const int esz = of32 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int64_t mrow0 = (int64_t)tm * BM + 32 * (FM * wm + i);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int rl = 8 * (q >> 2) + 4 * kh + (q & 3);   // 0..31
            const int64_t mr = mrow0 + rl;
            const float as = p.a_scale[mr < p.M ? mr : p.M - 1];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                float y;
                if constexpr (SW) {
                    const float g = acc[i][j][q] * as * cs[j] + cb[j];
                    const float u = acc[i][j + FN / 2][q] * as * cs[j + FN / 2] + cb[j + FN / 2];
                    y = silu(g) * u;
                } else {
                    y = acc[i][j][q] * as * cs[j] + cb[j];
                    if constexpr (EPI == EPI_GELU) y = gelu_tanh(y);
                }
                *(float *)(stg + rl * SROW + (32 * j + fr) * 4) = y;
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0);
        constexpr int RUNS = OUTC / 8;
#pragma unroll
        for (int it = 0; it < 32 * RUNS / 64; ++it) {
            const int idx = it * 64 + lane;
            const int rl = idx / RUNS, ch = idx % RUNS;
            const int64_t m = mrow0 + rl;
            const int64_t cg = col0 + ch * 8;
            const f32x4 v0 = *(const f32x4 *)(stg + rl * SROW + ch * 32);
            const f32x4 v1 = *(const f32x4 *)(stg + rl * SROW + ch * 32 + 16);
            if (m >= p.M || cg >= ncols) continue;
            char *dst;
            if constexpr (EPI == EPI_QKV) {
                if (cg < p.nq)              dst = (char *)p.out0 + qkv_index(p, m, cg, p.nq) * esz;
                else if (cg < p.nq + p.nkv) dst = (char *)p.out1 + qkv_index(p, m, cg - p.nq, p.nkv) * esz;
                else                        dst = (char *)p.out2 + qkv_index(p, m, cg - p.nq - p.nkv, p.nkv) * esz;
            } else {
                dst = (char *)p.out0 + (m * ncols + cg) * esz;
            }
            float y[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            if constexpr (EPI == EPI_LINEAR) {
                if (p.res_epi) {   // the down projection's residual add (this lane reads what it writes)
                    float r[8];
                    T::unpack(*(const u32x4 *)((const char *)p.res_epi + (m * ncols + cg) * 2), r);
#pragma unroll
                    for (int e = 0; e < 8; ++e) y[e] += r[e];
                }
            }
            if (of32) {
                *(f32x4 *)dst = (f32x4){y[0], y[1], y[2], y[3]};
                *(f32x4 *)(dst + 16) = (f32x4){y[4], y[5], y[6], y[7]};
            } else {
                *(u32x4 *)dst = T::pack(y);
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0);
    }
}

template <int ACT, int FM, int FN, int WGM, bool PK>
static hipError_t launch_gemm8_e(const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (a.epi) {
    case EPI_QKV:    return launch_k(gemm8_kernel<ACT, EPI_QKV, FM, FN, WGM, PK>, grid, s, a);
    case EPI_SWIGLU: return launch_k(gemm8_kernel<ACT, EPI_SWIGLU, FM, FN, WGM, PK>, grid, s, a);
    case EPI_GELU:   return launch_k(gemm8_kernel<ACT, EPI_GELU, FM, FN, WGM, PK>, grid, s, a);
    default:         return launch_k(gemm8_kernel<ACT, EPI_LINEAR, FM, FN, WGM, PK>, grid, s, a);
    }
}

template <int ACT, int FM, int FN, int WGM>
static hipError_t launch_gemm8_t(const ProjArgs &a, unsigned grid, hipStream_t s) {
    return a.w_layout ? launch_gemm8_e<ACT, FM, FN, WGM, true>(a, grid, s)
                      : launch_gemm8_e<ACT, FM, FN, WGM, false>(a, grid, s);
}

template <int ACT>
static hipError_t launch_gemm8_v(int tile, const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (tile) {
    case G8_256x256: return launch_gemm8_t<ACT, 4, 4, 2>(a, grid, s);
    case G8_32x256:  return launch_gemm8_t<ACT, 1, 2, 1>(a, grid, s);
    case G8_64x256:  return launch_gemm8_t<ACT, 2, 2, 1>(a, grid, s);
    default:         return launch_gemm8_t<ACT, 2, 2, 2>(a, grid, s);
    }
}

hipError_t launch_gemm8(int act, int tile, const ProjArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)((int64_t)a.tiles_m * a.tiles_n * a.splits);
    if (grid == 0) return hipSuccess;
    if (act == ACT_F16) return launch_gemm8_v<ACT_F16>(tile, a, grid, s);
    return launch_gemm8_v<ACT_BF16>(tile, a, grid, s);
}

const char *gemm8_kernel_name(int act, int tile, int epi) {
    static const char *tiles[4] = {"128x128", "256x256", "32x256", "64x256"};
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    static thread_local char buf[64];
    snprintf(buf, sizeof buf, "gemm8_kernel<%s,%s,%s>", act == ACT_F16 ? "f16" : "bf16", tiles[tile & 3], epis[epi & 3]);
    return buf;
}

}  // namespace fp
