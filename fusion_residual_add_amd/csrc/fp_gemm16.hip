// 16-bit prefill projection kernel of libfusedproj (gfx950): the product of
// the normalised activation rows with bf16 / f16 weights at token counts
// where the projection is bound by the matrix cores (the pages' prefill
// regime, "TensorRT-LLM 深度工程实践…", §3.1), then the epilogues of §2.3
// (GQA split, SwiGLU, tanh-GELU, the down projection's residual add).
//
// The normalised rows come from the row pass (norm_kernel), which forms h,
// the statistics and the rounded row once per token and writes it; this
// kernel reads it like a weight.  Forming the row inside the GEMM instead
// (the 128 x 512 kernel) re-reads x and the residual, two 16-bit operands,
// for every column tile and spends VALU work per MFMA: at prefill sizes the
// bytes each CU pulls per K step, not the MFMAs, set that kernel's rate, and
// one extra write and read of the [M, K] rows costs far less.
//
// One workgroup computes a 256 (tokens) x 256 (weight rows) tile with 4
// waves in a 2 x 2 layout, each wave 4 x 4 fragments of
// v_mfma_f32_32x32x16 with its 256 fp32 accumulators in AGPRs (one
// workgroup per CU).  K advances 32 per step through NST LDS stages of A and
// B (16 KB each), both filled straight from HBM / L2 (buffer_load ... lds,
// 16 bytes per lane, one 1 KB wave instruction = 16 rows x 64 bytes; 16-byte
// chunks XOR-swizzled by row so that a fragment read spreads over the
// banks).  The loads of a stage are issued NST - 1 steps before its
// MFMAs, so NST - 2 stages (64 or 96 KB per CU) are in flight while one is
// computed.  One workgroup barrier per step, in the middle of its MFMAs:
// before it, the MFMAs of the first K half run while the second half's
// fragments are read and the loads of a later stage are issued; after it
// (the next stage has landed for every wave), the second half's MFMAs run
// while the next step's first fragments are read.
// For SwiGLU the weight rows of a tile are 128 gate rows and the 128
// matching up rows, and each wave holds gate and up fragments of the same
// columns, so SiLU(g) * u is formed in registers.
#include "fp_device.hpp"

#include <cstdio>

namespace fp {

namespace g16 {
constexpr int BM = 256, BN = 256, BK = 32;
constexpr int ROWB = BK * 2;          // bytes of a tile row per stage
constexpr int TILE = 256 * ROWB;      // 16 KB per operand and stage
constexpr int STAGE = 2 * TILE;       // A, then B
// swizzled byte offset of 16-byte chunk c (0..3) of tile row r: the 8 rows
// one group of 8 lanes reads at a time land in 8 distinct 16-byte bank slots
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 1) & 3)) << 4); }
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char *lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
#else
    (void)r, (void)lds, (void)voff, (void)soff;
#endif
}
}  // namespace g16

template <int ACT, int EPI, int NST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm16_kernel(ProjArgs p) {
    using T = Act<ACT>;
    using namespace g16;
    constexpr bool SW = EPI == EPI_SWIGLU;
    static_assert(ACT != ACT_F32, "16-bit operands");
    static_assert(NST == 4 || NST == 5, "four or five stages (the epilogue stages one wave per stage buffer)");
    static_assert(NST * STAGE <= 160 * 1024, "LDS");
    // the stages as distinct LDS objects, so that the compiler can tell the
    // loads into one stage from the fragment reads of another
    __shared__ __attribute__((aligned(16))) unsigned char s0[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char s1[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char s2[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char s3[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char s4[NST == 5 ? STAGE : 16];
    unsigned char *const bufs[5] = {s0, s1, s2, s3, s4};

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 1, wn = wave >> 1;

    // ---- tile: XCD-aware remap, then grouped raster (8 row tiles per group)
    const int logical = xcd_remap(blockIdx.x, gridDim.x);
    int tm, tn;
    {
        constexpr int GROUP_M = 8;
        const int group = GROUP_M * p.tiles_n;
        const int gid = logical / group, first = gid * GROUP_M;
        const int gsz = min(p.tiles_m - first, GROUP_M);
        const int in = logical % group;
        tm = first + in % gsz;
        tn = in / gsz;
    }
    const int KT = (int)(p.K / BK);

    // ---- loads: wave w fills tile rows [64 w, 64 w + 64) of A and of B
    // with 4 instructions each; lane l of instruction i covers row
    // 64 w + 16 i + l / 4 at LDS chunk position l % 4, which holds the row's
    // global chunk (l % 4) ^ swizzle(row) = (l % 4) ^ ((l / 8) % 4).  Rows
    // past the operand are clamped to its last row (they only feed outputs
    // that are not stored), so every offset stays inside the operand and
    // below 2^32 (checked by the host).
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, (short)0,
                                                                        (uint32_t)(p.M * p.K * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)p.w, (short)0,
                                                                        (uint32_t)(p.Nw * p.K * 2), 0x00020000);
    const int gc = (lane & 3) ^ ((lane >> 3) & 3);
    uint32_t a_off[4], b_off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 64 * wave + 16 * i + (lane >> 2);
        int64_t ma = (int64_t)tm * BM + r;
        ma = ma < p.M ? ma : p.M - 1;
        a_off[i] = (uint32_t)(ma * p.K * 2) + gc * 16;
        int64_t wr;
        if constexpr (SW) wr = r < BN / 2 ? (int64_t)tn * (BN / 2) + r : p.F + (int64_t)tn * (BN / 2) + (r - BN / 2);
        else wr = (int64_t)tn * BN + r;
        wr = wr < p.Nw ? wr : p.Nw - 1;
        b_off[i] = (uint32_t)(wr * p.K * 2) + gc * 16;
    }
    auto issue = [&](int kt, unsigned char *st) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)kt * ROWB;
#pragma unroll
        for (int i = 0; i < 4; ++i) load_lds16(ra, st + (4 * wave + i) * 1024, a_off[i], soff);
#pragma unroll
        for (int i = 0; i < 4; ++i) load_lds16(rw, st + TILE + (4 * wave + i) * 1024, b_off[i], soff);
    };

    // ---- fragments: A rows 128 wm + 32 f + l % 32; B tile rows: SwiGLU the
    // gate blocks 64 wn + 32 f (f < 2) and the matching up blocks
    // 128 + 64 wn + 32 (f - 2), otherwise 128 wn + 32 f.  Lane l supplies k
    // 16 h + 8 (l / 32) .. + 7 of K half h: chunk 2 h + l / 32 of the row, the
    // same on both sides.  Every fragment row is l % 32 past a multiple of
    // 32, so its swizzle depends on the lane alone: one lane offset per
    // operand and K half, the rest a constant in the instruction.
    const int fr = lane & 31, kh = lane >> 5;
    const int lsw = (fr >> 1) & 3;
    const int va0 = 128 * wm * ROWB + fr * ROWB + ((kh ^ lsw) << 4);
    const int va1 = 128 * wm * ROWB + fr * ROWB + (((2 + kh) ^ lsw) << 4);
    const int wnb = (SW ? 64 : 128) * wn * ROWB;
    const int vb0 = TILE + wnb + fr * ROWB + ((kh ^ lsw) << 4);
    const int vb1 = TILE + wnb + fr * ROWB + (((2 + kh) ^ lsw) << 4);
    auto frag_a = [&](const unsigned char *st, int f, int h) __attribute__((always_inline)) {
        return *(const u32x4 *)(st + (h ? va1 : va0) + f * 32 * ROWB);
    };
    auto frag_b = [&](const unsigned char *st, int f, int h) __attribute__((always_inline)) {
        const int rb = SW ? (f < 2 ? 32 * f : BN / 2 + 32 * (f - 2)) : 32 * f;
        return *(const u32x4 *)(st + (h ? vb1 : vb0) + rb * ROWB);
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // Waits for this wave's loads of every stage but the NST - 2 issued
    // last, and for its LDS reads; then a workgroup barrier.  The empty asm
    // statements keep the compiler from moving memory accesses across it.
    auto sync_stage = [&]() __attribute__((always_inline)) {
        constexpr int VM = (NST - 2) * 8;
        __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8));
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
    };

    u32x4 af0[4], bf0[4];   // K half 0 of the current step
    // one K step on stage `cur`: `nxt` holds the next step's stage, `fill`
    // receives the loads of step kt + NST - 1 (past the end: a harmless
    // reload of the last step, never read)
    auto step = [&](const unsigned char *cur, const unsigned char *nxt, unsigned char *fill, int kt,
                    int kt1) __attribute__((always_inline)) {
        u32x4 af1[4], bf1[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            af1[f] = frag_a(cur, f, 1);
            bf1[f] = frag_b(cur, f, 1);
        }
        issue(kt + NST - 1 < kt1 ? kt + NST - 1 : kt1 - 1, fill);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = T::mfma32(af0[i], bf0[j], acc[i][j]);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
            if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // a fragment read
            else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // a stage load
        }
        __builtin_amdgcn_sched_barrier(0);
        sync_stage();
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            af0[f] = frag_a(nxt, f, 0);
            bf0[f] = frag_b(nxt, f, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = T::mfma32(af1[i], bf1[j], acc[i][j]);
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    if (KT > 0) {
        // prologue: stages 0 .. NST - 2 in flight, wait for the first
#pragma unroll
        for (int j = 0; j < NST - 1; ++j) issue(j < KT ? j : KT - 1, bufs[j]);
        sync_stage();
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            af0[f] = frag_a(bufs[0], f, 0);
            bf0[f] = frag_b(bufs[0], f, 0);
        }
        // step kt uses stage buffer kt % NST, a compile-time index in the
        // unrolled body: whole rounds of NST steps, then the remaining ones
        int kb = 0;
        for (; kb + NST <= KT; kb += NST) {
#pragma unroll
            for (int j = 0; j < NST; ++j) step(bufs[j], bufs[(j + 1) % NST], bufs[(j + NST - 1) % NST], kb + j, KT);
        }
#pragma unroll
        for (int j = 0; j < NST - 1; ++j)
            if (kb + j < KT) step(bufs[j], bufs[(j + 1) % NST], bufs[(j + NST - 1) % NST], kb + j, KT);
        // every load has landed before the epilogue reuses the stages
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- epilogue: bias, activation; staged per wave through its own stage
    // buffer in [row][col] order (rows padded by 32 bytes), then stored as
    // runs of 8 columns
    constexpr int OUTC = SW ? 64 : 128;   // output columns per wave
    constexpr int NJ = SW ? 2 : 4;        // output fragments per wave
    constexpr int SROW = OUTC * 4 + 32;   // staging row pitch, bytes
    static_assert(32 * SROW <= STAGE, "staging fits a stage buffer");
    unsigned char *stg = wave == 0 ? s0 : wave == 1 ? s1 : wave == 2 ? s2 : s3;
    const int64_t col0 = SW ? (int64_t)tn * (BN / 2) + OUTC * wn : (int64_t)tn * BN + OUTC * wn;
    const int64_t ncols = SW ? p.F : p.Nw;
    float cb[4];   // bias of this lane's columns (SwiGLU: gate, gate, up, up), zero when absent
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int jo = SW ? (j & 1) : j;
        int64_t c = col0 + 32 * jo + fr;
        c = c < ncols ? c : ncols - 1;
        const int64_t cw = SW && j >= 2 ? c + p.F : c;
        cb[j] = p.bias ? T::ld(p.bias, cw) : 0.f;
    }
    const bool of32 = p.out_f32 != 0;
    const int esz = of32 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t mrow0 = (int64_t)tm * BM + 128 * wm + 32 * i;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int rl = 8 * (q >> 2) + 4 * kh + (q & 3);   // 0..31
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                float y;
                if constexpr (SW) {
                    y = silu(acc[i][j][q] + cb[j]) * (acc[i][j + 2][q] + cb[j + 2]);
                } else {
                    y = acc[i][j][q] + cb[j];
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

template <int ACT, int NST>
static hipError_t launch_gemm16_t(const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (a.epi) {
    case EPI_QKV:    return launch_k(gemm16_kernel<ACT, EPI_QKV, NST>, grid, s, a);
    case EPI_SWIGLU: return launch_k(gemm16_kernel<ACT, EPI_SWIGLU, NST>, grid, s, a);
    case EPI_GELU:   return launch_k(gemm16_kernel<ACT, EPI_GELU, NST>, grid, s, a);
    default:         return launch_k(gemm16_kernel<ACT, EPI_LINEAR, NST>, grid, s, a);
    }
}

hipError_t launch_gemm16(int act, int nst, const ProjArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)((int64_t)a.tiles_m * a.tiles_n);
    if (grid == 0) return hipSuccess;
    if (act == ACT_F16) return nst == 5 ? launch_gemm16_t<ACT_F16, 5>(a, grid, s) : launch_gemm16_t<ACT_F16, 4>(a, grid, s);
    return nst == 5 ? launch_gemm16_t<ACT_BF16, 5>(a, grid, s) : launch_gemm16_t<ACT_BF16, 4>(a, grid, s);
}

const char *gemm16_kernel_name(int act, int nst, int epi) {
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    static thread_local char buf[64];
    snprintf(buf, sizeof buf, "gemm16_kernel<%s,256x256,%dst,%s>", act == ACT_F16 ? "f16" : "bf16", nst == 5 ? 5 : 4,
             epis[epi & 3]);
    return buf;
}

}  // namespace fp
