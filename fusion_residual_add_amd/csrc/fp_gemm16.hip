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
// Tile-packed weights (PK): the B tile of a stage is the stage's 64-byte K
// slices of the tile's 16-row blocks, 1 KB each and contiguous in the
// weight, so one wave load copies one of them as it is and the B tile keeps
// the packed order in LDS (block, slice, 16-byte group, row): the 16 lanes of
// a fragment read (16 rows, one 16-byte group) then read 256 contiguous
// bytes, no swizzle needed.  (Loading the packed weight into the row-major
// tile instead makes each load gather 16-byte pieces: measured 37 % slower
// on Llama-2-7B prefill, at the same L2 request count.)
#include "fp_device.hpp"

#include <cstdio>
#include <type_traits>

namespace fp {

namespace g16 {
constexpr int BM = 256, BN = 256;
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char *lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
#else
    (void)r, (void)lds, (void)voff, (void)soff;
#endif
}
// Stage geometry by stage count: two stages of K 64 (128-byte tile rows,
// one cache line each) or four / five stages of K 32 (64-byte rows).
template <int NST> struct Geo {
    static constexpr int BK = NST == 2 ? 64 : 32;
    static constexpr int ROWB = BK * 2;            // bytes of a tile row per stage
    static constexpr int CH = ROWB / 16;           // 16-byte chunks per row
    static constexpr int TILE = 256 * ROWB;        // bytes per operand and stage
    static constexpr int STAGE = 2 * TILE;         // A, then B
    static constexpr int RPI = 1024 / ROWB;        // tile rows per 1 KB wave load
    static constexpr int NI = 64 / RPI;            // loads per wave, operand and stage
    static constexpr int KS = BK / 16;             // MFMA K substeps per stage
    // LDS position of chunk c of tile row r is c ^ swz(r).  gfx950's LDS
    // serves a 16-byte-per-lane read 16 lanes at a time from 64 banks (256
    // bytes); the 16 consecutive rows those lanes read (same chunk) must land
    // on 16 distinct 16-byte bank slots.  128-byte rows: row r starts at slot
    // 8 (r % 2), and (r / 2) % 8 spreads each parity over the 8 chunks.
    // 64-byte rows: row r starts at slot 4 (r % 4), and (r / 4) % 4 spreads
    // each residue over the 4 chunks.
    __device__ static int swz(int r) { return NST == 2 ? (r >> 1) & 7 : (r >> 2) & 3; }
};
}  // namespace g16

template <int ACT, int EPI, int NST, bool PK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm16_kernel(ProjArgs p) {
    using T = Act<ACT>;
    using namespace g16;
    using G = Geo<NST>;
    constexpr int ROWB = G::ROWB, TILE = G::TILE, STAGE = G::STAGE, NI = G::NI, RPI = G::RPI, KS = G::KS;
    constexpr int SPS = ROWB / 64;   // packed B: 64-byte K slices per stage
    constexpr bool SW = EPI == EPI_SWIGLU;
    static_assert(ACT != ACT_F32, "16-bit operands");
    static_assert(NST == 2 || NST == 4 || NST == 5, "two stages of K 64 (an even number of them), or four / five of K 32");
    static_assert(NST * STAGE <= 160 * 1024, "LDS");
    // the stages as distinct LDS objects, so that the compiler can tell the
    // loads into one stage from the fragment reads of another
    __shared__ __attribute__((aligned(16))) unsigned char s0[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char s1[STAGE];
    __shared__ __attribute__((aligned(16))) unsigned char s2[NST >= 4 ? STAGE : 16];
    __shared__ __attribute__((aligned(16))) unsigned char s3[NST >= 4 ? STAGE : 16];
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
    const int KT = (int)(p.K / G::BK);

    // ---- loads: wave w fills tile rows [64 w, 64 w + 64) of A and of B
    // with NI instructions each; lane l of instruction i covers row
    // r = 64 w + RPI i + l / CH at LDS chunk position l % CH, which holds the
    // row's global chunk (l % CH) ^ swz(r).  Rows past the operand are
    // clamped to its last row (they only feed outputs that are not stored),
    // so every offset stays inside the operand and below 2^32 (checked by
    // the host).
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, (short)0,
                                                                        (uint32_t)(p.M * p.K * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void *)p.w, (short)0,
                                                                        (uint32_t)(p.Nw * p.K * 2), 0x00020000);
    uint32_t a_off[NI], b_off[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int r = 64 * wave + RPI * i + lane / G::CH;
        const int gc = (lane % G::CH) ^ G::swz(r);
        int64_t ma = (int64_t)tm * BM + r;
        ma = ma < p.M ? ma : p.M - 1;
        a_off[i] = (uint32_t)(ma * p.K * 2) + gc * 16;
        int64_t wr;
        if constexpr (PK) {
            // instruction i of wave w: block slice q = NI w + i of the stage
            // (16-row block q / SPS of the tile, slice q % SPS); a block past
            // the weight reads its last block (packed weights have whole
            // 128-row groups, so blocks are whole)
            const int q = NI * wave + i, br = 16 * (q / SPS);
            if constexpr (SW) wr = br < BN / 2 ? (int64_t)tn * (BN / 2) + br : p.F + (int64_t)tn * (BN / 2) + (br - BN / 2);
            else wr = (int64_t)tn * BN + br;
            wr = wr < p.Nw ? wr : p.Nw - 16;
            b_off[i] = (uint32_t)(packed_row_off(wr, p.F, p.K * 2, p.w_layout) + (q % SPS) * 8192) + lane * 16;
        } else {
            if constexpr (SW) wr = r < BN / 2 ? (int64_t)tn * (BN / 2) + r : p.F + (int64_t)tn * (BN / 2) + (r - BN / 2);
            else wr = (int64_t)tn * BN + r;
            wr = wr < p.Nw ? wr : p.Nw - 1;
            b_off[i] = (uint32_t)weight_off(p.w_layout, wr, gc * 16, p.F, p.K * 2);
        }
    }
    // stage kt: row bytes kt * ROWB of both operands, added as the scalar
    // offset (tile-packed weights: that byte's offset in the packed layout,
    // additive since ROWB is a multiple of 64)
    auto issue = [&](int kt, unsigned char *st) __attribute__((always_inline)) {
        const uint32_t soff = (uint32_t)kt * ROWB;
        const uint32_t wsoff = PK || p.w_layout ? (uint32_t)packed_col_off(soff) : soff;
#pragma unroll
        for (int i = 0; i < NI; ++i) load_lds16(ra, st + (NI * wave + i) * 1024, a_off[i], soff);
#pragma unroll
        for (int i = 0; i < NI; ++i) load_lds16(rw, st + TILE + (NI * wave + i) * 1024, b_off[i], wsoff);
    };

    // ---- fragments: A rows 128 wm + 32 f + l % 32; B tile rows: SwiGLU the
    // gate blocks 64 wn + 32 f (f < 2) and the matching up blocks
    // 128 + 64 wn + 32 (f - 2), otherwise 128 wn + 32 f.  Lane l supplies k
    // 16 t + 8 (l / 32) .. + 7 of K substep t: chunk 2 t + l / 32 of the row,
    // the same on both sides.  Every fragment row is l % 32 past a multiple
    // of 32, so its swizzle depends on the lane alone: one lane offset per
    // operand and substep, the rest a constant in the instruction.
    const int fr = lane & 31, kh = lane >> 5;
    const int lsw = G::swz(fr);
    const int wnb = (SW ? 64 : 128) * wn * ROWB;
    int va[KS], vb[KS];
#pragma unroll
    for (int t = 0; t < KS; ++t) {
        va[t] = 128 * wm * ROWB + fr * ROWB + (((2 * t + kh) ^ lsw) << 4);
        if constexpr (PK) {
            // packed B tile: tile row R, 16-byte chunk c at
            // ((R / 16) SPS + c / 4) KB + 256 (c % 4) + 16 (R % 16)
            const int c = 2 * t + kh, rw = (SW ? 64 : 128) * wn + fr;
            vb[t] = TILE + (((rw >> 4) * SPS + (c >> 2)) << 10) + ((c & 3) << 8) + ((fr & 15) << 4);
        } else {
            vb[t] = TILE + wnb + fr * ROWB + (((2 * t + kh) ^ lsw) << 4);
        }
    }
    auto frag_a = [&](const unsigned char *st, int f, int t) __attribute__((always_inline)) {
        return *(const u32x4 *)(st + va[t] + f * 32 * ROWB);
    };
    auto frag_b = [&](const unsigned char *st, int f, int t) __attribute__((always_inline)) {
        const int rb = SW ? (f < 2 ? 32 * f : BN / 2 + 32 * (f - 2)) : 32 * f;
        // rb is a multiple of 32: whole 16-row blocks either way
        return *(const u32x4 *)(st + vb[t] + (PK ? (rb >> 4) * SPS * 1024 : rb * ROWB));
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // Waits until this wave's loads of every stage but the VM / NI / 2 issued
    // last have landed, and for its LDS reads; then a workgroup barrier.  The
    // empty asm statements keep the compiler from moving memory accesses
    // across it.
    auto sync_stage = [&](auto vm) __attribute__((always_inline)) {
        constexpr int VM = decltype(vm)::value;
        __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8));
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
    };
    auto mfma_sub = [&](const u32x4 (&af)[4], const u32x4 (&bf)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = T::mfma32(af[i], bf[j], acc[i][j]);
    };
    auto read_sub = [&](const unsigned char *st, int t, u32x4 (&af)[4], u32x4 (&bf)[4]) __attribute__((always_inline)) {
        // A fragment 0 and the B fragments first: the first MFMAs need them
        af[0] = frag_a(st, 0, t);
#pragma unroll
        for (int f = 0; f < 4; ++f) bf[f] = frag_b(st, f, t);
#pragma unroll
        for (int f = 1; f < 4; ++f) af[f] = frag_a(st, f, t);
    };

    if constexpr (NST == 2) {
        // Two stages of K 64, four substeps each.  Step kt on stage `cur`:
        // substeps 0..2, each one's MFMAs overlapping the next one's fragment
        // reads; then the wait for stage kt + 1 (issued one step earlier) and
        // a barrier, after which every wave is done with `cur` and the loads
        // of step kt + 2 go into it (past the end: a harmless reload of the
        // last step, never read); then substep 3's MFMAs overlap the reads of
        // the next step's substep-0 fragments.  A load thus has a whole step
        // to arrive, and no MFMA waits on a fragment read after the barrier.
        u32x4 af[2][4], bf[2][4];   // fragment sets of alternating substeps
        auto step = [&](const unsigned char *cur, unsigned char *cur_w, const unsigned char *nxt, int kt)
            __attribute__((always_inline)) {
#pragma unroll
            for (int t = 0; t < KS - 1; ++t) {
                read_sub(cur, t + 1, af[(t + 1) & 1], bf[(t + 1) & 1]);
                mfma_sub(af[t & 1], bf[t & 1]);
#pragma unroll
                for (int m = 0; m < 16; ++m) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                // one MFMA
                    if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // a fragment read
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            sync_stage(std::integral_constant<int, 0>{});
            issue(kt + 2 < KT ? kt + 2 : KT - 1, cur_w);
            read_sub(nxt, 0, af[0], bf[0]);
            mfma_sub(af[1], bf[1]);
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                    // a stage load
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // K steps in pairs, each stage a fixed LDS object (the host takes
        // this form only for an even step count): with the stage chosen at
        // run time the compiler could not tell one step's loads from the
        // next step's reads and would wait for every load at each step.
        if (KT > 0) {
            issue(0, s0);
            issue(1, s1);
            sync_stage(std::integral_constant<int, 2 * NI>{});
            read_sub(s0, 0, af[0], bf[0]);
            for (int kt = 0; kt < KT; kt += 2) {
                step(s0, s0, s1, kt);
                step(s1, s1, s0, kt + 1);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    } else {
        // Four / five stages of K 32.  Step kt on stage buffer kt % NST:
        // before the barrier, the MFMAs of substep 0 run while substep 1's
        // fragments are read and the loads of step kt + NST - 1 are issued
        // (into the buffer of step kt - 1, which every wave finished reading
        // before the previous barrier; past the end: a harmless reload of the
        // last step, never read); the barrier follows the wait for stage
        // kt + 1 (every load but the NST - 2 stages issued after it); after
        // it, substep 1's MFMAs run while the next step's substep-0 fragments
        // are read.
        u32x4 af0[4], bf0[4];
        auto step = [&](const unsigned char *cur, const unsigned char *nxt, unsigned char *fill, int kt)
            __attribute__((always_inline)) {
            u32x4 af1[4], bf1[4];
            read_sub(cur, 1, af1, bf1);
            issue(kt + NST - 1 < KT ? kt + NST - 1 : KT - 1, fill);
            mfma_sub(af0, bf0);
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
                if (m < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // a fragment read
                else __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         // a stage load
            }
            __builtin_amdgcn_sched_barrier(0);
            sync_stage(std::integral_constant<int, (NST - 2) * 2 * NI>{});
            read_sub(nxt, 0, af0, bf0);
            mfma_sub(af1, bf1);
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
            sync_stage(std::integral_constant<int, (NST - 2) * 2 * NI>{});
            read_sub(bufs[0], 0, af0, bf0);
            // step kt uses stage buffer kt % NST, a compile-time index in the
            // unrolled body: whole rounds of NST steps, then the remaining ones
            int kb = 0;
            for (; kb + NST <= KT; kb += NST) {
#pragma unroll
                for (int j = 0; j < NST; ++j) step(bufs[j], bufs[(j + 1) % NST], bufs[(j + NST - 1) % NST], kb + j);
            }
#pragma unroll
            for (int j = 0; j < NST - 1; ++j)
                if (kb + j < KT) step(bufs[j], bufs[(j + 1) % NST], bufs[(j + NST - 1) % NST], kb + j);
            // every load has landed before the epilogue reuses the stages
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // ---- epilogue: bias, activation; staged per wave through its own stage
    // buffer in [row][col] order (rows padded by 32 bytes), then stored as
    // runs of 8 columns
    constexpr int OUTC = SW ? 64 : 128;   // output columns per wave
    constexpr int NJ = SW ? 2 : 4;        // output fragments per wave
    constexpr int SROW = OUTC * 4 + 32;   // staging row pitch, bytes
    // each wave stages in a stage buffer of its own (four / five stages) or
    // in half of one (two stages of twice the size)
    static_assert(32 * SROW <= (NST == 2 ? STAGE / 2 : STAGE), "staging fits");
    unsigned char *stg = NST == 2 ? (wave < 2 ? s0 : s1) + (wave & 1) * (STAGE / 2)
                                  : wave == 0 ? s0 : wave == 1 ? s1 : wave == 2 ? s2 : s3;
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

template <int ACT, int NST, bool PK>
static hipError_t launch_gemm16_e(const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (a.epi) {
    case EPI_QKV:    return launch_k(gemm16_kernel<ACT, EPI_QKV, NST, PK>, grid, s, a);
    case EPI_SWIGLU: return launch_k(gemm16_kernel<ACT, EPI_SWIGLU, NST, PK>, grid, s, a);
    case EPI_GELU:   return launch_k(gemm16_kernel<ACT, EPI_GELU, NST, PK>, grid, s, a);
    default:         return launch_k(gemm16_kernel<ACT, EPI_LINEAR, NST, PK>, grid, s, a);
    }
}

template <int ACT, int NST>
static hipError_t launch_gemm16_t(const ProjArgs &a, unsigned grid, hipStream_t s) {
    return a.w_layout ? launch_gemm16_e<ACT, NST, true>(a, grid, s) : launch_gemm16_e<ACT, NST, false>(a, grid, s);
}

hipError_t launch_gemm16(int act, int nst, const ProjArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)((int64_t)a.tiles_m * a.tiles_n);
    if (grid == 0) return hipSuccess;
    if (act == ACT_F16) {
        if (nst == 2) return launch_gemm16_t<ACT_F16, 2>(a, grid, s);
        return nst == 5 ? launch_gemm16_t<ACT_F16, 5>(a, grid, s) : launch_gemm16_t<ACT_F16, 4>(a, grid, s);
    }
    if (nst == 2) return launch_gemm16_t<ACT_BF16, 2>(a, grid, s);
    return nst == 5 ? launch_gemm16_t<ACT_BF16, 5>(a, grid, s) : launch_gemm16_t<ACT_BF16, 4>(a, grid, s);
}

const char *gemm16_kernel_name(int act, int nst, int epi) {
    static const char *epis[4] = {"qkv", "swiglu", "gelu", "linear"};
    static thread_local char buf[64];
    snprintf(buf, sizeof buf, "gemm16_kernel<%s,256x256,%dst,%s>", act == ACT_F16 ? "f16" : "bf16", nst == 5 ? 5 : nst == 2 ? 2 : 4,
             epis[epi & 3]);
    return buf;
}

}  // namespace fp
