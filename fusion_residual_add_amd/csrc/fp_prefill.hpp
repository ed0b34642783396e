// Prefill projection kernel of libfusedproj (gfx950): token counts where the
// projection is bound by the matrix cores (the pages' prefill regime,
// "TensorRT-LLM 深度工程实践…", §3.1).
//
// One workgroup computes a 128 (tokens) x 512 (weight rows) tile with 4
// waves side by side; each wave a 128 x 128 sub-tile as 4 x 4 fragments of
// v_mfma_f32_32x32x16 (bf16 / f16) with fp32 accumulators (256 per lane, all
// in AGPRs: the 32 x 32 shape keeps them in 16-register tuples that the
// allocator leaves in place).  K advances in steps of 64 through two LDS
// stages of A (normalised activations, 16 KB) and B (weights, 64 KB): the
// whole 160 KB of LDS.
//  * B: 16-bit weights go from HBM straight into LDS (buffer_load ... lds, 16
//    bytes per lane, one 1 KB wave instruction = 8 rows x 128 bytes); int8
//    and int4 weights go through registers and are dequantised to bf16 on
//    the way.
//  * A: x and the residual are read (L2 hits: a 128-row block is shared by
//    every column tile), re-formed as h, normalised with the row statistics
//    and gamma / beta, rounded to the activation dtype and written to LDS -
//    the normalised rows never reach memory (the LayerNorm + QKV fusion of
//    §2.3).  A tile 4 times wider than it is tall halves the rows each
//    workgroup normalises per MFMA compared with a square tile: the
//    normalisation is VALU work that has to hide in the MFMAs' shadow, the
//    weight tile costs no VALU at all.
// Both LDS tiles store 16-byte chunks XOR-swizzled by row, so that the rows
// of a fragment read spread over the banks.
// The epilogue applies bias and the GQA split / SwiGLU / tanh-GELU / nothing,
// stages the results through LDS and writes 16 bytes per lane.
#pragma once

#include "fp_device.hpp"

namespace fp {

namespace pf {
// 16 bytes per lane from a buffer straight into LDS: lane l writes lds + 16 l
// (the LDS address is taken from the wave-uniform pointer).  The builtin only
// exists in the device pass.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, unsigned char *lds, uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, soff, 0, 0);
#else
    (void)r, (void)lds, (void)voff, (void)soff;
#endif
}
constexpr int BM = 128, BN = 512, BK = 64;
constexpr int ROWB = BK * 2;                 // bytes per tile row (bf16 / f16)
constexpr int TILEA = BM * ROWB;             // 16 KB
constexpr int TILEB = BN * ROWB;             // 64 KB
// swizzled byte offset of 16-byte chunk c (0..7) of tile row r
__device__ __forceinline__ int swz(int r, int c) { return r * ROWB + ((c ^ ((r >> 1) & 7)) << 4); }
}  // namespace pf

// LN: LayerNorm (mean, beta); otherwise RMSNorm or no norm, whose
// normalisation is two multiplies (h * rstd * gamma) and has no beta to load.
// WQ: weight storage -- 0 the activation dtype (straight into LDS), 1 int8,
// 2 int4, 3 MXFP4 (all three through registers, dequantised into LDS), 5 the
// activation dtype tile-packed: a wave load copies one contiguous 1 KB
// block slice (16 rows x 64 bytes) and the B tile keeps the packed order in
// LDS (block, slice, 16-byte group, row), where the 16 lanes of a fragment
// read cover 256 contiguous bytes.  (Quantised weights go through registers,
// so either layout only changes their load addresses.)
template <int ACT, int WQ, int EPI, bool LN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void prefill_kernel(ProjArgs p) {
    using T = Act<ACT>;
    using namespace pf;
    // WI4: 4-bit weights of either kind ([N, K/2] bytes, 32 values per 16-byte vector)
    constexpr bool PK = WQ == 5;
    constexpr bool WI8 = WQ == 1, WMX = WQ == 3, WI4 = WQ == 2 || WMX, WREG = WQ != 0 && !PK;
    static_assert(ACT != ACT_F32, "16-bit activations");
    static_assert(WQ == 0 || PK || ACT == ACT_BF16, "int8 / int4 / MXFP4 weights feed bf16 MFMA");
    // A and B tiles of the two stages as four distinct LDS objects, so that
    // the compiler can tell the direct-to-LDS weight loads into one stage from
    // the fragment reads of the other (and waits for them only at the end of
    // the step, not before the first fragment read).  The B tiles are reused
    // as epilogue staging after the main loop.
    __shared__ __attribute__((aligned(16))) unsigned char lA0[TILEA];
    __shared__ __attribute__((aligned(16))) unsigned char lA1[TILEA];
    __shared__ __attribute__((aligned(16))) unsigned char lB0[TILEB];
    __shared__ __attribute__((aligned(16))) unsigned char lB1[TILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS bases stay scalar

    // ---- tile of this workgroup: XCD-aware remap, then grouped raster
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

    // ---- buffer resources: base and byte size in scalar registers, so each
    // stream needs one 32-bit per-lane offset and the K advance is a scalar
    // offset (keeps the vector register budget for the accumulators).
    // Absent optional operands get an empty range: their loads return zero.
    const uint32_t xbytes = (uint32_t)(p.M * p.K * 2);
    const bool has_res = p.res != nullptr;
    const bool has_beta = p.norm == 2 && p.beta != nullptr;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void *)p.x, (short)0, xbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc((void *)(has_res ? p.res : p.x), (short)0,
                                                                        has_res ? xbytes : 0u, 0x00020000);
    const void *gsrc = p.norm != 0 ? p.gamma : p.x;
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc((void *)gsrc, (short)0,
                                                                        p.norm != 0 ? (uint32_t)(p.K * 2) : 0u, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)(has_beta ? p.beta : gsrc), (short)0,
                                                                        has_beta ? (uint32_t)(p.K * 2) : 0u, 0x00020000);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void *)p.w, (short)0, (uint32_t)(WI4 ? p.Nw * p.K / 2 : p.Nw * p.K * (WI8 ? 1 : 2)), 0x00020000);
    // int4: the group scales [Nw, K / 128] fp32; MXFP4: the block scales [Nw, K / 32] E8M0
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(WI4 ? (const void *)p.w_scale : p.w), (short)0,
        WMX ? (uint32_t)(p.Nw * (p.K / 32)) : WI4 ? (uint32_t)(p.Nw * (p.K / 128) * 4) : 0u, 0x00020000);
    // norm none: gamma reads as zero and g1 turns it into one
    const float g1 = p.norm != 0 ? 0.f : 1.f;

    // ---- A side: thread -> 16-byte chunk a_c of tile rows a_r0 + 32 i (i < 4)
    const int a_c = tid & 7, a_r0 = tid >> 3;
    const float2 *stp = p.norm != 0 ? p.stats : (const float2 *)p.x;
    const float st_on = p.norm != 0 ? 1.f : 0.f;
    uint32_t a_off[4];                                   // bytes, without the K step
    float a_mu[4], a_rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int m = tm * BM + a_r0 + 32 * i;
        m = m < (int)p.M ? m : (int)p.M - 1;             // rows past M only feed unstored outputs
        a_off[i] = ((uint32_t)m * (uint32_t)p.K + a_c * 8) * 2;
        const float2 st = stp[m];
        a_mu[i] = st.x * st_on;
        a_rs[i] = st_on != 0.f ? st.y : 1.f;
    }

    // ---- B side
    // 16-bit weights: wave w loads tile rows [128 w, 128 w + 128) as 16
    // instructions of 8 rows; lane l of instruction i covers row
    // 128 w + 8 i + l / 8 at LDS chunk position l % 8, i.e. global chunk
    // (l % 8) ^ swizzle(row).
    // int8 weights: thread -> 16-byte int8 vector (tile row (tid / 4) + 64 i,
    // k bytes 16 (tid % 4) .. + 15), dequantised in registers.
    // int4 weights: thread -> 16-byte vector of 32 values (tile row
    // (tid / 2) + 128 i, k 32 (tid % 2) .. + 31 of the stage), with the row's
    // scale of the stage's group (a stage of 64 k lies in one group of 128).
    constexpr int NBO = WI8 ? 8 : WI4 ? 4 : 16;
    uint32_t b_off[NBO];                                 // bytes, without the K step
    uint32_t b_soff[WI4 ? 4 : 1];                        // int4: byte offset of the row's scales
    float b_sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b_sc[i] = 0.f;
    b_soff[0] = 0;
#pragma unroll
    for (int i = 0; i < NBO; ++i) {
        int br;
        if constexpr (WI8) br = (tid >> 2) + 64 * i;
        else if constexpr (WI4) br = (tid >> 1) + 128 * i;
        else if constexpr (PK) br = 128 * wave + 16 * (i >> 1);   // block slice 16 wave + i: block row, slice i % 2
        else br = 128 * wave + 8 * i + (lane >> 3);
        int64_t wrow;
        if constexpr (EPI == EPI_SWIGLU) {
            // 32-row blocks alternate gate / up: fragment pairs (2 j, 2 j + 1)
            // of a wave hold the gate and up values of the same outputs
            const int blk = br >> 5;
            int64_t j = (int64_t)tn * (BN / 2) + (blk >> 1) * 32 + (br & 31);
            j = j < p.F ? j : PK ? p.F - 16 : p.F - 1;   // (packed: whole blocks of 16 rows)
            wrow = (blk & 1) ? p.F + j : j;
        } else {
            wrow = (int64_t)tn * BN + br;
            wrow = wrow < p.Nw ? wrow : PK ? p.Nw - 16 : p.Nw - 1;
        }
        if constexpr (WI8) {
            b_off[i] = (uint32_t)weight_off(p.w_layout, wrow, (tid & 3) * 16, p.F, p.K);
            b_sc[i] = p.w_scale[wrow];
        } else if constexpr (WI4) {
            b_off[i] = (uint32_t)weight_off(p.w_layout, wrow, (tid & 1) * 16, p.F, p.K / 2);
            // MXFP4: the thread's 32 values of a stage are block 2 kt + (tid & 1) of the row
            b_soff[i] = WMX ? (uint32_t)(wrow * (p.K / 32)) + (tid & 1) : (uint32_t)(wrow * (p.K / 128) * 4);
        } else if constexpr (PK) {
            b_off[i] = (uint32_t)(packed_row_off(wrow, p.F, p.K * 2, p.w_layout) + (i & 1) * 8192) + lane * 16;
        } else {
            const int c = (lane & 7) ^ ((br >> 1) & 7);
            b_off[i] = (uint32_t)weight_off(p.w_layout, wrow, c * 16, p.F, p.K * 2);
        }
    }

    // ---- activation side, a rolling register pipeline: the rows of stage
    // kt + 1 are normalised into LDS while stage kt feeds the MFMAs, and each
    // row's registers are refilled with stage kt + 2 right after use, so every
    // load has a whole step to arrive.
    struct ARegs { u32x4 x[4], r[4], g, b; };
    struct BRegs {                  // int8 / int4 / MXFP4: the thread's weight vectors of a stage
        u32x4 q[WI4 ? 4 : 8];
        float s[WI4 ? 4 : 1];       // int4: their rows' scales for the stage
        unsigned sm[WMX ? 4 : 1];   // MXFP4: their blocks' scale codes
    };
    ARegs A;
    BRegs B;
    float gv[8], bv[8];             // gamma / beta of the stage being normalised
    auto ld16 = [](const __amdgpu_buffer_rsrc_t &rsrc, uint32_t voff, uint32_t soff) -> u32x4 {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, soff, 0));
    };
    auto a_issue = [&](int kt, int i) {
        const uint32_t kb = (uint32_t)kt * (BK * 2);
        A.x[i] = ld16(rx, a_off[i], kb);
        A.r[i] = ld16(rr, a_off[i], kb);
    };
    auto gb_issue = [&](int kt) {
        const uint32_t kb = (uint32_t)kt * (BK * 2);
        A.g = ld16(rg, a_c * 16, kb);
        if constexpr (LN) A.b = ld16(rb, a_c * 16, kb);
    };
    auto gb_unpack = [&]() {
        T::unpack(A.g, gv);
        if constexpr (LN) T::unpack(A.b, bv);
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[e] += g1;
    };
    // h = x + r (r reads as zero when absent; exact in fp32),
    // n = (h - mu) * rstd * gamma + beta, for words [w0, w0 + 2) of row i
    // (RMSNorm / no norm: mu = 0, no beta)
    auto a_norm = [&](int i, int w0, float (&n)[8]) {
#pragma unroll
        for (int w = w0; w < w0 + 2; ++w) {
            const unsigned xw = A.x[i][w], rv = A.r[i][w];
            if constexpr (LN) {
                const float d0 = (T::lo(xw) + T::lo(rv)) - a_mu[i];
                const float d1 = (T::hi(xw) + T::hi(rv)) - a_mu[i];
                n[2 * w] = fmaf(d0 * a_rs[i], gv[2 * w], bv[2 * w]);
                n[2 * w + 1] = fmaf(d1 * a_rs[i], gv[2 * w + 1], bv[2 * w + 1]);
            } else {
                n[2 * w] = ((T::lo(xw) + T::lo(rv)) * a_rs[i]) * gv[2 * w];
                n[2 * w + 1] = ((T::hi(xw) + T::hi(rv)) * a_rs[i]) * gv[2 * w + 1];
            }
        }
    };
    auto a_store = [&](unsigned char *la, int i, const float (&n)[8]) {
        *(u32x4 *)(la + swz(a_r0 + 32 * i, a_c)) = T::pack(n);
    };
    // ---- weight side.  A stage's weight bytes start at row byte kt times the
    // stage's bytes per row; its offset in the weight's layout is added as the
    // scalar offset to the lanes' offsets of stage 0 (additive in both layouts)
    auto wsoff = [&](uint32_t rb) -> uint32_t { return PK || p.w_layout ? (uint32_t)packed_col_off(rb) : rb; };
    auto bload_lds = [&](int kt, unsigned char *lb) {   // 16-bit weights, straight to LDS
        const uint32_t kb = wsoff((uint32_t)kt * (BK * 2));
#pragma unroll
        for (int i = 0; i < 16; ++i) load_lds16(rw, lb + (128 * wave + 8 * i) * ROWB, b_off[i], kb);
    };
    // int8 weights: vector i of stage kt into registers; dequantised into
    // the LDS tile of its stage (16 values -> two 16-byte bf16 chunks)
    auto bload_one = [&](int kt, int i) {
        if constexpr (WMX) {
            B.q[i] = ld16(rw, b_off[i], wsoff((uint32_t)kt * (BK / 2)));
            B.sm[i] = __builtin_amdgcn_raw_buffer_load_b8(rs, b_soff[i], (uint32_t)kt * 2, 0);
        } else if constexpr (WI4) {
            B.q[i] = ld16(rw, b_off[i], wsoff((uint32_t)kt * (BK / 2)));
            B.s[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, b_soff[i],
                                                                                    (uint32_t)(kt / 2) * 4, 0));
        } else {
            B.q[i] = ld16(rw, b_off[i], wsoff((uint32_t)kt * BK));
        }
    };
    auto bstore_one = [&](unsigned char *lb, int i) {
        u32x4 lo, hi;
        dequant16(B.q[i], b_sc[i], lo, hi);
        const int br = (tid >> 2) + 64 * i;
        const int c0 = (tid & 3) * 2;
        *(u32x4 *)(lb + swz(br, c0)) = lo;
        *(u32x4 *)(lb + swz(br, c0 + 1)) = hi;
    };
    // int4 / MXFP4: half hf of vector i (16 values, two 16-byte chunks) into the LDS tile
    auto bstore_half = [&](unsigned char *lb, int i, int hf) {
        const int br = (tid >> 1) + 128 * i;
        const int c0 = (tid & 1) * 4 + hf * 2;
        if constexpr (WMX) {
            const float sc = e8m0_to_f32(B.sm[i]);
            *(u32x4 *)(lb + swz(br, c0)) = dequant8_mxfp4(B.q[i][2 * hf], sc);
            *(u32x4 *)(lb + swz(br, c0 + 1)) = dequant8_mxfp4(B.q[i][2 * hf + 1], sc);
        } else {
            const float s = B.s[i], m8s = -8.0f * s;
            *(u32x4 *)(lb + swz(br, c0)) = dequant8_i4(B.q[i][2 * hf], s, m8s);
            *(u32x4 *)(lb + swz(br, c0 + 1)) = dequant8_i4(B.q[i][2 * hf + 1], s, m8s);
        }
    };

    // ---- accumulators: acc[i][j][q] = D[row i*32 + 8(q/4) + 4(lane/32) + q%4]
    //                                        [col j*32 + lane%32] of the wave tile
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // MFMAs of one stage: four K substeps of 16; lane l supplies row / column
    // l % 32 and the 16-byte chunk 2 t + l / 32 of both operands.  A stage is
    // run as 8 regions (substep t = r / 2, fragment columns 2 h, 2 h + 1 with
    // h = r % 2), each 8 MFMAs with half an activation row of the next stage
    // normalised between them (row r / 2; after its second half the row is
    // stored into `na` and its registers refilled from stage `kn`), while the
    // fragments of the following region are read from LDS.  Scheduling
    // barriers keep each region's instruction mix in place: every MFMA is
    // followed by a few VALU instructions, which run in its shadow.
    auto frag_a = [&](const unsigned char *la, int t, int i) {
        return *(const u32x4 *)(la + swz(i * 32 + (lane & 31), 2 * t + (lane >> 5)));
    };
    auto frag_b = [&](const unsigned char *lb, int t, int j) {
        if constexpr (PK) {   // packed B tile: row R, chunk c at ((R / 16) 2 + c / 4) KB + 256 (c % 4) + 16 (R % 16)
            const int r = wave * 128 + j * 32 + (lane & 31), c = 2 * t + (lane >> 5);
            return *(const u32x4 *)(lb + ((((r >> 4) * 2 + (c >> 2)) << 10) + ((c & 3) << 8) + ((r & 15) << 4)));
        }
        return *(const u32x4 *)(lb + swz(wave * 128 + j * 32 + (lane & 31), 2 * t + (lane >> 5)));
    };
    auto mma = [&](const unsigned char *la, const unsigned char *lb, unsigned char *na, unsigned char *nb, int kn) {
        u32x4 af[4], bf[2], nf[4], nbf[2];
        float n[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = frag_a(la, 0, i);
        bf[0] = frag_b(lb, 0, 0);
        bf[1] = frag_b(lb, 0, 1);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int t = r >> 1, h = r & 1;
            // fragments of region r + 1
            if (r < 7) {
                if (h == 0) {
                    nbf[0] = frag_b(lb, t, 2);
                    nbf[1] = frag_b(lb, t, 3);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) nf[i] = frag_a(la, t + 1, i);
                    nbf[0] = frag_b(lb, t + 1, 0);
                    nbf[1] = frag_b(lb, t + 1, 1);
                }
            }
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i][2 * h + jj] = T::mfma32(af[i], bf[jj], acc[i][2 * h + jj]);
            a_norm(r >> 1, 2 * h, n);
            if (h == 1) {
                a_store(na, r >> 1, n);
                a_issue(kn, r >> 1);
            }
            if constexpr (WI8) {
                // weights of the next stage, one vector per region, refilled
                // from stage kn right after
                bstore_one(nb, r);
                bload_one(kn, r);
            } else if constexpr (WI4) {
                // half a vector (16 values) per region, the vector refilled
                // after its second half
                bstore_half(nb, r >> 1, r & 1);
                if (r & 1) bload_one(kn, r >> 1);
            }
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                // the next region's fragment reads, two behind each of the
                // first three MFMAs (measured on MI355X: 1-3 % faster than all
                // six ahead of the first)
                if (m < 3) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, WREG ? 8 : 4, 0);   // then VALU
            }
            __builtin_amdgcn_sched_group_barrier(0x200, WREG ? 3 : 1, 0);   // LDS writes
            __builtin_amdgcn_sched_group_barrier(0x020, WREG ? 3 : 2, 0);   // refill loads
            __builtin_amdgcn_sched_barrier(0);
            if (r < 7) {
                bf[0] = nbf[0];
                bf[1] = nbf[1];
                if (h == 1) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) af[i] = nf[i];
                }
            }
        }
    };
    // wait for everything but the activation loads issued after the weights
    // of the step (gamma, beta for LayerNorm, and 8 row loads), and for this
    // thread's LDS writes; then a workgroup barrier.  (int8 weights roll
    // through registers like the activations: no load needs waiting for
    // here.)  The count relies on issue order: every weight load is fenced by
    // a scheduling barrier before anything else is issued.  The empty asm
    // statements keep the compiler from moving memory accesses across the
    // barrier.
    auto step_sync = [&]() {
        constexpr int VM = WREG ? 63 : (LN ? 10 : 9);   // int8 / int4: every load is a rolling register load
        __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (0 << 8));
        __asm__ __volatile__("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
    };

    if (kt0 < kt1) {
        // prologue: stage kt0 into LDS tile 0, then start loading stage kt0 + 1
        if constexpr (WREG) {
#pragma unroll
            for (int i = 0; i < NBO; ++i) bload_one(kt0, i);
        } else {
            bload_lds(kt0, lB0);
        }
        __builtin_amdgcn_sched_barrier(0);
        gb_issue(kt0);
#pragma unroll
        for (int i = 0; i < 4; ++i) a_issue(kt0, i);
        gb_unpack();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float n[8];
            a_norm(i, 0, n);
            a_norm(i, 2, n);
            a_store(lA0, i, n);
        }
        const int k1 = kt0 + 1 < kt1 ? kt0 + 1 : kt1 - 1;
        if constexpr (WI8) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                bstore_one(lB0, i);
                bload_one(k1, i);
            }
        } else if constexpr (WI4) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                bstore_half(lB0, i, 0);
                bstore_half(lB0, i, 1);
                bload_one(k1, i);
            }
        }
        gb_issue(k1);
#pragma unroll
        for (int i = 0; i < 4; ++i) a_issue(k1, i);
        step_sync();
        // stage identity alternates; both pointers of a pair come from one
        // condition, so alias analysis still separates the objects.  Every
        // step prepares the next stage (past the end: harmless reloads of the
        // last one, never used) so that the MFMA code exists once.
        for (int kt = kt0; kt < kt1; ++kt) {
            const bool odd = ((kt - kt0) & 1) != 0;
            const unsigned char *ca = odd ? lA1 : lA0, *cb = odd ? lB1 : lB0;
            unsigned char *na = odd ? lA0 : lA1, *nb = odd ? lB0 : lB1;
            const int kw = kt + 1 < kt1 ? kt + 1 : kt1 - 1;
            const int kn = kt + 2 < kt1 ? kt + 2 : kt1 - 1;
            if constexpr (!WREG) bload_lds(kw, nb);
            __builtin_amdgcn_sched_barrier(0);   // keeps the weight loads first (see step_sync)
            gb_unpack();
            gb_issue(kn);
            __builtin_amdgcn_sched_barrier(0);
            mma(ca, cb, na, nb, kn);
            step_sync();
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // ---- split-K (the arrival verdict lives in the first word of lA0, which
    // nobody reads any more)
    if (p.splits > 1) {
        float flat[256];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) flat[(i * 4 + j) * 16 + e] = acc[i][j][e];
        if (!splitk_reduce<256, true>(p, tile, z, p.splits, flat, (int *)lA0)) return;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = flat[(i * 4 + j) * 16 + e];
    }

    // ---- epilogue, one 32-row fragment row (i) of the wave tile at a time:
    // values (bias and activation applied, fp32) go to this wave's own LDS
    // area in [row][col] order, rows padded by 32 bytes so that the two lane
    // halves (4 rows apart) hit different banks; they are then read back as
    // runs of 8 columns, converted to the output dtype and stored 16 bytes at
    // a time.
    constexpr int OUTC = EPI == EPI_SWIGLU ? 64 : 128;   // output columns per wave
    constexpr int SROW = OUTC * 4 + 32;                  // staging row pitch, bytes
    static_assert(32 * SROW <= TILEB / 2, "staging fits half a B tile");
    unsigned char *stg = (wave < 2 ? lB0 : lB1) + (wave & 1) * (TILEB / 2);
    const int64_t col0 = EPI == EPI_SWIGLU ? (int64_t)tn * (BN / 2) + wave * 64 : (int64_t)tn * BN + wave * 128;
    const int64_t ncols = EPI == EPI_SWIGLU ? p.F : p.Nw;
    // bias of this lane's columns, zero when absent (SwiGLU: gate, up, gate, up)
    float bias_v[4] = {0.f, 0.f, 0.f, 0.f};
    if (p.bias) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t cg;
            if constexpr (EPI == EPI_SWIGLU) {
                const int64_t c = col0 + (j >> 1) * 32 + (lane & 31);
                cg = (c < ncols ? c : ncols - 1) + ((j & 1) ? p.F : 0);
            } else {
                const int64_t c = col0 + j * 32 + (lane & 31);
                cg = c < ncols ? c : ncols - 1;
            }
            bias_v[j] = T::ld(p.bias, cg);
        }
    }
    const bool of32 = p.out_f32 != 0;
    const int esz = of32 ? 4 : 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int rl = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);   // 0..31
            if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
                for (int j = 0; j < 4; j += 2) {
                    const int cl = (j >> 1) * 32 + (lane & 31);        // 0..63
                    const float gv2 = acc[i][j][q] + bias_v[j], uv = acc[i][j + 1][q] + bias_v[j + 1];
                    *(float *)(stg + rl * SROW + cl * 4) = silu(gv2) * uv;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int cl = j * 32 + (lane & 31);               // 0..127
                    float y = acc[i][j][q] + bias_v[j];
                    if constexpr (EPI == EPI_GELU) y = gelu_tanh(y);
                    *(float *)(stg + rl * SROW + cl * 4) = y;
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_s_waitcnt(0);
        // 32 rows x OUTC columns as runs of 8 columns
        constexpr int RUNS = OUTC / 8;
#pragma unroll
        for (int it = 0; it < 32 * RUNS / 64; ++it) {
            const int idx = it * 64 + lane;
            const int rl = idx / RUNS, ch = idx % RUNS;
            const int64_t m = (int64_t)tm * BM + i * 32 + rl;
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

template <int ACT, int WQ, bool LN>
inline hipError_t launch_prefill_n(const ProjArgs &a, unsigned grid, hipStream_t s) {
    switch (a.epi) {
    case EPI_QKV:
        return launch_k(prefill_kernel<ACT, WQ, EPI_QKV, LN>, grid, s, a);
    case EPI_SWIGLU:
        return launch_k(prefill_kernel<ACT, WQ, EPI_SWIGLU, LN>, grid, s, a);
    case EPI_GELU:
        return launch_k(prefill_kernel<ACT, WQ, EPI_GELU, LN>, grid, s, a);
    default:
        return launch_k(prefill_kernel<ACT, WQ, EPI_LINEAR, LN>, grid, s, a);
    }
}

template <int ACT, int WQ>
inline hipError_t launch_prefill_t(const ProjArgs &a, unsigned grid, hipStream_t s) {
    if (a.norm == 2) return launch_prefill_n<ACT, WQ, true>(a, grid, s);
    return launch_prefill_n<ACT, WQ, false>(a, grid, s);
}

}  // namespace fp
