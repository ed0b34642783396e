// Internal interface between the C-ABI layer (fp_api.cpp) and the HIP kernels
// (fp_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fusedproj.h"

namespace fp {

enum ActT { ACT_F32 = 0, ACT_F16 = 1, ACT_BF16 = 2 };
enum EpiKind { EPI_QKV = 0, EPI_SWIGLU = 1, EPI_GELU = 2, EPI_LINEAR = 3 };

// Tile families the kernels are instantiated for.
enum TileCfg {
    TILE_DEC16 = 0,   // BM 16,  BN 128, BK 64, waves 1x4  (decode, M <= 16)
    TILE_DEC32 = 1,   // BM 32,  BN 128, BK 64, waves 1x4  (decode, M <= 32)
    TILE_DEC64 = 2,   // BM 64,  BN 128, BK 64, waves 1x4  (decode, M <= 64)
    TILE_PF128 = 3,   // BM 128, BN 128, BK 64, waves 2x2  (prefill)
    TILE_COUNT = 4
};

struct TileShape { int bm, bn, bk; };
TileShape tile_shape(int cfg);

// Weight storage layouts (the layout bits of a call's w_dtype).
enum WLayout { WL_ROWS = 0, WL_PACKED = 1, WL_PACKED_GATE_UP = 2 };

// Tile-packed weights (fused_pack_weight).  The rows are taken in groups of
// 128 -- with the gate/up pairing, the gate rows 64 t .. 64 t + 63 followed
// by the matching up rows F + 64 t .. F + 64 t + 63 -- and a group is stored
// K slice by K slice: for each 64-byte slice s of the row bytes, its eight
// 16-row blocks, 1 KB each; inside a block, byte 256 g + 16 i + j holds byte
// 64 s + 16 g + j of the block's row i.  A workgroup that streams a group
// K slice by K slice then reads one contiguous run per step.
// Byte offset of logical row r's first byte:
__host__ __device__ inline int64_t packed_row_off(int64_t r, int64_t F, int64_t row_bytes, int layout) {
    int64_t t, i;
    if (layout == WL_PACKED_GATE_UP) {
        const bool up = r >= F;
        const int64_t j = up ? r - F : r;
        t = j >> 6;
        i = ((j >> 4) & 3) + (up ? 4 : 0);
    } else {
        t = r >> 7;
        i = (r >> 4) & 7;
    }
    return t * 128 * row_bytes + i * 1024 + (r & 15) * 16;
}
// ... to which row byte c adds (additively over a 64-byte-aligned base and a
// part inside its slice: packed_col_off(a + b) = packed_col_off(a) +
// packed_col_off(b) for a % 64 == 0, and for b < 64 - a % 64 with a % 16 == 0)
__host__ __device__ inline int64_t packed_col_off(int64_t c) {
    return (c >> 6) * 8192 + ((c >> 4) & 3) * 256 + (c & 15);
}
// byte offset of row byte c of weight row r in either layout
__host__ __device__ inline int64_t weight_off(int layout, int64_t r, int64_t c, int64_t F, int64_t row_bytes) {
    return layout == WL_ROWS ? r * row_bytes + c : packed_row_off(r, F, row_bytes, layout) + packed_col_off(c);
}

struct StatsArgs {
    const void *x, *res;
    void *h_out;
    float2 *stats;
    int norm;
    float eps;
    int64_t M, K;
    unsigned *counters;
    int n_counters;
    // per-token E4M3 quantisation (quant8_kernel only)
    const void *gamma, *beta;   // [K] act; beta LayerNorm only, may be null
    unsigned char *codes;       // [M, K] E4M3 codes of the normalised rows
    float *qscale;              // [M] dequantisation scale of each row
    // normalised rows in the activation dtype (norm_kernel only)
    void *rows;                 // [M, K] act
};

// Everything one projection launch needs.
struct ProjArgs {
    // prologue inputs
    const void *x;          // [M, K] act
    const void *res;        // [M, K] act or null
    const float2 *stats;    // [M] (mean, rstd) or null when norm == 0
    const void *gamma;      // [K] act
    const void *beta;       // [K] act or null
    int norm;               // 0 none, 1 rms, 2 layer
    // weights
    const void *w;          // [Nw, K] act or int8
    int w_layout;           // WLayout (packed: gate/up pairs against F, the SwiGLU width)
    const float *w_scale;   // int8 / E4M3: [Nw] fp32; int4: [Nw, K/128] fp32; MXFP4: [Nw, K/32] E8M0 bytes
    const void *bias;       // [Nw] act or null
    const void *res_epi;    // EPI_LINEAR: [M, F] act added to the output (residual stream), or null
    const float *a_scale;   // E4M3 path: [M] per-token scale of the quantised rows in x
    // epilogue
    int epi;                // EpiKind
    int out_f32;            // 1: store fp32, 0: store act dtype
    void *out0;             // q (QKV) or out
    void *out1;             // k (QKV)
    void *out2;             // v (QKV)
    int64_t nq, nkv;        // QKV column split: [0,nq) q, [nq,nq+nkv) k, rest v
    int qkv_hm;             // QKV outputs head-major [heads, M, head_dim] (else token-major)
    int64_t head_dim;       // QKV: D (head-major addressing)
    int64_t F;              // SwiGLU / GELU / linear output width
    // sizes
    int64_t M, K, Nw;       // Nw = weight rows
    // tiling
    int tiles_m, tiles_n, splits;
    int slots;              // partial-sum slots per tile (split count, or the most
                            // workgroups sharing one tile in the stream kernel)
    float *partials;        // [tile][slot][tile elements] partial sums
    unsigned *counters;     // per-tile arrival counters (splits > 1)
    // the stream kernel's own row pass (its RP form): workgroups 0 .. M - 1
    // each form one token row as norm_kernel does (rp: x, residual, gamma,
    // beta, h_out, rows, the split-K counters to clear) and publish it by
    // writing rp_tag to rp_flags[m]; every workgroup waits for all M flags
    // before it reads the rows (x above is then rp.rows)
    StatsArgs rp;
    unsigned long long *rp_flags;   // [M]
    unsigned long long rp_tag;      // this launch's tag (unique per launch in the process)
    unsigned long long rp_wait_tag; // the tag the waiting workgroups expect (rp_tag)
    int rp_spin;                    // polls before a waiting workgroup gives up
};


// Launch a kernel of 256-thread workgroups and return the status of this
// launch itself (hipLaunchKernel's return value), never an error that an
// earlier, unrelated HIP call left pending on the thread.
template <typename T> struct launch_arg { using type = T; };   // keeps P deduced from the kernel alone
template <typename... P>
inline hipError_t launch_k(void (*kernel)(P...), unsigned grid, hipStream_t s, typename launch_arg<P>::type... args) {
    void *argv[] = {(void *)&args...};
    return hipLaunchKernel((const void *)kernel, dim3(grid), dim3(256), argv, 0, s);
}

hipError_t launch_stats(int act, const StatsArgs &a, hipStream_t s);
// tiled family (fp_tiled.hip): prefill token counts and every fp32 call
hipError_t launch_tiled(int act, bool w_i8, int tile, const ProjArgs &a, hipStream_t s);
// weight-streaming family (fp_stream*.hip): 16-bit activations, M <= 64.
//  mf: 16-row token fragments (1, 2 or 4); nr: 16-row weight fragments per
//  wave (1 or 2; 2 for SwiGLU) -> 64 * nr weight rows per workgroup;
//  u: 32-wide k slices per chunk (8) -> K must be a multiple of 32 * u.
//  tiles_m must be 1.
struct StreamCfg {
    int mf, nr, u, kh = 1;   // kh: K parts per chunk (2: 32-row workgroups)
    int rp = 0;              // 1: the kernel's own row pass (ProjArgs::rp; 16-bit, int8, int4 and
                             // MXFP4 weights; hidden <= 8192, M <= the grid)
};
// grid_wgs workgroups share the (weight tile, K chunk) units evenly
hipError_t launch_stream(int act, int wq, const StreamCfg &c, const ProjArgs &a, int grid_wgs, hipStream_t s);
hipError_t launch_dequant(const int8_t *q, const float *scale, void *out, int64_t N, int64_t K,
                          hipStream_t s);

// names used by the event profiler
const char *stats_kernel_name(int act);
const char *proj_kernel_name(int act, bool w_i8, int tile, int epi);
const char *stream_kernel_name(int act, int wq, const StreamCfg &c, int epi);
// 128 x 512 family (fp_prefill*.hip): 16-bit activations, more than 64 tokens
hipError_t launch_prefill(int act, int wq, const ProjArgs &a, hipStream_t s);
const char *prefill_kernel_name(int act, int wq, int epi);
const char *dequant_kernel_name();
hipError_t launch_dequant_i4(const uint8_t *q, const float *scale, void *out, int64_t N, int64_t K,
                             hipStream_t s);
const char *dequant_i4_kernel_name();
hipError_t launch_dequant_mxfp4(const uint8_t *q, const uint8_t *scale, void *out, int64_t N, int64_t K,
                                hipStream_t s);
const char *dequant_mxfp4_kernel_name();
// E4M3 (W8A8) path: per-token quantisation of the normalised rows, then the
// FP8 GEMM on the codes (x = codes, a_scale, w = E4M3 weights, w_scale [Nw])
hipError_t launch_quant8(int act, const StatsArgs &a, hipStream_t s);
// tile-packed weights: pack (unpack = false) a row-major weight of n_rows rows
// of row_bytes bytes, or unpack it back (F: gate rows of the gate/up pairing)
hipError_t launch_pack(const void *src, void *dst, int64_t n_rows, int64_t row_bytes, int64_t F, int layout,
                       bool unpack, hipStream_t s);
const char *pack_kernel_name(bool unpack);
const char *quant8_kernel_name(int act);
// 256 x 256 prefill path: the row pass writes the normalised rows (h_out as
// stats_kernel, the rows into StatsArgs::rows), then the 16-bit GEMM reads
// them (x = rows, no norm) with the weights straight into LDS
hipError_t launch_norm(int act, const StatsArgs &a, hipStream_t s);
const char *norm_kernel_name(int act);
hipError_t launch_gemm16(int act, int nst, const ProjArgs &a, hipStream_t s);
const char *gemm16_kernel_name(int act, int nst, int epi);
// FP8 GEMM tiles (tokens x weight rows)
enum Gemm8Tile { G8_128x128 = 0, G8_256x256 = 1, G8_32x256 = 2, G8_64x256 = 3 };
hipError_t launch_gemm8(int act, int tile, const ProjArgs &a, hipStream_t s);
const char *gemm8_kernel_name(int act, int tile, int epi);

// A workspace for a call that brings none (fused_add_norm_qkv_noalloc):
// given the bytes the plan needs, sets *ws / *ws_bytes or returns a status
// with a message in msg.  Called after every argument has been validated.
typedef fp_status (*WorkspaceSource)(size_t need, void **ws, size_t *ws_bytes, char *msg, size_t cap);
fp_status add_norm_qkv_with_source(const void *x, const void *residual, void *h_out, const void *gamma,
                                   const void *beta, fp_norm norm, float eps, const void *w_qkv,
                                   const void *w_scale, const void *bias, void *q, void *k, void *v,
                                   int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads,
                                   int64_t head_dim, fp_dtype act_dtype, fp_dtype w_dtype,
                                   fp_dtype out_dtype, void *hip_stream, WorkspaceSource source);

}  // namespace fp
