// Internal interface between the C-ABI layer (fp_api.cpp) and the HIP kernels
// (fp_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

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
    const float *w_scale;   // [Nw] (int8 only)
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
};

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
};

hipError_t launch_stats(int act, const StatsArgs &a, hipStream_t s);
// tiled family (fp_tiled.hip): prefill token counts and every fp32 call
hipError_t launch_tiled(int act, bool w_i8, int tile, const ProjArgs &a, hipStream_t s);
// weight-streaming family (fp_stream*.hip): 16-bit activations, M <= 64.
//  mf: 16-row token fragments (1, 2 or 4); nr: 16-row weight fragments per
//  wave (1 or 2; 2 for SwiGLU) -> 64 * nr weight rows per workgroup;
//  u: 32-wide k slices per chunk (8) -> K must be a multiple of 32 * u.
//  tiles_m must be 1.
struct StreamCfg { int mf, nr, u; };
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
// E4M3 (W8A8) path: per-token quantisation of the normalised rows, then the
// FP8 GEMM on the codes (x = codes, a_scale, w = E4M3 weights, w_scale [Nw])
hipError_t launch_quant8(int act, const StatsArgs &a, hipStream_t s);
const char *quant8_kernel_name(int act);
// FP8 GEMM tiles (tokens x weight rows)
enum Gemm8Tile { G8_128x128 = 0, G8_256x256 = 1, G8_32x256 = 2, G8_64x256 = 3 };
hipError_t launch_gemm8(int act, int tile, const ProjArgs &a, hipStream_t s);
const char *gemm8_kernel_name(int act, int tile, int epi);

}  // namespace fp
