// Device-side building blocks shared by the kernels of libfusedproj (gfx950):
// vector types, round-to-nearest-even conversions, the int8 dequantisation,
// activation-dtype traits (unpack / pack / MFMA), wave reductions, the XCD-aware
// workgroup remap, the activations, the epilogue stores and the deterministic
// split-K reduction.
#pragma once

#include "fp_internal.h"

namespace fp {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// ---------------------------------------------------------------------------
// scalar conversions (round-to-nearest-even for every narrowing)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ unsigned to_bf16(float f) {
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)f);
}
// two fp32 values -> one word of two 16-bit values (first in the low half),
// round to nearest even, one packed conversion instruction each
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack2_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ unsigned pack2_f16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){a, b}, f16x2_t));
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
// Each pair is rounded by one packed conversion: bit for bit the words
// dequant_i8_bf16(q0, s) | dequant_i8_bf16(q1, s) << 16, in 2.5 instructions
// per value (sign-extending convert, multiply, half a packed conversion).
__device__ __forceinline__ void dequant16(u32x4 qv, float s, u32x4 &lo, u32x4 &hi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        unsigned w = qv[i];
        int q0 = (int)(w << 24) >> 24, q1 = (int)(w << 16) >> 24;
        int q2 = (int)(w << 8) >> 24, q3 = (int)w >> 24;
        unsigned p0 = pack2_bf16((float)q0 * s, (float)q1 * s);
        unsigned p1 = pack2_bf16((float)q2 * s, (float)q3 * s);
        if (i < 2) { lo[2 * i] = p0; lo[2 * i + 1] = p1; }
        else       { hi[2 * (i - 2)] = p0; hi[2 * (i - 2) + 1] = p1; }
    }
}

// int4 weights ("TensorRT-LLM 深度工程实践…", §3.3: 4-bit weights with 16-bit
// activations, one scale per group of 128 k, no zero point): 32 values of one
// 16-byte load (element 2i in the low nibble of byte i, two's complement)
// times their group scale s -> four 16-byte vectors of 8 bf16 values each,
// bf16_rne(f32_rne(q * s)).  The nibbles are turned into offset binary
// (u = q + 8 = nibble ^ 8) and spread into bytes, so each value is one byte
// convert (v_cvt_f32_ubyte) and one fma(u, s, -8 s): -8 s is exact and the
// fma rounds u * s - 8 s = q * s once, as the definition does (a zero
// result is +0, which the definition fixes).  About 3 instructions per value.  The single definition used by the weight loader
// and dequant_i4_kernel.
// 8 int4 values (one word) -> one 16-byte vector of 8 bf16 values
__device__ __forceinline__ u32x4 dequant8_i4(unsigned word, float s, float m8s) {
    const unsigned v = word ^ 0x88888888u;
    unsigned ev = v & 0x0F0F0F0Fu;                 // elements 0, 2, 4, 6
    unsigned od = (v >> 4) & 0x0F0F0F0Fu;          // elements 1, 3, 5, 7
    // keep the two spread words as they are: otherwise the compiler folds
    // the masks into a bit-field extract per value instead of using the
    // byte-select conversions (v_cvt_f32_ubyte1..3)
    asm("" : "+v"(ev), "+v"(od));
    u32x4 out;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const float f0 = fmaf((float)((ev >> (8 * b)) & 0xFFu), s, m8s);
        const float f1 = fmaf((float)((od >> (8 * b)) & 0xFFu), s, m8s);
        out[b] = pack2_bf16(f0, f1);
    }
    return out;
}

__device__ __forceinline__ void dequant32_i4(u32x4 qv, float s, u32x4 (&out)[4]) {
    const float m8s = -8.0f * s;
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = dequant8_i4(qv[w], s, m8s);
}

// MXFP4 weights ("TensorRT-LLM 深度工程实践…", §3.3: FP4 weights with 16-bit
// activations; §7.1: 32 FP4 elements sharing one 8-bit scale): E2M1 codes,
// element 2i of a word in the low nibble of byte i, times the block's E8M0
// scale 2^(s - 127).  The product is a 2-bit significand times a power of
// two, so the bf16 value is exact wherever bf16 reaches.  The scale code
// becomes its fp32 power of two (s = 0: the fp32 subnormal 2^-127), and one
// hardware conversion (v_cvt_scalef32_pk_bf16_fp4) turns each byte into two
// bf16 values.  The single definition used by the weight loaders and
// dequant_mxfp4_kernel.
__device__ __forceinline__ float e8m0_to_f32(unsigned s) {
    return __uint_as_float(s ? (s << 23) : 0x00400000u);
}
// E4M3 codes to bf16, exactly (every E4M3 value, subnormals included, is a
// bf16 value): two codes per conversion, the first code of each pair in the
// lower half (the hardware's scaled FP8 conversion with scale 1)
template <bool HIGH>
__device__ __forceinline__ unsigned e4m3x2_to_bf16x2(unsigned word) {
    return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(word, 1.0f, HIGH));
}
// 8 codes (two words) -> 8 bf16
__device__ __forceinline__ u32x4 decode8_e4m3(unsigned w0, unsigned w1) {
    return (u32x4){e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0), e4m3x2_to_bf16x2<false>(w1),
                   e4m3x2_to_bf16x2<true>(w1)};
}

__device__ __forceinline__ u32x4 dequant8_mxfp4(unsigned word, float scale) {
    u32x4 out;
    out[0] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 0));
    out[1] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 1));
    out[2] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 2));
    out[3] = __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, scale, 3));
    return out;
}
// 32 codes of one 16-byte load (one MXFP4 block) -> four vectors of 8 bf16
__device__ __forceinline__ void dequant32_mxfp4(u32x4 qv, unsigned scale_code, u32x4 (&out)[4]) {
    const float sc = e8m0_to_f32(scale_code);
#pragma unroll
    for (int w = 0; w < 4; ++w) out[w] = dequant8_mxfp4(qv[w], sc);
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
    __device__ static u32x4 pack(const float *f) {   // RNE, two values per conversion
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack2_bf16(f[2 * i], f[2 * i + 1]);
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
    // 32 x 32 x 16: lane l supplies row / column l % 32, k 8 (l / 32) .. + 7
    __device__ static f32x16 mfma32(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // the two values of a word (low half first)
    __device__ static float lo(unsigned w) { return bf16lo(w); }
    __device__ static float hi(unsigned w) { return bf16hi(w); }
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
    __device__ static u32x4 pack(const float *f) {   // RNE, two values per conversion
        u32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = pack2_f16(f[2 * i], f[2 * i + 1]);
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
    __device__ static f32x16 mfma32(Frag a, Frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static float lo(unsigned w) { return f16lo(w); }
    __device__ static float hi(unsigned w) { return f16hi(w); }
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

// Epilogue activations on the hardware's exp2 and reciprocal (v_exp_f32,
// v_rcp_f32: about 1 ulp each), a few instructions per value instead of a
// range-reduced expf and an IEEE division; the outputs are rounded to 16 bits
// afterwards.  Overflow behaves like the exact forms: exp2 -> +inf gives
// rcp -> 0 and a zero result for large negative inputs.
__device__ __forceinline__ float exp_neg(float x) {   // exp(-x)
    return __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
}
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + exp_neg(g)); }

// tanh-approximation GELU written through the identity
// 0.5 y (1 + tanh(z)) = y / (1 + exp(-2 z)), z = sqrt(2/pi) (y + 0.044715 y^3).
__device__ __forceinline__ float gelu_tanh(float y) {
    const float c2 = 2.0f * 0.7978845608028654f;
    const float z2 = c2 * fmaf(0.044715f * y, y * y, y);
    return y * __builtin_amdgcn_rcpf(1.0f + exp_neg(z2));
}

// ---------------------------------------------------------------------------
// epilogue stores
// ---------------------------------------------------------------------------
// Element index of column cc (relative to its block) of token m in the q, k
// or v output whose block is `width` columns wide: token-major
// [M, heads, D] -> m * width + cc, or head-major [heads, M, D] ->
// (h * M + m) * D + d with h = cc / D, d = cc % D.  A run of 8 columns
// starting at a multiple of 8 stays inside one head (D is a multiple of 16)
// and is contiguous in both layouts.
__device__ __forceinline__ int64_t qkv_index(const ProjArgs &p, int64_t m, int64_t cc, int64_t width) {
    if (!p.qkv_hm) return m * width + cc;
    const int h = (int)cc / (int)p.head_dim;
    return ((int64_t)h * p.M + m) * p.head_dim + (cc - (int64_t)h * p.head_dim);
}

// Column c of the projection (bias already added) to its destination: the GQA
// split for QKV (q | k | v column blocks, token- or head-major), tanh-GELU or nothing for
// the up projection, plus the residual for the down projection.  The residual
// element is read by the thread that writes the output element, so the output
// may be the residual buffer itself.
template <int ACT, int EPI>
__device__ __forceinline__ void store_col(const ProjArgs &p, int64_t m, int64_t c, float y) {
    using T = Act<ACT>;
    void *dst;
    int64_t idx;
    if constexpr (EPI == EPI_QKV) {
        if (c < p.nq)              { dst = p.out0; idx = qkv_index(p, m, c, p.nq); }
        else if (c < p.nq + p.nkv) { dst = p.out1; idx = qkv_index(p, m, c - p.nq, p.nkv); }
        else                       { dst = p.out2; idx = qkv_index(p, m, c - p.nq - p.nkv, p.nkv); }
    } else {
        if constexpr (EPI == EPI_GELU) y = gelu_tanh(y);
        dst = p.out0;
        idx = m * p.F + c;
        if constexpr (EPI == EPI_LINEAR)
            if (p.res_epi) y += T::ld(p.res_epi, idx);   // the down projection's residual add
    }
    if (p.out_f32) ((float *)dst)[idx] = y;
    else T::st(dst, idx, y);
}

// SwiGLU output j from the gate and up accumulators of the same column.
template <int ACT>
__device__ __forceinline__ void store_swiglu(const ProjArgs &p, int64_t m, int64_t j, float g, float u) {
    using T = Act<ACT>;
    if (p.bias) { g += T::ld(p.bias, j); u += T::ld(p.bias, p.F + j); }
    const float y = silu(g) * u;
    if (p.out_f32) ((float *)p.out0)[m * p.F + j] = y;
    else T::st(p.out0, m * p.F + j, y);
}

// ---------------------------------------------------------------------------
// deterministic split-K reduction
// ---------------------------------------------------------------------------
// Every contributor to a tile (a K split, or a workgroup sharing the tile in
// the stream kernel) stores its NACC accumulators per thread in its slot
// (coalesced: element r of thread t at r * 256 + t), then counts itself in
// at the tile's arrival counter.  The last of the `count` contributors to
// arrive reads all partials and sums them in slot order 0, 1, ..., count - 1
// (so the sum never depends on arrival order) and returns true; the others
// return false and go on without the tile.
//
// Publication across the XCDs' private, mutually non-coherent L2s: the
// partials are written and read only with agent-scope atomic accesses
// (gfx950: stores and loads with the sc1 bit, which complete at the
// device-wide coherence point instead of in an XCD's L2), and every thread
// waits for its own partial stores to be acknowledged (s_waitcnt 0) before
// the workgroup barrier that precedes thread 0's arrival at the tile's
// counter (an agent-scope atomic add).  A contributor's arrival is therefore
// issued only after all of its partials are visible device-wide, and the last
// arriver issues its partial loads only after it has read the final count
// (the barrier orders them; the loads depend on the broadcast verdict).  The
// memory model's way of writing this -- an acq_rel counter update and an
// acquire fence -- compiles to a whole-L2 write-back and invalidate at every
// arrival, and was measured at 7.4 us more per decode QKV call (20.4 ->
// 27.8 us, Llama-3-8B, 96 shared tiles) for partials that never sit in L2.
// The counters are cleared by the statistics kernel that precedes every
// split launch on the same stream.
// `flag`: an int of LDS for the arrival verdict, or null for a static one
// (kernels that use all of LDS pass a word of a tile buffer they are done
// with)
template <int NACC, bool EXT_FLAG = false>
__device__ __forceinline__ bool splitk_reduce(const ProjArgs &p, int tile, int slot, int count,
                                              float (&acc)[NACC], int *flag = nullptr) {
    int *s_last_p;
    if constexpr (EXT_FLAG) {
        s_last_p = flag;
    } else {
        __shared__ int s_last_own;
        s_last_p = &s_last_own;
    }
    int &s_last = *s_last_p;
    const int tid = threadIdx.x;
    const int64_t tile_elems = (int64_t)NACC * 256;
    float *mine = p.partials + ((int64_t)tile * p.slots + slot) * tile_elems;
#pragma unroll
    for (int r = 0; r < NACC; ++r)
        __hip_atomic_store(&mine[r * 256 + tid], acc[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);   // all of this thread's stores have completed
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&p.counters[tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        s_last = prev == (unsigned)(count - 1);
    }
    __syncthreads();
    if (!s_last) return false;
    const float *base = p.partials + (int64_t)tile * p.slots * tile_elems;
#pragma unroll
    for (int r = 0; r < NACC; ++r) acc[r] = 0.f;
    if constexpr (NACC > 64) {
        // large tiles: 64 values in flight at a time, split by split, in order
        for (int zz = 0; zz < count; ++zz) {
#pragma unroll
            for (int r0 = 0; r0 < NACC; r0 += 64) {
                float v[64];
#pragma unroll
                for (int r = 0; r < 64; ++r)
                    v[r] = __hip_atomic_load(&base[zz * tile_elems + (r0 + r) * 256 + tid], __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
                for (int r = 0; r < 64; ++r) acc[r0 + r] += v[r];
            }
        }
        return true;
    }
    // G splits' worth of partials in flight at once, then added in order
    constexpr int G = NACC >= 64 ? 1 : 64 / NACC;
    for (int z0 = 0; z0 < count; z0 += G) {
        float v[G][NACC];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < NACC; ++r)
                v[g][r] = z0 + g < count
                              ? __hip_atomic_load(&base[(z0 + g) * tile_elems + r * 256 + tid],
                                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                              : 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < NACC; ++r) acc[r] += v[g][r];
    }
    return true;
}

}  // namespace fp
