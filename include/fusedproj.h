/*
 * fusedproj — fused residual-add + norm + projection kernels for MI355X (gfx950).
 *
 * C ABI.  Every tensor is a plain pointer to HIP device memory owned by the
 * caller, row-major and contiguous; every size is int64_t.  Nothing here
 * allocates or frees device memory: scratch space is passed in as a
 * caller-owned workspace whose size fp_workspace_bytes() reports.
 *
 * The operations follow the TensorRT-LLM pages this library is built from:
 *  - "TensorRT-LLM 深度工程实践：从模型到生产级推理服务", §2.3 跨算子融合:
 *    the LayerNorm + QKV projection fusion sketch (per-token mean and
 *    variance, the reciprocal root of variance plus eps, gamma and beta, then the Q, K and V products
 *    written straight out without an intermediate tensor) and the SwiGLU
 *    sketch (SiLU of the gate product times the up product, one write);
 *    §2.2 图构建与算子映射: the QKV projection is one matmul followed by a
 *    reshape into GQA head groups;
 *  - "2. TensorRT-LLM 简介", 核心原理: residual + LayerNorm fusion, QKV
 *    fusion, per-op precision matching;
 *  - "TRT-LLM deep dive" (lib.uml.com.cn), 构建阶段详解 §3 Layer Fusion
 *    figure and 面试视角: Add / Bias / LayerNorm / GELU and LayerNorm +
 *    Linear + GELU each collapsed into a single kernel.
 *
 * Shared conventions
 *  - Token rows are independent; M (tokens) may be any value >= 0, M == 0 is
 *    a no-op that returns FP_OK (the per-token pointers x, residual, h_out and
 *    the outputs may then be NULL).
 *  - hidden (K) must be a positive multiple of 64.
 *  - Weights are [N, K] with K contiguous (the nn.Linear weight layout).
 *  - Residual add: h = x + residual, formed in fp32 (exact for 16-bit inputs).
 *    residual may be NULL (h = x).  If h_out is not NULL it receives
 *    round-to-nearest-even(h) in act_dtype (the residual stream for the next
 *    block); h_out must not alias x or residual.
 *  - Norm on h: FP_NORM_RMS   n = h / sqrt(mean(h^2) + eps) * gamma
 *               FP_NORM_LAYER n = (h - mean) / sqrt(var + eps) * gamma + beta
 *                             (biased variance; beta may be NULL = 0)
 *               FP_NORM_NONE  n = h (gamma and beta ignored)
 *    Row statistics are fp32.  n is rounded to act_dtype (RNE) and fed to the
 *    matrix cores.  Calls that the weight-streaming kernel takes (up to 64
 *    tokens) or the 256 x 256 GEMM takes (weights of the activation dtype
 *    and enough tokens to fill the GPU with 256 x 256 tiles: prefill; see
 *    fp_describe_plan, prep=norm_kernel) have a row pass write the rounded
 *    rows once into the workspace (M * hidden * 2 bytes of it), which the
 *    projection reads: the same values.  In streaming calls with hidden up
 *    to 8192 whose grid leaves a CU per token idle (kernel name ending in
 *    ",rows"), M extra workgroups of the streaming launch itself form the rows
 *    (one per token) and publish them through per-row flags in the workspace,
 *    tagged per launch, while the other workgroups request their first
 *    weights; under HIP graph capture (a replay would repeat the tag) and
 *    with the no_stream_rows override the row pass stays a launch of its own.
 *    In the other calls n never goes to memory.
 *  - Product: fp32 accumulation of n * W^T.
 *  - Int8 weights (w_dtype FP_I8, act_dtype FP_BF16 only): each element is
 *    dequantised as bf16_rne(f32_rne(q * w_scale[row])), bit-exactly the
 *    result of fused_dequant_i8_bf16.
 *  - Int4 weights (w_dtype FP_I4, act_dtype FP_BF16 only; the 4-bit
 *    weight-only configuration of "TensorRT-LLM 深度工程实践…" §3.3: group
 *    size 128, no zero point): the [N, hidden] weight is stored as
 *    [N, hidden/2] bytes, element k of a row in the low nibble of byte k/2
 *    for even k and in the high nibble for odd k, each nibble a
 *    two's-complement integer in [-8, 7]; w_scale is [N, hidden/128] fp32,
 *    one scale per row and group of 128 consecutive k; each element is
 *    dequantised as bf16_rne(f32_rne(q * w_scale[row][k / 128])), a zero
 *    result being +0, bit-exactly the result of fused_dequant_i4_bf16.  hidden must be a
 *    multiple of 128.  Calls that the weight-streaming kernel does not take
 *    (see fp_describe_plan) first dequantise the weight into the workspace
 *    (N * hidden * 2 bytes of it).
 *  - MXFP4 weights (w_dtype FP_MXFP4, act_dtype FP_BF16 only; the FP4
 *    weight configuration with 16-bit activations of "TensorRT-LLM
 *    深度工程实践…" §3.3, in the microscaling layout of §7.1: 32 FP4
 *    elements sharing one 8-bit scale): the [N, hidden] weight is stored as
 *    [N, hidden/2] bytes of E2M1 codes (1 sign, 2 exponent bits with bias 1,
 *    1 mantissa bit: +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), element k of a row in
 *    the low nibble of byte k/2 for even k and in the high nibble for odd k;
 *    w_scale points to [N, hidden/32] E8M0 bytes (scale 2^(s - 127); 255,
 *    NaN, is not accepted as data), one per row and block of 32 consecutive
 *    k; each element is dequantised as bf16_rne(e2m1(code) * 2^(s - 127)),
 *    exact for every s up to 252, bit-exactly the result of
 *    fused_dequant_mxfp4_bf16.  Calls that the streaming and 128 x 512
 *    kernels do not take dequantise the weight into the workspace first
 *    (N * hidden * 2 bytes of it).
 *  - FP8 W8A8 (w_dtype FP_E4M3, act_dtype FP_BF16 or FP_F16; the full-FP8
 *    configuration of "TensorRT-LLM 深度工程实践…" §3.3, whose activation
 *    range is taken from the data at run time): the weight is [N, hidden]
 *    E4M3 codes (the OCP 8-bit format: 1 sign, 4 exponent bits with bias 7,
 *    3 mantissa bits, no infinities, largest finite 448; torch's
 *    float8_e4m3fn) with w_scale [N] fp32, w = e4m3(code) * w_scale[row].
 *    Instead of rounding n to act_dtype, each token row of n (fp32) is
 *    quantised at run time: amax = max |n|, a_scale = amax / 448 and
 *    code = E4M3_rne(clamp(n * (448 / amax), -448, 448)) (a zero row gives
 *    zero codes); the product is then sum_k e4m3(a) e4m3(w) in fp32, times
 *    a_scale[m] * w_scale[c].  The codes and scales live in the workspace
 *    (M * hidden + 4 M bytes of it).  hidden must be a multiple of 128, and
 *    M * hidden and N * hidden must be below 2^32.  The product runs in the
 *    FP8 GEMM tiles, or, where the tuning table asks for the streaming
 *    family (up to 64 tokens, hidden a multiple of the streaming chunk), in
 *    the weight-streaming kernel with both operands decoded exactly to bf16
 *    in registers; the results are the same up to the order of the fp32
 *    sums.
 *  - Dtypes: act_dtype in {F32, F16, BF16}; w_dtype == act_dtype, or FP_I8 /
 *    FP_I4 / FP_MXFP4 with act_dtype FP_BF16, or FP_E4M3 with act_dtype
 *    FP_BF16 / FP_F16; out_dtype == act_dtype or FP_F32.  gamma, beta and
 *    bias are act_dtype; w_scale is fp32, except E8M0 bytes for FP_MXFP4.
 *  - Weight layout: w is row-major [N, hidden] (4-bit: [N, hidden / 2]
 *    bytes), or tile-packed by fused_pack_weight, which the caller states by
 *    OR-ing FP_LAYOUT_PACKED (QKV, down and non-SwiGLU gate/up calls) or
 *    FP_LAYOUT_PACKED_GATE_UP (the SwiGLU gate/up call) into w_dtype.  The
 *    results do not depend on the layout (the same kernels, the same order
 *    of sums); the packed layout lets the kernels stream a weight as long
 *    contiguous runs.  Scales (w_scale) stay row-major.
 *  - Every pointer must be 16-byte aligned.  No output range may overlap an
 *    input range, another output, or the workspace.
 *  - Execution is asynchronous on hip_stream (NULL = the default stream);
 *    the call returns once the kernels are enqueued.  Device faults surface at
 *    the caller's next synchronisation.
 *  - Errors: every argument is validated before any HIP call; on any status
 *    other than FP_OK nothing has been enqueued and no memory was touched,
 *    except FP_E_HIP (a launch failed; fp_last_error() has the HIP text).
 *  - The workspace holds per-row statistics, normalised rows, the rows'
 *    ready flags, split-K partial sums and arrival counters.  Its contents
 *    on entry do not matter.  Two calls that
 *    run concurrently must not share a workspace.
 *  - Results are deterministic: the same inputs give the same bits.
 */
#ifndef FUSEDPROJ_H
#define FUSEDPROJ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums are ints in C.  In C++ they get int as their underlying type, so
 * that any int a C caller passes is a value of the type until validation
 * rejects it (an enum without one only holds the values of its enumerators'
 * bit range). */
#ifdef __cplusplus
#define FP_ENUM(tag) enum tag : int
#else
#define FP_ENUM(tag) enum tag
#endif

typedef FP_ENUM(fp_dtype_e) { FP_F32 = 0, FP_F16 = 1, FP_BF16 = 2, FP_I8 = 3, FP_I4 = 4, FP_E4M3 = 5, FP_MXFP4 = 6 } fp_dtype;
/* Weight layout bits, OR'd into a call's w_dtype (and into the w_dtype of
 * fp_workspace_bytes, fp_down_workspace_bytes and fp_describe_plan): the
 * weight was tile-packed by fused_pack_weight with gate_up = 0 / 1.  Any
 * other bits above the low byte are FP_E_DTYPE.  The tuning table matches on
 * the element type alone. */
#define FP_LAYOUT_PACKED 0x100
#define FP_LAYOUT_PACKED_GATE_UP 0x200
typedef FP_ENUM(fp_norm_e) { FP_NORM_NONE = 0, FP_NORM_RMS = 1, FP_NORM_LAYER = 2 } fp_norm;
typedef FP_ENUM(fp_act_e) { FP_ACT_NONE = 0, FP_ACT_SWIGLU = 1, FP_ACT_GELU_TANH = 2 } fp_act;
/* Codes 0-6 keep the numbering of the boundary's first specification;
 * 7 and 8 were added after it (the workspace arguments and enum checks). */
typedef FP_ENUM(fp_status_e) {
    FP_OK = 0,
    FP_E_NULL = 1,      /* a required pointer is NULL */
    FP_E_SHAPE = 2,     /* a size is negative, zero where it must not be, or not a required multiple */
    FP_E_DTYPE = 3,     /* dtype combination not supported */
    FP_E_ALIGN = 4,     /* a pointer is not 16-byte aligned */
    FP_E_ALIAS = 5,     /* an output overlaps an input, another output or the workspace */
    FP_E_HIP = 6,       /* a kernel launch failed; see fp_last_error() */
    FP_E_WORKSPACE = 7, /* workspace missing or smaller than fp_workspace_bytes() */
    FP_E_ARG = 8        /* an enum or override value is out of range */
} fp_status;

/* Bytes of workspace a call with these sizes needs.  n_cols is the number of
 * weight rows of the projection: (n_heads + 2 n_kv_heads) * head_dim for
 * fused_add_norm_qkv, 2 * ffn for fused_gateup_act with FP_ACT_SWIGLU, ffn
 * otherwise.  Returns 0 for invalid sizes or dtypes. */
size_t fp_workspace_bytes(int64_t M, int64_t hidden, int64_t n_cols,
                          fp_dtype act_dtype, fp_dtype w_dtype);

/* Bytes of workspace fused_down_residual needs (K = ffn, hidden output
 * columns).  Returns 0 for invalid sizes or dtypes, and where the call needs
 * none. */
size_t fp_down_workspace_bytes(int64_t M, int64_t ffn, int64_t hidden,
                               fp_dtype act_dtype, fp_dtype w_dtype);

/* Residual add + norm -> QKV projection (+ bias) -> GQA split.
 * ("TensorRT-LLM 深度工程实践…", §2.3 LayerNorm + QKV fusion sketch; §2.2.)
 *  x, residual : [M, hidden] act_dtype (residual may be NULL)
 *  h_out       : [M, hidden] act_dtype or NULL
 *  gamma, beta : [hidden] act_dtype (gamma required unless FP_NORM_NONE)
 *  w_qkv       : [(H + 2 Hkv) * D, hidden], rows = Q heads, then K, then V
 *  w_scale     : required iff w_dtype is FP_I8 or FP_E4M3 (fp32
 *                [(H + 2 Hkv) * D]), FP_I4 (fp32 [(H + 2 Hkv) * D, hidden / 128])
 *                or FP_MXFP4 (E8M0 bytes [(H + 2 Hkv) * D, hidden / 32])
 *  bias        : [(H + 2 Hkv) * D] act_dtype or NULL
 *  q           : [M, H, D]   out_dtype, token-major
 *  k, v        : [M, Hkv, D] out_dtype, token-major
 *  Requires n_heads, n_kv_heads > 0, n_heads % n_kv_heads == 0,
 *  head_dim a positive multiple of 16. */
fp_status fused_add_norm_qkv(
    const void *x, const void *residual, void *h_out,
    const void *gamma, const void *beta, fp_norm norm, float eps,
    const void *w_qkv, const void *w_scale, const void *bias,
    void *q, void *k, void *v,
    int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
    fp_dtype act_dtype, fp_dtype w_dtype, fp_dtype out_dtype,
    void *workspace, size_t workspace_bytes, void *hip_stream);

/* fused_add_norm_qkv with head-major outputs, for an attention kernel that
 * reads one head's rows contiguously (each tensor-parallel rank computes
 * attention for its own group of heads: "TensorRT-LLM 深度工程实践…" §4.1;
 * the reshape into GQA head groups of §2.2):
 *  q    : [H, M, D]   out_dtype, q[h, m, d] = column h * D + d of token m
 *  k, v : [Hkv, M, D] out_dtype, likewise for the K and V column blocks
 * Every other argument, requirement and error as for fused_add_norm_qkv; the
 * values are the same, only their positions differ. */
fp_status fused_add_norm_qkv_hm(
    const void *x, const void *residual, void *h_out,
    const void *gamma, const void *beta, fp_norm norm, float eps,
    const void *w_qkv, const void *w_scale, const void *bias,
    void *q, void *k, void *v,
    int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
    fp_dtype act_dtype, fp_dtype w_dtype, fp_dtype out_dtype,
    void *workspace, size_t workspace_bytes, void *hip_stream);

/* fused_add_norm_qkv without a workspace argument and without any device
 * allocation, for callers that cannot allocate device memory: work recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The call's scratch (row statistics, split-K partial sums and
 * arrival counters) lives in a static device array of
 * FP_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends; its device address is taken once per device, on the first
 * call there.  Arguments, results and errors as for fused_add_norm_qkv,
 * except that a call needing more scratch than the array holds (see
 * fp_workspace_bytes) returns FP_E_WORKSPACE before touching the device.
 * All calls on one GPU share that GPU's array: calls that overlap on one GPU
 * (on two streams, or from two threads) race and must be ordered by the
 * caller.  The array's previous contents never matter. */
#define FP_NOALLOC_SCRATCH_BYTES (16u << 20)

fp_status fused_add_norm_qkv_noalloc(
    const void *x, const void *residual, void *h_out,
    const void *gamma, const void *beta, fp_norm norm, float eps,
    const void *w_qkv, const void *w_scale, const void *bias,
    void *q, void *k, void *v,
    int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim,
    fp_dtype act_dtype, fp_dtype w_dtype, fp_dtype out_dtype, void *hip_stream);

/* (Residual add + norm ->) gate/up or up projection (+ bias) -> activation.
 * ("TensorRT-LLM 深度工程实践…", §2.3 SwiGLU fusion sketch; "TRT-LLM deep
 * dive", Layer Fusion figure / LayerNorm + Linear + GELU.)
 *  act FP_ACT_SWIGLU   : w is [2 ffn, hidden], rows [0, ffn) gate and
 *                        [ffn, 2 ffn) up; out[m, j] = SiLU(g) * u with
 *                        g = acc[m, j] + bias[j], u = acc[m, ffn + j] + bias[ffn + j],
 *                        SiLU(g) = g / (1 + exp(-g))
 *  act FP_ACT_GELU_TANH: w is [ffn, hidden]; out = GELU_tanh(acc + bias),
 *                        GELU_tanh(y) = 0.5 y (1 + tanh(sqrt(2/pi)(y + 0.044715 y^3)))
 *  act FP_ACT_NONE     : w is [ffn, hidden]; out = acc + bias
 *  out : [M, ffn] out_dtype.  bias (act_dtype, length = rows of w) may be NULL.
 *  Requires ffn a positive multiple of 16.  Other arguments as above;
 *  with FP_NORM_NONE and residual NULL the input is x as given. */
fp_status fused_gateup_act(
    const void *x, const void *residual, void *h_out,
    const void *gamma, const void *beta, fp_norm norm, float eps,
    const void *w, const void *w_scale, const void *bias, void *out,
    int64_t M, int64_t hidden, int64_t ffn, fp_act act,
    fp_dtype act_dtype, fp_dtype w_dtype, fp_dtype out_dtype,
    void *workspace, size_t workspace_bytes, void *hip_stream);

/* Down projection with the residual add in its epilogue: the projection
 * after SwiGLU, whose output is added to the residual stream (the MLP's
 * down projection of "TensorRT-LLM 深度工程实践…" §4.1, and the Add folded
 * into its neighbouring kernel in the Layer Fusion figure of "TRT-LLM deep
 * dive", 构建阶段详解 §3):
 *   out[m, c] = residual[m, c] + bias[c] + sum_k a[m, k] * w[c, k]
 * accumulated in fp32 and rounded once to out_dtype.
 *  a        : [M, ffn] act_dtype (e.g. the fused_gateup_act output), used as
 *             given (no norm)
 *  w        : [hidden, ffn] act_dtype, or int8 / int4 / E4M3 with w_scale as
 *             for the other calls (K = ffn; with E4M3 the rows of a are
 *             quantised per token as n is there)
 *  bias     : [hidden] act_dtype or NULL
 *  residual : [M, hidden] act_dtype or NULL (no add)
 *  out      : [M, hidden] out_dtype; may be the residual buffer itself when
 *             out_dtype == act_dtype (the residual stream updated in place;
 *             each element is read and written by the same thread).  Any
 *             other overlap is FP_E_ALIAS.
 *  Requires ffn a positive multiple of 64 (128 for int4 and E4M3), hidden a positive
 *  multiple of 16.  Dtypes, alignment, workspace (fp_down_workspace_bytes(M,
 *  ffn, hidden, act_dtype, w_dtype); fp_workspace_bytes(M, ffn, hidden,
 *  act_dtype, w_dtype), which also covers a normalised-row region this call
 *  never uses, is always enough) and errors as for the other calls. */
fp_status fused_down_residual(const void *a, const void *w, const void *w_scale, const void *bias,
                              const void *residual, void *out, int64_t M, int64_t ffn, int64_t hidden,
                              fp_dtype act_dtype, fp_dtype w_dtype, fp_dtype out_dtype,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/* int8 per-output-row weight dequantisation to bf16, the same device
 * function the projection kernels use in their weight loader:
 * out[j, k] = bf16_rne(f32_rne(q[j, k] * scale[j])).
 *  q : [N, K] int8, scale : [N] fp32, out_bf16 : [N, K] bf16.
 *  Requires K a positive multiple of 16, N >= 0. */
fp_status fused_dequant_i8_bf16(const int8_t *q, const float *scale, void *out_bf16,
                                int64_t N, int64_t K, void *hip_stream);

/* int4 group-wise weight dequantisation to bf16, the same device function
 * the projections use for int4 weights:
 * out[j, k] = bf16_rne(f32_rne(q[j, k] * scale[j, k / 128])), zero as +0.
 *  q : [N, K/2] bytes (two values per byte, even k in the low nibble),
 *  scale : [N, K/128] fp32, out_bf16 : [N, K] bf16.
 *  Requires K a positive multiple of 128, N >= 0. */
fp_status fused_dequant_i4_bf16(const void *q, const float *scale, void *out_bf16,
                                int64_t N, int64_t K, void *hip_stream);

/* MXFP4 weight dequantisation to bf16, the same device function the
 * projections use for MXFP4 weights:
 * out[j, k] = bf16_rne(e2m1(q[j, k]) * 2^(scale[j, k / 32] - 127)).
 *  q : [N, K/2] bytes (two E2M1 codes per byte, even k in the low nibble),
 *  scale : [N, K/32] E8M0 bytes, out_bf16 : [N, K] bf16.
 *  Requires K a positive multiple of 32, N >= 0; q and out_bf16 16-byte
 *  aligned. */
fp_status fused_dequant_mxfp4_bf16(const void *q, const void *scale, void *out_bf16,
                                   int64_t N, int64_t K, void *hip_stream);

/* Tile-packed weights: the weight re-laid-out once, when a model is loaded,
 * so that the projections stream it as long contiguous runs (the pages'
 * deployment flow converts the checkpoint and re-lays the weights out for
 * the target GPU: "TensorRT-LLM 深度工程实践…", the build workflow, step 1,
 * weight preparation and conversion).  Measured on MI355X, the Llama-3-8B
 * decode gate/up call (a 235 MB weight streamed by 224 workgroups of 128
 * rows): 52.9 us on row-major weights, 44.0 us on packed ones.
 *
 * fused_pack_weight reads w, row-major [n_rows, K] elements of w_dtype
 * (F16, BF16, I8, E4M3: K elements per row; I4, MXFP4: K / 2 bytes), and
 * writes the same bytes to w_packed in this order: rows in groups of 128 --
 * with gate_up = 1 (weights of the SwiGLU call, n_rows = 2 * ffn: gate rows
 * [0, ffn), up rows [ffn, 2 ffn)) group t is gate rows 64 t .. 64 t + 63
 * followed by up rows ffn + 64 t .. ffn + 64 t + 63 -- and a group is stored
 * as its 64-byte K slices in order, each as its eight 16-row blocks in
 * order, 1 KB per block slice, in which byte 256 g + 16 i + j is byte
 * 64 s + 16 g + j of the block's row i (s: the slice, g < 4, i < 16,
 * j < 16).  Requires rows of a multiple of 64 bytes and n_rows a multiple of
 * 128 (gate_up: ffn a multiple of 64), both pointers 16-byte aligned and not
 * overlapping; FP_E_DTYPE for FP_F32.  fused_unpack_weight is the inverse.
 * Asynchronous on hip_stream; the caller owns both buffers. */
fp_status fused_pack_weight(const void *w, void *w_packed, int64_t n_rows, int64_t K, fp_dtype w_dtype,
                            int32_t gate_up, void *hip_stream);
fp_status fused_unpack_weight(const void *w_packed, void *w, int64_t n_rows, int64_t K, fp_dtype w_dtype,
                              int32_t gate_up, void *hip_stream);

/* Which kernel a call with these sizes would launch, and how: writes a
 * NUL-terminated line such as
 *   "family=stream kernel=stream_kernel<bf16,m32,n128,k256,swiglu> grid=256
 *    splits=1 slots=2 workspace=4227328"
 * into buf (truncated to cap bytes).  n_cols is the weight row count as for
 * fp_workspace_bytes; act selects the gate/up pairing (FP_ACT_SWIGLU) or not.
 * A diagnostic for tuning and tests: it reads the same tuning table and
 * plan overrides as the calls, touches no device and returns FP_E_SHAPE / FP_E_DTYPE /
 * FP_E_ARG / FP_E_NULL for arguments the calls would reject. */
fp_status fp_describe_plan(int64_t M, int64_t hidden, int64_t n_cols, fp_dtype act_dtype,
                           fp_dtype w_dtype, fp_act act, char *buf, size_t cap);

/* Launch-configuration tuning table.  The pages build their kernels by
 * running candidate configurations on the target GPU for the shapes at hand
 * and keeping the fastest ("TensorRT-LLM 深度工程实践…", §2.4 内核自动调优;
 * "TRT-LLM deep dive", 构建阶段详解 step 2 and 面试视角: micro-benchmarks of
 * GEMM configurations per GPU and input shape).  Here the micro-benchmark is
 * fusion_residual_add_amd.tune (Python, timing through these calls); its
 * result is a table of entries that override the built-in planner for calls
 * whose sizes match.
 *
 * An entry matches a call when m_lo <= M <= m_hi and hidden, n_cols (the
 * weight row count, as for fp_workspace_bytes), act_dtype, w_dtype and the
 * gate/up pairing (swiglu = 1 for FP_ACT_SWIGLU) are equal; the first match
 * wins.  Its fields, each 0 (or -1 for family) to keep the planner's choice:
 *  family : 0 the tiled kernel, 1 the weight-streaming kernel, 2 the
 *           128 x 512 kernel, 4 the row pass + 256 x 256 GEMM; ignored
 *           where that family cannot take the call (streaming: 16-bit
 *           activations, M <= 64, hidden a multiple of 256; 128 x 512:
 *           16-bit activations, x / residual and weight under 4 GiB each;
 *           256 x 256: as 128 x 512, with weights of the activation dtype).
 *           E4M3 weights: 1 (or -1 where the planner would) the
 *           weight-streaming kernel on the codes, any other value the FP8
 *           GEMM tiles;
 *  rows   : streaming kernel, weight rows per workgroup: 128, 64 (16-bit
 *           and E4M3 weights, no gate/up pairing, M <= 32), 32 (as 64, with
 *           hidden a multiple of 512: each K chunk split between two waves
 *           per 16 rows) or 256 (int8, int4, MXFP4 and E4M3 weights); other
 *           values are ignored;
 *  grid   : streaming kernel, workgroups (at most one per unit of work);
 *  splits : tiled, 128 x 512 and FP8 GEMM kernels, ways K is split.
 * Results stay within the parity bounds for any entry (only the order of the
 * fp32 partial sums changes) and are deterministic for a given table.
 * fp_workspace_bytes and fp_describe_plan read the same table, so install
 * it before sizing workspaces.  The plan overrides below, when set, take
 * precedence over the table.
 *
 * fp_tune_install copies n entries (replacing the previous table; n = 0
 * clears it); FP_E_ARG if a field is out of range, FP_E_NULL if entries is
 * NULL with n > 0.  The table is process-wide and guarded by a lock; install
 * it between calls, not while another thread is inside a call whose plan it
 * would change.  fp_tune_count returns the number of installed entries. */
typedef struct {
    int64_t m_lo, m_hi;
    int64_t hidden;
    int64_t n_cols;
    fp_dtype act_dtype;
    fp_dtype w_dtype;
    int32_t swiglu;
    int32_t family;
    int32_t rows;
    int32_t grid;
    int32_t splits;
} fp_tune_entry;

fp_status fp_tune_install(const fp_tune_entry *entries, int64_t n);
int64_t fp_tune_count(void);

/* Plan overrides, for experiments and tests that force a launch
 * configuration on every call (the tuning table above is the per-shape
 * form).  Each field 0 keeps the planner's (or the table's) choice:
 *  splits        : K splits of the tiled, 128 x 512 and FP8 kernels, and
 *                  workgroups per weight tile of the streaming kernel (1..64)
 *  stream_nr     : streaming kernel, weight rows per workgroup / 64 (1, 2, 4;
 *                  only the instantiated forms are taken, as for the table)
 *  stream_target : streaming kernel, workgroup budget (1..65535; 0 = 256)
 *  no_stream     : 1 = never the streaming kernel (E4M3 weights: the FP8
 *                  GEMM tiles at every token count)
 *  no_prefill    : 1 = never the 128 x 512 kernel
 *  fp8_tile      : FP8 GEMM tile by token rows: 32, 64, 128 or 256 (set:
 *                  the FP8 GEMM tiles, never the streaming kernel)
 *  no_gemm16     : 1 = never the row pass + 256 x 256 GEMM
 *  gemm16_stages : 256 x 256 GEMM, LDS stages: 2 (K 64 per stage; taken
 *                  where hidden is a multiple of 128), 4 or 5 (K 32)
 *  no_stream_rows: 1 = the streaming kernel never forms the normalised rows
 *                  itself (a separate row-pass launch forms them first, as
 *                  under HIP graph capture)
 *  stream_rows_expire: 1 = for tests of the bounded wait only: when the
 *                  streaming kernel forms the rows itself, its waiting
 *                  workgroups expect a tag that no workgroup publishes and
 *                  give up after a short wait, so every output of the call
 *                  is NaN (h_out is still written)
 * The initial values come from the environment variables FUSEDPROJ_SPLITS,
 * FUSEDPROJ_STREAM_NR, FUSEDPROJ_STREAM_TARGET, FUSEDPROJ_NO_STREAM,
 * FUSEDPROJ_NO_PREFILL, FUSEDPROJ_FP8_TILE, FUSEDPROJ_NO_GEMM16,
 * FUSEDPROJ_GEMM16_STAGES and FUSEDPROJ_NO_STREAM_ROWS (stream_rows_expire
 * only through fp_plan_override_set), read once, at the first call that plans a
 * launch; no call reads the environment after that.
 * fp_plan_override_set replaces the overrides (NULL restores the values read
 * from the environment); FP_E_ARG if a field is out of range.  Process-wide,
 * under the tuning table's lock; like the table, set it between calls.
 * fp_plan_override_get copies the current values. */
typedef struct {
    int32_t splits;
    int32_t stream_nr;
    int32_t stream_target;
    int32_t no_stream;
    int32_t no_prefill;
    int32_t fp8_tile;
    int32_t no_gemm16;
    int32_t gemm16_stages;
    int32_t no_stream_rows;
    int32_t stream_rows_expire;
} fp_plan_override;

fp_status fp_plan_override_set(const fp_plan_override *o);
fp_status fp_plan_override_get(fp_plan_override *o);

/* Static text for a status code. */
const char *fp_status_str(fp_status s);

/* Message for the last non-FP_OK status returned on this host thread. */
const char *fp_last_error(void);

/* Per-kernel timing with HIP events, for benchmarks.  Between
 * fp_profile_start() and fp_profile_stop() every kernel the library enqueues
 * is bracketed by two events on its stream.  fp_profile_stop() synchronises
 * those events and fills up to `capacity` records (one per kernel name) with
 * the number of launches and their summed duration; *count receives the
 * number of names.  Recording is per process and not thread-safe. */
typedef struct {
    char name[64];
    int64_t launches;
    double total_ms;
} fp_kernel_time;

fp_status fp_profile_start(void);
fp_status fp_profile_stop(fp_kernel_time *out, int capacity, int *count);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDPROJ_H */
