// C-ABI layer of libfusedproj: argument validation (before any HIP call),
// launch planning (tile family and split-K factor by token count), workspace
// layout, kernel launches on the caller's stream, error text, and an optional
// HIP-event profiler for benchmarks.
#include "fusedproj.h"
#include "fp_internal.h"

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>
#include <random>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

fp_status fail(fp_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

int act_size(int dt) { return dt == FP_F32 ? 4 : (dt == FP_I8 || dt == FP_E4M3) ? 1 : 2; }

int act_code(fp_dtype d) {
    return d == FP_F32 ? fp::ACT_F32 : d == FP_F16 ? fp::ACT_F16 : fp::ACT_BF16;
}

// ---------------------------------------------------------------------------
// launch plan
// ---------------------------------------------------------------------------
struct Plan {
    int family = 0;           // 0 tiled (128 x 128), 1 stream (decode), 2 prefill (128 x 512),
                              // 3 FP8 (per-token E4M3 quantisation, then the 128 x 128 FP8 GEMM),
                              // 4 gemm16 (the row pass writes the normalised rows, then the
                              //   256 x 256 16-bit GEMM reads them)
    int tile = 0;             // tiled: TileCfg
    fp::StreamCfg sc{1, 2, 8};
    int tiles_m = 0, tiles_n = 0, splits = 1;
    int grid = 0;             // stream: workgroups sharing the units evenly
    int slots = 1;            // partial-sum slots per tile (1: none needed)
    int64_t tile_elems = 0;   // accumulators per tile (split-K partial size)
    size_t stats_off = 0, ctr_off = 0, part_off = 0, total = 0;
    bool deq = false;         // int4 / MXFP4 weights staged as bf16 in the workspace first
    size_t deq_off = 0;
    size_t q_off = 0, qs_off = 0;   // FP8: activation codes [M, K] and row scales [M]
    int tile8 = 0;                  // FP8: fp::Gemm8Tile
    bool stream8 = false;           // FP8: the weight-streaming kernel on the codes (sc, grid) instead
    int nst = 4;                    // gemm16: LDS stages
    bool rows = false;              // gemm16: the row pass forms A (else A is the call's input)
    size_t rows_off = 0;            // gemm16: normalised rows [M, K]
    bool unpack = false;            // tile-packed weights unpacked into the workspace first (tiled family)
    size_t unpack_off = 0;
    size_t flags_off = 0;           // stream with sc.rp: the rows' ready flags [M] (8 bytes each)
    bool rows_expire = false;       // sc.rp: the waits expect an unpublished tag (tests of the bounded wait)
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

long env_long(const char *name, long dflt) {
    const char *s = getenv(name);
    if (!s || !*s) return dflt;
    return strtol(s, nullptr, 10);
}

// Launch-configuration overrides for one call: from the installed tuning
// table (fp_tune_install), then from the plan overrides (fp_plan_override_set,
// initially the FUSEDPROJ_* environment variables), which win.  Zero / -1
// fields leave the planner's choice.
struct Knobs {
    int family = -1;          // 0 tiled, 1 stream, 2 prefill, 4 gemm16; -1 the planner's
    long rows = 0;            // stream: weight rows per workgroup (64, 128, 256)
    long grid = 0;            // stream: workgroups
    long splits = 0;          // tiled / prefill / FP8: K splits
    long stream_splits = 0;   // stream: workgroups per tile (overrides only)
    long target = 256;        // stream: workgroup budget
    int fp8_tile = 0;         // FP8 GEMM tile by token rows (overrides only)
    int gemm16_stages = 0;    // gemm16: LDS stages, 2, 4 or 5 (overrides only)
    bool no_stream = false, no_prefill = false, no_gemm16 = false;
    bool no_stream_rows = false;   // stream: never the kernel's own row pass (overrides only)
    bool stream_rows_expire = false;   // stream: its waits expect an unpublished tag (tests only)
};

std::mutex g_tune_mu;
std::vector<fp_tune_entry> g_tune;

// the FUSEDPROJ_* environment, read once (thread-safe static initialisation)
const fp_plan_override &env_overrides() {
    static const fp_plan_override v = [] {
        fp_plan_override o{};
        o.splits = (int32_t)env_long("FUSEDPROJ_SPLITS", 0);
        o.stream_nr = (int32_t)env_long("FUSEDPROJ_STREAM_NR", 0);
        o.stream_target = (int32_t)env_long("FUSEDPROJ_STREAM_TARGET", 0);
        o.no_stream = env_long("FUSEDPROJ_NO_STREAM", 0) != 0;
        o.no_prefill = env_long("FUSEDPROJ_NO_PREFILL", 0) != 0;
        o.fp8_tile = (int32_t)env_long("FUSEDPROJ_FP8_TILE", 0);
        o.no_gemm16 = env_long("FUSEDPROJ_NO_GEMM16", 0) != 0;
        o.gemm16_stages = (int32_t)env_long("FUSEDPROJ_GEMM16_STAGES", 0);
        o.no_stream_rows = env_long("FUSEDPROJ_NO_STREAM_ROWS", 0) != 0;
        return o;
    }();
    return v;
}

bool g_ov_set = false;          // guarded by g_tune_mu
fp_plan_override g_ov{};        // guarded by g_tune_mu; valid when g_ov_set

const fp_plan_override &overrides_locked() {
    if (!g_ov_set) {
        g_ov = env_overrides();
        g_ov_set = true;
    }
    return g_ov;
}

Knobs knobs_for(int64_t M, int64_t K, int64_t Nw, fp_dtype act, fp_dtype wdt, bool swiglu) {
    Knobs kb;
    std::lock_guard<std::mutex> lk(g_tune_mu);
    for (const fp_tune_entry &e : g_tune) {
        if (M < e.m_lo || M > e.m_hi || e.hidden != K || e.n_cols != Nw || e.act_dtype != act ||
            e.w_dtype != wdt || (e.swiglu != 0) != swiglu)
            continue;
        kb.family = e.family;
        kb.rows = e.rows;
        kb.grid = e.grid;
        kb.splits = e.splits;
        break;
    }
    const fp_plan_override &o = overrides_locked();
    if (o.stream_target > 0) kb.target = o.stream_target;
    if (o.no_stream) {
        kb.no_stream = true;
        if (kb.family == 1) kb.family = -1;
    }
    if (o.no_prefill) {
        kb.no_prefill = true;
        if (kb.family == 2) kb.family = -1;
    }
    if (o.no_gemm16) {
        kb.no_gemm16 = true;
        if (kb.family == 4) kb.family = -1;
    }
    kb.gemm16_stages = o.gemm16_stages;
    kb.no_stream_rows = o.no_stream_rows != 0;
    kb.stream_rows_expire = o.stream_rows_expire != 0;
    if (o.stream_nr > 0) kb.rows = 64 * o.stream_nr;
    if (o.splits > 0) {
        kb.splits = o.splits;
        kb.stream_splits = o.splits;
        kb.grid = 0;
    }
    kb.fp8_tile = o.fp8_tile;
    return kb;
}

// The weight-streaming kernel's shape for one call (family 1, and the FP8
// call at decode token counts): token fragments, weight rows per
// workgroup, K chunk, the stream-K grid and the partial-sum slots.  qw:
// one-byte or 4-bit weights, dequantised or decoded in registers.
// K must be a multiple of the chunk (stream_chunk).  (Chunks twice as wide
// for E4M3, which the smaller activation registers would allow, measured
// slower on MI355X: Llama-3-8B decode QKV 20.2 -> 24.6 us, gate/up 32.5 ->
// 33.8 us: a longer pipeline ramp for the few chunks per workgroup.)
int stream_chunk(int64_t M) { return M > 32 ? 128 : 256; }

void plan_stream(Plan &p, int64_t M, int64_t K, int64_t Nw, fp_dtype wdt, bool qw, bool swiglu, const Knobs &kb,
                 bool packed) {
    p.sc.mf = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    // weight rows per workgroup 64 * nr: int8 weights at 33..64 tokens take
    // 256 when that still leaves >= 128 tiles (the A tile every workgroup
    // normalises is then amortised over twice the weight rows; measured on
    // MI355X: Llama-2-70B gate/up at 64 tokens 232 -> 186 us, while fewer
    // rows per workgroup stay faster at 1 and 16 tokens and for QKV)
    // 16-bit and E4M3 weights without the gate/up pairing at up to 32
    // tokens: 64 rows, so that more workgroups share the (smaller) weight
    // (measured on MI355X: Llama-3-8B QKV 1.1 us faster per call, E4M3 on
    // packed weights 2 us; with int8 weights, or at 33..64 tokens where the
    // A tile is four times as large, 64-row tiles are slower)
    p.sc.nr = qw && p.sc.mf >= 4 && Nw / 256 >= 128 ? 4 : 2;
    // On tile-packed weights at up to 32 tokens, int8 and MXFP4 gate/up
    // weights take 256 rows where the 256-row tiles fill 75-100 % of the
    // workgroups, one whole tile each (measured on MI355X by the tuner's HIP
    // events, Llama-2-70B gate/up, 224 tiles: int8 100.5 -> 90.2 us at 1
    // token, 97.6 -> 90.7 us at 16; MXFP4 87.2 -> 83.7 us at 16; int4 stays
    // faster at 128 rows)
    const int64_t t256 = (Nw + 255) / 256;
    if (packed && swiglu && (wdt == FP_I8 || wdt == FP_MXFP4) && p.sc.mf <= 2 && t256 <= kb.target &&
        t256 * 100 >= kb.target * 75)
        p.sc.nr = 4;
    const bool nr1_ok = !swiglu && (!qw || wdt == FP_E4M3) && p.sc.mf <= 2;   // the instantiated 64-row forms
    if (nr1_ok) p.sc.nr = 1;
    // requested rows: only the instantiated forms (64 for 16-bit and E4M3
    // weights without the gate/up pairing at up to 32 tokens, 256 for
    // quantised weights)
    if (kb.rows == 64 && nr1_ok) p.sc.nr = 1;
    if (kb.rows == 128 || (kb.rows == 256 && qw)) p.sc.nr = (int)(kb.rows / 64);
    // 32 rows (K halves: two waves per 16 rows, each streaming half of every
    // chunk) where the 32-row tiles fill three quarters of the workgroups or
    // more without outnumbering them, so that each workgroup streams one whole
    // tile where 64-row tiles would be split between two (measured on MI355X
    // with rocprofv3, Llama-3-8B QKV on tile-packed weights, 192 tiles, at 1 /
    // 16 / 32 tokens: bf16 14.1 / 14.4 / 15.8 -> 11.3 / 12.2 / 15.2 us, E4M3
    // 9.2 / 10.2 / 11.6 -> 7.6 / 8.5 / 11.3 us; where the 32-row tiles
    // outnumber the workgroups they are slower, Llama-2-7B QKV, 384 tiles:
    // 1.07 - 1.26x the 64-row time by HIP events)
    const int64_t t32 = (Nw + 31) / 32;
    const bool kh_ok = nr1_ok && K % (2 * stream_chunk(M)) == 0;
    p.sc.kh = 1;
    if (kb.rows == 0 && kh_ok && t32 <= kb.target && t32 * 100 >= kb.target * 75) {
        p.sc.nr = 1;
        p.sc.kh = 2;
    }
    if (kb.rows == 32 && kh_ok) {
        p.sc.nr = 1;
        p.sc.kh = 2;
    }
    p.sc.u = p.sc.kh * stream_chunk(M) / 32;   // K chunk 32 * u: must match the launcher
    const int nb = 64 * p.sc.nr / p.sc.kh;
    p.tiles_m = 1;
    p.tiles_n = (int)((Nw + nb - 1) / nb);
    // partial sums: 256 threads x the accumulators of 64 * nr rows (with K
    // halves, the second half's waves hold zeros)
    p.tile_elems = (int64_t)16 * p.sc.mf * 64 * p.sc.nr;
    const int64_t tiles = p.tiles_n, ksteps = K / (32 * p.sc.u), target = kb.target;
    // stream-K: `grid` workgroups take equal contiguous unit ranges of at
    // least 512 of K each (2 chunks of 256, 4 of 128; measured on MI355X:
    // shorter ranges pay the pipeline ramp too often, and 2 chunks of 256
    // beat 4 on the small QKV of Llama-2-70B's 8-way shard, 16.8 -> 14.9 us)
    const int64_t units = tiles * ksteps;
    const int64_t minc = 512 / (32 * p.sc.u);
    int64_t G = units / minc < target ? units / minc : target;
    // s workgroups per tile, each an equal 1/s of K, when that still
    // occupies most CUs and the call is short: a range that straddles two
    // tiles costs a few us (partial sums out and back, and the wait for
    // them), which outweighs the idle CUs only while the streaming itself
    // is short (measured on MI355X: Llama-3-8B gate/up, 224 tiles of 235
    // MB, s = 1: 51.3 -> 49.3 us with the weights in the last-level cache,
    // 0.3 % of the decode step with them streamed from HBM; the gate/up of
    // Llama-2-70B's 8-way shard, 56 tiles, s = 4: 24.6 -> 23.4 us;
    // Llama-2-70B int8 gate/up on row-major weights, 224 tiles of 470 MB, 6 %
    // slower so; there, an uneven 1/s of K, 32 chunks in 3, 1 us slower;
    // Llama-3-8B QKV on tile-packed weights, s = 2 of 64-row tiles (bf16) or
    // s = 4 of 128-row tiles (E4M3) on 192 workgroups: 1.5 / 3.0 us faster
    // than stream-K over 256, hence the three quarters).  On tile-packed
    // weights whole tiles also pay for weights over 256 MB at up to 32 tokens
    // (the int8 gate/up above) and an uneven 1/s of K is taken (Llama-2-70B
    // QKV, 80 tiles, s = 3 on 240 workgroups against stream-K over 256, by
    // the tuner's HIP events: int8 31.3 -> 28.5 us at 1 token, 32.1 -> 29.8
    // at 16, 48.1 -> 45.8 at 64; int4 28.4 -> 26.7 and MXFP4 30.3 -> 29.8 us
    // at 1 / 16 tokens); at 33..64 tokens a weight over 256 MB stays on
    // stream-K (int8 gate/up at 64 tokens: 127.3 us over 256 workgroups,
    // 129.3 us in whole tiles)
    const int64_t wbytes = (wdt == FP_I4 || wdt == FP_MXFP4) ? Nw * K / 2
                           : Nw * K * ((wdt == FP_I8 || wdt == FP_E4M3) ? 1 : 2);
    const bool small_w = wbytes <= (int64_t(256) << 20);
    if ((small_w || (packed && p.sc.mf <= 2)) && tiles > 0) {
        for (int64_t s = target / tiles < ksteps / minc ? target / tiles : ksteps / minc; s >= 1; --s) {
            if (tiles * s * 100 < target * 75) break;
            if (packed || ksteps % s == 0) {
                G = tiles * s;
                break;
            }
        }
    }
    if (kb.grid > 0) G = kb.grid;
    if (kb.stream_splits > 0) G = tiles * kb.stream_splits;
    if (G > units) G = units;
    if (G < 1) G = 1;
    p.grid = (int)G;
    // the most workgroups that share one tile
    auto owner = [&](int64_t v) { return ((v + 1) * G - 1) / units; };
    int64_t most = 1;
    for (int64_t t = 0; t < tiles; ++t) {
        const int64_t n = owner(t * ksteps + ksteps - 1) - owner(t * ksteps) + 1;
        if (n > most) most = n;
    }
    p.slots = (int)most;
}

// Decode token counts (M <= 64, 16-bit activations) use the weight-streaming
// kernel, which spreads (tile, K chunk) units evenly over one workgroup per
// CU; token counts above 64 the 128 x 512 prefill kernel while its 32-bit
// buffer offsets reach (activations and weights under 4 GiB each);
// everything else the tiled kernel (64-bit offsets).  When a tiled grid would hold too few workgroups, K is
// split.  Partial sums are reduced by the last contributor to arrive, in a
// fixed order.
// A tuning-table entry or FUSEDPROJ_* environment variables override the
// choices (Knobs); the workspace query and the call read them alike.  A
// requested family is used only where it can take the call: the streaming
// kernel needs 16-bit activations, M <= 64 and K a multiple of 256; the
// 128 x 512 kernel 16-bit activations and operands under 4 GiB.
// The 256 x 256 GEMM (family 4) takes 16-bit weights of the activation
// dtype from 512 tokens on (fewer leave too much of a 256-row tile as
// padding), when the call's 256 x 256 tiles fill the CUs at least once (at these
// sizes the 128 x 512 kernel is bound by the x and residual bytes it re-reads
// per column tile); the rows it reads are formed once by the row pass, in a
// workspace region of M * K 16-bit values (form_rows; the down projection
// reads its input as is).  Where that region would exceed ws_cap (the
// allocation-free entry point's static scratch) the 128 x 512 kernel takes
// the call instead.
Plan make_plan(int64_t M, int64_t K, int64_t Nw, fp_dtype act, fp_dtype wdt, bool swiglu, bool form_rows = true,
               size_t ws_cap = SIZE_MAX, int wl = fp::WL_ROWS) {
    Plan p;
    const Knobs kb = knobs_for(M, K, Nw, act, wdt, swiglu);
    if (wdt == FP_E4M3) {
        // FP8 W8A8: one family whatever the token count.  Up to 32 / 64
        // tokens: 32 x 256 / 64 x 256 tiles (the four waves share the token
        // rows), K split while fewer than one workgroup per CU runs and each
        // workgroup still streams at least 256 KB of weights, at most 8 ways
        // and at least 4 K steps of 128 per split (measured on MI355X,
        // Llama-3-8B decode shapes: gate/up, 112 tiles, 41.7 / 31.0 / 33.8 /
        // 46.6 us at 1 / 2 / 4 / 8 splits; QKV, 24 tiles, 26.2 / 19.2 / 15.5 /
        // 17.2 / 25.0 us at 1 / 2 / 4 / 8 / 16: the partial sums cost more
        // than a second workgroup per CU gains).  More tokens: 256 x 256
        // tiles (SwiGLU: 128 gate + 128 up rows), one workgroup per CU, when
        // they fill at least one round of CUs; otherwise 128 x 128 tiles, two
        // workgroups per CU, K split while fewer than two rounds of
        // workgroups run (same limits).  The fp8_tile override (32, 64,
        // 128 or 256) forces a tile.
        p.family = 3;
        // Up to 64 tokens with K a multiple of the chunk and no tile
        // requested, on tile-packed weights (or when requested, family 1):
        // the weight-streaming kernel on the codes, E4M3 weights decoded in
        // registers, shaped like a call with int8 weights (the same bytes per
        // weight).  Measured on MI355X, Llama-3-8B decode step (both calls):
        // packed weights 50.4 us streaming against 65.2 us in the FP8 tiles
        // (whose 8-row LDS loads lose on the packed order); row-major
        // weights 57.1 us streaming against 55.1 us in the tiles, which stay
        // the default there
        if (M <= 64 && K % stream_chunk(M) == 0 && kb.fp8_tile == 0 && !kb.no_stream &&
            (kb.family == 1 || (kb.family == -1 && wl != fp::WL_ROWS))) {
            p.stream8 = true;
            plan_stream(p, M, K, Nw, wdt, true, swiglu, kb, wl != fp::WL_ROWS);
            const int64_t tiles = p.tiles_n;
            size_t off = 0;
            p.ctr_off = off;
            if (p.slots > 1) off = align256(off + (size_t)tiles * 4);
            p.part_off = off;
            if (p.slots > 1) off = align256(off + (size_t)tiles * p.slots * p.tile_elems * 4);
            p.q_off = off;
            off = align256(off + (size_t)M * (size_t)K);
            p.qs_off = off;
            off = align256(off + (size_t)M * 4);
            p.total = off;
            return p;
        }
        const int64_t big_tiles = ((M + 255) / 256) * (swiglu ? (Nw / 2 + 127) / 128 : (Nw + 255) / 256);
        const long tile_env = kb.fp8_tile;
        if (tile_env == 32) p.tile8 = fp::G8_32x256;
        else if (tile_env == 64) p.tile8 = fp::G8_64x256;
        else if (tile_env == 128) p.tile8 = fp::G8_128x128;
        else if (tile_env == 256) p.tile8 = fp::G8_256x256;
        else if (M <= 32) p.tile8 = fp::G8_32x256;
        else if (M <= 64) p.tile8 = fp::G8_64x256;
        else p.tile8 = big_tiles >= 256 ? fp::G8_256x256 : fp::G8_128x128;
        static const int BMS[4] = {128, 256, 32, 64}, BNS[4] = {128, 256, 256, 256};
        const int bm = BMS[p.tile8], bn = BNS[p.tile8];
        p.tiles_m = (int)((M + bm - 1) / bm);
        p.tiles_n = (int)(swiglu ? (Nw / 2 + bn / 2 - 1) / (bn / 2) : (Nw + bn - 1) / bn);
        p.tile_elems = (int64_t)bm * bn;
        const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n, ksteps = K / 128;
        int64_t s = tiles > 0 ? (p.tile8 == fp::G8_128x128 ? 512 : 256) / tiles : 1;
        const int64_t cap = ksteps / 4 < 8 ? ksteps / 4 : 8;
        if (s > cap) s = cap;
        if (p.tile8 == fp::G8_32x256 || p.tile8 == fp::G8_64x256) {
            const int64_t by_bytes = tiles > 0 ? Nw * K / (tiles * (int64_t(256) << 10)) : 1;
            if (s > by_bytes) s = by_bytes;
        }
        if (kb.splits > 0) s = kb.splits < ksteps ? kb.splits : ksteps;
        if (s < 1 || p.tile8 == fp::G8_256x256) s = 1;   // the 256 x 256 kernel does not split K
        p.splits = p.slots = (int)s;
        size_t off = 0;
        p.ctr_off = off;
        if (p.slots > 1) off = align256(off + (size_t)tiles * 4);
        p.part_off = off;
        if (p.slots > 1) off = align256(off + (size_t)tiles * p.slots * p.tile_elems * 4);
        p.q_off = off;
        off = align256(off + (size_t)M * (size_t)K);
        p.qs_off = off;
        off = align256(off + (size_t)M * 4);
        p.total = off;
        return p;
    }
    const bool w4 = wdt == FP_I4 || wdt == FP_MXFP4;   // 4-bit weights, [N, K/2] bytes
    const fp_dtype wdt_stored = wdt;
    const size_t rows_bytes = form_rows ? align256((size_t)M * (size_t)K * 2) : 0;
    const bool stream_elig = act != FP_F32 && M <= 64 && K % 256 == 0 && rows_bytes <= ws_cap;
    const bool prefill_elig = act != FP_F32 && M * K * 2 < (int64_t(1) << 32) && Nw * K * 2 < (int64_t(1) << 32);
    const int64_t tiles256 = ((M + 255) / 256) * (swiglu ? (Nw / 2 + 127) / 128 : (Nw + 255) / 256);
    const bool g16_elig = prefill_elig && wdt == act && rows_bytes <= ws_cap;
    int fam;
    if (kb.family == 0 || (kb.family == 1 && stream_elig) || (kb.family == 2 && prefill_elig) ||
        (kb.family == 4 && g16_elig))
        fam = kb.family;
    else if (stream_elig && !kb.no_stream)
        fam = 1;
    else if (g16_elig && M >= 512 && tiles256 >= 256 && !kb.no_gemm16)
        fam = 4;
    else if (prefill_elig && M > 64 && !kb.no_prefill)
        fam = 2;
    else
        fam = 0;
    if (fam == 4) {
        p.family = 4;
        // two stages of K 64 need an even number of K steps (K a multiple
        // of 128); otherwise four stages of K 32
        const bool two = K % 128 == 0;
        p.nst = kb.gemm16_stages == 5 ? 5 : kb.gemm16_stages == 4 || !two ? 4 : 2;
        p.tiles_m = (int)((M + 255) / 256);
        p.tiles_n = (int)(swiglu ? (Nw / 2 + 127) / 128 : (Nw + 255) / 256);
        p.tile_elems = 256 * 256;
        p.rows = form_rows;
        p.rows_off = 0;
        p.total = rows_bytes;
        return p;
    }
    // int4 / MXFP4 weights: dequantised in registers by the streaming and 128 x 512
    // kernels; for the tiled family dequantised into the workspace first and
    // then run as bf16 weights
    if (w4 && fam == 0) wdt = FP_BF16;
    const bool qw = wdt == FP_I8 || wdt == FP_I4 || wdt == FP_MXFP4;   // weights dequantised in the loader
    int64_t tiles, ksteps, target;
    if (fam == 1) {
        p.family = 1;
        plan_stream(p, M, K, Nw, wdt, qw, swiglu, kb, wl != fp::WL_ROWS);
        tiles = p.tiles_n;
    } else if (fam == 2) {
        p.family = 2;
        p.tiles_m = (int)((M + 127) / 128);
        p.tiles_n = (int)((Nw + 511) / 512);
        p.tile_elems = 128 * 512;
        tiles = (int64_t)p.tiles_m * p.tiles_n;
        ksteps = K / 64;
        target = 256;
    } else {
        if (M <= 16) p.tile = fp::TILE_DEC16;
        else if (M <= 32) p.tile = fp::TILE_DEC32;
        else if (M <= 64) p.tile = fp::TILE_DEC64;
        else p.tile = fp::TILE_PF128;
        const fp::TileShape ts = fp::tile_shape(p.tile);
        p.tiles_m = (int)((M + ts.bm - 1) / ts.bm);
        p.tiles_n = (int)((Nw + ts.bn - 1) / ts.bn);
        p.tile_elems = (int64_t)ts.bm * ts.bn;
        tiles = (int64_t)p.tiles_m * p.tiles_n;
        ksteps = K / ts.bk;
        target = 512;
    }
    if (p.family != 1) {
        int64_t s = 1;
        if (p.family == 2) {
            // as many splits as still fit one round of workgroups (one per CU):
            // a second round costs more than the idle CUs of the first.  At
            // most 8 (a 128 x 512 partial tile is 256 KB each way).  Measured
            // on MI355X, Llama-2-70B int8 at 256 tokens: QKV (40 tiles) 115 ->
            // 103 us with 6 splits instead of 4; gate/up (224 tiles) 368 ->
            // 322 us unsplit instead of 2 splits.
            s = tiles > 0 ? target / tiles : 1;
            const int64_t cap = ksteps / 4 < 8 ? ksteps / 4 : 8;
            if (s > cap) s = cap;
            if (s < 1) s = 1;
        } else if (tiles > 0 && tiles < target) {
            s = (target + tiles - 1) / tiles;
        }
        int64_t smax = p.family == 2 ? 8 : ksteps / 4;
        if (smax < 1) smax = 1;
        if (s > smax) s = smax;
        if (s > 16) s = 16;
        if (s < 1) s = 1;
        if (kb.splits > 0) s = kb.splits < ksteps ? kb.splits : ksteps;
        p.splits = (int)s;
        p.slots = (int)s;
    }

    size_t off = 0;
    if (p.family == 1 && form_rows) {
        // the streaming kernel reads the rows the row pass forms (normalised,
        // in the activation dtype) instead of normalising in every workgroup;
        // the row pass runs inside the streaming kernel (sc.rp: M extra
        // workgroups, one per token, while the others' first weights are in
        // flight) for rows of up to 8192 values where the extra workgroups
        // fit in the workgroup budget next to the streaming grid (on CUs it
        // leaves idle), else as a launch of its own (also under graph
        // capture: see run)
        p.rows = true;
        p.rows_off = off;
        off += rows_bytes;
        p.flags_off = off;
        off = align256(off + (size_t)M * 8);
        p.sc.rp = K <= 8192 && p.grid + M <= kb.target && wdt != FP_E4M3 && !kb.no_stream_rows ? 1 : 0;
        p.rows_expire = kb.stream_rows_expire;
    } else {
        p.stats_off = off;
        off = align256(off + (size_t)M * 8);
    }
    p.ctr_off = off;
    if (p.slots > 1) off = align256(off + (size_t)tiles * 4);
    p.part_off = off;
    if (p.slots > 1) off = align256(off + (size_t)tiles * p.slots * p.tile_elems * 4);
    (void)wdt_stored;
    // the tiled kernel reads row-major weights only: tile-packed ones are
    // unpacked into the workspace first (before any dequantisation)
    if (wl != fp::WL_ROWS && p.family == 0) {
        p.unpack = true;
        p.unpack_off = off;
        off = align256(off + (size_t)Nw * (size_t)(w4 ? K / 2 : K * act_size(wdt_stored)));
    }
    if (w4 && p.family == 0) {
        p.deq = true;
        p.deq_off = off;
        off = align256(off + (size_t)Nw * (size_t)K * 2);
    }
    p.total = off;
    return p;
}

// A call's w_dtype: the element type in the low byte, the storage layout in
// the layout bits (FP_LAYOUT_*)
void split_wdt(fp_dtype w_dtype, fp_dtype &base, int &layout) {
    base = (fp_dtype)((int)w_dtype & 0xFF);
    const int bits = (int)w_dtype & ~0xFF;
    layout = bits == 0 ? fp::WL_ROWS : bits == FP_LAYOUT_PACKED ? fp::WL_PACKED
           : bits == FP_LAYOUT_PACKED_GATE_UP ? fp::WL_PACKED_GATE_UP : -1;
}

// bytes of one weight row of K elements
int64_t row_bytes(fp_dtype wdt, int64_t K) {
    return (wdt == FP_I4 || wdt == FP_MXFP4) ? K / 2 : K * act_size(wdt);
}

// The shape rules of the tile-packed layouts (fused_pack_weight): whole
// 128-row groups (gate/up pairs: whole 64-row halves) of whole 64-byte slices
fp_status check_layout(int layout, fp_dtype wdt, int64_t n_rows, int64_t K, int64_t gate_rows) {
    if (layout < 0) return fail(FP_E_DTYPE, "w_dtype carries unknown layout bits");
    if (layout == fp::WL_ROWS) return FP_OK;
    if (wdt == FP_F32) return fail(FP_E_DTYPE, "tile-packed weights are 16-bit, int8, int4, E4M3 or MXFP4");
    if (row_bytes(wdt, K) % 64 != 0)
        return fail(FP_E_SHAPE, "tile-packed weights need rows of a multiple of 64 bytes (K = %lld)", (long long)K);
    if (layout == fp::WL_PACKED && n_rows % 128 != 0)
        return fail(FP_E_SHAPE, "tile-packed weights need a multiple of 128 rows (%lld)", (long long)n_rows);
    if (layout == fp::WL_PACKED_GATE_UP && (gate_rows <= 0 || gate_rows % 64 != 0 || n_rows != 2 * gate_rows))
        return fail(FP_E_SHAPE, "gate/up-packed weights are for the SwiGLU call, with ffn a multiple of 64 "
                    "(ffn = %lld)", (long long)gate_rows);
    return FP_OK;
}

// ---------------------------------------------------------------------------
// validation helpers
// ---------------------------------------------------------------------------
struct Range {
    const char *name;
    uintptr_t lo, hi;   // [lo, hi)
};

bool overlaps(const Range &a, const Range &b) {
    return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo;
}

fp_status check_alias(const std::vector<Range> &ins, const std::vector<Range> &outs) {
    for (size_t i = 0; i < outs.size(); ++i) {
        for (const Range &r : ins)
            if (overlaps(outs[i], r))
                return fail(FP_E_ALIAS, "output '%s' overlaps input '%s'", outs[i].name, r.name);
        for (size_t j = i + 1; j < outs.size(); ++j)
            if (overlaps(outs[i], outs[j]))
                return fail(FP_E_ALIAS, "output '%s' overlaps output '%s'", outs[i].name, outs[j].name);
    }
    return FP_OK;
}

Range rng(const char *name, const void *p, int64_t bytes) {
    uintptr_t lo = (uintptr_t)p;
    return Range{name, lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

fp_status check_dtypes(fp_dtype act, fp_dtype wdt, fp_dtype odt) {
    if (act != FP_F32 && act != FP_F16 && act != FP_BF16)
        return fail(FP_E_DTYPE, "act_dtype %d not in {F32, F16, BF16}", (int)act);
    if (!(wdt == act || ((wdt == FP_I8 || wdt == FP_I4 || wdt == FP_MXFP4) && act == FP_BF16) ||
          (wdt == FP_E4M3 && (act == FP_BF16 || act == FP_F16))))
        return fail(FP_E_DTYPE, "w_dtype %d must equal act_dtype %d, or be I8 / I4 with BF16 activations, "
                    "or E4M3 with BF16 / F16 activations", (int)wdt, (int)act);
    if (!(odt == act || odt == FP_F32))
        return fail(FP_E_DTYPE, "out_dtype %d must equal act_dtype or be F32", (int)odt);
    return FP_OK;
}

// ---------------------------------------------------------------------------
// event profiler
// ---------------------------------------------------------------------------
struct ProfRec {
    char name[64];   // a copy: the name functions reuse one buffer per thread
    hipEvent_t a, b;
};
bool g_prof = false;
std::vector<ProfRec> g_recs;

struct ProfScope {
    ProfRec rec{};
    hipStream_t s;
    bool on;
    ProfScope(const char *name, hipStream_t st) : s(st), on(g_prof) {
        if (!on) return;
        snprintf(rec.name, sizeof rec.name, "%s", name);
        if (hipEventCreate(&rec.a) != hipSuccess || hipEventCreate(&rec.b) != hipSuccess) { on = false; return; }
        (void)hipEventRecord(rec.a, s);
    }
    ~ProfScope() {
        if (!on) return;
        (void)hipEventRecord(rec.b, s);
        g_recs.push_back(rec);
    }
};

fp_status hip_fail(hipError_t e, const char *what) {
    return fail(FP_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// the shared body of both projection entry points
// ---------------------------------------------------------------------------
struct Common {
    const void *x, *residual;
    void *h_out;
    const void *gamma, *beta;
    fp_norm norm;
    float eps;
    const void *w;
    const void *w_scale;      // fp32 (int8, int4, E4M3) or E8M0 bytes (MXFP4)
    const void *bias;
    int64_t M, K, Nw;
    fp_dtype act, wdt, odt;
    void *ws;
    size_t ws_bytes;
    hipStream_t stream;
    int wl = fp::WL_ROWS;     // storage layout of w (fp::WLayout; -1: unknown bits)
    int64_t gate_rows = 0;    // the SwiGLU call: ffn (the gate/up pairing of a packed w)
};

fp_status validate_common(const Common &c, const char *wname) {
    if (c.M < 0) return fail(FP_E_SHAPE, "M = %lld is negative", (long long)c.M);
    if (c.K <= 0 || c.K % 64 != 0)
        return fail(FP_E_SHAPE, "hidden = %lld must be a positive multiple of 64", (long long)c.K);
    if (c.norm != FP_NORM_NONE && c.norm != FP_NORM_RMS && c.norm != FP_NORM_LAYER)
        return fail(FP_E_ARG, "norm = %d is not a fp_norm value", (int)c.norm);
    fp_status st = check_dtypes(c.act, c.wdt, c.odt);
    if (st != FP_OK) return st;
    st = check_layout(c.wl, c.wdt, c.Nw, c.K, c.gate_rows);
    if (st != FP_OK) return st;
    if (!c.x && c.M > 0) return fail(FP_E_NULL, "x is NULL");
    if (!c.w) return fail(FP_E_NULL, "%s is NULL", wname);
    if (c.norm != FP_NORM_NONE && !c.gamma) return fail(FP_E_NULL, "gamma is NULL but norm is not NONE");
    if ((c.wdt == FP_I8 || c.wdt == FP_I4 || c.wdt == FP_E4M3 || c.wdt == FP_MXFP4) && !c.w_scale)
        return fail(FP_E_NULL, "w_scale is NULL for int8 / int4 / E4M3 / MXFP4 weights");
    if ((c.wdt == FP_I4 || c.wdt == FP_E4M3) && c.K % 128 != 0)
        return fail(FP_E_SHAPE, "hidden = %lld must be a multiple of 128 for int4 / E4M3 weights", (long long)c.K);
    if (c.wdt == FP_E4M3 && (c.M * c.K >= (int64_t(1) << 32) || c.Nw * c.K >= (int64_t(1) << 32)))
        return fail(FP_E_SHAPE, "E4M3: M * hidden and the weight's rows * hidden must be below 2^32");
    if (!(c.eps >= 0.0f) || c.eps > 1e30f) return fail(FP_E_ARG, "eps must be a finite value >= 0");
    const void *ptrs[] = {c.x, c.residual, c.h_out, c.gamma, c.beta, c.w, c.w_scale, c.bias, c.ws};
    const char *names[] = {"x", "residual", "h_out", "gamma", "beta", wname, "w_scale", "bias", "workspace"};
    for (int i = 0; i < 9; ++i)
        if (ptrs[i] && !aligned16(ptrs[i])) return fail(FP_E_ALIGN, "%s is not 16-byte aligned", names[i]);
    return FP_OK;
}

void add_inputs(const Common &c, std::vector<Range> &ins, const char *wname) {
    const int ea = act_size(c.act), ew = act_size(c.wdt);
    ins.push_back(rng("x", c.x, c.M * c.K * ea));
    if (c.residual) ins.push_back(rng("residual", c.residual, c.M * c.K * ea));
    if (c.gamma && c.norm != FP_NORM_NONE) ins.push_back(rng("gamma", c.gamma, c.K * ea));
    if (c.beta && c.norm == FP_NORM_LAYER) ins.push_back(rng("beta", c.beta, c.K * ea));
    ins.push_back(rng(wname, c.w, (c.wdt == FP_I4 || c.wdt == FP_MXFP4) ? c.Nw * c.K / 2 : c.Nw * c.K * ew));
    if (c.w_scale && (c.wdt == FP_I8 || c.wdt == FP_E4M3)) ins.push_back(rng("w_scale", c.w_scale, c.Nw * 4));
    if (c.w_scale && c.wdt == FP_I4) ins.push_back(rng("w_scale", c.w_scale, c.Nw * (c.K / 128) * 4));
    if (c.w_scale && c.wdt == FP_MXFP4) ins.push_back(rng("w_scale", c.w_scale, c.Nw * (c.K / 32)));
    if (c.bias) ins.push_back(rng("bias", c.bias, c.Nw * ea));
}

fp_status run_fp8(const Common &c, const Plan &plan, fp::ProjArgs &pa) {
    char *ws = (char *)c.ws;
    const int act = act_code(c.act);
    unsigned *ctr = plan.slots > 1 ? (unsigned *)(ws + plan.ctr_off) : nullptr;
    unsigned char *codes = (unsigned char *)(ws + plan.q_off);
    float *qscale = (float *)(ws + plan.qs_off);
    fp::StatsArgs sa{};
    sa.x = c.x;
    sa.res = c.residual;
    sa.h_out = c.h_out;
    sa.norm = (int)c.norm;
    sa.eps = c.eps;
    sa.M = c.M;
    sa.K = c.K;
    sa.counters = ctr;
    sa.n_counters = plan.slots > 1 ? plan.tiles_m * plan.tiles_n : 0;
    sa.gamma = c.gamma;
    sa.beta = c.norm == FP_NORM_LAYER ? c.beta : nullptr;
    sa.codes = codes;
    sa.qscale = qscale;
    {
        ProfScope ps(fp::quant8_kernel_name(act), c.stream);
        hipError_t e = fp::launch_quant8(act, sa, c.stream);
        if (e != hipSuccess) return hip_fail(e, "quant8_kernel launch");
    }
    pa.x = codes;
    pa.a_scale = qscale;
    pa.w = c.w;
    pa.w_layout = c.wl;
    pa.w_scale = (const float *)c.w_scale;
    pa.bias = c.bias;
    pa.out_f32 = c.odt == FP_F32;
    pa.M = c.M;
    pa.K = c.K;
    pa.Nw = c.Nw;
    pa.tiles_m = plan.tiles_m;
    pa.tiles_n = plan.tiles_n;
    pa.splits = plan.splits;
    pa.slots = plan.slots;
    pa.partials = plan.slots > 1 ? (float *)(ws + plan.part_off) : nullptr;
    pa.counters = ctr;
    if (plan.stream8) {
        pa.res = nullptr;
        pa.stats = nullptr;
        pa.norm = 0;
        ProfScope ps(fp::stream_kernel_name(act, 4, plan.sc, pa.epi), c.stream);
        hipError_t e = fp::launch_stream(act, 4, plan.sc, pa, plan.grid, c.stream);
        if (e != hipSuccess) return hip_fail(e, "stream_kernel launch");
        return FP_OK;
    }
    ProfScope ps(fp::gemm8_kernel_name(act, plan.tile8, pa.epi), c.stream);
    hipError_t e = fp::launch_gemm8(act, plan.tile8, pa, c.stream);
    if (e != hipSuccess) return hip_fail(e, "gemm8_kernel launch");
    return FP_OK;
}

// family 4: the row pass (h_out, the normalised rows) unless the call's
// input is the operand, then the 256 x 256 GEMM on the rows
fp_status run_gemm16(const Common &c, const Plan &plan, fp::ProjArgs &pa) {
    const int act = act_code(c.act);
    const void *rows = c.x;
    if (plan.rows) {
        fp::StatsArgs sa{};
        sa.x = c.x;
        sa.res = c.residual;
        sa.h_out = c.h_out;
        sa.norm = (int)c.norm;
        sa.eps = c.eps;
        sa.M = c.M;
        sa.K = c.K;
        sa.gamma = c.gamma;
        sa.beta = c.norm == FP_NORM_LAYER ? c.beta : nullptr;
        sa.rows = (char *)c.ws + plan.rows_off;
        ProfScope ps(fp::norm_kernel_name(act), c.stream);
        hipError_t e = fp::launch_norm(act, sa, c.stream);
        if (e != hipSuccess) return hip_fail(e, "norm_kernel launch");
        rows = sa.rows;
    }
    pa.x = rows;
    pa.res = nullptr;
    pa.stats = nullptr;
    pa.norm = 0;
    pa.w = c.w;
    pa.w_layout = c.wl;
    pa.bias = c.bias;
    pa.out_f32 = c.odt == FP_F32;
    pa.M = c.M;
    pa.K = c.K;
    pa.Nw = c.Nw;
    pa.tiles_m = plan.tiles_m;
    pa.tiles_n = plan.tiles_n;
    pa.splits = 1;
    pa.slots = 1;
    ProfScope ps(fp::gemm16_kernel_name(act, plan.nst, pa.epi), c.stream);
    hipError_t e = fp::launch_gemm16(act, plan.nst, pa, c.stream);
    if (e != hipSuccess) return hip_fail(e, "gemm16_kernel launch");
    return FP_OK;
}

// true while work on s is being captured into a HIP graph (or when that
// cannot be told: the separate row pass is right in either case)
bool stream_capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;
    return st != hipStreamCaptureStatusNone;
}

// A tag for one launch of the streaming kernel's own row pass: distinct for
// every launch in the process (a counter), and with its top bit set and a
// random start, so that neither a tag of an earlier launch nor other data
// left in a reused workspace equals it
unsigned long long next_rp_tag() {
    static std::atomic<unsigned long long> next{[] {
        std::random_device rd;
        return ((unsigned long long)rd() << 32 | rd()) | (1ull << 63);
    }()};
    return next.fetch_add(1, std::memory_order_relaxed);
}

fp_status run(const Common &c, const Plan &plan, fp::ProjArgs &pa) {
    if (c.M == 0) return FP_OK;
    if (plan.family == 3) return run_fp8(c, plan, pa);
    if (plan.family == 4) return run_gemm16(c, plan, pa);
    char *ws = (char *)c.ws;
    const int act = act_code(c.act);
    float2 *stats = c.norm != FP_NORM_NONE && !plan.rows ? (float2 *)(ws + plan.stats_off) : nullptr;
    unsigned *ctr = plan.slots > 1 ? (unsigned *)(ws + plan.ctr_off) : nullptr;
    const int n_ctr = plan.slots > 1 ? plan.tiles_m * plan.tiles_n : 0;
    // the streaming kernel forms the rows itself only outside graph capture:
    // a replay repeats the launch's tag, so the flags the previous replay
    // left would read as ready
    fp::StreamCfg sc = plan.sc;
    if (plan.family != 1 || !plan.rows || stream_capturing(c.stream)) sc.rp = 0;

    if (plan.rows) {
        // the row pass: h_out, the normalised rows (the A operand), and the
        // split-K counters cleared -- a launch of its own, or the streaming
        // kernel's first workgroups (sc.rp)
        fp::StatsArgs sa{};
        sa.x = c.x;
        sa.res = c.residual;
        sa.h_out = c.h_out;
        sa.norm = (int)c.norm;
        sa.eps = c.eps;
        sa.M = c.M;
        sa.K = c.K;
        sa.counters = ctr;
        sa.n_counters = n_ctr;
        sa.gamma = c.gamma;
        sa.beta = c.norm == FP_NORM_LAYER ? c.beta : nullptr;
        sa.rows = ws + plan.rows_off;
        if (sc.rp) {
            pa.rp = sa;
            pa.rp_flags = (unsigned long long *)(ws + plan.flags_off);
            pa.rp_tag = next_rp_tag();
            pa.rp_wait_tag = pa.rp_tag;
            pa.rp_spin = 1 << 20;
            if (plan.rows_expire) {   // tests of the bounded wait: a tag no launch publishes
                pa.rp_wait_tag = pa.rp_tag ^ (1ull << 62);
                pa.rp_spin = 64;
            }
        } else {
            ProfScope ps(fp::norm_kernel_name(act), c.stream);
            hipError_t e = fp::launch_norm(act, sa, c.stream);
            if (e != hipSuccess) return hip_fail(e, "norm_kernel launch");
        }
    } else if (stats || c.h_out || n_ctr) {
        fp::StatsArgs sa;
        sa.x = c.x;
        sa.res = c.residual;
        sa.h_out = c.h_out;
        sa.stats = stats;
        sa.norm = (int)c.norm;
        sa.eps = c.eps;
        sa.M = c.M;
        sa.K = c.K;
        sa.counters = ctr;
        sa.n_counters = n_ctr;
        ProfScope ps(fp::stats_kernel_name(act), c.stream);
        hipError_t e = fp::launch_stats(act, sa, c.stream);
        if (e != hipSuccess) return hip_fail(e, "stats_kernel launch");
    }
    pa.x = plan.rows ? (const void *)(ws + plan.rows_off) : c.x;
    pa.res = plan.rows ? nullptr : c.residual;
    pa.stats = stats;
    pa.gamma = c.gamma;
    pa.beta = c.norm == FP_NORM_LAYER ? c.beta : nullptr;
    pa.norm = plan.rows ? 0 : (int)c.norm;
    pa.w = c.w;
    pa.w_layout = c.wl;
    pa.w_scale = (const float *)c.w_scale;
    const bool wi8 = c.wdt == FP_I8;
    const int wq = c.wdt == FP_I8 ? 1 : plan.deq ? 0 : c.wdt == FP_I4 ? 2 : c.wdt == FP_MXFP4 ? 3 : 0;
    const void *wsrc = c.w;   // row-major weights for the dequantisation
    if (plan.unpack) {
        void *wu = ws + plan.unpack_off;
        ProfScope ps(fp::pack_kernel_name(true), c.stream);
        hipError_t e = fp::launch_pack(c.w, wu, c.Nw, row_bytes(c.wdt, c.K), c.gate_rows, c.wl, true, c.stream);
        if (e != hipSuccess) return hip_fail(e, "unpack_kernel launch");
        pa.w = wsrc = wu;
        pa.w_layout = fp::WL_ROWS;
    }
    if (plan.deq) {
        void *wb = ws + plan.deq_off;
        if (c.wdt == FP_MXFP4) {
            ProfScope ps(fp::dequant_mxfp4_kernel_name(), c.stream);
            hipError_t e = fp::launch_dequant_mxfp4((const uint8_t *)wsrc, (const uint8_t *)c.w_scale, wb, c.Nw, c.K,
                                                    c.stream);
            if (e != hipSuccess) return hip_fail(e, "dequant_mxfp4_kernel launch");
        } else {
            ProfScope ps(fp::dequant_i4_kernel_name(), c.stream);
            hipError_t e = fp::launch_dequant_i4((const uint8_t *)wsrc, (const float *)c.w_scale, wb, c.Nw, c.K,
                                                 c.stream);
            if (e != hipSuccess) return hip_fail(e, "dequant_i4_kernel launch");
        }
        pa.w = wb;
        pa.w_scale = nullptr;
    }
    pa.bias = c.bias;
    pa.out_f32 = c.odt == FP_F32;
    pa.M = c.M;
    pa.K = c.K;
    pa.Nw = c.Nw;
    pa.tiles_m = plan.tiles_m;
    pa.tiles_n = plan.tiles_n;
    pa.splits = plan.splits;
    pa.slots = plan.slots;
    pa.partials = plan.slots > 1 ? (float *)(ws + plan.part_off) : nullptr;
    pa.counters = ctr;
    if (plan.family == 1) {
        ProfScope ps(fp::stream_kernel_name(act, wq, sc, pa.epi), c.stream);
        hipError_t e = fp::launch_stream(act, wq, sc, pa, plan.grid, c.stream);
        if (e != hipSuccess) return hip_fail(e, "stream_kernel launch");
    } else if (plan.family == 2) {
        ProfScope ps(fp::prefill_kernel_name(act, wq, pa.epi), c.stream);
        hipError_t e = fp::launch_prefill(act, wq, pa, c.stream);
        if (e != hipSuccess) return hip_fail(e, "prefill_kernel launch");
    } else {
        ProfScope ps(fp::proj_kernel_name(act, wi8, plan.tile, pa.epi), c.stream);
        hipError_t e = fp::launch_tiled(act, wi8, plan.tile, pa, c.stream);
        if (e != hipSuccess) return hip_fail(e, "proj_kernel launch");
    }
    return FP_OK;
}

fp_status check_workspace(const Common &c, const Plan &plan, std::vector<Range> &outs) {
    if (c.M == 0) return FP_OK;
    if (plan.total > 0) {
        if (!c.ws) return fail(FP_E_WORKSPACE, "workspace is NULL; %zu bytes are needed", plan.total);
        if (c.ws_bytes < plan.total)
            return fail(FP_E_WORKSPACE, "workspace has %zu bytes; %zu are needed", c.ws_bytes, plan.total);
        outs.push_back(rng("workspace", c.ws, (int64_t)plan.total));
    }
    return FP_OK;
}

}  // namespace

extern "C" {

size_t fp_workspace_bytes(int64_t M, int64_t hidden, int64_t n_cols, fp_dtype act_dtype,
                          fp_dtype w_dtype) {
    fp_dtype wdt;
    int wl;
    split_wdt(w_dtype, wdt, wl);
    if (M < 0 || hidden <= 0 || hidden % 64 != 0 || n_cols <= 0 || wl < 0) return 0;
    if (check_dtypes(act_dtype, wdt, act_dtype) != FP_OK) return 0;
    if ((wdt == FP_I4 || wdt == FP_E4M3) && hidden % 128 != 0) return 0;
    if (M == 0) return 0;
    // gate/up-packed weights only go to the SwiGLU call
    const size_t a = wl == fp::WL_PACKED_GATE_UP ? 0 : make_plan(M, hidden, n_cols, act_dtype, wdt, false, true,
                                                                 SIZE_MAX, wl).total;
    const size_t b = make_plan(M, hidden, n_cols, act_dtype, wdt, true, true, SIZE_MAX, wl).total;
    return a > b ? a : b;
}

size_t fp_down_workspace_bytes(int64_t M, int64_t ffn, int64_t hidden, fp_dtype act_dtype, fp_dtype w_dtype) {
    fp_dtype wdt;
    int wl;
    split_wdt(w_dtype, wdt, wl);
    if (M <= 0 || ffn <= 0 || ffn % 64 != 0 || hidden <= 0 || wl < 0) return 0;
    if (check_dtypes(act_dtype, wdt, act_dtype) != FP_OK) return 0;
    if ((wdt == FP_I4 || wdt == FP_E4M3) && ffn % 128 != 0) return 0;
    return make_plan(M, ffn, hidden, act_dtype, wdt, false, false, SIZE_MAX, wl).total;
}

}  // extern "C"

namespace {

fp_status add_norm_qkv(const void *x, const void *residual, void *h_out, const void *gamma,
                       const void *beta, fp_norm norm, float eps, const void *w_qkv,
                       const void *w_scale, const void *bias, void *q, void *k, void *v,
                       int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads,
                       int64_t head_dim, fp_dtype act_dtype, fp_dtype w_dtype,
                       fp_dtype out_dtype, void *workspace, size_t workspace_bytes,
                       void *hip_stream, bool head_major, fp::WorkspaceSource source = nullptr) {
    if (n_heads <= 0 || n_kv_heads <= 0 || n_heads % n_kv_heads != 0)
        return fail(FP_E_SHAPE, "n_heads = %lld, n_kv_heads = %lld: both must be > 0 and n_heads a multiple of n_kv_heads",
                    (long long)n_heads, (long long)n_kv_heads);
    if (head_dim <= 0 || head_dim % 16 != 0)
        return fail(FP_E_SHAPE, "head_dim = %lld must be a positive multiple of 16", (long long)head_dim);
    fp_dtype wdt;
    int wl;
    split_wdt(w_dtype, wdt, wl);
    Common c{x, residual, h_out, gamma, beta, norm, eps, w_qkv, w_scale, bias,
             M, hidden, (n_heads + 2 * n_kv_heads) * head_dim, act_dtype, wdt, out_dtype,
             workspace, workspace_bytes, (hipStream_t)hip_stream};
    c.wl = wl;
    fp_status st = validate_common(c, "w_qkv");
    if (st != FP_OK) return st;
    if ((!q || !k || !v) && M > 0) return fail(FP_E_NULL, "q, k and v must all be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v))
        return fail(FP_E_ALIGN, "q, k and v must be 16-byte aligned");
    const int64_t nq = n_heads * head_dim, nkv = n_kv_heads * head_dim;
    const int eo = act_size(out_dtype), ea = act_size(act_dtype);
    std::vector<Range> ins, outs;
    add_inputs(c, ins, "w_qkv");
    if (h_out) outs.push_back(rng("h_out", h_out, M * hidden * ea));
    outs.push_back(rng("q", q, M * nq * eo));
    outs.push_back(rng("k", k, M * nkv * eo));
    outs.push_back(rng("v", v, M * nkv * eo));
    const Plan plan = make_plan(M, hidden, c.Nw, act_dtype, wdt, false, true,
                                source ? (size_t)FP_NOALLOC_SCRATCH_BYTES : SIZE_MAX, wl);
    // the workspace of a call that brings none: from the source, once every
    // argument has been checked (it may touch the device)
    if (source) {
        st = check_alias(ins, outs);
        if (st != FP_OK) return st;
        if (M > 0 && plan.total > 0) {
            char msg[256] = "";
            st = source(plan.total, &c.ws, &c.ws_bytes, msg, sizeof msg);
            if (st != FP_OK) return fail(st, "%s", msg);
        }
    }
    st = check_workspace(c, plan, outs);
    if (st != FP_OK) return st;
    st = check_alias(ins, outs);
    if (st != FP_OK) return st;

    fp::ProjArgs pa{};
    pa.epi = fp::EPI_QKV;
    pa.out0 = q;
    pa.out1 = k;
    pa.out2 = v;
    pa.nq = nq;
    pa.nkv = nkv;
    pa.qkv_hm = head_major ? 1 : 0;
    pa.head_dim = head_dim;
    pa.F = c.Nw;
    return run(c, plan, pa);
}

}  // namespace

namespace fp {
fp_status add_norm_qkv_with_source(const void *x, const void *residual, void *h_out, const void *gamma,
                                   const void *beta, fp_norm norm, float eps, const void *w_qkv,
                                   const void *w_scale, const void *bias, void *q, void *k, void *v,
                                   int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads,
                                   int64_t head_dim, fp_dtype act_dtype, fp_dtype w_dtype,
                                   fp_dtype out_dtype, void *hip_stream, WorkspaceSource source) {
    return add_norm_qkv(x, residual, h_out, gamma, beta, norm, eps, w_qkv, w_scale, bias, q, k, v, M, hidden,
                        n_heads, n_kv_heads, head_dim, act_dtype, w_dtype, out_dtype, nullptr, 0, hip_stream,
                        false, source);
}
}  // namespace fp

extern "C" {

fp_status fused_add_norm_qkv(const void *x, const void *residual, void *h_out, const void *gamma,
                             const void *beta, fp_norm norm, float eps, const void *w_qkv,
                             const void *w_scale, const void *bias, void *q, void *k, void *v,
                             int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads,
                             int64_t head_dim, fp_dtype act_dtype, fp_dtype w_dtype,
                             fp_dtype out_dtype, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
    return add_norm_qkv(x, residual, h_out, gamma, beta, norm, eps, w_qkv, w_scale, bias, q, k, v, M, hidden,
                        n_heads, n_kv_heads, head_dim, act_dtype, w_dtype, out_dtype, workspace,
                        workspace_bytes, hip_stream, false);
}

fp_status fused_add_norm_qkv_hm(const void *x, const void *residual, void *h_out, const void *gamma,
                                const void *beta, fp_norm norm, float eps, const void *w_qkv,
                                const void *w_scale, const void *bias, void *q, void *k, void *v,
                                int64_t M, int64_t hidden, int64_t n_heads, int64_t n_kv_heads,
                                int64_t head_dim, fp_dtype act_dtype, fp_dtype w_dtype,
                                fp_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                void *hip_stream) {
    return add_norm_qkv(x, residual, h_out, gamma, beta, norm, eps, w_qkv, w_scale, bias, q, k, v, M, hidden,
                        n_heads, n_kv_heads, head_dim, act_dtype, w_dtype, out_dtype, workspace,
                        workspace_bytes, hip_stream, true);
}

fp_status fused_gateup_act(const void *x, const void *residual, void *h_out, const void *gamma,
                           const void *beta, fp_norm norm, float eps, const void *w,
                           const void *w_scale, const void *bias, void *out, int64_t M,
                           int64_t hidden, int64_t ffn, fp_act act, fp_dtype act_dtype,
                           fp_dtype w_dtype, fp_dtype out_dtype, void *workspace,
                           size_t workspace_bytes, void *hip_stream) {
    if (act != FP_ACT_NONE && act != FP_ACT_SWIGLU && act != FP_ACT_GELU_TANH)
        return fail(FP_E_ARG, "act = %d is not a fp_act value", (int)act);
    if (ffn <= 0 || ffn % 16 != 0)
        return fail(FP_E_SHAPE, "ffn = %lld must be a positive multiple of 16", (long long)ffn);
    const int64_t Nw = act == FP_ACT_SWIGLU ? 2 * ffn : ffn;
    fp_dtype wdt;
    int wl;
    split_wdt(w_dtype, wdt, wl);
    Common c{x, residual, h_out, gamma, beta, norm, eps, w, w_scale, bias,
             M, hidden, Nw, act_dtype, wdt, out_dtype, workspace, workspace_bytes,
             (hipStream_t)hip_stream};
    c.wl = wl;
    c.gate_rows = act == FP_ACT_SWIGLU ? ffn : 0;
    fp_status st = validate_common(c, "w");
    if (st != FP_OK) return st;
    if (!out && M > 0) return fail(FP_E_NULL, "out is NULL");
    if (!aligned16(out)) return fail(FP_E_ALIGN, "out is not 16-byte aligned");
    const int eo = act_size(out_dtype), ea = act_size(act_dtype);
    std::vector<Range> ins, outs;
    add_inputs(c, ins, "w");
    if (h_out) outs.push_back(rng("h_out", h_out, M * hidden * ea));
    outs.push_back(rng("out", out, M * ffn * eo));
    const Plan plan = make_plan(M, hidden, Nw, act_dtype, wdt, act == FP_ACT_SWIGLU, true, SIZE_MAX, wl);
    st = check_workspace(c, plan, outs);
    if (st != FP_OK) return st;
    st = check_alias(ins, outs);
    if (st != FP_OK) return st;

    fp::ProjArgs pa{};
    pa.epi = act == FP_ACT_SWIGLU ? fp::EPI_SWIGLU : act == FP_ACT_GELU_TANH ? fp::EPI_GELU : fp::EPI_LINEAR;
    pa.out0 = out;
    pa.F = ffn;
    return run(c, plan, pa);
}

fp_status fused_down_residual(const void *a, const void *w, const void *w_scale, const void *bias,
                              const void *residual, void *out, int64_t M, int64_t ffn, int64_t hidden,
                              fp_dtype act_dtype, fp_dtype w_dtype, fp_dtype out_dtype, void *workspace,
                              size_t workspace_bytes, void *hip_stream) {
    if (hidden <= 0 || hidden % 16 != 0)
        return fail(FP_E_SHAPE, "hidden = %lld must be a positive multiple of 16", (long long)hidden);
    // the projection of a (K = ffn) onto hidden output columns, no norm prologue
    fp_dtype wdt;
    int wl;
    split_wdt(w_dtype, wdt, wl);
    Common c{a, nullptr, nullptr, nullptr, nullptr, FP_NORM_NONE, 0.0f, w, w_scale, bias,
             M, ffn, hidden, act_dtype, wdt, out_dtype, workspace, workspace_bytes,
             (hipStream_t)hip_stream};
    c.wl = wl;
    if (ffn <= 0 || ffn % 64 != 0)
        return fail(FP_E_SHAPE, "ffn = %lld must be a positive multiple of 64", (long long)ffn);
    fp_status st = validate_common(c, "w");
    if (st != FP_OK) return st;
    if (!out && M > 0) return fail(FP_E_NULL, "out is NULL");
    if (!aligned16(out) || !aligned16(residual)) return fail(FP_E_ALIGN, "out and residual must be 16-byte aligned");
    const int eo = act_size(out_dtype), ea = act_size(act_dtype);
    // in place (out == residual, same dtype): every output element is written by
    // the thread that read its residual element
    const bool in_place = residual && out == residual && out_dtype == act_dtype;
    std::vector<Range> ins, outs;
    add_inputs(c, ins, "w");
    ins[0].name = "a";
    if (residual && !in_place) ins.push_back(rng("residual", residual, M * hidden * ea));
    outs.push_back(rng("out", out, M * hidden * eo));
    const Plan plan = make_plan(M, ffn, hidden, act_dtype, wdt, false, false, SIZE_MAX, wl);
    st = check_workspace(c, plan, outs);
    if (st != FP_OK) return st;
    st = check_alias(ins, outs);
    if (st != FP_OK) return st;

    fp::ProjArgs pa{};
    pa.epi = fp::EPI_LINEAR;
    pa.out0 = out;
    pa.F = hidden;
    pa.res_epi = residual;
    return run(c, plan, pa);
}

fp_status fused_dequant_i8_bf16(const int8_t *q, const float *scale, void *out_bf16, int64_t N,
                                int64_t K, void *hip_stream) {
    if (N < 0) return fail(FP_E_SHAPE, "N = %lld is negative", (long long)N);
    if (K <= 0 || K % 16 != 0) return fail(FP_E_SHAPE, "K = %lld must be a positive multiple of 16", (long long)K);
    if (!q || !scale || !out_bf16) return fail(FP_E_NULL, "q, scale and out_bf16 must be non-NULL");
    if (!aligned16(q) || !aligned16(scale) || !aligned16(out_bf16))
        return fail(FP_E_ALIGN, "q, scale and out_bf16 must be 16-byte aligned");
    std::vector<Range> ins{rng("q", q, N * K), rng("scale", scale, N * 4)};
    std::vector<Range> outs{rng("out_bf16", out_bf16, N * K * 2)};
    fp_status st = check_alias(ins, outs);
    if (st != FP_OK) return st;
    if (N == 0) return FP_OK;
    hipStream_t s = (hipStream_t)hip_stream;
    ProfScope ps(fp::dequant_kernel_name(), s);
    hipError_t e = fp::launch_dequant(q, scale, out_bf16, N, K, s);
    if (e != hipSuccess) return hip_fail(e, "dequant_kernel launch");
    return FP_OK;
}

fp_status fused_dequant_i4_bf16(const void *q, const float *scale, void *out_bf16, int64_t N,
                                int64_t K, void *hip_stream) {
    if (N < 0) return fail(FP_E_SHAPE, "N = %lld is negative", (long long)N);
    if (K <= 0 || K % 128 != 0) return fail(FP_E_SHAPE, "K = %lld must be a positive multiple of 128", (long long)K);
    if (!q || !scale || !out_bf16) return fail(FP_E_NULL, "q, scale and out_bf16 must be non-NULL");
    if (!aligned16(q) || !aligned16(scale) || !aligned16(out_bf16))
        return fail(FP_E_ALIGN, "q, scale and out_bf16 must be 16-byte aligned");
    std::vector<Range> ins{rng("q", q, N * K / 2), rng("scale", scale, N * (K / 128) * 4)};
    std::vector<Range> outs{rng("out_bf16", out_bf16, N * K * 2)};
    fp_status st = check_alias(ins, outs);
    if (st != FP_OK) return st;
    if (N == 0) return FP_OK;
    hipStream_t s = (hipStream_t)hip_stream;
    ProfScope ps(fp::dequant_i4_kernel_name(), s);
    hipError_t e = fp::launch_dequant_i4((const uint8_t *)q, scale, out_bf16, N, K, s);
    if (e != hipSuccess) return hip_fail(e, "dequant_i4_kernel launch");
    return FP_OK;
}

fp_status fused_dequant_mxfp4_bf16(const void *q, const void *scale, void *out_bf16, int64_t N, int64_t K,
                                   void *hip_stream) {
    if (N < 0) return fail(FP_E_SHAPE, "N = %lld is negative", (long long)N);
    if (K <= 0 || K % 32 != 0) return fail(FP_E_SHAPE, "K = %lld must be a positive multiple of 32", (long long)K);
    if (!q || !scale || !out_bf16) return fail(FP_E_NULL, "q, scale and out_bf16 must be non-NULL");
    if (!aligned16(q) || !aligned16(out_bf16)) return fail(FP_E_ALIGN, "q and out_bf16 must be 16-byte aligned");
    std::vector<Range> ins{rng("q", q, N * K / 2), rng("scale", scale, N * (K / 32))};
    std::vector<Range> outs{rng("out_bf16", out_bf16, N * K * 2)};
    fp_status st = check_alias(ins, outs);
    if (st != FP_OK) return st;
    if (N == 0) return FP_OK;
    hipStream_t s = (hipStream_t)hip_stream;
    ProfScope ps(fp::dequant_mxfp4_kernel_name(), s);
    hipError_t e = fp::launch_dequant_mxfp4((const uint8_t *)q, (const uint8_t *)scale, out_bf16, N, K, s);
    if (e != hipSuccess) return hip_fail(e, "dequant_mxfp4_kernel launch");
    return FP_OK;
}

}  // extern "C"

namespace {
fp_status pack_common(const char *fn, const void *src, void *dst, int64_t n_rows, int64_t K, fp_dtype w_dtype,
                      int32_t gate_up, void *hip_stream, bool unpack) {
    if (w_dtype != FP_F16 && w_dtype != FP_BF16 && w_dtype != FP_I8 && w_dtype != FP_I4 && w_dtype != FP_E4M3 &&
        w_dtype != FP_MXFP4)
        return fail(FP_E_DTYPE, "%s: w_dtype %d is not F16, BF16, I8, I4, E4M3 or MXFP4", fn, (int)w_dtype);
    if (gate_up != 0 && gate_up != 1) return fail(FP_E_ARG, "%s: gate_up = %d (0 or 1)", fn, (int)gate_up);
    if (n_rows < 0 || K <= 0) return fail(FP_E_SHAPE, "%s: n_rows = %lld, K = %lld", fn, (long long)n_rows,
                                          (long long)K);
    if ((w_dtype == FP_I4 || w_dtype == FP_MXFP4) && K % 2 != 0)
        return fail(FP_E_SHAPE, "%s: K = %lld must be even for 4-bit weights", fn, (long long)K);
    const int layout = gate_up ? fp::WL_PACKED_GATE_UP : fp::WL_PACKED;
    fp_status st = check_layout(layout, w_dtype, n_rows, K, gate_up ? n_rows / 2 : 0);
    if (st != FP_OK) return st;
    if (!src || !dst) return fail(FP_E_NULL, "%s: both weight pointers must be non-NULL", fn);
    if (!aligned16(src) || !aligned16(dst)) return fail(FP_E_ALIGN, "%s: both weights must be 16-byte aligned", fn);
    const int64_t bytes = n_rows * row_bytes(w_dtype, K);
    std::vector<Range> ins{rng("source weight", src, bytes)}, outs{rng("destination weight", dst, bytes)};
    st = check_alias(ins, outs);
    if (st != FP_OK) return st;
    if (n_rows == 0) return FP_OK;
    hipStream_t s = (hipStream_t)hip_stream;
    ProfScope ps(fp::pack_kernel_name(unpack), s);
    hipError_t e = fp::launch_pack(src, dst, n_rows, row_bytes(w_dtype, K), n_rows / 2, layout, unpack, s);
    if (e != hipSuccess) return hip_fail(e, unpack ? "unpack_kernel launch" : "pack_kernel launch");
    return FP_OK;
}
}  // namespace

extern "C" {

fp_status fused_pack_weight(const void *w, void *w_packed, int64_t n_rows, int64_t K, fp_dtype w_dtype,
                            int32_t gate_up, void *hip_stream) {
    return pack_common("fused_pack_weight", w, w_packed, n_rows, K, w_dtype, gate_up, hip_stream, false);
}

fp_status fused_unpack_weight(const void *w_packed, void *w, int64_t n_rows, int64_t K, fp_dtype w_dtype,
                              int32_t gate_up, void *hip_stream) {
    return pack_common("fused_unpack_weight", w_packed, w, n_rows, K, w_dtype, gate_up, hip_stream, true);
}

fp_status fp_describe_plan(int64_t M, int64_t hidden, int64_t n_cols, fp_dtype act_dtype,
                           fp_dtype w_dtype, fp_act act, char *buf, size_t cap) {
    if (!buf || cap == 0) return fail(FP_E_NULL, "buf must be non-NULL with cap > 0");
    if (M < 0 || hidden <= 0 || hidden % 64 != 0 || n_cols <= 0)
        return fail(FP_E_SHAPE, "M = %lld, hidden = %lld (a positive multiple of 64), n_cols = %lld",
                    (long long)M, (long long)hidden, (long long)n_cols);
    if ((int)act < 0 || (int)act > 2) return fail(FP_E_ARG, "act = %d", (int)act);
    const fp_dtype w_dtype_arg = w_dtype;
    int wl;
    split_wdt(w_dtype_arg, w_dtype, wl);
    fp_status st = check_dtypes(act_dtype, w_dtype, act_dtype);
    if (st != FP_OK) return st;
    st = check_layout(wl, w_dtype, n_cols, hidden, act == FP_ACT_SWIGLU ? n_cols / 2 : 0);
    if (st != FP_OK) return st;
    if ((w_dtype == FP_I4 || w_dtype == FP_E4M3) && hidden % 128 != 0)
        return fail(FP_E_SHAPE, "hidden = %lld must be a multiple of 128 for int4 / E4M3 weights", (long long)hidden);
    const Plan p = make_plan(M, hidden, n_cols, act_dtype, w_dtype, act == FP_ACT_SWIGLU, true, SIZE_MAX, wl);
    if (p.family == 3) {
        const int a8 = act_code(act_dtype);
        const int e8 = act == FP_ACT_SWIGLU ? fp::EPI_SWIGLU : act == FP_ACT_GELU_TANH ? fp::EPI_GELU : fp::EPI_LINEAR;
        if (p.stream8)
            snprintf(buf, cap, "family=fp8 kernel=%s grid=%d splits=1 slots=%d workspace=%zu prep=%s",
                     fp::stream_kernel_name(a8, 4, p.sc, e8), p.grid, p.slots, M == 0 ? (size_t)0 : p.total,
                     fp::quant8_kernel_name(a8));
        else
            snprintf(buf, cap, "family=fp8 kernel=%s grid=%lld splits=%d slots=%d workspace=%zu prep=%s",
                     fp::gemm8_kernel_name(a8, p.tile8, e8), (long long)p.tiles_m * p.tiles_n * p.splits, p.splits,
                     p.slots, M == 0 ? (size_t)0 : p.total, fp::quant8_kernel_name(a8));
        return FP_OK;
    }
    const int a = act_code(act_dtype);
    const bool wi8 = w_dtype == FP_I8;
    const int wq = wi8 ? 1 : p.deq ? 0 : w_dtype == FP_I4 ? 2 : w_dtype == FP_MXFP4 ? 3 : 0;
    const int epi = act == FP_ACT_SWIGLU ? fp::EPI_SWIGLU : act == FP_ACT_GELU_TANH ? fp::EPI_GELU : fp::EPI_LINEAR;
    if (p.family == 4) {
        snprintf(buf, cap, "family=gemm16 kernel=%s grid=%lld splits=1 slots=1 workspace=%zu prep=%s",
                 fp::gemm16_kernel_name(a, p.nst, epi), (long long)p.tiles_m * p.tiles_n, M == 0 ? (size_t)0 : p.total,
                 fp::norm_kernel_name(a));
        return FP_OK;
    }
    const char *fam = p.family == 1 ? "stream" : p.family == 2 ? "prefill" : "tiled";
    const char *name = p.family == 1 ? fp::stream_kernel_name(a, wq, p.sc, epi)
                     : p.family == 2 ? fp::prefill_kernel_name(a, wq, epi)
                                     : fp::proj_kernel_name(a, wi8, p.tile, epi);
    const int64_t grid = p.family == 1 ? p.grid : (int64_t)p.tiles_m * p.tiles_n * p.splits;
    const char *deq = !p.deq ? "" : w_dtype == FP_MXFP4 ? "dequant_mxfp4_kernel" : "dequant_i4_kernel";
    char prep[96] = "";
    if (p.rows && !(p.family == 1 && p.sc.rp)) snprintf(prep, sizeof prep, " prep=%s", fp::norm_kernel_name(a));
    else if (p.unpack || p.deq)
        snprintf(prep, sizeof prep, " prep=%s%s%s", p.unpack ? "unpack_kernel" : "", p.unpack && p.deq ? "+" : "", deq);
    snprintf(buf, cap, "family=%s kernel=%s grid=%lld splits=%d slots=%d workspace=%zu%s", fam, name,
             (long long)grid, p.splits, p.slots, M == 0 ? (size_t)0 : p.total, prep);
    return FP_OK;
}

fp_status fp_tune_install(const fp_tune_entry *entries, int64_t n) {
    if (n < 0 || n > 65536) return fail(FP_E_ARG, "n = %lld entries (0 .. 65536)", (long long)n);
    if (n > 0 && !entries) return fail(FP_E_NULL, "entries is NULL");
    for (int64_t i = 0; i < n; ++i) {
        const fp_tune_entry &e = entries[i];
        const bool ok = e.m_lo >= 0 && e.m_hi >= e.m_lo && e.hidden > 0 && e.n_cols > 0 &&
                        e.family >= -1 && e.family <= 4 && e.family != 3 &&
                        (e.rows == 0 || e.rows == 32 || e.rows == 64 || e.rows == 128 || e.rows == 256) &&
                        e.grid >= 0 && e.grid <= 65535 && e.splits >= 0 && e.splits <= 64 &&
                        (e.swiglu == 0 || e.swiglu == 1) && check_dtypes(e.act_dtype, e.w_dtype, e.act_dtype) == FP_OK;
        if (!ok) return fail(FP_E_ARG, "tuning entry %lld is out of range", (long long)i);
    }
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_tune.assign(entries, entries + n);
    return FP_OK;
}

int64_t fp_tune_count(void) {
    std::lock_guard<std::mutex> lk(g_tune_mu);
    return (int64_t)g_tune.size();
}

fp_status fp_plan_override_set(const fp_plan_override *o) {
    const fp_plan_override v = o ? *o : env_overrides();
    const bool ok = v.splits >= 0 && v.splits <= 64 &&
                    (v.stream_nr == 0 || v.stream_nr == 1 || v.stream_nr == 2 || v.stream_nr == 4) &&
                    v.stream_target >= 0 && v.stream_target <= 65535 && (v.no_stream == 0 || v.no_stream == 1) &&
                    (v.no_prefill == 0 || v.no_prefill == 1) &&
                    (v.fp8_tile == 0 || v.fp8_tile == 32 || v.fp8_tile == 64 || v.fp8_tile == 128 || v.fp8_tile == 256) &&
                    (v.no_gemm16 == 0 || v.no_gemm16 == 1) &&
                    (v.gemm16_stages == 0 || v.gemm16_stages == 2 || v.gemm16_stages == 4 || v.gemm16_stages == 5) &&
                    (v.no_stream_rows == 0 || v.no_stream_rows == 1) &&
                    (v.stream_rows_expire == 0 || v.stream_rows_expire == 1);
    if (!ok) return fail(FP_E_ARG, "a plan override is out of range");
    std::lock_guard<std::mutex> lk(g_tune_mu);
    g_ov = v;
    g_ov_set = true;
    return FP_OK;
}

fp_status fp_plan_override_get(fp_plan_override *o) {
    if (!o) return fail(FP_E_NULL, "o is NULL");
    std::lock_guard<std::mutex> lk(g_tune_mu);
    *o = overrides_locked();
    return FP_OK;
}

const char *fp_status_str(fp_status s) {
    switch (s) {
    case FP_OK: return "ok";
    case FP_E_NULL: return "null pointer";
    case FP_E_SHAPE: return "invalid shape";
    case FP_E_DTYPE: return "unsupported dtype combination";
    case FP_E_ALIGN: return "misaligned pointer";
    case FP_E_ALIAS: return "output overlaps another buffer";
    case FP_E_WORKSPACE: return "workspace missing or too small";
    case FP_E_ARG: return "invalid enum argument";
    case FP_E_HIP: return "HIP error";
    }
    return "unknown status";
}

const char *fp_last_error(void) { return g_err.c_str(); }

fp_status fp_profile_start(void) {
    g_recs.clear();
    g_prof = true;
    return FP_OK;
}

fp_status fp_profile_stop(fp_kernel_time *out, int capacity, int *count) {
    g_prof = false;
    std::vector<fp_kernel_time> agg;
    fp_status st = FP_OK;
    for (const ProfRec &r : g_recs) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == FP_OK) st = hip_fail(e, "profiler event");
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
        size_t i = 0;
        for (; i < agg.size(); ++i)
            if (strcmp(agg[i].name, r.name) == 0) break;
        if (i == agg.size()) {
            fp_kernel_time t{};
            snprintf(t.name, sizeof t.name, "%s", r.name);
            agg.push_back(t);
        }
        agg[i].launches += 1;
        agg[i].total_ms += ms;
    }
    g_recs.clear();
    if (count) *count = (int)agg.size();
    for (int i = 0; out && i < capacity && i < (int)agg.size(); ++i) out[i] = agg[i];
    return st;
}

}  // extern "C"
