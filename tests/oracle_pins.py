"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what mathematics or an independent library fixes.  ``test_oracle_pins.py``
runs each as a test; ``test_oracle_mutants.py`` runs all of them against
deliberately broken copies of the oracle and requires that every copy fails at
least one pin.

Kinds of pin used here: closed forms evaluated in high-precision decimal
arithmetic, invariants (mean/variance after normalisation, shift and scale
invariance, identity / one-hot / zero weights, exact power-of-two scaling,
odd/even identities of the activations), exhaustive comparison against
IEEE casts of numpy / torch, and special cases that reduce to library routines
(torch fp64 layer_norm, rms_norm, silu, gelu, numpy matmul).
"""
from __future__ import annotations

import decimal
from decimal import Decimal

import numpy as np
import torch
import torch.nn.functional as TF

import oracle

decimal.getcontext().prec = 50


# ---------------------------------------------------------------------------
# small helpers (independent of the oracle)
# ---------------------------------------------------------------------------
def _dexp(x: Decimal) -> Decimal:
    return x.exp()


def _dtanh(x: Decimal) -> Decimal:
    e2 = (2 * x).exp()
    return (e2 - 1) / (e2 + 1)


def _silu_dec(g: float) -> float:
    g = Decimal(g)
    return float(g / (1 + _dexp(-g)))


def _gelu_dec(y: float) -> float:
    y = Decimal(y)
    c = (Decimal(2) / Decimal("3.14159265358979323846264338327950288419716939937510")).sqrt()
    return float(Decimal("0.5") * y * (1 + _dtanh(c * (y + Decimal("0.044715") * y ** 3))))


def _rng(seed=0):
    return np.random.default_rng(seed)


def _close(a, b, rtol=1e-13, atol=1e-13, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    assert np.all(err <= lim), f"{what}: max err {err.max():.3e}"


def _t(a, dt):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dt)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def pin_round_matches_ieee_casts():
    v = _rng(1).standard_normal(200000) * np.exp(_rng(2).uniform(-30, 30, 200000))
    assert np.array_equal(oracle.rne(v, "f32"), v.astype(np.float32).astype(np.float64))
    vh = v * 1e-3
    with np.errstate(over="ignore"):
        ref16 = vh.astype(np.float16).astype(np.float64)
    assert np.array_equal(oracle.rne(vh, "f16"), ref16)
    # bf16 from fp32 values (torch's fp32 -> bf16 cast is RNE and exact in its input)
    f = v.astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.rne(f.astype(np.float64), "bf16"), ref)


def pin_round_ties_and_limits():
    r = oracle.rne
    # ties go to the even neighbour
    assert r([1 + 2.0 ** -8], "bf16")[0] == 1.0
    assert r([1 + 3 * 2.0 ** -8], "bf16")[0] == 1 + 2.0 ** -6
    assert r([1 + 2.0 ** -11], "f16")[0] == 1.0
    assert r([1 + 3 * 2.0 ** -11], "f16")[0] == 1 + 2.0 ** -9
    assert r([1 + 2.0 ** -24], "f32")[0] == 1.0
    # just above a tie rounds up
    assert r([1 + 2.0 ** -8 + 2.0 ** -30], "bf16")[0] == 1 + 2.0 ** -7
    # overflow: largest finite, and the midpoint beyond it goes to infinity
    assert r([65504.0], "f16")[0] == 65504.0
    assert r([65519.0], "f16")[0] == 65504.0
    assert np.isinf(r([65520.0], "f16")[0])
    # subnormals keep a fixed quantum
    assert r([2.0 ** -24], "f16")[0] == 2.0 ** -24
    assert r([1.4 * 2.0 ** -25], "f16")[0] == 2.0 ** -24
    assert r([0.4 * 2.0 ** -24], "f16")[0] == 0.0
    assert r([2.0 ** -133], "bf16")[0] == 2.0 ** -133
    assert r([3 * 2.0 ** -135], "bf16")[0] == 2.0 ** -133


def pin_decode_exhaustive():
    allbits = np.arange(65536, dtype=np.uint16)
    # bf16: compare against torch's decode of every pattern
    t = torch.from_numpy(allbits.view(np.int16).copy()).view(torch.bfloat16)
    ref = t.to(torch.float64).numpy()
    got = oracle.decode(t)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    # fp16: numpy's decode of every pattern
    h = allbits.view(np.float16)
    ref = h.astype(np.float64)
    got = oracle.decode(h)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    # int8 and fp32 are plain conversions
    q = np.arange(-128, 128, dtype=np.int8)
    assert np.array_equal(oracle.decode(torch.from_numpy(q)), q.astype(np.float64))


# ---------------------------------------------------------------------------
# activations
# ---------------------------------------------------------------------------
_SILU_POINTS = [0.0, 1.0, -1.0, 2.0, -3.0, 0.5, 7.25, -11.0, 30.0]
_GELU_POINTS = [0.0, 1.0, -1.0, 2.0, 3.0, -0.3, 4.5, -6.0]


def pin_silu_closed_form():
    for g in _SILU_POINTS:
        ref = _silu_dec(g)
        _close(oracle.silu(g), ref, rtol=2e-15, atol=1e-300, what=f"silu({g})")
    # the published value of the logistic function at 1, times 1
    _close(oracle.silu(1.0), 0.7310585786300049, rtol=1e-15, what="silu(1)")
    # SiLU(-x) = SiLU(x) - x
    for g in np.linspace(-8, 8, 65):
        _close(oracle.silu(-g), oracle.silu(g) - g, rtol=1e-14, atol=1e-14, what="silu odd part")
    x = torch.linspace(-20, 20, 401, dtype=torch.float64)
    _close([oracle.silu(float(v)) for v in x], TF.silu(x).numpy(), rtol=1e-14, atol=1e-300,
           what="silu vs torch")


def pin_gelu_closed_form():
    for y in _GELU_POINTS:
        # 1 + tanh(.) cancels for large negative y: an absolute bound is the honest one
        _close(oracle.gelu_tanh(y), _gelu_dec(y), rtol=4e-15, atol=1e-15, what=f"gelu({y})")
    # GELU(x) - GELU(-x) = x, GELU(0) = 0
    assert oracle.gelu_tanh(0.0) == 0.0
    for y in np.linspace(-6, 6, 49):
        _close(oracle.gelu_tanh(y) - oracle.gelu_tanh(-y), y, rtol=1e-14, atol=1e-14,
               what="gelu odd identity")
    x = torch.linspace(-10, 10, 401, dtype=torch.float64)
    _close([oracle.gelu_tanh(float(v)) for v in x], TF.gelu(x, approximate="tanh").numpy(),
           rtol=1e-14, atol=1e-15, what="gelu vs torch")


# ---------------------------------------------------------------------------
# residual add and normalisation
# ---------------------------------------------------------------------------
def pin_residual_add_exact():
    rng = _rng(3)
    for act, dt in (("bf16", torch.bfloat16), ("f16", torch.float16), ("f32", torch.float32)):
        x = _t(rng.standard_normal((5, 64)), dt)
        r = _t(rng.standard_normal((5, 64)), dt)
        h, _, _ = oracle.add_norm(x, r, _t(np.ones(64), dt), None, "rms", 1e-5)
        exact = x.double() + r.double()
        ref = (x.float() + r.float()).to(dt).double().numpy()
        assert np.array_equal(h, ref), act
        if act != "f32":  # the fp32 sum of two 16-bit values is exact
            assert np.array_equal((x.float() + r.float()).double().numpy(), exact.numpy())
    # r = NULL means no residual: h_out is x itself
    x = _t(rng.standard_normal((3, 64)), torch.bfloat16)
    h, _, _ = oracle.add_norm(x, None, _t(np.ones(64), torch.bfloat16), None, "none", 0.0)
    assert np.array_equal(h, x.double().numpy())


def pin_layernorm_moments():
    rng = _rng(4)
    K = 256
    # values on a 2^-10 grid, so that shifting them by 4 is exact in fp32
    x = _t(np.round((rng.standard_normal((6, K)) * 3 + 0.7) * 1024) / 1024, torch.float32)
    r = _t(np.round(rng.standard_normal((6, K)) * 1024) / 1024, torch.float32)
    eps = 1e-5
    _, n, _ = oracle.add_norm(x, r, _t(np.ones(K), torch.float32),
                              _t(np.zeros(K), torch.float32), "layer", eps)
    h = x.double().numpy() + r.double().numpy()
    var = h.var(axis=1)
    e = float(np.float32(eps))
    assert np.all(np.abs(n.mean(axis=1)) <= 1e-12)
    _close(n.var(axis=1), var / (var + e), rtol=1e-12, what="LN variance closed form")
    # shift invariance: LN(h + c) == LN(h) (shift chosen exactly representable)
    xs = x + 4.0
    assert torch.equal(xs - 4.0, x)
    _, n2, _ = oracle.add_norm(xs, r, _t(np.ones(K), torch.float32),
                               _t(np.zeros(K), torch.float32), "layer", eps)
    _close(n2, n, rtol=1e-9, atol=1e-9, what="LN shift invariance")


def pin_rmsnorm_moments():
    rng = _rng(5)
    K = 512
    x = _t(rng.standard_normal((7, K)) * 2 + 0.3, torch.float32)
    r = _t(rng.standard_normal((7, K)), torch.float32)
    eps = 1e-5
    e = float(np.float32(eps))
    _, n, _ = oracle.add_norm(x, r, _t(np.ones(K), torch.float32), None, "rms", eps)
    h = x.double().numpy() + r.double().numpy()
    ms = (h * h).mean(axis=1)
    _close((n * n).mean(axis=1), ms / (ms + e), rtol=1e-12, what="RMS closed form")
    # scale invariance at eps = 0 with a power-of-two scale (exact)
    _, n0, _ = oracle.add_norm(x, r, _t(np.ones(K), torch.float32), None, "rms", 0.0)
    _, n1, _ = oracle.add_norm(x * 8, r * 8, _t(np.ones(K), torch.float32), None, "rms", 0.0)
    _close(n1, n0, rtol=1e-14, atol=1e-15, what="RMS scale invariance")
    # RMS does not subtract the mean: a constant row normalises to +-1 / sqrt(1+eps/c^2)
    c = 3.0
    xc = _t(np.full((1, K), c), torch.float32)
    _, nc, _ = oracle.add_norm(xc, None, _t(np.ones(K), torch.float32), None, "rms", eps)
    _close(nc, np.full((1, K), c / np.sqrt(c * c + e)), rtol=1e-15, what="RMS constant row")


def pin_norm_vs_torch_and_gamma():
    rng = _rng(6)
    K = 128
    x = _t(rng.standard_normal((9, K)), torch.float32)
    r = _t(rng.standard_normal((9, K)), torch.float32)
    g = _t(rng.uniform(0.5, 1.5, K), torch.float32)
    b = _t(rng.standard_normal(K) * 0.1, torch.float32)
    eps = 1e-5
    e = float(np.float32(eps))
    h = x.double() + r.double()
    _, n, a = oracle.add_norm(x, r, g, b, "layer", eps)
    ref = TF.layer_norm(h, (K,), g.double(), b.double(), e).numpy()
    _close(n, ref, rtol=1e-12, atol=1e-13, what="LN vs torch")
    _, n, _ = oracle.add_norm(x, r, g, None, "rms", eps)
    ref = TF.rms_norm(h, (K,), g.double(), e).numpy()
    _close(n, ref, rtol=1e-12, atol=1e-13, what="RMS vs torch")
    # gamma scales the normalised value, beta shifts it: doubling gamma doubles n exactly
    _, n2, _ = oracle.add_norm(x, r, g * 2, None, "rms", eps)
    _close(n2, 2 * n, rtol=0, atol=0, what="gamma power-of-two scaling")
    # NONE: n = h
    _, nn, _ = oracle.add_norm(x, r, g, None, "none", eps)
    assert np.array_equal(nn, h.numpy())


def pin_a_operand_is_rounded_normalised_row():
    rng = _rng(7)
    K = 64
    for dt, name in ((torch.bfloat16, "bf16"), (torch.float16, "f16")):
        x = _t(rng.standard_normal((4, K)), dt)
        r = _t(rng.standard_normal((4, K)), dt)
        g = _t(rng.uniform(0.8, 1.2, K), dt)
        _, n, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
        # every a is representable in the dtype and within half an ulp (plus
        # the single-precision evaluation error of R11) of n
        back = torch.from_numpy(a).to(dt).double().numpy()
        assert np.array_equal(back, a)
        ulp = 2.0 ** (np.floor(np.log2(np.abs(n))) - (7 if name == "bf16" else 10))
        assert np.all(np.abs(a - n) <= ulp / 2 + np.abs(n) * 2.0 ** -21)


def pin_single_precision_normalisation():
    """R11: the normalised value the product consumes is a single-precision
    evaluation: within a few fp32 roundings of the double-precision n (whose
    own pins are the closed forms above), exactly h for NONE, and the GEMM
    operand is that fp32 value cast to the activation dtype by torch."""
    rng = _rng(8)
    M, K = 256, 1024
    for dt in (torch.bfloat16, torch.float16, torch.float32):
        x = _t(rng.standard_normal((M, K)) * 1.5 + 0.7, dt)      # a mean far from zero
        r = _t(rng.standard_normal((M, K)), dt)
        g = _t(rng.uniform(0.5, 1.5, K), dt)
        b = _t(rng.standard_normal(K) * 0.3, dt)
        h = x.double() + r.double()
        for norm, beta in (("rms", None), ("layer", b), ("layer", None), ("none", None)):
            _, n, a = oracle.add_norm(x, r, g, beta, norm, 1e-5)
            n32 = oracle.add_norm_f32(x, r, g, beta, norm, 1e-5)
            # fp32 values
            assert np.array_equal(n32.astype(np.float32).astype(np.float64), n32)
            if norm == "none":
                assert np.array_equal(n32, h.float().double().numpy())
            else:
                hv = h.numpy()
                mu = hv.mean(1, keepdims=True) if norm == "layer" else 0.0
                var = ((hv - mu) ** 2).mean(1, keepdims=True)
                rstd = 1.0 / np.sqrt(var + float(np.float32(1e-5)))
                slack = np.abs(n) + np.abs(mu) * rstd * g.double().numpy() + \
                    (np.abs(b.double().numpy()) if beta is not None else 0.0)
                err = np.abs(n32 - n)
                assert np.all(err <= slack * 2.0 ** -21), (dt, norm, err.max())
                # and not the double value itself: single-precision rounding shows
                assert not np.array_equal(n32, n)
            # the operand is torch's cast of the fp32 values
            ref = torch.from_numpy(n32.astype(np.float32)).to(dt).double().numpy()
            assert np.array_equal(a, ref), (dt, norm)


def pin_matmul_special_cases():
    rng = _rng(8)
    M, K = 3, 16
    a = rng.standard_normal((M, K))
    # identity weight: acc == a exactly
    eye = np.eye(K, dtype=np.float32)
    assert np.array_equal(oracle.matmul_nt(a, eye), a)
    # one-hot rows pick columns (non-square: catches a transposed operand)
    N = 5
    cols = [7, 0, 15, 3, 3]
    oh = np.zeros((N, K), dtype=np.float32)
    for j, c in enumerate(cols):
        oh[j, c] = 1.0
    assert np.array_equal(oracle.matmul_nt(a, oh), a[:, cols])
    # zero weight
    assert np.array_equal(oracle.matmul_nt(a, np.zeros((N, K), np.float32)), np.zeros((M, N)))
    # power-of-two scaling of W is exact
    w = rng.standard_normal((N, K)).astype(np.float32)
    acc = oracle.matmul_nt(a, w)
    assert np.array_equal(oracle.matmul_nt(a, w * np.float32(4)), 4 * acc)
    # library routine
    _close(acc, a @ w.astype(np.float64).T, rtol=1e-13, atol=1e-13, what="matmul vs numpy")
    # brute force on a tiny integer case (exact)
    ai = rng.integers(-4, 5, (2, 3)).astype(np.float64)
    wi = rng.integers(-4, 5, (4, 3)).astype(np.float32)
    bf = [[sum(ai[m, k] * float(wi[j, k]) for k in range(3)) for j in range(4)] for m in range(2)]
    assert np.array_equal(oracle.matmul_nt(ai, wi), np.array(bf))


def pin_matmul_weight_dtypes():
    rng = _rng(9)
    a = rng.standard_normal((4, 32))
    w32 = rng.standard_normal((6, 32)).astype(np.float32)
    for dt in (torch.bfloat16, torch.float16):
        wt = torch.from_numpy(w32).to(dt)
        ref = a @ wt.double().numpy().T
        _close(oracle.matmul_nt(a, wt), ref, rtol=1e-13, atol=1e-13, what=str(dt))


def pin_dequant_i8_exhaustive():
    rng = _rng(10)
    q = np.tile(np.arange(-127, 128, dtype=np.int8), (64, 1))          # [64, 255]
    s = np.concatenate([
        rng.uniform(1e-5, 1e-3, 60).astype(np.float32),
        np.array([0.0, 2.0 ** -7, 0.02 / 127, 1.0], dtype=np.float32)])
    w, bits = oracle.dequant_i8(torch.from_numpy(q), torch.from_numpy(s))
    # reference 1: fp32 multiply (RNE) then torch's fp32 -> bf16 cast (RNE)
    prod32 = q.astype(np.float32) * s[:, None]
    ref = torch.from_numpy(prod32).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(w, ref.double().numpy())
    # reference 2: integer round-to-nearest-even on the fp32 bit pattern
    u = prod32.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rb = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    assert np.array_equal(bits, rb)
    # q = 0 or s = 0 gives exactly zero
    assert np.all(w[:, 127] == 0) and np.all(w[60] == 0)


def _bf16_direct_bits(v: np.ndarray) -> np.ndarray:
    """RNE of float64 values straight to bf16 (8 significant bits), normal range only."""
    u = v.view(np.uint64)
    lsb = (u >> np.uint64(45)) & np.uint64(1)
    r = (u + np.uint64((1 << 44) - 1) + lsb) >> np.uint64(45) << np.uint64(45)
    return (r.view(np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def pin_dequant_i8_double_rounding_cases():
    # scan consecutive fp32 scales; keep the (q, s) pairs where rounding q*s to
    # fp32 first changes the bf16 result -- the definition's two roundings must show
    mant = _rng(23).integers(0, 1 << 23, 32768).astype(np.uint32)
    s_all = ((np.uint32(118) << 23) | mant).view(np.float32)     # fp32 scales in [2^-9, 2^-8)
    q_all = np.arange(-127, 128, dtype=np.int8)
    qq, ss = np.meshgrid(q_all, s_all)
    exact = qq.astype(np.float64) * ss.astype(np.float64)
    direct = _bf16_direct_bits(exact)
    twice = torch.from_numpy(qq.astype(np.float32) * ss).to(torch.bfloat16)
    twice = twice.view(torch.int16).numpy().view(np.uint16)
    sel = np.nonzero(direct != twice)
    assert len(sel[0]) >= 5, "scan found too few double-rounding cases"
    rows = np.unique(sel[0])[:64]
    w, bits = oracle.dequant_i8(torch.from_numpy(np.ascontiguousarray(qq[rows])),
                                torch.from_numpy(np.ascontiguousarray(s_all[rows])))
    assert np.array_equal(bits, twice[rows])
    assert not np.array_equal(bits, direct[rows])


def _pack_i4(q: np.ndarray) -> np.ndarray:
    """[N, K] ints in [-8, 7] -> [N, K/2] bytes, even k in the low nibble
    (the storage the int4 weights are defined with), written independently of
    the input generator."""
    u = (q.astype(np.int64) % 16).astype(np.uint8)
    out = np.zeros((q.shape[0], q.shape[1] // 2), dtype=np.uint8)
    for k in range(q.shape[1]):
        out[:, k // 2] |= u[:, k] << (4 * (k % 2))
    return out


def pin_dequant_i4_exhaustive():
    # every nibble value at even and odd k in both groups of a 256-wide row,
    # with a different scale per (row, group): catches nibble order, sign
    # extension and group indexing
    rng = _rng(31)
    N, K = 40, 256
    k = np.arange(K)
    q = (((k[None, :] * 5 + np.arange(N)[:, None] * 3) % 16) - 8).astype(np.int8)      # [N, K]
    s = np.concatenate([rng.uniform(1e-4, 1e-2, (N - 3, 2)).astype(np.float32),
                        np.array([[0.0, 1.0], [2.0 ** -7, 3.0], [1.0, 0.02 / 7]], dtype=np.float32)])
    w, bits = oracle.dequant_i4(torch.from_numpy(_pack_i4(q)), torch.from_numpy(s))
    s_k = s[:, k // 128]
    prod32 = q.astype(np.float32) * s_k
    prod32[prod32 == 0] = 0.0                           # a zero product is +0 (reading R9)
    ref = torch.from_numpy(prod32).to(torch.bfloat16)
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(w, ref.double().numpy())
    assert np.all(bits[N - 3, :128] == 0)              # s = 0 gives +0, also for negative q
    assert np.array_equal(w[N - 3, 128:], q[N - 3, 128:].astype(np.float64))   # s = 1: the integers


def pin_dequant_i4_double_rounding_cases():
    # every fp32 scale in [2^-9, 2^-8): keep those where rounding q * s to fp32
    # first changes the bf16 result (a 4-bit q leaves few such scales)
    s_all = ((np.uint32(118) << 23) | np.arange(1 << 23, dtype=np.uint32)).view(np.float32)
    picks = []
    for qv in (3, 5, 7, -7):
        exact = np.float64(qv) * s_all.astype(np.float64)
        direct = _bf16_direct_bits(exact)
        twice = torch.from_numpy(np.float32(qv) * s_all).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        idx = np.nonzero(direct != twice)[0][:4]
        picks += [(qv, s_all[i], twice[i], direct[i]) for i in idx]
    assert len(picks) >= 8, "scan found too few double-rounding cases"
    # one row per case: q in every position of a 128-wide group with that scale
    q = np.array([[qv] * 128 for qv, _, _, _ in picks], dtype=np.int8)
    sc = np.array([[sv] for _, sv, _, _ in picks], dtype=np.float32)
    w, bits = oracle.dequant_i4(torch.from_numpy(_pack_i4(q)), torch.from_numpy(sc))
    assert np.array_equal(bits[:, 0], np.array([t for _, _, t, _ in picks], dtype=np.uint16))
    assert not np.array_equal(bits[:, 0], np.array([d for _, _, _, d in picks], dtype=np.uint16))
    assert np.all(bits == bits[:, :1])


# ---------------------------------------------------------------------------
# full calls
# ---------------------------------------------------------------------------
def _tiny(dt, M=3, K=64, seed=11):
    rng = _rng(seed)
    x = _t(rng.standard_normal((M, K)), dt)
    r = _t(rng.standard_normal((M, K)), dt)
    g = _t(rng.uniform(0.5, 1.5, K), dt)
    return x, r, g


def pin_qkv_split_layout():
    dt = torch.float32
    M, K, H, Hkv, D = 3, 64, 4, 2, 8
    N = (H + 2 * Hkv) * D
    x, r, g = _tiny(dt, M, K)
    rng = _rng(12)
    w = _t(rng.standard_normal((N, K)) / 8, dt)
    bias = _t(rng.standard_normal(N), dt)
    o = oracle.add_norm_qkv(x, r, g, None, "rms", 1e-5, w, None, bias, H, Hkv, D)
    _, _, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
    full = a @ w.double().numpy().T + bias.double().numpy()
    _close(o["q"].reshape(M, H * D), full[:, :H * D], rtol=1e-13, atol=1e-13, what="q block")
    _close(o["k"].reshape(M, Hkv * D), full[:, H * D:(H + Hkv) * D], rtol=1e-13, atol=1e-13,
           what="k block")
    _close(o["v"].reshape(M, Hkv * D), full[:, (H + Hkv) * D:], rtol=1e-13, atol=1e-13,
           what="v block")
    # one-hot rows: q[m, h, d] must read normalised column (h*D + d) % K
    oh = np.zeros((N, K), np.float32)
    for c in range(N):
        oh[c, (5 * c + 1) % K] = 1.0
    o = oracle.add_norm_qkv(x, r, g, None, "rms", 1e-5, torch.from_numpy(oh), None, None,
                            H, Hkv, D)
    for m in range(M):
        for h in range(H):
            for d in range(D):
                assert o["q"][m, h, d] == a[m, (5 * (h * D + d) + 1) % K]
        for h in range(Hkv):
            for d in range(D):
                c = H * D + h * D + d
                assert o["k"][m, h, d] == a[m, (5 * c + 1) % K]
                c2 = c + Hkv * D
                assert o["v"][m, h, d] == a[m, (5 * c2 + 1) % K]
    # h_out is the rounded residual stream
    assert np.array_equal(o["h_out"], (x.double() + r.double()).float().double().numpy())


def pin_qkv_mha_equal_split():
    dt = torch.bfloat16
    M, K, H, D = 2, 64, 2, 16
    x, r, g = _tiny(dt, M, K, seed=13)
    blk = _t(_rng(14).standard_normal((H * D, K)) / 8, dt)
    w = torch.cat([blk, blk, blk], 0)
    o = oracle.add_norm_qkv(x, r, g, None, "rms", 1e-5, w, None, None, H, H, D)
    assert np.array_equal(o["q"], o["k"]) and np.array_equal(o["k"], o["v"])


def pin_swiglu_epilogue():
    dt = torch.float32
    M, K, F = 3, 64, 24
    x, r, g = _tiny(dt, M, K, seed=15)
    rng = _rng(16)
    wg = rng.standard_normal((F, K)) / 8
    wu = rng.standard_normal((F, K)) / 8
    w = _t(np.concatenate([wg, wu]), dt)
    b = _t(rng.standard_normal(2 * F) * 0.1, dt)
    o = oracle.gateup_act(x, r, g, None, "rms", 1e-5, w, None, b, F, "swiglu")
    _, _, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
    at = torch.from_numpy(a)
    wd = w.double()
    gate = at @ wd[:F].T + b.double()[:F]
    up = at @ wd[F:].T + b.double()[F:]
    _close(o["out"], (TF.silu(gate) * up).numpy(), rtol=1e-12, atol=1e-13, what="swiglu vs torch")
    # up block zero, up bias one: out = SiLU(gate); gate <-> up swapped must differ
    w2 = torch.cat([w[:F], torch.zeros(F, K)], 0)
    b2 = torch.cat([b[:F], torch.ones(F)], 0)
    o2 = oracle.gateup_act(x, r, g, None, "rms", 1e-5, w2, None, b2, F, "swiglu")
    _close(o2["out"], TF.silu(gate).numpy(), rtol=1e-12, atol=1e-13, what="swiglu up=1")
    o3 = oracle.gateup_act(x, r, g, None, "rms", 1e-5, torch.cat([w[F:], w[:F]], 0), None,
                           torch.cat([b[F:], b[:F]], 0), F, "swiglu")
    assert not np.allclose(o3["out"], o["out"])


def pin_gelu_bias_epilogue():
    dt = torch.float16
    M, K, F = 2, 64, 16
    rng = _rng(17)
    x, r, g = _tiny(dt, M, K, seed=18)
    beta = _t(rng.standard_normal(K) * 0.02, dt)
    w = _t(rng.standard_normal((F, K)) * 0.1, dt)
    b = _t(rng.standard_normal(F) * 0.5, dt)
    o = oracle.gateup_act(x, r, g, beta, "layer", 1e-5, w, None, b, F, "gelu_tanh")
    _, _, a = oracle.add_norm(x, r, g, beta, "layer", 1e-5)
    y = torch.from_numpy(a) @ w.double().T + b.double()
    _close(o["out"], TF.gelu(y, approximate="tanh").numpy(), rtol=1e-12, atol=1e-13,
           what="gelu+bias vs torch")
    # zero weight: out = GELU(bias) for every row (bias before the activation)
    o0 = oracle.gateup_act(x, r, g, beta, "layer", 1e-5, torch.zeros(F, K, dtype=dt), None, b,
                           F, "gelu_tanh")
    ref = np.array([oracle.gelu_tanh(float(v)) for v in b.double()])
    for m in range(M):
        _close(o0["out"][m], ref, rtol=1e-15, atol=0, what="gelu(bias)")
        _close(o0["out"][m], [_gelu_dec(float(v)) for v in b.double()], rtol=4e-15,
               atol=1e-300, what="gelu(bias) closed form")
    # act NONE: plain projection plus bias
    on = oracle.gateup_act(x, r, g, beta, "layer", 1e-5, w, None, b, F, "none")
    _close(on["out"], y.numpy(), rtol=1e-13, atol=1e-13, what="linear + bias")


def pin_int8_projection_uses_dequantised_weights():
    rng = _rng(19)
    M, K, N = 2, 64, 12
    x, r, g = _tiny(torch.bfloat16, M, K, seed=20)
    q = torch.from_numpy(rng.integers(-127, 128, (N, K)).astype(np.int8))
    s = torch.from_numpy(rng.uniform(1e-4, 1e-3, N).astype(np.float32))
    _, _, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
    w_deq = (q.float() * s[:, None]).to(torch.bfloat16)
    o = oracle.gateup_act(x, r, g, None, "rms", 1e-5, q, s, None, N, "none")
    _close(o["out"], a @ w_deq.double().numpy().T, rtol=1e-13, atol=1e-13, what="int8 proj")


def pin_int4_projection_uses_dequantised_weights():
    rng = _rng(34)
    M, K, N = 2, 256, 10
    x, r, g = _tiny(torch.bfloat16, M, K, seed=35)
    q = rng.integers(-8, 8, (N, K)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, (N, K // 128)).astype(np.float32)
    _, _, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
    w_deq = torch.from_numpy(q.astype(np.float32) * s[:, np.arange(K) // 128]).to(torch.bfloat16)
    o = oracle.gateup_act(x, r, g, None, "rms", 1e-5, torch.from_numpy(_pack_i4(q)), torch.from_numpy(s),
                          None, N, "none")
    _close(o["out"], a @ w_deq.double().numpy().T, rtol=1e-13, atol=1e-13, what="int4 proj")


def pin_down_residual():
    rng = _rng(41)
    M, K, N = 3, 64, 10
    a = _t(rng.standard_normal((M, K)), torch.bfloat16)
    w = _t(rng.standard_normal((N, K)) / 8, torch.bfloat16)
    res = _t(rng.standard_normal((M, N)), torch.bfloat16)
    b = _t(rng.standard_normal(N) / 4, torch.bfloat16)
    ad, wd, rd, bd = (t.double().numpy() for t in (a, w, res, b))
    # the plain definition, the product by numpy
    _close(oracle.down_residual(a, w, None, b, res), rd + bd[None, :] + ad @ wd.T, rtol=1e-13, atol=1e-13,
           what="down + residual")
    # no residual, no bias: the product alone; zero weight: the residual (+ bias) exactly
    _close(oracle.down_residual(a, w, None, None, None), ad @ wd.T, rtol=1e-13, atol=1e-13, what="down")
    z = oracle.down_residual(a, torch.zeros_like(w), None, b, res)
    assert np.array_equal(z, rd + bd[None, :])
    # a one-hot row picks one weight column (catches a transposed operand)
    oh = torch.zeros(M, K, dtype=torch.bfloat16)
    oh[1, 7] = 1.0
    o = oracle.down_residual(oh, w, None, None, res)
    assert np.array_equal(o[1], rd[1] + wd[:, 7]) and np.array_equal(o[0], rd[0])
    # int8 weights go through their dequantisation
    q = torch.from_numpy(rng.integers(-127, 128, (N, K)).astype(np.int8))
    sc = torch.from_numpy(rng.uniform(1e-3, 1e-2, N).astype(np.float32))
    w_deq = (q.float() * sc[:, None]).to(torch.bfloat16).double().numpy()
    _close(oracle.down_residual(a, q, sc, None, res), rd + ad @ w_deq.T, rtol=1e-13, atol=1e-13, what="int8 down")


def pin_rounded_vs_unrounded_reading():
    # rounding the A operand is the only difference between the two readings
    dt = torch.bfloat16
    M, K, F = 2, 64, 8
    x, r, g = _tiny(dt, M, K, seed=21)
    w = _t(_rng(22).standard_normal((F, K)) / 8, dt)
    oa = oracle.gateup_act(x, r, g, None, "rms", 1e-5, w, None, None, F, "none", rounded=True)
    ob = oracle.gateup_act(x, r, g, None, "rms", 1e-5, w, None, None, F, "none", rounded=False)
    _, n, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
    _close(oa["out"], a @ w.double().numpy().T, rtol=1e-13, atol=1e-13, what="reading A")
    _close(ob["out"], n @ w.double().numpy().T, rtol=1e-13, atol=1e-13, what="reading B")
    assert not np.array_equal(oa["out"], ob["out"])


# ---------------------------------------------------------------------------
# E4M3 weights and per-token activation quantisation (R10)
# ---------------------------------------------------------------------------
def _e4m3_torch(codes) -> np.ndarray:
    """Values of E4M3 codes through torch's float8_e4m3fn dtype (a library cast)."""
    c = torch.as_tensor(np.asarray(codes, dtype=np.uint8))
    return c.view(torch.float8_e4m3fn).double().numpy()


def _finite_e4m3():
    """(codes, values) of every finite E4M3 code, from torch's decoding."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return codes, _e4m3_torch(codes)


def pin_e4m3_decode_exhaustive():
    vals = np.array([oracle.e4m3_value(c) for c in range(256)])
    ref = _e4m3_torch(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(vals), nan) and nan.sum() == 2          # S.1111.111 only
    assert np.array_equal(vals[~nan], ref[~nan])
    # landmarks of the format: largest finite, smallest normal and subnormal, one
    assert vals[0x7E] == 448.0 and vals[0xFE] == -448.0
    assert vals[0x08] == 2.0 ** -6 and vals[0x01] == 2.0 ** -9 and vals[0x38] == 1.0
    # positive codes increase strictly with their value
    assert np.all(np.diff(vals[:0x7F]) > 0)


def pin_e4m3_encode_nearest_even():
    codes, vals = _finite_e4m3()
    pos = np.sort(np.unique(vals[vals >= 0]))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = _rng(51)
    ts = np.concatenate([pos, -pos, mids, -mids, rng.uniform(-448, 448, 3000),
                         rng.standard_normal(2000) * 2.0 ** rng.integers(-12, 6, 2000)])
    got = np.array([oracle.e4m3_encode(t) for t in ts], dtype=np.uint8)
    # brute force: the nearest finite value, ties to the code with an even
    # mantissa, the sign of t kept
    for t, c in zip(ts, got):
        d = np.abs(vals - t)
        cand = codes[d == d.min()]
        cand = cand[(cand & 0x80) == (0x80 if np.signbit(t) else 0)] if len(cand) > 1 else cand
        if len(cand) > 1:
            cand = cand[(cand & 1) == 0]
        assert c == cand[0], (t, c, cand)
    # torch's cast agrees inside the range; past 448 the encoder saturates
    inr = np.abs(ts) <= 448
    assert np.array_equal(got[inr], torch.tensor(ts[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    assert oracle.e4m3_encode(1e6) == 0x7E and oracle.e4m3_encode(-470.0) == 0xFE


def _q8_route(v):
    """Per-row E4M3 quantisation in float32 arithmetic (R10 on fp32 rows):
    scale by fp32(448 / amax), clamp, torch's cast; returns (codes, values, s)."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.abs(v).max(1, keepdims=True)
    s = amax / np.float32(448.0)
    inv = np.where(amax > 0, np.float32(448.0) / np.where(amax > 0, amax, np.float32(1)), np.float32(0))
    t = np.clip(v * inv, np.float32(-448.0), np.float32(448.0))
    q = torch.from_numpy(np.ascontiguousarray(t, dtype=np.float32)).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy(), q.double().numpy() * s.astype(np.float64), s[:, 0].astype(np.float64)


def pin_e4m3_row_quantisation():
    rng = _rng(52)
    M, K = 5, 96
    n = (rng.standard_normal((M, K)) * rng.uniform(0.01, 30, (M, 1))).astype(np.float32).astype(np.float64)
    n[3] = 0.0                                                           # a zero row
    codes, a, s = oracle.quant_rows_e4m3(n)
    rc, ra, rs = _q8_route(n)
    assert np.array_equal(s, rs)
    for m in range(M):
        if rs[m] == 0:
            assert not codes[m].any() and not a[m].any()
            continue
        assert np.array_equal(codes[m], rc[m])
        assert np.array_equal(a[m], ra[m])
        # the largest magnitude lands on +-448 exactly
        k = np.abs(n[m]).argmax()
        assert abs(oracle.e4m3_value(codes[m, k])) == 448.0
    # a power-of-two rescale of a row keeps its codes and scales s_a
    c2, a2, s2 = oracle.quant_rows_e4m3(n * 2.0 ** 7)
    assert np.array_equal(c2, codes) and np.array_equal(s2, s * 2.0 ** 7)
    # relative error of a quantised element: at most half a step of 3 mantissa
    # bits (plus the fp32 scaling)
    amax = np.abs(n).max(1)
    big = np.abs(n) >= amax[:, None] * 2.0 ** -6
    assert np.all(np.abs(a - n)[big] <= np.abs(n)[big] * (2.0 ** -4 + 2.0 ** -20))
    # rows given in double are taken at their fp32 values
    c3, _, _ = oracle.quant_rows_e4m3(n + 1e-12 * np.sign(n))
    assert np.array_equal(c3, codes)


def pin_fp8_projection():
    rng = _rng(53)
    M, K, F = 3, 128, 6
    x, r, g = _tiny(torch.bfloat16, M, K, seed=54)
    wf = rng.standard_normal((2 * F, K)) / 8
    s_w = (np.abs(wf).max(1) / 448.0).astype(np.float32)
    wq = torch.tensor(wf / s_w[:, None]).to(torch.float8_e4m3fn)
    w_val = wq.double().numpy() * s_w.astype(np.float64)[:, None]
    n32 = oracle.add_norm_f32(x, r, g, None, "rms", 1e-5)      # R11, pinned above
    _, a, _ = _q8_route(n32)
    acc = a @ w_val.T
    o = oracle.gateup_act(x, r, g, None, "rms", 1e-5, wq, torch.from_numpy(s_w), None, F, "swiglu")
    ref = acc[:, :F] / (1 + np.exp(-acc[:, :F])) * acc[:, F:]
    _close(o["out"], ref, rtol=1e-12, atol=1e-14, what="fp8 swiglu")
    # the QKV call takes the same A operand
    oq = oracle.add_norm_qkv(x, r, g, None, "rms", 1e-5, wq[:8].contiguous(), torch.from_numpy(s_w[:8]), None,
                             2, 1, 2)
    _close(np.concatenate([oq["q"].reshape(M, -1), oq["k"].reshape(M, -1), oq["v"].reshape(M, -1)], 1),
           acc[:, :8], rtol=1e-12, atol=1e-14, what="fp8 qkv")
    # the down projection quantises its input rows the same way
    ad = _t(rng.standard_normal((M, K)), torch.bfloat16)
    res = _t(rng.standard_normal((M, 2 * F)), torch.bfloat16)
    _, aq, _ = _q8_route(ad.double().numpy())
    _close(oracle.down_residual(ad, wq, torch.from_numpy(s_w), None, res), res.double().numpy() + aq @ w_val.T,
           rtol=1e-12, atol=1e-14, what="fp8 down")


# ---------------------------------------------------------------------------
# MXFP4 weights (R12)
# ---------------------------------------------------------------------------
# E2M1 magnitudes of codes 0..7 as the OCP microscaling format lists them
_E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def pin_e2m1_decode_exhaustive():
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == _E2M1_TABLE and vals[8:] == [-v for v in _E2M1_TABLE]
    assert np.signbit(vals[8]) and not np.signbit(vals[0])                  # code 8 is -0
    # the normal codes as fp32 bit patterns: sign, exponent e - 1 + 127, one mantissa bit
    for c in range(16):
        e, m = (c >> 1) & 3, c & 1
        if e == 0:
            continue
        bits = ((c >> 3) << 31) | ((e - 1 + 127) << 23) | (m << 22)
        assert np.array([bits], dtype=np.uint32).view(np.float32)[0] == vals[c], c


def pin_e8m0_decode_exhaustive():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).double().numpy()                # torch's decoding
    got = np.array([oracle.e8m0_value(c) for c in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def pin_mxfp4_dequant_exhaustive():
    """Every E2M1 code at every scale 0..254, placed so that the nibble order
    and the block indexing matter: row j has scale j in its first block and
    scale 254 - j in its second; element k holds code k % 16."""
    N, K = 255, 64
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    scales = np.stack([np.arange(255), 254 - np.arange(255)], 1).astype(np.uint8)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    q = torch.from_numpy(packed).view(torch.float4_e2m1fn_x2)
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu)
    w, bits = oracle.dequant_mxfp4(q, s)
    table = np.array(_E2M1_TABLE + [-v for v in _E2M1_TABLE])
    sv = s.double().numpy()                                                  # torch's E8M0 decoding
    exact = table[codes] * np.repeat(sv, 32, axis=1)
    ref = torch.from_numpy(exact).to(torch.bfloat16)                        # torch's bf16 cast
    assert np.array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(w, ref.double().numpy(), equal_nan=True)
    # exact wherever bf16 reaches (no overflow below scale 253)
    assert np.array_equal(w[:253, :32], exact[:253, :32])


def pin_mxfp4_projection():
    rng = _rng(61)
    M, K, F = 3, 128, 6
    x, r, g = _tiny(torch.bfloat16, M, K, seed=62)
    codes = rng.integers(0, 16, (2 * F, K)).astype(np.uint8)
    scales = rng.integers(118, 128, (2 * F, K // 32)).astype(np.uint8)
    q = torch.from_numpy(codes[:, 0::2] | (codes[:, 1::2] << 4)).view(torch.float4_e2m1fn_x2)
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu)
    table = np.array(_E2M1_TABLE + [-v for v in _E2M1_TABLE])
    w_val = table[codes] * np.exp2(np.repeat(scales.astype(np.float64) - 127, 32, axis=1))
    _, _, a = oracle.add_norm(x, r, g, None, "rms", 1e-5)
    acc = a @ w_val.T
    o = oracle.gateup_act(x, r, g, None, "rms", 1e-5, q, s, None, F, "swiglu")
    ref = acc[:, :F] / (1 + np.exp(-acc[:, :F])) * acc[:, F:]
    _close(o["out"], ref, rtol=1e-12, atol=1e-14, what="mxfp4 swiglu")
    oq = oracle.add_norm_qkv(x, r, g, None, "rms", 1e-5, q[:8].contiguous(), s[:8].contiguous(), None, 2, 1, 2)
    _close(np.concatenate([oq["q"].reshape(M, -1), oq["k"].reshape(M, -1), oq["v"].reshape(M, -1)], 1),
           acc[:, :8], rtol=1e-12, atol=1e-14, what="mxfp4 qkv")
    ad = _t(rng.standard_normal((M, K)), torch.bfloat16)
    res = _t(rng.standard_normal((M, 2 * F)), torch.bfloat16)
    _close(oracle.down_residual(ad, q, s, None, res), res.double().numpy() + ad.double().numpy() @ w_val.T,
           rtol=1e-12, atol=1e-14, what="mxfp4 down")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
