"""CPU fp64 oracle of the fused residual-add + norm + projection path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product package.
The arithmetic lives in ``oracle.c`` (plain C, double precision); this module
compiles it with gcc and marshals numpy / torch CPU tensors into it.  It shares
no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_OUT = os.path.join(_HERE, "_build", "liboracle.so")

F32, F16, BF16, I8, I4, E4M3, MXFP4 = 0, 1, 2, 3, 4, 5, 6
MX_BLOCK = 32
E4M3_MAX = 448.0
I4_GROUP = 128
NORM = {"none": 0, "rms": 1, "layer": 2}
ACT = {"none": 0, "swiglu": 1, "gelu_tanh": 2}
DT = {"f32": F32, "f16": F16, "bf16": BF16, "i8": I8}

_lib = None


class using:
    """Temporarily route every call of this module to another build of the
    oracle (the tests use it to run the pins against deliberately broken
    copies and check that the pins notice)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self._saved = _lib
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._saved
        return False


def build(src: Optional[str] = None, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile oracle.c (or another copy of it) with gcc into a shared library
    (``sanitize``: with AddressSanitizer and UndefinedBehaviorSanitizer, for a
    process whose first library is gcc's libasan)."""
    src = src or _SRC
    out = out or _OUT
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp%d" % os.getpid()
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"] \
        if sanitize else []
    # no contraction: the single-precision steps of R11 round after every
    # operation except the one written as fmaf
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11", "-ffp-contract=off", *san,
           "-D_GNU_SOURCE", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: Optional[str] = None):
    """Load (building first if nothing is built) and declare the C signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _OUT
    if not os.path.exists(p):
        build()
    lib = ctypes.CDLL(p)
    vp, i64, dbl, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double, ctypes.c_int
    lib.or_round.argtypes = [dbl, ci]
    lib.or_round.restype = dbl
    lib.or_round_array.argtypes = [vp, vp, i64, ci]
    lib.or_decode_array.argtypes = [vp, ci, i64, vp]
    lib.or_silu.argtypes = [dbl]
    lib.or_silu.restype = dbl
    lib.or_gelu_tanh.argtypes = [dbl]
    lib.or_gelu_tanh.restype = dbl
    lib.or_num_threads.restype = ci
    lib.or_dequant_i8.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.or_dequant_i4.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.or_dequant_i4.restype = ci
    lib.or_i4_value.argtypes = [vp, i64]
    lib.or_i4_value.restype = ci
    lib.or_e4m3_value.argtypes = [ci]
    lib.or_e4m3_value.restype = dbl
    lib.or_e4m3_encode.argtypes = [dbl]
    lib.or_e4m3_encode.restype = ci
    lib.or_e2m1_value.argtypes = [ci]
    lib.or_e2m1_value.restype = dbl
    lib.or_e8m0_value.argtypes = [ci]
    lib.or_e8m0_value.restype = dbl
    lib.or_dequant_mxfp4.argtypes = [vp, vp, i64, i64, vp, vp]
    lib.or_dequant_mxfp4.restype = ci
    lib.or_quant_rows_e4m3.argtypes = [vp, i64, i64, vp, vp, vp]
    lib.or_quant_rows_e4m3.restype = ci
    lib.or_add_norm.argtypes = [vp, vp, vp, vp, ci, ci, dbl, i64, i64, vp, vp, vp, vp]
    lib.or_add_norm.restype = ci
    lib.or_matmul_nt.argtypes = [vp, vp, ci, vp, i64, i64, i64, vp]
    lib.or_matmul_nt.restype = ci
    lib.or_add_norm_qkv.argtypes = [vp, vp, vp, vp, ci, ci, dbl, vp, ci, vp, vp,
                                    i64, i64, i64, i64, i64, vp, vp, vp, vp, ci]
    lib.or_add_norm_qkv.restype = ci
    lib.or_gateup_act.argtypes = [vp, vp, vp, vp, ci, ci, dbl, vp, ci, vp, vp,
                                  i64, i64, i64, ci, vp, vp, ci]
    lib.or_gateup_act.restype = ci
    lib.or_down_residual.argtypes = [vp, ci, vp, ci, vp, vp, vp, i64, i64, i64, vp]
    lib.or_down_residual.restype = ci
    if path is None:
        _lib = lib
    return lib


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _raw(t):
    """(numpy array holding the stored bits, dtype code) of a CPU tensor/array."""
    if t is None:
        return None, None
    if isinstance(t, np.ndarray):
        a = np.ascontiguousarray(t)
        code = {np.dtype(np.float32): F32, np.dtype(np.int8): I8,
                np.dtype(np.float16): F16}[a.dtype]
        return a, code
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy(), BF16
    if t.dtype == torch.float16:
        return t.view(torch.int16).numpy(), F16
    if t.dtype == torch.float32:
        return t.numpy(), F32
    if t.dtype == torch.int8:
        return t.numpy(), I8
    if t.dtype == torch.float8_e4m3fn:       # E4M3 weight codes (R10)
        return t.view(torch.uint8).numpy(), E4M3
    if t.dtype == torch.uint8:               # int4 weights, two per byte (R9)
        return t.numpy(), I4
    if t.dtype == torch.float4_e2m1fn_x2:    # MXFP4 element codes, two per byte (R12)
        return t.view(torch.uint8).numpy(), MXFP4
    raise TypeError(f"oracle: unsupported dtype {t.dtype}")


def _scales(s):
    """Weight scales as the C functions take them: E8M0 bytes for MXFP4
    (torch float8_e8m0fnu), float32 otherwise."""
    if s is None:
        return None
    import torch
    if isinstance(s, torch.Tensor) and s.dtype == torch.float8_e8m0fnu:
        return np.ascontiguousarray(s.detach().cpu().contiguous().view(torch.uint8).numpy())
    return np.ascontiguousarray(_raw(s)[0], dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(shape):
    return np.zeros(shape, dtype=np.float64)


def rne(values, dtype: str) -> np.ndarray:
    """Round float64 values to ``dtype`` (ties to even), returned as float64."""
    v = np.ascontiguousarray(values, dtype=np.float64)
    out = np.empty_like(v)
    load().or_round_array(_ptr(v), _ptr(out), v.size, DT[dtype])
    return out


def decode(t) -> np.ndarray:
    a, code = _raw(t)
    out = np.empty(a.shape, dtype=np.float64)
    load().or_decode_array(_ptr(a), code, a.size, _ptr(out))
    return out


def silu(g: float) -> float:
    return load().or_silu(float(g))


def gelu_tanh(y: float) -> float:
    return load().or_gelu_tanh(float(y))


def num_threads() -> int:
    return load().or_num_threads()


def dequant_i8(q, s):
    """(w as float64, bf16 bit patterns as uint16) of int8 weights q [N, K], scales s [N]."""
    qa, _ = _raw(q)
    sa = np.ascontiguousarray(_raw(s)[0], dtype=np.float32)
    N, K = qa.shape
    w = _f64((N, K))
    bits = np.zeros((N, K), dtype=np.uint16)
    load().or_dequant_i8(_ptr(qa), _ptr(sa), N, K, _ptr(w), _ptr(bits))
    return w, bits


def dequant_i4(q, s):
    """(w as float64 [N, K], bf16 bit patterns as uint16) of int4 weights q
    [N, K/2] (uint8, two per byte, even k in the low nibble) with group scales
    s [N, K/128] (R9)."""
    qa, _ = _raw(q)
    sa = np.ascontiguousarray(_raw(s)[0], dtype=np.float32)
    N, K = qa.shape[0], 2 * qa.shape[1]
    w = _f64((N, K))
    bits = np.zeros((N, K), dtype=np.uint16)
    assert load().or_dequant_i4(_ptr(qa), _ptr(sa), N, K, _ptr(w), _ptr(bits)) == 0
    return w, bits


def dequant_mxfp4(q, s):
    """(w as float64 [N, K], bf16 bit patterns as uint16) of MXFP4 weights q
    [N, K/2] (float4_e2m1fn_x2: two E2M1 codes per byte, even k in the low
    nibble) with E8M0 block scales s [N, K/32] (float8_e8m0fnu) (R12)."""
    qa, _ = _raw(q)
    sa = _scales(s)
    N, K = qa.shape[0], 2 * qa.shape[1]
    w = _f64((N, K))
    bits = np.zeros((N, K), dtype=np.uint16)
    assert load().or_dequant_mxfp4(_ptr(qa), _ptr(sa), N, K, _ptr(w), _ptr(bits)) == 0
    return w, bits


def e2m1_value(code: int) -> float:
    """Value of one E2M1 code (R12)."""
    return load().or_e2m1_value(int(code))


def e8m0_value(code: int) -> float:
    """Value of one E8M0 scale code (R12)."""
    return load().or_e8m0_value(int(code))


def e4m3_value(code: int) -> float:
    """Value of one E4M3 code (R10)."""
    return load().or_e4m3_value(int(code))


def e4m3_encode(t: float) -> int:
    """Nearest E4M3 code of t (ties to the even code, magnitudes past 448 as 448)."""
    return load().or_e4m3_encode(float(t))


def quant_rows_e4m3(n):
    """Per-token E4M3 quantisation of float64 rows n [M, K] (R10):
    (codes uint8 [M, K], a = e4m3(code) * s_a float64 [M, K], s_a float64 [M])."""
    n = np.ascontiguousarray(n, dtype=np.float64)
    M, K = n.shape
    codes = np.zeros((M, K), dtype=np.uint8)
    a, s = _f64((M, K)), _f64((M,))
    assert load().or_quant_rows_e4m3(_ptr(n), M, K, _ptr(codes), _ptr(a), _ptr(s)) == 0
    return codes, a, s


def add_norm(x, r, gamma, beta, norm: str, eps: float):
    """(h_out, n, a) for the rows of x: the rounded residual stream, the
    double-precision normalised rows (R2 / R3), and the single-precision
    normalised rows of R11 rounded to the activation dtype (the GEMM operand
    of reading A)."""
    h, n, _, a = _add_norm(x, r, gamma, beta, norm, eps)
    return h, n, a


def add_norm_f32(x, r, gamma, beta, norm: str, eps: float) -> np.ndarray:
    """The single-precision normalised rows n32 of R11 (as float64 values)."""
    return _add_norm(x, r, gamma, beta, norm, eps)[2]


def _add_norm(x, r, gamma, beta, norm: str, eps: float):
    xa, act = _raw(x)
    M, K = xa.shape
    ra, _ = _raw(r)
    ga, _ = _raw(gamma)
    ba, _ = _raw(beta)
    h, n, n32, a = _f64((M, K)), _f64((M, K)), _f64((M, K)), _f64((M, K))
    rc = load().or_add_norm(_ptr(xa), _ptr(ra), _ptr(ga), _ptr(ba), act, NORM[norm],
                            float(np.float32(eps)), M, K, _ptr(h), _ptr(n), _ptr(n32), _ptr(a))
    assert rc == 0
    return h, n, n32, a


def matmul_nt(a: np.ndarray, w, w_scale=None) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    wa, wdt = _raw(w)
    sa = _scales(w_scale)
    M, K = a.shape
    N = wa.shape[0]
    acc = _f64((M, N))
    assert load().or_matmul_nt(_ptr(a), _ptr(wa), wdt, _ptr(sa), M, K, N, _ptr(acc)) == 0
    return acc


def add_norm_qkv(x, r, gamma, beta, norm: str, eps: float, w, w_scale, bias,
                 n_heads: int, n_kv_heads: int, head_dim: int,
                 rounded: bool = True) -> Dict[str, np.ndarray]:
    xa, act = _raw(x)
    M, K = xa.shape
    ra, _ = _raw(r)
    ga, _ = _raw(gamma)
    ba, _ = _raw(beta)
    wa, wdt = _raw(w)
    sa = _scales(w_scale)
    bia, _ = _raw(bias)
    q = _f64((M, n_heads, head_dim))
    k = _f64((M, n_kv_heads, head_dim))
    v = _f64((M, n_kv_heads, head_dim))
    h = _f64((M, K))
    rc = load().or_add_norm_qkv(_ptr(xa), _ptr(ra), _ptr(ga), _ptr(ba), act, NORM[norm],
                                float(np.float32(eps)), _ptr(wa), wdt, _ptr(sa), _ptr(bia),
                                M, K, n_heads, n_kv_heads, head_dim,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(h), int(rounded))
    assert rc == 0
    return {"q": q, "k": k, "v": v, "h_out": h}


def gateup_act(x, r, gamma, beta, norm: str, eps: float, w, w_scale, bias,
               ffn: int, act_fn: str, rounded: bool = True) -> Dict[str, np.ndarray]:
    xa, act = _raw(x)
    M, K = xa.shape
    ra, _ = _raw(r)
    ga, _ = _raw(gamma)
    ba, _ = _raw(beta)
    wa, wdt = _raw(w)
    sa = _scales(w_scale)
    bia, _ = _raw(bias)
    out = _f64((M, ffn))
    h = _f64((M, K))
    rc = load().or_gateup_act(_ptr(xa), _ptr(ra), _ptr(ga), _ptr(ba), act, NORM[norm],
                              float(np.float32(eps)), _ptr(wa), wdt, _ptr(sa), _ptr(bia),
                              M, K, ffn, ACT[act_fn], _ptr(out), _ptr(h), int(rounded))
    assert rc == 0
    return {"out": out, "h_out": h}


def down_residual(a, w, w_scale, bias, residual) -> np.ndarray:
    """out = residual + bias + a @ w^T in float64 (a [M, K] as stored, w [N, K])."""
    aa, act = _raw(a)
    M, K = aa.shape
    wa, wdt = _raw(w)
    N = wa.shape[0]
    sa = _scales(w_scale)
    ba, _ = _raw(bias)
    ra, _ = _raw(residual)
    out = _f64((M, N))
    assert load().or_down_residual(_ptr(aa), act, _ptr(wa), wdt, _ptr(sa), _ptr(ba), _ptr(ra),
                                   M, K, N, _ptr(out)) == 0
    return out


def workload_qkv(wl, inp, row_idx=None, rounded=True):
    """Oracle of the QKV call of a workload on (optionally a subset of) its rows."""
    x, r = inp["x"], inp["r"]
    if row_idx is not None:
        import torch
        idx = torch.as_tensor(row_idx, dtype=torch.long)
        x, r = x[idx].contiguous(), r[idx].contiguous()
    return add_norm_qkv(x, r, inp["gamma"], inp.get("beta"), wl.norm, wl.eps,
                        inp["w_qkv"], inp.get("s_qkv"), inp.get("b_qkv"),
                        wl.n_heads, wl.n_kv_heads, wl.head_dim, rounded=rounded)


def workload_gateup(wl, inp, row_idx=None, rounded=True):
    """Oracle of the gate/up (or up) call of a workload."""
    x, r = inp["x"], inp["r"]
    if row_idx is not None:
        import torch
        idx = torch.as_tensor(row_idx, dtype=torch.long)
        x, r = x[idx].contiguous(), r[idx].contiguous()
    return gateup_act(x, r, inp["gamma"], inp.get("beta"), wl.norm, wl.eps,
                      inp["w_gu"], inp.get("s_gu"), inp.get("b_gu"),
                      wl.ffn, wl.act_fn, rounded=rounded)
