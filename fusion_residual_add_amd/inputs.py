"""Seeded synthetic inputs for the fused projection path.

This module only *draws* inputs: it holds none of the arithmetic of the method
(no residual add, no normalisation, no matmul, no activation, no dequantisation).
Both the HIP path and the CPU oracle take their inputs from here, and from
nowhere else, so the two sides see bit-identical tensors.

Recipe (stated once, used everywhere):

* generator: numpy PCG64, ``numpy.random.default_rng(seed)``;
* draw order per workload: x, residual, gamma, beta, W_qkv, b_qkv, W_gu, b_gu
  (items a workload does not use are skipped, the order of the rest is kept);
* normal draws are float32 ziggurat samples (``standard_normal(dtype=float32)``)
  scaled by the standard deviation in float32; uniform draws are float64 and
  rounded to float32;
* float32 values are then rounded to the activation dtype by torch's cast,
  which is round-to-nearest-even;
* weights are drawn directly in the ``[N, K]`` (output-major, K contiguous)
  layout that the library consumes;
* int8 weights: a float32 weight is drawn as above, then quantised per output
  row with the symmetric max-abs rule ``s = max|w| / 127`` (float32) and
  ``q = clip(rint(w / s), -127, 127)``.  The stored inputs of the method are
  ``(q, s)``; how they were produced is not part of the path;
* int4 weights (4-bit weights with 16-bit activations, group 128, no zero
  point): per output row and group of 128 consecutive k,
  ``s = max|w| / 7`` (float32) and ``q = clip(rint(w / s), -8, 7)``, packed
  two per byte along k (even k in the low nibble), scales ``[N, K/128]``;
* MXFP4 weights (FP4 weights with 16-bit activations, one 8-bit power-of-two
  scale per 32 consecutive k): per row and block, the shared exponent
  ``e = floor(log2(max|w|)) - 2`` (2 being the largest E2M1 exponent), scale
  code ``e + 127``, element codes the nearest E2M1 value (ties to the even
  code) of ``w / 2^e`` saturated at +-6, packed two per byte along k.

Workload shapes follow the five transformer-block configurations that the
fused-projection pages are measured on: a tiny fp32 block, a Llama-3-8B decode
step, a Llama-2-7B prefill batch, a GPT-style fp16 LayerNorm + GELU block, and
a Llama-2-70B layer with int8 weights at four token counts.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "quantize_rows_i8", "quantize_groups_i4",
           "quantize_rows_e4m3", "quantize_blocks_mxfp4"]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    hidden: int
    act: str                    # "f32" | "f16" | "bf16"
    wdt: str                    # "f32" | "f16" | "bf16" | "i8" | "i4" | "e4m3" | "mxfp4"
    norm: str                   # "rms" | "layer"
    eps: float
    x_std: float
    r_std: float
    gamma_lo: float
    gamma_hi: float
    beta_std: Optional[float]   # LayerNorm only
    w_std: float
    # QKV projection (None when the workload has no QKV call)
    n_heads: Optional[int]
    n_kv_heads: Optional[int]
    head_dim: Optional[int]
    # gate/up or up projection
    ffn: int
    act_fn: str                 # "swiglu" | "gelu_tanh" | "none"
    bias_std: Optional[float]   # bias of the gate/up (or up) projection

    @property
    def n_qkv(self) -> int:
        if self.n_heads is None:
            return 0
        return (self.n_heads + 2 * self.n_kv_heads) * self.head_dim

    @property
    def n_gu(self) -> int:
        return 2 * self.ffn if self.act_fn == "swiglu" else self.ffn

    def with_m(self, M: int) -> "Workload":
        return dataclasses.replace(self, M=M, name=f"{self.name.split('@')[0]}@M{M}")


def _llama70b(M: int) -> Workload:
    return Workload(
        name=f"llama2-70b-int8w@M{M}", M=M, hidden=8192, act="bf16", wdt="i8",
        norm="rms", eps=1e-5, x_std=1.0, r_std=1.0, gamma_lo=0.8, gamma_hi=1.2,
        beta_std=None, w_std=0.02, n_heads=64, n_kv_heads=8, head_dim=128,
        ffn=28672, act_fn="swiglu", bias_std=None)


def _llama70b_tp8(M: int) -> Workload:
    """One GPU's share of the Llama-2-70B int8 layer under 8-way tensor
    parallelism: 8 of the 64 Q heads, 1 of the 8 KV heads, 3584 of the 28672
    gate/up rows (each with its matching up row)."""
    return dataclasses.replace(_llama70b(M), name=f"llama2-70b-int8w-tp8@M{M}", n_heads=8, n_kv_heads=1,
                               ffn=28672 // 8)


def _llama70b_i4(M: int) -> Workload:
    """The Llama-2-70B layer with int4 weights, one scale per 128 k (the
    4-bit weight-only configuration of the pages' quantisation section)."""
    return dataclasses.replace(_llama70b(M), name=f"llama2-70b-int4w@M{M}", wdt="i4")


def _llama70b_mxfp4(M: int) -> Workload:
    """The Llama-2-70B layer with MXFP4 weights (E2M1 elements, one E8M0 scale
    per 32 k) and bf16 activations (the pages' FP4 weight configuration)."""
    return dataclasses.replace(_llama70b(M), name=f"llama2-70b-mxfp4w@M{M}", wdt="mxfp4")


def _fp8(base: Workload, name: str) -> Workload:
    """A workload's shapes with E4M3 weights (per-row scales) and per-token
    E4M3 activations (the pages' full-FP8 configuration)."""
    return dataclasses.replace(base, name=name, wdt="e4m3")


WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 block: M=4, hidden=256, 4 Q / 2 KV heads of 64, ffn=512
    "tiny-f32": Workload(
        name="tiny-f32", M=4, hidden=256, act="f32", wdt="f32", norm="rms",
        eps=1e-5, x_std=1.0, r_std=1.0, gamma_lo=0.5, gamma_hi=1.5,
        beta_std=None, w_std=1.0 / 16.0, n_heads=4, n_kv_heads=2, head_dim=64,
        ffn=512, act_fn="swiglu", bias_std=None),
    # Llama-3-8B-shaped decode step, bf16
    "llama3-8b-decode": Workload(
        name="llama3-8b-decode", M=32, hidden=4096, act="bf16", wdt="bf16",
        norm="rms", eps=1e-5, x_std=1.0, r_std=1.0, gamma_lo=0.8, gamma_hi=1.2,
        beta_std=None, w_std=0.02, n_heads=32, n_kv_heads=8, head_dim=128,
        ffn=14336, act_fn="swiglu", bias_std=None),
    # Llama-2-7B-shaped prefill (32 x 512 tokens), bf16, MHA; the tiny block's
    # distributions with the weight std taken as 1/sqrt(hidden)
    "llama2-7b-prefill": Workload(
        name="llama2-7b-prefill", M=16384, hidden=4096, act="bf16", wdt="bf16",
        norm="rms", eps=1e-5, x_std=1.0, r_std=1.0, gamma_lo=0.5, gamma_hi=1.5,
        beta_std=None, w_std=1.0 / 64.0, n_heads=32, n_kv_heads=32,
        head_dim=128, ffn=11008, act_fn="swiglu", bias_std=None),
    # GPT-style fp16 block: add + LayerNorm -> up GEMM + bias + tanh-GELU
    "gpt-fp16-gelu": Workload(
        name="gpt-fp16-gelu", M=2048, hidden=4096, act="f16", wdt="f16",
        norm="layer", eps=1e-5, x_std=1.0, r_std=1.0, gamma_lo=0.8,
        gamma_hi=1.2, beta_std=0.02, w_std=0.02, n_heads=None,
        n_kv_heads=None, head_dim=None, ffn=16384, act_fn="gelu_tanh",
        bias_std=0.02),
    "llama2-70b-int8w@M1": _llama70b(1),
    "llama2-70b-int8w@M16": _llama70b(16),
    "llama2-70b-int8w@M64": _llama70b(64),
    "llama2-70b-int8w@M256": _llama70b(256),
    "llama2-70b-int8w-tp8@M1": _llama70b_tp8(1),
    "llama2-70b-int8w-tp8@M16": _llama70b_tp8(16),
    "llama2-70b-int8w-tp8@M64": _llama70b_tp8(64),
    "llama2-70b-int4w@M1": _llama70b_i4(1),
    "llama2-70b-int4w@M16": _llama70b_i4(16),
    "llama2-70b-int4w@M256": _llama70b_i4(256),
    "llama2-70b-mxfp4w@M1": _llama70b_mxfp4(1),
    "llama2-70b-mxfp4w@M16": _llama70b_mxfp4(16),
    "llama2-70b-mxfp4w@M64": _llama70b_mxfp4(64),
    "llama2-70b-mxfp4w@M256": _llama70b_mxfp4(256),
}


# the same prefill batch with the tiny block's weight spread taken literally
# (std 1/16 = 1/sqrt(256)): outputs about four times larger
WORKLOADS["llama2-7b-prefill-w16"] = dataclasses.replace(WORKLOADS["llama2-7b-prefill"],
                                                         name="llama2-7b-prefill-w16", w_std=1.0 / 16.0)
WORKLOADS["llama2-7b-prefill-fp8"] = _fp8(WORKLOADS["llama2-7b-prefill"], "llama2-7b-prefill-fp8")
WORKLOADS["llama3-8b-decode-fp8"] = _fp8(WORKLOADS["llama3-8b-decode"], "llama3-8b-decode-fp8")
WORKLOADS["gpt-fp16-gelu-fp8"] = _fp8(WORKLOADS["gpt-fp16-gelu"], "gpt-fp16-gelu-fp8")


def workload(name: str) -> Workload:
    return WORKLOADS[name]


_TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(std)
    return v


def _uniform(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def _to_act(v: np.ndarray, act: str) -> torch.Tensor:
    return torch.from_numpy(v).to(_TORCH_DT[act])


def quantize_rows_i8(w: np.ndarray):
    """Symmetric per-output-row int8 storage of a float32 ``[N, K]`` weight.

    ``s[j] = max_k |w[j, k]| / 127`` in float32 and
    ``q[j, k] = clip(rint(w[j, k] / s[j]), -127, 127)``; a zero row gets s = 0
    and q = 0.  This produces the *stored* weights; the method only ever reads
    ``(q, s)``.  Rows are processed in blocks to bound host memory.
    """
    N, K = w.shape
    q = np.empty((N, K), dtype=np.int8)
    s = np.empty((N,), dtype=np.float32)
    step = max(1, (1 << 24) // max(K, 1))
    for j0 in range(0, N, step):
        blk = w[j0:j0 + step]
        amax = np.abs(blk).max(axis=1).astype(np.float32)
        sc = (amax / np.float32(127.0)).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        qq = np.rint(blk / safe[:, None])
        qq = np.clip(qq, -127, 127)
        qq[sc == 0] = 0
        q[j0:j0 + step] = qq.astype(np.int8)
        s[j0:j0 + step] = sc
    return torch.from_numpy(q), torch.from_numpy(s)


I4_GROUP = 128


def quantize_groups_i4(w: np.ndarray):
    """Symmetric int4 storage of a float32 ``[N, K]`` weight, one scale per
    row and group of 128 consecutive k.

    ``s[j, g] = max |w[j, 128 g : 128 g + 128]| / 7`` in float32 and
    ``q = clip(rint(w / s), -8, 7)`` (an all-zero group gets s = 0, q = 0);
    returns ``(q packed [N, K/2] uint8, s [N, K/128] float32)`` with element
    2i of a row in the low nibble of byte i and 2i + 1 in the high nibble,
    each a 4-bit two's-complement value.
    """
    N, K = w.shape
    assert K % I4_GROUP == 0, "int4 weights need K a multiple of 128"
    G = K // I4_GROUP
    q = np.empty((N, K // 2), dtype=np.uint8)
    s = np.empty((N, G), dtype=np.float32)
    step = max(1, (1 << 24) // max(K, 1))
    for j0 in range(0, N, step):
        blk = w[j0:j0 + step].reshape(-1, G, I4_GROUP)
        amax = np.abs(blk).max(axis=2).astype(np.float32)
        sc = (amax / np.float32(7.0)).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        qq = np.clip(np.rint(blk / safe[:, :, None]), -8, 7)
        qq[sc == 0] = 0
        nib = (qq.astype(np.int16).reshape(blk.shape[0], K) & 0xF).astype(np.uint8)
        q[j0:j0 + step] = nib[:, 0::2] | (nib[:, 1::2] << 4)
        s[j0:j0 + step] = sc
    return torch.from_numpy(q), torch.from_numpy(s)


E4M3_MAX = 448.0


def quantize_rows_e4m3(w: np.ndarray):
    """E4M3 storage of a float32 ``[N, K]`` weight, one scale per output row.

    ``s[j] = max_k |w[j, k]| / 448`` in float32 and the codes are torch's
    nearest-even float8_e4m3fn conversion of ``w / s`` (clipped to +-448); a
    zero row gets s = 0 and zero codes.  Returns ``(codes [N, K]
    float8_e4m3fn, s [N] float32)``; the method only ever reads them.
    """
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.float8_e4m3fn)
    s = np.empty((N,), dtype=np.float32)
    step = max(1, (1 << 24) // max(K, 1))
    for j0 in range(0, N, step):
        blk = w[j0:j0 + step]
        amax = np.abs(blk).max(axis=1).astype(np.float32)
        sc = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        safe = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
        t = np.clip(blk / safe[:, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
        t[sc == 0] = 0
        q[j0:j0 + step] = torch.from_numpy(t).to(torch.float8_e4m3fn)
        s[j0:j0 + step] = sc
    return q, torch.from_numpy(s)


MX_BLOCK = 32
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


_E2M1_MIDS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_MID_UP = (False, True, False, True, False, True, False)   # midpoints whose lower code is odd


def _e2m1_codes(t: torch.Tensor) -> torch.Tensor:
    """Nearest E2M1 code of each value (ties to the even code, i.e. the one
    with mantissa bit 0), magnitudes saturated at 6, sign kept (-0 for
    negative values that round to zero): the number of midpoints below the
    magnitude, plus one at a midpoint whose lower neighbour is odd."""
    a = t.abs()
    idx = torch.zeros(t.shape, dtype=torch.uint8)
    for mid, up in zip(_E2M1_MIDS, _E2M1_MID_UP):
        idx += (a > mid) | (a == mid) & up
    return idx | torch.signbit(t).to(torch.uint8) * 8


def quantize_blocks_mxfp4(w: np.ndarray):
    """MXFP4 storage of a float32 ``[N, K]`` weight: per row and block of 32
    consecutive k, the shared exponent e = floor(log2(max |w|)) - 2 (clamped to
    the E8M0 range; an all-zero block takes e = 0), the scale code e + 127 and
    the element codes _e2m1_codes(w / 2^e).  Returns ``(codes [N, K/2]
    float4_e2m1fn_x2, element 2i of a row in the low nibble of byte i,
    scales [N, K/32] float8_e8m0fnu)``; the method only ever reads them."""
    N, K = w.shape
    assert K % MX_BLOCK == 0, "MXFP4 weights need K a multiple of 32"
    G = K // MX_BLOCK
    q = torch.empty((N, K // 2), dtype=torch.uint8)
    s = torch.empty((N, G), dtype=torch.uint8)
    step = max(1, (1 << 24) // max(K, 1))
    for j0 in range(0, N, step):
        blk = torch.from_numpy(np.ascontiguousarray(w[j0:j0 + step], dtype=np.float32)).view(-1, G, MX_BLOCK)
        amax = blk.abs().amax(dim=2)
        # floor(log2(amax)) exactly: amax = f 2^x with f in [0.5, 1) gives x - 1
        e = torch.where(amax > 0, torch.frexp(amax).exponent - 3, 0).clamp(-127, 127)
        codes = _e2m1_codes(torch.ldexp(blk, -e[:, :, None].to(torch.float32))).view(blk.shape[0], K)
        q[j0:j0 + step] = codes[:, 0::2] | (codes[:, 1::2] << 4)
        s[j0:j0 + step] = (e + 127).to(torch.uint8)
    return q.view(torch.float4_e2m1fn_x2), s.view(torch.float8_e8m0fnu)


def _weight(rng, wl: Workload, N: int):
    w = _normal(rng, (N, wl.hidden), wl.w_std)
    if wl.wdt == "e4m3":
        return quantize_rows_e4m3(w)
    if wl.wdt == "i8":
        q, s = quantize_rows_i8(w)
        return q, s
    if wl.wdt == "i4":
        return quantize_groups_i4(w)
    if wl.wdt == "mxfp4":
        return quantize_blocks_mxfp4(w)
    return _to_act(w, wl.wdt), None


def generate(wl: Workload, seed: int = 0, parts=("qkv", "gu")) -> Dict[str, torch.Tensor]:
    """All host tensors of one workload (CPU torch tensors, contiguous).

    Keys: x, r, gamma, beta (LayerNorm only), and per projection
    w_qkv / s_qkv / b_qkv and w_gu / s_gu / b_gu.  ``s_*`` is present only for
    int8, int4 and E4M3 weights; ``b_*`` only when the workload has that bias.  ``parts``
    selects which projections to draw, but the draw order (and hence every
    value) does not depend on it: skipped weights are still drawn.
    """
    rng = np.random.default_rng(seed)
    out: Dict[str, torch.Tensor] = {}
    M, K = wl.M, wl.hidden
    out["x"] = _to_act(_normal(rng, (M, K), wl.x_std), wl.act)
    out["r"] = _to_act(_normal(rng, (M, K), wl.r_std), wl.act)
    out["gamma"] = _to_act(_uniform(rng, (K,), wl.gamma_lo, wl.gamma_hi), wl.act)
    if wl.norm == "layer":
        out["beta"] = _to_act(_normal(rng, (K,), wl.beta_std), wl.act)
    if wl.n_qkv:
        w, s = _weight(rng, wl, wl.n_qkv)
        if "qkv" in parts:
            out["w_qkv"] = w
            if s is not None:
                out["s_qkv"] = s
        del w, s
    w, s = _weight(rng, wl, wl.n_gu)
    if "gu" in parts:
        out["w_gu"] = w
        if s is not None:
            out["s_gu"] = s
    del w, s
    if wl.bias_std is not None:
        out["b_gu"] = _to_act(_normal(rng, (wl.n_gu,), wl.bias_std), wl.act)
    if "down" in parts:
        # the down projection (drawn last, so asking for it changes no other
        # value): its input a [M, ffn] ~ N(0, 1) stands for the gate/up output,
        # its weight [hidden, ffn] has the workload's weight distribution, and
        # r doubles as the residual it adds
        out["a_down"] = _to_act(_normal(rng, (M, wl.ffn), 1.0), wl.act)
        w = _normal(rng, (wl.hidden, wl.ffn), wl.w_std)
        if wl.wdt == "i8":
            out["w_down"], out["s_down"] = quantize_rows_i8(w)
        elif wl.wdt == "i4":
            out["w_down"], out["s_down"] = quantize_groups_i4(w)
        elif wl.wdt == "e4m3":
            out["w_down"], out["s_down"] = quantize_rows_e4m3(w)
        elif wl.wdt == "mxfp4":
            out["w_down"], out["s_down"] = quantize_blocks_mxfp4(w)
        else:
            out["w_down"] = _to_act(w, wl.wdt)
        del w
    return out


def device_normal(shape, std: float, dtype: torch.dtype, device, seed: int) -> torch.Tensor:
    """Seeded N(0, std) draws made on the device, for inputs too large to draw
    on the host (past 4 GiB): torch's generator on ``device`` seeded with
    ``seed``, float32 samples scaled by std, rounded to ``dtype`` (RNE), drawn
    in slices of at most 2^28 elements so the float32 staging stays small."""
    return _device_draw(shape, dtype, device, seed, lambda t, g: t.normal_(0.0, std, generator=g))


def device_uniform(shape, lo: float, hi: float, dtype: torch.dtype, device, seed: int) -> torch.Tensor:
    """Seeded U(lo, hi) draws made on the device; as ``device_normal``."""
    return _device_draw(shape, dtype, device, seed, lambda t, g: t.uniform_(lo, hi, generator=g))


def _device_draw(shape, dtype, device, seed, fill) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        tmp = torch.empty(n, dtype=torch.float32, device=device)
        fill(tmp, g)
        flat[i:i + n].copy_(tmp)
        del tmp
    return out


def rows(t: torch.Tensor, idx) -> torch.Tensor:
    """Gather token rows (rows are independent in every step of the path)."""
    return t[torch.as_tensor(idx, dtype=torch.long)].contiguous()
