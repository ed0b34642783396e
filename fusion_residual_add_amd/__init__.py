"""fusion_residual_add_amd: fused residual-add + norm + projection kernels for MI355X.

Python binding over the C ABI of ``libfusedproj.so`` (include/fusedproj.h).
This layer only marshals arguments: it checks that tensors are contiguous
device tensors of the expected dtype, allocates output / workspace tensors with
PyTorch when the caller does not pass them, and passes raw pointers and the
current HIP stream to the library.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import torch

from . import _lib
from ._lib import FP_ACT, FP_NORM

__all__ = ["fused_add_norm_qkv", "fused_add_norm_qkv_noalloc", "fused_gateup_act", "fused_down_residual", "fused_dequant_i8_bf16",
           "fused_dequant_i4_bf16", "fused_dequant_mxfp4_bf16",
           "workspace_bytes", "describe_plan", "FusedProjError", "profile_start", "profile_stop",
           "library_path", "tune_install", "tune_clear", "tune_count", "plan_override",
           "set_plan_override", "get_plan_override", "PackedWeight", "pack_weight", "unpack_weight"]

# torch.uint8 weights are int4 pairs (two values per byte, even k in the low nibble)
# torch.float4_e2m1fn_x2 weights are MXFP4 element pairs (two per byte, even
# k in the low nibble), with torch.float8_e8m0fnu block scales
_DT = {torch.float32: _lib.FP_F32, torch.float16: _lib.FP_F16,
       torch.bfloat16: _lib.FP_BF16, torch.int8: _lib.FP_I8, torch.uint8: _lib.FP_I4,
       torch.float8_e4m3fn: _lib.FP_E4M3, torch.float4_e2m1fn_x2: _lib.FP_MXFP4}
_PACKED4 = (torch.uint8, torch.float4_e2m1fn_x2)
_LAYOUT = {"rows": 0, "packed": _lib.FP_LAYOUT_PACKED, "packed_gate_up": _lib.FP_LAYOUT_PACKED_GATE_UP}


class PackedWeight:
    """A weight tile-packed by fused_pack_weight (see ``pack_weight``).

    ``data`` has the dtype and shape of the row-major weight and holds the same
    bytes in the packed order; ``gate_up`` is the gate/up pairing, for the
    SwiGLU gate/up call.  The projection calls take it wherever they take a
    weight; their results do not depend on the layout."""
    __slots__ = ("data", "gate_up")

    def __init__(self, data: torch.Tensor, gate_up: bool):
        self.data = data
        self.gate_up = bool(gate_up)

    @property
    def dtype(self) -> torch.dtype:
        return self.data.dtype

    @property
    def shape(self):
        return self.data.shape

    @property
    def device(self):
        return self.data.device

    @property
    def layout(self) -> str:
        return "packed_gate_up" if self.gate_up else "packed"


def _wcode(w) -> Tuple[torch.Tensor, int]:
    """The weight tensor and its w_dtype code (element type | layout bits)."""
    if isinstance(w, PackedWeight):
        return w.data, _DT[w.data.dtype] | _LAYOUT[w.layout]
    return w, _DT[w.dtype]


def _elems_per_row(w: torch.Tensor) -> int:
    return w.shape[1] * 2 if w.dtype in _PACKED4 else w.shape[1]


def pack_weight(w: torch.Tensor, gate_up: bool = False, out: Optional[torch.Tensor] = None) -> PackedWeight:
    """fused_pack_weight: the tile-packed copy of a row-major weight [N, K]
    (4-bit: [N, K / 2]) -- once, when a model is loaded.  ``gate_up``: the
    weight of the SwiGLU gate/up call ([gate; up], N = 2 ffn)."""
    lib = _lib.load()
    _ptr(w, "w")
    if w.dim() != 2:
        raise ValueError(f"w must be 2-D, got shape {tuple(w.shape)}")
    if out is None:
        out = torch.empty_like(w)
    if out.shape != w.shape or out.dtype != w.dtype:
        raise ValueError("out must have the shape and dtype of w")
    st = lib.fused_pack_weight(w.data_ptr(), _ptr(out, "out", w.device), w.shape[0], _elems_per_row(w),
                               _DT[w.dtype], int(bool(gate_up)), _stream(w.device))
    _check("fused_pack_weight", st)
    return PackedWeight(out, gate_up)


def unpack_weight(pw: PackedWeight, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fused_unpack_weight: the row-major weight back from a PackedWeight."""
    lib = _lib.load()
    w = pw.data
    _ptr(w, "w")
    if out is None:
        out = torch.empty_like(w)
    if out.shape != w.shape or out.dtype != w.dtype:
        raise ValueError("out must have the shape and dtype of the packed weight")
    st = lib.fused_unpack_weight(w.data_ptr(), _ptr(out, "out", w.device), w.shape[0], _elems_per_row(w),
                                 _DT[w.dtype], int(pw.gate_up), _stream(w.device))
    _check("fused_unpack_weight", st)
    return out


def _scale_dtype(w: torch.Tensor) -> torch.dtype:
    return torch.float8_e8m0fnu if w.dtype == torch.float4_e2m1fn_x2 else torch.float32


def _check_weight(w: torch.Tensor, w_scale: Optional[torch.Tensor], Nw: int, K: int, name: str):
    """Shapes of the weight and its scales for the weight dtype."""
    want = (Nw, K // 2) if w.dtype in _PACKED4 else (Nw, K)
    if tuple(w.shape) != want:
        raise ValueError(f"{name} has shape {tuple(w.shape)}, expected {want}")
    if w.dtype in (torch.int8, torch.float8_e4m3fn) and w_scale is not None and tuple(w_scale.shape) != (Nw,):
        raise ValueError(f"w_scale has shape {tuple(w_scale.shape)}, expected {(Nw,)}")
    if w.dtype == torch.uint8 and w_scale is not None and tuple(w_scale.shape) != (Nw, K // 128):
        raise ValueError(f"w_scale has shape {tuple(w_scale.shape)}, expected {(Nw, K // 128)}")
    if w.dtype == torch.float4_e2m1fn_x2 and w_scale is not None and tuple(w_scale.shape) != (Nw, K // 32):
        raise ValueError(f"w_scale has shape {tuple(w_scale.shape)}, expected {(Nw, K // 32)}")


class FusedProjError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        self.status = status
        name = _lib.STATUS[status] if 0 <= status < len(_lib.STATUS) else str(status)
        super().__init__(f"{fn}: {name}: {msg}")


def library_path() -> str:
    return _lib.LIB_PATH


def _check(fn: str, status: int):
    if status != 0:
        lib = _lib.load()
        raise FusedProjError(fn, status, lib.fp_last_error().decode())


def _ptr(t: Optional[torch.Tensor], name: str, device=None, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


_WS: Dict[Tuple[int, int], torch.Tensor] = {}


def workspace_bytes(M: int, hidden: int, n_cols: int, act_dtype: torch.dtype,
                    w_dtype: torch.dtype, layout: str = "rows") -> int:
    return int(_lib.load().fp_workspace_bytes(M, hidden, n_cols, _DT[act_dtype], _DT[w_dtype] | _LAYOUT[layout]))


def down_workspace_bytes(M: int, ffn: int, hidden: int, act_dtype: torch.dtype, w_dtype: torch.dtype,
                         layout: str = "rows") -> int:
    return int(_lib.load().fp_down_workspace_bytes(M, ffn, hidden, _DT[act_dtype], _DT[w_dtype] | _LAYOUT[layout]))


def describe_plan(M: int, hidden: int, n_cols: int, act_dtype: torch.dtype, w_dtype: torch.dtype,
                  act: str = "none", layout: str = "rows") -> dict:
    """The kernel and launch shape a call with these sizes would use (no device
    work): {"family", "kernel", "grid", "splits", "slots", "workspace"}.
    ``layout``: "rows", "packed" or "packed_gate_up" (see pack_weight)."""
    import ctypes
    lib = _lib.load()
    buf = ctypes.create_string_buffer(256)
    st = lib.fp_describe_plan(M, hidden, n_cols, _DT[act_dtype], _DT[w_dtype] | _LAYOUT[layout], _lib.FP_ACT[act],
                              buf, 256)
    if st != 0:
        raise FusedProjError("fp_describe_plan", st, lib.fp_last_error().decode())
    out = dict(kv.split("=", 1) for kv in buf.value.decode().split(" "))
    for k in ("grid", "splits", "slots", "workspace"):
        out[k] = int(out[k])
    return out


def _workspace(device: torch.device, stream: int, nbytes: int) -> Optional[torch.Tensor]:
    """Per (device, stream) cached workspace: calls on one stream are ordered,
    so they may share it."""
    if nbytes == 0:
        return None
    key = (device.index, stream)
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def fused_add_norm_qkv(x: torch.Tensor, residual: Optional[torch.Tensor], gamma: Optional[torch.Tensor],
                       w_qkv: torch.Tensor | PackedWeight, n_heads: int, n_kv_heads: int, head_dim: int, *,
                       beta: Optional[torch.Tensor] = None, norm: str = "rms", eps: float = 1e-5,
                       w_scale: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                       write_h: bool = True, out_dtype: Optional[torch.dtype] = None,
                       h_out: Optional[torch.Tensor] = None, q: Optional[torch.Tensor] = None,
                       k: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, head_major: bool = False):
    """residual add + norm -> QKV projection (+bias) -> q [M,H,D], k/v [M,Hkv,D]
    (``head_major``: q [H,M,D], k/v [Hkv,M,D], through fused_add_norm_qkv_hm).

    Returns (q, k, v, h_out) where h_out = rne(x + residual) (None when
    ``write_h`` is False and no h_out tensor was passed)."""
    lib = _lib.load()
    _ptr(x, "x")
    dev = x.device
    M, K = x.shape
    act = x.dtype
    odt = out_dtype or act
    w_qkv, wcode = _wcode(w_qkv)
    Nw = (n_heads + 2 * n_kv_heads) * head_dim
    _check_weight(w_qkv, w_scale, Nw, K, "w_qkv")
    qs = (n_heads, M, head_dim) if head_major else (M, n_heads, head_dim)
    kvs = (n_kv_heads, M, head_dim) if head_major else (M, n_kv_heads, head_dim)
    if q is None:
        q = torch.empty(qs, dtype=odt, device=dev)
    if k is None:
        k = torch.empty(kvs, dtype=odt, device=dev)
    if v is None:
        v = torch.empty(kvs, dtype=odt, device=dev)
    for t, shape, name in ((q, qs, "q"), (k, kvs, "k"), (v, kvs, "v")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if h_out is None and write_h:
        h_out = torch.empty_like(x)
    stream = _stream(dev)
    need = int(lib.fp_workspace_bytes(M, K, Nw, _DT[act], wcode))
    ws = workspace if workspace is not None else _workspace(dev, stream, need)
    fn = lib.fused_add_norm_qkv_hm if head_major else lib.fused_add_norm_qkv
    st = fn(
        _ptr(x, "x", dev, act), _ptr(residual, "residual", dev, act), _ptr(h_out, "h_out", dev, act),
        _ptr(gamma, "gamma", dev, act), _ptr(beta, "beta", dev, act), FP_NORM[norm], float(eps),
        _ptr(w_qkv, "w_qkv", dev), _ptr(w_scale, "w_scale", dev, _scale_dtype(w_qkv)),
        _ptr(bias, "bias", dev, act), _ptr(q, "q", dev, odt), _ptr(k, "k", dev, odt),
        _ptr(v, "v", dev, odt), M, K, n_heads, n_kv_heads, head_dim,
        _DT[act], wcode, _DT[odt],
        None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), stream)
    _check("fused_add_norm_qkv", st)
    return q, k, v, h_out


NOALLOC_SCRATCH_BYTES = 16 << 20     # FP_NOALLOC_SCRATCH_BYTES of include/fusedproj.h


def fused_add_norm_qkv_noalloc(x: torch.Tensor, residual: Optional[torch.Tensor], gamma: Optional[torch.Tensor],
                               w_qkv: torch.Tensor | PackedWeight, n_heads: int, n_kv_heads: int, head_dim: int, *,
                               q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               h_out: Optional[torch.Tensor] = None, beta: Optional[torch.Tensor] = None,
                               norm: str = "rms", eps: float = 1e-5, w_scale: Optional[torch.Tensor] = None,
                               bias: Optional[torch.Tensor] = None):
    """fused_add_norm_qkv_noalloc: the QKV call with the library's static device
    scratch instead of a workspace.  The caller passes every output (q, k, v
    token-major, h_out or None) so that nothing is allocated here either."""
    lib = _lib.load()
    _ptr(x, "x")
    dev = x.device
    M, K = x.shape
    act = x.dtype
    odt = q.dtype
    w_qkv, wcode = _wcode(w_qkv)
    Nw = (n_heads + 2 * n_kv_heads) * head_dim
    _check_weight(w_qkv, w_scale, Nw, K, "w_qkv")
    for t, shape, name in ((q, (M, n_heads, head_dim), "q"), (k, (M, n_kv_heads, head_dim), "k"),
                           (v, (M, n_kv_heads, head_dim), "v")):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    st = lib.fused_add_norm_qkv_noalloc(
        _ptr(x, "x", dev, act), _ptr(residual, "residual", dev, act), _ptr(h_out, "h_out", dev, act),
        _ptr(gamma, "gamma", dev, act), _ptr(beta, "beta", dev, act), FP_NORM[norm], float(eps),
        _ptr(w_qkv, "w_qkv", dev), _ptr(w_scale, "w_scale", dev, _scale_dtype(w_qkv)),
        _ptr(bias, "bias", dev, act), _ptr(q, "q", dev, odt), _ptr(k, "k", dev, odt),
        _ptr(v, "v", dev, odt), M, K, n_heads, n_kv_heads, head_dim,
        _DT[act], wcode, _DT[odt], _stream(dev))
    _check("fused_add_norm_qkv_noalloc", st)
    return q, k, v, h_out


def fused_gateup_act(x: torch.Tensor, residual: Optional[torch.Tensor], gamma: Optional[torch.Tensor],
                     w: torch.Tensor | PackedWeight, ffn: int, act: str = "swiglu", *,
                     beta: Optional[torch.Tensor] = None, norm: str = "rms", eps: float = 1e-5,
                     w_scale: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                     out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                     h_out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(residual add + norm ->) gate/up or up projection (+bias) -> activation; returns out [M, ffn]."""
    lib = _lib.load()
    _ptr(x, "x")
    dev = x.device
    M, K = x.shape
    adt = x.dtype
    odt = out_dtype or adt
    w, wcode = _wcode(w)
    Nw = 2 * ffn if act == "swiglu" else ffn
    _check_weight(w, w_scale, Nw, K, "w")
    if out is None:
        out = torch.empty((M, ffn), dtype=odt, device=dev)
    stream = _stream(dev)
    need = int(lib.fp_workspace_bytes(M, K, Nw, _DT[adt], wcode))
    ws = workspace if workspace is not None else _workspace(dev, stream, need)
    st = lib.fused_gateup_act(
        _ptr(x, "x", dev, adt), _ptr(residual, "residual", dev, adt), _ptr(h_out, "h_out", dev, adt),
        _ptr(gamma, "gamma", dev, adt), _ptr(beta, "beta", dev, adt), FP_NORM[norm], float(eps),
        _ptr(w, "w", dev), _ptr(w_scale, "w_scale", dev, _scale_dtype(w)), _ptr(bias, "bias", dev, adt),
        _ptr(out, "out", dev, odt), M, K, ffn, FP_ACT[act], _DT[adt], wcode, _DT[odt],
        None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), stream)
    _check("fused_gateup_act", st)
    return out


def fused_down_residual(a: torch.Tensor, w: torch.Tensor | PackedWeight, residual: Optional[torch.Tensor] = None, *,
                        w_scale: Optional[torch.Tensor] = None, bias: Optional[torch.Tensor] = None,
                        out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Down projection plus residual: out = residual + bias + a @ w^T; returns out [M, hidden].
    ``out`` may be ``residual`` itself (updated in place) when the dtypes match."""
    lib = _lib.load()
    _ptr(a, "a")
    dev = a.device
    M, F = a.shape
    adt = a.dtype
    odt = out_dtype or adt
    w, wcode = _wcode(w)
    Nw = w.shape[0]
    _check_weight(w, w_scale, Nw, F, "w")
    if out is None:
        out = torch.empty((M, Nw), dtype=odt, device=dev)
    stream = _stream(dev)
    need = int(lib.fp_down_workspace_bytes(M, F, Nw, _DT[adt], wcode))
    ws = workspace if workspace is not None else _workspace(dev, stream, need)
    st = lib.fused_down_residual(
        _ptr(a, "a", dev, adt), _ptr(w, "w", dev), _ptr(w_scale, "w_scale", dev, _scale_dtype(w)),
        _ptr(bias, "bias", dev, adt), _ptr(residual, "residual", dev, adt), _ptr(out, "out", dev, odt),
        M, F, Nw, _DT[adt], wcode, _DT[odt],
        None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), stream)
    _check("fused_down_residual", st)
    return out


def fused_dequant_i8_bf16(q: torch.Tensor, scale: torch.Tensor,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    lib = _lib.load()
    _ptr(q, "q")
    dev = q.device
    N, K = q.shape
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    st = lib.fused_dequant_i8_bf16(_ptr(q, "q", dev, torch.int8), _ptr(scale, "scale", dev, torch.float32),
                                   _ptr(out, "out", dev, torch.bfloat16), N, K, _stream(dev))
    _check("fused_dequant_i8_bf16", st)
    return out


def fused_dequant_i4_bf16(q: torch.Tensor, scale: torch.Tensor,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int4 weights q [N, K/2] (uint8, two per byte) with scales [N, K/128] -> bf16 [N, K]."""
    lib = _lib.load()
    _ptr(q, "q")
    dev = q.device
    N, K = q.shape[0], 2 * q.shape[1]
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    st = lib.fused_dequant_i4_bf16(_ptr(q, "q", dev, torch.uint8), _ptr(scale, "scale", dev, torch.float32),
                                   _ptr(out, "out", dev, torch.bfloat16), N, K, _stream(dev))
    _check("fused_dequant_i4_bf16", st)
    return out


def fused_dequant_mxfp4_bf16(q: torch.Tensor, scale: torch.Tensor,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """MXFP4 weights q [N, K/2] (float4_e2m1fn_x2, two codes per byte) with E8M0
    block scales [N, K/32] (float8_e8m0fnu) -> bf16 [N, K]."""
    lib = _lib.load()
    _ptr(q, "q")
    dev = q.device
    N, K = q.shape[0], 2 * q.shape[1]
    if out is None:
        out = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    st = lib.fused_dequant_mxfp4_bf16(_ptr(q, "q", dev, torch.float4_e2m1fn_x2),
                                      _ptr(scale, "scale", dev, torch.float8_e8m0fnu),
                                      _ptr(out, "out", dev, torch.bfloat16), N, K, _stream(dev))
    _check("fused_dequant_mxfp4_bf16", st)
    return out


def profile_start():
    _check("fp_profile_start", _lib.load().fp_profile_start())


def profile_stop() -> Dict[str, Tuple[int, float]]:
    """{kernel name: (launches, total ms)} for the kernels enqueued since profile_start()."""
    import ctypes
    lib = _lib.load()
    buf = (_lib.KernelTime * 64)()
    n = ctypes.c_int(0)
    _check("fp_profile_stop", lib.fp_profile_stop(buf, 64, ctypes.byref(n)))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n.value, 64))}


_FAMILY = {None: -1, "tiled": 0, "stream": 1, "prefill": 2, "gemm16": 4}


def tune_install(entries) -> None:
    """Install a launch-configuration table (fp_tune_install; replaces the
    previous one).  Each entry is a dict with m_lo, m_hi, hidden, n_cols,
    act_dtype, w_dtype (torch dtypes) and swiglu (bool), and optionally family
    ("tiled", "stream", "prefill", "gemm16" or None for the planner's), rows, grid and
    splits (0 for the planner's).  See fusion_residual_add_amd.tune for the
    micro-benchmark that produces such tables."""
    entries = list(entries)
    arr = (_lib.TuneEntry * max(len(entries), 1))()
    for i, e in enumerate(entries):
        arr[i] = _lib.TuneEntry(int(e["m_lo"]), int(e["m_hi"]), int(e["hidden"]), int(e["n_cols"]),
                                _DT[e["act_dtype"]], _DT[e["w_dtype"]], int(bool(e["swiglu"])),
                                _FAMILY[e.get("family")], int(e.get("rows", 0)), int(e.get("grid", 0)),
                                int(e.get("splits", 0)))
    _check("fp_tune_install", _lib.load().fp_tune_install(arr, len(entries)))


def tune_clear() -> None:
    """Remove every tuning entry: the built-in planner decides again."""
    tune_install([])


def tune_count() -> int:
    return int(_lib.load().fp_tune_count())


_OVERRIDE_FIELDS = ("splits", "stream_nr", "stream_target", "no_stream", "no_prefill", "fp8_tile", "no_gemm16",
                    "gemm16_stages", "no_stream_rows", "stream_rows_expire")


def get_plan_override() -> dict:
    """The current plan overrides (fp_plan_override_get)."""
    o = _lib.PlanOverride()
    _check("fp_plan_override_get", _lib.load().fp_plan_override_get(o))
    return {k: int(getattr(o, k)) for k in _OVERRIDE_FIELDS}


def set_plan_override(values: Optional[dict]) -> None:
    """Replace the plan overrides (fp_plan_override_set): a dict with any of
    splits, stream_nr, stream_target, no_stream, no_prefill, fp8_tile, no_gemm16, gemm16_stages,
    no_stream_rows, stream_rows_expire (missing
    fields 0 = the planner's choice); None restores the values the FUSEDPROJ_*
    environment variables held when the library first planned a call."""
    import ctypes
    lib = _lib.load()
    if values is None:
        _check("fp_plan_override_set", lib.fp_plan_override_set(None))
        return
    unknown = set(values) - set(_OVERRIDE_FIELDS)
    if unknown:
        raise ValueError(f"unknown plan override fields {sorted(unknown)}")
    o = _lib.PlanOverride(*(int(values.get(k, 0)) for k in _OVERRIDE_FIELDS))
    _check("fp_plan_override_set", lib.fp_plan_override_set(ctypes.byref(o)))


class plan_override:
    """Context manager: ``with plan_override(splits=3, no_stream=1): ...``
    forces those launch choices on every call inside, then restores the
    previous overrides."""

    def __init__(self, **values):
        self.values = values
        self.prev = None

    def __enter__(self):
        self.prev = get_plan_override()
        set_plan_override(self.values)
        return self

    def __exit__(self, *exc):
        set_plan_override(self.prev)
        return False
