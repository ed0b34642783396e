"""The C ABI on a machine without a GPU: the library loads, exports every symbol
the header declares, sizes workspaces, and rejects bad arguments before any
HIP call (so these calls never touch memory; the pointers below are fake)."""
import ctypes
import os
import re

import pytest
import torch

import fusion_residual_add_amd as fra
from fusion_residual_add_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fusedproj.h")

FAKE = 0x10000           # 16-byte aligned, never dereferenced
F32, F16, BF16, I8, I4, E4M3 = 0, 1, 2, 3, 4, 5


def lib():
    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    L = lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    L = lib()
    for s in range(len(_lib.STATUS)):
        assert L.fp_status_str(s)
    assert L.fp_status_str(99) == b"unknown status"


def test_workspace_bytes():
    L = lib()
    assert L.fp_workspace_bytes(0, 4096, 6144, BF16, BF16) == 0
    assert L.fp_workspace_bytes(32, 4095, 6144, BF16, BF16) == 0      # hidden not multiple of 64
    assert L.fp_workspace_bytes(32, 4096, 6144, F16, I8) == 0         # int8 needs bf16 activations
    dec = L.fp_workspace_bytes(32, 4096, 6144, BF16, BF16)
    assert dec >= 32 * 8 and dec % 256 == 0
    big = L.fp_workspace_bytes(16384, 4096, 12288, BF16, BF16)
    assert big >= 16384 * 8


def qkv(**kw):
    a = dict(x=FAKE, residual=FAKE + 0x1000000, h_out=None, gamma=FAKE + 0x2000000, beta=None,
             norm=1, eps=1e-5, w=FAKE + 0x3000000, w_scale=None, bias=None,
             q=FAKE + 0x40000000, k=FAKE + 0x50000000, v=FAKE + 0x60000000, M=0, hidden=4096,
             H=32, Hkv=8, D=128, act=BF16, wdt=BF16, odt=BF16, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    fn = lib().fused_add_norm_qkv_hm if a.pop("head_major", False) else lib().fused_add_norm_qkv
    st = fn(a["x"], a["residual"], a["h_out"], a["gamma"], a["beta"], a["norm"],
                                  a["eps"], a["w"], a["w_scale"], a["bias"], a["q"], a["k"], a["v"],
                                  a["M"], a["hidden"], a["H"], a["Hkv"], a["D"], a["act"], a["wdt"],
                                  a["odt"], a["ws"], a["ws_bytes"], a["stream"])
    return _lib.STATUS[st], lib().fp_last_error().decode()


def gu(**kw):
    a = dict(x=FAKE, residual=None, h_out=None, gamma=FAKE + 0x2000000, beta=None, norm=1, eps=1e-5,
             w=FAKE + 0x3000000, w_scale=None, bias=None, out=FAKE + 0x40000000, M=0, hidden=4096,
             ffn=14336, act=1, adt=BF16, wdt=BF16, odt=BF16, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    st = lib().fused_gateup_act(a["x"], a["residual"], a["h_out"], a["gamma"], a["beta"], a["norm"],
                                a["eps"], a["w"], a["w_scale"], a["bias"], a["out"], a["M"], a["hidden"],
                                a["ffn"], a["act"], a["adt"], a["wdt"], a["odt"], a["ws"], a["ws_bytes"],
                                a["stream"])
    return _lib.STATUS[st], lib().fp_last_error().decode()


def test_m_zero_is_a_noop():
    assert qkv(M=0)[0] == "FP_OK"
    assert qkv(M=0, head_major=True)[0] == "FP_OK"
    assert gu(M=0)[0] == "FP_OK"


@pytest.mark.parametrize("kw,status", [
    (dict(M=1, x=None), "FP_E_NULL"),
    (dict(w=None), "FP_E_NULL"),
    (dict(gamma=None), "FP_E_NULL"),
    (dict(M=1, q=None), "FP_E_NULL"),
    (dict(wdt=I8), "FP_E_NULL"),                       # int8 without scales
    (dict(wdt=I4), "FP_E_NULL"),                       # int4 without scales
    (dict(wdt=I4, hidden=320, w_scale=FAKE + 0x70000000), "FP_E_SHAPE"),   # int4: hidden % 128
    (dict(act=F16, wdt=I4, w_scale=FAKE + 0x70000000), "FP_E_DTYPE"),
    (dict(wdt=E4M3), "FP_E_NULL"),                     # E4M3 without scales
    (dict(wdt=E4M3, hidden=320, w_scale=FAKE + 0x70000000), "FP_E_SHAPE"),   # E4M3: hidden % 128
    (dict(act=F32, odt=F32, wdt=E4M3, w_scale=FAKE + 0x70000000), "FP_E_DTYPE"),   # fp32 activations
    (dict(M=-1), "FP_E_SHAPE"),
    (dict(hidden=4000), "FP_E_SHAPE"),
    (dict(hidden=0), "FP_E_SHAPE"),
    (dict(H=30, Hkv=8), "FP_E_SHAPE"),
    (dict(Hkv=0), "FP_E_SHAPE"),
    (dict(D=100), "FP_E_SHAPE"),
    (dict(act=I8), "FP_E_DTYPE"),
    (dict(act=F16, wdt=BF16), "FP_E_DTYPE"),
    (dict(act=F16, wdt=I8, w_scale=FAKE + 0x70000000), "FP_E_DTYPE"),
    (dict(odt=F16), "FP_E_DTYPE"),
    (dict(norm=7), "FP_E_ARG"),
    (dict(eps=-1.0), "FP_E_ARG"),
    (dict(x=FAKE + 8), "FP_E_ALIGN"),
    (dict(q=FAKE + 0x40000004), "FP_E_ALIGN"),
    (dict(M=32, ws=None), "FP_E_WORKSPACE"),
    (dict(M=32, ws=FAKE + 0x7000000, ws_bytes=16), "FP_E_WORKSPACE"),
    (dict(M=32, ws=FAKE + 0x7000000, ws_bytes=1 << 30, q=FAKE + 0x3000000), "FP_E_ALIAS"),   # q over w
    (dict(M=32, ws=FAKE + 0x7000000, ws_bytes=1 << 30, k=FAKE + 0x40000000), "FP_E_ALIAS"),  # k over q
    (dict(M=32, ws=FAKE + 0x7000000, ws_bytes=1 << 30, h_out=FAKE + 0x1000000), "FP_E_ALIAS"),  # in place
    (dict(M=32, ws=FAKE + 0x40000000, ws_bytes=1 << 30), "FP_E_ALIAS"),  # workspace over q
])
def test_qkv_rejects(kw, status):
    got, msg = qkv(**kw)
    assert got == status, msg
    assert msg
    # the head-major entry point validates alike (same sizes, same ranges)
    got_hm, _ = qkv(head_major=True, **kw)
    assert got_hm == status


@pytest.mark.parametrize("kw,status", [
    (dict(M=1, out=None), "FP_E_NULL"),
    (dict(ffn=1000), "FP_E_SHAPE"),
    (dict(ffn=0), "FP_E_SHAPE"),
    (dict(act=9), "FP_E_ARG"),
    (dict(adt=F32, wdt=F16), "FP_E_DTYPE"),
    (dict(out=FAKE + 0x40000002), "FP_E_ALIGN"),
    (dict(M=4, ws=FAKE + 0x7000000, ws_bytes=1 << 30, out=FAKE + 0x2000000 - 64), "FP_E_ALIAS"),  # over gamma
])
def test_gateup_rejects(kw, status):
    got, msg = gu(**kw)
    assert got == status, msg


def test_dequant_rejects():
    L = lib()
    assert _lib.STATUS[L.fused_dequant_i8_bf16(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 0, 64, None)] == "FP_OK"
    assert _lib.STATUS[L.fused_dequant_i8_bf16(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 4, 60, None)] == "FP_E_SHAPE"
    assert _lib.STATUS[L.fused_dequant_i8_bf16(None, FAKE + 0x1000000, FAKE + 0x2000000, 4, 64, None)] == "FP_E_NULL"
    assert _lib.STATUS[L.fused_dequant_i8_bf16(FAKE, FAKE + 0x1000000, FAKE + 0x80, 4, 64, None)] == "FP_E_ALIAS"


def test_dequant_i4_rejects():
    L = lib()
    f = L.fused_dequant_i4_bf16
    assert _lib.STATUS[f(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 0, 128, None)] == "FP_OK"
    assert _lib.STATUS[f(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 4, 192, None)] == "FP_E_SHAPE"
    assert _lib.STATUS[f(FAKE, None, FAKE + 0x2000000, 4, 128, None)] == "FP_E_NULL"
    assert _lib.STATUS[f(FAKE, FAKE + 0x1000000, FAKE + 0x8, 4, 128, None)] == "FP_E_ALIGN"
    # the [4, 128] bf16 output (1 KB) over the packed weight ([4, 64] bytes)
    assert _lib.STATUS[f(FAKE, FAKE + 0x1000000, FAKE - 0x100, 4, 128, None)] == "FP_E_ALIAS"


def test_int4_plans():
    for var in _ENV:
        os.environ.pop(var, None)
    u8 = torch.uint8
    # decode token counts, hidden a multiple of 256: streamed, dequantised in registers
    p = _plan(16, 8192, 57344, w=u8, fn="swiglu")
    assert p["kernel"] == "stream_kernel<bf16-i4w,m16,n128,k256,swiglu>" and "prep" not in p
    assert _plan(64, 8192, 57344, w=u8, fn="swiglu")["kernel"] == "stream_kernel<bf16-i4w,m64,n256,k128,swiglu>"
    # more than 64 tokens: the 128 x 512 kernel, dequantised in registers too
    p = _plan(256, 8192, 57344, w=u8, fn="swiglu")
    assert p["family"] == "prefill" and p["kernel"] == "prefill_kernel<bf16-i4w,128x512,swiglu>"
    assert "prep" not in p and p["workspace"] < 57344 * 8192
    # the tiled kernel: dequantised into the workspace, then the bf16 kernel
    p = _plan(8, 384, 512, w=u8)
    assert p["family"] == "tiled" and p["prep"] == "dequant_i4_kernel"
    assert fra.workspace_bytes(8, 384, 512, torch.bfloat16, u8) >= 512 * 384 * 2
    assert fra.workspace_bytes(16, 8192, 57344, torch.bfloat16, u8) < 57344 * 8192


def test_fp8_plans():
    for var in _ENV:
        os.environ.pop(var, None)
    e = torch.float8_e4m3fn
    # one family at every token count: per-token quantisation, then the FP8 GEMM
    p = _plan(32, 4096, 28672, w=e, fn="swiglu")
    assert p["family"] == "fp8" and p["prep"] == "quant8_kernel<bf16>"
    assert p["kernel"] == "gemm8_kernel<bf16,32x256,swiglu>"
    assert p["splits"] == 2 and p["grid"] == 112 * 2          # 112 tiles of 128 gate + 128 up rows, split in two
    assert _plan(64, 4096, 28672, w=e, fn="swiglu")["kernel"] == "gemm8_kernel<bf16,64x256,swiglu>"
    p = _plan(1, 4096, 6144, w=e)
    assert p["splits"] == 4 and p["grid"] == 24 * 4            # each split streams 256 KB of weights
    p = _plan(200, 4096, 6144, w=e)
    assert p["kernel"] == "gemm8_kernel<bf16,128x128,linear>" and p["splits"] == 5 and p["grid"] == 2 * 48 * 5
    # enough 256 x 256 tiles for a round of CUs: the large tiles, unsplit
    p = _plan(16384, 4096, 22016, w=e, fn="swiglu")
    assert p["kernel"] == "gemm8_kernel<bf16,256x256,swiglu>" and p["splits"] == 1 and p["grid"] == 64 * 86
    assert _plan(16384, 4096, 12288, w=e)["grid"] == 64 * 48
    p = _plan(100, 512, 512, act=torch.float16, w=e, fn="gelu_tanh")
    assert p["kernel"] == "gemm8_kernel<f16,128x128,gelu>"
    # the workspace holds the codes and row scales (and the partials when split)
    assert fra.workspace_bytes(16384, 4096, 22016, torch.bfloat16, e) >= 16384 * 4096 + 16384 * 4
    assert fra.workspace_bytes(32, 4096, 28672, torch.bfloat16, e) >= 112 * 2 * 32 * 256 * 4
    assert fra.workspace_bytes(8, 320, 512, torch.bfloat16, e) == 0      # hidden % 128
    os.environ["FUSEDPROJ_SPLITS"] = "3"
    os.environ["FUSEDPROJ_FP8_TILE"] = "128"
    try:
        p = _plan(1, 4096, 6144, w=e)
        assert p["splits"] == 3 and p["kernel"] == "gemm8_kernel<bf16,128x128,linear>"
        os.environ["FUSEDPROJ_FP8_TILE"] = "256"
        assert _plan(1, 4096, 6144, w=e)["splits"] == 1      # the 256 x 256 kernel does not split K
    finally:
        os.environ.pop("FUSEDPROJ_SPLITS")
        os.environ.pop("FUSEDPROJ_FP8_TILE")


def test_binding_refuses_cpu_tensors():
    import torch
    import fusion_residual_add_amd as fra
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fra.fused_gateup_act(x, None, torch.ones(64, dtype=torch.bfloat16),
                             torch.zeros(32, 64, dtype=torch.bfloat16), 16, "swiglu")


# ---------------------------------------------------------------------------
# kernel routing (host logic, no device): which family each shape takes
# ---------------------------------------------------------------------------
def _plan(M, K, N, act=torch.bfloat16, w=torch.bfloat16, fn="none"):
    return fra.describe_plan(M, K, N, act, w, fn)


def test_plan_routing_families(monkeypatch):
    for var in ("FUSEDPROJ_SPLITS", "FUSEDPROJ_NO_STREAM", "FUSEDPROJ_NO_PREFILL", "FUSEDPROJ_STREAM_NR",
                "FUSEDPROJ_STREAM_TARGET"):
        monkeypatch.delenv(var, raising=False)
    # decode token counts with K a multiple of 256: the weight-streaming kernel
    p = _plan(32, 4096, 2 * 14336, fn="swiglu")
    assert p["family"] == "stream" and p["kernel"] == "stream_kernel<bf16,m32,n128,k256,swiglu>"
    # 224 tiles of a 235 MB weight: one whole tile per workgroup, nothing shared
    assert p["grid"] == 224 and p["slots"] == 1
    # the same tile count on a 470 MB weight: stream-K over 256 workgroups
    p = _plan(64, 8192, 57344, w=torch.int8, fn="swiglu")
    assert p["grid"] == 256 and p["slots"] >= 2
    # 16-bit QKV weights at up to 32 tokens: 64-row tiles (96 of them), stream-K
    # over 256 workgroups
    p = _plan(32, 4096, 6144)
    assert p["kernel"] == "stream_kernel<bf16,m32,n64,k256,linear>" and p["grid"] == 256 and p["slots"] >= 2
    # 33..64 tokens keep 128-row tiles
    assert _plan(64, 4096, 6144)["kernel"] == "stream_kernel<bf16,m64,n128,k128,linear>"
    # Llama-2-70B's 8-way shard: QKV (10 tiles x 32 chunks) on 160 workgroups of
    # 2 chunks; gate/up (56 tiles x 32 chunks) 4 workgroups per tile, 8 chunks each
    p = _plan(1, 8192, 1280, w=torch.int8)
    assert p["grid"] == 160 and p["slots"] == 16
    p = _plan(1, 8192, 7168, w=torch.int8, fn="swiglu")
    assert p["grid"] == 224 and p["slots"] == 4
    assert _plan(1, 8192, 10240, w=torch.int8)["kernel"] == "stream_kernel<bf16-i8w,m16,n128,k256,linear>"
    # 33..64 tokens: 128-wide chunks; int8 large-N gate/up: 256 rows per workgroup
    assert _plan(64, 8192, 57344, w=torch.int8, fn="swiglu")["kernel"] == "stream_kernel<bf16-i8w,m64,n256,k128,swiglu>"
    assert _plan(64, 8192, 10240, w=torch.int8)["kernel"] == "stream_kernel<bf16-i8w,m64,n128,k128,linear>"
    # K not a multiple of 256 at decode sizes, and every fp32 call: the tiled kernel
    assert _plan(32, 320, 512)["family"] == "tiled"
    assert _plan(4, 256, 512, act=torch.float32, w=torch.float32)["family"] == "tiled"
    # more than 64 tokens: the 128 x 512 kernel
    p = _plan(16384, 4096, 12288)
    assert p["family"] == "prefill" and p["kernel"] == "prefill_kernel<bf16,128x512,linear>"
    assert p["grid"] == 128 * 24 and p["splits"] == 1
    # split K so that the workgroups fill one round of CUs: 40 tiles -> 6 splits
    # (240 workgroups); 224 tiles -> unsplit (2 splits would take two rounds)
    p = _plan(256, 8192, 10240, w=torch.int8)
    assert p["family"] == "prefill" and p["splits"] == 6 and p["grid"] == 240
    p = _plan(256, 8192, 57344, w=torch.int8, fn="swiglu")
    assert p["splits"] == 1 and p["grid"] == 224
    assert _plan(2048, 4096, 16384, act=torch.float16, w=torch.float16, fn="gelu_tanh")["kernel"] == \
        "prefill_kernel<f16,128x512,gelu>"
    # past 4 GiB of activations or of weights the 128 x 512 kernel's 32-bit
    # buffer offsets do not reach: the tiled kernel; decode counts stream any size
    m_big = (1 << 32) // (2 * 4096) + 64
    assert _plan(m_big, 4096, 256)["family"] == "tiled"
    assert _plan(m_big - 128, 4096, 256)["family"] == "prefill"
    f_big = (1 << 32) // (2 * 2 * 8192) + 32
    assert _plan(96, 8192, 2 * f_big, fn="swiglu")["family"] == "tiled"
    assert _plan(96, 8192, 2 * f_big - 128, fn="swiglu")["family"] == "prefill"
    assert _plan(8, 8192, 2 * f_big, fn="swiglu")["family"] == "stream"


def test_plan_grid_slots_consistent(monkeypatch):
    """The stream kernel's partial-sum slots cover the most workgroups that share
    one tile, for unit counts that do and do not divide evenly."""
    monkeypatch.delenv("FUSEDPROJ_STREAM_TARGET", raising=False)
    for splits in ("1", "2", "3", "5", "7"):
        monkeypatch.setenv("FUSEDPROJ_SPLITS", splits)
        for M, K, N in ((1, 2048, 640), (32, 4096, 6144), (20, 1024, 928)):
            p = _plan(M, K, N)
            tiles = -(-N // 64)               # 64-row tiles: 16-bit weights, no pairing, <= 32 tokens
            chunks = K // 256
            units = tiles * chunks
            G = min(tiles * int(splits), units)
            assert p["grid"] == G
            owner = lambda v: ((v + 1) * G - 1) // units
            most = max(owner(t * chunks + chunks - 1) - owner(t * chunks) + 1 for t in range(tiles))
            assert p["slots"] == most


def test_plan_env_overrides(monkeypatch):
    monkeypatch.setenv("FUSEDPROJ_NO_STREAM", "1")
    assert _plan(32, 4096, 6144)["family"] == "tiled"
    monkeypatch.delenv("FUSEDPROJ_NO_STREAM")
    monkeypatch.setenv("FUSEDPROJ_NO_PREFILL", "1")
    assert _plan(300, 4096, 6144)["family"] == "tiled"


def test_plan_rejects():
    with pytest.raises(fra.FusedProjError):
        _plan(32, 4000, 6144)                  # hidden not a multiple of 64
    with pytest.raises(fra.FusedProjError):
        _plan(32, 4096, 6144, act=torch.float16, w=torch.int8)


_ENV = ("FUSEDPROJ_SPLITS", "FUSEDPROJ_NO_STREAM", "FUSEDPROJ_NO_PREFILL", "FUSEDPROJ_STREAM_NR",
        "FUSEDPROJ_STREAM_TARGET", "FUSEDPROJ_FP8_TILE")


def _entry(**kw):
    e = dict(m_lo=17, m_hi=32, hidden=4096, n_cols=6144, act_dtype=torch.bfloat16,
             w_dtype=torch.bfloat16, swiglu=False)
    e.update(kw)
    return e


def test_tuning_table_overrides_matching_calls(monkeypatch):
    for var in _ENV:
        monkeypatch.delenv(var, raising=False)
    base, base_gu, base_33 = _plan(32, 4096, 6144), _plan(32, 4096, 6144, fn="swiglu"), _plan(33, 4096, 6144)
    try:
        fra.tune_install([_entry(family="stream", rows=128, grid=192)])
        assert fra.tune_count() == 1
        p = _plan(32, 4096, 6144)
        assert p["kernel"] == "stream_kernel<bf16,m32,n128,k256,linear>" and p["grid"] == 192
        assert _plan(17, 4096, 6144)["grid"] == 192
        # other token counts, the gate/up pairing and other sizes keep the planner's choice
        assert _plan(33, 4096, 6144) == base_33
        assert _plan(32, 4096, 6144, fn="swiglu") == base_gu
        assert _plan(32, 4096, 6400) == fra.describe_plan(32, 4096, 6400, torch.bfloat16, torch.bfloat16)
        # the workspace query reads the same table
        assert fra.workspace_bytes(32, 4096, 6144, torch.bfloat16, torch.bfloat16) >= p["workspace"]
        # any family that can take the call, with its split
        fra.tune_install([_entry(family="tiled", splits=3)])
        p = _plan(32, 4096, 6144)
        assert p["family"] == "tiled" and p["splits"] == 3
        fra.tune_install([_entry(family="prefill", splits=2)])
        p = _plan(32, 4096, 6144)
        assert p["family"] == "prefill" and p["splits"] == 2 and p["grid"] == 12 * 2
        # a family that cannot take the call is ignored (fp32 activations stream nowhere)
        fra.tune_install([_entry(family="stream", act_dtype=torch.float32, w_dtype=torch.float32)])
        assert _plan(32, 4096, 6144, act=torch.float32, w=torch.float32)["family"] == "tiled"
        # 64 rows per workgroup only where that form exists: ignored for the gate/up pairing
        fra.tune_install([_entry(rows=64, swiglu=True)])
        assert _plan(32, 4096, 6144, fn="swiglu") == base_gu
        fra.tune_install([_entry(rows=128)])
        assert _plan(32, 4096, 6144)["kernel"] == "stream_kernel<bf16,m32,n128,k256,linear>"
        # the first matching entry wins; the environment overrides win over the table
        fra.tune_install([_entry(grid=128), _entry(grid=64)])
        assert _plan(32, 4096, 6144)["grid"] == 128
        fra.tune_install([_entry(family="stream")])
        monkeypatch.setenv("FUSEDPROJ_NO_STREAM", "1")
        assert _plan(32, 4096, 6144)["family"] == "tiled"
        monkeypatch.delenv("FUSEDPROJ_NO_STREAM")
        fra.tune_clear()
        assert fra.tune_count() == 0 and _plan(32, 4096, 6144) == base
    finally:
        fra.tune_clear()


@pytest.mark.parametrize("bad", [dict(rows=96), dict(m_lo=40, m_hi=8), dict(family=3), dict(splits=65),
                                 dict(grid=-1), dict(hidden=0), dict(act_dtype=torch.float16, w_dtype=torch.int8)],
                         ids=lambda b: ",".join(f"{k}={v}" for k, v in b.items()))
def test_tuning_table_rejects(bad):
    good = _entry(grid=200)
    try:
        fra.tune_install([good])
        e = dict(good)
        if "family" in bad and bad["family"] == 3:
            arr = (_lib.TuneEntry * 1)()
            arr[0] = _lib.TuneEntry(17, 32, 4096, 6144, BF16, BF16, 0, 3, 0, 0, 0)
            assert lib().fp_tune_install(arr, 1) == _lib.STATUS.index("FP_E_ARG")
        else:
            e.update(bad)
            with pytest.raises(fra.FusedProjError):
                fra.tune_install([good, e])
        # a rejected table leaves the installed one in place
        assert fra.tune_count() == 1 and _plan(32, 4096, 6144)["grid"] == 200
    finally:
        fra.tune_clear()


def test_tuning_table_json_round_trip(tmp_path):
    from fusion_residual_add_amd import tune
    entries = [_entry(family="stream", rows=256, grid=240, w_dtype=torch.uint8, hidden=8192, n_cols=10240),
               _entry(family="tiled", splits=4, act_dtype=torch.float32, w_dtype=torch.float32),
               _entry(rows=256, w_dtype=torch.int8), _entry(splits=3, w_dtype=torch.float8_e4m3fn)]
    path = str(tmp_path / "table.json")
    tune.save(entries, path)
    back = tune.load(path)
    assert back == entries
    try:
        fra.tune_install(back)
        assert fra.tune_count() == 4
        p = _plan(20, 8192, 10240, w=torch.uint8)
        assert p["kernel"] == "stream_kernel<bf16-i4w,m32,n256,k256,linear>" and p["grid"] == 240
    finally:
        fra.tune_clear()


def test_tuner_candidates_fp8_splits():
    from fusion_residual_add_amd import tune
    c = tune.candidates(32, 4096, 28672, torch.bfloat16, torch.float8_e4m3fn, True)
    assert {x["plan"]["family"] for x in c} == {"fp8"}
    assert sorted(x["plan"]["splits"] for x in c) == [1, 2, 3, 4, 6, 8]
    assert fra.tune_count() == 0


def test_tuner_candidates_cover_every_family():
    from fusion_residual_add_amd import tune
    for w in (torch.bfloat16, torch.int8, torch.uint8):
        fams = {c["plan"]["family"] for c in tune.candidates(16, 1024, 1024, torch.bfloat16, w, False)}
        assert fams == {"stream", "prefill", "tiled"}, (w, fams)
        kernels = {c["plan"]["kernel"] for c in tune.candidates(16, 1024, 1024, torch.bfloat16, w, False)}
        if w != torch.bfloat16:
            assert any(",n256," in k for k in kernels), kernels   # 256 rows per workgroup for int8 / int4
    assert fra.tune_count() == 0
