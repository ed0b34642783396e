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


def qkv_noalloc(**kw):
    a = dict(x=FAKE, residual=FAKE + 0x1000000, h_out=None, gamma=FAKE + 0x2000000, beta=None,
             norm=1, eps=1e-5, w=FAKE + 0x3000000, w_scale=None, bias=None,
             q=FAKE + 0x40000000, k=FAKE + 0x50000000, v=FAKE + 0x60000000, M=0, hidden=4096,
             H=32, Hkv=8, D=128, act=BF16, wdt=BF16, odt=BF16, stream=None)
    a.update(kw)
    st = lib().fused_add_norm_qkv_noalloc(a["x"], a["residual"], a["h_out"], a["gamma"], a["beta"], a["norm"],
                                          a["eps"], a["w"], a["w_scale"], a["bias"], a["q"], a["k"], a["v"],
                                          a["M"], a["hidden"], a["H"], a["Hkv"], a["D"], a["act"], a["wdt"],
                                          a["odt"], a["stream"])
    return _lib.STATUS[st], lib().fp_last_error().decode()


def test_noalloc_rejects_before_touching_the_device():
    """The allocation-free QKV call validates every argument, and the scratch
    it would need, before any HIP call (only error paths run here: a valid
    call would launch kernels on these fake addresses)."""
    assert qkv_noalloc(M=0)[0] == "FP_OK"
    # Llama-2-70B int8 QKV at 256 tokens needs 60 MiB of partial sums: more than the static scratch
    st, msg = qkv_noalloc(M=256, hidden=8192, H=64, Hkv=8, D=128, wdt=I8, w_scale=FAKE + 0x70000000)
    assert st == "FP_E_WORKSPACE" and "static scratch holds 16777216" in msg, msg
    assert fra.workspace_bytes(256, 8192, 10240, torch.bfloat16, torch.int8) > fra.NOALLOC_SCRATCH_BYTES
    assert qkv_noalloc(M=1, x=None)[0] == "FP_E_NULL"
    assert qkv_noalloc(M=32, hidden=4000)[0] == "FP_E_SHAPE"
    assert qkv_noalloc(M=32, D=100)[0] == "FP_E_SHAPE"
    assert qkv_noalloc(M=32, wdt=I8)[0] == "FP_E_NULL"                       # int8 without scales
    assert qkv_noalloc(M=32, act=F16, wdt=BF16)[0] == "FP_E_DTYPE"
    assert qkv_noalloc(M=32, q=FAKE + 0x3000000)[0] == "FP_E_ALIAS"         # q over the weight
    assert qkv_noalloc(M=32, x=FAKE + 8)[0] == "FP_E_ALIGN"
    # the header's limit is the binding's
    text = open(HEADER).read()
    assert "#define FP_NOALLOC_SCRATCH_BYTES (16u << 20)" in text and fra.NOALLOC_SCRATCH_BYTES == 16 << 20


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


def test_int4_plans(plan_override):
    plan_override()
    u8 = torch.uint8
    # decode token counts, hidden a multiple of 256: streamed, dequantised in
    # registers (the row pass forms the normalised rows)
    p = _plan(16, 8192, 57344, w=u8, fn="swiglu")
    assert p["kernel"] == "stream_kernel<bf16-i4w,m16,n128,k256,swiglu>" and p["prep"] == "norm_kernel<bf16>"
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


def test_mxfp4_plans_and_rejections(plan_override):
    plan_override()
    mx = torch.float4_e2m1fn_x2
    # decode token counts, hidden a multiple of 256: streamed, dequantised in registers
    p = _plan(16, 8192, 57344, w=mx, fn="swiglu")
    assert p["kernel"] == "stream_kernel<bf16-mxfp4w,m16,n128,k256,swiglu>" and p["prep"] == "norm_kernel<bf16>"
    assert _plan(64, 8192, 57344, w=mx, fn="swiglu")["kernel"] == "stream_kernel<bf16-mxfp4w,m64,n256,k128,swiglu>"
    # more than 64 tokens: the 128 x 512 kernel, any hidden that is a multiple of 64
    p = _plan(256, 8192, 10240, w=mx)
    assert p["kernel"] == "prefill_kernel<bf16-mxfp4w,128x512,linear>" and p["splits"] == 6
    assert _plan(300, 320, 512, w=mx)["kernel"] == "prefill_kernel<bf16-mxfp4w,128x512,linear>"
    # the tiled kernel: staged as bf16 in the workspace
    p = _plan(8, 320, 512, w=mx)
    assert p["family"] == "tiled" and p["prep"] == "dequant_mxfp4_kernel"
    assert fra.workspace_bytes(8, 320, 512, torch.bfloat16, mx) >= 512 * 320 * 2
    # MXFP4 weights take bf16 activations and need their scales
    assert qkv(M=4, wdt=6)[0] == "FP_E_NULL"
    assert qkv(M=4, act=F16, wdt=6, w_scale=FAKE + 0x70000000)[0] == "FP_E_DTYPE"
    # the E8M0 scales [N, K/32] are an input range: a q over them is an alias
    st, msg = qkv(M=4, wdt=6, w_scale=FAKE + 0x40000000 + 64, ws=FAKE + 0x7000000, ws_bytes=1 << 30)
    assert st == "FP_E_ALIAS" and "w_scale" in msg
    L = lib()
    assert _lib.STATUS[L.fused_dequant_mxfp4_bf16(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 4, 48, None)] == "FP_E_SHAPE"
    assert _lib.STATUS[L.fused_dequant_mxfp4_bf16(FAKE, None, FAKE + 0x2000000, 4, 64, None)] == "FP_E_NULL"
    assert _lib.STATUS[L.fused_dequant_mxfp4_bf16(FAKE, FAKE + 0x1000000, FAKE + 0x2000008, 4, 64, None)] == "FP_E_ALIGN"
    assert _lib.STATUS[L.fused_dequant_mxfp4_bf16(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, 0, 64, None)] == "FP_OK"


def test_fp8_plans(plan_override):
    plan_override()
    e = torch.float8_e4m3fn
    # one family at every token count: per-token quantisation, then a GEMM on the codes
    p = _plan(32, 4096, 28672, w=e, fn="swiglu")
    assert p["family"] == "fp8" and p["prep"] == "quant8_kernel<bf16>"
    assert p["kernel"] == "gemm8_kernel<bf16,32x256,swiglu>"
    assert p["splits"] == 2 and p["grid"] == 112 * 2          # 112 tiles of 128 gate + 128 up rows, split in two
    assert _plan(64, 4096, 28672, w=e, fn="swiglu")["kernel"] == "gemm8_kernel<bf16,64x256,swiglu>"
    p = _plan(1, 4096, 6144, w=e)
    assert p["splits"] == 4 and p["grid"] == 24 * 4            # each split streams 256 KB of weights
    assert fra.workspace_bytes(32, 4096, 28672, torch.bfloat16, e) >= 112 * 2 * 32 * 256 * 4
    # the weight-streaming kernel on the codes for tile-packed weights or
    # when requested (up to 64 tokens, hidden a multiple of the chunk), with
    # the weight rows per workgroup and grid of int8 weights (one byte per
    # weight as well)
    p = fra.describe_plan(32, 4096, 28672, torch.bfloat16, e, "swiglu", layout="packed_gate_up")
    assert p["kernel"] == "stream_kernel<bf16-e4m3,m32,n128,k256,swiglu>" and p["grid"] == 224, p
    p = fra.describe_plan(32, 4096, 6144, torch.bfloat16, e, layout="packed")
    assert p["kernel"] == "stream_kernel<bf16-e4m3,m32,n32,k512,linear>" and p["grid"] == 192, p
    assert p["slots"] == 1
    assert fra.describe_plan(200, 4096, 6144, torch.bfloat16, e, layout="packed")["kernel"].startswith("gemm8")
    with fra.plan_override(fp8_tile=32):
        assert fra.describe_plan(32, 4096, 6144, torch.bfloat16, e, layout="packed")["kernel"].startswith("gemm8")
    try:
        for M, N, sw in ((1, 6144, False), (32, 28672, True), (64, 6144, False), (64, 57344, True), (40, 768, False)):
            fn = "swiglu" if sw else "none"
            fra.tune_install([dict(m_lo=0, m_hi=64, hidden=K, n_cols=N, act_dtype=torch.bfloat16, w_dtype=e,
                                   swiglu=sw, family="stream") for K in (768, 4096)])
            a, b = _plan(M, 4096 if N != 768 else 768, N, w=e, fn=fn), _plan(M, 4096, N, w=torch.int8, fn=fn)
            assert a["family"] == "fp8" and a["kernel"].startswith("stream_kernel<bf16-e4m3,"), a
            # 32 (192 tiles of 6144 rows) or 64 weight rows per workgroup
            # without the gate/up pairing at up to 32 tokens (as 16-bit
            # weights), else int8's shapes
            if M <= 32 and not sw:
                assert (",n32,k512," if N == 6144 else ",n64,") in a["kernel"], a
            elif N != 768:
                # (the int8 call's kernel forms the rows itself; the E4M3
                # call's quantisation pass stays a launch of its own)
                assert a["kernel"].split(",", 1)[1] == b["kernel"].split(",", 1)[1].replace(",rows>", ">") and \
                    a["grid"] == b["grid"], (a, b)
        fra.tune_install([dict(m_lo=0, m_hi=64, hidden=4096, n_cols=6144, act_dtype=torch.float16, w_dtype=e,
                               swiglu=False, family="stream")])
        assert _plan(16, 4096, 6144, act=torch.float16, w=e)["kernel"] == "stream_kernel<f16-e4m3,m16,n32,k512,linear>"
        fra.tune_install([dict(m_lo=0, m_hi=64, hidden=K, n_cols=6144, act_dtype=torch.bfloat16, w_dtype=e,
                               swiglu=False, family="stream", rows=64) for K in (640, 4096)])
        # the codes, row scales and the partial sums of tiles shared by workgroups
        p = _plan(1, 4096, 6144, w=e)
        assert p["slots"] > 1 and p["workspace"] >= 4096 + 4 + 96 * p["slots"] * 16 * 64 * 4
        # hidden not a multiple of 256, or a tile requested: the FP8 GEMM tiles
        assert _plan(8, 640, 6144, w=e)["kernel"] == "gemm8_kernel<bf16,32x256,linear>"
        with fra.plan_override(fp8_tile=64):
            assert _plan(1, 4096, 6144, w=e)["kernel"] == "gemm8_kernel<bf16,64x256,linear>"
        with fra.plan_override(no_stream=1):
            assert _plan(1, 4096, 6144, w=e)["kernel"] == "gemm8_kernel<bf16,32x256,linear>"
    finally:
        fra.tune_clear()
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
    assert fra.workspace_bytes(8, 320, 512, torch.bfloat16, e) == 0      # hidden % 128
    with fra.plan_override(splits=3, fp8_tile=128):
        p = _plan(1, 4096, 6144, w=e)
        assert p["splits"] == 3 and p["kernel"] == "gemm8_kernel<bf16,128x128,linear>"
    with fra.plan_override(splits=3, fp8_tile=256):
        assert _plan(1, 4096, 6144, w=e)["splits"] == 1      # the 256 x 256 kernel does not split K


PK, PKGU = 0x100, 0x200     # FP_LAYOUT_PACKED, FP_LAYOUT_PACKED_GATE_UP


def test_packed_layout_rejects():
    # QKV of Llama-3-8B: 6144 rows, packable
    assert qkv(M=0, wdt=BF16 | PK)[0] == "FP_OK"
    assert qkv(M=32, wdt=BF16 | PK, ws=FAKE + 0x7000000, ws_bytes=1 << 30)[0] != "FP_E_SHAPE"
    assert qkv(wdt=BF16 | PKGU)[0] == "FP_E_SHAPE"           # the gate/up pairing is for the SwiGLU call
    assert qkv(wdt=BF16 | 0x400)[0] == "FP_E_DTYPE"          # unknown layout bits
    assert qkv(wdt=BF16 | PK | PKGU)[0] == "FP_E_DTYPE"
    assert qkv(act=F32, odt=F32, wdt=F32 | PK)[0] == "FP_E_DTYPE"
    assert qkv(H=5, Hkv=1, D=48, hidden=4096, wdt=BF16 | PK)[0] == "FP_E_SHAPE"   # 336 rows
    assert qkv(hidden=4096, wdt=I4 | PK)[0] == "FP_E_NULL"   # (scales checked first) int4 packs
    # SwiGLU: gate/up pairs of whole 64-row halves; plain packing also taken
    assert gu(wdt=BF16 | PKGU)[0] == "FP_OK"
    assert gu(wdt=BF16 | PK)[0] == "FP_OK"
    assert gu(ffn=14336 + 32, wdt=BF16 | PKGU)[0] == "FP_E_SHAPE"
    assert gu(act=2, ffn=1024, wdt=BF16 | PKGU)[0] == "FP_E_SHAPE"    # GELU: no pairing
    assert gu(act=2, ffn=1024, wdt=BF16 | PK)[0] == "FP_OK"
    assert gu(act=2, ffn=1040, wdt=BF16 | PK)[0] == "FP_E_SHAPE"      # 1040 rows
    L = lib()
    assert L.fp_workspace_bytes(32, 4096, 6144, BF16, BF16 | 0x400) == 0
    # the query covers both calls on that layout (plans may differ by layout)
    need = {lay: max(fra.describe_plan(32, 4096, 6144, torch.bfloat16, torch.bfloat16, fn, layout=lay)["workspace"]
                     for fn in ("none", "swiglu")) for lay in ("rows", "packed")}
    assert L.fp_workspace_bytes(32, 4096, 6144, BF16, BF16 | PK) == need["packed"]
    assert L.fp_workspace_bytes(32, 4096, 6144, BF16, BF16) == need["rows"]


def test_pack_weight_rejects():
    L = lib()
    f, g = L.fused_pack_weight, L.fused_unpack_weight
    S = lambda st: _lib.STATUS[st]
    for fn in (f, g):
        assert S(fn(FAKE, FAKE + 0x1000000, 0, 64, BF16, 0, None)) == "FP_OK"           # nothing to do
        assert S(fn(FAKE, FAKE + 0x1000000, 100, 64, BF16, 0, None)) == "FP_E_SHAPE"    # rows % 128
        assert S(fn(FAKE, FAKE + 0x1000000, 128, 16, BF16, 0, None)) == "FP_E_SHAPE"    # 32-byte rows
        assert S(fn(FAKE, FAKE + 0x1000000, 128, 64, I4, 0, None)) == "FP_E_SHAPE"      # 32-byte int4 rows
        assert S(fn(FAKE, FAKE + 0x1000000, 192, 64, BF16, 1, None)) == "FP_E_SHAPE"    # ffn 96
        assert S(fn(FAKE, FAKE + 0x1000000, 128, 64, F32, 0, None)) == "FP_E_DTYPE"
        assert S(fn(FAKE, FAKE + 0x1000000, 128, 64, BF16, 2, None)) == "FP_E_ARG"
        assert S(fn(None, FAKE + 0x1000000, 128, 64, BF16, 0, None)) == "FP_E_NULL"
        assert S(fn(FAKE, FAKE + 0x1000008, 128, 64, BF16, 0, None)) == "FP_E_ALIGN"
        assert S(fn(FAKE, FAKE + 0x100, 128, 64, BF16, 0, None)) == "FP_E_ALIAS"        # 16 KB each


def test_packed_plans(plan_override):
    plan_override()
    b = torch.bfloat16
    # the same kernel and grid as row-major weights; the tiled family unpacks first
    for M, K, N, fn in ((32, 4096, 28672, "swiglu"), (32, 4096, 6144, "none"), (16384, 4096, 22016, "swiglu"),
                        (300, 4096, 6144, "none")):
        lay = "packed_gate_up" if fn == "swiglu" else "packed"
        a, r = fra.describe_plan(M, K, N, b, b, fn, layout=lay), fra.describe_plan(M, K, N, b, b, fn)
        assert a == r, (a, r)
    p = fra.describe_plan(40, 320, 6144, b, b, layout="packed")
    assert p["family"] == "tiled" and p["prep"] == "unpack_kernel"
    assert p["workspace"] >= fra.describe_plan(40, 320, 6144, b, b)["workspace"] + 6144 * 320 * 2
    p = fra.describe_plan(40, 512, 1024, b, torch.uint8, "swiglu", layout="packed_gate_up")
    # the streaming grid leaves CUs for one workgroup per token: the kernel forms the rows
    assert p["family"] == "stream" and p["kernel"].endswith(",rows>") and "prep" not in p, p
    with fra.plan_override(no_stream=1):
        p = fra.describe_plan(40, 512, 1024, b, torch.uint8, "swiglu", layout="packed_gate_up")
        assert p["family"] == "tiled" and p["prep"] == "unpack_kernel+dequant_i4_kernel", p
        assert fra.workspace_bytes(40, 512, 1024, b, torch.uint8, "packed_gate_up") >= 1024 * 256 + 1024 * 512 * 2


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


def test_plan_routing_families(plan_override):
    plan_override()
    # decode token counts with K a multiple of 256: the weight-streaming kernel
    p = _plan(32, 4096, 2 * 14336, fn="swiglu")
    assert p["family"] == "stream" and p["kernel"] == "stream_kernel<bf16,m32,n128,k256,swiglu,rows>"
    # 224 tiles of a 235 MB weight: one whole tile per workgroup, nothing shared
    assert p["grid"] == 224 and p["slots"] == 1
    # the same tile count on a 470 MB weight: stream-K over 256 workgroups
    p = _plan(64, 8192, 57344, w=torch.int8, fn="swiglu")
    assert p["grid"] == 256 and p["slots"] >= 2
    # 16-bit QKV weights at up to 32 tokens: 32-row tiles with K halves (192
    # of them: at least three quarters of the CUs), one whole tile per workgroup
    p = _plan(32, 4096, 6144)
    assert p["kernel"] == "stream_kernel<bf16,m32,n32,k512,linear,rows>" and p["grid"] == 192 and p["slots"] == 1
    # more 32-row tiles than workgroups (Llama-2-7B QKV): 64-row tiles, one each
    p = _plan(16, 4096, 12288)
    assert p["kernel"] == "stream_kernel<bf16,m16,n64,k256,linear,rows>" and p["grid"] == 192 and p["slots"] == 1
    # requested: 64 rows, two workgroups per tile; or 32 rows where 64 would be chosen
    with fra.plan_override(stream_nr=1):
        p = _plan(32, 4096, 6144)
        assert p["kernel"] == "stream_kernel<bf16,m32,n64,k256,linear,rows>" and p["grid"] == 192 and p["slots"] == 2
    try:
        fra.tune_install([dict(m_lo=0, m_hi=64, hidden=4096, n_cols=12288, act_dtype=torch.bfloat16,
                               w_dtype=torch.bfloat16, swiglu=False, family="stream", rows=32)])
        assert _plan(16, 4096, 12288)["kernel"] == "stream_kernel<bf16,m16,n32,k512,linear>"
        # not for gate/up pairs, 4-bit or int8 weights, 33..64 tokens or hidden not a multiple of 512
        fra.tune_install([dict(m_lo=0, m_hi=64, hidden=K, n_cols=N, act_dtype=torch.bfloat16, w_dtype=w,
                               swiglu=sw, family="stream", rows=32)
                          for K in (768, 4096) for N in (6144, 28672) for w in (torch.bfloat16, torch.int8)
                          for sw in (False, True)])
        assert ",n128," in _plan(16, 4096, 28672, fn="swiglu")["kernel"]
        assert ",n128," in _plan(16, 4096, 6144, w=torch.int8)["kernel"]
        assert ",n128," in _plan(48, 4096, 6144)["kernel"]
        assert ",n64," in _plan(16, 768, 6144)["kernel"]
    finally:
        fra.tune_clear()
    # 33..64 tokens keep 128-row tiles
    assert _plan(64, 4096, 6144)["kernel"] == "stream_kernel<bf16,m64,n128,k128,linear,rows>"
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
    # more than 64 tokens, 16-bit weights, at least 256 tiles of 256 x 256: the
    # row pass writes the normalised rows, the 256 x 256 GEMM reads them
    p = _plan(16384, 4096, 12288)
    assert p["family"] == "gemm16" and p["kernel"] == "gemm16_kernel<bf16,256x256,2st,linear>"
    assert p["grid"] == 64 * 48 and p["splits"] == 1 and p["prep"] == "norm_kernel<bf16>"
    assert p["workspace"] == 16384 * 4096 * 2
    p = _plan(16384, 4096, 2 * 11008, fn="swiglu")
    assert p["kernel"] == "gemm16_kernel<bf16,256x256,2st,swiglu>" and p["grid"] == 64 * 86
    # hidden not a multiple of 128: four stages of K 32
    assert _plan(16384, 4160, 12288)["kernel"] == "gemm16_kernel<bf16,256x256,4st,linear>"
    # fewer tiles: the 128 x 512 kernel (192 tiles of 256 x 256 here)
    p = _plan(1024, 4096, 12288)
    assert p["family"] == "prefill" and p["kernel"] == "prefill_kernel<bf16,128x512,linear>"
    assert p["grid"] == 8 * 24 and p["splits"] == 1
    # split K so that the workgroups fill one round of CUs: 40 tiles -> 6 splits
    # (240 workgroups); 224 tiles -> unsplit (2 splits would take two rounds)
    p = _plan(256, 8192, 10240, w=torch.int8)
    assert p["family"] == "prefill" and p["splits"] == 6 and p["grid"] == 240
    p = _plan(256, 8192, 57344, w=torch.int8, fn="swiglu")
    assert p["splits"] == 1 and p["grid"] == 224
    assert _plan(2048, 4096, 16384, act=torch.float16, w=torch.float16, fn="gelu_tanh")["kernel"] == \
        "gemm16_kernel<f16,256x256,2st,gelu>"
    assert _plan(512, 4096, 16384, act=torch.float16, w=torch.float16, fn="gelu_tanh")["kernel"] == \
        "prefill_kernel<f16,128x512,gelu>"
    # past 4 GiB of activations or of weights the 128 x 512 kernel's 32-bit
    # buffer offsets do not reach: the tiled kernel; decode counts stream any size
    m_big = (1 << 32) // (2 * 4096) + 64
    assert _plan(m_big, 4096, 256)["family"] == "tiled"
    assert _plan(m_big - 128, 4096, 256)["family"] == "gemm16"
    assert _plan(m_big - 128, 4096, 256, w=torch.int8)["family"] == "prefill"
    f_big = (1 << 32) // (2 * 2 * 8192) + 32
    assert _plan(96, 8192, 2 * f_big, fn="swiglu")["family"] == "tiled"
    assert _plan(96, 8192, 2 * f_big - 128, fn="swiglu")["family"] == "prefill"
    assert _plan(8, 8192, 2 * f_big, fn="swiglu")["family"] == "stream"


def test_plan_grid_slots_consistent(plan_override):
    """The stream kernel's partial-sum slots cover the most workgroups that share
    one tile, for unit counts that do and do not divide evenly."""
    for splits in ("1", "2", "3", "5", "7"):
        plan_override(splits=int(splits))
        for M, K, N in ((1, 2048, 640), (32, 4096, 6144), (20, 1024, 928)):
            p = _plan(M, K, N)
            # 64-row tiles of 256-wide chunks, or 32-row tiles of 512-wide
            # chunks (16-bit weights, no pairing, <= 32 tokens)
            nb, ck = (int(f[1:]) for f in p["kernel"].split(",")[2:4])
            assert (nb, ck) in ((64, 256), (32, 512)), p
            tiles = -(-N // nb)
            chunks = K // ck
            units = tiles * chunks
            G = min(tiles * int(splits), units)
            assert p["grid"] == G
            owner = lambda v: ((v + 1) * G - 1) // units
            most = max(owner(t * chunks + chunks - 1) - owner(t * chunks) + 1 for t in range(tiles))
            assert p["slots"] == most


def test_plan_overrides(plan_override):
    plan_override(no_stream=1)
    assert _plan(32, 4096, 6144)["family"] == "tiled"
    plan_override(no_prefill=1)
    assert _plan(300, 4096, 6144)["family"] == "tiled"
    assert _plan(32, 4096, 6144)["family"] == "stream"
    plan_override(stream_nr=2)
    assert _plan(8, 4096, 6144)["kernel"] == "stream_kernel<bf16,m16,n128,k256,linear,rows>"
    plan_override(stream_target=64)
    assert _plan(8, 4096, 28672, fn="swiglu")["grid"] == 64
    plan_override(no_gemm16=1)
    assert _plan(16384, 4096, 12288)["family"] == "prefill"
    plan_override(gemm16_stages=5)
    assert _plan(16384, 4096, 12288)["kernel"] == "gemm16_kernel<bf16,256x256,5st,linear>"
    plan_override(gemm16_stages=4)
    assert _plan(16384, 4096, 12288)["kernel"] == "gemm16_kernel<bf16,256x256,4st,linear>"
    plan_override(gemm16_stages=2)
    assert _plan(16384, 4096, 12288)["kernel"] == "gemm16_kernel<bf16,256x256,2st,linear>"
    assert _plan(16384, 4160, 12288)["kernel"] == "gemm16_kernel<bf16,256x256,4st,linear>"
    plan_override(no_gemm16=1, no_prefill=1)
    assert _plan(16384, 4096, 12288)["family"] == "tiled"
    plan_override(no_stream_rows=1)
    p = _plan(32, 4096, 6144)
    assert p["kernel"] == "stream_kernel<bf16,m32,n32,k512,linear>" and p["prep"] == "norm_kernel<bf16>"
    plan_override()
    assert fra.get_plan_override() == dict(splits=0, stream_nr=0, stream_target=0, no_stream=0, no_prefill=0,
                                           fp8_tile=0, no_gemm16=0, gemm16_stages=0, no_stream_rows=0,
                                           stream_rows_expire=0)
    # out-of-range values are rejected and leave the overrides as they were
    plan_override(splits=2)
    for bad in (dict(splits=65), dict(splits=-1), dict(stream_nr=3), dict(no_stream=2), dict(fp8_tile=100),
                dict(stream_target=70000), dict(no_gemm16=2), dict(gemm16_stages=3), dict(no_stream_rows=2),
                dict(stream_rows_expire=2)):
        with pytest.raises(fra.FusedProjError) as ei:
            fra.set_plan_override(bad)
        assert ei.value.status == 8                     # FP_E_ARG
        assert fra.get_plan_override()["splits"] == 2
    with pytest.raises(ValueError):
        fra.set_plan_override(dict(bogus=1))


def test_plan_overrides_read_environment_once():
    """The FUSEDPROJ_* variables are read once, at the library's first plan, in
    a fresh process; changing them afterwards has no effect."""
    import subprocess
    import sys
    code = (
        "import os, torch, fusion_residual_add_amd as fra\n"
        "p = fra.describe_plan(32, 4096, 6144, torch.bfloat16, torch.bfloat16)\n"
        "assert p['family'] == 'tiled' and p['splits'] == 3, p\n"
        "os.environ['FUSEDPROJ_NO_STREAM'] = '0'\n"
        "os.environ['FUSEDPROJ_SPLITS'] = '5'\n"
        "assert fra.describe_plan(32, 4096, 6144, torch.bfloat16, torch.bfloat16) == p\n"
        "fra.set_plan_override({})\n"
        "assert fra.describe_plan(32, 4096, 6144, torch.bfloat16, torch.bfloat16)['family'] == 'stream'\n"
        "fra.set_plan_override(None)\n"
        "assert fra.describe_plan(32, 4096, 6144, torch.bfloat16, torch.bfloat16) == p\n"
        "print('env-once ok')\n")
    env = dict(os.environ, FUSEDPROJ_NO_STREAM="1", FUSEDPROJ_SPLITS="3")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0 and "env-once ok" in res.stdout, res.stdout + res.stderr


def test_status_numbering():
    """Codes 0-6 as the boundary's specification numbers them; 7 and 8 appended."""
    assert _lib.STATUS[:7] == ["FP_OK", "FP_E_NULL", "FP_E_SHAPE", "FP_E_DTYPE", "FP_E_ALIGN", "FP_E_ALIAS",
                               "FP_E_HIP"]
    assert _lib.STATUS[7:] == ["FP_E_WORKSPACE", "FP_E_ARG"]
    texts = [lib().fp_status_str(i).decode() for i in range(9)]
    assert texts[6] == "HIP error" and texts[7].startswith("workspace") and texts[8].startswith("invalid")


def test_plan_rejects():
    with pytest.raises(fra.FusedProjError):
        _plan(32, 4000, 6144)                  # hidden not a multiple of 64
    with pytest.raises(fra.FusedProjError):
        _plan(32, 4096, 6144, act=torch.float16, w=torch.int8)


def _entry(**kw):
    e = dict(m_lo=17, m_hi=32, hidden=4096, n_cols=6144, act_dtype=torch.bfloat16,
             w_dtype=torch.bfloat16, swiglu=False)
    e.update(kw)
    return e


def test_tuning_table_overrides_matching_calls(plan_override):
    plan_override()
    base, base_gu, base_33 = _plan(32, 4096, 6144), _plan(32, 4096, 6144, fn="swiglu"), _plan(33, 4096, 6144)
    try:
        fra.tune_install([_entry(family="stream", rows=128, grid=192)])
        assert fra.tune_count() == 1
        p = _plan(32, 4096, 6144)
        assert p["kernel"] == "stream_kernel<bf16,m32,n128,k256,linear,rows>" and p["grid"] == 192
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
        assert _plan(32, 4096, 6144)["kernel"] == "stream_kernel<bf16,m32,n128,k256,linear,rows>"
        # the first matching entry wins; the plan overrides win over the table
        fra.tune_install([_entry(grid=128), _entry(grid=64)])
        assert _plan(32, 4096, 6144)["grid"] == 128
        fra.tune_install([_entry(family="stream")])
        plan_override(no_stream=1)
        assert _plan(32, 4096, 6144)["family"] == "tiled"
        plan_override()
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
    g8 = [x["plan"] for x in c if x["plan"]["kernel"].startswith("gemm8_kernel")]
    st = [x["plan"] for x in c if x["plan"]["kernel"].startswith("stream_kernel<bf16-e4m3")]
    assert len(g8) + len(st) == len(c)
    assert sorted(p["splits"] for p in g8) == [1, 2, 3, 4, 6, 8]
    # the streaming kernel at 128 and 256 rows per workgroup and several grids
    assert {p["kernel"].split(",")[2] for p in st} == {"n128", "n256"} and len({p["grid"] for p in st}) > 3
    assert fra.tune_count() == 0


def test_tuner_candidates_cover_every_family():
    from fusion_residual_add_amd import tune
    for w in (torch.bfloat16, torch.int8, torch.uint8):
        fams = {c["plan"]["family"] for c in tune.candidates(16, 1024, 1024, torch.bfloat16, w, False)}
        assert fams == {"stream", "prefill", "tiled"} | ({"gemm16"} if w == torch.bfloat16 else set()), (w, fams)
        kernels = {c["plan"]["kernel"] for c in tune.candidates(16, 1024, 1024, torch.bfloat16, w, False)}
        if w != torch.bfloat16:
            assert any(",n256," in k for k in kernels), kernels   # 256 rows per workgroup for int8 / int4
        else:   # 16-bit weights without gate/up pairing: 32, 64 and 128 rows
            assert {k.split(",")[2] for k in kernels if k.startswith("stream")} == {"n32", "n64", "n128"}, kernels
    # E4M3 QKV at decode counts: every instantiated row count of the streaming kernel
    c = tune.candidates(16, 4096, 6144, torch.bfloat16, torch.float8_e4m3fn, False)
    st = {x["plan"]["kernel"].split(",")[2] for x in c if x["plan"]["kernel"].startswith("stream")}
    assert st == {"n32", "n64", "n128", "n256"}, st
    assert fra.tune_count() == 0
