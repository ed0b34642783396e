"""Tile-packed weights (fused_pack_weight / fused_unpack_weight) through the C ABI.

* The packed bytes against the layout's definition written out here with
  numpy reshapes (rows in groups of 128 -- gate/up pairing: 64 gate rows,
  then the 64 matching up rows --, a group as its 64-byte K slices, a slice
  as its eight 16-row blocks of 1 KB, byte 256 g + 16 i + j of a block being
  byte 64 s + 16 g + j of its row i), and unpacking back to the row-major
  bytes, for every weight dtype.
* Every kernel family reading packed weights against the same call on the
  row-major weights, bit for bit: the kernels differ only in the addresses
  they load from, so every sum and its order are the same.  The row-major
  calls themselves are held to the oracle by the parity tests; one case per
  family is checked against the oracle here as well.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, TDT, check, small, to_dev, _sample_rows

pytestmark = pytest.mark.gpu

WDT = {"bf16": torch.bfloat16, "f16": torch.float16, "i8": torch.int8, "i4": torch.uint8,
       "e4m3": torch.float8_e4m3fn, "mxfp4": torch.float4_e2m1fn_x2}


def expected_packed(wb: np.ndarray, gate_up: bool) -> np.ndarray:
    """The packed bytes of a row-major weight wb (uint8 [N, row bytes])."""
    N, RB = wb.shape
    if gate_up:
        F = N // 2
        order = np.concatenate([np.r_[np.arange(64 * t, 64 * t + 64), F + np.arange(64 * t, 64 * t + 64)]
                                for t in range(F // 64)])
        wb = wb[order]
    T, S = N // 128, RB // 64
    x = wb.reshape(T, 8, 16, S, 4, 16)                    # group, block, row, slice, 16-byte group, byte
    return x.transpose(0, 3, 1, 4, 2, 5).reshape(N, RB)   # group, slice, block, 16-byte group, row, byte


@pytest.mark.parametrize("gate_up", [False, True])
@pytest.mark.parametrize("wdt", list(WDT))
@pytest.mark.parametrize("rows,row_bytes", [(128, 64), (256, 512), (384, 192)])
def test_pack_layout(wdt, gate_up, rows, row_bytes):
    rng = np.random.default_rng(rows + row_bytes)
    wb = rng.integers(0, 256, size=(rows, row_bytes), dtype=np.uint8)
    w = torch.from_numpy(wb).to(DEV)
    elt = 2 if wdt in ("bf16", "f16") else 1
    w = w.view(WDT[wdt]).reshape(rows, row_bytes // elt)
    if gate_up and rows % 128:
        pytest.skip("gate/up pairs need ffn a multiple of 64")
    pw = fra.pack_weight(w, gate_up=gate_up)
    back = fra.unpack_weight(pw)
    torch.cuda.synchronize()
    got = pw.data.view(torch.uint8).reshape(rows, row_bytes).cpu().numpy()
    assert np.array_equal(got, expected_packed(wb, gate_up))
    assert np.array_equal(back.view(torch.uint8).reshape(rows, row_bytes).cpu().numpy(), wb)
    assert pw.dtype == w.dtype and tuple(pw.shape) == tuple(w.shape)


def test_pack_rejects():
    w = torch.zeros(100, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fra.FusedProjError, match="FP_E_SHAPE"):
        fra.pack_weight(w)                                   # 100 rows
    w = torch.zeros(128, 64, dtype=torch.float32, device=DEV)
    with pytest.raises(fra.FusedProjError, match="FP_E_DTYPE"):
        fra.pack_weight(w)
    w = torch.zeros(192, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fra.FusedProjError, match="FP_E_SHAPE"):
        fra.pack_weight(w, gate_up=True)                     # ffn 96


# family, act, weight dtype, tokens, hidden, gate/up activation
CASES = [
    ("stream", "bf16", "bf16", 1, 512, "swiglu"), ("stream", "bf16", "bf16", 20, 768, "swiglu"),
    ("stream", "f16", "f16", 64, 512, "gelu_tanh"), ("stream", "bf16", "bf16", 32, 1024, "none"),
    ("stream", "bf16", "i8", 33, 512, "swiglu"), ("stream", "bf16", "i4", 16, 512, "swiglu"),
    ("stream", "bf16", "mxfp4", 48, 512, "swiglu"), ("stream", "bf16", "e4m3", 24, 512, "swiglu"),
    ("stream", "f16", "e4m3", 60, 512, "gelu_tanh"),
    ("prefill", "bf16", "bf16", 130, 512, "swiglu"), ("prefill", "f16", "f16", 200, 384, "gelu_tanh"),
    ("prefill", "bf16", "i8", 100, 512, "swiglu"), ("prefill", "bf16", "i4", 150, 512, "none"),
    ("prefill", "bf16", "mxfp4", 90, 512, "swiglu"),
    ("gemm16", "bf16", "bf16", 300, 512, "swiglu"), ("gemm16", "f16", "f16", 520, 640, "gelu_tanh"),
    ("gemm16", "bf16", "bf16", 260, 384, "swiglu"),
    ("tiled", "bf16", "bf16", 40, 384, "swiglu"), ("tiled", "bf16", "i4", 40, 384, "swiglu"),
    ("tiled", "bf16", "mxfp4", 20, 256, "swiglu"), ("tiled", "bf16", "i8", 70, 256, "gelu_tanh"),
    ("fp8", "bf16", "e4m3", 1, 512, "swiglu"), ("fp8", "bf16", "e4m3", 64, 512, "swiglu"),
    ("fp8", "f16", "e4m3", 200, 512, "gelu_tanh"), ("fp8", "bf16", "e4m3", 600, 512, "swiglu"),
    # overrides: 256 weight rows per streaming workgroup; the 256 x 256 FP8 tile
    ("stream-nr4", "bf16", "i8", 64, 512, "swiglu"), ("stream-nr4", "bf16", "e4m3", 40, 512, "swiglu"),
    ("fp8-256", "bf16", "e4m3", 300, 512, "swiglu"),
]


def _table(wl, fam):
    """Tuning entries that send the workload's three calls to one family."""
    fam = fam.split("-")[0]
    if fam == "fp8":
        return
    act, wdt = TDT[wl.act], WDT[wl.wdt]
    common = dict(m_lo=0, m_hi=1 << 40, act_dtype=act, w_dtype=wdt, family=fam)
    fra.tune_install([dict(common, hidden=wl.hidden, n_cols=wl.n_qkv, swiglu=False),
                      dict(common, hidden=wl.hidden, n_cols=wl.n_gu, swiglu=wl.act_fn == "swiglu"),
                      dict(common, hidden=wl.ffn, n_cols=wl.hidden, swiglu=False)])


@pytest.fixture
def table():
    yield _table
    fra.tune_clear()


def _run(wl, d, w_qkv, w_gu, w_down):
    q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], w_qkv, wl.n_heads, wl.n_kv_heads, wl.head_dim,
                                        beta=d.get("beta"), norm=wl.norm, eps=wl.eps, w_scale=d.get("s_qkv"),
                                        out_dtype=torch.float32)
    out = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], w_gu, wl.ffn, wl.act_fn, beta=d.get("beta"),
                               norm=wl.norm, eps=wl.eps, w_scale=d.get("s_gu"), out_dtype=torch.float32)
    dn = fra.fused_down_residual(d["a_down"], w_down, d["r"], w_scale=d.get("s_down"))
    return [t.clone() for t in (q, k, v, out, dn)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(str(x) for x in c))
def test_packed_calls(case, table, plan_override):
    fam, act, wdt, M, hidden, act_fn = case
    wl = small(act=act, wdt=wdt, M=M, hidden=hidden, H=8, Hkv=2, D=64, ffn=256, act_fn=act_fn)
    _table(wl, fam)
    if fam == "stream-nr4":
        plan_override(stream_nr=4)
    if fam == "fp8-256":
        plan_override(fp8_tile=256)
    if fam == "fp8":
        # the FP8 tiles for both layouts (packed decode shapes default to the
        # streaming kernel, checked against the oracle below)
        plan_override(no_stream=1)
    inp = inputs.generate(wl, seed=21, parts=("qkv", "gu", "down"))
    d = to_dev(inp)
    a_dt, w_dt = TDT[act], WDT[wdt]
    sw = act_fn == "swiglu"
    plans = [fra.describe_plan(M, hidden, wl.n_qkv, a_dt, w_dt, "none", layout="packed"),
             fra.describe_plan(M, hidden, wl.n_gu, a_dt, w_dt, act_fn, layout="packed_gate_up" if sw else "packed"),
             fra.describe_plan(M, wl.ffn, hidden, a_dt, w_dt, "none", layout="packed")]
    print(f"packed {case}: " + " | ".join(p["kernel"] + (" " + p["prep"] if "prep" in p else "") for p in plans),
          flush=True)
    want = {"stream": "stream_kernel", "stream-nr4": "stream_kernel", "prefill": "prefill_kernel",
            "gemm16": "gemm16_kernel", "tiled": "proj_kernel", "fp8-256": "gemm8_kernel"}.get(fam)
    if want:
        assert plans[1]["kernel"].startswith(want), plans[1]
    if fam == "tiled":
        assert "unpack_kernel" in plans[1]["prep"]
    rows = _run(wl, d, d["w_qkv"], d["w_gu"], d["w_down"])
    pk = _run(wl, d, fra.pack_weight(d["w_qkv"]), fra.pack_weight(d["w_gu"], gate_up=sw),
              fra.pack_weight(d["w_down"]))
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "k", "v", "gate/up", "down"), rows, pk):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{name}: packed result differs"
    rg = oracle.workload_gateup(wl, inp)
    check("out", pk[3], rg["out"])
    if fam == "fp8":
        plan_override()
        dflt = _run(wl, d, fra.pack_weight(d["w_qkv"]), fra.pack_weight(d["w_gu"], gate_up=sw),
                    fra.pack_weight(d["w_down"]))
        torch.cuda.synchronize()
        rq = oracle.workload_qkv(wl, inp)
        check("q", dflt[0], rq["q"])
        check("v", dflt[2], rq["v"])
        check("out", dflt[3], rg["out"])


def test_packed_layout_mismatch():
    wl = small(M=4, hidden=256, H=8, Hkv=2, D=64, ffn=256)
    d = to_dev(inputs.generate(wl, seed=22))
    # a gate/up-paired weight is for the SwiGLU call only
    with pytest.raises(fra.FusedProjError, match="FP_E_SHAPE"):
        fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], fra.PackedWeight(d["w_qkv"], True), 8, 2, 64)
    # a weight of whole 64-row halves only: ffn 80 is not
    wl = small(M=4, hidden=256, ffn=80)
    d = to_dev(inputs.generate(wl, seed=22))
    with pytest.raises(fra.FusedProjError, match="FP_E_SHAPE"):
        fra.fused_gateup_act(d["x"], d["r"], d["gamma"], fra.PackedWeight(d["w_gu"], True), 80, "swiglu")


@pytest.mark.parametrize("name", ["llama3-8b-decode", "llama3-8b-decode-fp8", "llama2-7b-prefill"])
def test_packed_full_size(name, plan_override):
    """The workloads at full size: packed and row-major results bit for bit
    on the same kernels; FP8 decode, whose packed default is the streaming
    kernel, then also against the oracle on sampled rows."""
    wl = inputs.workload(name)
    inp = inputs.generate(wl, seed=5)
    d = to_dev(inp)
    sw = wl.act_fn == "swiglu"
    fp8 = wl.wdt == "e4m3"
    if fp8:
        plan_override(no_stream=1)

    def both(w_qkv, w_gu):
        q, k, v, _ = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], w_qkv, wl.n_heads, wl.n_kv_heads,
                                            wl.head_dim, beta=d.get("beta"), norm=wl.norm, eps=wl.eps,
                                            w_scale=d.get("s_qkv"), write_h=False)
        out = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], w_gu, wl.ffn, wl.act_fn, beta=d.get("beta"),
                                   norm=wl.norm, eps=wl.eps, w_scale=d.get("s_gu"))
        return q.clone(), out.clone()

    a = both(d["w_qkv"], d["w_gu"])
    pq, pg = fra.pack_weight(d["w_qkv"]), fra.pack_weight(d["w_gu"], gate_up=sw)
    b = both(pq, pg)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int16), b[1].view(torch.int16))
    if fp8:
        plan_override()
        assert fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.float8_e4m3fn, "swiglu",
                                 layout="packed_gate_up")["kernel"].startswith("stream_kernel")
        q, out = both(pq, pg)
        torch.cuda.synchronize()
        rows = _sample_rows(wl.M, 8)
        rq = oracle.workload_qkv(wl, inp, row_idx=rows)
        rg = oracle.workload_gateup(wl, inp, row_idx=rows)
        check("q", q[rows], rq["q"])
        check("out", out[rows], rg["out"])
