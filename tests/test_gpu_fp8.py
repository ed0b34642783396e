"""FP8 W8A8 (E4M3 weights with per-row scales, per-token E4M3 activations)
through the C ABI against the oracle: both projections and the down
projection, bf16 and fp16 activations, every norm and epilogue, ragged token
and column counts, split K, rows that quantise to zero, and the workloads at
full size on sampled token rows.  Both GEMMs on the codes are covered: the
FP8 GEMM tiles (the planner's choice; every tile form, split K) and the
weight-streaming kernel, requested through the tuning table (up to 64 tokens
with hidden a multiple of the chunk; 128 or 256 weight rows per workgroup,
whole tiles or K ranges shared by several workgroups).

Both sides decide every activation code in double precision (the oracle's
exact normalisation, the quantisation kernel's fp64 statistics and scaling
narrowed with round-to-odd), so the codes agree unless a scaled value lies
within double rounding of a midpoint between two E4M3 values; the outputs
then differ only by the fp32 accumulation and scaling, and the tolerances of
test_gpu_parity apply.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, TDT, check, full_size_check, run_gu, run_qkv, small, to_dev, _sample_rows

pytestmark = pytest.mark.gpu
E4M3 = torch.float8_e4m3fn


def _force_stream(wl, down=False):
    """Tuning entries that send this workload's FP8 calls to the weight-streaming kernel."""
    common = dict(m_lo=0, m_hi=64, act_dtype=TDT[wl.act], w_dtype=E4M3, family="stream")
    ents = [dict(common, hidden=wl.hidden, n_cols=wl.n_qkv, swiglu=False),
            dict(common, hidden=wl.hidden, n_cols=wl.n_gu, swiglu=wl.act_fn == "swiglu")]
    if down:
        ents.append(dict(common, hidden=wl.ffn, n_cols=wl.hidden, swiglu=False))
    fra.tune_install(ents)


@pytest.fixture
def stream_table():
    yield _force_stream
    fra.tune_clear()


def _stream_ok(M, K):
    return M <= 64 and K % (128 if M > 32 else 256) == 0

FP8 = [
    dict(M=1, hidden=256), dict(M=5, hidden=384, ffn=208), dict(M=17, hidden=512, H=8, Hkv=2, D=64),
    dict(M=33, hidden=256), dict(M=64, hidden=1024, ffn=336), dict(M=65, hidden=384),
    dict(M=130, hidden=512, ffn=400), dict(M=257, hidden=256, ffn=208, act_fn="none", bias=True),
    dict(M=40, hidden=512, norm="layer"), dict(M=90, hidden=256, norm="layer", act_fn="gelu_tanh", bias=True),
    dict(act="f16", M=37, hidden=384), dict(act="f16", M=150, hidden=512, norm="layer", act_fn="gelu_tanh",
                                            bias=True, ffn=272),
    dict(M=3, H=5, Hkv=1, D=48, hidden=640, ffn=48), dict(M=129, H=8, Hkv=8, D=16, hidden=512),
    dict(act="f16", M=9, hidden=1024, ffn=176, norm="layer", act_fn="gelu_tanh", bias=True),
    dict(act="f16", M=50, hidden=512, H=5, Hkv=1, D=48, ffn=80),
]


def _fp8(**cfg):
    bias = cfg.pop("bias", False)
    return small(wdt="e4m3", bias=bias, **cfg)


@pytest.mark.parametrize("kernel", ["planner", "stream"])
@pytest.mark.parametrize("cfg", FP8, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("native", [False, True], ids=["f32out", "nativeout"])
def test_fp8_small(cfg, native, kernel, stream_table):
    wl = _fp8(**dict(cfg))
    if kernel == "stream":
        if not _stream_ok(wl.M, wl.hidden):
            pytest.skip("the streaming kernel does not take this shape")
        stream_table(wl)
    inp = inputs.generate(wl, seed=7)
    d = to_dev(inp)
    odt = None if native else torch.float32
    adt = d["x"].dtype
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, adt, E4M3, wl.act_fn)
    print(f"fp8 {wl.name} {plan['kernel']} splits={plan['splits']} native={native}", flush=True)
    assert plan["family"] == "fp8"
    assert plan["kernel"].startswith("stream_kernel" if kernel == "stream" else "gemm8_kernel"), plan
    q, k, v, h = run_qkv(wl, d, odt)
    out = run_gu(wl, d, odt)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("k", k, rq["k"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])
    assert np.array_equal(h.double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"


@pytest.mark.parametrize("splits", [1, 3, 8])
@pytest.mark.parametrize("M,kernel", [(1, "stream"), (48, "stream"), (1, "gemm8"), (48, "gemm8"), (200, "gemm8")])
def test_fp8_splits(splits, M, kernel, plan_override, stream_table):
    # the FP8 GEMM tiles split K in `splits` (the last split to arrive adds
    # the partial sums); the weight-streaming kernel gives each weight tile
    # `splits` workgroups (at most one per K chunk) that share it the same way
    plan_override(splits=int(splits))
    wl = _fp8(M=M, hidden=1024, ffn=208)
    if kernel == "stream":
        stream_table(wl)
    inp = inputs.generate(wl, seed=8)
    d = to_dev(inp)
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.float8_e4m3fn, "swiglu")
    print(f"fp8 splits {splits} M={M}: {plan['kernel']} grid={plan['grid']} slots={plan['slots']}", flush=True)
    if kernel == "stream":
        assert plan["kernel"].startswith("stream_kernel<bf16-e4m3") and (plan["slots"] > 1) == (splits > 1), plan
    else:
        assert plan["kernel"].startswith("gemm8_kernel") and plan["splits"] == splits, plan
    q, k, v, _ = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])


@pytest.mark.parametrize("tile", ["32", "64", "128", "256"])
@pytest.mark.parametrize("M", [1, 40, 100, 300])
def test_fp8_tiles(tile, M, plan_override):
    # every tile form at token counts below, inside and above its own height
    plan_override(fp8_tile=int(tile))
    wl = _fp8(M=M, hidden=512, ffn=272, H=6, Hkv=2, D=32, act_fn="swiglu", bias=True)
    inp = inputs.generate(wl, seed=15)
    d = to_dev(inp)
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.float8_e4m3fn, "swiglu")
    print(f"fp8 tile {tile} M={M}: {plan['kernel']} splits={plan['splits']}", flush=True)
    assert f",{tile}x" in plan["kernel"]
    q, k, v, _ = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("k", k, rq["k"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])


@pytest.mark.parametrize("target", [0, 7])
@pytest.mark.parametrize("nr", [2, 4])
@pytest.mark.parametrize("M", [1, 20, 64])
def test_fp8_stream_forms(M, nr, target, plan_override, stream_table):
    # 128 / 256 weight rows per workgroup; target 7: a few workgroups that
    # each stream several tiles, with ranges shared across tile boundaries
    plan_override(stream_nr=nr, stream_target=target)
    wl = _fp8(M=M, hidden=1536, ffn=336, H=6, Hkv=2, D=64, act_fn="swiglu", bias=True)
    stream_table(wl)
    inp = inputs.generate(wl, seed=16)
    d = to_dev(inp)
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.float8_e4m3fn, "swiglu")
    print(f"fp8 stream M={M} nr={nr} target={target}: {plan['kernel']} grid={plan['grid']} "
          f"slots={plan['slots']}", flush=True)
    assert plan["kernel"].startswith("stream_kernel<bf16-e4m3") and f",n{64 * nr}," in plan["kernel"]
    if target:
        assert plan["grid"] <= target
    q, k, v, h = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, None)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("k", k, rq["k"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])
    assert np.array_equal(h.double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"


def test_fp8_zero_rows_and_bias():
    # rows whose normalised values are all zero quantise to zero codes with a
    # zero scale: the output is the bias alone
    wl = _fp8(M=20, hidden=256, ffn=64, act_fn="none", bias=True, norm="none")
    inp = inputs.generate(wl, seed=9)
    inp["r"][3] = -inp["x"][3]
    inp["x"][11] = 0
    inp["r"][11] = 0
    d = to_dev(inp)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rg = oracle.workload_gateup(wl, inp)
    check("out", out, rg["out"])
    b = inp["b_gu"].double().numpy()
    assert np.array_equal(out[3].double().cpu().numpy(), b)
    assert np.array_equal(out[11].double().cpu().numpy(), b)


@pytest.mark.parametrize("kernel", ["gemm8", "stream"])
def test_fp8_deterministic_and_m_zero(kernel, plan_override, stream_table):
    plan_override(splits=4)
    wl = _fp8(M=24, hidden=512, ffn=144)
    if kernel == "stream":
        stream_table(wl)
    d = to_dev(inputs.generate(wl, seed=10))
    a = run_gu(wl, d)
    b = run_gu(wl, d)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    e = fra.fused_gateup_act(d["x"][:0], d["r"][:0], d["gamma"], d["w_gu"], wl.ffn, "swiglu", w_scale=d["s_gu"])
    assert e.shape == (0, wl.ffn)


DOWN8 = [dict(M=1, hidden=320, ffn=512), dict(M=20, hidden=512, ffn=1024), dict(M=150, hidden=256, ffn=768),
         dict(act="f16", M=40, hidden=512, ffn=512), dict(M=7, hidden=192, ffn=1536)]


@pytest.mark.parametrize("kernel", ["planner", "stream"])
@pytest.mark.parametrize("cfg", DOWN8, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("mode", ["f32out", "nativeout", "inplace"])
def test_fp8_down(cfg, mode, kernel, stream_table):
    wl = _fp8(**dict(cfg))
    if kernel == "stream":
        if not _stream_ok(wl.M, wl.ffn):
            pytest.skip("the streaming kernel does not take this shape")
        stream_table(wl, down=True)
    inp = inputs.generate(wl, seed=12, parts=("down",))
    d = to_dev(inp)
    plan = fra.describe_plan(wl.M, wl.ffn, wl.hidden, d["a_down"].dtype, E4M3)
    assert plan["kernel"].startswith("stream_kernel" if kernel == "stream" else "gemm8_kernel"), plan
    print(f"fp8 down {wl.name} {mode}: {plan['kernel']}", flush=True)
    if mode == "inplace":
        res = d["r"].clone()
        out = fra.fused_down_residual(d["a_down"], d["w_down"], res, w_scale=d["s_down"], out=res)
        assert out.data_ptr() == res.data_ptr()
    else:
        out = fra.fused_down_residual(d["a_down"], d["w_down"], d["r"], w_scale=d["s_down"],
                                      out_dtype=torch.float32 if mode == "f32out" else None)
    torch.cuda.synchronize()
    ref = oracle.down_residual(inp["a_down"], inp["w_down"], inp["s_down"], None, inp["r"])
    check("out", out, ref)


FULL8 = ["llama3-8b-decode-fp8", "llama2-7b-prefill-fp8", "gpt-fp16-gelu-fp8"]


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", FULL8)
def test_fp8_workload_full_size(name, seed):
    full_size_check(inputs.workload(name), seed)


def test_fp8_stream_full_size(stream_table):
    wl = inputs.workload("llama3-8b-decode-fp8")
    stream_table(wl)
    assert fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, E4M3, "swiglu")["kernel"].startswith(
        "stream_kernel<bf16-e4m3")
    full_size_check(wl, 3)


# the quantisation kernel's forms: one workgroup per row (up to 1024 tokens)
# or one wave per row, the row kept in registers (up to 16 vectors of 8 per
# thread) or read again for every pass
@pytest.mark.parametrize("M,hidden", [(3, 33024), (1030, 8192), (1100, 8320), (1500, 512)],
                         ids=["wg-reload", "wave-regs16", "wave-reload", "wave-regs1"])
def test_fp8_quant_forms(M, hidden):
    wl = _fp8(M=M, hidden=hidden, ffn=32, H=2, Hkv=1, D=16, norm="layer")
    inp = inputs.generate(wl, seed=14)
    d = to_dev(inp)
    q, k, v, h = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rows = _sample_rows(M, 16)
    rq = oracle.workload_qkv(wl, inp, row_idx=rows)
    rg = oracle.workload_gateup(wl, inp, row_idx=rows)
    check("q", q[rows], rq["q"])
    check("v", v[rows], rq["v"])
    check("out", out[rows], rg["out"])
    assert np.array_equal(h[rows].double().cpu().numpy(), rq["h_out"])
