"""The row pass + 256 x 256 GEMM (family gemm16) through the C ABI against the
oracle.

The planner takes this family for 16-bit weights of the activation dtype
from 512 tokens on when the call's 256 x 256 tiles fill the GPU; here it is
forced through the tuning table on small shapes that span several 256 x 256
tiles with ragged tails in M, in the weight rows and in the gate/up pairs,
with K step counts below, at and past whole rounds of the LDS stages, every
stage count (two stages of K 64 where hidden allows, four or five of K 32),
every norm, residual present or absent, bias, every epilogue, fp32 and
native outputs, head-major q / k / v and the down projection (in place).
Checked:
  * the normalised rows the row pass leaves at the start of the workspace,
    bit for bit against the oracle's rows of the single-precision reading
    (the GEMM operand), and h_out bit for bit;
  * the outputs to the parity bounds of test_gpu_parity;
  * the full-size prefill workloads (planner's choice) on sampled rows, with
    every stage count.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, TDT, check, full_size_check, small, to_dev

pytestmark = pytest.mark.gpu


def _force(wl, down=False):
    """Tuning entries that send this workload's calls to the gemm16 family."""
    act = TDT[wl.act]
    common = dict(m_lo=0, m_hi=1 << 40, act_dtype=act, w_dtype=act)
    ents = [dict(common, hidden=wl.hidden, n_cols=wl.n_qkv, swiglu=False, family="gemm16"),
            dict(common, hidden=wl.hidden, n_cols=wl.n_gu, swiglu=wl.act_fn == "swiglu", family="gemm16")]
    if down:
        ents.append(dict(common, hidden=wl.ffn, n_cols=wl.hidden, swiglu=False, family="gemm16"))
    fra.tune_install(ents)


@pytest.fixture
def forced():
    yield _force
    fra.tune_clear()


CASES = [
    dict(M=300, hidden=320),                                  # K 10 steps of 32
    dict(M=257, hidden=256, ffn=208),                         # one row past a tile; 8 K steps
    dict(M=1, hidden=512), dict(M=5, hidden=64, ffn=48),      # one token; K of 2 steps
    dict(M=600, hidden=1024, H=8, Hkv=2, D=64, ffn=400),
    dict(M=513, hidden=768, norm="layer", act_fn="gelu_tanh", bias=True, ffn=272),
    dict(M=256, hidden=384, norm="layer", ffn=144),
    dict(M=130, hidden=512, act_fn="none", bias=True, ffn=1008),
    dict(M=400, hidden=640, act="f16", ffn=336),
    dict(M=270, hidden=512, act="f16", norm="layer", act_fn="gelu_tanh", bias=True, ffn=528),
]


@pytest.mark.parametrize("stages", [2, 4, 5])
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_gemm16_small(cfg, stages, forced, plan_override):
    cfg = dict(cfg)
    bias = cfg.pop("bias", False)
    wl = small(bias=bias, **cfg)
    forced(wl)
    plan_override(gemm16_stages=stages)
    inp = inputs.generate(wl, seed=12)
    if bias:
        inp["b_qkv"] = inputs._to_act(np.random.default_rng(9).standard_normal(wl.n_qkv).astype(np.float32)
                                      * np.float32(0.1), wl.act)
    d = to_dev(inp)
    act = TDT[wl.act]
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_qkv, act, act)
    print(f"gemm16 {wl.name} {plan['kernel']} grid={plan['grid']} stages={stages}", flush=True)
    # two stages need hidden a multiple of 128 (an even number of K steps of 64)
    want = 4 if stages == 2 and wl.hidden % 128 else stages
    assert plan["family"] == "gemm16" and f"{want}st" in plan["kernel"]
    need = fra.workspace_bytes(wl.M, wl.hidden, wl.n_gu, act, act)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    for native in (False, True):
        odt = act if native else torch.float32
        q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                            wl.head_dim, beta=d.get("beta"), norm=wl.norm, eps=wl.eps,
                                            bias=d.get("b_qkv"), out_dtype=odt, workspace=ws)
        rows = ws[:wl.M * wl.hidden * 2].view(act).reshape(wl.M, wl.hidden).clone()
        out = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], d["w_gu"], wl.ffn, wl.act_fn, beta=d.get("beta"),
                                   norm=wl.norm, eps=wl.eps, bias=d.get("b_gu"), out_dtype=odt, workspace=ws)
        torch.cuda.synchronize()
        rq = oracle.workload_qkv(wl, inp)
        rg = oracle.workload_gateup(wl, inp)
        _, _, a_ref = oracle.add_norm(inp["x"], inp["r"], inp["gamma"], inp.get("beta"), wl.norm, wl.eps)
        assert np.array_equal(rows.double().cpu().numpy(), a_ref), "normalised rows not bit-exact"
        assert np.array_equal(h.double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"
        check("q", q, rq["q"])
        check("k", k, rq["k"])
        check("v", v, rq["v"])
        check("out", out, rg["out"])


@pytest.mark.parametrize("norm", ["none", "rms"])
def test_gemm16_without_residual(norm, forced):
    wl = small(M=520, hidden=512, norm=norm, ffn=272)
    forced(wl)
    inp = inputs.generate(wl, seed=13)
    d = to_dev(inp)
    out = fra.fused_gateup_act(d["x"], None, d["gamma"], d["w_gu"], wl.ffn, "swiglu", norm=norm, eps=wl.eps,
                               out_dtype=torch.float32)
    q, k, v, h = fra.fused_add_norm_qkv(d["x"], None, d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                        wl.head_dim, norm=norm, eps=wl.eps, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rg = oracle.gateup_act(inp["x"], None, inp["gamma"], None, norm, wl.eps, inp["w_gu"], None, None, wl.ffn,
                           "swiglu")
    rq = oracle.add_norm_qkv(inp["x"], None, inp["gamma"], None, norm, wl.eps, inp["w_qkv"], None, None,
                             wl.n_heads, wl.n_kv_heads, wl.head_dim)
    check("out", out, rg["out"])
    check("q", q, rq["q"])
    check("v", v, rq["v"])
    assert np.array_equal(h.double().cpu().numpy(), inp["x"].double().numpy())


@pytest.mark.parametrize("M", [300, 700])
def test_gemm16_head_major_and_down(M, forced):
    wl = small(M=M, hidden=512, ffn=1024, H=4, Hkv=2, D=64)
    forced(wl, down=True)
    inp = inputs.generate(wl, seed=14, parts=("qkv", "down"))
    d = to_dev(inp)
    plan = fra.describe_plan(M, wl.ffn, wl.hidden, torch.bfloat16, torch.bfloat16)
    assert plan["family"] == "gemm16"
    # the down projection reads its input as is: no row region in its workspace
    assert fra.down_workspace_bytes(M, wl.ffn, wl.hidden, torch.bfloat16, torch.bfloat16) == 0
    res = d["r"].clone()
    out = fra.fused_down_residual(d["a_down"], d["w_down"], res, out=res)
    out32 = fra.fused_down_residual(d["a_down"], d["w_down"], d["r"], out_dtype=torch.float32)
    q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                        wl.head_dim, head_major=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.down_residual(inp["a_down"], inp["w_down"], None, None, inp["r"])
    check("down", out, ref)
    check("down32", out32, ref)
    rq = oracle.workload_qkv(wl, inp)
    check("q", q, rq["q"].transpose(1, 0, 2))
    check("k", k, rq["k"].transpose(1, 0, 2))
    check("v", v, rq["v"].transpose(1, 0, 2))


def test_gemm16_against_128x512_kernel(forced, plan_override):
    """The same call through both prefill families: the normalised rows are the
    same values, so the outputs differ only by the order of the fp32 sums."""
    wl = small(M=640, hidden=1024, ffn=528, H=8, Hkv=2, D=64)
    d = to_dev(inputs.generate(wl, seed=15))
    forced(wl)
    a = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], d["w_gu"], wl.ffn, "swiglu", eps=wl.eps,
                             out_dtype=torch.float32).clone()
    fra.tune_clear()
    plan_override(no_gemm16=1)
    assert fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.bfloat16, "swiglu")["family"] == "prefill"
    b = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], d["w_gu"], wl.ffn, "swiglu", eps=wl.eps,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    diff = (a - b).abs().max().item()
    assert diff <= 1e-3 * max(1.0, b.abs().max().item()), diff


@pytest.mark.parametrize("stages", [2, 4, 5])
@pytest.mark.parametrize("name", ["llama2-7b-prefill", "gpt-fp16-gelu"])
def test_gemm16_full_size(name, stages, plan_override):
    plan_override(gemm16_stages=stages)
    wl = inputs.workload(name)
    act = TDT[wl.act]
    assert fra.describe_plan(wl.M, wl.hidden, wl.n_gu, act, act, wl.act_fn)["family"] == "gemm16"
    full_size_check(wl, seed=2)
