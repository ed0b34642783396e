"""The weight-streaming kernel's 32-row form through the C ABI against the
oracle.  In this form the four waves of a workgroup are two groups of 16
weight rows times the two halves of each K chunk, and the halves' fp32 sums
meet in LDS before the epilogue; the form takes 16-bit and E4M3 weights
without the gate/up pairing (the QKV call, the GELU / plain gate/up call) at
up to 32 tokens with hidden a multiple of 512.  It is requested through the
tuning table (rows = 32).

Cases: bf16, fp16 and E4M3 weights; ragged weight-row counts (a last tile of
16 rows); row-major and tile-packed weights; one whole tile per workgroup
(the planner's grid), each tile's K split over two workgroups, and a few
workgroups whose K ranges cross tile boundaries (partial sums between
workgroups, to which the second half's waves add zeros).  The halves only
reorder fp32 partial sums, so the tolerances of test_gpu_parity apply, and
the 32-row form on packed weights is the same sums as on row-major ones, bit
for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import TDT, check, run_gu, run_qkv, small, to_dev

pytestmark = pytest.mark.gpu
WDT = {"bf16": torch.bfloat16, "f16": torch.float16, "e4m3": torch.float8_e4m3fn}


@pytest.fixture
def khalves_table():
    def install(wl, rows=32):
        common = dict(m_lo=0, m_hi=64, act_dtype=TDT[wl.act], w_dtype=WDT[wl.wdt], family="stream", rows=rows)
        ents = [dict(common, hidden=wl.hidden, n_cols=wl.n_qkv, swiglu=False)]
        if wl.act_fn != "swiglu":
            ents.append(dict(common, hidden=wl.hidden, n_cols=wl.n_gu, swiglu=False))
        fra.tune_install(ents)
    yield install
    fra.tune_clear()


CASES = [
    dict(M=1, hidden=512, H=6, Hkv=2, D=64),                                      # 640 rows: 20 tiles
    dict(M=17, hidden=1024, H=10, Hkv=2, D=32, ffn=336, act_fn="gelu_tanh", bias=True),   # 448 / 336: ragged
    dict(M=32, hidden=2048, H=4, Hkv=2, D=64, ffn=272, act_fn="none"),
    dict(act="f16", M=9, hidden=512, norm="layer", act_fn="gelu_tanh", ffn=208, bias=True),
    dict(wdt="e4m3", M=5, hidden=1024, H=6, Hkv=1, D=64, ffn=176, act_fn="gelu_tanh"),
    dict(wdt="e4m3", act="f16", M=32, hidden=512, H=5, Hkv=1, D=48, ffn=80, act_fn="none", bias=True),
    dict(wdt="e4m3", M=20, hidden=1536, H=6, Hkv=2, D=64, norm="layer"),
]
ENVS = [{}, {"splits": 2}, {"stream_target": 7}]


def _kernels(wl):
    kw = dict(layout="rows")
    out = [fra.describe_plan(wl.M, wl.hidden, wl.n_qkv, TDT[wl.act], WDT[wl.wdt], **kw)]
    if wl.act_fn != "swiglu":
        out.append(fra.describe_plan(wl.M, wl.hidden, wl.n_gu, TDT[wl.act], WDT[wl.wdt], wl.act_fn, **kw))
    return out


@pytest.mark.parametrize("env", ENVS, ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()) or "planner")
@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_khalves_parity(cfg, env, plan_override, khalves_table):
    plan_override(**env)
    cfg = dict(cfg)
    wl = small(**cfg)
    khalves_table(wl)
    for p in _kernels(wl):
        print(f"khalves {cfg} {env}: {p['kernel']} grid={p['grid']} slots={p['slots']}", flush=True)
        assert p["kernel"].startswith("stream_kernel<") and ",n32,k512," in p["kernel"], p["kernel"]
        if "splits" in env and wl.hidden >= 1024:   # two chunks of 512 at least
            assert p["slots"] == 2
    inp = inputs.generate(wl, seed=23)
    d = to_dev(inp)
    q, k, v, h = run_qkv(wl, d, torch.float32)
    outs = [run_gu(wl, d, None)] if wl.act_fn != "swiglu" else []
    qn, kn, vn, _ = run_qkv(wl, d, None, write_h=False)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    for name, got in (("q", q), ("k", k), ("v", v), ("q native", qn), ("k native", kn), ("v native", vn)):
        check(name, got, rq[name[0]])
    assert np.array_equal(h.double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"
    if outs:
        check("out", outs[0], oracle.workload_gateup(wl, inp)["out"])


@pytest.mark.parametrize("cfg", [CASES[0], CASES[2], CASES[4], CASES[6]],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_khalves_packed(cfg, khalves_table):
    """Packed weights (a multiple of 128 rows) through the 32-row form: the
    same sums as on the row-major weights, bit for bit."""
    wl = small(**dict(cfg))
    if wl.n_qkv % 128:
        pytest.skip("tile-packed weights need a multiple of 128 rows")
    khalves_table(wl)
    d = to_dev(inputs.generate(wl, seed=29))
    pw = fra.pack_weight(d["w_qkv"])
    p = fra.describe_plan(wl.M, wl.hidden, wl.n_qkv, TDT[wl.act], WDT[wl.wdt], layout="packed")
    print(f"khalves packed {cfg}: {p['kernel']} grid={p['grid']}", flush=True)
    assert ",n32,k512," in p["kernel"]
    ref = run_qkv(wl, d, torch.float32, write_h=False)
    got = run_qkv(wl, dict(d, w_qkv=pw), torch.float32, write_h=False)
    torch.cuda.synchronize()
    for a, b in zip(ref[:3], got[:3]):
        assert torch.equal(a, b)


def test_khalves_matches_64_rows(khalves_table):
    """The 32-row form against the 64-row form of the same call: the same
    products, summed in another order (fp32), so equal within rounding."""
    wl = small(M=16, hidden=4096, H=32, Hkv=8, D=128)
    d = to_dev(inputs.generate(wl, seed=31))
    res = {}
    for rows in (32, 64):
        khalves_table(wl, rows=rows)
        p = fra.describe_plan(wl.M, wl.hidden, wl.n_qkv, TDT[wl.act], WDT[wl.wdt])
        print(f"khalves rows={rows}: {p['kernel']} grid={p['grid']} slots={p['slots']}", flush=True)
        assert f",n{rows}," in p["kernel"]
        res[rows] = run_qkv(wl, d, torch.float32, write_h=False)
    torch.cuda.synchronize()
    for a, b in zip(res[32][:3], res[64][:3]):
        err = (a - b).abs().max().item()
        assert err <= 1e-4 * max(1.0, b.abs().max().item()), err
