"""int4 group-wise weights (4-bit weights, 16-bit activations, one scale per
row and group of 128 k, no zero point) through the C ABI against the oracle.

The weight-streaming kernel (decode token counts, hidden a multiple of 256)
and the 128 x 512 kernel (more than 64 tokens) dequantise the weights in
registers; the tiled kernel's calls dequantise them into the workspace and
run the bf16 kernel.  Both paths, both calls,
fp32 and bf16 outputs, the 256-row streaming form, and the dequantisation
bits (the same device function in both paths) are checked; tolerances as in
test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, check, full_size_check, run_gu, run_qkv, small, to_dev, _sample_rows

pytestmark = pytest.mark.gpu


def test_dequant_i4_bits():
    rng = np.random.default_rng(5)
    N, K = 300, 1024
    q = torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8))
    s = rng.uniform(1e-4, 1e-2, (N, K // 128)).astype(np.float32)
    s[0, :] = 0.0
    s[1, :] = 1.0
    s[2, 0] = 2.0 ** -7
    s = torch.from_numpy(s)
    got = fra.fused_dequant_i4_bf16(q.to(DEV), s.to(DEV))
    torch.cuda.synchronize()
    _, bits = oracle.dequant_i4(q, s)
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), bits)


INT4 = [
    dict(M=1, hidden=512), dict(M=5, hidden=768, ffn=208), dict(M=17, hidden=1024, H=8, Hkv=2, D=64),
    dict(M=32, hidden=512), dict(M=40, hidden=768), dict(M=64, hidden=1024, ffn=336),
    dict(M=3, hidden=384),                       # hidden not a multiple of 256: staged, tiled kernel
    dict(M=100, hidden=512), dict(M=300, hidden=1024, ffn=400),   # 128 x 512 kernel
    dict(M=257, hidden=384, ffn=208, act_fn="none", bias=True),
    dict(M=9, hidden=512, act_fn="none", bias=True, ffn=144),
]


@pytest.mark.parametrize("cfg", INT4, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("native", [False, True], ids=["f32out", "nativeout"])
def test_int4_small(cfg, native):
    cfg = dict(cfg)
    bias = cfg.pop("bias", False)
    wl = small(wdt="i4", bias=bias, **cfg)
    inp = inputs.generate(wl, seed=6)
    d = to_dev(inp)
    odt = None if native else torch.float32
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.uint8, wl.act_fn)
    print(f"int4 {wl.name} {plan['kernel']} {plan.get('prep', '')} native={native}", flush=True)
    stream = wl.M <= 64 and wl.hidden % 256 == 0
    assert (plan["family"] == "stream") == stream
    assert ("dequant" in plan.get("prep", "")) == (plan["family"] == "tiled")   # staged only for the tiled kernel
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


@pytest.mark.parametrize("env", [{"stream_nr": 4}, {"stream_nr": 4, "splits": 3},
                                 {"no_stream": 1, "splits": 3}],
                         ids=lambda e: ",".join(f"{k[10:]}={v}" for k, v in e.items()))
@pytest.mark.parametrize("M", [1, 48])
def test_int4_256_rows(env, M, plan_override):
    plan_override(**env)
    wl = small(wdt="i4", M=M, hidden=1024, H=10, Hkv=2, D=32, ffn=464)
    inp = inputs.generate(wl, seed=7)
    d = to_dev(inp)
    print(f"int4 256-row stream {env} M={M}", flush=True)
    q, k, v, h = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", ["llama2-70b-int4w@M1", "llama2-70b-int4w@M16", "llama2-70b-int4w@M256"])
def test_int4_workload_full_size(name, seed):
    full_size_check(inputs.workload(name), seed)


@pytest.mark.parametrize("splits", ["1", "2", "3", "5"])
def test_int4_prefill_splits(splits, plan_override):
    """The 128 x 512 kernel's int4 path with K split (group scales per stage of each split)."""
    plan_override(splits=int(splits))
    wl = small(wdt="i4", M=200, hidden=1024, H=8, Hkv=2, D=64, ffn=336)
    inp = inputs.generate(wl, seed=8)
    d = to_dev(inp)
    print(f"int4 prefill splits={splits}", flush=True)
    q, k, v, h = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("k", k, rq["k"])
    check("out", out, rg["out"])
