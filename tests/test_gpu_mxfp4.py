"""MXFP4 weights (E2M1 codes, one E8M0 scale per row and 32 k; bf16
activations) through the C ABI against the oracle.

The weight-streaming kernel (decode token counts, hidden a multiple of 256)
and the 128 x 512 kernel (more than 64 tokens) dequantise the weights in
registers with the hardware's scaled FP4 conversion; the tiled kernel's
calls dequantise them into the workspace first.  Checked: the dequantisation
bits of every code at every scale (the same device function as the weight
loaders), every kernel family with both calls and fp32 / bf16 outputs, the
256-row streaming form and K splits, the down projection, head-major q / k /
v and the Llama-2-70B layer at full size; tolerances as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, check, full_size_check, run_gu, run_qkv, small, to_dev

pytestmark = pytest.mark.gpu

MX = torch.float4_e2m1fn_x2


def test_dequant_mxfp4_every_code_and_scale():
    # row j: scale j on its first 32 k, 254 - j on the next 32; element k code k % 16
    N, K = 255, 64
    codes = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    scales = np.stack([np.arange(255), 254 - np.arange(255)], 1).astype(np.uint8)
    q = torch.from_numpy(codes[:, 0::2] | (codes[:, 1::2] << 4)).view(MX)
    s = torch.from_numpy(scales).view(torch.float8_e8m0fnu)
    got = fra.fused_dequant_mxfp4_bf16(q.to(DEV), s.to(DEV))
    torch.cuda.synchronize()
    _, bits = oracle.dequant_mxfp4(q, s)
    g = got.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(g != bits)
    assert len(bad) == 0, f"{len(bad)} mismatches, first (row, k) {bad[:4].tolist()}: " \
                          f"got {[hex(g[i, j]) for i, j in bad[:4]]} want {[hex(bits[i, j]) for i, j in bad[:4]]}"


def test_dequant_mxfp4_random_weights():
    wl = small(wdt="mxfp4", M=1, hidden=1024, ffn=400)
    inp = inputs.generate(wl, seed=9, parts=("gu",))
    got = fra.fused_dequant_mxfp4_bf16(inp["w_gu"].to(DEV), inp["s_gu"].to(DEV))
    torch.cuda.synchronize()
    _, bits = oracle.dequant_mxfp4(inp["w_gu"], inp["s_gu"])
    assert np.array_equal(got.cpu().view(torch.int16).numpy().view(np.uint16), bits)


MXFP4 = [
    dict(M=1, hidden=512), dict(M=5, hidden=768, ffn=208), dict(M=17, hidden=1024, H=8, Hkv=2, D=64),
    dict(M=32, hidden=512), dict(M=40, hidden=768), dict(M=64, hidden=1024, ffn=336),
    dict(M=3, hidden=320),                       # hidden not a multiple of 256: staged, tiled kernel
    dict(M=100, hidden=512), dict(M=300, hidden=1024, ffn=400),   # 128 x 512 kernel
    dict(M=257, hidden=320, ffn=208, act_fn="none", bias=True),
    dict(M=9, hidden=512, act_fn="none", bias=True, ffn=144),
    dict(M=70, hidden=768, norm="layer", act_fn="gelu_tanh", bias=True, ffn=272),
]


@pytest.mark.parametrize("cfg", MXFP4, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("native", [False, True], ids=["f32out", "nativeout"])
def test_mxfp4_small(cfg, native):
    cfg = dict(cfg)
    bias = cfg.pop("bias", False)
    wl = small(wdt="mxfp4", bias=bias, **cfg)
    inp = inputs.generate(wl, seed=6)
    if bias:
        inp["b_qkv"] = inputs._to_act(np.random.default_rng(9).standard_normal(wl.n_qkv).astype(np.float32)
                                      * np.float32(0.1), wl.act)
    d = to_dev(inp)
    odt = None if native else torch.float32
    plan = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, MX, wl.act_fn)
    print(f"mxfp4 {wl.name} {plan['kernel']} {plan.get('prep', '')} native={native}", flush=True)
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


@pytest.mark.parametrize("ov", [{"stream_nr": 4}, {"stream_nr": 4, "splits": 3}, {"splits": 5},
                                {"no_stream": 1, "splits": 3}, {"no_stream": 1, "no_prefill": 1}],
                         ids=lambda e: ",".join(f"{k}={v}" for k, v in e.items()))
@pytest.mark.parametrize("M", [1, 20, 48, 130])
def test_mxfp4_launch_configs(ov, M, plan_override):
    plan_override(**ov)
    wl = small(wdt="mxfp4", M=M, hidden=1024, H=10, Hkv=2, D=32, ffn=464)
    inp = inputs.generate(wl, seed=17)
    d = to_dev(inp)
    print(f"mxfp4 configs {ov} M={M}: "
          f"{fra.describe_plan(M, wl.hidden, wl.n_gu, torch.bfloat16, MX, wl.act_fn)['kernel']}", flush=True)
    q, k, v, h = run_qkv(wl, d, torch.float32)
    out = run_gu(wl, d, torch.float32)
    torch.cuda.synchronize()
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])


@pytest.mark.parametrize("M", [16, 200])
def test_mxfp4_down_and_head_major(M):
    wl = small(wdt="mxfp4", M=M, hidden=512, ffn=1024, H=4, Hkv=2, D=64)
    inp = inputs.generate(wl, seed=21, parts=("qkv", "down"))
    d = to_dev(inp)
    res = d["r"].clone()
    out = fra.fused_down_residual(d["a_down"], d["w_down"], res, w_scale=d["s_down"], out=res)
    q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                        wl.head_dim, w_scale=d["s_qkv"], head_major=True,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.down_residual(inp["a_down"], inp["w_down"], inp["s_down"], None, inp["r"])
    check("down", out, ref)
    rq = oracle.workload_qkv(wl, inp)
    check("q", q, rq["q"].transpose(1, 0, 2))
    check("v", v, rq["v"].transpose(1, 0, 2))


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", ["llama2-70b-mxfp4w@M1", "llama2-70b-mxfp4w@M16", "llama2-70b-mxfp4w@M64",
                                  "llama2-70b-mxfp4w@M256"])
def test_mxfp4_workload_full_size(name, seed):
    full_size_check(inputs.workload(name), seed)
