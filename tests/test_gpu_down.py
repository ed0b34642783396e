"""The down projection with the residual add in its epilogue
(fused_down_residual) against the oracle: every kernel family, weight dtype
and output dtype, with and without residual and bias, the residual stream
updated in place, and the down projections of the workloads at full size on
sampled token rows.  Tolerances as in test_gpu_parity.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, check, small, tile_rows, to_dev, _sample_rows

pytestmark = pytest.mark.gpu


def _run(d, native, bias=None, in_place=False, out=None):
    odt = None if native else torch.float32
    if in_place:
        res = d["r_down"].clone()
        out = fra.fused_down_residual(d["a_down"], d["w_down"], res, w_scale=d.get("s_down"), bias=bias, out=res)
        assert out.data_ptr() == res.data_ptr()
        return out
    return fra.fused_down_residual(d["a_down"], d["w_down"], d.get("r_down"), w_scale=d.get("s_down"),
                                   bias=bias, out_dtype=odt, out=out)


def _inputs(wl, seed, residual=True):
    inp = inputs.generate(wl, seed=seed, parts=("down",))
    if residual:
        # the residual stream the down projection adds to: [M, hidden]
        inp["r_down"] = inp["r"]
    return inp


DOWN = [
    dict(M=1, hidden=320, ffn=512), dict(M=20, hidden=512, ffn=1024), dict(M=64, hidden=256, ffn=768),
    dict(M=8, hidden=256, ffn=320),                         # ffn not a multiple of 256: tiled kernel
    dict(M=100, hidden=512, ffn=512), dict(M=300, hidden=320, ffn=1024),   # 128 x 512 kernel
    dict(act="f32", M=5, hidden=256, ffn=256), dict(act="f32", M=130, hidden=128, ffn=192),
    dict(act="f16", M=40, hidden=512, ffn=512),
    dict(wdt="i8", M=16, hidden=512, ffn=1024), dict(wdt="i8", M=200, hidden=256, ffn=512),
    dict(wdt="i4", M=16, hidden=512, ffn=1024), dict(wdt="i4", M=150, hidden=256, ffn=512),
]


@pytest.mark.parametrize("cfg", DOWN, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("mode", ["f32out", "nativeout", "bias", "noresidual", "inplace"])
def test_down_residual(cfg, mode):
    if cfg.get("act") == "f32" and mode == "nativeout":
        pytest.skip("fp32 activations: the native output is the fp32 output")
    wl = small(**cfg)
    inp = _inputs(wl, seed=12, residual=mode != "noresidual")
    d = to_dev(inp)
    bias = None
    if mode == "bias":
        bias = inputs._to_act(np.random.default_rng(2).standard_normal(wl.hidden).astype(np.float32)
                              * np.float32(0.1), wl.act)
    plan = fra.describe_plan(wl.M, wl.ffn, wl.hidden, d["a_down"].dtype, d["w_down"].dtype)
    print(f"down {wl.name} ffn={wl.ffn} hidden={wl.hidden} {mode}: {plan['kernel']}", flush=True)
    out = _run(d, mode in ("nativeout", "inplace"), None if bias is None else bias.to(DEV), mode == "inplace")
    torch.cuda.synchronize()
    ref = oracle.down_residual(inp["a_down"], inp["w_down"], inp.get("s_down"), bias, inp.get("r_down"))
    check("out", out, ref)


def test_down_rejects_partial_overlap():
    wl = small(M=16, hidden=256, ffn=512)
    d = to_dev(_inputs(wl, seed=13))
    big = torch.empty(16 * 256 + 64, dtype=torch.bfloat16, device=DEV)
    res = big[:16 * 256].view(16, 256)
    res.copy_(d["r_down"])
    out = big[64:].view(16, 256)               # shifted by 64 elements: overlaps, not in place
    with pytest.raises(fra.FusedProjError):
        fra.fused_down_residual(d["a_down"], d["w_down"], res, out=out)
    with pytest.raises(fra.FusedProjError):    # writing over the input
        fra.fused_down_residual(d["a_down"], d["w_down"], d["r_down"], out=d["a_down"].view(-1)[:16 * 256].view(16, 256))


@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("name", ["llama3-8b-decode", "llama2-7b-prefill", "llama2-70b-int8w@M16",
                                  "llama2-70b-int4w@M16"])
def test_down_workload_full_size(name, seed):
    wl = inputs.workload(name)
    print(f"down {name} seed {seed}: generating", flush=True)
    inp = _inputs(wl, seed=seed)
    d = to_dev(inp)
    rows = tile_rows(wl.M, seed)
    got = {}
    for native in (False, True):
        o = torch.full((wl.M, wl.hidden), float("nan"), dtype=torch.float32 if not native else d["a_down"].dtype,
                       device=DEV)
        _run(d, native, out=o)
        assert bool(torch.isfinite(o).all()), f"down {name}: unwritten or non-finite elements"
        got[native] = o[torch.from_numpy(rows).to(DEV)].cpu()
    torch.cuda.synchronize()
    print(f"down {name}: oracle on {len(rows)} rows", flush=True)
    idx = torch.as_tensor(rows, dtype=torch.long)
    ref = oracle.down_residual(inp["a_down"][idx].contiguous(), inp["w_down"], inp.get("s_down"), None,
                               inp["r_down"][idx].contiguous())
    for native in (False, True):
        print(name, native, check("out", got[native], ref), flush=True)
