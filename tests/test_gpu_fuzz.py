"""Seeded random configurations against the oracle: token counts, widths,
head layouts, dtypes (bf16, fp16, fp32, int8, int4 and E4M3 weights), norms,
epilogues, bias, residual and output dtype drawn at random (fixed seeds), so
that combinations no hand-written case names still meet the parity bounds.
Each case prints its configuration before running."""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import check, run_gu, run_qkv, small, to_dev

pytestmark = pytest.mark.gpu


def _config(seed):
    rng = np.random.default_rng(1000 + seed)
    kind = str(rng.choice(["bf16", "bf16", "f16", "f32", "i8", "i4"]))
    act = "bf16" if kind in ("i8", "i4") else kind
    wdt = kind if kind in ("i8", "i4") else None
    step = 128 if kind == "i4" else 64
    # half the time a multiple of 256 (the streaming kernel's K granularity)
    hidden = int(rng.choice([rng.integers(1, 9) * 256, rng.integers(1, 17) * step]))
    M = int(rng.choice([rng.integers(1, 65), rng.integers(65, 400)]))
    Hkv = int(rng.integers(1, 5))
    H = Hkv * int(rng.integers(1, 5))
    D = 16 * int(rng.integers(1, 9))
    ffn = 16 * int(rng.integers(1, 40))
    norm = str(rng.choice(["rms", "rms", "layer", "none"]))
    act_fn = str(rng.choice(["swiglu", "swiglu", "gelu_tanh", "none"]))
    bias = bool(rng.integers(0, 2))
    native = bool(rng.integers(0, 2)) and act != "f32"
    return dict(act=act, wdt=wdt, M=M, hidden=hidden, H=H, Hkv=Hkv, D=D, ffn=ffn, norm=norm, act_fn=act_fn,
                bias=bias), native


@pytest.mark.parametrize("seed", range(48))
def test_random_configuration(seed):
    _run_case(seed, *_config(seed))


def _config_fp8(seed):
    rng = np.random.default_rng(2000 + seed)
    act = str(rng.choice(["bf16", "bf16", "f16"]))
    hidden = 128 * int(rng.integers(1, 33))
    M = int(rng.choice([rng.integers(1, 65), rng.integers(65, 600)]))
    Hkv = int(rng.integers(1, 5))
    H = Hkv * int(rng.integers(1, 5))
    D = 16 * int(rng.integers(1, 9))
    ffn = 16 * int(rng.integers(1, 40))
    norm = str(rng.choice(["rms", "rms", "layer", "none"]))
    act_fn = str(rng.choice(["swiglu", "swiglu", "gelu_tanh", "none"]))
    bias = bool(rng.integers(0, 2))
    native = bool(rng.integers(0, 2))
    return dict(act=act, wdt="e4m3", M=M, hidden=hidden, H=H, Hkv=Hkv, D=D, ffn=ffn, norm=norm, act_fn=act_fn,
                bias=bias), native


# E4M3 weights with per-token E4M3 activations (FP8 W8A8), 24 more seeds
@pytest.mark.parametrize("seed", range(24))
def test_random_fp8_configuration(seed):
    _run_case(seed, *_config_fp8(seed))


def _run_case(seed, cfg, native):
    wl = small(**cfg)
    inp = inputs.generate(wl, seed=seed)
    if cfg["bias"]:
        inp["b_qkv"] = inputs._to_act(np.random.default_rng(seed).standard_normal(wl.n_qkv).astype(np.float32)
                                      * np.float32(0.1), wl.act)
    d = to_dev(inp)
    plans = [fra.describe_plan(wl.M, wl.hidden, n, d["x"].dtype, d["w_qkv"].dtype, a)["kernel"]
             for n, a in ((wl.n_qkv, "none"), (wl.n_gu, wl.act_fn))]
    print(f"seed {seed}: {cfg} native={native} kernels={plans}", flush=True)
    odt = None if native else torch.float32
    q, k, v, h = run_qkv(wl, d, odt)
    out = run_gu(wl, d, odt)
    torch.cuda.synchronize()
    rq = oracle.add_norm_qkv(inp["x"], inp["r"], inp["gamma"], inp.get("beta"), wl.norm, wl.eps,
                             inp["w_qkv"], inp.get("s_qkv"), inp.get("b_qkv"), wl.n_heads, wl.n_kv_heads,
                             wl.head_dim)
    rg = oracle.workload_gateup(wl, inp)
    check("q", q, rq["q"])
    check("k", k, rq["k"])
    check("v", v, rq["v"])
    check("out", out, rg["out"])
    assert np.array_equal(h.double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"
