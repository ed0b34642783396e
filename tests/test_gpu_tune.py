"""The tuning table and the micro-benchmark autotuner on the GPU.

Every candidate configuration the tuner can install for a shape (kernel
family, rows per workgroup, workgroup count, K split; including the 128 x 512
kernel at decode token counts and the tiled kernel at any count; the K split
of the FP8 kernel) must give
results within the parity bounds against the oracle; the tuner itself must
time the candidates and return a valid entry or keep the planner's choice.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs, tune

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _wl(M, wdt="bf16", act_fn="swiglu"):
    return inputs.Workload(
        name=f"tune-{M}-{wdt}", M=M, hidden=1024, act="bf16", wdt=wdt, norm="rms", eps=1e-5,
        x_std=1.0, r_std=1.0, gamma_lo=0.5, gamma_hi=1.5, beta_std=None, w_std=0.05, n_heads=8,
        n_kv_heads=2, head_dim=64, ffn=336, act_fn=act_fn, bias_std=None)


def _check(name, got, ref):
    g = got.detach().double().cpu().numpy().reshape(ref.shape)
    err = np.abs(g - ref)
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= 5e-3 and err.max() <= 2e-2, f"{name}: max-abs {err.max():.3e} rel-fro {rel:.3e}"


@pytest.mark.parametrize("M,wdt", [(5, "bf16"), (40, "i8"), (100, "bf16"), (5, "e4m3"), (100, "e4m3")])
def test_every_candidate_meets_parity(M, wdt):
    wl = _wl(M, wdt)
    inp = inputs.generate(wl, seed=4)
    d = {k: v.to(DEV) for k, v in inp.items()}
    rq = oracle.workload_qkv(wl, inp)
    rg = oracle.workload_gateup(wl, inp)
    act, w = torch.bfloat16, d["w_qkv"].dtype
    try:
        for call, n_cols, swiglu in (("qkv", d["w_qkv"].shape[0], False), ("gu", d["w_gu"].shape[0], True)):
            for cand in tune.candidates(M, wl.hidden, n_cols, act, w, swiglu):
                cfg = {k: v for k, v in cand.items() if k != "plan"}
                fra.tune_install([tune._entry(M, M, wl.hidden, n_cols, act, w, swiglu, cfg)] if cfg else [])
                print(f"M={M} {wdt} {call}: {cand['plan']['kernel']} grid {cand['plan']['grid']} "
                      f"splits {cand['plan']['splits']}", flush=True)
                if call == "qkv":
                    q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads,
                                                        wl.n_kv_heads, wl.head_dim, norm="rms", eps=wl.eps,
                                                        w_scale=d.get("s_qkv"), out_dtype=torch.float32)
                    torch.cuda.synchronize()
                    _check("q", q, rq["q"])
                    _check("k", k, rq["k"])
                    _check("v", v, rq["v"])
                    assert np.array_equal(h.double().cpu().numpy(), rq["h_out"])
                else:
                    out = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], d["w_gu"], wl.ffn, "swiglu",
                                               norm="rms", eps=wl.eps, w_scale=d.get("s_gu"),
                                               out_dtype=torch.float32)
                    torch.cuda.synchronize()
                    _check("out", out, rg["out"])
    finally:
        fra.tune_clear()


def test_tuner_times_candidates_and_returns_an_entry_or_none():
    wl = _wl(24)
    r = tune.tune_call(wl, "gu", reps=3, rounds=2, log=lambda s: print(s, flush=True))
    assert r["default_us"] > 0 and len(r["results"]) >= 5
    assert all(us > 0 for _, us in r["results"])
    e = r["entry"]
    if e is not None:
        fra.tune_install([e])
        try:
            assert fra.tune_count() == 1
        finally:
            fra.tune_clear()
    assert fra.tune_count() == 0


def test_tuner_fp8_splits():
    # E4M3 weights: the FP8 GEMM tiles at every K split and the
    # weight-streaming kernel on the codes at several grids, all checked
    # against the planner's result inside tune_call
    wl = _wl(24, "e4m3")
    r = tune.tune_call(wl, "gu", reps=3, rounds=2, log=lambda s: print(s, flush=True))
    assert r["default_us"] > 0 and len(r["results"]) >= 3
    kernels = {c["kernel"].split("<")[0] for c, _ in r["results"]}
    assert kernels == {"gemm8_kernel", "stream_kernel"}, kernels
    assert fra.tune_count() == 0

