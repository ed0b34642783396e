"""The allocation-free QKV call (fused_add_norm_qkv_noalloc, static device
scratch) against the workspace call it varies (fused_add_norm_qkv) and the
oracle: two calls in a row on one device, the second with a smaller input,
each checked bit for bit against the workspace call's outputs and to the
parity bounds against the oracle.  The first shape splits its 96 weight
tiles of 64 rows between workgroups (64 rows requested: the planner's own
choice for it, 32-row tiles with K halves, gives every workgroup a whole
tile), so the partial sums and arrival counters in the scratch are
exercised; the second reuses the scratch the first left behind.  The
planner's 32-row form is checked against the workspace call as well.
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, check, small, to_dev

pytestmark = pytest.mark.gpu


def _noalloc_vs_workspace(wl, seed, out_dtype):
    inp = inputs.generate(wl, seed=seed, parts=("qkv",))
    d = to_dev(inp)
    M = wl.M
    print(f"noalloc {wl.name} M={M} hidden={wl.hidden} out={out_dtype}: "
          f"{fra.describe_plan(M, wl.hidden, wl.n_qkv, d['x'].dtype, d['w_qkv'].dtype)}", flush=True)
    q = torch.full((M, wl.n_heads, wl.head_dim), float("nan"), dtype=out_dtype, device=DEV)
    k = torch.full((M, wl.n_kv_heads, wl.head_dim), float("nan"), dtype=out_dtype, device=DEV)
    v = torch.full_like(k, float("nan"))
    h = torch.full_like(d["x"], float("nan"))
    kw = dict(beta=d.get("beta"), norm=wl.norm, eps=wl.eps, w_scale=d.get("s_qkv"))
    fra.fused_add_norm_qkv_noalloc(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads, wl.head_dim,
                                   q=q, k=k, v=v, h_out=h, **kw)
    rq, rk, rv, rh = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                            wl.head_dim, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    for name, a, b in (("q", q, rq), ("k", k, rk), ("v", v, rv), ("h_out", h, rh)):
        assert torch.equal(a.view(torch.uint8), b.contiguous().view(torch.uint8)), f"{name} differs from the workspace call"
    ref = oracle.workload_qkv(wl, inp)
    check("q", q, ref["q"])
    check("k", k, ref["k"])
    check("v", v, ref["v"])
    assert np.array_equal(h.double().cpu().numpy(), ref["h_out"])


def test_noalloc_two_calls_second_smaller(plan_override):
    plan_override(stream_nr=1)
    big = inputs.workload("llama3-8b-decode")                     # 32 tokens, 96 shared tiles
    assert fra.describe_plan(big.M, big.hidden, big.n_qkv, torch.bfloat16, torch.bfloat16)["slots"] > 1
    _noalloc_vs_workspace(big, seed=0, out_dtype=torch.float32)
    smaller = small(M=5, hidden=1024, H=8, Hkv=2, D=64)             # fewer tokens, narrower rows
    _noalloc_vs_workspace(smaller, seed=1, out_dtype=torch.bfloat16)


def test_noalloc_khalves():
    big = inputs.workload("llama3-8b-decode")
    p = fra.describe_plan(big.M, big.hidden, big.n_qkv, torch.bfloat16, torch.bfloat16)
    assert ",n32," in p["kernel"] and p["slots"] == 1, p
    _noalloc_vs_workspace(big, seed=2, out_dtype=torch.bfloat16)


def test_noalloc_rejects_beyond_the_scratch():
    wl = inputs.workload("llama2-70b-int8w@M256")
    need = fra.workspace_bytes(wl.M, wl.hidden, wl.n_qkv, torch.bfloat16, torch.int8)
    assert need > fra.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((wl.M, wl.hidden), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((wl.n_qkv, wl.hidden), dtype=torch.int8, device=DEV)
    s = torch.ones(wl.n_qkv, dtype=torch.float32, device=DEV)
    q = torch.empty((wl.M, wl.n_heads, wl.head_dim), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((wl.M, wl.n_kv_heads, wl.head_dim), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fra.FusedProjError) as ei:
        fra.fused_add_norm_qkv_noalloc(x, None, torch.ones(wl.hidden, dtype=torch.bfloat16, device=DEV), w,
                                       wl.n_heads, wl.n_kv_heads, wl.head_dim, q=q, k=k, v=torch.empty_like(k),
                                       w_scale=s)
    assert ei.value.status == 7 and "static scratch" in str(ei.value)   # FP_E_WORKSPACE
