"""The weight-streaming kernel's own row pass through the C ABI.

At decode token counts the rows the streaming kernel multiplies (h = x +
residual, normalised, rounded to the activation dtype) are formed either by a
row-pass launch before the kernel, or by the kernel itself: its first M
workgroups each form one token row while every workgroup's first weights are
in flight, publish it with a per-launch tag, and every workgroup waits for
all M rows before it reads them.  Both forms run the same row arithmetic and
the same streaming kernel on the same rows, so their outputs and h_out must be
identical, bit for bit; the rows also reach the oracle's parity bounds (the
full-size workloads of test_gpu_parity take this form by default).

Cases: bf16 / fp16 / int8 / int4 / MXFP4 weights; QKV (with h_out), SwiGLU,
tanh-GELU and plain epilogues; RMSNorm, LayerNorm with and without beta, no
norm with a residual; 1 .. 64 tokens; hidden up to 8192; row-major and
tile-packed weights; consecutive calls on one workspace (flags of earlier
launches left in it) without synchronising between them; the bounded wait,
forced from the host (every wait expires: NaN outputs, the launch ends).
"""
import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs
from test_gpu_parity import DEV, TDT, check, run_gu, run_qkv, small, to_dev

pytestmark = pytest.mark.gpu
WDT = {"bf16": torch.bfloat16, "f16": torch.float16, "i8": torch.int8, "i4": torch.uint8, "mxfp4": torch.uint8}

CASES = [
    dict(M=1, hidden=512),
    dict(M=5, hidden=1024, act_fn="gelu_tanh", bias=True, ffn=272),
    dict(M=17, hidden=2048, norm="layer", H=8, Hkv=2, D=64),
    dict(M=32, hidden=4096, H=32, Hkv=8, D=128, ffn=512),
    dict(M=33, hidden=1024, H=32, Hkv=8, D=128, act_fn="none", ffn=4096),
    dict(M=64, hidden=768, norm="layer", act="f16", H=16, Hkv=16, D=128, act_fn="gelu_tanh", bias=True, ffn=8192),
    dict(M=16, hidden=8192, H=8, Hkv=1, D=128, ffn=256),
    dict(M=9, hidden=512, wdt="i8", H=16, Hkv=4, D=128, ffn=2048),
    dict(M=64, hidden=1024, wdt="i8", norm="layer", H=32, Hkv=8, D=128, ffn=4096),
    dict(M=3, hidden=1024, wdt="i4", ffn=256),
    dict(M=24, hidden=2048, wdt="mxfp4", H=16, Hkv=4, D=128, ffn=2048),
    dict(M=12, hidden=512, norm="none", H=16, Hkv=4, D=64, ffn=1024),
]


def _wl(cfg):
    cfg = dict(cfg)
    bias = cfg.pop("bias", False)
    return small(bias=bias, **cfg)


def _layout(w):
    return w.layout if isinstance(w, fra.PackedWeight) else "rows"


def _both(wl, d, plan_override, out_dtype=torch.float32):
    """The two calls with the separate row pass, then with the kernel's own."""
    res = {}
    for own in (False, True):
        plan_override(no_stream_rows=0 if own else 1)
        pq = fra.describe_plan(wl.M, wl.hidden, wl.n_qkv, TDT[wl.act], d["w_qkv"].dtype,
                               layout=_layout(d["w_qkv"]))
        pg = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, TDT[wl.act], d["w_gu"].dtype, wl.act_fn,
                               layout=_layout(d["w_gu"]))
        print(f"rows own={own}: qkv {pq['kernel']} grid={pq['grid']} {pq.get('prep', '')}; "
              f"gu {pg['kernel']} grid={pg['grid']} {pg.get('prep', '')}", flush=True)
        for p in (pq, pg):
            assert p["family"] == "stream", p
            if own and p["grid"] + wl.M <= 256:   # M more workgroups fit: the kernel's own rows
                assert p["kernel"].endswith(",rows>") and "prep" not in p, p
            else:
                assert p["prep"].startswith("norm_kernel"), p
        if own:
            assert pq["kernel"].endswith(",rows>") or pg["kernel"].endswith(",rows>"), "no call takes the form"

        q, k, v, h = run_qkv(wl, d, out_dtype)
        out = run_gu(wl, d, out_dtype)
        res[own] = (q, k, v, h, out)
    torch.cuda.synchronize()
    return res[False], res[True]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_rows_in_kernel_matches_row_pass(cfg, plan_override):
    wl = _wl(cfg)
    inp = inputs.generate(wl, seed=41)
    if wl.norm == "layer" and wl.M % 2:   # LayerNorm without beta
        del inp["beta"]
    d = to_dev(inp)
    if wl.norm == "none":
        d["gamma"] = None
    sep, own = _both(wl, d, plan_override)
    for name, a, b in zip(("q", "k", "v", "h_out", "out"), sep, own):
        assert torch.equal(a, b), f"{name}: the kernel's own rows differ from the row pass"
    # and the oracle's bounds
    rq, rg = oracle.workload_qkv(wl, inp), oracle.workload_gateup(wl, inp)
    for name, got in zip("qkv", own[:3]):
        check(name, got, rq[name])
    assert np.array_equal(own[3].double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"
    check("out", own[4], rg["out"])


@pytest.mark.parametrize("cfg", [CASES[3], CASES[8], CASES[10]],
                         ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_rows_in_kernel_packed(cfg, plan_override):
    """Tile-packed weights: the kernel's own rows, the same outputs as the
    row pass on the same packed weights."""
    wl = _wl(cfg)
    d = to_dev(inputs.generate(wl, seed=43))
    if wl.n_qkv % 128 or wl.ffn % 64:
        pytest.skip("tile-packed weights need whole 128-row groups")
    d["w_qkv"] = fra.pack_weight(d["w_qkv"])
    d["w_gu"] = fra.pack_weight(d["w_gu"], gate_up=wl.act_fn == "swiglu")
    res = {}
    for own in (False, True):
        plan_override(no_stream_rows=0 if own else 1)
        res[own] = (*run_qkv(wl, d, None), run_gu(wl, d, None))
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "k", "v", "h_out", "out"), res[False], res[True]):
        assert torch.equal(a, b), name


@pytest.mark.parametrize("cfg", [dict(M=32, hidden=4096, H=32, Hkv=8, D=128, ffn=512),
                                 dict(M=32, hidden=512, H=4, Hkv=2, D=64, ffn=256)],
                         ids=["large", "l2-resident"])
def test_rows_in_kernel_consecutive_calls_one_workspace(cfg, plan_override):
    """Four calls on one workspace, back to back without synchronising: each
    launch waits for its own rows (a new tag), never for the flags an
    earlier launch left, so every result equals the separate row pass's.
    The second shape's weights, rows and flags (under 1 MB) all stay in the
    XCDs' L2s from one call to the next, so a row line that an earlier launch
    left in an L2 would be read stale by a later one."""
    wl = _wl(cfg)
    ins = [to_dev(inputs.generate(wl, seed=s)) for s in (51, 52, 53, 54)]
    plan_override(no_stream_rows=1)
    ref = [(*run_qkv(wl, d, None), run_gu(wl, d, None)) for d in ins]
    torch.cuda.synchronize()
    plan_override(no_stream_rows=0)
    need = max(fra.workspace_bytes(wl.M, wl.hidden, wl.n_qkv, torch.bfloat16, torch.bfloat16),
               fra.workspace_bytes(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.bfloat16))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    got = []
    for d in ins:
        q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                            wl.head_dim, eps=wl.eps, workspace=ws)
        out = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], d["w_gu"], wl.ffn, wl.act_fn, eps=wl.eps,
                                   workspace=ws)
        got.append((q, k, v, h, out))
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        for name, x, y in zip(("q", "k", "v", "h_out", "out"), a, b):
            assert torch.equal(x, y), f"call {i}: {name}"


@pytest.mark.parametrize("name", ["llama3-8b-decode", "llama2-70b-int8w@M1", "llama2-70b-int8w@M16",
                                  "llama2-70b-int4w@M16", "llama2-70b-mxfp4w@M16"])
def test_rows_in_kernel_full_size(name, plan_override):
    """The decode workloads at full size: the kernel's own rows give the
    separate row pass's outputs, bit for bit (the oracle comparison of the
    same calls is in test_gpu_parity / test_gpu_int4 / test_gpu_mxfp4)."""
    wl = inputs.workload(name)
    d = to_dev(inputs.generate(wl, seed=1))
    # tile-packed, as a model loads them (on row-major weights the 70B
    # shapes stream over all 256 workgroups, leaving no CU for the rows)
    d["w_qkv"] = fra.pack_weight(d["w_qkv"])
    d["w_gu"] = fra.pack_weight(d["w_gu"], gate_up=True)
    sep, own = _both(wl, d, plan_override, out_dtype=None)
    for nm, a, b in zip(("q", "k", "v", "h_out", "out"), sep, own):
        assert torch.equal(a, b), f"{name}: {nm}"


def test_rows_in_kernel_wait_is_bounded(plan_override):
    """The bounded wait, forced from the host (the stream_rows_expire
    override): the waiting workgroups expect a tag that no workgroup
    publishes, so every wait runs out after a short bound.  The launch ends,
    every output is NaN (QKV here on tiles that several workgroups share, so
    the NaN also travels through the partial sums), h_out is still exact, and
    the next call on the same workspace is right again."""
    wl = _wl(dict(M=16, hidden=2048, H=6, Hkv=2, D=64, ffn=512))
    inp = inputs.generate(wl, seed=53)
    d = to_dev(inp)
    pq = fra.describe_plan(wl.M, wl.hidden, wl.n_qkv, torch.bfloat16, torch.bfloat16)
    pg = fra.describe_plan(wl.M, wl.hidden, wl.n_gu, torch.bfloat16, torch.bfloat16, wl.act_fn)
    print(f"bounded wait: qkv {pq['kernel']} grid={pq['grid']} slots={pq['slots']}; gu {pg['kernel']}", flush=True)
    assert pq["kernel"].endswith(",rows>") and pq["slots"] > 1, pq
    assert pg["kernel"].endswith(",rows>"), pg
    need = max(fra.workspace_bytes(wl.M, wl.hidden, n, torch.bfloat16, torch.bfloat16) for n in (wl.n_qkv, wl.n_gu))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)

    def calls():
        q, k, v, h = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], d["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                            wl.head_dim, eps=wl.eps, workspace=ws, out_dtype=torch.float32)
        out = fra.fused_gateup_act(d["x"], d["r"], d["gamma"], d["w_gu"], wl.ffn, wl.act_fn, eps=wl.eps,
                                   workspace=ws, out_dtype=torch.float32)
        torch.cuda.synchronize()
        return q, k, v, h, out

    rq, rg = oracle.workload_qkv(wl, inp), oracle.workload_gateup(wl, inp)
    plan_override(stream_rows_expire=1)
    q, k, v, h, out = calls()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        assert torch.isnan(t).all(), f"{name}: an expired wait must leave NaN"
    assert np.array_equal(h.double().cpu().numpy(), rq["h_out"]), "h_out not bit-exact"
    plan_override(stream_rows_expire=0)
    q, k, v, h, out = calls()
    for name, got in (("q", q), ("k", k), ("v", v)):
        check(name, got, rq[name])
    check("out", out, rg["out"])
