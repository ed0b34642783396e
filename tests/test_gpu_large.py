"""Inputs past 4 GiB: activations or weights whose byte offsets do not fit in
32 bits.

The 128 x 512 kernel addresses its operands through 32-bit buffer offsets, so
a call whose x / residual or weight exceeds 4 GiB is routed to the tiled
kernel (64-bit offsets) at prefill token counts; the weight-streaming kernel
takes any size at decode token counts (64-bit row pointers).  Each case checks
the routing, then the outputs on sampled token rows against the oracle,
including rows and weight rows past the 4 GiB boundary; h_out bit for bit.
Inputs are drawn on the GPU from seeded generators (inputs.device_normal /
device_uniform): RMSNorm, x and r ~ N(0, 1), gamma ~ U(0.5, 1.5), weights
N(0, 1/64), as in the Llama-2-7B prefill recipe.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
BF = torch.bfloat16
EPS = 1e-5


def check(name, got: torch.Tensor, ref: np.ndarray):
    """fp32-stored outputs: max-abs <= 2e-2 and relative Frobenius <= 5e-3."""
    g = got.detach().double().cpu().numpy().reshape(ref.shape)
    assert np.all(np.isfinite(g)), f"{name}: non-finite output"
    err = np.abs(g - ref)
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= 5e-3 and err.max() <= 2e-2, f"{name}: max-abs {err.max():.3e} rel-fro {rel:.3e}"


def _rows(M, boundary, n_rand=6, seed=0):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, boundary - 1, boundary, boundary + 1, M - 1]
    extra = rng.choice(np.arange(2, M - 1), n_rand, replace=False).tolist()
    return sorted(set(r for r in fixed + extra if 0 <= r < M))


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def test_activations_past_4gib():
    K, H, Hkv, D, F = 4096, 2, 1, 64, 64
    M = (1 << 32) // (2 * K) + 64          # x and r: 64 rows past 4 GiB each
    assert M * K * 2 > (1 << 32)
    for n_cols, act in (((H + 2 * Hkv) * D, "none"), (2 * F, "swiglu")):
        plan = fra.describe_plan(M, K, n_cols, BF, BF, act)
        assert plan["family"] == "tiled", plan
    print(f"activations past 4 GiB: M={M} K={K}: drawing", flush=True)
    x = inputs.device_normal((M, K), 1.0, BF, DEV, seed=101)
    r = inputs.device_normal((M, K), 1.0, BF, DEV, seed=102)
    gamma = inputs.device_uniform((K,), 0.5, 1.5, BF, DEV, seed=103)
    wq = inputs.device_normal(((H + 2 * Hkv) * D, K), 1 / 64, BF, DEV, seed=104)
    wg = inputs.device_normal((2 * F, K), 1 / 64, BF, DEV, seed=105)
    print("activations past 4 GiB: GPU calls", flush=True)
    q, k, v, h = fra.fused_add_norm_qkv(x, r, gamma, wq, H, Hkv, D, norm="rms", eps=EPS, out_dtype=torch.float32)
    out = fra.fused_gateup_act(x, r, gamma, wg, F, "swiglu", norm="rms", eps=EPS, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = _rows(M, (1 << 32) // (2 * K))
    idx = torch.as_tensor(rows, dtype=torch.long, device=DEV)
    xs, rs = x[idx].cpu(), r[idx].cpu()
    got = {n: t[idx].cpu() for n, t in (("q", q), ("k", k), ("v", v), ("h", h), ("out", out))}
    del x, r, q, k, v, h, out
    print(f"activations past 4 GiB: oracle on rows {rows}", flush=True)
    g_c = gamma.cpu()
    rq = oracle.add_norm_qkv(xs, rs, g_c, None, "rms", EPS, wq.cpu(), None, None, H, Hkv, D)
    rg = oracle.gateup_act(xs, rs, g_c, None, "rms", EPS, wg.cpu(), None, None, F, "swiglu")
    for n in ("q", "k", "v"):
        check(n, got[n], rq[n])
    check("out", got["out"], rg["out"])
    assert np.array_equal(got["h"].double().numpy(), rq["h_out"]), "h_out not bit-exact"


@pytest.mark.parametrize("M", [8, 96])
def test_weights_past_4gib(M):
    K = 8192
    F = (1 << 32) // (2 * 2 * K) + 32      # the [2F, K] gate/up weight: 64 rows past 4 GiB
    assert 2 * F * K * 2 > (1 << 32)
    plan = fra.describe_plan(M, K, 2 * F, BF, BF, "swiglu")
    assert plan["family"] == ("stream" if M <= 64 else "tiled"), plan
    print(f"weights past 4 GiB: M={M} F={F} K={K}: drawing", flush=True)
    x = inputs.device_normal((M, K), 1.0, BF, DEV, seed=201)
    r = inputs.device_normal((M, K), 1.0, BF, DEV, seed=202)
    gamma = inputs.device_uniform((K,), 0.5, 1.5, BF, DEV, seed=203)
    w = inputs.device_normal((2 * F, K), 1 / 64, BF, DEV, seed=204)
    print(f"weights past 4 GiB: M={M}: GPU call", flush=True)
    out = fra.fused_gateup_act(x, r, gamma, w, F, "swiglu", norm="rms", eps=EPS, out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows = list(range(M)) if M <= 8 else _rows(M, M // 2, n_rand=4)
    idx = torch.as_tensor(rows, dtype=torch.long, device=DEV)
    xs, rs, got = x[idx].cpu(), r[idx].cpu(), out[idx].cpu()
    w_c = w.cpu()
    del out, w
    print(f"weights past 4 GiB: M={M}: oracle on rows {rows}", flush=True)
    rg = oracle.gateup_act(xs, rs, gamma.cpu(), None, "rms", EPS, w_c, None, None, F, "swiglu")
    check("out", got, rg["out"])
