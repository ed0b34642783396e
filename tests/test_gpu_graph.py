"""Captured graphs and concurrent streams.

A serving loop replays the two projection calls from a captured HIP graph
(torch.cuda.CUDAGraph over the library's own launches): every replay must
give exactly the bits of eager calls on the same inputs, with eager work and
synchronisations between replays.  Calls on two streams, each with its own
workspace, may overlap: each must give the bits of the same call made alone.
Each case covers one kernel family (weight streaming with shared tiles, its
32-row form with K halves, its int8 form, the 128 x 512 kernel with split K,
the fp32 tiled kernel).
"""
import pytest
import torch

import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TDT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

CASES = [
    dict(act="bf16", M=32, hidden=2048, H=8, Hkv=2, D=64, ffn=512),   # weight streaming, two per tile
    dict(act="bf16", M=16, hidden=1024, H=64, Hkv=16, D=64, ffn=256),  # QKV: 32-row tiles with K halves
    dict(act="bf16", wdt="i8", M=16, hidden=2048, H=4, Hkv=2, D=32, ffn=400),
    dict(act="bf16", M=200, hidden=512, H=4, Hkv=2, D=64, ffn=384),   # 128 x 512 tiles, K split
    dict(act="f32", M=40, hidden=256, H=4, Hkv=2, D=32, ffn=96),      # tiled kernel
]


def _workload(act="bf16", wdt=None, M=32, hidden=512, H=4, Hkv=2, D=32, ffn=128):
    return inputs.Workload(
        name=f"graph-{act}-{wdt}-{M}", M=M, hidden=hidden, act=act, wdt=wdt or act, norm="rms", eps=1e-5,
        x_std=1.0, r_std=1.0, gamma_lo=0.5, gamma_hi=1.5, beta_std=None, w_std=0.05, n_heads=H,
        n_kv_heads=Hkv, head_dim=D, ffn=ffn, act_fn="swiglu", bias_std=None)


class Layer:
    """Static buffers of one (QKV, gate/up) pair of calls."""

    def __init__(self, wl, weights):
        dt = TDT[wl.act]
        M = wl.M
        self.wl, self.w = wl, weights
        self.x = torch.empty(M, wl.hidden, dtype=dt, device=DEV)
        self.r = torch.empty_like(self.x)
        self.h = torch.empty_like(self.x)
        self.q = torch.empty(M, wl.n_heads, wl.head_dim, dtype=dt, device=DEV)
        self.k = torch.empty(M, wl.n_kv_heads, wl.head_dim, dtype=dt, device=DEV)
        self.v = torch.empty_like(self.k)
        self.out = torch.empty(M, wl.ffn, dtype=dt, device=DEV)
        wdt = weights["w_qkv"].dtype
        need = max(fra.workspace_bytes(M, wl.hidden, n, dt, wdt)
                   for n in (weights["w_qkv"].shape[0], weights["w_gu"].shape[0]))
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)

    def load(self, xr):
        self.x.copy_(xr["x"])
        self.r.copy_(xr["r"])

    def run(self):
        wl, w = self.wl, self.w
        fra.fused_add_norm_qkv(self.x, self.r, w["gamma"], w["w_qkv"], wl.n_heads, wl.n_kv_heads, wl.head_dim,
                               norm=wl.norm, eps=wl.eps, w_scale=w.get("s_qkv"), h_out=self.h,
                               q=self.q, k=self.k, v=self.v, workspace=self.ws)
        fra.fused_gateup_act(self.x, self.r, w["gamma"], w["w_gu"], wl.ffn, wl.act_fn, norm=wl.norm, eps=wl.eps,
                             w_scale=w.get("s_gu"), out=self.out, workspace=self.ws)

    def outputs(self):
        return [t.clone() for t in (self.q, self.k, self.v, self.h, self.out)]


def _sets(wl, n):
    """Shared weights (seed 0) and n activation sets (seeds 0 .. n-1)."""
    full = [inputs.generate(wl, seed=s) for s in range(n)]
    weights = {k: v.to(DEV) for k, v in full[0].items() if k not in ("x", "r")}
    acts = [{k: full[s][k].to(DEV) for k in ("x", "r")} for s in range(n)]
    return weights, acts


def _same(got, ref, what):
    for name, a, b in zip(("q", "k", "v", "h", "out"), got, ref):
        assert torch.equal(a, b), f"{what}: {name} differs from the eager call"


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_graph_replays_match_eager(cfg):
    wl = _workload(**cfg)
    weights, acts = _sets(wl, 3)
    layer = Layer(wl, weights)
    eager = []
    for a in acts:
        layer.load(a)
        layer.run()
        eager.append(layer.outputs())
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.run()                      # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.run()

    for rep, s in enumerate((0, 1, 2, 1, 0)):
        layer.load(acts[s])
        graph.replay()
        torch.cuda.synchronize()
        _same(layer.outputs(), eager[s], f"replay {rep} (set {s})")
        # eager work of the program between replays
        layer.load(acts[(s + 1) % 3])
        layer.run()
        torch.cuda.synchronize()
        _same(layer.outputs(), eager[(s + 1) % 3], f"eager call after replay {rep}")


@pytest.mark.parametrize("cfg", CASES[:3], ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_two_streams_overlap(cfg):
    wl = _workload(**cfg)
    weights, acts = _sets(wl, 2)
    layers = [Layer(wl, weights), Layer(wl, weights)]
    eager = []
    for L, a in zip(layers, acts):
        L.load(a)
        L.run()
        eager.append(L.outputs())
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for L in layers:
        L.q.zero_()
        L.out.zero_()
    torch.cuda.synchronize()
    for _ in range(4):                   # interleaved enqueues: the calls overlap on the device
        for L, st in zip(layers, streams):
            with torch.cuda.stream(st):
                L.run()
    torch.cuda.synchronize()
    for i, L in enumerate(layers):
        _same(L.outputs(), eager[i], f"stream {i}")
