"""Benchmark of the fused projection path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic tokens:
fused_add_norm_qkv (residual add, row statistics, normalisation into the MFMA
A-tile, QKV GEMM, GQA split) followed by fused_gateup_act (the same prologue,
gate/up GEMM, SwiGLU), i.e. the two calls of a transformer block's fused
projections.  The default workload is the Llama-3-8B-shaped decode step
(M = 32 tokens, hidden 4096, 32 Q / 8 KV heads of 128, ffn 14336, bf16),
which is HBM-bound, so the headline value is algorithmic HBM GB/s.
The prefill workload (Llama-2-7B shape, M = 16384) is timed as a secondary
line in TFLOP/s.

Inputs are resident in HBM before the timed region.  Several weight sets are
rotated so that the 256 MB last-level cache cannot serve the weights of one
step from the previous one.  Per-kernel durations come from the library's
HIP-event profiler (events on the stream the kernels are launched on).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5033.2   # MI355X dense fp8 MFMA
MALL_BYTES = 256 << 20


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fusion_residual_add_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode())
            h.update(fh.read())
    return h.hexdigest()[:16]


def algo_bytes(wl, call: str) -> int:
    """Algorithmic HBM bytes of one call: every input read once, every output
    written once; the normalised rows and the GEMM intermediates are not
    counted (the fusion keeps them on chip)."""
    ea = {"f32": 4, "f16": 2, "bf16": 2}[wl.act]
    ew = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i4": 0.5, "e4m3": 1}[wl.wdt]
    if call == "down":                               # a [M, ffn], residual and out [M, hidden], weights
        N, K = wl.hidden, wl.ffn
        b = wl.M * K * ea + 2 * wl.M * N * ea + int(N * K * ew)
        if wl.wdt in ("i8", "e4m3"):
            b += 4 * N
        if wl.wdt == "i4":
            b += 4 * N * (K // 128)
        return b
    M, K = wl.M, wl.hidden
    b = 2 * M * K * ea + K * ea                      # x, residual, gamma
    if wl.norm == "layer":
        b += K * ea                                  # beta
    if call == "qkv":
        N = wl.n_qkv
        b += int(N * K * ew) + M * K * ea + M * N * ea    # weights, h_out, q/k/v
    else:
        N = wl.n_gu
        b += int(N * K * ew) + M * wl.ffn * ea       # weights, out
        if wl.bias_std is not None:
            b += N * ea
    if wl.wdt in ("i8", "e4m3"):
        b += 4 * N                                   # per-row scales
    if wl.wdt == "i4":
        b += 4 * N * (K // 128)                      # per-row, per-128-k group scales
    return b


def flops(wl, call: str) -> int:
    if call == "down":
        return 2 * wl.M * wl.ffn * wl.hidden
    N = wl.n_qkv if call == "qkv" else wl.n_gu
    return 2 * wl.M * wl.hidden * N


class Runner:
    """Device copies of a workload with R rotating weight sets."""

    def __init__(self, wl, seed=0, min_sets=1, down=False):
        import torch
        from fusion_residual_add_amd import inputs
        self.wl = wl
        dev = torch.device("cuda:0")
        host = inputs.generate(wl, seed=seed, parts=("qkv", "gu", "down") if down else ("qkv", "gu"))
        self.base = {k: v.to(dev) for k, v in host.items()}
        wbytes = sum(t.numel() * t.element_size() for k, t in self.base.items() if k.startswith("w_"))
        self.R = max(min_sets, (2 * MALL_BYTES) // max(wbytes, 1) + 1)
        self.sets = [self.base]
        for i in range(1, self.R):
            s = dict(self.base)
            for k in list(s):
                if k.startswith("w_"):
                    w = self.base[k]                              # distinct buffers, same statistics
                    s[k] = w.view(torch.uint8).roll(i, 0).contiguous().view(w.dtype) if w.element_size() == 1 \
                        else w.roll(i, 0).contiguous()
            self.sets.append(s)
        import fusion_residual_add_amd as fra
        self.fra = fra
        M = wl.M
        self.q = torch.empty((M, wl.n_heads or 1, wl.head_dim or 1), dtype=self.base["x"].dtype, device=dev)
        self.k = torch.empty((M, wl.n_kv_heads or 1, wl.head_dim or 1), dtype=self.base["x"].dtype, device=dev)
        self.v = torch.empty_like(self.k)
        self.h = torch.empty_like(self.base["x"])
        self.out = torch.empty((M, wl.ffn), dtype=self.base["x"].dtype, device=dev)
        # the residual stream the down projection updates in place
        self.h_down = self.base["r"].clone() if down else None
        self.ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
        need = 0
        act_t = self.base["x"].dtype
        for call, N in (("qkv", wl.n_qkv), ("gu", wl.n_gu)):
            if N:
                w = self.base["w_qkv" if call == "qkv" else "w_gu"]
                need = max(need, fra.workspace_bytes(M, wl.hidden, N, act_t, w.dtype))
        if down:
            need = max(need, fra.workspace_bytes(M, wl.ffn, wl.hidden, act_t, self.base["w_down"].dtype))
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def qkv(self, i):
        s, wl = self.sets[i % self.R], self.wl
        self.fra.fused_add_norm_qkv(s["x"], s["r"], s["gamma"], s["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                    wl.head_dim, beta=s.get("beta"), norm=wl.norm, eps=wl.eps,
                                    w_scale=s.get("s_qkv"), bias=s.get("b_qkv"), h_out=self.h,
                                    q=self.q, k=self.k, v=self.v, workspace=self.ws)

    def gu(self, i):
        s, wl = self.sets[i % self.R], self.wl
        self.fra.fused_gateup_act(s["x"], s["r"], s["gamma"], s["w_gu"], wl.ffn, wl.act_fn,
                                  beta=s.get("beta"), norm=wl.norm, eps=wl.eps, w_scale=s.get("s_gu"),
                                  bias=s.get("b_gu"), out=self.out, workspace=self.ws)

    def down(self, i):
        s = self.sets[i % self.R]
        self.fra.fused_down_residual(s["a_down"], s["w_down"], self.h_down, w_scale=s.get("s_down"),
                                     out=self.h_down)

    def step(self, i):
        if self.wl.n_qkv:
            self.qkv(i)
        self.gu(i)


def time_steps(fn, steps, warmup):
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def profile_call(runner, call: str, n: int):
    """Average duration (ms) of each library kernel over n calls of one kind."""
    import torch
    fn = {"qkv": runner.qkv, "gu": runner.gu, "down": runner.down}[call]
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    runner.fra.profile_start()
    for i in range(n):
        fn(i)
    prof = runner.fra.profile_stop()
    return {k: t / c for k, (c, t) in prof.items()}


def load_traffic(kernel_key: str):
    """HBM traffic per launch measured with rocprofv3 counters (profiles/traffic.json),
    valid only while the kernel sources are unchanged since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash():
        return None
    ent = d.get("kernels", {}).get(kernel_key)
    return None if ent is None else ent.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters and kernel-trace summaries
# ---------------------------------------------------------------------------
_ACT = {"0": "f32", "1": "f16", "2": "bf16"}
_EPI = {"0": "qkv", "1": "swiglu", "2": "gelu", "3": "linear"}


def library_kernel_name(cxx: str) -> str:
    """The library profiler's name of a kernel from the demangled C++ name rocprofv3 prints."""
    import re
    # the second template argument: the weight storage (false / 0: the
    # activation dtype, true / 1: int8, 2: int4)
    m = re.search(r"fp::stream_kernel<(\d), (true|false|\d), (\d+), (\d+), (\d+), (\d)(?:, (?:true|false))?>", cxx)
    if m:
        wq = {"true": "1", "false": "0"}.get(m.group(2), m.group(2))
        act = {"1": "bf16-i8w", "2": "bf16-i4w"}.get(wq) or _ACT[m.group(1)]
        return (f"stream_kernel<{act},m{16 * int(m.group(3))},n{64 * int(m.group(4))},"
                f"k{32 * int(m.group(5))},{_EPI[m.group(6)]}>")
    m = re.search(r"fp::prefill_kernel<(\d), (true|false|\d), (\d)(?:, (?:true|false))?>", cxx)
    if m:
        wq = {"true": "1", "false": "0"}.get(m.group(2), m.group(2))
        act = {"1": "bf16-i8w", "2": "bf16-i4w"}.get(wq) or _ACT[m.group(1)]
        return f"prefill_kernel<{act},128x512,{_EPI[m.group(3)]}>"
    m = re.search(r"fp::stats_kernel<(\d), \d+>", cxx)
    if m:
        return f"stats_kernel<{_ACT[m.group(1)]}>"
    m = re.search(r"fp::quant8_kernel<(\d), \d+, \d+>", cxx)
    if m:
        return f"quant8_kernel<{_ACT[m.group(1)]}>"
    m = re.search(r"fp::gemm8_kernel<(\d), (\d), (\d), (\d), (\d)>", cxx)
    if m:
        fm, fn, wgm = int(m.group(3)), int(m.group(4)), int(m.group(5))
        return f"gemm8_kernel<{_ACT[m.group(1)]},{32 * fm * wgm}x{32 * fn * (4 // wgm)},{_EPI[m.group(2)]}>"
    return cxx


def traffic_probe(wl_name: str) -> None:
    """Workload run under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE): an
    elementwise pass over 1 GiB (reads 1 GiB, writes 1 GiB: the calibration of
    the counters) and six calls of each projection of the workload."""
    import torch
    from fusion_residual_add_amd import inputs
    n = (1 << 30) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()
    wl = inputs.workload(wl_name)
    run = Runner(wl)
    for i in range(6):
        if wl.n_qkv:
            run.qkv(i)
        run.gu(i)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": wl_name, "calibration_bytes": 2 * n}), flush=True)


def _counter_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                per.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return per


def traffic_summarize(wl_name: str, fetch_dir: str, write_dir: str, cmds: str) -> None:
    """profiles/traffic.json and a text summary from the two counter runs of --traffic-probe."""
    import statistics
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)
    calib = 1 << 30
    cal = [k for k in fetch if "neg" in k.lower()]
    if not cal:
        raise SystemExit("calibration kernel not found in the counter output")
    kf = calib / (statistics.median(fetch[cal[0]]) * 1024.0)
    kw = calib / (statistics.median(write[cal[0]]) * 1024.0)
    kernels, lines = {}, []
    for name in sorted(fetch):
        if "fp::" not in name:
            continue
        f_b = statistics.median(fetch[name]) * 1024.0 * kf
        w_b = statistics.median(write.get(name, [0.0])) * 1024.0 * kw
        lib = library_kernel_name(name)
        kernels[f"{wl_name}:{lib}"] = {"bytes_per_launch": round(f_b + w_b), "fetch_bytes": round(f_b),
                                       "write_bytes": round(w_b), "launches": len(fetch[name])}
        lines.append(f"| `{lib}` | {len(fetch[name])} | {f_b / 1e6:.2f} | {w_b / 1e6:.2f} | {(f_b + w_b) / 1e6:.2f} |")
    out = {"source_hash": kernel_source_hash(), "workload": wl_name,
           "calibration": {"kernel": cal[0], "bytes_each_way": calib, "fetch_factor": round(kf, 4),
                           "write_factor": round(kw, 4)},
           "kernels": kernels}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    md = [f"# HBM traffic per launch, {wl_name}", "",
          "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, L2 to memory), one rocprofv3 run each,",
          "scaled by what they read for an elementwise pass that reads and writes 1 GiB",
          f"(fetch factor {kf:.4f}, write factor {kw:.4f}).", "",
          "Commands (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):", "", "```", cmds, "```", "",
          "| kernel | dispatches | fetch MB | write MB | total MB |", "|---|---|---|---|---|"] + lines
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl_name}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(out))


def trace_summarize(tag: str, trace_dir: str, cmd: str) -> None:
    """profiles/kernel_trace_<tag>.md from a `rocprofv3 --kernel-trace --stats` output directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {trace_dir}")
    rows = []
    with open(files[0]) as fh:
        for row in csv.DictReader(fh):
            rows.append(row)
    md = [f"# Kernel trace, {tag}", "", "Command (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):",
          "", "```", cmd, "```", "", "| kernel (library name) | calls | avg us | min us | max us | share |",
          "|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| `{library_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def all_configs(steps: int) -> None:
    """One JSON line per workload: per-call kernel times and the roofline
    fraction of each call (HBM GB/s when the call is bandwidth-bound, MFMA
    TFLOP/s otherwise)."""
    import torch
    from fusion_residual_add_amd import inputs
    for name in inputs.WORKLOADS:
        wl = inputs.workload(name)
        run = Runner(wl, down=True)
        ms = time_steps(run.step, steps, 3)
        calls = {}
        for call in (["qkv"] if wl.n_qkv else []) + ["gu", "down"]:
            prof = profile_call(run, call, 20)
            total = sum(prof.values())
            b, f = algo_bytes(wl, call), flops(wl, call)
            mfma_peak = MFMA_FP8_PEAK_TFLOPS if wl.wdt == "e4m3" else \
                MFMA_BF16_PEAK_TFLOPS if wl.act != "f32" else 157.3
            mem_bound = f / b < mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)
            peak = HBM_PEAK_GBS if mem_bound else mfma_peak
            rate = b / (total * 1e-3) / 1e9 if mem_bound else f / (total * 1e-3) / 1e12
            calls[call] = {"kernels_us": {k: round(v * 1e3, 2) for k, v in prof.items()},
                           "bound": "hbm" if mem_bound else "mfma",
                           "rate": round(rate, 1), "unit": "GB/s" if mem_bound else "TFLOP/s",
                           "frac": round(rate / peak, 4)}
        print(json.dumps({"workload": name, "M": wl.M, "hidden": wl.hidden, "act": wl.act, "weights": wl.wdt,
                          "ms_per_step": round(ms, 5), "calls": calls}), flush=True)
        del run
        torch.cuda.empty_cache()


def all_configs_summarize(path: str, cmd: str) -> None:
    """profiles/all_configs.md from the JSON lines of --all-configs."""
    md = ["# Every workload, per call", "", "Command (from the repository root):", "", "```", cmd, "```", "",
          "Rates are per call, statistics kernel included: algorithmic HBM GB/s for bandwidth-bound calls",
          "(8000 GB/s peak), MFMA TFLOP/s otherwise (2516.6 bf16/fp16, 157.3 fp32).", "",
          "| workload | call | kernels (us) | rate | fraction of peak |", "|---|---|---|---|---|"]
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            for call, c in d["calls"].items():
                ks = ", ".join(f"`{k}` {v}" for k, v in c["kernels_us"].items())
                md.append(f"| {d['workload']} | {call} | {ks} | {c['rate']} {c['unit']} | {c['frac']:.3f} |")
    with open(os.path.join(ROOT, "profiles", "all_configs.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def cpu_baseline(wl, budget_s: float = 12.0):
    import oracle
    from fusion_residual_add_amd import inputs
    inp = inputs.generate(wl, seed=0)
    oracle.load()
    n, t0 = 0, time.perf_counter()
    while True:
        if wl.n_qkv:
            oracle.workload_qkv(wl, inp)
        oracle.workload_gateup(wl, inp)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 100:
            break
    per_step = el / n
    step_bytes = (algo_bytes(wl, "qkv") if wl.n_qkv else 0) + algo_bytes(wl, "gu")
    return {"value": round(step_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"the full {wl.name} step (both calls, all {wl.M} tokens) run {n} times "
                      f"in {el:.1f} s, {per_step * 1e3:.1f} ms per step"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3-8b-decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--traffic-probe", action="store_true",
                    help="calibration pass + projection calls, to run under rocprofv3 --pmc")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from the two counter runs of --traffic-probe")
    ap.add_argument("--trace-summarize", nargs=2, metavar=("TAG", "TRACE_DIR"),
                    help="write profiles/kernel_trace_TAG.md from a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--cmd", default="", help="the profiling command(s), recorded in the summary")
    ap.add_argument("--all-configs-summarize", metavar="JSON_LINES",
                    help="write profiles/all_configs.md from the output of --all-configs")
    ap.add_argument("--all-configs", action="store_true",
                    help="per-call times and roofline fractions of every workload, one JSON line each")
    ap.add_argument("--tune-file", metavar="JSON",
                    help="install this launch-configuration table (python -m fusion_residual_add_amd.tune "
                         "--out) before timing; the default is the built-in planner")
    args = ap.parse_args()
    if args.traffic_summarize:
        traffic_summarize(args.workload, *args.traffic_summarize, args.cmd)
        return
    if args.trace_summarize:
        trace_summarize(*args.trace_summarize, args.cmd)
        return
    if args.all_configs_summarize:
        all_configs_summarize(args.all_configs_summarize, args.cmd)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the projections shard by heads / by gate-up pairs without communication; "
              "see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from fusion_residual_add_amd import inputs
    if not os.path.exists(os.path.join(ROOT, "fusion_residual_add_amd", "libfusedproj.so")):
        import __graft_entry__
        __graft_entry__.build()

    if args.tune_file:
        import fusion_residual_add_amd as fra
        from fusion_residual_add_amd import tune
        fra.tune_install(tune.load(args.tune_file))
    if args.traffic_probe:
        traffic_probe(args.workload)
        return
    if args.all_configs:
        all_configs(min(args.steps, 20))
        return
    wl = inputs.workload(args.workload)
    run = Runner(wl)
    ms = time_steps(run.step, args.steps, args.warmup)
    step_bytes = (algo_bytes(wl, "qkv") if wl.n_qkv else 0) + algo_bytes(wl, "gu")
    step_flops = (flops(wl, "qkv") if wl.n_qkv else 0) + flops(wl, "gu")
    mfma_peak = MFMA_FP8_PEAK_TFLOPS if wl.wdt == "e4m3" else MFMA_BF16_PEAK_TFLOPS
    decode = step_flops / step_bytes < mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9)

    # dominant kernel: the gate/up projection
    prof_gu = profile_call(run, "gu", 50)
    gu_kernel = max(prof_gu, key=lambda k: prof_gu[k])
    gu_ms = prof_gu[gu_kernel]
    per_call = {"gu": {k: round(v * 1e3, 2) for k, v in prof_gu.items()}}
    if wl.n_qkv:
        prof_q = profile_call(run, "qkv", 50)
        per_call["qkv"] = {k: round(v * 1e3, 2) for k, v in prof_q.items()}
    if decode:
        achieved = algo_bytes(wl, "gu") / (gu_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        value, unit = step_bytes / (ms * 1e-3) / 1e9, "GB/s"
    else:
        achieved = flops(wl, "gu") / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": round(achieved / mfma_peak, 4)}
        value, unit = step_flops / (ms * 1e-3) / 1e12, "TFLOP/s"
    roof["kernel"] = gu_kernel
    roof["kernel_avg_us"] = round(gu_ms * 1e3, 2)
    roof["algo_bytes_per_launch"] = algo_bytes(wl, "gu")
    roof["traffic"] = load_traffic(f"{wl.name}:{gu_kernel}")

    line = {
        "metric": "fused-layer TFLOP/s (prefill) and HBM GB/s (decode), % of MI355X roofline",
        "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3" if wl.wdt == "e4m3" else wl.act, "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "hidden": wl.hidden, "n_heads": wl.n_heads,
                   "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "ffn": wl.ffn,
                   "act_fn": wl.act_fn, "norm": wl.norm, "weights": wl.wdt,
                   "calls": (["fused_add_norm_qkv"] if wl.n_qkv else []) + [f"fused_gateup_act({wl.act_fn})"],
                   "step_algo_bytes": step_bytes, "step_flops": step_flops,
                   "weight_sets_rotated": run.R},
        "roofline": roof,
        "kernel_us": per_call,
        "tuning_table": args.tune_file,
    }
    del run
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        for name in ("llama2-7b-prefill", "llama2-7b-prefill-fp8", "llama3-8b-decode-fp8"):
            pwl = inputs.workload(name)
            pr = Runner(pwl)
            pms = time_steps(pr.step, args.prefill_steps if pwl.M > 64 else 100, 3)
            pfl = flops(pwl, "qkv") + flops(pwl, "gu")
            pby = algo_bytes(wl=pwl, call="qkv") + algo_bytes(wl=pwl, call="gu")
            pprof = profile_call(pr, "gu", 5)
            pk = max(pprof, key=lambda k: pprof[k])
            pq = profile_call(pr, "qkv", 5)
            if pwl.M > 64:      # prefill: matrix-core bound
                ppeak = MFMA_FP8_PEAK_TFLOPS if pwl.wdt == "e4m3" else MFMA_BF16_PEAK_TFLOPS
                pval, punit = pfl / (pms * 1e-3) / 1e12, "TFLOP/s"
            else:               # decode: HBM bound (algorithmic bytes)
                ppeak, pval, punit = HBM_PEAK_GBS, pby / (pms * 1e-3) / 1e9, "GB/s"
            sec[name] = {"value": round(pval, 2), "unit": punit,
                         "ms_per_step": round(pms, 4),
                         "dtype": "e4m3" if pwl.wdt == "e4m3" else pwl.act, "peak": ppeak,
                         "frac_of_peak": round(pval / ppeak, 4),
                         "kernel_us": {"gu": {k: round(v * 1e3, 1) for k, v in pprof.items()},
                                       "qkv": {k: round(v * 1e3, 1) for k, v in pq.items()}}}
            del pr
            torch.cuda.empty_cache()
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
