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
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA
MFMA_FP8_PEAK_TFLOPS = 5033.2   # MI355X dense fp8 MFMA
MALL_BYTES = 256 << 20


_COMMENT_OR_STRING = re.compile(r'"(?:\\.|[^"\\\n])*"|//[^\n]*|/\*.*?\*/', re.S)


def code_text(src: str) -> str:
    """C++ / HIP source with its comments removed (string literals kept) and
    every run of white space made one space."""
    return " ".join(_COMMENT_OR_STRING.sub(lambda m: m.group(0) if m.group(0).startswith('"') else " ", src).split())


def kernel_source_hash(csrc: str = "") -> str:
    """Hash of the library sources' code (comments excluded: they change no
    kernel), which keys the stored traffic counters to the code they were
    taken on."""
    h = hashlib.sha256()
    csrc = csrc or os.path.join(ROOT, "fusion_residual_add_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode())
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def algo_bytes(wl, call: str) -> int:
    """Algorithmic HBM bytes of one call: every input read once, every output
    written once; the normalised rows and the GEMM intermediates are not
    counted (the fusion keeps them on chip)."""
    ea = {"f32": 4, "f16": 2, "bf16": 2}[wl.act]
    ew = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1, "i4": 0.5, "e4m3": 1, "mxfp4": 0.5}[wl.wdt]
    if call == "down":                               # a [M, ffn], residual and out [M, hidden], weights
        N, K = wl.hidden, wl.ffn
        b = wl.M * K * ea + 2 * wl.M * N * ea + int(N * K * ew)
        if wl.wdt in ("i8", "e4m3"):
            b += 4 * N
        if wl.wdt == "i4":
            b += 4 * N * (K // 128)
        if wl.wdt == "mxfp4":
            b += N * (K // 32)
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
    if wl.wdt == "mxfp4":
        b += N * (K // 32)                           # one E8M0 byte per row and 32 k
    return b


def flops(wl, call: str) -> int:
    if call == "down":
        return 2 * wl.M * wl.ffn * wl.hidden
    N = wl.n_qkv if call == "qkv" else wl.n_gu
    return 2 * wl.M * wl.hidden * N


class Runner:
    """Device copies of a workload with R rotating weight sets.  layout
    "packed": the fused calls read tile-packed copies of the weights (made
    once here, as at model load; a weight whose shape the layout does not
    take stays row-major), the torch reference the row-major ones."""

    def __init__(self, wl, seed=0, min_sets=1, down=False, layout="rows"):
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
        self.layout = layout
        self.fsets = self.sets          # the weights the fused calls read
        self.packed = []
        if layout == "packed":
            self.fsets = []
            for st in self.sets:
                f = dict(st)
                for k in [k for k in st if k.startswith("w_")]:
                    try:
                        f[k] = fra.pack_weight(st[k], gate_up=(k == "w_gu" and wl.act_fn == "swiglu"))
                        if k not in self.packed:
                            self.packed.append(k)
                    except fra.FusedProjError:
                        pass
                self.fsets.append(f)
            torch.cuda.synchronize()
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
        lay = lambda k: (("packed_gate_up" if k == "w_gu" and wl.act_fn == "swiglu" else "packed")
                         if k in self.packed else "rows")
        for call, N in (("qkv", wl.n_qkv), ("gu", wl.n_gu)):
            if N:
                k = "w_qkv" if call == "qkv" else "w_gu"
                need = max(need, fra.workspace_bytes(M, wl.hidden, N, act_t, self.base[k].dtype, lay(k)))
        if down:
            need = max(need, fra.workspace_bytes(M, wl.ffn, wl.hidden, act_t, self.base["w_down"].dtype,
                                                 lay("w_down")))
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=dev)

    def qkv(self, i):
        s, wl = self.fsets[i % self.R], self.wl
        self.fra.fused_add_norm_qkv(s["x"], s["r"], s["gamma"], s["w_qkv"], wl.n_heads, wl.n_kv_heads,
                                    wl.head_dim, beta=s.get("beta"), norm=wl.norm, eps=wl.eps,
                                    w_scale=s.get("s_qkv"), bias=s.get("b_qkv"), h_out=self.h,
                                    q=self.q, k=self.k, v=self.v, workspace=self.ws)

    def gu(self, i):
        s, wl = self.fsets[i % self.R], self.wl
        self.fra.fused_gateup_act(s["x"], s["r"], s["gamma"], s["w_gu"], wl.ffn, wl.act_fn,
                                  beta=s.get("beta"), norm=wl.norm, eps=wl.eps, w_scale=s.get("s_gu"),
                                  bias=s.get("b_gu"), out=self.out, workspace=self.ws)

    def down(self, i):
        s = self.fsets[i % self.R]
        self.fra.fused_down_residual(s["a_down"], s["w_down"], self.h_down, w_scale=s.get("s_down"),
                                     out=self.h_down)

    def step(self, i):
        if self.wl.n_qkv:
            self.qkv(i)
        self.gu(i)

    def unfused(self, i):
        """The same step as separate torch ops on the same tensors (16-bit
        weights only): h = x + r, the norm, the projection through
        torch.nn.functional.linear (hipBLASLt), q / k / v as views of its
        output, then the norm again for the gate/up projection and SiLU(g) * u
        (or bias + tanh-GELU) as elementwise ops.  Every intermediate goes
        through HBM, which is what the fused calls avoid."""
        import torch.nn.functional as Fn
        s, wl = self.sets[i % self.R], self.wl
        K = wl.hidden

        def norm(h):
            if wl.norm == "rms":
                return Fn.rms_norm(h, (K,), s["gamma"], wl.eps)
            return Fn.layer_norm(h, (K,), s["gamma"], s.get("beta"), wl.eps)

        h = s["x"] + s["r"]
        if wl.n_qkv:
            qkv = Fn.linear(norm(h), s["w_qkv"], s.get("b_qkv"))
            qkv.split([wl.n_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim, wl.n_kv_heads * wl.head_dim], 1)
        gu = Fn.linear(norm(h), s["w_gu"], s.get("b_gu"))
        if wl.act_fn == "swiglu":
            return Fn.silu(gu[:, :wl.ffn]) * gu[:, wl.ffn:]
        if wl.act_fn == "gelu_tanh":
            return Fn.gelu(gu, approximate="tanh")
        return gu


def time_steps(fn, steps, warmup):
    """Mean ms per step over exactly `steps` steps after `warmup` untimed ones,
    bracketed by device synchronisation on both sides."""
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


def repeat_stats(fn, steps, repeats=5):
    """`repeats` more timed runs of `steps` steps each: median / p10 / p90 of
    their ms per step (the spread the single timed run does not show)."""
    import statistics
    runs = sorted(time_steps(fn, steps, 2) for _ in range(repeats))
    q = statistics.quantiles(runs, n=10, method="inclusive") if len(runs) > 1 else runs * 9
    return {"n": repeats, "steps_each": steps, "ms_per_step_median": round(statistics.median(runs), 5),
            "ms_per_step_p10": round(q[0], 5), "ms_per_step_p90": round(q[-1], 5),
            "ms_per_step_min": round(runs[0], 5), "ms_per_step_max": round(runs[-1], 5)}


class ClockSampler:
    """GPU clocks and power while the timed repeats run (the pages insist that
    throughput be compared at a stated clock): sysfs pp_dpm_sclk / pp_dpm_mclk
    (current level marked '*') and hwmon power of the device's PCI function,
    sampled every 5 ms by a thread; without sysfs access, rocm-smi's clock
    report before and after."""

    def __init__(self):
        import glob
        self.dev = None
        self.samples = {"sclk_mhz": [], "mclk_mhz": [], "power_w": []}
        self.smi = []
        try:
            import torch
            p = torch.cuda.get_device_properties(0)
            bdf = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
            cand = f"/sys/bus/pci/devices/{bdf}"
            if os.path.exists(os.path.join(cand, "pp_dpm_sclk")):
                self.dev = cand
        except Exception:
            pass
        if self.dev is None:
            found = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
            if len(found) == 1:
                self.dev = os.path.dirname(found[0])
        self.hwmon = None
        if self.dev:
            for name in ("power1_average", "power1_input"):
                g = glob.glob(os.path.join(self.dev, "hwmon", "hwmon*", name))
                if g:
                    self.hwmon = g[0]
                    break

    @staticmethod
    def _cur(path):
        import re
        with open(path) as fh:
            for line in fh:
                if "*" in line:
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    if m:
                        return int(m.group(1))
        return None

    def _smi(self):
        import re
        import subprocess
        try:
            out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20).stdout
        except (OSError, subprocess.SubprocessError):
            return None
        return {k: int(v) for k, v in re.findall(r"(\w+) clock level: \d+: \((\d+)Mhz\)", out)}

    def _run(self):
        import time as _t
        while not self._stop:
            for key, fn in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
                try:
                    v = self._cur(os.path.join(self.dev, fn))
                    if v is not None:
                        self.samples[key].append(v)
                except OSError:
                    pass
            if self.hwmon:
                try:
                    with open(self.hwmon) as fh:
                        self.samples["power_w"].append(int(fh.read()) / 1e6)
                except (OSError, ValueError):
                    pass
            _t.sleep(0.005)

    def __enter__(self):
        import threading
        self._stop = False
        if self.dev:
            self._t = threading.Thread(target=self._run, daemon=True)
            self._t.start()
        else:
            self.smi.append(self._smi())
        return self

    def __exit__(self, *exc):
        self._stop = True
        if self.dev:
            self._t.join()
        else:
            self.smi.append(self._smi())
        return False

    def report(self):
        import statistics
        if self.dev:
            out = {"source": f"sysfs {self.dev} (pp_dpm_sclk / pp_dpm_mclk current level, hwmon power), "
                             "sampled every 5 ms over the timed repeats"}
            for k, v in self.samples.items():
                out[k] = None if not v else {"median": statistics.median(v), "min": min(v), "max": max(v),
                                             "samples": len(v)}
            return out
        return {"source": "rocm-smi --showclocks before and after the timed repeats (no sysfs access)",
                "before": self.smi[0] if self.smi else None, "after": self.smi[-1] if self.smi else None}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


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


def load_traffic(kernel_key: str, layout: str = "packed"):
    """HBM traffic per launch measured with rocprofv3 counters (profiles/traffic.json),
    valid only while the kernel sources are unchanged since the counters were taken
    and for the weight layout they were taken on."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != kernel_source_hash() or d.get("layout", "rows") != layout:
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
    # activation dtype, true / 1: int8, 2: int4, 3: MXFP4, 4: E4M3 with E4M3 activation codes)
    # the seventh: K parts per chunk (2: 32 weight rows per workgroup of one 16-row fragment);
    # the eighth: nonzero when the kernel forms the normalised rows itself
    m = re.search(r"fp::stream_kernel<(\d), (true|false|\d), (\d+), (\d+), (\d+), (\d)(?:, (\d))?(?:, (\d))?>", cxx)
    if m:
        wq = {"true": "1", "false": "0"}.get(m.group(2), m.group(2))
        act = {"1": "bf16-i8w", "2": "bf16-i4w", "3": "bf16-mxfp4w"}.get(wq) or _ACT[m.group(1)]
        if wq == "4":
            act = _ACT[m.group(1)] + "-e4m3"
        kh = int(m.group(7) or 1)
        rows = ",rows" if int(m.group(8) or 0) else ""
        return (f"stream_kernel<{act},m{16 * int(m.group(3))},n{64 * int(m.group(4)) // kh},"
                f"k{32 * int(m.group(5))},{_EPI[m.group(6)]}{rows}>")
    m = re.search(r"fp::prefill_kernel<(\d), (true|false|\d), (\d)(?:, (?:true|false))?>", cxx)
    if m:
        wq = {"true": "1", "false": "0"}.get(m.group(2), m.group(2))
        act = {"1": "bf16-i8w", "2": "bf16-i4w", "3": "bf16-mxfp4w"}.get(wq) or _ACT[m.group(1)]
        return f"prefill_kernel<{act},128x512,{_EPI[m.group(3)]}>"
    m = re.search(r"fp::stats_kernel<(\d), \d+(?:, \d+)?>", cxx)
    if m:
        return f"stats_kernel<{_ACT[m.group(1)]}>"
    m = re.search(r"fp::quant8_kernel<(\d), \d+, \d+>", cxx)
    if m:
        return f"quant8_kernel<{_ACT[m.group(1)]}>"
    m = re.search(r"fp::norm_kernel<(\d), \d+, \d+>", cxx)
    if m:
        return f"norm_kernel<{_ACT[m.group(1)]}>"
    m = re.search(r"fp::gemm16_kernel<(\d), (\d), (\d)(?:, (?:true|false))?>", cxx)
    if m:
        return f"gemm16_kernel<{_ACT[m.group(1)]},256x256,{m.group(3)}st,{_EPI[m.group(2)]}>"
    if "fp::pack_kernel(" in cxx:
        return "pack_kernel"
    m = re.search(r"fp::gemm8_kernel<(\d), (\d), (\d), (\d), (\d)(?:, (?:true|false))?>", cxx)
    if m:
        fm, fn, wgm = int(m.group(3)), int(m.group(4)), int(m.group(5))
        return f"gemm8_kernel<{_ACT[m.group(1)]},{32 * fm * wgm}x{32 * fn * (4 // wgm)},{_EPI[m.group(2)]}>"
    return cxx


def traffic_probe(wl_name: str, layout: str = "rows") -> None:
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
    run = Runner(wl, layout=layout)
    for i in range(6):
        if wl.n_qkv:
            run.qkv(i)
        run.gu(i)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": wl_name, "calibration_bytes": 2 * n}), flush=True)


def blas_probe(wl_name: str) -> None:
    """hipBLASLt's plain GEMMs of the workload's projection shapes (torch's
    F.linear on an already normalised 16-bit input), six calls of each, to run
    under rocprofv3 --pmc beside --traffic-probe: the counters of the library
    GEMM the fused kernels are compared with."""
    import torch
    import torch.nn.functional as F
    from fusion_residual_add_amd import inputs
    wl = inputs.workload(wl_name)
    if wl.wdt != wl.act:
        raise SystemExit("--blas-probe: 16-bit weights of the activation dtype only")
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[wl.act]
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn(wl.M, wl.hidden, device="cuda", dtype=torch.float32, generator=g).to(dt)
    shapes = ([wl.n_qkv] if wl.n_qkv else []) + [wl.n_gu]
    for n in shapes:
        w = (torch.randn(n, wl.hidden, device="cuda", dtype=torch.float32, generator=g) * wl.w_std).to(dt)
        for _ in range(6):
            F.linear(a, w)
        torch.cuda.synchronize()
        del w
    print(json.dumps({"blas_probe": wl_name, "shapes": [[wl.M, n, wl.hidden] for n in shapes]}), flush=True)


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


def traffic_summarize(wl_name: str, fetch_dir: str, write_dir: str, cmds: str, layout: str = "packed") -> None:
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
    out = {"source_hash": kernel_source_hash(), "workload": wl_name, "layout": layout,
           "calibration": {"kernel": cal[0], "bytes_each_way": calib, "fetch_factor": round(kf, 4),
                           "write_factor": round(kw, 4)},
           "kernels": kernels}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    md = [f"# HBM traffic per launch, {wl_name} ({layout} weights)", "",
          "Counters FETCH_SIZE and WRITE_SIZE (KiB per dispatch, L2 to memory), one rocprofv3 run each,",
          "scaled by what they read for an elementwise pass that reads and writes 1 GiB",
          f"(fetch factor {kf:.4f}, write factor {kw:.4f}).", "",
          "Commands (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):", "", "```", cmds, "```", "",
          "| kernel | dispatches | fetch MB | write MB | total MB |", "|---|---|---|---|---|"] + lines
    with open(os.path.join(ROOT, "profiles", f"traffic_{wl_name}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(json.dumps(out))


def _trace_rows(trace_dir: str):
    """Per-kernel rows (name, calls, avg / min / max ns, share, grid, workgroup,
    VGPRs, LDS) from a rocprofv3 --kernel-trace output directory: the rocpd
    SQLite database (this ROCm's default) or a *kernel_stats.csv."""
    import csv
    import glob
    dbs = glob.glob(os.path.join(trace_dir, "**", "*_results.db"), recursive=True)
    if dbs:
        import sqlite3
        con = sqlite3.connect(dbs[0])
        q = ("select name, count(*), avg(duration), min(duration), max(duration), sum(duration), grid_x, "
             "workgroup_x, vgpr_count, accum_vgpr_count, lds_size from kernels group by name, grid_x "
             "order by sum(duration) desc")
        rows = list(con.execute(q))
        total = sum(r[5] for r in rows) or 1
        return [dict(name=r[0], calls=r[1], avg=r[2], min=r[3], max=r[4], share=100.0 * r[5] / total,
                     grid=r[6] // max(r[7], 1), vgpr=r[8] + r[9], lds=r[10]) for r in rows]
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *_results.db or *kernel_stats.csv under {trace_dir}")
    out = []
    with open(files[0]) as fh:
        for row in csv.DictReader(fh):
            out.append(dict(name=row["Name"], calls=int(row["Calls"]), avg=float(row["AverageNs"]),
                            min=float(row["MinNs"]), max=float(row["MaxNs"]), share=float(row["Percentage"]),
                            grid=None, vgpr=None, lds=None))
    return out


def counters_summarize(tag: str, dirs, cmd: str) -> None:
    """profiles/counters_<tag>.md from rocprofv3 --pmc runs (csv output) of
    --traffic-probe: per library kernel, the median of each counter over its
    dispatches, and what follows from them.  GRBM_GUI_ACTIVE is summed over the
    8 XCDs (each has its own graphics register block), so the shader clock is
    GRBM_GUI_ACTIVE / 8 over the dispatch's duration; SQ_VALU_MFMA_BUSY_CYCLES
    is summed over the 1024 SIMDs, so MFMA busy = it / (1024 x cycles)."""
    import csv
    import glob
    import statistics
    per, dur = {}, {}
    for d in dirs:
        for fpath in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fpath) as fh:
                for row in csv.DictReader(fh):
                    n = row["Kernel_Name"]
                    if "fp::" in n:
                        key = n
                    elif "Cijk" in n:   # hipBLASLt: one name for several shapes, told apart by the grid
                        key = f"{n[:100]} (grid {int(row['Grid_Size']) // 256} workgroups)"
                    else:
                        continue
                    per.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                    dur.setdefault(key, []).append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    md = [f"# Hardware counters, {tag}", "", "Commands (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):",
          "", "```", cmd, "```", "",
          "Medians over the dispatches of each kernel.  GRBM_GUI_ACTIVE is summed over the 8 XCDs: the shader clock",
          "is GRBM_GUI_ACTIVE / 8 / duration.  SQ_VALU_MFMA_BUSY_CYCLES is summed over the 1024 SIMDs: MFMA busy =",
          "it / (1024 x GRBM_GUI_ACTIVE / 8).  SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: the share of wave time spent",
          "waiting at s_waitcnt.  Clock-based ratios only for dispatches longer than 200 us (for short ones",
          "GRBM_GUI_ACTIVE counts beyond the dispatch's timestamps).", ""]
    for n in sorted(per):
        c = {k: statistics.median(v) for k, v in per[n].items()}
        t = statistics.median(dur[n]) * 1e-9
        md.append(f"## `{library_kernel_name(n)}`")
        md.append("")
        md.append(f"median duration under the profiler {t * 1e6:.1f} us")
        # for short dispatches GRBM_GUI_ACTIVE also counts activity outside the
        # dispatch's own timestamps (the implied clock exceeds the part's
        # 2.4 GHz), so the clock-based ratios are given for long ones only
        if "GRBM_GUI_ACTIVE" in c and t > 200e-6:
            cyc = c["GRBM_GUI_ACTIVE"] / 8
            md.append(f"; shader clock {cyc / t / 1e9:.2f} GHz")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                md.append(f"; MFMA busy {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (1024 * cyc):.3f} of SIMD cycles")
            if "TA_TA_BUSY" in c:
                md.append(f"; TA busy {c['TA_TA_BUSY'] / (256 * cyc):.3f} of CU cycles")
            if "TCP_PENDING_STALL_CYCLES" in c:
                md.append(f"; TCP pending-stall {c['TCP_PENDING_STALL_CYCLES'] / (256 * cyc):.3f} of CU cycles")
        if "SQ_WAIT_INST_ANY" in c and c.get("SQ_WAVE_CYCLES"):
            md.append(f"; waiting at s_waitcnt {c['SQ_WAIT_INST_ANY'] / c['SQ_WAVE_CYCLES']:.3f} of wave time")
        if "TCC_HIT" in c and "TCC_MISS" in c:
            md.append(f"; L2 hit rate {c['TCC_HIT'] / max(c['TCC_HIT'] + c['TCC_MISS'], 1):.3f}")
        md.append("")
        md.append("")
        md.append("| counter | median per dispatch |")
        md.append("|---|---|")
        for k in sorted(c):
            md.append(f"| {k} | {c[k]:.0f} |")
        md.append("")
    path = os.path.join(ROOT, "profiles", f"counters_{tag}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def trace_summarize(tag: str, trace_dir: str, cmd: str) -> None:
    """profiles/kernel_trace_<tag>.md from a `rocprofv3 --kernel-trace --stats` output directory."""
    rows = _trace_rows(trace_dir)
    md = [f"# Kernel trace, {tag}", "", "Command (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):",
          "", "```", cmd, "```", "",
          "| kernel (library name, or the first 100 characters) | calls | avg us | min us | max us | share | "
          "workgroups | VGPRs | LDS bytes |", "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        name = library_kernel_name(r["name"])
        name = name if len(name) <= 100 else name[:100] + "..."
        md.append(f"| `{name}` | {r['calls']} | {r['avg'] / 1e3:.2f} | {r['min'] / 1e3:.2f} | {r['max'] / 1e3:.2f} | "
                  f"{r['share']:.1f}% | {r['grid']} | {r['vgpr']} | {r['lds']} |")
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{tag}.md"), "w") as fh:
        fh.write("\n".join(md) + "\n")
    print("\n".join(md))


def all_configs(steps: int, layout: str = "rows") -> None:
    """One JSON line per workload: per-call kernel times and the roofline
    fraction of each call (HBM GB/s when the call is bandwidth-bound, MFMA
    TFLOP/s otherwise)."""
    import torch
    from fusion_residual_add_amd import inputs
    for name in inputs.WORKLOADS:
        wl = inputs.workload(name)
        run = Runner(wl, down=True, layout=layout)
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
                          "weights_packed": run.packed, "ms_per_step": round(ms, 5), "calls": calls}), flush=True)
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


def fusion_gain(steps: int, repeats: int, layout: str = "rows") -> None:
    """Fused calls against the same step as torch ops on the same GPU, per
    16-bit workload (the pages' fusion-gain comparison), with hipBLASLt's
    plain GEMMs of the same shapes (torch.nn.functional.linear on an
    already-normalised input: the GEMM alone, no add / norm / activation) and
    torch's own streaming kernels as context for the HBM rate (a float32 sum
    over 1 GiB of bf16: reads only; a 1 GiB copy: reads and writes).  One
    JSON line per workload, medians of `repeats` runs of `steps` steps, with
    the clocks sampled during the fused runs."""
    import torch
    import torch.nn.functional as Fn
    from fusion_residual_add_amd import inputs
    import statistics
    src = torch.ones((1 << 30) // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    def med(fn, n):
        return statistics.median(time_steps(fn, n, 3) for _ in range(repeats))
    rd = med(lambda i: src.sum(dtype=torch.float32), 20)
    cp = med(lambda i: dst.copy_(src), 20)
    print(json.dumps({"stream_context": {"sum_read_GBps": round((1 << 30) / (rd * 1e-3) / 1e9, 1),
                                         "copy_GBps": round(2 * (1 << 30) / (cp * 1e-3) / 1e9, 1)}}), flush=True)
    del src, dst
    torch.cuda.empty_cache()
    for name in ("llama3-8b-decode", "llama2-7b-prefill", "gpt-fp16-gelu"):
        wl = inputs.workload(name)
        run = Runner(wl, layout=layout)
        n = steps if wl.M <= 64 else max(20, steps // 10)
        with ClockSampler() as clk:
            fused = med(run.step, n)
        unf = med(run.unfused, n)
        s0 = run.sets
        gemm = {}
        for call, key in (("qkv", "w_qkv"), ("gu", "w_gu")):
            if key not in run.base:
                continue
            a = torch.randn((wl.M, wl.hidden), dtype=run.base["x"].dtype, device="cuda")
            t = med(lambda i: Fn.linear(a, s0[i % run.R][key]), n)
            gemm[call] = {"us": round(t * 1e3, 2), "TFLOP/s": round(flops(wl, call) / (t * 1e-3) / 1e12, 1)}
        prof = {c: profile_call(run, c, n) for c in (["qkv"] if wl.n_qkv else []) + ["gu"]}
        fused_kernels = {c: {k: round(v * 1e3, 2) for k, v in p.items()} for c, p in prof.items()}
        step_flops = (flops(wl, "qkv") if wl.n_qkv else 0) + flops(wl, "gu")
        step_bytes = (algo_bytes(wl, "qkv") if wl.n_qkv else 0) + algo_bytes(wl, "gu")
        print(json.dumps({"workload": name, "M": wl.M, "steps": n, "repeats": repeats,
                          "fused_ms": round(fused, 5), "unfused_ms": round(unf, 5),
                          "fused_speedup": round(unf / fused, 3),
                          "fused_TFLOPs": round(step_flops / (fused * 1e-3) / 1e12, 1),
                          "fused_GBps": round(step_bytes / (fused * 1e-3) / 1e9, 1),
                          "fused_kernels_us": fused_kernels, "hipblaslt_gemm_only": gemm,
                          "clocks": clk.report()}), flush=True)
        del run
        torch.cuda.empty_cache()


def fusion_gain_summarize(path: str, cmd: str) -> None:
    """profiles/fusion_gain.md from the JSON lines of --fusion-gain."""
    ctx, rows = None, []
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            if "stream_context" in d:
                ctx = d["stream_context"]
            else:
                rows.append(d)
    md = ["# Fused calls against the unfused torch step, same GPU", "", "Command (from the repository root):", "",
          "```", cmd, "```", "",
          "Unfused = the same step as torch ops on the same tensors: h = x + r, the norm, F.linear (hipBLASLt),",
          "q / k / v as views, the norm again, F.linear, SiLU(g) * u (or bias + tanh-GELU).  `hipBLASLt GEMM",
          "only` = F.linear of the same shapes on an already-normalised input.  Medians of the repeats.", ""]
    if ctx:
        md += [f"torch streaming kernels on this GPU: float32 sum over 1 GiB of bf16 {ctx['sum_read_GBps']} GB/s "
               f"(reads), 1 GiB copy {ctx['copy_GBps']} GB/s (reads + writes).", ""]
    md += ["| workload | fused ms | unfused ms | fused speedup | fused rate | fused kernels (us) | "
           "hipBLASLt GEMM only | sclk MHz (median, min-max) |", "|---|---|---|---|---|---|---|---|"]
    for d in rows:
        rate = f"{d['fused_GBps']} GB/s" if d["M"] <= 64 else f"{d['fused_TFLOPs']} TFLOP/s"
        ks = "; ".join(f"{c}: " + ", ".join(f"`{k}` {v}" for k, v in kk.items())
                       for c, kk in d["fused_kernels_us"].items())
        gm = ", ".join(f"{c} {g['us']} us ({g['TFLOP/s']} TFLOP/s)" for c, g in d["hipblaslt_gemm_only"].items())
        c = d["clocks"].get("sclk_mhz") if isinstance(d["clocks"], dict) else None
        clk = f"{c['median']} ({c['min']}-{c['max']})" if c else json.dumps(d["clocks"].get("after"))
        md.append(f"| {d['workload']} | {d['fused_ms']} | {d['unfused_ms']} | {d['fused_speedup']} | {rate} | "
                  f"{ks} | {gm} | {clk} |")
    with open(os.path.join(ROOT, "profiles", "fusion_gain.md"), "w") as fh:
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
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"the full {wl.name} step (both calls, all {wl.M} tokens) run {n} times "
                      f"in {el:.1f} s, {per_step * 1e3:.1f} ms per step"}


def cpu_baseline_rows(wl, n_rows: int = 64):
    """The oracle on a sample of token rows of a prefill-sized step (rows are
    independent, so the time scales with the row count): both calls on
    n_rows evenly spaced rows, reported as the FLOP rate of that sample."""
    import numpy as np
    import oracle
    from fusion_residual_add_amd import inputs
    inp = inputs.generate(wl, seed=0)
    oracle.load()
    rows = np.linspace(0, wl.M - 1, n_rows).astype(np.int64)
    t0 = time.perf_counter()
    if wl.n_qkv:
        oracle.workload_qkv(wl, inp, row_idx=rows)
    oracle.workload_gateup(wl, inp, row_idx=rows)
    el = time.perf_counter() - t0
    fl = 2 * n_rows * wl.hidden * ((wl.n_qkv or 0) + wl.n_gu)
    return {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"both calls of {wl.name} on {n_rows} of its {wl.M} token rows in {el:.2f} s "
                      f"({fl / 1e9:.1f} GFLOP); the full step would take about {el * wl.M / n_rows:.0f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3-8b-decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--layout", choices=("rows", "packed"), default="packed",
                    help="weight layout the fused calls read: tile-packed once at load (fused_pack_weight, as a "
                         "deployment converts its checkpoint) or row-major")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=5,
                    help="extra timed runs of --steps steps each, for the median / p10 / p90 spread")
    ap.add_argument("--blas-probe", action="store_true",
                    help="hipBLASLt GEMMs of the workload's shapes, to run under rocprofv3 --pmc")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="calibration pass + projection calls, to run under rocprofv3 --pmc")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from the two counter runs of --traffic-probe")
    ap.add_argument("--trace-summarize", nargs=2, metavar=("TAG", "TRACE_DIR"),
                    help="write profiles/kernel_trace_TAG.md from a rocprofv3 --kernel-trace --stats run")
    ap.add_argument("--counters-summarize", nargs="+", metavar=("TAG", "PMC_DIR"),
                    help="write profiles/counters_TAG.md from rocprofv3 --pmc csv runs of --traffic-probe")
    ap.add_argument("--cmd", default="", help="the profiling command(s), recorded in the summary")
    ap.add_argument("--all-configs-summarize", metavar="JSON_LINES",
                    help="write profiles/all_configs.md from the output of --all-configs")
    ap.add_argument("--all-configs", action="store_true",
                    help="per-call times and roofline fractions of every workload, one JSON line each")
    ap.add_argument("--fusion-gain", action="store_true",
                    help="fused against unfused torch steps and hipBLASLt GEMMs, one JSON line per workload")
    ap.add_argument("--fusion-gain-summarize", metavar="JSON_LINES",
                    help="write profiles/fusion_gain.md from the output of --fusion-gain")
    ap.add_argument("--tune-file", metavar="JSON",
                    help="install this launch-configuration table (python -m fusion_residual_add_amd.tune "
                         "--out) before timing; the default is the built-in planner")
    args = ap.parse_args()
    if args.traffic_summarize:
        traffic_summarize(args.workload, *args.traffic_summarize, args.cmd, args.layout)
        return
    if args.trace_summarize:
        trace_summarize(*args.trace_summarize, args.cmd)
        return
    if args.counters_summarize:
        counters_summarize(args.counters_summarize[0], args.counters_summarize[1:], args.cmd)
        return
    if args.all_configs_summarize:
        all_configs_summarize(args.all_configs_summarize, args.cmd)
        return
    if args.fusion_gain_summarize:
        fusion_gain_summarize(args.fusion_gain_summarize, args.cmd)
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
        traffic_probe(args.workload, args.layout)
        return
    if args.blas_probe:
        blas_probe(args.workload)
        return
    if args.all_configs:
        all_configs(min(args.steps, 20), args.layout)
        return
    if args.fusion_gain:
        fusion_gain(args.steps, args.repeats, args.layout)
        return
    wl = inputs.workload(args.workload)
    run = Runner(wl, layout=args.layout)
    ms = time_steps(run.step, args.steps, args.warmup)
    with ClockSampler() as clk:
        reps = repeat_stats(run.step, args.steps, args.repeats)
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
    roof["traffic"] = load_traffic(f"{wl.name}:{gu_kernel}", args.layout)
    unfused = None
    if wl.wdt == wl.act:
        ums = time_steps(run.unfused, args.steps, args.warmup)
        unfused = {"ms_per_step": round(ums, 5), "fused_speedup": round(ums / ms, 3),
                   "what": "the same step as torch ops (add, norm, F.linear through hipBLASLt, SiLU * up)"}

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
                   "weight_sets_rotated": run.R, "weights_layout": args.layout,
                   "weights_packed": run.packed},
        "roofline": roof,
        "repeats": reps,
        "clocks": clk.report(),
        "kernel_us": per_call,
        "unfused_torch": unfused,
        "tuning_table": args.tune_file,
    }
    del run
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        for name in ("llama2-7b-prefill", "llama2-7b-prefill-fp8", "llama3-8b-decode-fp8"):
            pwl = inputs.workload(name)
            pr = Runner(pwl, layout=args.layout)
            nsteps = args.prefill_steps if pwl.M > 64 else 100
            pms = time_steps(pr.step, nsteps, 3)
            with ClockSampler() as pclk:
                preps = repeat_stats(pr.step, nsteps, args.repeats)
            pfl = flops(pwl, "qkv") + flops(pwl, "gu")
            pby = algo_bytes(wl=pwl, call="qkv") + algo_bytes(wl=pwl, call="gu")
            pprof = profile_call(pr, "gu", 5)
            pq = profile_call(pr, "qkv", 5)
            if pwl.M > 64:      # prefill: matrix-core bound
                ppeak = MFMA_FP8_PEAK_TFLOPS if pwl.wdt == "e4m3" else MFMA_BF16_PEAK_TFLOPS
                pval, punit = pfl / (pms * 1e-3) / 1e12, "TFLOP/s"
            else:               # decode: HBM bound (algorithmic bytes)
                ppeak, pval, punit = HBM_PEAK_GBS, pby / (pms * 1e-3) / 1e9, "GB/s"
            ent = {"value": round(pval, 2), "unit": punit, "steps": nsteps, "weights_packed": pr.packed,
                   "ms_per_step": round(pms, 4), "repeats": preps, "clocks": pclk.report(),
                   "dtype": "e4m3" if pwl.wdt == "e4m3" else pwl.act, "peak": ppeak,
                   "frac_of_peak": round(pval / ppeak, 4),
                   "kernel_us": {"gu": {k: round(v * 1e3, 1) for k, v in pprof.items()},
                                 "qkv": {k: round(v * 1e3, 1) for k, v in pq.items()}}}
            if pwl.wdt == pwl.act:
                ums = time_steps(pr.unfused, nsteps, 3)
                ent["unfused_torch"] = {"ms_per_step": round(ums, 4), "fused_speedup": round(ums / pms, 3)}
            sec[name] = ent
            del pr
            torch.cuda.empty_cache()
            if not args.no_cpu_baseline and name == "llama2-7b-prefill":
                sec[name]["cpu_baseline"] = cpu_baseline_rows(pwl)
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
