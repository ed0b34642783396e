"""Micro-benchmark autotuner for the launch configuration of the projections.

The pages build their kernels by timing candidate configurations of each
GEMM on the target GPU for the shapes at hand and keeping the fastest
("TensorRT-LLM 深度工程实践…", §2.4 内核自动调优; "TRT-LLM deep dive",
构建阶段详解 step 2 and 面试视角).  This module does that for one MI355X
call shape at a time:

* candidates: every configuration the library can run for the shape -- the
  kernel family, and for the weight-streaming kernel the weight rows per
  workgroup (32, 64, 128 or 256, as the weight dtype allows) and the
  workgroup count, for the tiled and 128 x 512 kernels the
  K split -- deduplicated by the plan each one produces (fp_describe_plan);
* each candidate is installed as a one-entry table (fp_tune_install), run
  once with fp32 outputs and checked against the planner's own result (the
  configurations only reorder fp32 partial sums), then timed over several
  interleaved rounds by the library's per-kernel HIP events (the device time
  of the call's kernels, so host launch overhead cannot mask a difference),
  weights rotated through copies so that they stream from HBM as they would
  in a model;
* the fastest candidate becomes a table entry for exactly that token count
  (none when the planner's choice is already the fastest).

Inputs are the seeded synthetic workloads of ``inputs``.  The tables are JSON
(``save`` / ``load``) and are installed with ``fusion_residual_add_amd.tune_install``.

    python -m fusion_residual_add_amd.tune --workload llama3-8b-decode --out table.json
"""
from __future__ import annotations

import argparse
import json
import statistics
import sys
from typing import Dict, List, Optional

import torch

import fusion_residual_add_amd as fra
from fusion_residual_add_amd import inputs

MALL_BYTES = 256 << 20            # MI355X last-level (Infinity) cache
_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16, "i8": torch.int8,
           "i4": torch.uint8, "e4m3": torch.float8_e4m3fn, "mxfp4": torch.float4_e2m1fn_x2}
_NAMES = {v: k for k, v in _DTYPES.items()}


def candidates(M: int, hidden: int, n_cols: int, act: torch.dtype, wdt: torch.dtype,
               swiglu: bool, layout: str = "rows") -> List[Dict]:
    """Launch configurations for one call shape (plan overrides; {} is the
    planner's own choice), one per distinct plan."""
    fn = "swiglu" if swiglu else "none"
    raw: List[Dict] = [{}]
    stream_ok = act != torch.float32 and M <= 64 and hidden % 256 == 0
    big = M * hidden * 2 >= (1 << 32) or n_cols * hidden * 2 >= (1 << 32)
    if stream_ok:
        # the instantiated rows per workgroup: 128 always; 64 and 32 (K halves,
        # hidden a multiple of 512) for 16-bit and E4M3 weights without the
        # gate/up pairing at up to 32 tokens; 256 for one-byte and 4-bit weights
        quant = wdt in (torch.int8, torch.uint8, torch.float8_e4m3fn, torch.float4_e2m1fn_x2)
        rows = [128]
        if not swiglu and M <= 32 and wdt not in (torch.int8, torch.uint8, torch.float4_e2m1fn_x2):
            rows.append(64)
            if hidden % 512 == 0:
                rows.append(32)
        if quant:
            rows.append(256)
        for r in rows:
            for g in (128, 160, 192, 224, 240, 256):
                raw.append(dict(family="stream", rows=r, grid=g))
    if act != torch.float32 and not big:
        for s in (1, 2, 3, 4, 6, 8):
            raw.append(dict(family="prefill", splits=s))
        if wdt == act:
            raw.append(dict(family="gemm16"))
    for s in (1, 2, 4, 8):
        raw.append(dict(family="tiled", splits=s))
    seen, out = set(), []
    try:
        for c in raw:
            fra.tune_install([_entry(M, M, hidden, n_cols, act, wdt, swiglu, c)] if c else [])
            p = fra.describe_plan(M, hidden, n_cols, act, wdt, fn, layout=layout)
            key = (p["kernel"], p["grid"], p["splits"])
            if key not in seen:
                seen.add(key)
                out.append(dict(c, plan=p))
    finally:
        fra.tune_clear()
    return out


def _entry(m_lo, m_hi, hidden, n_cols, act, wdt, swiglu, cfg) -> Dict:
    e = dict(m_lo=m_lo, m_hi=m_hi, hidden=hidden, n_cols=n_cols, act_dtype=act, w_dtype=wdt,
             swiglu=bool(swiglu))
    for k in ("family", "rows", "grid", "splits"):
        if k in cfg:
            e[k] = cfg[k]
    return e


class _Call:
    """Device inputs of one call of a workload, with rotated weight copies
    (layout "packed": tile-packed copies, where the shape allows)."""

    def __init__(self, wl, call: str, seed: int = 0, layout: str = "rows"):
        dev = torch.device("cuda:0")
        host = inputs.generate(wl, seed=seed, parts=(call,))
        self.wl, self.call = wl, call
        self.d = {k: v.to(dev) for k, v in host.items()}
        wkey = "w_qkv" if call == "qkv" else "w_gu"
        w = self.d[wkey]
        wbytes = w.numel() * w.element_size()
        n_sets = max(1, (2 * MALL_BYTES) // max(wbytes, 1) + 1)
        roll = (lambda i: w.view(torch.uint8).roll(i, 0).contiguous().view(w.dtype)) if w.element_size() == 1 \
            else (lambda i: w.roll(i, 0).contiguous())
        self.ws = [w] + [roll(i) for i in range(1, n_sets)]
        self.wkey = wkey
        self.n_cols = w.shape[0]
        self.swiglu = call == "gu" and wl.act_fn == "swiglu"
        self.layout = "rows"
        if layout == "packed":
            try:
                self.ws = [fra.pack_weight(x, gate_up=self.swiglu) for x in self.ws]
                self.layout = "packed_gate_up" if self.swiglu else "packed"
            except fra.FusedProjError:
                pass

    def run(self, i: int, out_dtype=None):
        wl, d = self.wl, self.d
        w = self.ws[i % len(self.ws)]
        if self.call == "qkv":
            q, k, v, _ = fra.fused_add_norm_qkv(d["x"], d["r"], d["gamma"], w, wl.n_heads, wl.n_kv_heads,
                                                wl.head_dim, beta=d.get("beta"), norm=wl.norm, eps=wl.eps,
                                                w_scale=d.get("s_qkv"), bias=d.get("b_qkv"), write_h=False,
                                                out_dtype=out_dtype)
            return torch.cat([q.reshape(wl.M, -1), k.reshape(wl.M, -1), v.reshape(wl.M, -1)], 1)
        return fra.fused_gateup_act(d["x"], d["r"], d["gamma"], w, wl.ffn, wl.act_fn, beta=d.get("beta"),
                                    norm=wl.norm, eps=wl.eps, w_scale=d.get("s_gu"), bias=d.get("b_gu"),
                                    out_dtype=out_dtype)


def tune_call(wl, call: str, reps: int = 20, rounds: int = 5, log=None, layout: str = "rows") -> Dict:
    """Time every candidate of one call of workload ``wl``; returns
    {"entry": table entry or None, "results": [(candidate, median us)], "default_us": ...}."""
    c = _Call(wl, call, layout=layout)
    act, wdt = c.d["x"].dtype, c.ws[0].dtype
    M, K = wl.M, wl.hidden
    cands = candidates(M, K, c.n_cols, act, wdt, c.swiglu, c.layout)
    times: List[List[float]] = [[] for _ in cands]
    ref = None
    try:
        for j, cand in enumerate(cands):          # correctness against the planner's result
            fra.tune_install([_entry(M, M, K, c.n_cols, act, wdt, c.swiglu, cand)] if j else [])
            got = c.run(0, out_dtype=torch.float32).double()
            torch.cuda.synchronize()
            if ref is None:
                ref = got
            else:
                err = (got - ref).abs().max().item()
                if not err <= 1e-3 * max(1.0, ref.abs().max().item()):
                    raise RuntimeError(f"candidate {cand} differs from the planner's result by {err}")
        for _ in range(rounds):
            for j, cand in enumerate(cands):
                fra.tune_install([_entry(M, M, K, c.n_cols, act, wdt, c.swiglu, cand)] if j else [])
                for i in range(3):
                    c.run(i)
                torch.cuda.synchronize()
                # device time of the call's kernels (HIP events around each
                # launch), so that host launch overhead cannot hide differences
                fra.profile_start()
                for i in range(reps):
                    c.run(i)
                prof = fra.profile_stop()
                times[j].append(sum(ms for _, ms in prof.values()) / reps * 1e3)
    finally:
        fra.tune_clear()
    med = [statistics.median(t) for t in times]
    results = sorted(zip(cands, med), key=lambda x: x[1])
    best, best_us = results[0]
    entry = None
    if best and best_us < 0.99 * med[0]:
        entry = _entry(M, M, K, c.n_cols, act, wdt, c.swiglu, best)
    if log:
        log(f"{wl.name} {call}: planner {cands[0]['plan']['kernel']} grid {cands[0]['plan']['grid']} "
            f"splits {cands[0]['plan']['splits']}: {med[0]:.1f} us; best {best.get('plan', {}).get('kernel')} "
            f"grid {best['plan']['grid']} splits {best['plan']['splits']}: {best_us:.1f} us"
            f"{' (entry)' if entry else ' (planner kept)'}")
    return {"entry": entry, "default_us": med[0],
            "results": [({k: v for k, v in cnd.items() if k != "plan"} | {"kernel": cnd["plan"]["kernel"],
                          "grid": cnd["plan"]["grid"], "splits": cnd["plan"]["splits"]}, us)
                        for cnd, us in results]}


def tune_workload(name: str, reps: int = 20, rounds: int = 5, log=print, layout: str = "rows") -> List[Dict]:
    """Table entries for both calls of a named workload (only where a candidate
    beats the planner by more than 1 %)."""
    wl = inputs.workload(name)
    out = []
    for call in (("qkv", "gu") if wl.n_qkv else ("gu",)):
        r = tune_call(wl, call, reps=reps, rounds=rounds, log=log, layout=layout)
        if r["entry"]:
            out.append(r["entry"])
    return out


def save(entries: List[Dict], path: str) -> None:
    rows = []
    for e in entries:
        e = dict(e)
        e["act_dtype"], e["w_dtype"] = _NAMES[e["act_dtype"]], _NAMES[e["w_dtype"]]
        rows.append(e)
    with open(path, "w") as fh:
        json.dump(rows, fh, indent=1)


def load(path: str) -> List[Dict]:
    with open(path) as fh:
        rows = json.load(fh)
    for e in rows:
        e["act_dtype"], e["w_dtype"] = _DTYPES[e["act_dtype"]], _DTYPES[e["w_dtype"]]
    return rows


def main(argv: Optional[List[str]] = None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", action="append", required=True, help="a workload name (repeatable)")
    ap.add_argument("--out", help="write the table here (JSON)")
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--rounds", type=int, default=5)
    ap.add_argument("--layout", choices=("rows", "packed"), default="rows",
                    help="time the calls on row-major or tile-packed weights")
    args = ap.parse_args(argv)
    entries = []
    for name in args.workload:
        entries += tune_workload(name, reps=args.reps, rounds=args.rounds,
                                 log=lambda s: print(s, flush=True), layout=args.layout)
    if args.out:
        save(entries, args.out)
    print(f"{len(entries)} table entries", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
