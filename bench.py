#!/usr/bin/env python3
"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--only-headline] [--no-cpu]

Prints ONE JSON line. A step is one fused forward (fa_fwd) over the headline
workload: B=4, H=16, N=8192, d=128, bfloat16 Q/K/V/O, non-causal, inputs
resident in HBM. Throughput counts 4*B*H*N^2*d FLOPs per step (halved for
causal), the same count for every backend. Also reported:

- ``roofline``: the forward kernel against the dense bf16 MFMA peak (2.5
  PFLOP/s published for MI355X), with its average launch time measured by HIP
  events on the stream the kernel is launched on; ``traffic`` (HBM bytes per
  launch, from rocprofv3 FETCH_SIZE + WRITE_SIZE scaled by the same counters
  on a plain copy of known size) is read from profiles/ and is null if the
  kernel sources changed since those counters were taken;
- ``cpu_baseline``: the float64 CPU oracle timed on a bounded sample of the
  same workload on the host cores (a reported baseline, not the target);
- ``extra``: per-launch min/median/max of the headline; the backward (dQ, dK, dV;
  FLOPs counted as 2.5x the forward's, the five products of the backward); the causal headline, the
  other workloads (including the FP8 path: rotation/quantisation of Q, K, V plus
  the FP8 forward) and the FP8 quantiser's HBM throughput; the tiny fp32 case and
  the short-sequence sweep in GB/s of algorithmic bytes, warm and with the
  last-level cache flushed; split-key decoding (one new token against a key/value
  cache) in GB/s of algorithmic bytes (K and V read once, Q read, O and LSE written); the
  forward with grouped key/value heads, a sliding window and packed sequences, in TFLOP/s
  of the (query, key) pairs each query sees (4 d FLOPs per pair).

``cpu_baseline.per_workload`` times the same oracle on whole heads of every forward workload
(the FP8 one twice: on the original and on the dequantised inputs).

``--summarize DIR [--kernel RE] [--last K]`` prints kernel-trace and counter statistics of a
rocprofv3 csv output directory (only each kernel's last K dispatches with --last: the timed
launches); ``--source-hashes`` prints the code-only hashes of each kernel family's sources.
``--calib-copy`` runs only a 1 GiB device-to-device copy (used to calibrate the
rocprofv3 byte counters); ``--only-headline`` skips the extra workloads;
``--only-bwd`` times only the backward on the headline shape (for kernel traces
of the backward kernels) and prints its own JSON line; ``--only-decode`` does the
same for split-key decoding on the grouped-head 8K-cache workload, ``--only fp8``
for the FP8 forward (inputs quantised once, untimed), ``--only fp8-prep`` for the
rotation and quantisation of one tensor of that workload, and ``--only NAME`` for the
bf16 or fp32 forward on the named workload (e.g. short_b64h16n512_d128; with
``--causal`` its causal variant).
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0         # MI355X dense fp8 MFMA, published
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E, published
HEADLINE = "b4h16n8k_d128"
EXT_BENCH = ("gqa_b2_hq16_hkv4_n8k_d128_causal", "swa_b2_hq16_hkv4_n8k_d128_w4096", "varlen_16docs_hq16_hkv4_n16k_d128")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_fa_fwd_bf16_b4h16n8k_d128.txt")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--only-headline", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--calib-copy", action="store_true")
    p.add_argument("--only-bwd", action="store_true")
    p.add_argument("--only-decode", action="store_true")
    p.add_argument("--only", default=None, help="fp8, fp8-prep, or a forward workload name")
    p.add_argument("--causal", action="store_true", help="--only: the causal variant of a workload that has one")
    p.add_argument("--only-ext", default=None, help="one grouped-head / window / packed workload")
    p.add_argument("--source-hashes", action="store_true", help="print the kernel families' source hashes")
    p.add_argument("--summarize", default=None, metavar="DIR",
                   help="statistics of a rocprofv3 output directory (kernel trace and/or counters)")
    p.add_argument("--kernel", default="fwd_kernel", help="--summarize: regular expression of kernel names")
    p.add_argument("--last", type=int, default=0, help="--summarize: only the last N dispatches of each kernel")
    return p.parse_args()


# the sources each kernel family is compiled from (headline: the bf16 forward)
KERNEL_SOURCES = {
    "fwd_bf16": ("fa_common.h", "fa_fwd_kernel.h", "fa_fwd_bf16.hip"),
    "fwd_fp8": ("fa_common.h", "fa_fwd_kernel.h", "fa_fp8.hip"),
    "fwd_short": ("fa_common.h", "fa_fwd_kernel.h", "fa_tile.h", "fa_fwd_short.hip"),
    "fwd_f32": ("fa_common.h", "fa_fwd_f32.hip"),
    "bwd": ("fa_common.h", "fa_fwd_kernel.h", "fa_tile.h", "fa_bwd.hip"),
    "decode": ("fa_common.h", "fa_fwd_kernel.h", "fa_tile.h", "fa_decode.hip"),
}
HEADLINE_SOURCES = KERNEL_SOURCES["fwd_bf16"]


def code_only(text: str) -> str:
    """C++ source without its comments, whitespace collapsed (the kernel sources hold no string
    literals with comment markers): what the compiler sees, so that editing a comment does not
    make stored measurements of the code stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(family: str = "fwd_bf16") -> str:
    """Hash of a kernel family's sources (code only), to tell whether stored measurements of
    those kernels are still current (the headline's: family fwd_bf16)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_06_amd", "csrc")
    for name in KERNEL_SOURCES[family]:
        h.update(name.encode())
        h.update(code_only(open(os.path.join(csrc, name)).read()).encode())
    return h.hexdigest()[:16]


def source_hashes() -> dict:
    return {fam: kernel_source_hash(fam) for fam in KERNEL_SOURCES}


def read_traffic():
    """Stored HBM bytes per launch of the headline kernel, or None if missing or stale."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def visible_pairs(n: int, causal: bool, left: int, right: int) -> int:
    """(query, key) pairs of one head of a sequence of n tokens under the causal mask and the
    window (left, right) (negative: no limit): query i sees keys max(0, i - left) ..
    min(n - 1, i + right, i if causal)."""
    total = 0
    for i in range(n):
        hi = n - 1
        if causal:
            hi = min(hi, i)
        if right >= 0:
            hi = min(hi, i + right)
        lo = max(0, i - left) if left >= 0 else 0
        total += max(0, hi - lo + 1)
    return total


def progress(msg: str) -> None:
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def ramp(torch, fn, ms: float = 100.0) -> None:
    """Untimed calls of fn for about `ms` of GPU time, so the clock has risen from idle."""
    t0 = time.perf_counter()
    fn()
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-5) * 1e3
    for _ in range(int(ms / one)):
        fn()
    torch.cuda.synchronize()


def time_launches(torch, fn, steps: int, warmup: int, ramp_ms: float = 0.0) -> float:
    """Average milliseconds per call of fn (which launches on the current stream), after
    `warmup` untimed calls (and, for the secondary workloads, ~ramp_ms of untimed calls)."""
    if ramp_ms > 0:
        ramp(torch, fn, ramp_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def launch_stats(torch, fn, n: int = 20, flush=None):
    """Per-launch milliseconds (min, median, max) over n launches, each bracketed by its own
    events on the current stream; flush() (untimed) runs before each launch if given."""
    times = []
    for _ in range(n):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b))
    times.sort()
    return {"min": round(times[0], 4), "median": round(times[len(times) // 2], 4), "max": round(times[-1], 4)}


def calib_copy(torch):
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ms = time_launches(torch, lambda: dst.copy_(src), 10, 2)
    print(json.dumps({"calib_copy_bytes": n, "ms": ms, "GB/s": 2 * n / ms / 1e6}))


def cpu_baseline(w, budget_s: float = 15.0):
    """Time the float64 oracle on whole heads of the workload until ~budget_s of CPU work."""
    import numpy as np

    from exact_attention_06_amd.workloads import make_qkv
    from oracle.attention import attention_head_fp64

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.seed, "bf16")   # the same inputs as the GPU run
    heads, secs = 0, 0.0
    while secs < budget_s and heads < w.B * w.H:
        b, hi = divmod(heads, w.H)
        qh, kh, vh = (x[b, hi].float().numpy().astype(np.float64) for x in (q, k, v))
        t0 = time.perf_counter()
        attention_head_fp64(qh, kh, vh, w.scale, False)
        secs += time.perf_counter() - t0
        heads += 1
    flops = heads * 4.0 * w.N * w.N * w.d
    return {
        "value": flops / secs / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"first {heads} of {w.B * w.H} heads of the workload (all {w.N} query rows each, "
                  f"non-causal), float64 three-pass oracle, {secs:.1f} s; value = 4*N^2*d per head / time",
        "seconds": round(secs, 2), "host_cpus": os.cpu_count(),
    }


def _short_name(name: str) -> str:
    """A kernel name without its argument list (the first '(' outside template brackets)."""
    anon = "(anonymous namespace)"
    text = name.replace(anon, "\x00")
    depth = 0
    for i, ch in enumerate(text):
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            text = text[:i]
            break
    return text.replace("\x00", anon).strip()


def summarize(d: str, kernel_re: str, last: int) -> int:
    """Statistics of one rocprofv3 ``--output-format csv`` directory for the kernels whose name
    matches kernel_re: from a kernel trace, per kernel the dispatch count and the average, median,
    min and max duration; from a counter collection, per kernel and counter the median value per
    dispatch. With ``last`` > 0 only each kernel's last `last` dispatches count (in dispatch
    order): the timed launches of a bench run, after its warm-up."""
    import csv
    import glob
    import statistics
    from collections import defaultdict

    rx = re.compile(kernel_re)
    found = False
    for f in sorted(glob.glob(os.path.join(d, "*kernel_trace.csv"))):
        found = True
        by = defaultdict(list)
        for r in csv.DictReader(open(f)):
            if rx.search(r["Kernel_Name"]):
                by[r["Kernel_Name"]].append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        print(f"# kernel trace {os.path.basename(f)}: kernels matching '{kernel_re}'"
              + (f", last {last} dispatches of each" if last else ", every dispatch"))
        print("# columns: kernel | dispatches | used | average ns | median ns | min ns | max ns")
        for name, ts in sorted(by.items()):
            ts.sort()
            sel = ts[-last:] if last else ts
            du = [e - b for b, e in sel]
            print(f"{_short_name(name)} | {len(ts)} | {len(sel)} | {statistics.mean(du):.0f} | "
                  f"{statistics.median(du):.0f} | {min(du)} | {max(du)}")
    for f in sorted(glob.glob(os.path.join(d, "*counter_collection.csv"))):
        found = True
        vals = defaultdict(lambda: defaultdict(float))   # (kernel, dispatch) -> counter -> value
        for r in csv.DictReader(open(f)):
            if rx.search(r["Kernel_Name"]):
                vals[(r["Kernel_Name"], int(r["Dispatch_Id"]))][r["Counter_Name"]] += float(r["Counter_Value"])
        per_kernel = defaultdict(list)
        for (name, disp), cv in vals.items():
            per_kernel[name].append((disp, cv))
        print(f"# counters {os.path.basename(f)}: median per dispatch, kernels matching '{kernel_re}'"
              + (f", last {last} dispatches of each" if last else ", every dispatch"))
        for name, rows in sorted(per_kernel.items()):
            rows.sort()
            sel = rows[-last:] if last else rows
            print(f"## {_short_name(name)} ({len(sel)} of {len(rows)} dispatches)")
            for c in sorted(sel[0][1]):
                print(f"{c}: {statistics.median(cv[c] for _, cv in sel):.6g}")
    if not found:
        print(f"no kernel trace or counter collection in {d}", file=sys.stderr)
        return 1
    return 0


def cpu_oracle_per_workload(budget_s: float = 2.0) -> dict:
    """The float64 oracle on whole heads of every forward workload, each until ~budget_s of CPU
    work (at least one head; every head of the small ones), on the same seeded inputs as the GPU
    runs. The oracle materialises the full score matrix, causal or not: fp64 FLOPs done are
    4 N^2 d per head; "attention_TFLOP/s" counts them as the GPU figures do (halved for causal).
    The FP8 workload twice: on the original float32 inputs (the O_true reference) and on the
    dequantised rotated inputs (O_deq; the quantisation itself untimed)."""
    import numpy as np

    from exact_attention_06_amd.workloads import WORKLOADS, make_fp8_inputs, make_qkv
    from oracle.attention import attention_head_fp64
    from oracle.fp8 import block_dequantize, block_quantize, rotate_to_f32

    def run(w, causal, heads_fn):
        heads, secs = 0, 0.0
        while heads < w.B * w.H and (heads == 0 or secs < budget_s):
            b, h = divmod(heads, w.H)
            args = heads_fn(b, h)
            t0 = time.perf_counter()
            attention_head_fp64(*args, w.scale, causal)
            secs += time.perf_counter() - t0
            heads += 1
        done = heads * 4.0 * w.N * w.N * w.d
        counted = done / (2 if causal else 1)
        return {"heads_timed": heads, "heads": w.B * w.H, "seconds": round(secs, 3),
                "fp64_GFLOP/s": round(done / secs / 1e9, 1), "attention_TFLOP/s": round(counted / secs / 1e12, 4),
                "whole_workload_s_est": round(secs / heads * w.B * w.H, 1)}

    out = {}
    for name, causal in [("tiny_f32", False), ("b4h16n2k_d128", False), ("b4h16n2k_d128", True),
                         ("long_n16k_d128", True), ("b8h16n4k_d64", False), ("b8h16n4k_d256", False),
                         ("b4h16n8k_d128", False), ("b4h16n8k_d128", True)]:
        w = WORKLOADS[name]
        q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype)
        out[f"{name}{'_causal' if causal else ''}"] = run(w, causal, lambda b, h: (q[b, h], k[b, h], v[b, h]))
        del q, k, v
        progress(f"cpu oracle {name} causal={causal} done")
    w = WORKLOADS["fp8_b4h16n8k_d128"]
    q, k, v, signs = make_fp8_inputs(w.B, w.H, w.N, w.d, w.seed)
    sg = signs.numpy()
    out["fp8_b4h16n8k_d128_O_true"] = run(w, False, lambda b, h: (q[b, h], k[b, h], v[b, h]))

    def deq(b, h):
        qc, qs = block_quantize(rotate_to_f32(q[b, h].numpy(), sg))
        kc, ks = block_quantize(rotate_to_f32(k[b, h].numpy(), sg))
        vc, vs = block_quantize(v[b, h].numpy())
        return (block_dequantize(qc, qs), block_dequantize(kc, ks), block_dequantize(vc, vs))
    out["fp8_b4h16n8k_d128_O_deq"] = run(w, False, deq)
    progress("cpu oracle fp8 done")
    del q, k, v
    _ = np
    return out


def main():
    args = parse_args()
    if args.summarize is not None:
        return summarize(args.summarize, args.kernel, args.last)
    if args.source_hashes:
        print(json.dumps(source_hashes()))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the library runs "
              "on one GPU per call and the attention forward is not sharded across GPUs.", file=sys.stderr)
        return 2
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calib_copy:
        calib_copy(torch)
        return 0

    from exact_attention_06_amd import fa_fwd, fa_fwd_fp8, fa_prep_fp8
    from exact_attention_06_amd.workloads import WORKLOADS, make_fp8_inputs, make_qkv

    def bwd_case(wx, causal, steps, warmup, ramp_ms):
        """Backward (dQ, dK, dV) after one forward; FLOPs counted as the page's five products,
        2.5x the forward's."""
        from exact_attention_06_amd import fa_bwd
        from exact_attention_06_amd.workloads import make_dout
        q, k, v = (x.cuda() for x in make_qkv(wx.B, wx.H, wx.N, wx.d, wx.seed, wx.dtype))
        do = make_dout(wx.B, wx.H, wx.N, wx.d, wx.seed).cuda()
        o, lse = fa_fwd(q, k, v, causal=causal)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        delta = torch.empty((2, wx.B, wx.H, wx.N), dtype=torch.float32, device="cuda")
        m = time_launches(torch, lambda: fa_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, causal=causal),
                          steps, warmup, ramp_ms)
        progress(f"bwd {wx.name} causal={causal}: {m:.3f} ms")
        return {"ms": round(m, 4), "TFLOP/s": round(2.5 * wx.flops(causal) / m / 1e9, 1)}

    def decode_case(wd, steps, warmup, ramp_ms):
        from exact_attention_06_amd import fa_decode, fa_decode_workspace_size
        from exact_attention_06_amd.workloads import make_decode_inputs
        q, k, v = (x.cuda() for x in make_decode_inputs(wd.B, wd.Hq, wd.Hkv, wd.Nq, wd.Nk, wd.d, wd.seed))
        o = torch.empty_like(q)
        lse = torch.empty((wd.B, wd.Hq, wd.Nq), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(16, fa_decode_workspace_size(wd.B, wd.Hq, wd.Hkv, wd.Nq, wd.Nk, wd.d)),
                         dtype=torch.uint8, device="cuda")
        m = time_launches(torch, lambda: fa_decode(q, k, v, o, lse, ws, causal=wd.causal), steps, warmup, ramp_ms)
        nb = wd.kv_bytes()
        progress(f"decode {wd.name}: {m:.4f} ms, {nb / m / 1e6:.0f} GB/s")
        return {"ms": round(m, 4), "bytes": nb, "GB/s": round(nb / m / 1e6, 1),
                "frac_of_8TBs": round(nb / m / 1e6 / PEAK_HBM_GBS, 4)}

    def ext_case(name, steps, warmup, ramp_ms):
        # grouped heads / sliding window / packed documents: FLOPs of the visible (query, key) pairs
        from exact_attention_06_amd import fa_fwd_ext
        from exact_attention_06_amd.workloads import EXT_WORKLOADS, make_ext_inputs
        we = EXT_WORKLOADS[name]
        q, k, v, cu = make_ext_inputs(we)
        lens = [we.N] * we.B if cu is None else [int(x) for x in (cu[1:] - cu[:-1])]
        pairs = sum(visible_pairs(n, we.causal, we.window[0], we.window[1]) for n in lens)
        fl = 4.0 * we.d * we.Hq * pairs
        q, k, v = q.cuda(), k.cuda(), v.cuda()
        cud = None if cu is None else cu.cuda()
        mx = we.N if cu is None else max(lens)
        o = torch.empty_like(q)
        lse = torch.empty((we.B, we.Hq, we.N), dtype=torch.float32, device="cuda")
        m = time_launches(torch, lambda: fa_fwd_ext(q, k, v, o, lse, causal=we.causal, window=we.window,
                                                    cu_seqlens=cud, max_seqlen=mx), steps, warmup, ramp_ms)
        progress(f"{name}: {m:.3f} ms, {fl / m / 1e9:.1f} TFLOP/s")
        return {"ms": round(m, 4), "TFLOP/s": round(fl / m / 1e9, 1), "visible_pairs_per_head": pairs}

    if args.only_ext is not None:
        if args.only_ext not in EXT_BENCH:
            print(f"--only-ext: one of {list(EXT_BENCH)}", file=sys.stderr)
            return 2
        r = ext_case(args.only_ext, args.steps, args.warmup, 100.0)
        print(json.dumps({"metric": "attention fwd TFLOP/s over visible pairs (4*d each)", "value": r["TFLOP/s"],
                          "unit": "TFLOP/s", "ms_per_step": r["ms"], "steps": args.steps,
                          "config": {"workload": args.only_ext}}))
        return 0

    if args.only_decode:
        from exact_attention_06_amd.workloads import DECODE_WORKLOADS
        wd = DECODE_WORKLOADS["decode_b16_hq32_hkv8_nk8k_d128"]
        r = decode_case(wd, args.steps, args.warmup, 100.0)
        print(json.dumps({"metric": "decode HBM GB/s (K, V read once; Q, O, LSE)", "value": r["GB/s"], "unit": "GB/s",
                          "ms_per_step": r["ms"], "steps": args.steps,
                          "config": {"workload": f"fa_decode B={wd.B} Hq={wd.Hq} Hkv={wd.Hkv} Nq={wd.Nq} "
                                                 f"Nk={wd.Nk} d={wd.d} bf16"}}))
        return 0

    if args.only == "fp8-prep":
        # the rotation + quantisation of one tensor of the FP8 workload (Q: rotated)
        wf = WORKLOADS["fp8_b4h16n8k_d128"]
        q, _, _, signs = (x.cuda() for x in make_fp8_inputs(wf.B, wf.H, wf.N, wf.d, wf.seed))
        q8, sq = fa_prep_fp8(q, signs)
        m = time_launches(torch, lambda: fa_prep_fp8(q, signs, q8, sq), args.steps, args.warmup, 100.0)
        nbytes = q.numel() * 5 + sq.numel() * 4
        print(json.dumps({"metric": "FP8 rotation + quantisation GB/s (4 B read + 1 B written per element)",
                          "value": round(nbytes / m / 1e6, 1), "unit": "GB/s", "ms_per_step": round(m, 4),
                          "steps": args.steps,
                          "config": {"workload": f"fa_prep_fp8 B={wf.B} H={wf.H} N={wf.N} d={wf.d} rotated"}}))
        return 0
    if args.only == "fp8":
        wf = WORKLOADS["fp8_b4h16n8k_d128"]
        q, k, v, signs = (x.cuda() for x in make_fp8_inputs(wf.B, wf.H, wf.N, wf.d, wf.seed))
        q8, sq = fa_prep_fp8(q, signs)
        k8, sk = fa_prep_fp8(k, signs)
        v8, sv = fa_prep_fp8(v)
        del q, k, v
        o = torch.empty((wf.B, wf.H, wf.N, wf.d), dtype=torch.float32, device="cuda")
        lse = torch.empty((wf.B, wf.H, wf.N), dtype=torch.float32, device="cuda")
        m = time_launches(torch, lambda: fa_fwd_fp8(q8, k8, v8, sq, sk, sv, o, lse), args.steps, args.warmup, 100.0)
        print(json.dumps({"metric": "attention fwd TFLOP/s (4*B*H*N^2*d), e4m3 inputs", "value": round(wf.flops(False) / m / 1e9, 1),
                          "unit": "TFLOP/s", "ms_per_step": round(m, 4), "steps": args.steps,
                          "config": {"workload": f"fa_fwd_fp8 B={wf.B} H={wf.H} N={wf.N} d={wf.d} non-causal"}}))
        return 0
    if args.only is not None:
        if args.only not in WORKLOADS or WORKLOADS[args.only].dtype == "fp8":
            print(f"--only: fp8 or one of {sorted(n for n, x in WORKLOADS.items() if x.dtype != 'fp8')}", file=sys.stderr)
            return 2
        wx = WORKLOADS[args.only]
        causal = wx.causal[0]
        if args.causal:
            if True not in wx.causal:
                print(f"--causal: {args.only} has no causal variant", file=sys.stderr)
                return 2
            causal = True
        q, k, v = (x.cuda() for x in make_qkv(wx.B, wx.H, wx.N, wx.d, wx.seed, wx.dtype))
        o = torch.empty_like(q)
        lse = torch.empty((wx.B, wx.H, wx.N), dtype=torch.float32, device="cuda")
        m = time_launches(torch, lambda: fa_fwd(q, k, v, o, lse, causal=causal), args.steps, args.warmup, 100.0)
        nbytes = 4 * q.numel() * q.element_size() + lse.numel() * 4
        print(json.dumps({"metric": "attention fwd", "TFLOP/s": round(wx.flops(causal) / m / 1e9, 2),
                          "GB/s": round(nbytes / m / 1e6, 1), "ms_per_step": round(m, 4), "steps": args.steps,
                          "bytes": nbytes, "config": {"workload": f"{wx.name} causal={causal}"}}))
        return 0

    if args.only_bwd:
        wb = WORKLOADS[HEADLINE]
        r = bwd_case(wb, False, args.steps, args.warmup, 100.0)
        print(json.dumps({"metric": "attention bwd TFLOP/s (2.5 x 4*B*H*N^2*d)", "value": r["TFLOP/s"],
                          "unit": "TFLOP/s", "ms_per_step": r["ms"], "steps": args.steps,
                          "config": {"workload": f"fa_bwd B={wb.B} H={wb.H} N={wb.N} d={wb.d} bf16 non-causal"}}))
        return 0

    def bf16_case(w, causal, steps, warmup, ramp_ms=0.0):
        q, k, v = (x.cuda() for x in make_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
        ms = time_launches(torch, lambda: fa_fwd(q, k, v, o, lse, causal=causal), steps, warmup, ramp_ms)
        del q, k, v, o, lse
        return ms

    # ---------------- headline
    w = WORKLOADS[HEADLINE]
    flops = w.flops(False)
    ms = bf16_case(w, False, args.steps, args.warmup)
    tflops = flops / (ms * 1e-3) / 1e12
    progress(f"headline {ms:.3f} ms, {tflops:.1f} TFLOP/s")
    qh, kh, vh = (x.cuda() for x in make_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype))
    oh = torch.empty_like(qh)
    lh = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    per_launch = launch_stats(torch, lambda: fa_fwd(qh, kh, vh, oh, lh), 20)
    del qh, kh, vh, oh, lh
    traffic = read_traffic()
    result = {
        "metric": "attention fwd TFLOP/s (4*B*H*N^2*d) and % of MFMA peak, bf16 N=8k d=128",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded iid N(0,1))",
        "config": {"workload": f"fa_fwd B={w.B} H={w.H} N={w.N} d={w.d} bf16 non-causal",
                   "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": False},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic},
    }
    extra = {"headline_per_launch_ms": per_launch}
    if not args.only_headline:
        s2, w2 = max(5, args.steps // 2), 2
        ms_c = bf16_case(w, True, args.steps, args.warmup, 100.0)
        extra["headline_causal"] = {"ms": round(ms_c, 4), "TFLOP/s": round(w.flops(True) / ms_c / 1e9, 1)}
        for name, causal in [("b4h16n2k_d128", False), ("b4h16n2k_d128", True), ("long_n16k_d128", True),
                             ("b8h16n4k_d64", False), ("b8h16n4k_d256", False)]:
            wx = WORKLOADS[name]
            m = bf16_case(wx, causal, s2, w2, 100.0)
            extra[f"{name}{'_causal' if causal else ''}"] = {
                "ms": round(m, 4), "TFLOP/s": round(wx.flops(causal) / m / 1e9, 1)}
            progress(f"{name} causal={causal}: {m:.3f} ms")
        for name, causal in [("b4h16n8k_d128", False), ("b4h16n8k_d128", True), ("b4h16n2k_d128", False),
                             ("b4h16n2k_d128", True), ("b8h16n4k_d64", False)]:
            extra[f"bwd_{name}{'_causal' if causal else ''}"] = bwd_case(WORKLOADS[name], causal, s2, w2, 100.0)
        # FP8 path: prep of Q, K (rotated) and V, then the FP8 forward
        wf = WORKLOADS["fp8_b4h16n8k_d128"]
        q, k, v, signs = (x.cuda() for x in make_fp8_inputs(wf.B, wf.H, wf.N, wf.d, wf.seed))
        q8, sq = fa_prep_fp8(q, signs)
        k8, sk = fa_prep_fp8(k, signs)
        v8, sv = fa_prep_fp8(v)
        o = torch.empty((wf.B, wf.H, wf.N, wf.d), dtype=torch.float32, device="cuda")
        lse = torch.empty((wf.B, wf.H, wf.N), dtype=torch.float32, device="cuda")
        m_fwd = time_launches(torch, lambda: fa_fwd_fp8(q8, k8, v8, sq, sk, sv, o, lse), s2, w2, 100.0)
        m_prep = time_launches(torch, lambda: fa_prep_fp8(q, signs, q8, sq), s2, w2, 100.0)
        prep_bytes = q.numel() * 5 + sq.numel() * 4
        extra["fp8_b4h16n8k_d128"] = {
            "fwd_ms": round(m_fwd, 4), "fwd_TFLOP/s": round(wf.flops(False) / m_fwd / 1e9, 1),
            "prep_ms_per_tensor": round(m_prep, 4),
            "prep_GB/s": round(prep_bytes / m_prep / 1e6, 1),
            "path_ms": round(m_fwd + 3 * m_prep, 4),
            "path_TFLOP/s": round(wf.flops(False) / (m_fwd + 3 * m_prep) / 1e9, 1),
        }
        del q, k, v, q8, k8, v8, o, lse
        progress(f"fp8: fwd {m_fwd:.3f} ms, prep {m_prep:.3f} ms per tensor")
        # tiny fp32 case (launch/latency bound) and short sequences (HBM bound): GB/s of the
        # algorithmic bytes (Q, K, V read, O, LSE written), warm and with the 256 MB
        # last-level cache flushed by a 512 MB write before each launch
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        flush = lambda: scratch.fill_(1)
        for name in ("tiny_f32", "short_b64h16n128_d128", "short_b64h16n256_d128", "short_b64h16n512_d128"):
            wx = WORKLOADS[name]
            q, k, v = (x.cuda() for x in make_qkv(wx.B, wx.H, wx.N, wx.d, wx.seed, wx.dtype))
            o = torch.empty_like(q)
            lse = torch.empty((wx.B, wx.H, wx.N), dtype=torch.float32, device="cuda")
            nbytes = 4 * q.numel() * q.element_size() + lse.numel() * 4
            fn = lambda: fa_fwd(q, k, v, o, lse)
            ramp(torch, fn)
            warm = launch_stats(torch, fn, 20)
            cold = launch_stats(torch, fn, 20, flush)
            extra[name] = {"bytes": nbytes, "warm_ms": warm, "cold_ms": cold,
                           "warm_GB/s": round(nbytes / warm["median"] / 1e6, 1),
                           "cold_GB/s": round(nbytes / cold["median"] / 1e6, 1),
                           "TFLOP/s_warm": round(wx.flops(False) / warm["median"] / 1e9, 2)}
            progress(f"{name}: warm {warm['median']:.4f} ms, cold {cold['median']:.4f} ms")
            del q, k, v, o, lse
        # what the same protocol allows: a device copy moving the bytes of the N = 128 shape
        # (half read, half written), warm and after the same flush
        nb = extra["short_b64h16n128_d128"]["bytes"]
        src = torch.empty(nb // 2, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(3)
        cp = lambda: dst.copy_(src)
        ramp(torch, cp, 30.0)
        cw, cc = launch_stats(torch, cp, 20), launch_stats(torch, cp, 20, flush)
        extra["copy_same_bytes_as_n128"] = {"bytes": 2 * (nb // 2), "warm_GB/s": round(2 * (nb // 2) / cw["median"] / 1e6, 1),
                                            "cold_GB/s": round(2 * (nb // 2) / cc["median"] / 1e6, 1)}
        del scratch, src, dst
        from exact_attention_06_amd.workloads import DECODE_WORKLOADS
        for name in ("decode_b16_hq32_hkv8_nk8k_d128", "decode_b2_h32_nk32k_d128"):
            extra[name] = decode_case(DECODE_WORKLOADS[name], args.steps, args.warmup, 100.0)
        for name in EXT_BENCH:
            extra[name] = ext_case(name, s2, w2, 100.0)
        result["extra"] = extra
    # calibration GEMM (hipBLASLt via torch): what a plain bf16 GEMM sustains on this GPU now
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    c = torch.empty_like(a)
    g_ms = time_launches(torch, lambda: torch.mm(a, b, out=c), 10, 3, 100.0)
    gemm_tflops = 2.0 * 8192 ** 3 / g_ms / 1e9
    result["calibration_gemm"] = {"shape": "8192x8192x8192 bf16 torch.mm", "TFLOP/s": round(gemm_tflops, 1),
                                  "attention_frac_of_gemm": round(tflops / gemm_tflops, 4)}
    del a, b, c
    progress(f"calibration gemm {gemm_tflops:.1f} TFLOP/s")
    result["source_hashes"] = source_hashes()
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w)
        progress("cpu baseline done")
        if not args.only_headline:
            result["cpu_baseline"]["per_workload"] = cpu_oracle_per_workload()
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
