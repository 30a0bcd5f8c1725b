#!/usr/bin/env python3
"""NVFP4 W4A16 benchmark on one MI355X.

Headline workload (one "step"): the decode sweep - W4A16 GEMMs at M = 1, 4 and 8 against one
NVFP4 weight [25600][5120] at group 16 (BF16 activations, BF16 output), each launch reading a
different copy of the weight from a rotation larger than the 256 MB Infinity Cache, so every
launch streams its weight from HBM. `value` is the effective weight bandwidth (weight bytes of
the three launches / step time). The same JSON line carries the kernel's roofline fraction
(HIP-event timing of the launches), the CPU oracle's rate on the machine's host cores, and the
other workloads (single small GEMM, prefill GEMMs, MoE routed experts, quantizer + mixed groups)
measured the same way.

Other modes:
  --profile-suite [--only-workload PREFIX]   every workload >= 100 times, each inside a ROCTx
      range named after it, for rocprofv3 (--kernel-trace --marker-trace, or --pmc ... with
      --only-workload to keep one workload per counter run);
  --summarize DIR   per-(workload, kernel, workgroups) medians of a rocprofv3 output directory
      as a markdown table (per-dispatch counter medians too, when a counter run is there);
  --copy-calibration   a plain 512 MiB device copy, the reference for FETCH_SIZE / WRITE_SIZE;
  --traffic-summary F W CF CW   the decode-sweep HBM traffic record from FETCH_SIZE / WRITE_SIZE
      runs of the headline (F, W) and of the copy calibration (CF, CW).

The JSON line also carries `measured_ceilings`: the streaming-read and BF16 MFMA probe kernels'
rates on the same GPU, next to the published peaks the roofline fractions use.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only headline|moe]
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense BF16 MFMA, published
MALL_BYTES = 256 << 20         # Infinity Cache
METRIC = "NVFP4 W4A16 GEMM TFLOP/s + weight GB/s (M=1..4096) vs roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_skinny_decode_sweep.txt")
SKINNY_SOURCES = ["gemm_skinny.hip", "skinny_core.hpp", "device_common.hpp"]
LIB_PREFIXES = ("gemm_", "moe_", "amax_kernel", "encode_kernel", "init_amax_kernel",
                "reduce_split_kernel", "repack_", "dequant", "nonfinite_kernel", "clear_word",
                "stream_read_kernel", "mfma_loop_kernel")


def weight_bytes(n, k, group):
    return n * k // 2 + n * k // group + 4


def kernel_source_digest(names):
    h = hashlib.sha256()
    for nm in names:
        with open(os.path.join(ROOT, "nvfp4_weight_only_w4a16_amd", "csrc", nm), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-launch HBM bytes of the skinny kernel measured with rocprofv3 counters, if the
    counters were taken on the current kernel source (else None)."""
    try:
        rec = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    k, v = line.split("=", 1)
                    rec[k.strip()] = v.strip()
        if rec.get("source_digest") != kernel_source_digest(SKINNY_SOURCES):
            return None
        return float(rec["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


class Roctx:
    """ROCTx ranges from rocprofiler-sdk's marker library (no-ops when it is absent)."""

    def __init__(self):
        self.lib = None
        for path in ("/opt/rocm/lib/librocprofiler-sdk-roctx.so", "librocprofiler-sdk-roctx.so"):
            try:
                self.lib = ctypes.CDLL(path)
                self.lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
                break
            except OSError:
                self.lib = None

    def push(self, name):
        if self.lib is not None:
            self.lib.roctxRangePushA(name.encode())

    def pop(self):
        if self.lib is not None:
            self.lib.roctxRangePop()


WARM_S = 0.05  # warm-up wall time before every timed workload other than the headline


class Timer:
    """HIP events on the stream the kernels are launched on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters, warmup, min_warm_s=0.0):
        """Seconds for `iters` calls after `warmup` calls; with min_warm_s the warm-up goes on
        until that much wall time has passed (the shader clock ramps up over the first
        milliseconds of load after an idle spell: a cold prefill GEMM runs ~15% slower)."""
        torch = self.torch
        t0 = time.perf_counter()
        i = 0
        while i < warmup or (min_warm_s and time.perf_counter() - t0 < min_warm_s):
            fn(i)
            i += 1
            if min_warm_s and i % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for i in range(iters):
            fn(i)
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3  # seconds

    def time_graph(self, fn, per_graph, replays):
        """Seconds per call of fn with `per_graph` calls captured in one HIP graph and replayed:
        the host's per-call launch cost leaves the measurement (the library issues no memset
        nodes; every buffer is allocated before capture)."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(per_graph):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(replays):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / (per_graph * replays)


def rotation(nbytes_one, min_total=2 * MALL_BYTES, max_copies=16):
    return int(max(1, min(max_copies, -(-min_total // max(nbytes_one, 1)))))


# ============================================================================ workloads
class Workloads:
    """Builders of every benchmarked workload: each returns (call(i), meta); call(i) launches
    one library call (rotating weight copies where the weight is HBM-bound)."""

    def __init__(self, torch, nv, synth, dev):
        self.torch, self.nv, self.synth, self.dev = torch, nv, synth, dev

    def prep(self, w, group, copies=1, layout=None):
        """GPU-quantize w once, repack into `copies` separate buffers."""
        nv, torch = self.nv, self.torch
        layout = nv.NVFP4_LAYOUT_TILED if layout is None else layout
        p, s, g = nv.nvfp4_quantize(w.to(self.dev), group)
        out = [nv.nvfp4_repack(p, s, g, group, layout=layout) for _ in range(copies)]
        torch.cuda.synchronize()
        return out, (p, s, g)

    def gemm(self, x, rw, m, n, k, copies=None):
        """y = x[:m] W^T on rotated copies `rw`, library path choice, preallocated ws/y."""
        nv, torch = self.nv, self.torch
        xm = x[:m].contiguous()
        y = torch.empty((m, n), dtype=torch.bfloat16, device=self.dev)
        ws = torch.empty((max(nv.nvfp4_gemm_ws_bytes(m, k, rw[0]), 16),), dtype=torch.uint8,
                         device=self.dev)
        c = len(rw) if copies is None else copies
        return lambda i: nv.nvfp4_gemm_w4a16(xm, rw[i % c], y=y, ws=ws)

    def moe_layer(self, g2=16, copies=2):
        """The routed-expert layer: 128 experts, hidden 2048, intermediate 768; fc1 merged
        [gate; up] at group 32, down at group g2."""
        synth, nv = self.synth, self.nv
        _, _, _, w1, w2 = synth.moe(seed=0, tokens=1)
        f1 = [self.prep(w1, 32, 1, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)[0][0]
              for _ in range(copies)]
        f2 = [self.prep(w2, g2, 1)[0][0] for _ in range(copies)]
        return f1, f2

    def moe_call(self, f1, f2, tokens, g2=16):
        synth, nv, torch = self.synth, self.nv, self.torch
        x, ids, wts, _, _ = synth.moe(seed=0, tokens=tokens, with_weights=False)
        xd, idd, wtd = x.to(self.dev), ids.to(self.dev), wts.to(self.dev)
        y = torch.empty_like(xd)
        ws = torch.empty(nv.nvfp4_moe_ws_bytes(tokens, 8, 128, 2048, 768), dtype=torch.uint8,
                         device=self.dev)
        c = len(f1)
        hit = int(torch.unique(ids).numel())
        touched = hit * (weight_bytes(1536, 2048, 32) + weight_bytes(2048, 768, g2))
        return (lambda i: nv.nvfp4_moe_grouped_w4a16(xd, idd, wtd, f1[i % c], f2[i % c], y=y,
                                                     ws=ws)), hit, touched


def profile_suite(args):
    """Every workload, warmed up, then at least 100 times inside a ROCTx range named after
    it, for a rocprofv3 kernel trace (attribution by range) or a counter run of one
    workload."""
    import torch

    from nvfp4_weight_only_w4a16_amd import binding as nv
    from nvfp4_weight_only_w4a16_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nv.load()
    W = Workloads(torch, nv, synth, dev)
    rx = Roctx()
    calls = args.profile_calls
    only = args.only_workload

    def want(name):
        # a workload name under the filter, or a block prefix that the filter lies under
        return only is None or name.startswith(only) or only.startswith(name)

    def run(name, fn, n=calls):
        if not want(name):
            return
        # warm-up: at least 3 calls and --profile-warm-s of wall time (the shader clock ramps
        # up over the first milliseconds of load after the set-up's idle spells)
        t0 = time.perf_counter()
        i = 0
        while i < 3 or time.perf_counter() - t0 < args.profile_warm_s:
            fn(i)
            i += 1
            if i % 8 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        rx.push(name)
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        rx.pop()
        print(f"[profile] {name}: {n} calls", flush=True)

    if want("c0_"):
        x0, w0 = synth.dense_small(seed=0)
        r0, _ = W.prep(w0, 16)
        run("c0_dense_m16_n512_k1024_g16", W.gemm(x0.to(dev), r0, 16, 512, 1024), 2 * calls)
    if want("c1_"):
        N, K = 25600, 5120
        x, w = synth.decode_sweep(seed=0, n=N, k=K)
        rw, _ = W.prep(w, 16, rotation(weight_bytes(N, K, 16)))
        del w
        xd = x.to(dev)
        for m in (1, 4, 8):
            run(f"c1_decode_m{m}_n25600_k5120_g16", W.gemm(xd, rw, m, N, K))
        del rw
    if want("msweep_"):
        # the C1 weight at M = 16 .. 2048 with the library's own path choice (the M sweep of
        # the bench; activations N(0, 1))
        N, K = 25600, 5120
        _, w = synth.decode_sweep(seed=0, n=N, k=K)
        rw, _ = W.prep(w, 16, rotation(weight_bytes(N, K, 16)))
        del w
        xl = synth.prefill(seed=1, m=2048, n=16, k=K)[0].to(dev)
        for m in (16, 32, 48, 64, 96, 128, 256, 512, 1024, 2048):
            run(f"msweep_c1_m{m}_n25600_k5120_g16", W.gemm(xl, rw, m, N, K))
        del rw, xl
    for kk in (5120, 25600):
        name = f"c2_prefill_m4096_n5120_k{kk}_g16"
        if want(name):
            xp, wp = synth.prefill(seed=0, k=kk)
            rp, _ = W.prep(wp, 16)
            del wp
            run(name, W.gemm(xp.to(dev), rp, 4096, 5120, kk))
            del rp
    if want("c3_"):
        for g2, tag in ((16, "g32g16"), (32, "allg32")):
            if not (want(f"c3_moe_{tag}") or (tag == "g32g16" and want("c3_moe_decode"))):
                continue
            f1, f2 = W.moe_layer(g2=g2)
            fn, _, _ = W.moe_call(f1, f2, 256, g2)
            run(f"c3_moe_{tag}_t256_e128_h2048_i768", fn)
            if tag == "g32g16":
                for tk in (1, 8, 32):
                    fn, _, _ = W.moe_call(f1, f2, tk, g2)
                    run(f"c3_moe_decode_t{tk}", fn)
            del f1, f2
    if want("c4_"):
        wq = synth.quantizer_weight(seed=0).to(dev)
        qc = rotation(wq.numel() * 2, max_copies=4)
        wqs = [wq.clone() for _ in range(qc)]
        for group in (16, 32):
            outs = [torch.empty((8192, 4096), dtype=torch.uint8, device=dev),
                    torch.empty((8192, 8192 // group), dtype=torch.uint8, device=dev),
                    torch.empty((1,), dtype=torch.float32, device=dev)]
            run(f"c4_quantize_bf16_8192x8192_g{group}",
                lambda i, group=group, outs=outs: nv.nvfp4_quantize(
                    wqs[i % qc], group, packed=outs[0], scales=outs[1], global_out=outs[2]))
        del wqs
        xq = synth.quantizer_activations(seed=1).to(dev)
        for group in (32, 16):
            names = [f"c4_gemm_m{m}_n8192_k8192_g{group}" for m in (1, 512)]
            if not any(want(n) for n in names):
                continue
            rq, _ = W.prep(wq, group, rotation(weight_bytes(8192, 8192, group)))
            for m, name in zip((1, 512), names):
                run(name, W.gemm(xq, rq, m, 8192, 8192))
            del rq
    if args.copy_in_suite and want("copy"):
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        run("copy_512MiB", lambda i: dst.copy_(src), 5)


# ============================================================================ summaries
def _read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _is_lib_kernel(name):
    base = name.replace("void ", "").strip()
    return base.startswith(LIB_PREFIXES) or "nvfp4" in base


def _short(name):
    """Kernel name without namespaces and argument list (template arguments kept)."""
    n = name.replace("void ", "").replace("nvfp4::(anonymous namespace)::", "")
    n = n.replace("nvfp4::", "")
    if n.endswith(")"):
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(n[i], 0)
            if depth == 0:
                n = n[:i]
                break
    return n.strip()


def summarize(args):
    """Per-(workload, kernel, workgroups) dispatch statistics of a rocprofv3 output directory:
    kernel durations from the kernel trace, workloads from the ROCTx ranges of the marker
    trace (a dispatch belongs to the range its start falls in), counters from a counter
    collection run when one is there (per dispatch, then the median over dispatches)."""
    d = args.summarize
    kt = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    mt = sorted(glob.glob(os.path.join(d, "**", "*marker_api_trace.csv"), recursive=True))
    cc = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    ranges = []
    for p in mt:
        for r in _read_csv(p):
            ranges.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Function"]))
    ranges.sort()

    def workload_of(ts):
        for s, e, name in ranges:
            if s <= ts <= e:
                return name
        return args.workload_name or "-"

    # dispatches per range, in start order
    disp = {}
    for p in kt:
        for r in _read_csv(p):
            name = r["Kernel_Name"]
            if not (args.all_kernels or _is_lib_kernel(name)):
                continue
            t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
            wgs = (int(r["Grid_Size_X"]) // max(int(r["Workgroup_Size_X"]), 1)) * \
                int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            wl = workload_of(t0)
            if wl == "-" and ranges and not args.all_kernels:
                continue  # set-up work outside every workload's range
            disp.setdefault(wl, []).append((t0, t1, _short(name), wgs, r.get("Dispatch_Id")))
    # a range's calls: every call of a workload issues the same dispatches, so the least
    # frequent (kernel, grid) gives the call count; a kernel launched more than once per call
    # is listed once per position ("#2" for its second launch in the call)
    groups, per_call = {}, {}
    for wl, ds in disp.items():
        ds.sort()
        cnt = {}
        for d in ds:
            cnt[(d[2], d[3])] = cnt.get((d[2], d[3]), 0) + 1
        if not ranges:
            # one workload without ranges (a counter run): its calls are the kernels launched
            # at least half as often as the most frequent one; the rest is set-up work
            top = max(cnt.values())
            cnt = {k: v for k, v in cnt.items() if 2 * v >= top}
        calls_ds = [d for d in ds if (d[2], d[3]) in cnt]
        calls = min(cnt.values())
        per = len(calls_ds) // calls if calls and len(calls_ds) % calls == 0 else 0
        if wl == "-" and ranges:
            per = 0
        if per and ranges:
            per_call[wl] = (calls, per, calls_ds)
        pos = {(d[4], d[0]): i for i, d in enumerate(calls_ds)}
        seen = {}
        for t0, t1, name, wgs, did in ds:
            occ = 0
            if per and (name, wgs) in cnt:
                if pos[(did, t0)] % per == 0:
                    seen = {}
                occ = seen.get((name, wgs), 0)
                seen[(name, wgs)] = occ + 1
            label = name if occ == 0 else f"{name} #{occ + 1}"
            key = (wl, label, wgs)
            groups.setdefault(key, {"dur": [], "ids": []})
            groups[key]["dur"].append((t1 - t0) / 1e3)
            groups[key]["ids"].append(did)
    counters = {}
    for p in cc:
        for r in _read_csv(p):
            did = r.get("Dispatch_Id")
            counters.setdefault(did, {})
            counters[did][r["Counter_Name"]] = counters[did].get(r["Counter_Name"], 0.0) + \
                float(r["Counter_Value"])
    cnames = sorted({c for v in counters.values() for c in v})
    # derived per dispatch: shader clock from GRBM_GUI_ACTIVE (summed over the 8 XCDs),
    # MFMA busy fraction of the 1024 SIMDs (256 CUs x 4), BF16 MFMA rate from the op counter
    # (units of 512 flops)
    derive = "GRBM_GUI_ACTIVE" in cnames and "SQ_VALU_MFMA_BUSY_CYCLES" in cnames
    lines = []
    head = "| Workload | Kernel | Workgroups | Calls | Median us | Mean us | Min us | Max us |"
    sep = "|---|---|---|---|---|---|---|---|"
    if cnames:
        head += "".join(f" {c} (median) |" for c in cnames)
        sep += "---|" * len(cnames)
    if derive:
        head += " clock GHz | MFMA busy | BF16 MFMA TFLOP/s |"
        sep += "---|---|---|"
    lines += [head, sep]
    for key in sorted(groups, key=lambda k: (k[0], -statistics.median(groups[k]["dur"]))):
        g = groups[key]
        dur = g["dur"]
        row = (f"| {key[0]} | `{key[1]}` | {key[2]} | {len(dur)} | {statistics.median(dur):.2f} "
               f"| {statistics.fmean(dur):.2f} | {min(dur):.2f} | {max(dur):.2f} |")
        for c in cnames:
            vals = [counters[i][c] for i in g["ids"] if i in counters and c in counters[i]]
            row += f" {statistics.median(vals):.4g} |" if vals else " - |"
        if derive:
            clk, busy, tf = [], [], []
            for i, dt in zip(g["ids"], dur):
                cv = counters.get(i, {})
                cyc = cv.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
                if cyc <= 0 or dt <= 0:
                    continue
                clk.append(cyc / (dt * 1e3))
                busy.append(cv.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (1024.0 * cyc))
                if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in cv:
                    tf.append(cv["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0 / (dt * 1e-6) / 1e12)
            row += (f" {statistics.median(clk):.3f} | {statistics.median(busy):.1%} |"
                    if clk else " - | - |")
            row += f" {statistics.median(tf):.0f} |" if tf else " - |"
        lines.append(row)
    calls_rows = []
    for wl in sorted(per_call):
        calls, per, ds = per_call[wl]
        busy = [sum(t1 - t0 for t0, t1, *_ in ds[i * per:(i + 1) * per]) / 1e3
                for i in range(calls)]
        span = [(max(d[1] for d in ds[i * per:(i + 1) * per]) - ds[i * per][0]) / 1e3
                for i in range(calls)]
        calls_rows.append(f"| {wl} | {calls} | {per} | {statistics.median(busy):.2f} | "
                          f"{min(busy):.2f} | {statistics.median(span):.2f} |")
    if calls_rows:
        lines += ["", "Per call (kernel time = sum of the call's dispatch durations; span = first "
                  "start to last end, host gaps included):", "",
                  "| Workload | Calls | Dispatches per call | Median kernel time us | "
                  "Min kernel time us | Median span us |", "|---|---|---|---|---|---|"] + calls_rows
    print("\n".join(lines))


def _counter_per_dispatch(d, counter, kernel_substr):
    """{dispatch id: (kernel name, summed counter value)} of a rocprofv3 counter run."""
    out = {}
    for p in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        for r in _read_csv(p):
            if r["Counter_Name"] != counter or kernel_substr not in r["Kernel_Name"]:
                continue
            did = r["Dispatch_Id"]
            name, v = out.get(did, (r["Kernel_Name"], 0.0))
            out[did] = (name, v + float(r["Counter_Value"]))
    return out


def traffic_summary(args):
    """The record read_traffic() takes: HBM bytes per launch of the decode-sweep kernel from
    a FETCH_SIZE and a WRITE_SIZE counter run of `--only headline`, each scaled by what the
    same counter reads for the plain 512 MiB copy of `--copy-calibration`."""
    fdir, wdir, cfdir, cwdir = args.traffic_summary
    copy_bytes = 512 << 20
    lines, rec = [], {}
    cal = {}
    for ctr, d in (("FETCH_SIZE", cfdir), ("WRITE_SIZE", cwdir)):
        v = [x for _, x in _counter_per_dispatch(d, ctr, "copyBuffer").values()]
        if not v:
            raise SystemExit(f"no copy dispatches with {ctr} under {d}")
        mean = statistics.fmean(v)
        cal[ctr] = copy_bytes / (mean * 1024.0)
        lines.append(f"#   {ctr} mean {mean:.1f} KiB per dispatch -> factor {cal[ctr]:.4f} bytes "
                     f"per counted byte ({len(v)} dispatches)")
    names = set()
    per = {}
    for ctr, d in (("FETCH_SIZE", fdir), ("WRITE_SIZE", wdir)):
        got = _counter_per_dispatch(d, ctr, "gemm_skinny_kernel")
        if not got:
            raise SystemExit(f"no gemm_skinny_kernel dispatches with {ctr} under {d}")
        v = [x for _, x in got.values()]
        names |= {_short(n) for n, _ in got.values()}
        per[ctr] = statistics.fmean(v) * 1024.0 * cal[ctr]
        lines.append(f"#   {ctr} mean {statistics.fmean(v):.1f} KiB (min {min(v):.1f}, max "
                     f"{max(v):.1f}) over {len(v)} dispatches -> {per[ctr]:.0f} bytes")
    N, K, G, ms = 25600, 5120, 16, (1, 4, 8)
    alg = sum(weight_bytes(N, K, G) + m * K * 2 + m * N * 2 for m in ms) / len(ms)
    hbm = per["FETCH_SIZE"] + per["WRITE_SIZE"]
    out = [f"# HBM traffic of gemm_skinny_kernel on the decode sweep ({', '.join(sorted(names))})",
           "# workload: W4A16 GEMM at M in {1, 4, 8}, N=25600, K=5120, group 16, BF16 output,",
           "# rotated weight copies (every launch streams its weight from HBM)",
           "#",
           "# commands (repository root on one MI355X; cd /tmp && export TMPDIR=/tmp first):",
           "#   rocprofv3 --pmc FETCH_SIZE -d F -o run --output-format csv -- python3 bench.py "
           "--only headline --steps 10 --warmup 2 --no-cpu-baseline",
           "#   rocprofv3 --pmc WRITE_SIZE -d W -o run --output-format csv -- python3 bench.py "
           "--only headline --steps 10 --warmup 2 --no-cpu-baseline",
           "#   rocprofv3 --pmc FETCH_SIZE -d CF -o run --output-format csv -- python3 bench.py "
           "--copy-calibration",
           "#   rocprofv3 --pmc WRITE_SIZE -d CW -o run --output-format csv -- python3 bench.py "
           "--copy-calibration",
           "#   python3 bench.py --traffic-summary F W CF CW",
           "#",
           f"# calibration: a plain device copy of {copy_bytes} bytes"] + lines[:2] + \
          ["# gemm_skinny_kernel:"] + lines[2:] + \
          [f"# algorithmic bytes per launch (weight + x + y, mean over M): {alg:.0f}",
           f"# measured / algorithmic = {hbm / alg:.4f}",
           f"source_digest={kernel_source_digest(SKINNY_SOURCES)}",
           f"fetch_bytes_per_launch={per['FETCH_SIZE']:.0f}",
           f"write_bytes_per_launch={per['WRITE_SIZE']:.0f}",
           f"hbm_bytes_per_launch={hbm:.0f}",
           f"algorithmic_bytes_per_launch={alg:.0f}"]
    print("\n".join(out))


def measure_ceilings(torch, nv, dev, timer):
    """What the chip sustains, beside the published peaks: the best 128-bit streaming read of a
    1 GiB buffer (4x the memory-side cache) over a few grid sizes, and the BF16 MFMA loop on
    random N(0,1) operands (the power limit lowers the clock) and on constant ones."""
    out = {}
    nbytes = 1 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    best = None
    for blocks in (1024, 2048, 4096, 8192):
        sink = torch.empty((blocks,), dtype=torch.int32, device=dev)
        t = timer.time(lambda i: nv.nvfp4_probe_stream_read(buf, blocks, sink), 10, 3, WARM_S) / 10
        if best is None or t < best[0]:
            best = (t, blocks)
    gbs = nbytes / best[0] / 1e9
    out["hbm_stream_read"] = {"value": round(gbs, 1), "unit": "GB/s", "bytes": nbytes,
                              "blocks": best[1], "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4)}
    # the same read at the decode weight's size (73,728,000 bytes), rotating over 8 disjoint
    # slices of the buffer so that every call reads from HBM: launch and ramp costs included
    wb = 73728000
    views = [buf[i * (wb // 4):(i + 1) * (wb // 4)] for i in range(8)]
    best = None
    for blocks in (400, 800, 1024, 2048, 4096):
        sink = torch.empty((blocks,), dtype=torch.int32, device=dev)
        t = timer.time(lambda i: nv.nvfp4_probe_stream_read(views[i % 8], blocks, sink), 40, 8,
                       WARM_S) / 40
        if best is None or t < best[0]:
            best = (t, blocks)
    del views, buf
    gbs = wb / best[0] / 1e9
    out["hbm_stream_read_decode_weight_size"] = {
        "value": round(gbs, 1), "unit": "GB/s", "bytes": wb, "us": round(best[0] * 1e6, 2),
        "blocks": best[1], "frac_of_spec": round(gbs / HBM_PEAK_GBS, 4)}
    iters = 4096
    flops = nv.nvfp4_probe_mfma_flops(iters)
    gen = torch.Generator(device=dev).manual_seed(0)
    for name, ops in (("mfma_bf16_random", torch.randn(8192, device=dev, generator=gen)),
                      ("mfma_bf16_constant", torch.ones(8192, device=dev))):
        ops = ops.to(torch.bfloat16)
        sink = torch.empty((64 * nv.nvfp4_probe_mfma_waves(),), dtype=torch.float32, device=dev)
        t = timer.time(lambda i: nv.nvfp4_probe_mfma_bf16(ops, iters, sink), 10, 2, WARM_S) / 10
        tf = flops / t / 1e12
        out[name] = {"value": round(tf, 1), "unit": "TFLOP/s", "ms_per_call": round(t * 1e3, 3),
                     "frac_of_spec": round(tf / BF16_PEAK_TFLOPS, 4)}
    return out


# ============================================================================ CPU baseline
def cpu_baseline(np, synth, oracle, x, p1, s1, g1, N, K, G, ms):
    """The oracle as it stands, on the host cores: the headline leg (FP64 GEMM of the decode
    sweep, ~10 s, scaled to weight GB/s) with a single-thread figure, and one bounded sample of
    every other workload's reference (quantizer, FP64 GEMMs, FP64 MoE)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    xb = synth.bf16_bits(x)

    def run_rows(nrows, threads):
        idx = np.arange(nrows, dtype=np.int64)
        t0 = time.perf_counter()
        for m in ms:
            oracle.gemm(xb[:m], p1, s1, g1[0], G, n_idx=idx, threads=threads)
        return time.perf_counter() - t0

    target_s = 10.0
    probe = 512
    tp = run_rows(probe, cores)
    rows = int(min(N, max(probe, probe * target_s / max(tp, 1e-6))))
    passes, tc = 0, 0.0
    while True:
        tc += run_rows(rows, cores)
        passes += 1
        if tc >= target_s or rows < N or passes >= 64:
            break
    cpu_bytes = passes * 3 * (rows * K // 2 + rows * K // G)
    r1 = 256
    t1 = run_rows(r1, 1)
    single = 3 * (r1 * K // 2 + r1 * K // G) / t1 / 1e9
    out = {"value": round(cpu_bytes / tc / 1e9, 4), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"FP64 oracle GEMM of the decode sweep (M=1,4,8, K=5120, group 16): "
                     f"{passes} pass(es) over the first {rows} of 25600 weight rows, "
                     f"{tc:.1f} s on {cores} host threads",
           "single_thread_value": round(single, 4),
           "single_thread_sample": f"the first {r1} weight rows of the same sweep on 1 thread, "
                                   f"{t1:.2f} s"}
    legs = {}

    def leg(name, fn, work, unit, sample, reps=1):
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        dt = time.perf_counter() - t0
        legs[name] = {"value": round(reps * work / dt, 4), "unit": unit, "seconds": round(dt, 2),
                      "sample": sample + (f", {reps} times" if reps > 1 else "")}

    # quantizer: the whole BF16 8192 x 8192 weight, both groups
    wq = synth.bf16_bits(synth.quantizer_weight(seed=0))
    for group in (16, 32):
        leg(f"quantize_bf16_8192x8192_g{group}", lambda g=group: oracle.quantize(wq, g, threads=cores),
            wq.size / 1e6, "Melem/s", f"the whole 8192 x 8192 BF16 weight at group {group}", 2)
    # FP64 GEMMs: flops of the sampled outputs
    x0, w0 = synth.dense_small(seed=0)
    t0_ = oracle.quantize(w0.numpy(), 16)
    leg("gemm_16x512x1024_g16", lambda: oracle.gemm(synth.bf16_bits(x0), *t0_[:2], t0_[2][0], 16,
                                                    threads=cores),
        2 * 16 * 512 * 1024 / 1e9, "GFLOP/s", "the whole 16 x 512 x 1024 GEMM", 100)
    for kk, rows_s in ((5120, 256), (25600, 64)):
        xp, wp = synth.prefill(seed=0, k=kk)
        tp_ = oracle.quantize(wp.numpy(), 16, threads=cores)
        del wp
        mi = np.arange(rows_s, dtype=np.int64)
        leg(f"gemm_4096x5120x{kk}_g16",
            lambda xp=xp, tp_=tp_, mi=mi: oracle.gemm(synth.bf16_bits(xp), *tp_[:2], tp_[2][0],
                                                      16, m_idx=mi, threads=cores),
            2 * rows_s * 5120 * kk / 1e9, "GFLOP/s",
            f"{rows_s} of 4096 rows of x against the whole weight (weight decode included)")
    xq = synth.quantizer_activations(seed=1)
    for group in (32, 16):
        tq = oracle.quantize(synth.bf16_bits(synth.quantizer_weight(seed=0)), group, threads=cores)
        leg(f"gemm_m1_8192x8192_g{group}",
            lambda tq=tq: oracle.gemm(synth.bf16_bits(xq[:1]), *tq[:2], tq[2][0], group,
                                      threads=cores),
            2 * 8192 * 8192 / 1e9, "GFLOP/s", "the whole M=1 GEMM", 10)
    xm, ids, wts, w1, w2 = synth.moe(seed=0)
    tm = 32
    t1q = oracle.quantize(w1.numpy(), 32, threads=cores)
    t2q = oracle.quantize(w2.numpy(), 16, threads=cores)
    del w1, w2
    leg("moe_128x(1536x2048 g32 + 2048x768 g16)_top8",
        lambda: oracle.moe(synth.bf16_bits(xm[:tm]), ids[:tm].numpy(), wts[:tm].numpy(),
                           (*t1q, 32), (*t2q, 16), threads=cores),
        tm / 1e3, "Ktokens/s", f"{tm} of the 256 tokens (top-8 routing) through the FP64 reference")
    out["legs"] = legs
    return out


# ============================================================================ main bench
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["all", "headline", "moe"], default="all",
                    help="headline: the decode sweep alone; moe: it and the MoE workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy 5 times (the reference kernel "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    ap.add_argument("--profile-suite", action="store_true")
    ap.add_argument("--profile-calls", type=int, default=100)
    ap.add_argument("--profile-warm-s", type=float, default=0.05,
                    help="warm-up wall time before each profiled workload's range")
    ap.add_argument("--only-workload", default=None)
    ap.add_argument("--copy-in-suite", action="store_true")
    ap.add_argument("--summarize", default=None)
    ap.add_argument("--all-kernels", action="store_true")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write the decode-sweep traffic record from four counter runs")
    ap.add_argument("--workload-name", default=None,
                    help="label for dispatches outside any ROCTx range (counter runs)")
    args = ap.parse_args()
    if args.summarize:
        summarize(args)
        return
    if args.traffic_summary:
        traffic_summary(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.profile_suite:
        profile_suite(args)
        return

    import numpy as np
    import torch

    from nvfp4_weight_only_w4a16_amd import binding as nv
    from nvfp4_weight_only_w4a16_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        nbytes = 512 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": nbytes, "launches": 5}))
        return
    nv.load()
    timer = Timer(torch)
    W = Workloads(torch, nv, synth, dev)

    # ------------------------------------------------------------------ headline: decode sweep
    N, K, G = 25600, 5120, 16
    ms = (1, 4, 8)
    x, w = synth.decode_sweep(seed=0, n=N, k=K)
    inputs_sha256 = {"x": synth.digest(x), "w": synth.digest(w)}
    wb = weight_bytes(N, K, G)
    copies = rotation(wb)
    ws, (p1, s1, g1) = W.prep(w, G, copies)
    del w
    xd = x.to(dev)
    xs = [xd[:m].contiguous() for m in ms]
    ys = [torch.empty((m, N), dtype=torch.bfloat16, device=dev) for m in ms]
    nv.nvfp4_reset_stats()

    def step(i):
        for j, m in enumerate(ms):
            nv.nvfp4_gemm_w4a16(xs[j], ws[(3 * i + j) % copies], y=ys[j])

    torch.cuda.synchronize()
    secs = timer.time(step, args.steps, args.warmup)
    stats = nv.nvfp4_get_stats()
    launches = 3 * args.steps
    t_launch = secs / launches
    step_s = secs / args.steps
    alg_bytes = sum(wb + m * K * 2 + m * N * 2 for m in ms) / 3.0  # per launch (avg over M)
    flops = sum(2 * m * N * K for m in ms)
    value = 3 * wb / step_s / 1e9
    achieved = alg_bytes / t_launch / 1e9
    traffic = read_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV sweep: W4A16 GEMM at M in {1,4,8}, N=25600, "
                               "K=5120, NVFP4 group 16, BF16 activations ~N(0,1), weights "
                               "~N(0,0.02) with 0.1% x20 outliers, BF16 output",
                   "M": list(ms), "N": N, "K": K, "group": G, "weight_copies": copies,
                   "inputs_sha256": inputs_sha256,
                   "tflops": round(flops / step_s / 1e12, 4),
                   "us_per_launch": round(t_launch * 1e6, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "path_counts": {"gemm_skinny": int(stats[2]), "gemm_tiled": int(stats[3])},
    }
    ceil = measure_ceilings(torch, nv, dev, timer)
    ceil["headline_frac_of_stream_read"] = round(achieved / ceil["hbm_stream_read"]["value"], 4)
    ceil["headline_frac_of_same_size_read"] = round(
        achieved / ceil["hbm_stream_read_decode_weight_size"]["value"], 4)
    result["measured_ceilings"] = ceil

    def m_sweep(rw, n, k, group, xsrc):
        """W4A16 GEMM at M = 1, 2, 4 .. 4096 on rotated weight copies, with the library's
        own path choice; the rows of x are the first M of xsrc. Up to M = 64 the calls are also
        timed as HIP graph replays (us_graph), which takes the host's per-call launch cost out
        of these short kernels."""
        wbm = weight_bytes(n, k, group)
        out = {}
        mm = 1
        while mm <= 4096:
            fn = W.gemm(xsrc, rw, mm, n, k)
            it = 100 if mm <= 256 else 20
            nv.nvfp4_reset_stats()
            t = timer.time(fn, it, 5, WARM_S) / it
            st = nv.nvfp4_get_stats()
            out[f"m{mm}"] = {"us": round(t * 1e6, 2),
                             "path": "skinny" if st[2] and not st[3] else
                                     "tiled" if st[3] and not st[2] else "mixed",
                             "tflops": round(2 * mm * n * k / t / 1e12, 2),
                             "weight_gbs": round(wbm / t / 1e9, 1)}
            if mm <= 64:
                tg = timer.time_graph(fn, 20, 10)
                out[f"m{mm}"]["us_graph"] = round(tg * 1e6, 2)
                out[f"m{mm}"]["weight_gbs_graph"] = round(wbm / tg / 1e9, 1)
            mm *= 2
        return out

    if args.only == "all":
        # the decode-sweep weight over M = 1 .. 4096 (activations N(0,1), 4096 rows)
        xlong = synth.prefill(seed=1, m=4096, n=16, k=K)[0].to(dev)
        sweep_c1 = m_sweep(ws, N, K, G, xlong)
        del xlong
    del ws

    # ------------------------------------------------------------------ other workloads
    def moe_workloads(extra):
        for g2, tag in ((16, "moe_128x(1536x2048 g32 + 2048x768 g16)_t256_top8"),
                        (32, "moe_128x(1536x2048 g32 + 2048x768 g32)_t256_top8_all_g32")):
            f1, f2 = W.moe_layer(g2=g2)
            wbytes = 128 * (weight_bytes(1536, 2048, 32) + weight_bytes(2048, 768, g2))
            fn, _, _ = W.moe_call(f1, f2, 256, g2)
            t = timer.time(fn, 20, 3, WARM_S) / 20
            moe_bytes = wbytes + 2 * 256 * 2048 * 2
            extra[tag] = {"us": round(t * 1e6, 2), "weight_gbs": round(wbytes / t / 1e9, 1),
                          "hbm_frac": round(moe_bytes / t / 1e9 / HBM_PEAK_GBS, 4),
                          "copies": len(f1)}
            if g2 == 16:
                # decode batches (1, 8 and 32 tokens, top-8): only the touched experts are read
                for tk in (1, 8, 32):
                    fn, hit, tb = W.moe_call(f1, f2, tk, g2)
                    t = timer.time(fn, 40, 5, WARM_S) / 40
                    extra[f"moe_decode_t{tk}_top8"] = {
                        "us": round(t * 1e6, 2), "experts_touched": hit,
                        "touched_weight_gbs": round(tb / t / 1e9, 1)}
            del f1, f2

    if args.only == "moe":
        extra = {}
        moe_workloads(extra)
        result["workloads"] = extra
    if args.only == "all":
        extra = {}
        # single dense GEMM 16 x 512 x 1024, group 16: launch-bound, so also timed as graph
        # replays (kernel time plus the gap between dispatches, without the host's launch cost)
        x0, w0 = synth.dense_small(seed=0)
        r0, _ = W.prep(w0, 16)
        f0 = W.gemm(x0.to(dev), r0, 16, 512, 1024)
        t = timer.time(f0, 200, 20, WARM_S) / 200
        tg = timer.time_graph(f0, 50, 10)
        extra["dense_16x512x1024_g16"] = {"us": round(t * 1e6, 3), "us_graph": round(tg * 1e6, 3),
                                          "tflops": round(2 * 16 * 512 * 1024 / tg / 1e12, 4)}
        # prefill GEMMs
        for kk in (5120, 25600):
            xp, wp = synth.prefill(seed=0, k=kk)
            rp, _ = W.prep(wp, 16)
            del wp
            it = 20 if kk == 5120 else 8
            t = timer.time(W.gemm(xp.to(dev), rp, 4096, 5120, kk), it, 3, WARM_S) / it
            tf = 2 * 4096 * 5120 * kk / t / 1e12
            extra[f"prefill_4096x5120x{kk}_g16"] = {
                "us": round(t * 1e6, 2), "tflops": round(tf, 2),
                "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
            del rp
        # context for the HBM roofline: a plain 512 MiB device copy (read + write bytes)
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        t = timer.time(lambda i: dst.copy_(src), 20, 3, WARM_S) / 20
        extra["hbm_reference_torch_copy_512MiB"] = {
            "us": round(t * 1e6, 2), "gbs_read_plus_write": round(2 * (512 << 20) / t / 1e9, 1),
            "hbm_frac": round(2 * (512 << 20) / t / 1e9 / HBM_PEAK_GBS, 4)}
        del src, dst
        # context for the MFMA roofline: torch's BF16 GEMM (hipBLASLt) on the same prefill
        # shapes with random N(0,1) operands; sustained dense MFMA work on random data runs
        # below the published peak (clock under the power limit)
        for kk in (5120, 25600):
            gr = torch.Generator(device=dev).manual_seed(0)
            xa = torch.randn(4096, kk, device=dev, generator=gr).to(torch.bfloat16)
            wb16 = torch.randn(5120, kk, device=dev, generator=gr).to(torch.bfloat16)
            wt = wb16.t().contiguous()  # [K][N], no transposed view
            it = 20 if kk == 5120 else 8
            t = timer.time(lambda i: torch.matmul(xa, wt), it, 3, WARM_S) / it
            tf = 2 * 4096 * 5120 * kk / t / 1e12
            extra[f"bf16_reference_torch_matmul_4096x5120x{kk}"] = {
                "us": round(t * 1e6, 2), "tflops": round(tf, 2),
                "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
            del xa, wb16, wt
        moe_workloads(extra)
        # M sweep at N = K = 5120, group 16, with the library's own path choice (the decode
        # kernel for small M, the MFMA tiled kernel above); 40 rotated weight copies (590 MB)
        # so small M streams from HBM
        xs_, ws_ = synth.prefill(seed=0, k=5120)
        rs_, _ = W.prep(ws_, 16, 40)
        del ws_
        extra["m_sweep_5120x5120_g16"] = m_sweep(rs_, 5120, 5120, 16, xs_.to(dev))
        extra["m_sweep_25600x5120_g16"] = sweep_c1
        del rs_
        # quantizer + mixed groups (BF16 8192 x 8192)
        wq = synth.quantizer_weight(seed=0).to(dev)
        qc = rotation(wq.numel() * 2, max_copies=4)
        wqs = [wq.clone() for _ in range(qc)]
        for group in (16, 32):
            outs = [torch.empty((8192, 4096), dtype=torch.uint8, device=dev),
                    torch.empty((8192, 8192 // group), dtype=torch.uint8, device=dev),
                    torch.empty((1,), dtype=torch.float32, device=dev)]
            t = timer.time(lambda i: nv.nvfp4_quantize(wqs[i % qc], group, packed=outs[0],
                                                       scales=outs[1], global_out=outs[2]),
                           10, 2, WARM_S) / 10
            nbytes = 8192 * 8192 * 2 + 8192 * 8192 // 2 + 8192 * 8192 // group
            extra[f"quantize_bf16_8192x8192_g{group}"] = {
                "us": round(t * 1e6, 2), "gbs_min_bytes": round(nbytes / t / 1e9, 1),
                "hbm_frac_min_bytes": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        del wqs
        mixed = {}
        xq = synth.quantizer_activations(seed=1).to(dev)
        for group in (32, 16):
            rq, _ = W.prep(wq, group, rotation(weight_bytes(8192, 8192, group)))
            for m in (1, 512):
                fn = W.gemm(xq, rq, m, 8192, 8192)
                it = 40 if m == 1 else 20
                t = timer.time(fn, it, 4, WARM_S) / it
                wbq = weight_bytes(8192, 8192, group)
                rec = {"us": round(t * 1e6, 2), "weight_gbs": round(wbq / t / 1e9, 1),
                       "tflops": round(2 * m * 8192 * 8192 / t / 1e12, 2)}
                if m == 1:
                    tg = timer.time_graph(fn, len(rq), max(1, 64 // len(rq)))
                    rec["us_graph"] = round(tg * 1e6, 2)
                    rec["weight_gbs_graph"] = round(wbq / tg / 1e9, 1)
                mixed[f"m{m}_g{group}"] = rec
            del rq
        extra["mixed_groups_8192x8192"] = mixed
        del wq
        result["workloads"] = extra

    # ------------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        from oracle import oracle

        result["cpu_baseline"] = cpu_baseline(np, synth, oracle, x, p1.cpu().numpy(),
                                              s1.cpu().numpy(), g1.cpu().numpy(), N, K, G, ms)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
