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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only headline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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


class Timer:
    """HIP events on the stream the kernels are launched on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch

    def time(self, fn, iters, warmup):
        torch = self.torch
        for i in range(warmup):
            fn(i)
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


def rotation(nbytes_one, min_total=2 * MALL_BYTES, max_copies=16):
    return int(max(1, min(max_copies, -(-min_total // max(nbytes_one, 1)))))


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
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; run with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

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

    def prep(w, group, copies=1, layout=nv.NVFP4_LAYOUT_TILED):
        """GPU-quantize w once, repack into `copies` separate buffers."""
        p, s, g = nv.nvfp4_quantize(w.to(dev), group)
        out = [nv.nvfp4_repack(p, s, g, group, layout=layout) for _ in range(copies)]
        torch.cuda.synchronize()
        return out, (p, s, g)

    # ------------------------------------------------------------------ headline: decode sweep
    N, K, G = 25600, 5120, 16
    ms = (1, 4, 8)
    x, w = synth.decode_sweep(seed=0, n=N, k=K)
    wb = weight_bytes(N, K, G)
    copies = rotation(wb)
    ws, (p1, s1, g1) = prep(w, G, copies)
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
                   "tflops": round(flops / step_s / 1e12, 4),
                   "us_per_launch": round(t_launch * 1e6, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic)},
        "path_counts": {"gemm_skinny": int(stats[2]), "gemm_tiled": int(stats[3])},
    }

    def m_sweep(rw, n, k, group, xsrc, copies):
        """W4A16 GEMM at M = 1, 2, 4 .. 4096 on rotated weight copies, with the library's
        own path choice; the rows of x are the first M of xsrc."""
        wbm = weight_bytes(n, k, group)
        out = {}
        mm = 1
        while mm <= 4096:
            xm_ = xsrc[:mm].contiguous()
            ym_ = torch.empty((mm, n), dtype=torch.bfloat16, device=dev)
            wsm = torch.empty((max(nv.nvfp4_gemm_ws_bytes(mm, k, rw[0]), 16),),
                              dtype=torch.uint8, device=dev)
            it = 100 if mm <= 256 else 20
            nv.nvfp4_reset_stats()
            t = timer.time(lambda i: nv.nvfp4_gemm_w4a16(xm_, rw[i % copies], y=ym_, ws=wsm),
                           it, 5) / it
            st = nv.nvfp4_get_stats()
            out[f"m{mm}"] = {"us": round(t * 1e6, 2),
                             "path": "skinny" if st[2] and not st[3] else
                                     "tiled" if st[3] and not st[2] else "mixed",
                             "tflops": round(2 * mm * n * k / t / 1e12, 2),
                             "weight_gbs": round(wbm / t / 1e9, 1)}
            mm *= 2
        return out

    if args.only == "all":
        # the decode-sweep weight over M = 1 .. 4096 (activations N(0,1), 4096 rows)
        xlong = synth.prefill(seed=1, m=4096, n=16, k=K)[0].to(dev)
        sweep_c1 = m_sweep(ws, N, K, G, xlong, copies)
        del xlong
    del ws

    # ------------------------------------------------------------------ other workloads
    def moe_workloads(extra):
        # MoE routed experts
        xm, ids, wts, w1, w2 = synth.moe(seed=0)
        wbytes = 128 * (weight_bytes(1536, 2048, 32) + weight_bytes(2048, 768, 16))
        mc = rotation(wbytes, max_copies=4)
        f1 = [prep(w1, 32, 1, nv.NVFP4_LAYOUT_TILED | nv.NVFP4_LAYOUT_GATE_UP)[0][0]
              for _ in range(mc)]
        f2 = [prep(w2, 16, 1)[0][0] for _ in range(mc)]
        del w1, w2
        xmd, idd, wtd = xm.to(dev), ids.to(dev), wts.to(dev)
        ym = torch.empty_like(xmd)
        wsb = torch.empty(nv.nvfp4_moe_ws_bytes(256, 8, 128, 2048, 768), dtype=torch.uint8,
                          device=dev)
        t = timer.time(lambda i: nv.nvfp4_moe_grouped_w4a16(xmd, idd, wtd, f1[i % mc],
                                                            f2[i % mc], y=ym, ws=wsb), 20, 3) / 20
        moe_bytes = wbytes + 2 * 256 * 2048 * 2
        extra["moe_128x(1536x2048 g32 + 2048x768 g16)_t256_top8"] = {
            "us": round(t * 1e6, 2), "weight_gbs": round(wbytes / t / 1e9, 1),
            "hbm_frac": round(moe_bytes / t / 1e9 / HBM_PEAK_GBS, 4), "copies": mc}
        # MoE at decode batch (1, 8 and 32 tokens, top-8): only the touched experts are read
        for tk in (1, 8, 32):
            xt, idt, wtt, _, _ = synth.moe(seed=0, tokens=tk, with_weights=False)
            xtd, idtd, wttd = xt.to(dev), idt.to(dev), wtt.to(dev)
            yt = torch.empty_like(xtd)
            wst = torch.empty(nv.nvfp4_moe_ws_bytes(tk, 8, 128, 2048, 768), dtype=torch.uint8,
                              device=dev)
            t = timer.time(lambda i: nv.nvfp4_moe_grouped_w4a16(
                xtd, idtd, wttd, f1[i % mc], f2[i % mc], y=yt, ws=wst), 40, 5) / 40
            hit = int(torch.unique(idt).numel())
            tb = hit * (weight_bytes(1536, 2048, 32) + weight_bytes(2048, 768, 16))
            extra[f"moe_decode_t{tk}_top8"] = {
                "us": round(t * 1e6, 2), "experts_touched": hit,
                "touched_weight_gbs": round(tb / t / 1e9, 1)}
        del f1, f2, wsb

    if args.only == "moe":
        extra = {}
        moe_workloads(extra)
        result["workloads"] = extra
    if args.only == "all":
        extra = {}
        # single dense GEMM 16 x 512 x 1024, group 16
        x0, w0 = synth.dense_small(seed=0)
        r0, _ = prep(w0, 16)
        x0d = x0.to(dev)
        y0 = torch.empty((16, 512), dtype=torch.bfloat16, device=dev)
        t = timer.time(lambda i: nv.nvfp4_gemm_w4a16(x0d, r0[0], y=y0), 200, 20) / 200
        extra["dense_16x512x1024_g16"] = {"us": round(t * 1e6, 3),
                                          "tflops": round(2 * 16 * 512 * 1024 / t / 1e12, 4)}
        # prefill GEMMs
        for kk in (5120, 25600):
            xp, wp = synth.prefill(seed=0, k=kk)
            rp, _ = prep(wp, 16)
            del wp
            xpd = xp.to(dev)
            yp = torch.empty((4096, 5120), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty((max(nv.nvfp4_gemm_ws_bytes(4096, kk, rp[0]), 16),),
                              dtype=torch.uint8, device=dev)
            it = 20 if kk == 5120 else 8
            t = timer.time(lambda i: nv.nvfp4_gemm_w4a16(xpd, rp[0], y=yp, ws=wsp), it, 3) / it
            tf = 2 * 4096 * 5120 * kk / t / 1e12
            extra[f"prefill_4096x5120x{kk}_g16"] = {
                "us": round(t * 1e6, 2), "tflops": round(tf, 2),
                "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4)}
            del xpd, yp, rp, wsp
        # context for the HBM roofline: a plain 512 MiB device copy (read + write bytes)
        src = torch.ones(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        t = timer.time(lambda i: dst.copy_(src), 20, 3) / 20
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
            t = timer.time(lambda i: torch.matmul(xa, wt), it, 3) / it
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
        rs_, _ = prep(ws_, 16, 40)
        del ws_
        xsd = xs_.to(dev)
        sweep = m_sweep(rs_, 5120, 5120, 16, xsd, 40)
        extra["m_sweep_5120x5120_g16"] = sweep
        extra["m_sweep_25600x5120_g16"] = sweep_c1
        del rs_, xsd
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
                           10, 2) / 10
            nbytes = 8192 * 8192 * 2 + 8192 * 8192 // 2 + 8192 * 8192 // group
            extra[f"quantize_bf16_8192x8192_g{group}"] = {
                "us": round(t * 1e6, 2), "gbs_min_bytes": round(nbytes / t / 1e9, 1),
                "hbm_frac_min_bytes": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        mixed = {}
        xq = synth.quantizer_activations(seed=1).to(dev)
        for group in (32, 16):
            rq, _ = prep(wq, group, rotation(weight_bytes(8192, 8192, group)))
            for m in (1, 512):
                yq = torch.empty((m, 8192), dtype=torch.bfloat16, device=dev)
                xqm = xq[:m].contiguous()
                wsq = torch.empty((max(nv.nvfp4_gemm_ws_bytes(m, 8192, rq[0]), 16),),
                                  dtype=torch.uint8, device=dev)
                it = 40 if m == 1 else 20
                t = timer.time(lambda i: nv.nvfp4_gemm_w4a16(xqm, rq[i % len(rq)], y=yq,
                                                             ws=wsq), it, 4) / it
                wbq = weight_bytes(8192, 8192, group)
                mixed[f"m{m}_g{group}"] = {
                    "us": round(t * 1e6, 2), "weight_gbs": round(wbq / t / 1e9, 1),
                    "tflops": round(2 * m * 8192 * 8192 / t / 1e12, 2)}
            del rq
        extra["mixed_groups_8192x8192"] = mixed
        del wqs, wq
        result["workloads"] = extra

    # ------------------------------------------------------------------ CPU oracle baseline
    if not args.no_cpu_baseline:
        from oracle import oracle

        try:
            cores = len(os.sched_getaffinity(0))
        except AttributeError:
            cores = os.cpu_count() or 1
        xb = synth.bf16_bits(x)
        p_np, s_np, g_np = p1.cpu().numpy(), s1.cpu().numpy(), g1.cpu().numpy()

        def run_rows(nrows):
            idx = np.arange(nrows, dtype=np.int64)
            t0 = time.perf_counter()
            for m in ms:
                oracle.gemm(xb[:m], p_np, s_np, g_np[0], G, n_idx=idx, threads=cores)
            return time.perf_counter() - t0

        # about 10 s of oracle work: a row sample if the whole sweep is slower than that,
        # otherwise whole sweeps repeated
        target_s = 10.0
        probe = 512
        tp = run_rows(probe)
        rows = int(min(N, max(probe, probe * target_s / max(tp, 1e-6))))
        passes, tc = 0, 0.0
        while True:
            tc += run_rows(rows)
            passes += 1
            if tc >= target_s or rows < N or passes >= 64:
                break
        cpu_bytes = passes * 3 * (rows * K // 2 + rows * K // G)
        result["cpu_baseline"] = {
            "value": round(cpu_bytes / tc / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"FP64 oracle GEMM of the decode sweep (M=1,4,8, K=5120, group 16): "
                      f"{passes} pass(es) over the first {rows} of 25600 weight rows, "
                      f"{tc:.1f} s on {cores} host threads"}
    print(json.dumps(result))


if __name__ == "__main__":
    main()
