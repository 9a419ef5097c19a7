"""Benchmark of DiT dense joint attention on one MI355X.

A step is one attention forward over one batch of synthetic inputs: for the
default workload, B=1, H=24, N=16896 (512 text + 128x128 image tokens),
d=128, bf16 in and out. Inputs are resident in HBM before timing starts.

Prints ONE JSON line. ``value`` is TFLOP/s by 4*B*H*N^2*d over the wall
clock of K back-to-back steps (synchronised on both sides), each step one
call of the library with a caller-owned workspace (the schedule that splits
the last round of query tiles along the keys). ``roofline`` uses the
per-launch kernel time from events recorded on the stream the kernel runs
on. ``cpu_baseline`` times the fp64 CPU oracle on every row of the same
workload (or, with --cpu-rows, on a row sample: each output row depends on
one query row, so a sample is the same computation, only fewer rows), and
``check`` compares the output of the last timed step with that oracle.
``clocks`` are the GPU's shader and memory clocks read by a child process
(amd-smi) before and after the timed work; ``cold`` times single calls after
a 512 MiB scrub of the caches; ``no_workspace`` times the short entry point
dit_attn_fwd, which runs one workgroup per query tile; ``sustained`` is the
rate of the timed step over the second half of about four seconds of
back-to-back calls run after the companions (the timed ``value`` covers the
first calls of the process, before the card's power management settles).
``fp8``, ``fp8_mx`` and ``blocksparse`` are companion figures of the same
workload: the e4m3 path with per-tensor scales, the e4m3 path with one scale
per 32 values (scaled MFMA), and block-sparse attention over the text key
blocks plus a seeded fraction of the image key blocks (TFLOP/s over the keys
actually visited).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DiT attention fwd TFLOP/s at 16896-token shape; % of MI355X MFMA peak"
PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2}     # MI355X dense MFMA, 2.4 GHz
HBM_PEAK_GBS = 8000.0
KERNEL_SOURCES = ["attn_common.h", "attn_fwd_bf16.h", "attn_fwd_bf16_pipe.h", "attn_fwd_fp8_pipe.h", "quant_mx.h",
                  "dit_attn.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "diffusion_transformer_attention_non_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kind: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, warmup: int, steps: int):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in evs]
    return wall, per


def cpu_baseline(q, k, v, scale, max_rows: int = 0):
    """Time the fp64 oracle over batch entry 0 (every batch entry when B > 1
    and every row is asked for); return (record, rows, oracle output)."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                      default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    B, H, N, d = q.shape
    full = max_rows <= 0 or max_rows >= N
    nb = B if full else 1
    q64, k64, v64 = (t[:nb].double().numpy() for t in (q, k, v))
    rows = np.arange(N) if full else np.linspace(0, N - 1, max_rows).astype(np.int64)
    t0 = time.perf_counter()
    o_ref, _ = oracle.attention(q64, k64, v64, scale, rows=rows)
    t = time.perf_counter() - t0
    flops = 4.0 * nb * H * rows.size * N * d
    cpu = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    what = "every query row of the workload" if full else f"{rows.size} of {N} query rows x {H} heads of batch entry 0"
    rec = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"fp64 numpy oracle on {what} ({flops / 1e9:.1f} GFLOP in {t:.1f} s); host CPU: {cpu}"}
    return rec, rows, o_ref, nb


def output_error(o_dev, o_ref, rows, nb):
    """max / mean |O_gpu - O_oracle| over the rows the oracle computed."""
    import numpy as np
    import torch
    idx = torch.as_tensor(rows, device=o_dev.device)
    got = o_dev[:nb].index_select(2, idx).float().cpu().double().numpy()
    err = np.abs(got - o_ref)
    return {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "elements": int(err.size)}


def read_clocks():
    """Current shader (sclk) and memory (mclk) clocks in MHz of GPU 0, read by
    a child process; None where the tool is missing or prints no such field."""
    import re
    import subprocess
    out = {"sclk_mhz": None, "mclk_mhz": None, "source": None}
    for cmd in (["amd-smi", "metric", "-g", "0", "-c"], ["rocm-smi", "-d", "0", "--showclocks"]):
        try:
            text = subprocess.run(cmd, capture_output=True, text=True, timeout=30).stdout
        except (OSError, subprocess.SubprocessError):
            continue
        if cmd[0] == "amd-smi":
            # blocks "GFX_0:" / "MEM_0:" each followed by an indented "CLK: <n> MHz"
            g = re.search(r"GFX_0:\s*\n\s*CLK:\s*([\d.]+)\s*MHz", text)
            m = re.search(r"MEM_0:\s*\n\s*CLK:\s*([\d.]+)\s*MHz", text)
        else:
            g = re.search(r"sclk clock level:[^(]*\(([\d.]+)\s*Mhz\)", text, re.I)
            m = re.search(r"mclk clock level:[^(]*\(([\d.]+)\s*Mhz\)", text, re.I)
        if g or m:
            out.update(sclk_mhz=float(g.group(1)) if g else None, mclk_mhz=float(m.group(1)) if m else None,
                       source=cmd[0])
            break
    return out


def time_cold(fn, steps: int, scrub_mib: int = 512):
    """Median per-call kernel ms with a scrub of scrub_mib MiB written between calls."""
    import torch
    scrub = torch.empty(scrub_mib << 20, dtype=torch.uint8, device="cuda")
    per = []
    for i in range(steps):
        scrub.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b))
    del scrub
    return statistics.median(per)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t2i_2048")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-e4m3 companion measurement")
    ap.add_argument("--sparse-density", type=float, default=0.25,
                    help="fraction of image key blocks in the block-sparse companion's lists (0 skips it)")
    ap.add_argument("--layout", choices=["bhnd", "bnhd"], default="bhnd",
                    help="rows of q, k, v and o packed as [B][H][N][d] (default) or taken from [B][N][H][d] "
                         "buffers through dit_attn_fwd_strided")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="query rows per head for cpu_baseline (0: every row of the workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the clock readings, the cold-cache and the no-workspace companion timings")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (to calibrate "
                         "the FETCH_SIZE / WRITE_SIZE counters against known bytes) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every (b, h) slice is independent, so heads or batch entries shard across GPUs with no "
              "exchange inside attention). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_copy": n, "copies": 3}), flush=True)
        return 0
    import diffusion_transformer_attention_non_amd as dit
    from workloads import WORKLOADS, make_qkv

    w = WORKLOADS[args.workload]
    scale = 1.0 / math.sqrt(w.d)
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(w)
    B, H, N, d = w.B, w.H, w.N, w.d
    if args.layout == "bnhd":
        # (B, H, N, d) views of (B, N, H, d) buffers, as a QKV projection writes them
        qd, kd, vd = (t.permute(0, 2, 1, 3).contiguous().to(dev).permute(0, 2, 1, 3) for t in (q, k, v))
        od = torch.empty((B, N, H, d), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
    else:
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        od = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    handle = stream.cuda_stream
    in_strides, out_strides = qd.stride()[:3], od.stride()[:3]
    # the caller-owned workspace, sized by the plan (allocated before timing)
    fp8_on = not args.no_fp8 and d == 128          # the e4m3 kernel is d = 128 only
    ws_bytes = dit.workspace_bytes(B, H, N, d, dit.DIT_ATTN_BF16)
    if fp8_on:
        ws_bytes = max(ws_bytes, dit.workspace_bytes(B, H, N, d, dit.DIT_ATTN_FP8_E4M3))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    _, plan = dit.dit_attn_plan(B, H, N, d, dit.DIT_ATTN_BF16, 0, False, 0, ws_bytes)
    clocks_before = None if args.no_extras else read_clocks()

    def step():
        st = dit.dit_attn_fwd_strided(qd, kd, vd, od, B, H, N, d, scale, dit.DIT_ATTN_BF16, in_strides,
                                      out_strides, None, None, ws, ws_bytes, handle)
        if st != 0:
            raise dit.DitAttnError(st, "dit_attn_fwd_strided")

    wall, per = time_launches(step, args.warmup, args.steps)
    o_timed = od.clone()
    flops = w.flops
    ms_per_step = wall / args.steps * 1e3
    value = flops / (wall / args.steps) / 1e12
    k_mean = statistics.fmean(per)
    achieved = flops / (k_mean * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    traffic = load_traffic("attn_fwd_bf16", w.name)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: Q, K, V iid N(0,1) rounded to bf16, seed 0",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "n_text": w.n_text,
                   "n_image": w.n_image, "causal": False, "scale": scale, "layout": args.layout,
                   "schedule": ["tile", "split", "stream-k"][plan.schedule], "workspace_bytes": ws_bytes},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "kernel_ms": {"mean": round(k_mean, 4), "median": round(statistics.median(per), 4),
                      "p95": round(sorted(per)[int(0.95 * (len(per) - 1))], 4), "min": round(min(per), 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic},
    }

    if fp8_on:
        if args.layout == "bnhd":      # quantise the (B, N, H, d) buffers, view them as (B, H, N, d)
            quant = [dit.quantize_e4m3(t.permute(0, 2, 1, 3)) for t in (qd, kd, vd)]
            q8, k8, v8 = (c.permute(0, 2, 1, 3) for c, _ in quant)
        else:
            quant = [dit.quantize_e4m3(t) for t in (qd, kd, vd)]
            q8, k8, v8 = (c for c, _ in quant)
        descale = torch.cat([ds for _, ds in quant]).contiguous()

        def step8():
            st = dit.dit_attn_fwd_strided(q8, k8, v8, od, B, H, N, d, scale, dit.DIT_ATTN_FP8_E4M3,
                                          q8.stride()[:3], out_strides, descale, None, ws, ws_bytes, handle)
            if st != 0:
                raise dit.DitAttnError(st, "dit_attn_fwd_strided")

        wall8, per8 = time_launches(step8, args.warmup, args.steps)
        o8_timed = od.clone()
        v8_tflops = flops / (wall8 / args.steps) / 1e12
        k8_mean = statistics.fmean(per8)
        line["fp8"] = {"workload": w.name + "_fp8", "value": round(v8_tflops, 2), "unit": "TFLOP/s",
                       "ms_per_step": round(wall8 / args.steps * 1e3, 4),
                       "pct_of_fp8_peak": round(100.0 * v8_tflops / PEAK_TFLOPS["fp8"], 2),
                       "roofline": {"bound": "mfma", "achieved": round(flops / (k8_mean * 1e-3) / 1e12, 2),
                                    "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                                    "frac": round(flops / (k8_mean * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
                                    "traffic": load_traffic("attn_fwd_fp8", w.name)}}

    if not args.no_fp8 and args.layout == "bhnd" and d == 128:
        # block-scaled e4m3 (32-value blocks, E8M0 scales) on the scaled MFMA
        (qm, qsc), (km, ksc) = dit.quantize_mx(qd, "d"), dit.quantize_mx(kd, "d")
        vm, vsc = dit.quantize_mx(vd, "tokens")

        def step_mx():
            st = dit.dit_attn_fwd_mx(qm, km, vm, qsc, ksc, vsc, od, B, H, N, d, scale, None, ws, ws_bytes, handle)
            if st != 0:
                raise dit.DitAttnError(st, "dit_attn_fwd_mx")

        wallm, perm = time_launches(step_mx, args.warmup, args.steps)
        km_mean = statistics.fmean(perm)
        line["fp8_mx"] = {"workload": w.name + "_mx", "value": round(flops / (wallm / args.steps) / 1e12, 2),
                          "unit": "TFLOP/s", "ms_per_step": round(wallm / args.steps * 1e3, 4),
                          "roofline": {"bound": "mfma", "achieved": round(flops / (km_mean * 1e-3) / 1e12, 2),
                                       "peak": PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                                       "frac": round(flops / (km_mean * 1e-3) / 1e12 / PEAK_TFLOPS["fp8"], 4),
                                       "traffic": None}}

    if args.sparse_density > 0 and args.layout == "bhnd" and d == 128:
        from workloads import random_kv_blocks
        blocks, counts = random_kv_blocks(B, H, N, args.sparse_density, seed=w.seed)
        ws_sparse = dit.workspace_bytes(B, H, N, d, dit.DIT_ATTN_BF16, max_blocks=blocks.shape[-1])
        ws_s = torch.empty(max(ws_sparse, 16), dtype=torch.uint8, device=dev)
        # keys each query row visits, summed over rows (the listed blocks' real sizes)
        nq, mb = counts.shape[-1], blocks.shape[-1]
        visited = 0
        for bh in range(B * H):
            for t in range(nq):
                c = int(counts.view(-1, nq)[bh, t])
                keys = sum(min(64, N - 64 * u) for u in blocks.view(-1, nq, mb)[bh, t, :c].tolist())
                visited += min(256, N - 256 * t) * keys
        blocks_d, counts_d = blocks.to(dev), counts.to(dev)

        def step_sparse():
            st = dit.dit_attn_fwd_blocksparse(qd, kd, vd, od, B, H, N, d, scale, dit.DIT_ATTN_BF16, blocks_d,
                                              counts_d, mb, None, None, None, ws_s, ws_sparse, handle)
            if st != 0:
                raise dit.DitAttnError(st, "dit_attn_fwd_blocksparse")

        walls, pers = time_launches(step_sparse, args.warmup, args.steps)
        sflops = 4.0 * d * visited
        ks_mean = statistics.fmean(pers)
        line["blocksparse"] = {
            "workload": f"{w.name}, text blocks + {args.sparse_density:.2f} of image key blocks per 256-query block",
            "visited_fraction": round(visited / (B * H * N * N), 4),
            "value": round(sflops / (walls / args.steps) / 1e12, 2), "unit": "TFLOP/s over visited keys",
            "ms_per_step": round(walls / args.steps * 1e3, 4),
            "speedup_vs_dense": round((wall / args.steps) / (walls / args.steps), 3),
            "roofline": {"bound": "mfma", "achieved": round(sflops / (ks_mean * 1e-3) / 1e12, 2), "peak": peak,
                         "unit": "TFLOP/s", "frac": round(sflops / (ks_mean * 1e-3) / 1e12 / peak, 4),
                         "traffic": None}}

    if not args.no_extras:
        # what the matrix cores sustain on changing random operands, right after the timed calls:
        # the power-limited reference for the attention kernels on this card
        ceil = {"bf16": dit.mfma_ceiling(dit.DIT_ATTN_BF16)}
        ceil["bf16"]["frac"] = round(achieved / ceil["bf16"]["tflops"], 4)
        if "fp8" in line:
            ceil["fp8"] = dit.mfma_ceiling(dit.DIT_ATTN_FP8_E4M3)
            ceil["fp8"]["frac"] = round(line["fp8"]["roofline"]["achieved"] / ceil["fp8"]["tflops"], 4)
        ceil["kind"] = ("dit_attn_mfma_ceiling: independent 32x32 products back to back, one wave per SIMD, "
                        "operands drawn from a counter hash and changing every product; frac = the kernel's "
                        "achieved rate over this one")
        line["mfma_ceiling"] = ceil

        # clocks under load: a thread reads them from a child process while
        # about four seconds of back-to-back calls run; a reading taken after
        # the queue drained (the stream already idle) is marked as such
        import threading
        n_load = max(10, int(4.0 / (wall / args.steps)))
        during, done = [], threading.Event()

        def sample():
            time.sleep(0.5)
            while not done.is_set() and len(during) < 4:
                rec = read_clocks()
                rec["busy"] = not done.is_set()
                during.append(rec)

        th = threading.Thread(target=sample)
        th.start()
        # the same calls timed by events: the rate they settle at over the
        # second half (the timed `value` above covers the first calls of the
        # process, before the card's power management has settled)
        half = n_load // 2
        e0, e_mid, e_end = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record()
        for i in range(n_load):
            if i == half:
                e_mid.record()
            step()
        e_end.record()
        torch.cuda.synchronize()
        done.set()
        th.join()
        line["clocks"] = {"idle_before": clocks_before, "under_load": [r for r in during if r["busy"]],
                          "calls_enqueued": n_load}
        ms_first, ms_second = e0.elapsed_time(e_mid), e_mid.elapsed_time(e_end)
        line["sustained"] = {
            "value": round(flops * (n_load - half) / (ms_second * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
            "first_half_value": round(flops * half / (ms_first * 1e-3) / 1e12, 2),
            "calls": n_load, "seconds": round((ms_first + ms_second) * 1e-3, 2),
            "kind": "back-to-back calls of the timed step after the companions; value over the second half"}

        def step_short():
            st = dit.dit_attn_fwd(qd, kd, vd, od, B, H, N, d, scale, dit.DIT_ATTN_BF16, handle)
            if st != 0:
                raise dit.DitAttnError(st, "dit_attn_fwd")

        if args.layout == "bhnd":
            walln, pern = time_launches(step_short, args.warmup, args.steps)
            line["no_workspace"] = {"entry_point": "dit_attn_fwd", "schedule": "tile",
                                    "value": round(flops / (walln / args.steps) / 1e12, 2), "unit": "TFLOP/s",
                                    "kernel_ms_mean": round(statistics.fmean(pern), 4)}
        cold = time_cold(step, min(args.steps, 10))
        line["cold"] = {"scrub_mib": 512, "kernel_ms_median": round(cold, 4),
                        "value": round(flops / (cold * 1e-3) / 1e12, 2), "unit": "TFLOP/s"}

    if not args.no_cpu_baseline:
        rec, rows, o_ref, nb = cpu_baseline(q, k, v, scale, args.cpu_rows)
        line["cpu_baseline"] = rec
        check = {"bf16": output_error(o_timed, o_ref, rows, nb), "spec_max_abs": 2e-2, "spec_mean_abs": 2e-3}
        check["bf16"]["within_spec"] = check["bf16"]["max_abs"] <= 2e-2 and check["bf16"]["mean_abs"] <= 2e-3
        if "fp8" in line:
            check["fp8"] = output_error(o8_timed, o_ref, rows, nb)
            check["fp8"]["within_spec"] = check["fp8"]["max_abs"] <= 6e-2
            check["spec_max_abs_fp8"] = 6e-2
        line["check"] = check
    line["context"] = ("pages (NVIDIA B200, FLUX 3 Image Klein, 2048x2048): Base text-to-image denoise "
                       "14.24 s of 14.70 s; dense BF16 attention ~60% of DiT kernel time")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
