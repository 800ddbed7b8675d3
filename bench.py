#!/usr/bin/env python3
"""Throughput of the flash-attention training forward (O + L) on one MI355X.

One step = one forward pass over each of the two training-scale workloads:
  d64_b8_h16_q4096_k4096_causal          (head_dim 64, B8 H16, 4k tokens)
  d256_gqa_b2_h16kv4_q8192_k8192_causal  (head_dim 256, GQA 16/4, 8k tokens)
with seeded synthetic bf16 inputs already resident in HBM. Reported value:
metric FLOP (4*B*H*ql*kl*D, halved for causal) of the step / step time, in
TFLOP/s. Each kernel launch is bracketed by HIP events on the stream it runs
on. The CPU oracle is timed on a strided sample of the same rows on the host.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|both]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0
# untimed calls before each of the extra (non-headline) timings: enough for
# the clocks and the fresh buffers' address translations to settle
EXTRA_WARMUP = 20
HEADLINE = ["d64_b8_h16_q4096_k4096_causal", "d256_gqa_b2_h16kv4_q8192_k8192_causal"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the forward kernel's sources: the stored counters hold only while these are unchanged
KERNEL_SOURCES = [os.path.join(ROOT, "flash_attention_forward_fa_amd", "csrc", n)
                  for n in ("fa_fwd_kernel.h", "fa_common.h", "fa_fwd.hip")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """sha256[:16] over the forward kernel's source files, in order."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def device_info(dev_index):
    """The GPU's own figures (HIP device attributes): compute units, peak
    clock, and the dense bf16 MFMA peak they give at 4096 FLOP per clock and
    CU; the published peak stays the roofline's. None where HIP is not found."""
    import ctypes
    import torch
    p = torch.cuda.get_device_properties(dev_index)
    out = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
           "compute_units": p.multi_processor_count, "l2_bytes": getattr(p, "L2_cache_size", None),
           "hbm_bytes": p.total_memory}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate (peak clock, kHz) is attribute 5 in
        # hip_runtime_api.h's hipDeviceAttribute_t
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, dev_index) == 0 and v.value > 0:
            out["peak_clock_mhz"] = v.value / 1e3
            out["bf16_peak_from_device_tflops"] = (p.multi_processor_count * v.value * 1e3 * 4096
                                                   / 1e12)
    except OSError:
        pass
    return out


def stored_counters(workload):
    """rocprofv3 --pmc figures of the workload's forward launch (HBM bytes from
    FETCH_SIZE/WRITE_SIZE, MFMA/VALU/LDS activity from the SQ counters), if they
    were taken on the current kernel source; else an empty dict."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {}
    entry = t.get(workload)
    if not entry or entry.get("kernel_source_sha") != kernel_source_hash():
        return {}
    return entry


def cpu_baseline(workloads, inputs, target_rows):
    """The oracle, as it stands, on every row of each workload (or a strided
    sample of target_rows rows)."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    total_flop = 0.0
    total_s = 0.0
    parts = []
    for w in workloads:
        n_rows = w.B * w.H * w.ql
        stride = max(1, n_rows // target_rows[w.name])
        rows = np.arange(0, n_rows, stride, dtype=np.int64)
        t0 = time.perf_counter()
        oracle.fwd_workload(w, inputs[w.name], rows=rows, n_threads=threads)
        dt = time.perf_counter() - t0
        flop = w.metric_flop * rows.size / n_rows
        total_flop += flop
        total_s += dt
        which = "every row" if stride == 1 else f"every {stride}th row"
        parts.append(f"{w.name}: {which} ({rows.size} rows, {dt:.1f} s)")
        log(f"cpu_baseline {w.name}: {rows.size} rows in {dt:.2f} s "
            f"({flop / dt / 1e9:.2f} GFLOP/s)")
    host_cores = os.cpu_count()
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = host_cores
    return {"value": total_flop / total_s / 1e12, "unit": "TFLOP/s", "cores": threads,
            "threads": threads, "host_cores": host_cores, "host_cores_usable": usable,
            "kind": "oracle", "sample": "; ".join(parts) +
            f"; metric FLOP of the sampled rows / oracle wall time; the oracle ran {threads} "
            f"threads on a host with {host_cores} logical cores ({usable} usable by this "
            "process)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="both")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="timed backward calls per workload after the forward (0: none)")
    ap.add_argument("--window-steps", type=int, default=10,
                    help="timed sliding-window forward calls per workload (0: none)")
    ap.add_argument("--d128-steps", type=int, default=10,
                    help="timed head_dim-128 forward and backward calls (0: none)")
    ap.add_argument("--split-steps", type=int, default=10,
                    help="timed long-cache calls, plain and split-KV (0: none)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows per workload for the CPU baseline (0: default sample)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run 3 device-to-device copies of MIB MiB (a plain copy kernel of "
                         "known traffic, to calibrate rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards by batch or KV-head group with no communication).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fagen
    import flash_attention_forward_fa_amd as fa

    names = HEADLINE if args.workload == "both" else [args.workload]
    workloads = [fagen.WORKLOADS[n] for n in names]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    inputs, dev_inputs, outputs = {}, {}, {}
    for w in workloads:
        t0 = time.perf_counter()
        inp = fagen.generate(w)
        inputs[w.name] = inp
        to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        dev_inputs[w.name] = (to(inp["q"]), to(inp["k"]), to(inp["v"]))
        q = dev_inputs[w.name][0]
        outputs[w.name] = (torch.empty_like(q),
                           torch.empty((w.B, w.H, w.ql), dtype=torch.float32, device=dev))
        log(f"inputs {w.name}: generated and uploaded in {time.perf_counter() - t0:.1f} s")

    def launch(w):
        q, k, v = dev_inputs[w.name]
        O, L = outputs[w.name]
        fa.train_fwd(q, k, v, scale=w.scale, causal=w.causal, out=O, lse=L)

    for i in range(args.warmup):
        for w in workloads:
            launch(w)
    torch.cuda.synchronize()
    log(f"warmup: {args.warmup} steps done")

    ev = {w.name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.steps)] for w in workloads}
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(args.steps):
        for w in workloads:
            a, b = ev[w.name][s]
            a.record(stream)
            launch(w)
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    log(f"timed: {args.steps} steps in {wall:.3f} s wall")

    # The backward of the same calls (not part of the headline metric): its own
    # HIP-event timing, fewer steps, the forward's O and L as inputs and a
    # seeded upstream gradient.
    bwd = {}
    if args.backward_steps > 0:
        for w in workloads:
            q, k, v = dev_inputs[w.name]
            O, L = outputs[w.name]
            dO = torch.from_numpy(fagen.normal_bf16(w.seed, 6, (w.B, w.H, w.ql, w.D))
                                  .view(np.int16)).view(torch.bfloat16).to(dev)
            for _ in range(EXTRA_WARMUP):
                fa.train_bwd(q, k, v, O, L, dO, scale=w.scale, causal=w.causal)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.backward_steps):
                fa.train_bwd(q, k, v, O, L, dO, scale=w.scale, causal=w.causal)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.backward_steps
            # the FA-2 count: dQ, dK, dV, dP and the recomputed S, 2.5x the forward
            flop = 2.5 * w.metric_flop
            bwd[w.name] = {"ms_avg": ms, "flop_fa2": flop, "tflops": flop / (ms * 1e-3) / 1e12,
                           "frac_of_peak": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
            log(f"{w.name}: backward {ms * 1e3:.1f} us/call, {bwd[w.name]['tflops']:.1f} TFLOP/s "
                f"(FA-2 count)")

    # The sliding-window forward (fa_train_fwd_swa) on the same inputs, window
    # 1024 (D=64) or 2048 (D=256); not part of the headline metric. Its FLOP
    # count is exact: 4*D per visible score.
    swa = {}
    if args.window_steps > 0:
        for w in workloads:
            q, k, v = dev_inputs[w.name]
            O, L = outputs[w.name]
            win = 1024 if w.D == 64 else 2048
            for _ in range(EXTRA_WARMUP):
                fa.train_fwd_swa(q, k, v, win, scale=w.scale, out=O, lse=L)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(args.window_steps):
                fa.train_fwd_swa(q, k, v, win, scale=w.scale, out=O, lse=L)
            b.record(stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.window_steps
            off = max(w.kl - w.ql, 0)
            q_abs = off + np.arange(w.ql, dtype=np.int64)
            visible = int((np.minimum(q_abs, w.kl - 1) - np.maximum(q_abs - win, 0) + 1)
                          .clip(min=0).sum()) * w.B * w.H
            flop = 4 * w.D * visible
            swa[w.name] = {"window": win, "ms_avg": ms, "flop": flop,
                           "tflops": flop / (ms * 1e-3) / 1e12,
                           "frac_of_peak": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
            log(f"{w.name}: sliding window {win}: {ms * 1e3:.1f} us/call, "
                f"{swa[w.name]['tflops']:.1f} TFLOP/s (4*D per visible score)")
            if args.backward_steps > 0:
                # its backward on the window forward's O and L (FA-2 count, 10*D
                # FLOP per visible score)
                dO = torch.from_numpy(fagen.normal_bf16(w.seed, 6, (w.B, w.H, w.ql, w.D))
                                      .view(np.int16)).view(torch.bfloat16).to(dev)
                for _ in range(EXTRA_WARMUP):
                    fa.train_bwd_swa(q, k, v, O, L, dO, win, scale=w.scale)
                torch.cuda.synchronize()
                a.record(stream)
                for _ in range(args.window_steps):
                    fa.train_bwd_swa(q, k, v, O, L, dO, win, scale=w.scale)
                b.record(stream)
                torch.cuda.synchronize()
                bms = a.elapsed_time(b) / args.window_steps
                bflop = 2.5 * flop
                swa[w.name].update({"backward_ms_avg": bms, "backward_flop_fa2": bflop,
                                    "backward_tflops": bflop / (bms * 1e-3) / 1e12})
                log(f"{w.name}: sliding window {win} backward: {bms * 1e3:.1f} us/call, "
                    f"{swa[w.name]['backward_tflops']:.1f} TFLOP/s (FA-2 count)")
        # leave the causal forward's outputs in place for anything read later
        for w in workloads:
            launch(w)
        torch.cuda.synchronize()

    # head_dim 128 (B2, 32 query heads on 8 kv heads, 4096 tokens, causal), the
    # forward and its backward; not part of the headline metric.
    d128 = {}
    if args.d128_steps > 0:
        w = fagen.Workload("d128_b2_h32kv8_q4096_k4096_causal", 2, 32, 8, 4096, 4096, 128, True,
                           seed_offset=8000)
        inp = fagen.generate(w)
        to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        q, k, v = to(inp["q"]), to(inp["k"]), to(inp["v"])
        dO = to(fagen.normal_bf16(w.seed, 6, (w.B, w.H, w.ql, w.D)))
        O, L = fa.train_fwd(q, k, v, scale=w.scale, causal=True)
        for _ in range(EXTRA_WARMUP):
            fa.train_fwd(q, k, v, scale=w.scale, causal=True, out=O, lse=L)
            fa.train_bwd(q, k, v, O, L, dO, scale=w.scale, causal=True)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.d128_steps):
            fa.train_fwd(q, k, v, scale=w.scale, causal=True, out=O, lse=L)
        b.record(stream)
        torch.cuda.synchronize()
        fms = a.elapsed_time(b) / args.d128_steps
        a.record(stream)
        for _ in range(args.d128_steps):
            fa.train_bwd(q, k, v, O, L, dO, scale=w.scale, causal=True)
        b.record(stream)
        torch.cuda.synchronize()
        bms = a.elapsed_time(b) / args.d128_steps
        d128 = {"workload": w.name, "ms_avg": fms, "metric_flop": w.metric_flop,
                "tflops": w.metric_flop / (fms * 1e-3) / 1e12,
                "frac_of_peak": w.metric_flop / (fms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "backward_ms_avg": bms,
                "backward_tflops": 2.5 * w.metric_flop / (bms * 1e-3) / 1e12}
        log(f"{w.name}: {fms * 1e3:.1f} us/call, {d128['tflops']:.1f} TFLOP/s; backward "
            f"{bms * 1e3:.1f} us/call, {d128['backward_tflops']:.1f} TFLOP/s (FA-2 count)")
        del q, k, v, dO, O, L

    # Few query tiles against a long KV cache (head_dim 128, 32 query
    # heads on 8 kv heads, causal): prefill of 512 tokens and decoding 1 token
    # (batch 1 and 8) against 32768 keys, the plain launch against the split-KV
    # one (suggest_n_split chunks), and the same keys in a block-paged cache
    # (fa_paged_fwd, same chunks); not part of the headline metric. FLOP:
    # 4*D per visible score; K+V GB/s: the cache's bytes over the call's time.
    split_kv = {}
    if args.split_steps > 0:
        for name, B, ql, kl in (("prefill_b1_h32kv8_q512_k32768_d128", 1, 512, 32768),
                                ("decode_b1_h32kv8_q1_k32768_d128", 1, 1, 32768),
                                ("decode_b8_h32kv8_q1_k32768_d128", 8, 1, 32768)):
            w = fagen.Workload(name, B, 32, 8, ql, kl, 128, True, seed_offset=9300 + ql)
            n_split = fa.suggest_n_split(B, 32, ql, 128, n_kv_heads=8)
            inp = fagen.generate(w)
            to = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
            q, k, v = to(inp["q"]), to(inp["k"]), to(inp["v"])
            O = torch.empty_like(q)
            L = torch.empty((w.B, w.H, w.ql), dtype=torch.float32, device=dev)
            ws = torch.empty(fa.fa_train_fwd_split_workspace(w.B, w.H, w.ql, w.D, n_split),
                             dtype=torch.uint8, device=dev)
            off = max(kl - ql, 0)
            visible = int(np.minimum(off + np.arange(ql) + 1, kl).sum()) * w.B * w.H
            flop = 4 * w.D * visible
            res = {"n_split": n_split, "flop": flop, "kv_bytes": 2 * 2 * w.B * w.Hkv * kl * w.D}
            for label, call in (("plain", lambda: fa.train_fwd(q, k, v, scale=w.scale, causal=True,
                                                               out=O, lse=L)),
                                ("split", lambda: fa.train_fwd_split(q, k, v, n_split,
                                                                     scale=w.scale, causal=True,
                                                                     workspace=ws, out=O,
                                                                     lse=L))):
                for _ in range(EXTRA_WARMUP):
                    call()
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(args.split_steps):
                    call()
                b.record(stream)
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / args.split_steps
                res[f"{label}_ms_avg"] = ms
                res[f"{label}_tflops"] = flop / (ms * 1e-3) / 1e12
                res[f"{label}_kv_gbs"] = res["kv_bytes"] / (ms * 1e-3) / 1e9
            # the same keys in a block-paged cache (blocks of 64 and of 16
            # keys in a seeded shuffled order), read through fa_paged_fwd
            # with the same chunks
            for bs, tag in ((64, "paged_split"), (16, "paged16_split")):
                per = kl // bs
                order = torch.from_numpy(np.random.default_rng(ql + B).permutation(B * per)
                                         .astype(np.int64)).to(dev)
                kc = torch.empty((B * per, w.Hkv, bs, w.D), dtype=torch.bfloat16, device=dev)
                vc = torch.empty_like(kc)
                kc[order] = k.view(B, w.Hkv, per, bs, w.D).permute(0, 2, 1, 3, 4).reshape(
                    B * per, w.Hkv, bs, w.D)
                vc[order] = v.view(B, w.Hkv, per, bs, w.D).permute(0, 2, 1, 3, 4).reshape(
                    B * per, w.Hkv, bs, w.D)
                table = order.view(B, per).to(torch.int32)
                lens = torch.full((B,), kl, dtype=torch.int32, device=dev)
                call = lambda: fa.paged_fwd(q, kc, vc, table, lens, scale=w.scale,
                                            causal=True, n_split=n_split, workspace=ws,
                                            out=O, lse=L)
                for _ in range(EXTRA_WARMUP):
                    call()
                torch.cuda.synchronize()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(args.split_steps):
                    call()
                b.record(stream)
                torch.cuda.synchronize()
                ms = a.elapsed_time(b) / args.split_steps
                res[f"{tag}_ms_avg"] = ms
                res[f"{tag}_tflops"] = flop / (ms * 1e-3) / 1e12
                res[f"{tag}_kv_gbs"] = res["kv_bytes"] / (ms * 1e-3) / 1e9
                del kc, vc, table, lens
            split_kv[name] = res
            log(f"{name}: plain {res['plain_ms_avg'] * 1e3:.1f} us, split({n_split}) "
                f"{res['split_ms_avg'] * 1e3:.1f} us ({res['split_tflops']:.1f} TFLOP/s, "
                f"K+V {res['split_kv_gbs']:.0f} GB/s)"
                + (f", paged split {res['paged_split_ms_avg'] * 1e3:.1f} us (64-key blocks), "
                   f"{res['paged16_split_ms_avg'] * 1e3:.1f} us (16-key blocks)"
                   if "paged_split_ms_avg" in res else ""))
            del q, k, v, O, L, ws

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {args.copy_calibration} MiB done")

    per = {}
    total_ms = 0.0
    total_flop = 0
    for w in workloads:
        ms = [a.elapsed_time(b) for a, b in ev[w.name]]
        avg = float(np.mean(ms))
        total_ms += avg
        total_flop += w.metric_flop
        # Q and O (bf16), K and V (bf16, each read once), L (f32)
        alg_bytes = (2 * 2 * w.B * w.H * w.ql * w.D + 2 * 2 * w.B * w.Hkv * w.kl * w.D
                     + 4 * w.B * w.H * w.ql)
        per[w.name] = {"ms_avg": avg, "ms_min": float(np.min(ms)), "ms_median": float(np.median(ms)),
                       "tflops": w.metric_flop / (avg * 1e-3) / 1e12,
                       "frac_of_peak": w.metric_flop / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                       "metric_flop": w.metric_flop, "algorithmic_bytes": alg_bytes}
        log(f"{w.name}: {avg * 1e3:.1f} us/launch, {per[w.name]['tflops']:.1f} TFLOP/s "
            f"({100 * per[w.name]['frac_of_peak']:.1f}% of bf16 peak)")

    dom = max(workloads, key=lambda w: per[w.name]["ms_avg"])
    dp = per[dom.name]
    ctr = stored_counters(dom.name)
    roofline = {"bound": "mfma", "achieved": dp["tflops"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": dp["tflops"] / PEAK_BF16_TFLOPS,
                "traffic": ctr.get("bytes_per_launch"),
                "mfma_util": ctr.get("mfma_util"), "valu_busy": ctr.get("valu_busy"),
                "lds_util": ctr.get("lds_util"),
                "kernel": f"fa_train_fwd: one mixed fa_fwd_kernel<{dom.D}, causal> launch",
                "workload": dom.name}

    value = total_flop / (total_ms * 1e-3) / 1e12
    result = {
        "metric": "fwd TFLOP/s (O+L, bf16, causal, D=64/256) and % of MI355X bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": total_ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "config": {"workload": "+".join(names),
                   "workloads": {w.name: {"B": w.B, "H": w.H, "Hkv": w.Hkv, "ql": w.ql,
                                          "kl": w.kl, "D": w.D, "causal": w.causal,
                                          "sigma": w.sigma} for w in workloads},
                   "parallelism": "none (one GPU)"},
        "per_workload": per,
        "roofline": roofline,
        "device": device_info(dev.index if dev.index is not None else 0),
    }
    if bwd:
        result["backward"] = bwd
    if swa:
        result["sliding_window"] = swa
    if d128:
        result["head_dim_128"] = d128
    if split_kv:
        result["split_kv"] = split_kv
    if not args.no_cpu_baseline:
        target = {w.name: (args.cpu_rows or (524288 if w.D == 64 else 262144)) for w in workloads}
        result["cpu_baseline"] = cpu_baseline(workloads, inputs, target)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
