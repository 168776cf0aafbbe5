#!/usr/bin/env python3
"""Benchmark of the NF4 + double-quantized QLoRA frozen-base linear layer on
one MI355X.

One step = forward of the three LLaMA-7B MLP linears (gate_proj and up_proj
4096->11008, down_proj 11008->4096; batch 8 x seq 512 = M 4096 rows; LoRA
r = 64, alpha = 16), then their backward (dX, dA, dB) in reverse order, on
seeded synthetic inputs already resident in HBM.  `value` is the step's
algorithmic TFLOP/s: per layer fwd 2MNK + 2Mr(K+N), bwd 2MNK + 4Mr(N+K)
(the frozen base's dW, which the method never forms, is not counted).

Also reported, each against its roofline:
  rows.quantize     qlora_quantize_nf4_dq, GB/s on 4 B in + 0.5159 B out per weight
  rows.dequant      qlora_dequant_bf16, GB/s on 0.5159 B in + 2 B out per weight
  rows.fwd / .bwd   per-pass TFLOP/s
  rows.small_m      65B up_proj (8192->22016) forward at M = 1, 4, 16, GB/s on the
                    packed-weight bytes, rotating 6 weight copies (558 MB) so the
                    256 MB last-level cache cannot hold them: the whole call, and
                    the streaming kernel alone; M1_single_level: M = 1 with
                    single-level float32 block constants (4.5 bits)
  kernels           per-kernel average duration from the library's event timer
  roofline          the dominant kernel (largest summed time in a step)
  cpu_baseline      the CPU oracle (NumPy fp64) on a bounded sample of the step

roofline.traffic (HBM bytes per launch of the dominant kernel) comes from
profiles/traffic_counters.json when its source digest matches the library
sources.  That file is written by --ingest-pmc from two rocprofv3 counter
runs of this script with --calib-copy-mib (FETCH_SIZE, then WRITE_SIZE);
both counters are scaled by what they read for the calibration copy, an
elementwise kernel that reads and writes exactly that many bytes.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused NF4-QLoRA linear fwd+bwd TFLOP/s & GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense BF16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
# HBM traffic counters per kernel family, each valid for the sources it was
# taken with (see source_digest)
TRAFFIC_FILES = {"tile": os.path.join(ROOT, "profiles", "traffic_counters.json"),
                 "gemv": os.path.join(ROOT, "profiles", "traffic_counters_gemv.json")}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)  # ~0.2 s of timed steps at the 7B MLP shape
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="mlp_7b")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--no-extras", action="store_true", help="skip quantize/dequant/small-M rows")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB (counter calibration)")
    p.add_argument("--small-m-only", action="store_true",
                   help="print only rows.small_m (the small-M forward), as one JSON line")
    p.add_argument("--configs-only", action="store_true",
                   help="print only the 7B q_proj and 65B block rows (M = 512), as one JSON line")
    p.add_argument("--layer-only", action="store_true",
                   help="print only rows.decoder_layer (the 7B decoder layer and its attention core), as one JSON "
                        "line; use with --no-extras")
    p.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write the traffic-counter file of --pmc-target from two rocprofv3 --pmc output folders "
                        "(FETCH_SIZE, WRITE_SIZE) of a run with --calib-copy-mib, then exit")
    p.add_argument("--pmc-target", choices=sorted(TRAFFIC_FILES), default="tile",
                   help="kernel family whose counters --ingest-pmc records (tile: the 7B MLP step; gemv: the "
                        "small-M forward, from a --small-m-only run)")
    return p.parse_args()


# each kernel family's translation unit and the headers it includes: its
# traffic counters stay valid until one of these changes
COUNTER_SOURCES = {"tile": ("nf4_tile.hip", "nf4_tile.h", "lora_gemm.h", "qlora_internal.h", "qlora_device.h"),
                   "gemv": ("nf4_gemv.hip", "nf4_tile.h", "lora_gemm.h", "qlora_internal.h", "qlora_device.h")}


def source_digest(target: str = "tile") -> str:
    h = hashlib.sha256()
    for f in sorted(os.path.join(ROOT, "bit_nf4_quantized_qlora_amd", "csrc", n) for n in COUNTER_SOURCES[target]):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def layer_flops(M, N, K, r):
    fwd = 2 * M * N * K + 2 * M * r * (K + N)
    bwd = 2 * M * N * K + 4 * M * r * (N + K)
    return fwd, bwd


# rocprofv3 kernel names -> the names the library's event timer uses
KERNEL_ALIASES = {"k_nf4_tile<false>": "k_fwd_nf4", "k_nf4_tile<true>": "k_bwd_dx_nf4",
                  "k_nf4_tile<false, false>": "k_fwd_nf4", "k_nf4_tile<true, false>": "k_bwd_dx_nf4",
                  "k_nf4_tile<false, true>": "k_fwd_bf16w",
                  "k_gemv_nf4<false>": "k_gemv_nf4", "k_gemv_nf4<true>": "k_gemv_nf4_single"}


def short_kernel_name(name: str) -> str:
    base = name.replace("qlora::(anonymous namespace)::", "").replace("qlora::", "")
    base = base.split("(")[0].replace("void ", "").strip()
    return KERNEL_ALIASES.get(base, base)


def load_traffic(target: str) -> dict:
    """{kernel: counters} of one family when its file matches the current
    sources, else {}."""
    path = TRAFFIC_FILES[target]
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        tc = json.load(f)
    return tc.get("kernels", {}) if tc.get("source_sha256") == source_digest(target) else {}


def ingest_pmc(fetch_dir: str, write_dir: str, target: str) -> None:
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) -> bytes per launch, each
    scaled so the calibration copy reads and writes its known size."""
    def load(folder, counter):
        per = collections.defaultdict(float)  # (kernel, dispatch) -> value
        for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if row["Counter_Name"] == counter:
                        per[(short_kernel_name(row["Kernel_Name"]), row["Dispatch_Id"])] += float(row["Counter_Value"])
        by = collections.defaultdict(list)
        for (k, _), v in per.items():
            by[k].append(v)
        return by
    fetch, write = load(fetch_dir, "FETCH_SIZE"), load(write_dir, "WRITE_SIZE")
    calib_path = os.path.join(fetch_dir, "calib_copy.json")
    with open(calib_path) as fh:
        copy_bytes = json.load(fh)["copy_bytes_read"]
    # the calibration copy: the elementwise kernel with the largest dispatch
    cands = [k for k in fetch if "elementwise" in k]
    ck = max(cands, key=lambda k: max(fetch[k]))
    f_raw, w_raw = max(fetch[ck]), max(write[ck])
    f_scale, w_scale = copy_bytes / f_raw, copy_bytes / w_raw
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k.startswith("k_"):
            fm, wm = sum(fetch[k]) / len(fetch[k]), sum(write[k]) / len(write[k])
            kernels[k] = {"dispatches": len(fetch[k]), "fetch_raw_per_launch": round(fm, 1),
                          "write_raw_per_launch": round(wm, 1),
                          "fetch_bytes_per_launch": round(fm * f_scale), "write_bytes_per_launch": round(wm * w_scale)}
    out = {"source_sha256": source_digest(target), "sources": list(COUNTER_SOURCES[target]),
           "counters": ["FETCH_SIZE", "WRITE_SIZE"],
           "calibration": {"kernel": ck, "copy_bytes": copy_bytes, "fetch_raw": f_raw, "write_raw": w_raw,
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": kernels}
    with open(TRAFFIC_FILES[target], "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out["calibration"]))
    for k, v in kernels.items():
        print(f"{k:28s} {v['dispatches']:4d} fetch {v['fetch_bytes_per_launch'] / 1e6:10.1f} MB  "
              f"write {v['write_bytes_per_launch'] / 1e6:10.1f} MB per launch")


def main():
    args = parse()
    if args.ingest_pmc:
        ingest_pmc(*args.ingest_pmc, args.pmc_target)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_nf4_quantized_qlora_amd import inputs as I
    from bit_nf4_quantized_qlora_amd import qlora as q

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    wl = I.WORKLOADS[args.workload]
    M = wl.ms[0]
    r, alpha = wl.r, wl.alpha
    stream = torch.cuda.current_stream()

    def dev16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    calib = calib_copy(torch, dev, args.calib_copy_mib) if args.calib_copy_mib else None

    if args.configs_only:
        print(json.dumps({c: config_rows(q, I, c, dev, lambda: torch.cuda.Event(enable_timing=True), dev16)
                          for c in ("q_proj_7b", "block_65b")}), flush=True)
        return

    if args.small_m_only:
        print(json.dumps({"small_m": small_m_rows(q, I, np, torch, dev, dev16, lambda: torch.cuda.Event(enable_timing=True))}),
              flush=True)
        return

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # ---------------------------------------------------------------- setup
    layers = []
    quant_ms, quant_bytes, deq_ms, deq_bytes = 0.0, 0, 0.0, 0
    for li, L in enumerate(wl.layers):
        W = torch.from_numpy(I.weight(wl, li)).to(dev)
        w = q.NF4Weight.empty(L.n, L.k, dev)
        qws = torch.empty(q.qlora_quantize_workspace_bytes(L.n, L.k), dtype=torch.uint8, device=dev)
        q.qlora_quantize_nf4_dq(W, w, qws)                          # untimed first call
        pb, sb, ng = q.qlora_nf4_sizes(L.n, L.k)
        enc_bytes = pb + sb + 4 * ng + 4
        if not args.no_extras:
            reps = 5
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                q.qlora_quantize_nf4_dq(W, w, qws)
            e1.record()
            torch.cuda.synchronize()
            quant_ms += e0.elapsed_time(e1) / reps
            quant_bytes += 4 * L.n * L.k + enc_bytes
            Wh = torch.empty(L.n, L.k, dtype=torch.bfloat16, device=dev)
            q.qlora_dequant_bf16(w, Wh)
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(reps):
                q.qlora_dequant_bf16(w, Wh)
            e1.record()
            torch.cuda.synchronize()
            deq_ms += e0.elapsed_time(e1) / reps
            deq_bytes += enc_bytes + 2 * L.n * L.k
            del Wh
        del W, qws
        A, B = I.adapters(wl, li)
        t = {"L": L, "w": w, "X": dev16(I.activation(wl, li, M)), "dY": dev16(I.grad_output(wl, li, M)),
             "A": dev16(A), "B": dev16(B)}
        t["Y"] = torch.empty(M, L.n, dtype=torch.bfloat16, device=dev)
        t["H"] = torch.empty(M, r, dtype=torch.float32, device=dev)
        t["dX"] = torch.empty(M, L.k, dtype=torch.bfloat16, device=dev)
        t["dA"] = torch.empty(r, L.k, dtype=torch.bfloat16, device=dev)
        t["dB"] = torch.empty(L.n, r, dtype=torch.bfloat16, device=dev)
        layers.append(t)
    ws_bytes = max(q.qlora_linear_workspace_bytes(M, t["L"].n, t["L"].k, r) for t in layers)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.empty_cache()
    if args.layer_only:
        print(json.dumps({"decoder_layer": layer_rows(q, I, layers, dev, ev, M, r, alpha, wl.adapter_bound)}),
              flush=True)
        return

    def fwd_pass():
        for t in layers:
            q.qlora_linear_fwd(t["w"], t["X"], t["A"], t["B"], r, alpha, t["Y"], t["H"], ws)

    def bwd_pass():
        for t in reversed(layers):
            q.qlora_linear_bwd(t["w"], t["X"], t["dY"], t["A"], t["B"], r, alpha, t["H"], t["dX"], t["dA"],
                               t["dB"], ws)

    def step():
        fwd_pass()
        bwd_pass()

    fwd_flops = bwd_flops = 0
    for t in layers:
        f, b = layer_flops(M, t["L"].n, t["L"].k, r)
        fwd_flops += f
        bwd_flops += b
    step_flops = fwd_flops + bwd_flops

    # ---------------------------------------------------------- timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    # per-pass times
    def timed(fn, n):
        a, b = ev(), ev()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    fwd_ms = timed(fwd_pass, max(3, args.steps // 2))
    bwd_ms = timed(bwd_pass, max(3, args.steps // 2))

    # per-step spread: the same steps one at a time, events around each
    evs = [(ev(), ev()) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in evs)
    spread = {"p10": round(float(np.percentile(per_step, 10)), 4), "p50": round(float(np.percentile(per_step, 50)), 4),
              "p90": round(float(np.percentile(per_step, 90)), 4)}

    # --------------------------------------- per-kernel event timing (second pass)
    prof = traced(q, step, args.steps)
    kernels = {name: {"launches_per_step": n / args.steps, "avg_us": 1e3 * ms / n,
                      "ms_per_step": ms / args.steps} for name, (n, ms) in prof.items()}
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    # algorithmic flops of one launch (same M*N*K for every MLP layer): the
    # forward GEMM carries the LoRA up-projection, the dX GEMM the G A term
    fwd_launch = sum(2 * M * t["L"].n * t["L"].k + 2 * M * t["L"].n * r for t in layers) / len(layers)
    dx_launch = sum(2 * M * t["L"].n * t["L"].k + 2 * M * t["L"].k * r for t in layers) / len(layers)
    per_launch_flops = {"k_fwd_nf4": fwd_launch, "k_bwd_dx_nf4": dx_launch, "k_bwd_dx": dx_launch}
    traffic = None
    tile_tc = load_traffic("tile")
    if dom in tile_tc:
        traffic = tile_tc[dom]["fetch_bytes_per_launch"] + tile_tc[dom]["write_bytes_per_launch"]
    if dom in per_launch_flops:
        ach = per_launch_flops[dom] / (kernels[dom]["avg_us"] * 1e-6) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                    "flops_per_launch": per_launch_flops[dom], "avg_launch_us": round(kernels[dom]["avg_us"], 2)}
    else:
        roofline = {"bound": "unknown", "kernel": dom, "achieved": None, "peak": None, "unit": None,
                    "frac": None, "traffic": traffic}

    rows = {
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 1),
                "frac_bf16_peak": round(fwd_flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1),
                "frac_bf16_peak": round(bwd_flops / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
    }
    if not args.no_extras:
        for cname in ("q_proj_7b", "block_65b"):
            rows[cname] = config_rows(q, I, cname, dev, ev, dev16)
        rows["quantize"] = {"ms_all_layers": round(quant_ms, 4),
                            "gbps": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
                            "frac_hbm_peak": round(quant_bytes / (quant_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        rows["dequant"] = {"ms_all_layers": round(deq_ms, 4),
                           "gbps": round(deq_bytes / (deq_ms * 1e-3) / 1e9, 1),
                           "frac_hbm_peak": round(deq_bytes / (deq_ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}
        rows["small_m"] = small_m_rows(q, I, np, torch, dev, dev16, ev)
        rows["storage_types"] = storage_rows(q, I, wl, layers, dev, ev, ws, M, r, alpha, step_flops)
        rows["storage_types"]["bf16_weights_fwd"] = bf16_weight_rows(q, layers, dev, ev, ws, M, r, alpha)
        rows["merge"] = merge_rows(q, layers, dev, ev, r, alpha)
        rows["adamw"] = adamw_rows(q, layers, dev, ev)
        if wl.name == "mlp_7b":
            rows["mlp_block"] = block_rows(q, layers, dev, ev, ws, M, r, alpha, step_flops)
            rows["decoder_layer"] = layer_rows(q, I, layers, dev, ev, M, r, alpha, wl.adapter_bound)


    attainable = None
    if not args.no_extras:
        attainable = attainable_peaks(torch, dev, ev)
        attainable["mfma_bf16_tflops"] = round(q.mfma_peak_tflops(), 1)
        attainable["mfma_how"] = ("tracing library's k_mfma_peak: v_mfma_f32_16x16x32_bf16 back to back on 8 "
                                  "independent accumulator tiles per wave, 2 waves per SIMD, no memory traffic; "
                                  "fastest of 5 launches")
        if roofline.get("achieved") is not None:
            roofline["frac_attainable"] = round(roofline["achieved"] / attainable["mfma_bf16_tflops"], 4)
        for k, v in rows["small_m"].items():
            if isinstance(v, dict) and "kernel_gbps_packed" in v:
                v["kernel_frac_attainable_read"] = round(v["kernel_gbps_packed"] / attainable["hbm_read_gbps"], 4)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, I, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama7b_mlp_gate_up_down_fwd_bwd", "layers": [[t["L"].name, t["L"].n, t["L"].k]
                                                                           for t in layers],
                   "M": M, "global_batch": 8, "seq_len": 512, "lora_r": r, "lora_alpha": alpha,
                   "weights": "NF4+DQ (block 64, 8-bit E4M3 constants per 256)", "parallelism": "single_gpu"},
        "frac_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "wall_s_timed": round(wall, 3),
        "step_ms_spread": spread,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": rows,
        "kernels": {k: {kk: round(vv, 3) for kk, vv in v.items()} for k, v in sorted(kernels.items())},
        "source_sha256": source_digest("tile"),
    }
    if calib:
        out["calib_copy"] = calib
    if attainable:
        out["attainable"] = attainable
    print(json.dumps(out), flush=True)


def config_rows(q, I, name, dev, ev, dev16, steps=20, warmup=10):
    """One workload's step at its own shapes (every layer's forward, then
    every backward in reverse order, independent seeded inputs per layer, as
    the main step): time per step, TFLOP/s against the BF16 peak, the
    per-kernel times from a traced pass, and each layer's launch plan (tile
    path and contraction splits)."""
    import torch
    wl = I.WORKLOADS[name]
    M, r, alpha = wl.ms[0], wl.r, wl.alpha
    layers = []
    for li, L in enumerate(wl.layers):
        W = torch.from_numpy(I.weight(wl, li)).to(dev)
        w = q.NF4Weight.empty(L.n, L.k, dev)
        qws = torch.empty(q.qlora_quantize_workspace_bytes(L.n, L.k), dtype=torch.uint8, device=dev)
        q.qlora_quantize_nf4_dq(W, w, qws)
        del W, qws
        A, B = I.adapters(wl, li)
        layers.append({"L": L, "w": w, "X": dev16(I.activation(wl, li, M)), "dY": dev16(I.grad_output(wl, li, M)),
                       "A": dev16(A), "B": dev16(B),
                       "Y": torch.empty(M, L.n, dtype=torch.bfloat16, device=dev),
                       "H": torch.empty(M, r, dtype=torch.float32, device=dev),
                       "dX": torch.empty(M, L.k, dtype=torch.bfloat16, device=dev),
                       "dA": torch.empty(r, L.k, dtype=torch.bfloat16, device=dev),
                       "dB": torch.empty(L.n, r, dtype=torch.bfloat16, device=dev)})
    ws = torch.empty(max(q.qlora_linear_workspace_bytes(M, t["L"].n, t["L"].k, r) for t in layers),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    def fwd_pass():
        for t in layers:
            q.qlora_linear_fwd(t["w"], t["X"], t["A"], t["B"], r, alpha, t["Y"], t["H"], ws)

    def bwd_pass():
        for t in reversed(layers):
            q.qlora_linear_bwd(t["w"], t["X"], t["dY"], t["A"], t["B"], r, alpha, t["H"], t["dX"], t["dA"],
                               t["dB"], ws)

    def step():
        fwd_pass()
        bwd_pass()

    def timed(fn, n):
        a, b = ev(), ev()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ms = timed(step, steps)
    fwd_ms, bwd_ms = timed(fwd_pass, steps), timed(bwd_pass, steps)
    ff = bf = 0
    for t in layers:
        f, b = layer_flops(M, t["L"].n, t["L"].k, r)
        ff, bf = ff + f, bf + b
    prof = traced(q, step, 5)
    graph_ms, graph_same = graph_step(torch, step, [t[k] for t in layers for k in ("Y", "H", "dX", "dA", "dB")],
                                      timed, steps)
    tf = lambda fl, m: round(fl / (m * 1e-3) / 1e12, 1)
    out = {"workload": f"{name}: " + ", ".join(f"{t['L'].name} {t['L'].k}->{t['L'].n}" for t in layers) +
                       f"; M = {M}, r = {r}",
           "ms": round(ms, 4), "tflops": tf(ff + bf, ms), "frac_bf16_peak": round((ff + bf) / (ms * 1e-3) / 1e12 /
                                                                                    PEAK_BF16_TFLOPS, 4),
           "fwd_ms": round(fwd_ms, 4), "fwd_tflops": tf(ff, fwd_ms), "bwd_ms": round(bwd_ms, 4),
           "bwd_tflops": tf(bf, bwd_ms), "flops_per_step": ff + bf,
           "graph": {"ms": round(graph_ms, 4), "tflops": tf(ff + bf, graph_ms),
                     "frac_bf16_peak": round((ff + bf) / (graph_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "replays_equal_eager": graph_same,
                     "how": "the same step captured once as a HIP graph (torch.cuda.graph on the current stream) "
                            "and replayed: no host launch cost per kernel; three replays compared bit for bit "
                            "with the eager step's outputs first"},
           "plans": {t["L"].name: q.qlora_linear_plan(M, t["L"].n, t["L"].k, r) for t in layers},
           "kernels_us": {k: {"launches_per_step": n / 5, "avg_us": round(1e3 * v / n, 2)}
                          for k, (n, v) in sorted(prof.items())}}
    del layers, ws
    torch.cuda.empty_cache()
    return out


def graph_step(torch, step, outs, timed, steps):
    """Capture step() as a HIP graph and replay it: the replay time per step,
    and whether three replays (outputs overwritten with NaN before each)
    equal the eager step's outputs bit for bit."""
    bits = lambda v: v.view(torch.int32) if v.dtype == torch.float32 else v.view(torch.int16)
    step()
    torch.cuda.synchronize()
    ref = [v.clone() for v in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one run off the capture first, as torch asks
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    same = True
    for _ in range(3):
        for v in outs:
            v.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        same = same and all(torch.equal(bits(v), bits(r)) for v, r in zip(outs, ref))
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms = timed(g.replay, steps)
    del g
    return ms, same


def calib_copy(torch, dev, mib):
    """A plain elementwise copy of known size (counter calibration): each
    traffic counter is scaled by what it reads for this kernel."""
    nbytes = mib << 20
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):  # an elementwise kernel (a plain copy_ may go to a DMA engine)
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    calib = {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "kernel": "elementwise mul by 1"}
    del src, dst
    torch.cuda.empty_cache()
    if os.environ.get("QLORA_CALIB_DIR"):
        with open(os.path.join(os.environ["QLORA_CALIB_DIR"], "calib_copy.json"), "w") as fh:
            json.dump(calib, fh)
    return calib


def traced(q, fn, reps):
    """Per-kernel event times of `reps` calls of fn through the tracing build
    of the library (same kernels; events recorded on each launch's stream):
    {kernel: (launches, total ms)}.  One untimed call first loads its code."""
    import torch
    q.use_tracing_library(True)
    try:
        fn()
        torch.cuda.synchronize()
        q.qlora_profile_begin()
        for _ in range(reps):
            fn()
        return q.qlora_profile_end()
    finally:
        q.use_tracing_library(False)


def storage_rows(q, I, wl, layers, dev, ev, ws, M, r, alpha, step_flops):
    """The same fwd+bwd step with the comparison storage types: Float4 (E2M1)
    and Float4 (E3M0) codes instead of NF4, and single-level float32 block
    constants (double
    quantization off, 4.5 bits) instead of the double-quantized ones.  Each
    variant's step is timed alternately with the NF4+DQ step (same inputs,
    same workspace), 3 rounds of 3 warm-up + 10 timed steps, minimum per
    variant; plus its standalone dequantization rate on its own bytes."""
    import torch
    variants = {"nf4_dq": (q.QLORA_CODEBOOK_NF4, q.QLORA_SCALES_DQ),
                "fp4_dq": (q.QLORA_CODEBOOK_FP4_E2M1, q.QLORA_SCALES_DQ),
                "fp4e3m0_dq": (q.QLORA_CODEBOOK_FP4_E3M0, q.QLORA_SCALES_DQ),
                "nf4_fp32_absmax": (q.QLORA_CODEBOOK_NF4, q.QLORA_SCALES_FP32),
                "fp4_fp32_absmax": (q.QLORA_CODEBOOK_FP4_E2M1, q.QLORA_SCALES_FP32)}
    weights = {}
    for name, (cb, sc) in variants.items():
        ws_list = []
        for li, t in enumerate(layers):
            if name == "nf4_dq":
                ws_list.append(t["w"])
                continue
            L = t["L"]
            W = torch.from_numpy(I.weight(wl, li)).to(dev)
            w = q.NF4Weight.empty(L.n, L.k, dev, codebook=cb, scales=sc)
            qws = torch.empty(q.qlora_quantize_workspace_bytes(L.n, L.k), dtype=torch.uint8, device=dev)
            q.qlora_quantize_nf4_dq(W, w, qws)
            del W, qws
            ws_list.append(w)
        weights[name] = ws_list

    def step(wlist):
        for t, w in zip(layers, wlist):
            q.qlora_linear_fwd(w, t["X"], t["A"], t["B"], r, alpha, t["Y"], t["H"], ws)
        for t, w in zip(reversed(layers), reversed(wlist)):
            q.qlora_linear_bwd(w, t["X"], t["dY"], t["A"], t["B"], r, alpha, t["H"], t["dX"], t["dA"], t["dB"], ws)

    best = {n: float("inf") for n in variants}
    for _ in range(3):
        for name in variants:
            for _ in range(3):
                step(weights[name])
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for _ in range(10):
                step(weights[name])
            b.record()
            torch.cuda.synchronize()
            best[name] = min(best[name], a.elapsed_time(b) / 10)
    out = {}
    for name, (cb, sc) in variants.items():
        deq_ms, deq_bytes, store_bytes, nw = 0.0, 0, 0, 0
        for t, w in zip(layers, weights[name]):
            L = t["L"]
            pb, sb, ng = q.qlora_nf4_sizes(L.n, L.k)
            enc = pb + (4 * sb if sc == q.QLORA_SCALES_FP32 else sb + 4 * ng + 4)
            Wh = torch.empty(L.n, L.k, dtype=torch.bfloat16, device=dev)
            q.qlora_dequant_bf16(w, Wh)
            a, b = ev(), ev()
            a.record()
            for _ in range(5):
                q.qlora_dequant_bf16(w, Wh)
            b.record()
            torch.cuda.synchronize()
            deq_ms += a.elapsed_time(b) / 5
            deq_bytes += enc + 2 * L.n * L.k
            store_bytes += enc - (0 if sc == q.QLORA_SCALES_FP32 else 4)
            nw += L.n * L.k
            del Wh
        out[name] = {"step_ms": round(best[name], 4),
                     "tflops": round(step_flops / (best[name] * 1e-3) / 1e12, 1),
                     "step_vs_nf4_dq": round(best[name] / best["nf4_dq"], 4),
                     "dequant_gbps": round(deq_bytes / (deq_ms * 1e-3) / 1e9, 1),
                     "bits_per_weight": round(8 * store_bytes / nw, 6)}
    out["how"] = ("same 7B MLP step and inputs per storage type, alternated with nf4_dq, min of 3 x 10 steps; "
                  "dequant rate on each type's own bytes (codes + constants + bf16 out)")
    for name in variants:
        if name != "nf4_dq":
            del weights[name]
    torch.cuda.empty_cache()
    return out


def bf16_weight_rows(q, layers, dev, ev, ws, M, r, alpha):
    """The 16-bit baseline on the same kernels: the forward of the three
    layers with NF4+DQ weights (codes expanded in the tile kernel, block-scale
    table job) against the same forward with the weights already in BF16
    (W_hat, the same tile kernel reading BF16 tiles: no expansion, no table),
    both through the tracing library, alternated, 3 rounds of 3 warm-up +
    10 timed passes, minimum each; plus each tile kernel's average launch.
    Bytes per weight read by the tile kernel: 0.516 (NF4+DQ) vs 2 (BF16)."""
    import torch
    W16 = []
    for t in layers:
        Wh = torch.empty(t["L"].n, t["L"].k, dtype=torch.bfloat16, device=dev)
        q.qlora_dequant_bf16(t["w"], Wh)
        W16.append(Wh)

    def fwd_nf4():
        for t in layers:
            q.qlora_linear_fwd(t["w"], t["X"], t["A"], t["B"], r, alpha, t["Y"], t["H"], ws)

    def fwd_bf16():
        for t, Wh in zip(layers, W16):
            q.qlora_profile_linear_fwd_bf16w(Wh, t["X"], t["A"], t["B"], r, alpha, t["Y"], t["H"], ws)

    best = {"nf4_dq": float("inf"), "bf16": float("inf")}
    q.use_tracing_library(True)
    try:
        for _ in range(3):
            for name, fn in (("nf4_dq", fwd_nf4), ("bf16", fwd_bf16)):
                for _ in range(3):
                    fn()
                torch.cuda.synchronize()
                a, b = ev(), ev()
                a.record()
                for _ in range(10):
                    fn()
                b.record()
                torch.cuda.synchronize()
                best[name] = min(best[name], a.elapsed_time(b) / 10)
    finally:
        q.use_tracing_library(False)
    kn = traced(q, fwd_nf4, 5).get("k_fwd_nf4")
    kb = traced(q, fwd_bf16, 5).get("k_fwd_bf16w")
    out = {"fwd_ms_nf4_dq": round(best["nf4_dq"], 4), "fwd_ms_bf16": round(best["bf16"], 4),
           "fwd_nf4_over_bf16": round(best["nf4_dq"] / best["bf16"], 4)}
    if kn and kb:
        out["tile_us_nf4_dq"] = round(1e3 * kn[1] / kn[0], 2)
        out["tile_us_bf16"] = round(1e3 * kb[1] / kb[0], 2)
        out["tile_nf4_over_bf16"] = round(kn[1] / kn[0] / (kb[1] / kb[0]), 4)
    out["how"] = ("7B MLP forward (gate, up, down; M = 4096): NF4+DQ expanded in the tile kernel vs the same tile "
                  "kernel on W_hat in BF16 (qlora_profile_linear_fwd_bf16w), identical outputs bit for bit")
    del W16
    torch.cuda.empty_cache()
    return out


def merge_rows(q, layers, dev, ev, r, alpha):
    """Adapter merge (deployment step) on the three layers: W' = W_hat + s B A
    in float64 (2r flops per weight), its bf16 copy and the NF4+DQ
    re-encoding of W'.  Timed whole (events) and per kernel (library timer)."""
    import torch
    nmax = max(t["L"].n * t["L"].k for t in layers)
    mws = torch.empty(max(q.qlora_merge_workspace_bytes(t["L"].n, t["L"].k) for t in layers), dtype=torch.uint8,
                      device=dev)
    outs = [q.NF4Weight.empty(t["L"].n, t["L"].k, dev) for t in layers]
    Wb = torch.empty(nmax, dtype=torch.bfloat16, device=dev)

    def run():
        for t, o in zip(layers, outs):
            q.qlora_merge_adapters(t["w"], t["A"], t["B"], r, alpha, Wb[: t["L"].n * t["L"].k], o, mws)

    run()
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for _ in range(3):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 3
    prof = traced(q, run, 1)
    flops = sum(2 * r * t["L"].n * t["L"].k for t in layers)
    kern = {k: round(1e3 * v[1] / v[0], 1) for k, v in prof.items()}
    km = prof.get("k_merge", (1, ms))[1]
    del mws, outs, Wb
    torch.cuda.empty_cache()
    return {"ms_all_layers": round(ms, 4), "kernels_us": kern,
            "merge_fp64_tflops": round(flops / (km * 1e-3) / 1e12, 2),
            "merge_frac_fp64_peak": round(flops / (km * 1e-3) / 1e12 / 78.6, 4),
            "how": "W_hat + s B A in float64 (2r flops per weight) + bf16 copy + NF4+DQ re-encoding, 3 layers"}


def adamw_rows(q, layers, dev, ev):
    """One AdamW step over the three layers' adapters (A and B: r (k + n)
    parameters each), moments in HBM and, the paged layout, in pinned host
    memory mapped for the device.  28 B per parameter move in either case
    (16 of them, the moments, cross the host link in the paged one)."""
    import ctypes
    import torch
    count = sum(t["A"].numel() + t["B"].numel() for t in layers)
    P = torch.zeros(count, dtype=torch.float32, device=dev)
    P16 = torch.empty(count, dtype=torch.bfloat16, device=dev)
    G = torch.full((count,), 1e-3, dtype=torch.bfloat16, device=dev)
    md = torch.zeros(count, dtype=torch.float32, device=dev)
    vd = torch.zeros(count, dtype=torch.float32, device=dev)

    def timed(m, v, reps=20):
        for i in range(3):
            q.qlora_adamw_step(P, P16, G, m, v, 2e-4, 0.9, 0.999, 1e-8, 0.01, 1 + i)
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for i in range(reps):
            q.qlora_adamw_step(P, P16, G, m, v, 2e-4, 0.9, 0.999, 1e-8, 0.01, 4 + i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    out = {"params": count}
    ms = timed(md, vd)
    out["hbm_state"] = {"us": round(1e3 * ms, 2), "gbps": round(28 * count / (ms * 1e-3) / 1e9, 1)}
    mh = torch.zeros(count, dtype=torch.float32).pin_memory()
    vh = torch.zeros(count, dtype=torch.float32).pin_memory()
    hip = ctypes.CDLL("libamdhip64.so")
    ptrs = []
    for t in (mh, vh):
        d = ctypes.c_void_p()
        ptrs.append(d.value if hip.hipHostGetDevicePointer(ctypes.byref(d), ctypes.c_void_p(t.data_ptr()), 0) == 0
                    else None)
    if all(ptrs):
        ms = timed(ptrs[0], ptrs[1], reps=5)
        out["pinned_host_state"] = {"us": round(1e3 * ms, 2),
                                    "host_link_gbps": round(16 * count / (ms * 1e-3) / 1e9, 1)}
    out["how"] = "3 MLP layers' A and B; state in HBM, then in pinned host memory addressed by the kernel"
    del P, P16, G, md, vd, mh, vh
    torch.cuda.empty_cache()
    return out


def block_rows(q, layers, dev, ev, ws, M, r, alpha, step_flops):
    """The same three layers chained as the LLaMA MLP block: gate and up on
    one X, SwiGLU, down on its output; backward through down, the gate/up
    outputs recomputed from X (checkpointing), SwiGLU's backward, gate and
    up, and the sum of the two input gradients."""
    import torch
    g, u, d = layers
    X = g["X"]
    n = g["L"].n
    h = torch.empty(M, n, dtype=torch.bfloat16, device=dev)
    dh, dg, du = (torch.empty(M, n, dtype=torch.bfloat16, device=dev) for _ in range(3))
    dX = torch.empty_like(g["dX"])

    def fwd():
        q.qlora_linear_fwd(g["w"], X, g["A"], g["B"], r, alpha, g["Y"], g["H"], ws)
        q.qlora_linear_fwd(u["w"], X, u["A"], u["B"], r, alpha, u["Y"], u["H"], ws)
        q.qlora_swiglu_fwd(g["Y"], u["Y"], h)
        q.qlora_linear_fwd(d["w"], h, d["A"], d["B"], r, alpha, d["Y"], d["H"], ws)

    def bwd():
        q.qlora_linear_bwd(d["w"], h, d["dY"], d["A"], d["B"], r, alpha, d["H"], dh, d["dA"], d["dB"], ws)
        q.qlora_linear_fwd(g["w"], X, g["A"], g["B"], r, alpha, g["Y"], None, ws)    # recompute
        q.qlora_linear_fwd(u["w"], X, u["A"], u["B"], r, alpha, u["Y"], None, ws)
        q.qlora_swiglu_bwd(g["Y"], u["Y"], dh, dg, du)
        q.qlora_linear_bwd(g["w"], X, dg, g["A"], g["B"], r, alpha, g["H"], g["dX"], g["dA"], g["dB"], ws)
        q.qlora_linear_bwd(u["w"], X, du, u["A"], u["B"], r, alpha, u["H"], u["dX"], u["dA"], u["dB"], ws)
        q.qlora_add_bf16(g["dX"], u["dX"], dX)

    for _ in range(5):
        fwd()
        bwd()
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for _ in range(10):
        fwd()
        bwd()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 10
    recompute = sum(2 * M * t["L"].n * t["L"].k + 2 * M * r * (t["L"].n + t["L"].k) for t in (g, u))
    out = {"ms": round(ms, 4), "tflops": round(step_flops / (ms * 1e-3) / 1e12, 1),
           "tflops_with_recompute": round((step_flops + recompute) / (ms * 1e-3) / 1e12, 1),
           "how": "gate, up -> SwiGLU -> down; backward recomputes gate/up outputs; tflops counts the three "
                  "layers' fwd+bwd flops (the step's), the second figure adds the recomputed forwards"}
    del h, dh, dg, du, dX
    torch.cuda.empty_cache()
    return out


def layer_rows(q, I, layers, dev, ev, M, r, alpha, adapter_bound, seq=512, heads=32, head_dim=128):
    """The LLaMA-7B decoder layer: q, k, v, o (4096 x 4096 NF4+DQ, each with
    its own adapters) around the causal attention core (M / 512 sequences of
    512 tokens, 32 heads of 128), the residuals and the MLP layers above;
    the backward recomputes from X the activations up to the SwiGLU output
    (checkpointing).  Then the
    attention core alone at the same shape.  Attention flops count the
    causal pairs only: per head 4 d per pair forward (QK^T, PV) and 8 d
    backward (dV, dP, dQ, dK)."""
    import numpy as np
    import torch
    from bit_nf4_quantized_qlora_amd.layer import DecoderLayer
    g, u, d = layers
    hidden, batch = heads * head_dim, M // seq
    d16 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
    weights = {"gate": g["w"], "up": u["w"], "down": d["w"]}
    adapters = {"gate": (g["A"], g["B"]), "up": (u["A"], u["B"]), "down": (d["A"], d["B"])}
    qws = torch.empty(q.qlora_quantize_workspace_bytes(hidden, hidden), dtype=torch.uint8, device=dev)
    for i, nm in enumerate(("q", "k", "v", "o")):
        w = q.NF4Weight.empty(hidden, hidden, device=dev)
        q.qlora_quantize_nf4_dq(torch.from_numpy(I.custom_weight(hidden, hidden, 500 + i)).to(dev), w, qws)
        weights[nm] = w
        adapters[nm] = (d16(I.custom_bf16((r, hidden), 510 + i, 1, bound=adapter_bound)),
                        d16(I.custom_bf16((hidden, r), 510 + i, 2, bound=adapter_bound)))
    del qws
    lay = DecoderLayer(weights, adapters, r, alpha, batch, seq, heads, head_dim, device=dev)
    X, dY = g["X"], d["dY"]
    Y, dX = (torch.empty(M, hidden, dtype=torch.bfloat16, device=dev) for _ in range(2))

    def timed(fn, n=10, warm=3):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    ms = timed(lambda: (lay.fwd(X, Y), lay.bwd(X, dY, dX)))
    lin_f = lin_b = 0
    for nm, w in weights.items():
        f, b_ = layer_flops(M, w.n, w.k, r)
        lin_f, lin_b = lin_f + f, lin_b + b_
    pairs = batch * heads * seq * (seq + 1) // 2
    att_f, att_b = 4 * head_dim * pairs, 8 * head_dim * pairs
    down_f = layer_flops(M, weights["down"].n, weights["down"].k, r)[0]
    flops, recompute = lin_f + lin_b + att_f + att_b, lin_f - down_f + att_f   # the backward recomputes up to h
    a = lay.act
    g_ = lay.grad
    fwd_ms = timed(lambda: q.qlora_attention_fwd(a["q"], a["k"], a["v"], a["attn"], lay.lse, batch, seq, heads,
                                                 head_dim, lay.ws))
    bwd_ms = timed(lambda: q.qlora_attention_bwd(a["q"], a["k"], a["v"], g_["dattn"], lay.lse, g_["dq"],
                                                 g_["dk"], g_["dv"], batch, seq, heads, head_dim, lay.ws))
    tf = lambda fl, m: round(fl / (m * 1e-3) / 1e12, 1)
    out = {"ms": round(ms, 4), "tflops": tf(flops, ms), "tflops_with_recompute": tf(flops + recompute, ms),
           "attention": {"fwd_ms": round(fwd_ms, 4), "fwd_tflops": tf(att_f, fwd_ms),
                         "bwd_ms": round(bwd_ms, 4), "bwd_tflops": tf(att_b, bwd_ms),
                         "frac_bf16_peak": round((att_f + att_b) / ((fwd_ms + bwd_ms) * 1e-3) / 1e12
                                                 / PEAK_BF16_TFLOPS, 4)},
           "how": f"q,k,v,o (4096x4096) + gate,up,down NF4+DQ with r={r} adapters, causal attention over {batch} "
                  f"sequences of {seq} ({heads} heads of {head_dim}), SwiGLU, residuals; fwd + checkpointed bwd (recomputes up to the SwiGLU output); "
                  "tflops counts the 7 projections' fwd+bwd and the causal attention pairs, the second figure adds "
                  "the recomputed forward"}
    del lay, Y, dX
    torch.cuda.empty_cache()
    return out


def attainable_peaks(torch, dev, ev):
    """What the box sustains, measured beside the run (the second denominator
    next to the spec peaks): an elementwise copy and a read-only reduction
    over 1 GiB (the fastest of three torch reductions), and a large vendor
    BF16 GEMM (8192^3, hipBLASLt via torch.matmul) as context.  Medians of 10
    timed calls after 3 warm-ups.  The matrix-core denominator itself is the
    library's MFMA microbenchmark (mfma_bf16_tflops, added by the caller)."""
    def med(fn, n=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return sorted(ts)[len(ts) // 2]
    nb = 1 << 30
    src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    copy_ms = med(lambda: torch.mul(src, 1.0, out=dst))
    v = src.view(-1, 1 << 16)
    reads = {"sum_all": med(lambda: torch.sum(src)), "sum_rows": med(lambda: torch.sum(v, dim=1)),
             "amax_rows": med(lambda: torch.amax(v, dim=1))}
    read_best = min(reads, key=reads.get)
    read_ms = reads[read_best]
    del src, dst, v
    n = 8192
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    gemm_ms = med(lambda: torch.matmul(a, b))
    del a, b
    torch.cuda.empty_cache()
    return {"hbm_copy_gbps": round(2 * nb / (copy_ms * 1e-3) / 1e9, 1),
            "hbm_read_gbps": round(nb / (read_ms * 1e-3) / 1e9, 1), "hbm_read_kernel": read_best,
            "bf16_gemm_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 1),
            "how": "1 GiB elementwise copy; fastest of three 1 GiB torch reductions; torch.matmul bf16 8192^3; medians of 10"}


def small_m_rows(q, I, np, torch, dev, dev16, ev, copies=6):
    """65B up_proj forward at M = 1, 4, 16 on rotating weight copies; and at
    M = 1 with single-level float32 block constants (4.5 bits) for the
    bandwidth double quantization saves on the same kernel."""
    wl = I.WORKLOADS["up_65b"]
    L = wl.layers[0]
    W = torch.from_numpy(I.weight(wl, 0)).to(dev)
    qws = torch.empty(q.qlora_quantize_workspace_bytes(L.n, L.k), dtype=torch.uint8, device=dev)

    def encode(scales):
        lst = []
        for _ in range(copies):
            w = q.NF4Weight.empty(L.n, L.k, dev, scales=scales)
            q.qlora_quantize_nf4_dq(W, w, qws)
            lst.append(w)
        return lst

    ws_list = encode(q.QLORA_SCALES_DQ)
    torch.cuda.synchronize()
    pb, sb, ng = q.qlora_nf4_sizes(L.n, L.k)
    packed_bytes = pb + sb + 4 * ng
    A, B = I.adapters(wl, 0)
    Ad, Bd = dev16(A), dev16(B)
    out = {"workload": f"up_proj {L.k}->{L.n}", "packed_weight_bytes": packed_bytes, "copies": copies}
    for m in list(wl.ms) + ["1_single_level"]:
        if m == "1_single_level":  # the DQ copies make room for the 4.5-bit ones
            del ws_list
            torch.cuda.empty_cache()
            ws_list = encode(q.QLORA_SCALES_FP32)
            torch.cuda.synchronize()
            packed_bytes = pb + 4 * sb
            m = 1
            key = "M1_single_level"
        else:
            key = f"M{m}"
        X = dev16(I.activation(wl, 0, m))
        Y = torch.empty(m, L.n, dtype=torch.bfloat16, device=dev)
        H = torch.empty(m, wl.r, dtype=torch.float32, device=dev)
        lws = torch.empty(q.qlora_linear_workspace_bytes(m, L.n, L.k, wl.r), dtype=torch.uint8, device=dev)
        for i in range(2 * copies):
            q.qlora_linear_fwd(ws_list[i % copies], X, Ad, Bd, wl.r, wl.alpha, Y, H, lws)
        reps = 10 * copies
        a, b = ev(), ev()
        a.record()
        for i in range(reps):
            q.qlora_linear_fwd(ws_list[i % copies], X, Ad, Bd, wl.r, wl.alpha, Y, H, lws)
        b.record()
        torch.cuda.synchronize()
        us = 1e3 * a.elapsed_time(b) / reps
        gbps = packed_bytes / (us * 1e-6) / 1e9
        row = {"us": round(us, 2), "gbps_packed": round(gbps, 1), "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        if key != f"M{m}":
            row["weight_bytes"] = packed_bytes
        # the streaming kernel on its own (library event timer, separate pass)
        it = iter(range(10 ** 9))
        prof = traced(q, lambda: q.qlora_linear_fwd(ws_list[next(it) % copies], X, Ad, Bd, wl.r, wl.alpha, Y, H, lws),
                      reps)
        gemv_tc = load_traffic("gemv").get("k_gemv_nf4" if key == f"M{m}" else "k_gemv_nf4_single")
        if gemv_tc:
            row["kernel_traffic_bytes"] = {"fetch": gemv_tc["fetch_bytes_per_launch"],
                                           "write": gemv_tc["write_bytes_per_launch"],
                                           "fetch_vs_packed": round(gemv_tc["fetch_bytes_per_launch"] / packed_bytes, 4)}
        if "k_gemv_nf4" in prof:
            n, ms = prof["k_gemv_nf4"]
            kus = 1e3 * ms / n
            row["kernel"] = "k_gemv_nf4"
            row["kernel_us"] = round(kus, 2)
            row["kernel_gbps_packed"] = round(packed_bytes / (kus * 1e-6) / 1e9, 1)
            row["kernel_frac_hbm_peak"] = round(packed_bytes / (kus * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
        if key == "M1":  # the same calls as one replayed HIP graph (a decode loop's usual form)
            def calls():
                for i in range(copies):
                    q.qlora_linear_fwd(ws_list[i], X, Ad, Bd, wl.r, wl.alpha, Y, H, lws)

            def timed_g(fn, n):
                a, b = ev(), ev()
                a.record()
                for _ in range(n):
                    fn()
                b.record()
                torch.cuda.synchronize()
                return a.elapsed_time(b) / n

            gms, same = graph_step(torch, calls, [Y, H], timed_g, 10)
            row["graph"] = {"us": round(1e3 * gms / copies, 2), "replays_equal_eager": same,
                            "how": f"the {copies} rotating calls captured once as a HIP graph and replayed 10 "
                                   "times (per call: no host launch cost); replays compared bit for bit first"}
        out[key] = row
    del W, qws
    return out


def cpu_baseline(wl, I, target_s):
    """The CPU oracle (as it stands) on a bounded sample of the step: every
    layer sliced to its first 2048 weight rows (its own NF4+DQ tensor,
    encoded untimed), all M rows; timed = oracle dequantization to BF16 +
    fp64 forward + fp64 backward, repeated until target_s has elapsed."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import linear, nf4_dq
    n_s = 2048
    M = wl.ms[0]
    prep = []
    flops = 0
    for li, L in enumerate(wl.layers):
        ns = min(n_s, L.n)
        W = I.weight(wl, li, rows=slice(0, ns))
        enc = nf4_dq.quantize_nf4_dq(W)
        A, B = I.adapters(wl, li)
        X = nf4_dq.bf16_bits_to_f64(I.activation(wl, li, M))
        dY = nf4_dq.bf16_bits_to_f64(I.grad_output(wl, li, M))[:, :ns]
        prep.append((enc, ns, L.k, X, dY, nf4_dq.bf16_bits_to_f64(A), nf4_dq.bf16_bits_to_f64(B)[:ns]))
        f, b = layer_flops(M, ns, L.k, wl.r)
        flops += f + b
    reps, t0 = 0, time.perf_counter()
    while True:
        for enc, ns, k, X, dY, A, B in prep:
            Wh = nf4_dq.bf16_bits_to_f64(
                nf4_dq.dequant_bf16(enc["packed"], enc["scale_code"], enc["group_amax"], enc["offset"], ns, k))
            _, H = linear.fwd(X, Wh, A, B, wl.alpha)
            linear.bwd(X, dY, Wh, A, B, wl.alpha, H=H)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or reps >= 20:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    return {"value": round(flops * reps / el / 1e12, 4), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"mlp layers sliced to their first {n_s} weight rows, all {M} rows of X; "
                      f"oracle bf16 dequant + fp64 fwd + bwd; {reps} rep(s) in {el:.1f} s",
            "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
