"""Benchmark of the Spense linear layer on one MI355X.

Workload: 32B-class FFN gate/up projection W[25600, 5120] e4m3 with
per-channel fp32 scales, dense tail = last 25% of K, X[M, 5120] bf16 for
M in {1, 4, 16} (decode).  One step = one spense_linear launch per batch size
(bf16 output), weights already resident in HBM.  Packed weight copies are
rotated so the working set exceeds the 256 MB Infinity Cache and every launch
streams its weights from HBM.  The all-dense MFMA baseline (same kernel
template, dense fraction 1.0) is timed the same way for the speedup.

Prints one JSON line.  Extra keys: per-M timings, dense baseline, pack time,
roofline of the linear kernel, and the CPU oracle baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
WORKLOAD = "gateup_fp8"
CSRC = os.path.join(ROOT, "sparse_dense_gemm_amd", "csrc")
# the kernels and the launch planner that picks them decide the HBM traffic
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("spense_kernels.hip", "spense_internal.h", "spense_api.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "spense_linear_gateup_fp8_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="force the split-K factor (0 = automatic)")
    ap.add_argument("--ms", type=str, default="", help="override batch sizes, e.g. 1,4,16")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 512 MiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(per_launch_alg_bytes):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_dense_gemm_amd as sdg
    import synth

    wl = synth.WORKLOADS[WORKLOAD]
    spec = wl.layers[0]
    Ms = tuple(int(m) for m in args.ms.split(",")) if args.ms else wl.Ms
    Mmax = max(Ms)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.time()
    W, s, X, D = synth.layer_inputs(spec, Mmax)
    gen_s = time.time() - t0
    Wd = torch.from_numpy(W).to(dev)
    sd = torch.from_numpy(s).to(dev)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    stream = torch.cuda.current_stream()

    # ---- pack: once per weight; timed on its own ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    h0 = sdg.spense_pack(Wd, sdg.DT_FP8, scales=sd, dense_cols=D)
    pack_ms = (time.perf_counter() - t0) * 1e3
    info = sdg.spense_info(h0)
    wbytes = info["weight_bytes"]
    copies = max(4, -(-2 * MALL_BYTES // info["device_bytes"]) + 1)
    handles = [h0] + [sdg.spense_pack(Wd, sdg.DT_FP8, scales=sd, dense_cols=D) for _ in range(copies - 1)]
    # all-dense baseline: same kernel template with K_s = 0
    hd0 = sdg.spense_pack(Wd, sdg.DT_FP8, scales=sd, dense_fraction=1.0)
    dinfo = sdg.spense_info(hd0)
    dcopies = max(4, -(-2 * MALL_BYTES // dinfo["device_bytes"]) + 1)
    dhandles = [hd0] + [sdg.spense_pack(Wd, sdg.DT_FP8, scales=sd, dense_fraction=1.0) for _ in range(dcopies - 1)]
    del Wd
    Ys = {M: torch.empty((M, spec.N), dtype=torch.bfloat16, device=dev) for M in Ms}

    def run(hs, M, i):
        sdg.spense_linear_splits(hs[i % len(hs)], Xd[:M], Ys[M], args.splits, stream=stream)

    # ---- warmup ----
    for i in range(args.warmup):
        for M in Ms:
            run(handles, M, i)
            run(dhandles, M, i)
    torch.cuda.synchronize()

    # ---- timed region: K steps of the Spense layer (one launch per batch size) ----
    ev = {M: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for M in Ms}
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for M in Ms:
        ev[M][0].record(stream)
        for i in range(args.steps):
            run(handles, M, i)
        ev[M][1].record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    spense_us = {M: ev[M][0].elapsed_time(ev[M][1]) * 1e3 / args.steps for M in Ms}

    # ---- dense baseline, same protocol (outside the Spense timed region) ----
    dev_ = {M: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for M in Ms}
    torch.cuda.synchronize()
    for M in Ms:
        dev_[M][0].record(stream)
        for i in range(args.steps):
            run(dhandles, M, i)
        dev_[M][1].record(stream)
    torch.cuda.synchronize()
    dense_us = {M: dev_[M][0].elapsed_time(dev_[M][1]) * 1e3 / args.steps for M in Ms}

    def alg_bytes(wb, M):
        return wb + 4 * spec.N + 2 * M * spec.K + 2 * M * spec.N  # weights + scales + X + Y(bf16)

    per_m = {}
    for M in Ms:
        per_m[str(M)] = {
            "spense_us": round(spense_us[M], 3),
            "dense_us": round(dense_us[M], 3),
            "speedup_vs_dense": round(dense_us[M] / spense_us[M], 4),
            "weight_GBs": round(wbytes / spense_us[M] / 1e3, 1),
            "weight_frac_of_peak": round(wbytes / spense_us[M] / 1e3 / HBM_PEAK_GBS, 4),
            "dense_weight_GBs": round(dinfo["weight_bytes"] / dense_us[M] / 1e3, 1),
        }
    total_us = sum(spense_us.values())
    value = len(Ms) * wbytes / total_us / 1e3  # GB/s on compressed + dense weight bytes
    alg = sum(alg_bytes(wbytes, M) for M in Ms)
    achieved = alg / total_us / 1e3
    traffic = load_traffic(alg / len(Ms))

    for hh in handles + dhandles:
        sdg.spense_free(hh)
    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, W, s, X, D, Ms, wbytes)

    out = {
        "metric": "Spense linear us + achieved HBM GB/s at decode M=1..64; speedup vs dense GEMM",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_s * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 weights x bf16 activations, fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": "FFN gate/up W[25600,5120] e4m3 + per-channel scales, dense tail 25% (1280 cols), "
                               "X bf16, M in {" + ",".join(map(str, Ms)) + "}",
                   "N": spec.N, "K": spec.K, "K_d": spec.K_d, "Ms": list(Ms), "weight_copies": copies,
                   "splits": args.splits or "auto"},
        "per_m": per_m,
        "speedup_vs_dense": round(sum(dense_us.values()) / total_us, 4),
        "spense_weight_bytes": wbytes,
        "dense_weight_bytes": dinfo["weight_bytes"],
        "pack_ms_wall": round(pack_ms, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
        "input_gen_s": round(gen_s, 2),
    }
    print(json.dumps(out))


def cpu_baseline(spec, W, s, X, D, Ms, wbytes):
    """The oracle, as it stands, on the same layer: one packed form, then the
    float64 layer output for each batch size.  Throughput on the same weight bytes."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    pi, K_s, _ = oracle.resolve_dense_set(spec.K, dense_cols=D)
    p = oracle.pack(W, oracle.DT_FP8, pi, K_s)
    # repeat whole passes over the batch sizes until about 10 s of CPU work
    passes = 0
    t0 = time.perf_counter()
    while passes < 20 and (passes == 0 or time.perf_counter() - t0 < 10.0):
        for M in Ms:
            oracle.linear_ref(X[:M], oracle.DT_BF16, p, s)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(passes * len(Ms) * wbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"full layer, oracle linear_ref for M in {list(Ms)}, {passes} passes ({dt:.1f} s); pack excluded"}


if __name__ == "__main__":
    main()
