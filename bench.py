"""Benchmark of the Spense linear layer on one MI355X.

Default workload (the headline line): 32B-class FFN gate/up projection
W[25600, 5120] e4m3 with per-channel fp32 scales, dense tail = last 25% of K,
X[M, 5120] bf16 for M in {1, 4, 16} (decode).  One step = one spense_linear
launch per batch size (bf16 output), weights already resident in HBM.  Packed
weight copies are rotated so the working set exceeds the 256 MB Infinity Cache
and every launch streams its weights from HBM.  The all-dense baseline (same
kernels, dense fraction 1.0) is timed the same way for the speedup.

Other workloads (``--workload``):
  gateup_fp8_rows  the gate/up layer in output-split form: the last 25% of the rows
                 dense, the others 2:4 along K, M in {1, 4, 16}
  down_fp8       FFN down W[5120, 25600] e4m3, 6400 chosen dense columns, M in {1, 8, 32, 64}
  glu32b_fp8     the whole GLU MLP block (H = 5120, I = 25600, e4m3): gate/up output-split and
                 down input-split over 6400 chosen dense intermediate indices, permuted into a
                 contiguous block at pack time; one step = one spense_glu call per batch size
                 (two launches), against the all-dense block through the same path
  layer32b_fp8   32B-class decoder linear set (QKV, O, gate+up, down), e4m3, dense
                 tail fraction in {0, 12.5, 25, 50}%, M = 32; one step = the four
                 layers of every fraction
  layer36b_fp8   36B-class decoder linear set, e4m3, 25% chosen dense columns per
                 layer, M in {128, 2048}
  layer36b_bf16  the same with bf16 weights
  layer36b_w8a8  the layer36b_fp8 set in W8A8 form: activations quantised per token to
                 e4m3 (absmax / 448) in the same pass that re-orders their columns, then
                 the fp8 structured-sparse product; one step = spense_linear_w8a8 per
                 layer (quantisation included), against the all-dense layers through the
                 same path
A layer set streams more than the Infinity Cache per pass, so its packed
weights are not rotated.

Before the W warmup steps, the warmup step runs back to back for about 100 ms
(``spin_up_ms`` in the output): the GPU reaches its loaded clock state only
after some milliseconds of continuous work, and the timed steps measure the
sustained rate.

Prints one JSON line.  Extra keys: per-M (and per-layer) timings, dense
baseline, roofline of the linear kernel, and the CPU oracle baseline.
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
# Dense bf16 matrix peak.  The structured-sparse instruction performs half the
# multiply-adds of a dense one in the same time, so 2.5 PFLOP/s is also its
# peak on the nonzero multiply-adds that the algorithmic flops count.
MFMA_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0  # dense e4m3 matrix peak (W8A8)
MALL_BYTES = 256 << 20
CSRC = os.path.join(ROOT, "sparse_dense_gemm_amd", "csrc")
# the kernels and the launch planner that picks them decide the HBM traffic
KERNEL_SRCS = [os.path.join(CSRC, f) for f in ("spense_kernels.hip", "spense_tile.hip", "spense_device.h",
                                              "spense_internal.h", "spense_api.cpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "spense_linear_gateup_fp8_traffic.json")
METRIC = "Spense linear us + achieved HBM GB/s at decode M=1..64; speedup vs dense GEMM"

SETS = {
    "gateup_fp8": ["gateup_fp8"],
    "gateup_fp8_rows": ["gateup_fp8_rows"],
    "down_fp8": ["down_fp8"],
    "glu32b_fp8": ["glu32b_fp8"],
    "layer32b_fp8": ["layer32b_fp8_d0", "layer32b_fp8_d12p5", "layer32b_fp8_d25", "layer32b_fp8_d50"],
    "layer36b_fp8": ["layer36b_fp8"],
    "layer36b_bf16": ["layer36b_bf16"],
    "layer36b_w8a8": ["layer36b_fp8"],
}
A8_SETS = {"layer36b_w8a8"}  # run through spense_linear_w8a8
HEADLINE_VARIANT = {"layer32b_fp8": "layer32b_fp8_d25"}


# Untimed load before the warmup steps.  The GPU leaves its idle clock state
# only after some milliseconds of continuous work: a launch of the 94 MB gate/up
# layer took 19-22 us during the first ~15 ms of back-to-back launches and a
# steady 17.8 us after that, so the timed steps follow at least this much load.
SPIN_UP_S = 0.1


def spin_up(torch, step, seconds=SPIN_UP_S):
    """Runs step(i) in rounds of 8 until `seconds` of wall time have passed,
    each round synchronised (the launch queue stays short).  Returns the ms."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8):
            step(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return (time.perf_counter() - t0) * 1e3


def lead_in(launch):
    """One untimed launch just before the first timing event of a sequence:
    with the device idle, that event would fire at once and the first timed
    kernel would start only when the host has issued it (about one host call,
    7-10 us, spread over the K steps); behind a running kernel the next launch
    is already queued when the event fires."""
    launch()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gateup_fp8", choices=sorted(SETS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--splits", type=int, default=0, help="force the split-K factor (0 = automatic)")
    ap.add_argument("--ms", type=str, default="", help="override batch sizes, e.g. 1,4,16")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run a plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the all-dense baseline (profiling runs: every linear launch is then a Spense one)")
    return ap.parse_args()


def kernel_hash() -> str:
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic():
    """HBM bytes per launch from committed rocprofv3 counter runs, if they match these sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


class Layer:
    """One layer's inputs on the device and its packed handles (Spense and all-dense)."""

    def __init__(self, sdg, torch, dev, spec, Mmax, rotate, with_dense=True):
        import synth

        self.spec = spec
        W, s, X, D = synth.layer_inputs(spec, Mmax)
        self.host = (W, s, X, D)
        bits = W.view(np.int16) if W.dtype == np.uint16 else W
        Wd = torch.from_numpy(bits).to(dev)
        self.sd = torch.from_numpy(s).to(dev) if s is not None else None
        self.Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
        self.Y = torch.empty((Mmax, spec.N), dtype=torch.bfloat16, device=dev)
        wdt = spec.wdtype

        def copies(info):  # enough rotated copies to stream more than twice the Infinity Cache
            return max(4, -(-2 * MALL_BYTES // info["device_bytes"]) + 1) if rotate else 1

        if spec.form == "output":  # dense rows (the last N_d), 2:4 rows along K
            rows = np.arange(spec.N - spec.N_d, spec.N, dtype=np.int32)

            def pack():
                return sdg.spense_pack_rows(Wd, wdt, scales=self.sd, dense_rows=rows)
        else:
            def pack():
                return sdg.spense_pack(Wd, wdt, scales=self.sd, dense_cols=D)

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h0 = pack()
        self.pack_ms = (time.perf_counter() - t0) * 1e3
        info = sdg.spense_info(h0)
        self.wbytes = info["weight_bytes"]
        self.handles = [h0] + [pack() for _ in range(copies(info) - 1)]
        self.dhandles, self.dbytes = [], None
        if with_dense:
            hd0 = sdg.spense_pack(Wd, wdt, scales=self.sd, dense_fraction=1.0)
            dinfo = sdg.spense_info(hd0)
            self.dbytes = dinfo["weight_bytes"]
            self.dhandles = [hd0] + [sdg.spense_pack(Wd, wdt, scales=self.sd, dense_fraction=1.0)
                                     for _ in range(copies(dinfo) - 1)]
        del Wd

    def flops(self, M):
        """2 x nonzero multiply-adds: the algorithmic flops of the layer."""
        sp = self.spec
        if sp.form == "output":
            return 2.0 * M * sp.K * ((sp.N - sp.N_d) / 2 + sp.N_d)
        K_s = sp.K - sp.K_d
        return 2.0 * M * sp.N * (K_s / 2 + sp.K_d)

    def alg_bytes(self, M):
        sp = self.spec
        scale_b = 4 * sp.N if self.sd is not None else 0
        return self.wbytes + scale_b + 2 * M * sp.K + 2 * M * sp.N  # weights + scales + X + Y(bf16)

    def free(self, sdg):
        for h in self.handles + self.dhandles:
            sdg.spense_free(h)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the layer runs on a single MI355X; use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import sparse_dense_gemm_amd as sdg
    import synth

    variants = SETS[args.workload]
    wls = [synth.WORKLOADS[v] for v in variants]
    if wls[0].extra.get("glu"):
        return run_glu(args, torch, sdg, synth, wls[0])
    Ms = tuple(int(m) for m in args.ms.split(",")) if args.ms else wls[0].Ms
    Mmax = max(Ms)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    single = len(wls) == 1 and len(wls[0].layers) == 1
    hv = variants.index(HEADLINE_VARIANT.get(args.workload, variants[0]))

    t0 = time.time()
    sets = [[Layer(sdg, torch, dev, spec, Mmax, rotate=single, with_dense=not args.no_dense) for spec in wl.layers]
            for wl in wls]
    gen_s = time.time() - t0

    a8 = args.workload in A8_SETS

    def call(h, X, Y):
        if a8:
            sdg.spense_linear_w8a8(h, X, Y, splits=args.splits, stream=stream)
        else:
            sdg.spense_linear_splits(h, X, Y, args.splits, stream=stream)

    def run_set(layers, M, i, dense):
        for L in layers:
            hs = L.dhandles if dense else L.handles
            call(hs[i % len(hs)], L.Xd[:M], L.Y[:M])

    # ---- prime: every packed copy once at every batch size (a handle sizes its
    # split-K and gather workspaces on first use), then the warmup steps ----
    for M in Ms:
        for layers in sets:
            for L in layers:
                for h in L.handles + L.dhandles:
                    call(h, L.Xd[:M], L.Y[:M])
    def warm_step(i):
        for M in Ms:
            for layers in sets:
                run_set(layers, M, i, False)
            if not args.no_dense:
                run_set(sets[hv], M, i, True)

    spin_ms = spin_up(torch, warm_step)
    for i in range(args.warmup):
        warm_step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps (one launch per layer, batch size and set variant) ----
    ev = {}
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    lead_in(lambda: run_set(sets[0], Ms[0], 0, False))
    for vi, layers in enumerate(sets):
        for M in Ms:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                run_set(layers, M, i, False)
            e1.record(stream)
            ev[(vi, M)] = (e0, e1)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    spense_us = {k: a.elapsed_time(b) * 1e3 / args.steps for k, (a, b) in ev.items()}

    # ---- dense baseline (the same layers packed with dense fraction 1.0), same protocol ----
    dev_ = {}
    torch.cuda.synchronize()
    if not args.no_dense:
        lead_in(lambda: run_set(sets[hv], Ms[0], 0, True))
    for M in Ms if not args.no_dense else ():
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            run_set(sets[hv], M, i, True)
        e1.record(stream)
        dev_[M] = (e0, e1)
    torch.cuda.synchronize()
    dense_us = {M: a.elapsed_time(b) * 1e3 / args.steps for M, (a, b) in dev_.items()}

    # ---- per-layer times inside a pass of a layer set (events between the launches) ----
    per_layer = {}
    if not single:
        layers = sets[hv]
        lead_in(lambda: call(layers[0].handles[0], layers[0].Xd[:Ms[0]], layers[0].Y[:Ms[0]]))
        for M in Ms:
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(layers) + 1)] for _ in range(args.steps)]
            for i in range(args.steps):
                for j, L in enumerate(layers):
                    evs[i][j].record(stream)
                    call(L.handles[0], L.Xd[:M], L.Y[:M])
                evs[i][-1].record(stream)
            torch.cuda.synchronize()
            per_layer[str(M)] = {L.spec.name: round(sum(e[j].elapsed_time(e[j + 1]) for e in evs) * 1e3 / args.steps, 3)
                                 for j, L in enumerate(layers)}

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = sets[hv]
    wbytes = sum(L.wbytes for L in head)
    dbytes = None if args.no_dense else sum(L.dbytes for L in head)
    per_m = {}
    for M in Ms:
        t = spense_us[(hv, M)]
        du = dense_us.get(M)
        per_m[str(M)] = {
            "spense_us": round(t, 3),
            "dense_us": None if du is None else round(du, 3),
            "speedup_vs_dense": None if du is None else round(du / t, 4),
            "weight_GBs": round(wbytes / t / 1e3, 1),
            "weight_frac_of_peak": round(wbytes / t / 1e3 / HBM_PEAK_GBS, 4),
            "dense_weight_GBs": None if du is None else round(dbytes / du / 1e3, 1),
            "alg_TFLOPs": round(sum(L.flops(M) for L in head) / t / 1e6, 1),
        }
    total_us = sum(spense_us[(hv, M)] for M in Ms)
    value = len(Ms) * wbytes / total_us / 1e3  # GB/s on compressed + dense weight bytes
    big = [M for M in Ms if M >= 1024]
    if big:
        # prefill batches dominate the step and are bound by the matrix units
        t_big = sum(spense_us[(hv, M)] for M in big)
        ach = sum(sum(L.flops(M) for L in head) for M in big) / t_big / 1e6
        peak = FP8_PEAK_TFLOPS if a8 else MFMA_PEAK_TFLOPS
        roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "traffic": None, "batch_sizes": big}
    else:
        ach = sum(sum(L.alg_bytes(M) for L in head) for M in Ms) / total_us / 1e3
        traffic = load_traffic() if args.workload == "gateup_fp8" and not args.ms else None
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic}

    variants_out = {}
    if len(sets) > 1:
        for vi, v in enumerate(variants):
            variants_out[v] = {"dense_fraction": wls[vi].extra.get("fraction"),
                               "weight_bytes": sum(L.wbytes for L in sets[vi]),
                               **{f"M{M}_us": round(spense_us[(vi, M)], 3) for M in Ms},
                               **{f"M{M}_speedup_vs_dense": (None if M not in dense_us else
                                                             round(dense_us[M] / spense_us[(vi, M)], 4)) for M in Ms}}

    pack_ms = round(sum(L.pack_ms for L in head), 3)
    cpu = None if args.no_cpu_baseline else cpu_baseline(head, Ms, single, a8)
    for layers in sets:
        for L in layers:
            L.free(sdg)

    if args.workload == "gateup_fp8":
        wdesc = ("FFN gate/up W[25600,5120] e4m3 + per-channel scales, dense tail 25% (1280 cols), X bf16, "
                 "M in {" + ",".join(map(str, Ms)) + "}")
    else:
        wdesc = wls[hv].title + (f" (batch sizes {list(Ms)})" if args.ms else "")
        if a8:
            wdesc += ", W8A8: per-token e4m3 activations"
    cfg = {"workload": wdesc, "key": args.workload, "Ms": list(Ms), "splits": args.splits or "auto"}
    if single:
        cfg.update({"N": head[0].spec.N, "K": head[0].spec.K, "K_d": head[0].spec.K_d,
                    "weight_copies": len(head[0].handles)})
    else:
        cfg["layers"] = [{"name": L.spec.name, "N": L.spec.N, "K": L.spec.K, "K_d": L.spec.K_d} for L in head]
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spin_up_ms": round(spin_ms, 1),
        "ms_per_step": round(wall_s * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("e4m3" if head[0].spec.wdtype == synth.DT_FP8 else "bf16")
        + (" weights x per-token e4m3 activations" if a8 else " weights x bf16 activations") + ", fp32 accumulate",
        "data": "synthetic",
        "config": cfg,
        "per_m": per_m,
        "speedup_vs_dense": None if args.no_dense else round(sum(dense_us.values()) / total_us, 4),
        "spense_weight_bytes": wbytes,
        "dense_weight_bytes": dbytes,
        "pack_ms_wall": pack_ms,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "input_gen_s": round(gen_s, 2),
    }
    if per_layer:
        out["per_layer_us"] = per_layer
    if variants_out:
        out["variants"] = variants_out
    print(json.dumps(out))


def run_glu(args, torch, sdg, synth, wl):
    """The GLU block workload: spense_glu per batch size, all-dense block as the baseline."""
    gu, dn = wl.layers
    H, I = dn.N, dn.K
    Ms = tuple(int(m) for m in args.ms.split(",")) if args.ms else wl.Ms
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t0 = time.time()
    Wgu, sgu, X, _ = synth.layer_inputs(gu, max(Ms))
    Wd, sd, _, D = synth.layer_inputs(dn, max(Ms))
    gen_s = time.time() - t0
    Wgu_d, Wd_d = torch.from_numpy(Wgu).to(dev), torch.from_numpy(Wd).to(dev)
    sgu_d, sd_d = torch.from_numpy(sgu).to(dev), torch.from_numpy(sd).to(dev)
    Xd = torch.from_numpy(X.view(np.int16)).to(dev).view(torch.bfloat16)
    A = torch.empty((max(Ms), I), dtype=torch.bfloat16, device=dev)
    Y = torch.empty((max(Ms), H), dtype=torch.bfloat16, device=dev)

    def pack(**kw):
        return sdg.spense_pack_glu(Wgu_d, Wd_d, gu.wdtype, H=H, I=I, s_gu=sgu_d, s_down=sd_d, **kw)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hs = [pack(dense_idx=D)]
    pack_ms = (time.perf_counter() - t0) * 1e3
    info = sdg.spense_info(hs[0])
    n_copies = max(2, -(-2 * MALL_BYTES // info["device_bytes"]) + 1)
    hs += [pack(dense_idx=D) for _ in range(n_copies - 1)]
    hd = [pack(dense_fraction=1.0) for _ in range(n_copies)]
    wbytes, dbytes = info["weight_bytes"], sdg.spense_info(hd[0])["weight_bytes"]

    def step(handles, M, i):
        sdg.spense_glu(handles[i % len(handles)], Xd[:M], A[:M], Y[:M], stream=stream)

    for M in Ms:
        for h in hs + hd:
            step([h], M, 0)
    def warm_step(i):
        for M in Ms:
            step(hs, M, i)
            step(hd, M, i)

    spin_ms = spin_up(torch, warm_step)
    for i in range(args.warmup):
        warm_step(i)
    torch.cuda.synchronize()
    ev = {}
    t_wall = time.perf_counter()
    lead_in(lambda: step(hs, Ms[0], 0))
    for M in Ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(hs, M, i)
        e1.record(stream)
        ev[M] = (e0, e1)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    us = {M: a.elapsed_time(b) * 1e3 / args.steps for M, (a, b) in ev.items()}
    dev_ = {}
    lead_in(lambda: step(hd, Ms[0], 0))
    for M in Ms:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(hd, M, i)
        e1.record(stream)
        dev_[M] = (e0, e1)
    torch.cuda.synchronize()
    dus = {M: a.elapsed_time(b) * 1e3 / args.steps for M, (a, b) in dev_.items()}

    # SpenseGPT+ selection of the dense set (offline, before packing): scores
    # from T calibration rows, their intermediate activations taken from the
    # dense block itself, then the top-I_d selection
    T = 512
    Xc = torch.from_numpy(synth.make_x(T, H, synth.DT_BF16, np.random.default_rng(7)).view(np.int16)).to(dev).view(
        torch.bfloat16)
    Ac = torch.empty((T, I), dtype=torch.bfloat16, device=dev)
    Yc = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    sdg.spense_glu(hd[0], Xc, Ac, Yc, stream=stream)
    score = torch.empty(I, dtype=torch.float32, device=dev)
    reps, t_score, t_sel = 5, 0.0, 0.0
    for r in range(reps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        sdg.spense_score_glu(Wgu_d, Wd_d, gu.wdtype, H=H, I=I, X_cal=Xc, A_cal=Ac, score=score, s_gu=sgu_d,
                             s_down=sd_d, stream=stream)
        t1 = time.perf_counter()
        sel = sdg.spense_select_dense(score, int(len(D)), stream=stream)
        t2 = time.perf_counter()
        if r:  # the first call is a warmup
            t_score += t1 - t0
            t_sel += t2 - t1
    score_bytes = Wgu.nbytes + Wd.nbytes + 2 * T * (H + I) * 2
    scoring = {"T": T, "score_ms": round(t_score / reps * 1e3, 3), "select_ms": round(t_sel / reps * 1e3, 3),
               "score_GBs": round(score_bytes / (t_score / reps) / 1e9, 1), "k": int(len(sel)),
               "note": "host wall time per call (each call allocates scratch and synchronises)"}
    del Wgu_d, Wd_d
    for h in hs + hd:
        sdg.spense_free(h)

    def alg(M):  # weights + scales + X + A written and read + Y (bf16)
        return wbytes + 4 * (2 * I + H) + 2 * M * H + 2 * 2 * M * I + 2 * M * H

    per_m = {str(M): {"spense_us": round(us[M], 3), "dense_us": round(dus[M], 3),
                      "speedup_vs_dense": round(dus[M] / us[M], 4),
                      "weight_GBs": round(wbytes / us[M] / 1e3, 1),
                      "weight_frac_of_peak": round(wbytes / us[M] / 1e3 / HBM_PEAK_GBS, 4),
                      "dense_weight_GBs": round(dbytes / dus[M] / 1e3, 1)} for M in Ms}
    total = sum(us.values())
    ach = sum(alg(M) for M in Ms) / total / 1e3
    cpu = None
    if not args.no_cpu_baseline:
        import oracle  # the CPU baseline leg only

        # whole passes over a restricted block until about 10 s of CPU work
        rows, M0 = 256, min(Ms)
        passes = 0
        t0 = time.perf_counter()
        while True:
            oracle.glu_block_ref(X[:M0], oracle.DT_BF16, Wgu[:rows], Wgu[I:I + rows], Wd[:, :rows], gu.wdtype,
                                 np.arange(rows - rows // 4, rows), sgu[:rows], sgu[I:I + rows], sd)
            passes += 1
            dt = time.perf_counter() - t0
            if dt >= 10.0 or passes >= 1000:
                break
        nbytes = wbytes * rows / I * passes
        cpu = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": oracle_threads(), "kind": "oracle",
               **host_cpu(),
               "sample": f"block restricted to the first {rows} intermediate indices (last quarter dense), "
                         f"M={M0}, {passes} passes ({dt:.1f} s)"}
    out = {
        "metric": METRIC, "value": round(len(Ms) * wbytes / total / 1e3, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "spin_up_ms": round(spin_ms, 1),
        "ms_per_step": round(wall_s * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "e4m3 weights x bf16 activations, fp32 accumulate", "data": "synthetic",
        "config": {"workload": wl.title, "key": wl.key, "Ms": list(Ms), "H": H, "I": I, "I_d": int(len(D)),
                   "weight_copies": n_copies},
        "per_m": per_m, "speedup_vs_dense": round(sum(dus.values()) / total, 4),
        "spense_weight_bytes": wbytes, "dense_weight_bytes": dbytes, "pack_ms_wall": round(pack_ms, 3),
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": cpu, "input_gen_s": round(gen_s, 2), "spensegpt_plus_scoring": scoring,
    }
    print(json.dumps(out))


def host_cpu() -> dict:
    """The host CPU the baseline ran on: model name and logical CPUs visible to this process."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        nproc = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": nproc}


def oracle_threads() -> int:
    """Threads the oracle's BLAS pool runs (what the CPU baseline actually used)."""
    try:
        from threadpoolctl import threadpool_info

        return int(max([p.get("num_threads", 1) for p in threadpool_info()] + [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(layers, Ms, single, a8=False):
    """The oracle, as it stands, on the same layer(s): one packed form, then the
    float64 layer output.  A single layer: whole passes over the batch sizes
    until about 10 s of CPU work.  A layer set: the first 256 output rows of
    each layer at the smallest batch size.  Throughput on the weight bytes covered."""
    import oracle

    cores = oracle_threads()
    if single:
        L = layers[0]
        W, s, X, D = L.host
        if L.spec.form == "output":
            rho, N_s, _ = oracle.resolve_dense_rows(L.spec.N, L.spec.K, dense_fraction=L.spec.N_d / L.spec.N)
            p = oracle.pack_rows(W, L.spec.wdtype, rho, N_s)
            run = oracle.linear_rows_ref
        else:
            pi, K_s, _ = oracle.resolve_dense_set(L.spec.K, dense_cols=D)
            p = oracle.pack(W, L.spec.wdtype, pi, K_s)
            run = oracle.linear_ref
        # repeat whole passes over the batch sizes until about 10 s of CPU work
        passes = 0
        t0 = time.perf_counter()
        while passes < 20 and (passes == 0 or time.perf_counter() - t0 < 10.0):
            for M in Ms:
                run(X[:M], oracle.DT_BF16, p, s)
            passes += 1
        dt = time.perf_counter() - t0
        return {"value": round(passes * len(Ms) * L.wbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores),
                "kind": "oracle", **host_cpu(),
                "sample": f"full layer, oracle linear_ref for M in {list(Ms)}, {passes} passes ({dt:.1f} s); pack excluded"}
    rows, M = 256, min(Ms)
    nbytes, dt = 0.0, 0.0
    for L in layers:
        W, s, X, D = L.host
        pi, K_s, _ = oracle.resolve_dense_set(L.spec.K, dense_cols=D)
        p = oracle.pack(W[:rows], L.spec.wdtype, pi, K_s)
        t0 = time.perf_counter()
        if a8:
            q, sx = oracle.quantize_tokens_ref(X[:M], oracle.DT_BF16)
            oracle.linear_w8a8_ref(q, sx, p, s[:rows])
        else:
            oracle.linear_ref(X[:M], oracle.DT_BF16, p, None if s is None else s[:rows])
        dt += time.perf_counter() - t0
        nbytes += L.wbytes * rows / L.spec.N
    what = "quantize_tokens_ref + linear_w8a8_ref" if a8 else "linear_ref"
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(cores), "kind": "oracle", **host_cpu(),
            "sample": f"oracle {what} on the first {rows} output rows of each layer, M={M} ({dt:.1f} s); "
                      "pack excluded"}


if __name__ == "__main__":
    main()
