#!/usr/bin/env python3
"""Benchmark of the ternary BitLinear forward path on one MI355X.

A step is one forward pass of every BitLinear of the chosen workload over one
batch of synthetic input (RMSNorm -> int8 quantisation -> I2_S ternary x int8
contraction -> rescale), all in the HIP library.  Default workload: the seven
BitLinears of one decoder layer at decode (M = 1; q/o 2560x2560, k/v
2560->640, gate/up 2560->6912, down 6912->2560).

value = algorithmic bytes of a step / wall time of a step (GB/s), with inputs
resident in HBM.  Algorithmic bytes per BitLinear = N*K/4 (packed W) +
4*M*K (x) + 4*K (gamma) + 4*M*N (y).  The packed weights are rotated over
enough copies (>= 768 MB in total) that every step streams them from HBM,
not from the 256 MB last-level cache.

Prints one JSON line (see the "metric" of the workload).  Options:
  --gpus N (only 1 is supported), --steps K, --warmup W,
  --workload decode|prefill|ffn70b-1|ffn70b-16|sweep-M,
  --no-cpu-baseline, --no-secondary, --pack-only.
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

METRIC = "BitLinear GB/s (M=1 GEMV) and int8 TOPS (M=512 GEMM), % of roofline"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0    # MI355X dense int8 MFMA, published (5.0 POP/s)
ROTATE_BYTES = 768 << 20


def workload_by_name(name: str):
    from ternary_bit_linear_amd import workloads as wl
    if name == "decode":
        return wl.DECODE_LAYER
    if name == "prefill":
        return wl.PREFILL_LAYER
    if name.startswith("ffn70b-"):
        return wl.ffn70b(int(name.split("-")[1]))
    if name.startswith("sweep-"):
        return wl.sweep(int(name.split("-")[1]))
    if name == "tiny":
        return wl.TINY
    raise SystemExit(f"unknown workload {name}")


class Prepared:
    """Device-resident inputs of a workload, with rotated weight copies."""

    def __init__(self, torch, api, work):
        self.work = work
        self.lin = []
        packed_total = 0
        for i, L in enumerate(work.linears):
            x, w, _, g = work.inputs(i)
            X = torch.from_numpy(x).cuda()
            G = torch.from_numpy(g).cuda()
            P, s = api.pack_i2s(torch.from_numpy(w).cuda())
            Y = torch.empty((L.M, L.N), dtype=torch.float32, device="cuda")
            WS = api.new_workspace(L.M, L.K)
            self.lin.append({"L": L, "x": X, "g": G, "P": [P], "s": s, "y": Y, "ws": WS})
            packed_total += P.numel()
        self.copies = max(2, -(-ROTATE_BYTES // packed_total))
        for d in self.lin:
            d["P"] += [d["P"][0].clone() for _ in range(self.copies - 1)]
        torch.cuda.synchronize()

    def step(self, api, r: int):
        """One step: every BitLinear of the workload, as one batched call
        (decode-sized ones share a launch; bit-identical to single calls)."""
        api.forward_batch([(d["x"], d["P"][r % self.copies], d["s"], d["g"], self.work.eps,
                            d["y"], d["ws"]) for d in self.lin])


def capture(torch, fn):
    """Capture fn() (which enqueues on the current stream) into a HIP graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # untimed eager pass (allocator / module warm-up before capture)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_steps(torch, api, prep, steps, warmup):
    """ms per step over exactly `steps` steps, replayed from one HIP graph
    (the host does not pace the GPU), after `warmup` untimed steps."""
    gw = capture(torch, lambda: [prep.step(api, r) for r in range(max(1, warmup))])
    gt = capture(torch, lambda: [prep.step(api, warmup + r) for r in range(steps)])
    gw.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gt.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps  # ms per step


def time_launches(torch, api, prep, reps=None):
    """Mean duration of each BitLinear's forward launch: a HIP graph of
    `reps` back-to-back launches of that one shape (rotating weight copies),
    timed with events on the launch stream."""
    out = {}
    reps = reps or prep.copies
    for d in prep.lin:
        L = d["L"]

        def run(d=d, L=L):
            for r in range(reps):
                api.forward(d["x"], d["P"][r % prep.copies], d["s"], d["g"], prep.work.eps, L.N,
                            out=d["y"], workspace=d["ws"])
        g = capture(torch, run)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out[L.name] = (L, e0.elapsed_time(e1) * 1e-3 / reps)  # s per launch
        del g
    return out


def linear_bytes(L):
    return L.N * L.K // 4 + 4 * L.M * L.K + 4 * L.K + 4 * L.M * L.N


# Sources of the batched decode kernel (the traffic record is valid for
# these only).
KERNEL_SOURCES = [os.path.join(ROOT, "ternary_bit_linear_amd", "csrc", f)
                  for f in ("common.hpp", "gemv_shot.hip")]


def sources_sha256() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_from_profiles(name: str):
    """HBM bytes per launch from the committed PMC summary
    profiles/traffic_<name>.json, if it was taken on the current kernel
    sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("sources_sha256") != sources_sha256():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(work, budget_s=12.0):
    """The oracle, untuned, on the host cores: whole steps of the workload
    (inputs prepared outside the timed region), repeated until the budget is
    spent; scaled to GB/s of algorithmic bytes.  For workloads whose step is
    too large, a subset of the weight rows is used and scaled."""
    from oracle import oracle as orc
    orc.lib()
    items = []
    total_bytes = 0
    row_frac = 1.0
    macs = sum(L.M * L.N * L.K for L in work.linears)
    if macs > 2e9:
        row_frac = 2e9 / macs
    for i, L in enumerate(work.linears):
        x, w, _, g = work.inputs(i)
        n_keep = max(1, int(L.N * row_frac))
        p, s = orc.pack_i2s(w[:n_keep])
        items.append((x, p, s, g, n_keep))
        total_bytes += linear_bytes(L)
    t0 = time.perf_counter()
    n = 0
    while True:
        for x, p, s, g, n_keep in items:
            orc.forward(x, p, s, g, work.eps, n_keep)
        n += 1
        el = time.perf_counter() - t0
        if el > budget_s or n >= 100000:
            break
    per_step = el / n / row_frac
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    sample = (f"{n} oracle forward step(s) of the whole workload" if row_frac == 1.0 else
              f"{n} oracle step(s) over {row_frac:.4f} of the weight rows, scaled")
    return {"value": round(total_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "sample": sample, "seconds": round(el, 2)}


def secondary_prefill(torch, api, steps, warmup):
    """int8 TOPS of the prefill layer (M = 512): 2*M*N*K over the forward time."""
    from ternary_bit_linear_amd import workloads as wl
    prep = Prepared(torch, api, wl.PREFILL_LAYER)
    ms = time_steps(torch, api, prep, steps, warmup)
    ops = wl.PREFILL_LAYER.int_ops()
    tops = ops / (ms * 1e-3) / 1e12
    by = time_launches(torch, api, prep)
    per = {}
    for name, (L, t) in by.items():
        per[name] = {"M": L.M, "K": L.K, "N": L.N, "us": round(t * 1e6, 2),
                     "TOPS": round(2 * L.M * L.N * L.K / t / 1e12, 1)}
    del prep
    torch.cuda.empty_cache()
    # The square M = 512 point (K = N = 8192) of the sweep, same measurement.
    sq = wl.sweep(512)
    prep = Prepared(torch, api, sq)
    ms_sq = time_steps(torch, api, prep, steps, warmup)
    tops_sq = sq.int_ops() / (ms_sq * 1e-3) / 1e12
    del prep
    torch.cuda.empty_cache()
    return {"workload": wl.PREFILL_LAYER.name, "metric": "int8 TOPS (M=512 GEMM)",
            "value": round(tops, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4), "per_linear": per,
            "square_m512": {"workload": sq.name, "value": round(tops_sq, 2), "unit": "TOPS",
                            "ms_per_step": round(ms_sq, 4),
                            "frac_of_int8_peak": round(tops_sq / INT8_PEAK_TOPS, 4)}}


def secondary_pack(torch, api, reps=5):
    """I2_S packing of the packing workload (fp32 ternary x 0.02, N = 8192 x
    K = 28672; seeded on the device): GB/s of algorithmic bytes (4NK read +
    NK/4 + 32 written) over the whole synchronous bitlinear_pack_i2s call."""
    from ternary_bit_linear_amd import workloads as wl
    N, K = wl.PACK_SHAPE
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5000)
    t = torch.randint(-1, 2, (N, K), generator=gen, device="cuda", dtype=torch.int8)
    w = t.to(torch.float32).mul_(0.02)
    del t
    api.pack_i2s(w)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        api.pack_i2s(w)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / reps
    nbytes = 4 * N * K + N * K // 4 + 32
    del w
    torch.cuda.empty_cache()
    return {"workload": f"I2_S pack, N={N} x K={K}", "metric": "pack GB/s (whole call)",
            "value": round(nbytes / sec / 1e9, 1), "unit": "GB/s", "us_per_call": round(sec * 1e6, 1),
            "frac_of_hbm_peak": round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--pack-only", action="store_true",
                    help="time only the I2_S packer over --steps calls and print its line")
    ap.add_argument("--pmc-app", action="store_true",
                    help="no timing: run --steps steps of the workload and a 256 MiB device "
                         "copy (the calibration kernel for HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU N-split is described in DESIGN.md, not built)", file=sys.stderr)
        sys.exit(2)

    import torch
    from ternary_bit_linear_amd import api
    api.lib()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.pack_only:
        print(json.dumps(secondary_pack(torch, api, reps=max(1, args.steps))), flush=True)
        return
    work = workload_by_name(args.workload)
    prep = Prepared(torch, api, work)
    if args.pmc_app:
        for r in range(args.steps):
            prep.step(api, r)
        torch.cuda.synchronize()
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")  # 256 MiB
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_app": work.name, "steps": args.steps, "copy_bytes": a.numel() * 4}))
        return
    ms = time_steps(torch, api, prep, args.steps, args.warmup)
    step_bytes = sum(linear_bytes(L) for L in work.linears)
    gbs = step_bytes / (ms * 1e-3) / 1e9
    by = time_launches(torch, api, prep)
    M = work.linears[0].M
    decode = M <= 16
    # Decode BitLinears with M == 1 and K <= 8192 take the fused kernel and a
    # step of them is one launch (up to 8 per launch).
    fused_all = all(L.M == 1 and L.K <= 8192 for L in work.linears)
    launches = -(-len(work.linears) // 8)
    if decode and fused_all:
        avg_s = ms * 1e-3 / launches
        ach = step_bytes / launches / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles(args.workload),
                "kernel": "gemv_shot_kernel (one-shot decode: RMSNorm + int8 quant + "
                          f"I2_S x int8 MFMA, {len(work.linears)} BitLinears per launch)",
                "launches_per_step": launches,
                "avg_launch_us": round(avg_s * 1e6, 3),
                "bytes_per_launch": step_bytes // launches}
    else:
        dom_name, (dom_L, dom_s) = max(by.items(), key=lambda kv: linear_bytes(kv[1][0]))
        if decode:
            ach = linear_bytes(dom_L) / dom_s / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": traffic_from_profiles(args.workload),
                    "kernel": "act_quant + gemv (decode route)",
                    "launch": f"{dom_name} M={dom_L.M} K={dom_L.K} N={dom_L.N}",
                    "avg_launch_us": round(dom_s * 1e6, 3),
                    "bytes_per_launch": linear_bytes(dom_L)}
        else:
            # A step of prefill-sized BitLinears is one batched quantisation
            # launch plus one grouped tile-kernel launch per 8 BitLinears:
            # the rate is int ops over the step, quantisation included.
            groups = -(-len(work.linears) // 8)
            ach = work.int_ops() / (ms * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": INT8_PEAK_TOPS,
                    "unit": "TOPS", "frac": round(ach / INT8_PEAK_TOPS, 4),
                    "traffic": None,
                    "kernel": "act_quant_batch_kernel + gemm_group_kernel (I2_S x int8 MFMA), "
                              f"{len(work.linears)} BitLinears per launch pair",
                    "launches_per_step": 2 * groups,
                    "avg_step_us": round(ms * 1e3, 3),
                    "int_ops_per_step": work.int_ops()}
    per_linear = {n: {"M": L.M, "K": L.K, "N": L.N, "us": round(t * 1e6, 3),
                      "GBs": round(linear_bytes(L) / t / 1e9, 1)}
                  for n, (L, t) in by.items()}

    out = {
        "metric": METRIC,
        "value": round(gbs, 2) if decode else round(work.int_ops() / (ms * 1e-3) / 1e12, 2),
        "unit": "GB/s" if decode else "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": work.name, "M": M,
                   "linears": [[L.name, L.K, L.N] for L in work.linears],
                   "algorithmic_bytes_per_step": step_bytes,
                   "weight_copies_rotated": prep.copies},
        "roofline": roof,
        "per_linear_single_launch": per_linear,
    }
    del prep
    torch.cuda.empty_cache()
    if not args.no_secondary and args.workload == "decode":
        out["secondary"] = secondary_prefill(torch, api, max(20, args.steps // 4), 5)
        torch.cuda.empty_cache()
        out["secondary"]["pack"] = secondary_pack(torch, api)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(work)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
