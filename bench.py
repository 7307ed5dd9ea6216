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

Prints one JSON line (see the "metric" of the workload).  Beside the main
value: the prefill layer (M = 512) and the square K = N = 8192 sweep
(M = 1 .. 2048) in int8 TOPS / GB/s, the 70B FFN BitLinears at M = 1 and 16,
the single 256 x 256 BitLinear, the packer, the FFN block, half-precision
I/O, a dequantised-weights library comparison and the layer without
RMSNorm, each with its roofline fraction; measured ceilings (one-launch HBM
read at the decode sizes, back-to-back int8 MFMA); and the oracle on the
host cores (all threads and one thread).  Options:
  --gpus N (only 1 is supported), --steps K, --warmup W,
  --workload decode|prefill|decode-mM|ffn70b-1|ffn70b-16|sweep-M|tiny,
  --no-cpu-baseline, --no-secondary, --pack-only, --ffn-only, --io-only,
  --dense-only, --pmc-app.
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
    if name.startswith("decode-m"):
        return wl.decode_layer(int(name.split("-m")[1]))
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


# Untimed GPU work before every timed region.  The MI355X runs short
# launches faster once it has been under load for some milliseconds: the
# decode layer's 200 timed steps took 6.65-6.67 us each right after 20
# warm-up steps (0.13 ms of work), 6.39-6.43 us after 13-100 ms of warm-up
# steps (one long graph, or short ones with a synchronisation every ~7 ms),
# and were back at 6.66 us after a 50 ms pause; K = N = 8192 at M = 512
# 44.5 against 42.1 us, the prefill layer 62.2 against 57.8 us.  Hundreds of
# short graph replays issued without a synchronisation made the timed steps
# slower and erratic instead (6.6-7.4 us), so the warm-up goes in chunks of
# at least CLOCK_CHUNK_S of work, each followed by a synchronisation.
CLOCK_WARM_S = 0.025
CLOCK_CHUNK_S = 0.005


def warm_clock(torch, g):
    """Replays graph g (untimed) in chunks of at least CLOCK_CHUNK_S seconds
    of GPU work, synchronising after each, until about CLOCK_WARM_S seconds
    have run; returns the seconds of GPU work run."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    one = max(e0.elapsed_time(e1) * 1e-3, 1e-6)
    per_chunk = max(1, int(CLOCK_CHUNK_S / one + 0.999))
    chunks = max(0, int(CLOCK_WARM_S / (per_chunk * one) + 0.5))
    for _ in range(chunks):
        for _ in range(per_chunk):
            g.replay()
        torch.cuda.synchronize()
    return one * (1 + chunks * per_chunk)


def replay_timed(torch, gw, gt, steps):
    """Seconds per step of graph gt (`steps` steps), timed with HIP events on
    the current stream, after the warm-up graph gw (the `warmup` untimed
    steps) and the clock warm-up over replays of gw."""
    gw.replay()
    warm_clock(torch, gw)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    gt.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / steps


def time_steps(torch, api, prep, steps, warmup):
    """ms per step over exactly `steps` steps, replayed from one HIP graph
    (the host does not pace the GPU), after `warmup` untimed steps and the
    clock warm-up."""
    gw = capture(torch, lambda: [prep.step(api, r) for r in range(max(1, warmup))])
    gt = capture(torch, lambda: [prep.step(api, warmup + r) for r in range(steps)])
    return replay_timed(torch, gw, gt, steps) * 1e3  # ms per step


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
        out[L.name] = (L, replay_timed(torch, g, g, reps))  # s per launch
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def set_oracle_threads(n):
    """OpenMP threads of the oracle (its library is built with -fopenmp;
    results do not depend on the count)."""
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except OSError:
        return False


def cpu_baseline(work, budget_s=12.0, threads=None):
    """The oracle, untuned, on the host cores: whole steps of the workload
    (inputs prepared outside the timed region), repeated until the budget is
    spent; scaled to GB/s of algorithmic bytes.  For workloads whose step is
    too large, a subset of the weight rows is used and scaled.  threads:
    OpenMP threads (None: all of them)."""
    from oracle import oracle as orc
    orc.lib()
    all_cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    used = all_cores if threads is None else threads
    set_oracle_threads(used)
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
    set_oracle_threads(all_cores)
    sample = (f"{n} oracle forward step(s) of the whole workload" if row_frac == 1.0 else
              f"{n} oracle step(s) over {row_frac:.4f} of the weight rows, scaled")
    return {"value": round(total_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": used,
            "kind": "oracle", "sample": sample, "seconds": round(el, 2),
            "ms_per_step": round(per_step * 1e3, 3), "cpu_model": cpu_model()}


def time_fn(torch, fn, steps, warmup):
    """Seconds per call of fn(r) (which enqueues on the current stream):
    HIP events around a graph replay of `steps` calls, after `warmup`
    untimed ones."""
    gw = capture(torch, lambda: [fn(r) for r in range(max(1, warmup))])
    gt = capture(torch, lambda: [fn(warmup + r) for r in range(steps)])
    t = replay_timed(torch, gw, gt, steps)
    del gw, gt
    return t


def roofline_of(L_list, sec, kernel):
    """Roofline block of a step of BitLinears taking `sec` seconds: the bound
    is min(int8 peak, intensity x HBM peak) over the step's algorithmic bytes
    and int ops; `achieved` is in that bound's unit."""
    nbytes = sum(linear_bytes(L) for L in L_list)
    ops = sum(2 * L.M * L.N * L.K for L in L_list)
    if ops / nbytes * HBM_PEAK_GBS * 1e9 < INT8_PEAK_TOPS * 1e12:
        ach = nbytes / sec / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "avg_step_us": round(sec * 1e6, 2),
                "kernel": kernel}
    ach = ops / sec / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
            "frac": round(ach / INT8_PEAK_TOPS, 4), "avg_step_us": round(sec * 1e6, 2),
            "kernel": kernel}


class DeviceLinears:
    """BitLinears whose ternary weights are drawn on the device (seeded,
    with the workload's P(0) and scale; x and gamma from the workload's host
    recipe), packed once and rotated over >= 768 MB of copies.  For timing
    legs of large shapes, where drawing the weights on the host would
    dominate the run."""

    def __init__(self, torch, api, linears, seed, eps=1e-6, packs=None):
        from ternary_bit_linear_amd import workloads as wl
        self.eps = eps
        self.lin = []
        total = 0
        gen = torch.Generator(device="cuda")
        for i, L in enumerate(linears):
            if packs is not None:
                P, sc = packs[i]
            else:
                gen.manual_seed(seed + 3 * i + 1)
                u = torch.rand((L.N, L.K), generator=gen, device="cuda")
                w = torch.where(u < L.p0, 0.0, torch.where(u < L.p0 + (1 - L.p0) / 2, 1.0, -1.0))
                del u
                w.mul_(L.scale)
                P, sc = api.pack_i2s(w)
                del w
            x = torch.from_numpy(wl.activations(seed + 3 * i, L.M, L.K, L.outlier_frac)).cuda()
            g = torch.from_numpy(wl.gamma(seed + 3 * i + 2, L.K, L.gamma)).cuda()
            y = torch.empty((L.M, L.N), dtype=torch.float32, device="cuda")
            self.lin.append({"L": L, "x": x, "g": g, "P": [P], "s": sc, "y": y,
                             "ws": api.new_workspace(L.M, L.K)})
            total += P.numel()
        self.copies = max(2, -(-ROTATE_BYTES // total))
        for d in self.lin:
            d["P"] += [d["P"][0].clone() for _ in range(self.copies - 1)]
        torch.cuda.synchronize()

    def packs(self):
        return [(d["P"][0], d["s"]) for d in self.lin]

    def step(self, api, r):
        api.forward_batch([(d["x"], d["P"][r % self.copies], d["s"], d["g"], self.eps, d["y"],
                            d["ws"]) for d in self.lin])

    def single(self, api, d, r):
        api.forward(d["x"], d["P"][r % self.copies], d["s"], d["g"], self.eps, d["L"].N,
                    out=d["y"], workspace=d["ws"])


def secondary_prefill(torch, api, steps, warmup):
    """int8 TOPS of the prefill layer (M = 512): 2*M*N*K over the forward
    time (one batched quantisation launch and one grouped contraction
    launch per step), and each BitLinear alone."""
    from ternary_bit_linear_amd import workloads as wl
    prep = Prepared(torch, api, wl.PREFILL_LAYER)
    ms = time_steps(torch, api, prep, steps, warmup)
    ops = wl.PREFILL_LAYER.int_ops()
    tops = ops / (ms * 1e-3) / 1e12
    by = time_launches(torch, api, prep)
    per = {}
    for name, (L, t) in by.items():
        per[name] = {"M": L.M, "K": L.K, "N": L.N, "us": round(t * 1e6, 2),
                     "TOPS": round(2 * L.M * L.N * L.K / t / 1e12, 1),
                     "roofline": roofline_of([L], t, "act_quant + contraction")}
    del prep
    torch.cuda.empty_cache()
    roof = roofline_of(list(wl.PREFILL_LAYER.linears), ms * 1e-3,
                       "act_quant_batch_kernel + grouped contraction (7 BitLinears per launch "
                       "pair)")
    roof_mfma = {"bound": "mfma", "achieved": round(tops, 2), "peak": INT8_PEAK_TOPS,
                 "unit": "TOPS", "frac": round(tops / INT8_PEAK_TOPS, 4)}
    return {"workload": wl.PREFILL_LAYER.name, "metric": "int8 TOPS (M=512 GEMM)",
            "value": round(tops, 2), "unit": "TOPS", "ms_per_step": round(ms, 4),
            "frac_of_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
            "roofline": roof, "roofline_vs_int8_peak": roof_mfma, "per_linear": per}


def secondary_sweep(torch, api, steps, warmup):
    """The square BitLinear K = N = 8192 at M = 1 .. 2048 tokens, one
    forward per step (quantisation and contraction launches included), with
    the roofline of each point (HBM-bound up to M = 64, MFMA-bound from
    M = 256)."""
    from ternary_bit_linear_amd import workloads as wl
    res = {}
    packs = None
    for M in (1, 4, 16, 64, 256, 512, 2048):
        work = wl.sweep(M)
        dl = DeviceLinears(torch, api, work.linears, 5000 + M, work.eps, packs)
        packs = dl.packs()
        sec = time_fn(torch, lambda r: dl.step(api, r), steps, warmup)
        L = work.linears[0]
        res[f"M{M}"] = {"M": M, "us": round(sec * 1e6, 2),
                        "GBs": round(linear_bytes(L) / sec / 1e9, 1),
                        "TOPS": round(2 * M * L.N * L.K / sec / 1e12, 1),
                        "roofline": roofline_of([L], sec, "act_quant + contraction, one "
                                                "forward")}
        del dl
        torch.cuda.empty_cache()
    return {"workload": "square BitLinear K=N=8192, M = 1..2048 (weights drawn on the device)",
            **res}


def secondary_ffn70b(torch, api, steps, warmup):
    """The 70B-shaped FFN BitLinears (gate / up 8192 -> 28672, down
    28672 -> 8192) one forward at a time, at M = 1 and M = 16: GB/s of
    algorithmic bytes and the HBM roofline fraction of each."""
    from ternary_bit_linear_amd import workloads as wl
    res = {}
    packs = None
    for M in (1, 16):
        work = wl.ffn70b(M)
        dl = DeviceLinears(torch, api, work.linears, 4000, work.eps, packs)
        packs = dl.packs()
        per = {}
        for d in dl.lin:
            L = d["L"]
            sec = time_fn(torch, lambda r, d=d: dl.single(api, d, r), max(4, steps // 2), 2)
            per[L.name] = {"M": M, "K": L.K, "N": L.N, "us": round(sec * 1e6, 2),
                           "GBs": round(linear_bytes(L) / sec / 1e9, 1),
                           "roofline": roofline_of([L], sec, "one forward (all its launches)")}
        sec = time_fn(torch, lambda r: dl.step(api, r), max(4, steps // 2), 2)
        per["all_three_batched"] = {"us": round(sec * 1e6, 2),
                                    "roofline": roofline_of(list(work.linears), sec,
                                                            "forward_batch of the three")}
        res[f"M{M}"] = per
        del dl
        torch.cuda.empty_cache()
    del packs
    torch.cuda.empty_cache()
    return {"workload": "70B-shaped FFN BitLinears (weights drawn on the device)", **res}


def secondary_tiny(torch, api, steps, warmup):
    """The single 256 x 256 BitLinear at M = 1 (correctness-sized: its time
    is the launch floor, so no roofline claim)."""
    from ternary_bit_linear_amd import workloads as wl
    prep = Prepared(torch, api, wl.TINY)
    ms = time_steps(torch, api, prep, steps, warmup)
    del prep
    return {"workload": wl.TINY.name, "us": round(ms * 1e3, 2)}


def measured_ceilings(torch, api):
    """Measured ceilings: one launch reading the decode layer's weight bytes
    (17.6 MB) and a 70B FFN matrix (58.7 MB) from HBM (buffers rotated over
    >= 768 MB so the reads miss the last-level cache), a device copy of the
    same sizes, and back-to-back int8 MFMAs over the whole device."""
    res = {}
    for name, nbytes in (("decode_layer_17.6MB", 17636352), ("ffn70b_matrix_58.7MB", 58720256)):
        nbytes = nbytes // 16 * 16
        copies = max(2, -(-ROTATE_BYTES // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i & 255)
                for i in range(copies)]
        sink = api.probe_read(bufs[0])
        sec = time_fn(torch, lambda r: api.probe_read(bufs[r % copies], sink), 50, 5)
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        sec_c = time_fn(torch, lambda r: dst.copy_(bufs[r % copies]), 50, 5)
        res[name] = {"read_GBs": round(nbytes / sec / 1e9, 1), "read_us": round(sec * 1e6, 2),
                     "copy_GBs_read_plus_write": round(2 * nbytes / sec_c / 1e9, 1),
                     "copy_us": round(sec_c * 1e6, 2)}
        del bufs, dst, sink
        torch.cuda.empty_cache()
    iters, wgs = 4096, 512
    sink = api.probe_mfma(iters, wgs)
    sec = time_fn(torch, lambda r: api.probe_mfma(iters, wgs, sink), 10, 2)
    ops = 4 * 65536 * iters * 4 * wgs
    res["int8_mfma_back_to_back"] = {"TOPS": round(ops / sec / 1e12, 1),
                                     "frac_of_published": round(ops / sec / 1e12 / INT8_PEAK_TOPS,
                                                                4),
                                     "workgroups": wgs, "rounds_per_wave": iters}
    return res


def secondary_ffn(torch, api, steps, warmup):
    """The BitNet FFN block (gate, up, squared-ReLU product, down with its
    sub-norm) as one bitlinear_ffn_forward call per step, on the 2B4T
    shapes (H = 2560, F = 6912) at decode (M = 1, GB/s of algorithmic
    bytes) and prefill (M = 512, int8 TOPS), and the 70B shapes (H = 8192,
    F = 28672) at M = 1.  Beside it the same block from the plain entry
    points (gate and up in one forward_batch call, relu(g)^2 * u in torch,
    then the down forward).  Weights: seeded ternary x scale generated on
    the device, packed copies rotated past the last-level cache."""
    from ternary_bit_linear_amd import workloads as wl
    res = {}
    for name, M, H, F in (("2b4t_decode", 1, 2560, 6912), ("2b4t_prefill", 512, 2560, 6912),
                          ("70b_decode", 1, 8192, 28672)):
        gen = torch.Generator(device="cuda")
        packs = []
        for i, (n, k, sc) in enumerate(((F, H, 0.02), (F, H, 0.015), (H, F, 0.025))):
            gen.manual_seed(6000 + i)
            t = torch.randint(-1, 2, (n, k), generator=gen, device="cuda", dtype=torch.int8)
            w = t.to(torch.float32).mul_(sc)
            del t
            packs.append(api.pack_i2s(w))
            del w
        wbytes = 3 * H * F // 4
        copies = max(2, -(-ROTATE_BYTES // wbytes))
        rot = [[(p.clone() if c else p, sc) for p, sc in packs] for c in range(copies)]
        x = torch.from_numpy(wl.activations(6100, M, H, 0.01)).cuda()
        gi = torch.from_numpy(wl.gamma(6101, H, "u0.8-1.2")).cuda()
        gs = torch.from_numpy(wl.gamma(6102, F, "u0.8-1.2")).cuda()
        y = torch.empty((M, H), dtype=torch.float32, device="cuda")
        ws = torch.empty(api.ffn_workspace_bytes(M, H, F), dtype=torch.uint8, device="cuda")
        g_t = torch.empty((M, F), dtype=torch.float32, device="cuda")
        u_t = torch.empty_like(g_t)
        a_t = torch.empty_like(g_t)
        ws_g, ws_u = api.new_workspace(M, H), api.new_workspace(M, H)
        ws_d = api.new_workspace(M, F)

        def fused(r):
            gp, up, dp = rot[r % copies]
            api.ffn_forward(x, gi, 1e-6, gp, up, dp, gs, out=y, workspace=ws)

        def plain(r):
            (gp, sg), (up, su), (dp, sd) = rot[r % copies]
            api.forward_batch([(x, gp, sg, gi, 1e-6, g_t, ws_g), (x, up, su, gi, 1e-6, u_t, ws_u)])
            torch.mul(torch.relu(g_t).square_(), u_t, out=a_t)
            api.forward(a_t, dp, sd, gs, 1e-6, H, out=y, workspace=ws_d)

        def timed(fn):
            gw = capture(torch, lambda: [fn(r) for r in range(max(1, warmup))])
            gt = capture(torch, lambda: [fn(warmup + r) for r in range(steps)])
            t = replay_timed(torch, gw, gt, steps)
            del gw, gt
            return t  # s per step

        t_f = timed(fused)
        t_p = timed(plain)
        nbytes = wbytes + 4 * M * H + 4 * H + 4 * F + 4 * M * H
        ops = 2 * M * 3 * H * F
        r = {"M": M, "H": H, "F": F, "us": round(t_f * 1e6, 2),
             "plain_entry_points_us": round(t_p * 1e6, 2),
             "speedup_vs_plain": round(t_p / t_f, 3)}
        if M <= 16:
            r.update({"GBs": round(nbytes / t_f / 1e9, 1),
                      "frac_of_hbm_peak": round(nbytes / t_f / 1e9 / HBM_PEAK_GBS, 4),
                      "algorithmic_bytes": nbytes})
        else:
            r.update({"TOPS": round(ops / t_f / 1e12, 1),
                      "frac_of_int8_peak": round(ops / t_f / 1e12 / INT8_PEAK_TOPS, 4)})
        res[name] = r
        del rot, packs, x, gi, gs, y, ws, g_t, u_t, a_t, ws_g, ws_u, ws_d
        torch.cuda.empty_cache()
    return {"workload": "BitNet FFN block: down(sub_norm(relu(gate(x))^2 * up(x)))", **res}


def secondary_io(torch, api, steps, warmup):
    """The decoder layer's BitLinears with bf16 activations in and out, as
    one bitlinear_forward_io_batch call per step (decode: one one-shot
    launch; prefill: typed quantisation, contraction, rescale per
    BitLinear), beside the fp32 step."""
    from ternary_bit_linear_amd import workloads as wl
    res = {}
    for key, work in (("decode_bf16", wl.DECODE_LAYER), ("prefill_bf16", wl.PREFILL_LAYER)):
        prep = Prepared(torch, api, work)
        io = []
        for d in prep.lin:
            L = d["L"]
            io.append({"x": d["x"].to(torch.bfloat16),
                       "y": torch.empty((L.M, L.N), dtype=torch.bfloat16, device="cuda"),
                       "ws": torch.empty(int(api.lib().bitlinear_io_workspace_bytes(L.M, L.K, L.N)),
                                         dtype=torch.uint8, device="cuda")})

        def step(r):
            api.forward_io_batch([(b["x"], d["P"][r % prep.copies], d["s"], d["g"], work.eps,
                                   b["y"], b["ws"]) for d, b in zip(prep.lin, io)])
        gw = capture(torch, lambda: [step(r) for r in range(max(1, warmup))])
        gt = capture(torch, lambda: [step(warmup + r) for r in range(steps)])
        t = replay_timed(torch, gw, gt, steps)
        del gw, gt
        t32 = time_steps(torch, api, prep, steps, warmup) * 1e-3
        nbytes = sum(L.N * L.K // 4 + 2 * L.M * L.K + 4 * L.K + 2 * L.M * L.N for L in work.linears)
        r = {"us": round(t * 1e6, 2), "fp32_step_us": round(t32 * 1e6, 2)}
        if work.linears[0].M <= 16:
            r["GBs"] = round(nbytes / t / 1e9, 1)
        else:
            r["TOPS"] = round(work.int_ops() / t / 1e12, 1)
        res[key] = r
        del prep, io
        torch.cuda.empty_cache()
    return {"workload": "decoder-layer BitLinears with bf16 activation I/O", **res}


def secondary_nonorm(torch, api, steps, warmup):
    """The decoder layer's BitLinears without RMSNorm (gamma NULL: the layer
    with use_rms_norm off), one forward_batch call per step, beside the
    step with RMSNorm."""
    from ternary_bit_linear_amd import workloads as wl
    work = wl.DECODE_LAYER
    prep = Prepared(torch, api, work)

    def step(r):
        api.forward_batch([(d["x"], d["P"][r % prep.copies], d["s"], None, work.eps, d["y"],
                            d["ws"]) for d in prep.lin])
    gw = capture(torch, lambda: [step(r) for r in range(max(1, warmup))])
    gt = capture(torch, lambda: [step(warmup + r) for r in range(steps)])
    t = replay_timed(torch, gw, gt, steps)
    del gw, gt
    t_norm = time_steps(torch, api, prep, steps, warmup) * 1e-3
    nbytes = sum(L.N * L.K // 4 + 4 * L.M * L.K + 4 * L.M * L.N for L in work.linears)
    del prep
    torch.cuda.empty_cache()
    return {"workload": "decoder-layer BitLinears at decode without RMSNorm (gamma NULL)",
            "us": round(t * 1e6, 2), "with_rmsnorm_us": round(t_norm * 1e6, 2),
            "GBs": round(nbytes / t / 1e9, 1)}


def secondary_dense(torch, api, steps, warmup):
    """Comparison: the decoder layer run the way the pages' BLAS route runs
    a prompt batch -- weights dequantised once (bitlinear_dequant_i2s, to
    bf16) and a library GEMM per BitLinear (torch.mm on bf16, no activation
    quantisation) -- beside the I2_S path, at decode and prefill.  The dense
    weights are rotated past the last-level cache like the packed ones."""
    from ternary_bit_linear_amd import workloads as wl
    res = {}
    for key, work in (("decode", wl.DECODE_LAYER), ("prefill", wl.PREFILL_LAYER)):
        prep = Prepared(torch, api, work)
        dense_bytes = sum(2 * L.N * L.K for L in work.linears)
        copies = max(2, -(-ROTATE_BYTES // dense_bytes))
        mats = []
        for d in prep.lin:
            L = d["L"]
            w = api.dequant_i2s(d["P"][0], L.N, L.K, torch.bfloat16)
            wt = w.t().contiguous()  # [K][N]: a plain (non-transposed) right operand
            del w
            mats.append({"x": d["x"].to(torch.bfloat16), "wt": [wt] + [wt.clone() for _ in range(copies - 1)],
                         "y": torch.empty((L.M, L.N), dtype=torch.bfloat16, device="cuda")})
        torch.cuda.synchronize()

        def step(r):
            for m in mats:
                torch.mm(m["x"], m["wt"][r % copies], out=m["y"])
        gw = capture(torch, lambda: [step(r) for r in range(max(1, warmup))])
        gt = capture(torch, lambda: [step(warmup + r) for r in range(steps)])
        t = replay_timed(torch, gw, gt, steps)
        del gw, gt
        t_i2s = time_steps(torch, api, prep, steps, warmup) * 1e-3
        res[key] = {"dense_bf16_library_us": round(t * 1e6, 2), "i2s_us": round(t_i2s * 1e6, 2),
                    "i2s_speedup": round(t / t_i2s, 3),
                    "dense_weight_bytes": dense_bytes,
                    "packed_weight_bytes": sum(L.N * L.K // 4 for L in work.linears)}
        del prep, mats
        torch.cuda.empty_cache()
    return {"workload": "decoder-layer BitLinears: dequantised bf16 weights + library GEMM "
                        "(torch.mm) against the I2_S path", **res}


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
    ap.add_argument("--dense-only", action="store_true",
                    help="time only the dequantised-bf16 library comparison and print its line")
    ap.add_argument("--io-only", action="store_true",
                    help="time only the bf16-I/O legs (--steps steps each) and print their line")
    ap.add_argument("--ffn-only", action="store_true",
                    help="time only the FFN block legs (--steps steps each) and print their line")
    ap.add_argument("--sweep-only", action="store_true",
                    help="time only the K = N = 8192 sweep and print its line")
    ap.add_argument("--ffn70b-only", action="store_true",
                    help="time only the 70B FFN BitLinears at M = 1 and 16 and print their line")
    ap.add_argument("--ceilings-only", action="store_true",
                    help="measure only the read / copy / MFMA ceilings and print their line")
    ap.add_argument("--pmc-app", action="store_true",
                    help="no timing: run --steps steps of the workload and a 256 MiB device "
                         "copy (the calibration kernel for HBM byte counters), then exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: one GPU only; --gpus must be 1 "
              "(the library runs one GPU per process; a multi-GPU split of N is not built)",
              file=sys.stderr)
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
    if args.dense_only:
        print(json.dumps(secondary_dense(torch, api, max(1, args.steps), args.warmup)), flush=True)
        return
    if args.io_only:
        print(json.dumps(secondary_io(torch, api, max(1, args.steps), args.warmup)), flush=True)
        return
    if args.ffn_only:
        print(json.dumps(secondary_ffn(torch, api, max(1, args.steps), args.warmup)), flush=True)
        return
    if args.sweep_only:
        print(json.dumps(secondary_sweep(torch, api, max(1, args.steps), args.warmup)), flush=True)
        return
    if args.ffn70b_only:
        print(json.dumps(secondary_ffn70b(torch, api, max(1, args.steps), args.warmup)),
              flush=True)
        return
    if args.ceilings_only:
        print(json.dumps(measured_ceilings(torch, api)), flush=True)
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
                # HIP-event time per launch over the graph-replayed timed
                # region (back-to-back steps, launch gaps included)
                "avg_step_us": round(avg_s * 1e6, 3),
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
                    "avg_step_us": round(dom_s * 1e6, 3),
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
                    "kernel": "act_quant_batch_kernel + grouped I2_S x int8 MFMA contraction, "
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
        "clock_warmup_s": CLOCK_WARM_S, "clock_warmup_chunk_s": CLOCK_CHUNK_S,
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
        sec_steps = max(20, args.steps // 4)
        out["secondary"] = secondary_prefill(torch, api, sec_steps, 5)
        torch.cuda.empty_cache()
        out["secondary"]["sweep"] = secondary_sweep(torch, api, sec_steps, 5)
        out["secondary"]["square_m512"] = {
            "workload": "square BitLinear K=N=8192 M=512",
            **{k: out["secondary"]["sweep"]["M512"][k] for k in ("us", "TOPS", "roofline")}}
        torch.cuda.empty_cache()
        out["secondary"]["ffn70b_linears"] = secondary_ffn70b(torch, api, sec_steps, 5)
        torch.cuda.empty_cache()
        out["secondary"]["tiny"] = secondary_tiny(torch, api, sec_steps, 5)
        torch.cuda.empty_cache()
        out["secondary"]["pack"] = secondary_pack(torch, api)
        torch.cuda.empty_cache()
        out["secondary"]["ffn"] = secondary_ffn(torch, api, max(20, args.steps // 4), 5)
        torch.cuda.empty_cache()
        out["secondary"]["io"] = secondary_io(torch, api, max(20, args.steps // 4), 5)
        torch.cuda.empty_cache()
        out["secondary"]["dense_comparison"] = secondary_dense(torch, api, max(20, args.steps // 4), 5)
        torch.cuda.empty_cache()
        out["secondary"]["no_rmsnorm"] = secondary_nonorm(torch, api, max(20, args.steps // 4), 5)
        torch.cuda.empty_cache()
        out["measured_ceilings"] = measured_ceilings(torch, api)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(work)
        one = cpu_baseline(work, budget_s=8.0, threads=1)
        out["cpu_baseline"]["single_thread"] = {k: one[k] for k in
                                                ("value", "unit", "cores", "sample", "seconds",
                                                 "ms_per_step")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
