#!/usr/bin/env python3
"""Benchmark of the tile-hybrid dense / 2:4 GEMV on one MI355X.

Default workload: Llama-3.1-8B-shaped up projection, W 14336 x 4096 bf16,
128 x 128 tiles, 2509 of 3584 tiles 2:4 sparse (35.0% sparsity), decode
batch M = 1.  A step is one pass of every row of the hot path on one batch:
  gemv      hybrid decode product, M = 1                    <- the metric
  dense     the same kernel with the all-dense tile map     <- speedup base
  gemm      prefill product, M = 64, matrix-core kernel
  unpack    hybrid streams -> W'
  pack      W -> hybrid streams (rotating copy)
The timed region runs the K steps row by row (all GEMVs, then the GEMMs,
unpacks and packs) so no GEMV competes with the write-back of a packing
kernel's output.  Each kernel is bracketed by HIP events on the stream it
runs on (rows.*.us_mean, us_median; rates use the median).  The metric kernel is also timed as a burst: 2C
launches captured in a HIP graph and replayed between one event pair (C =
rotating copies); `value` is the hybrid GEMV's algorithmic bytes per launch
divided by that per-launch time, which is what a per-dispatch profiler
reports (an event pair per launch adds the event packets' own latency).  Packed copies rotate through more than 1 GiB per
kind (stepping by 3 copies) so the 256 MB last-level cache holds nothing
from the previous use of a copy.

After the timed steps, the grouped decode launch is compared with separate
launches on one decoder layer (JSON key "grouped"), the sparse + low-rank
decode product is compared with the plain one (JSON key "lowrank"), 4:8
tiles with 2:4 ones (JSON key "nm48"), and the prefill GEMM is
measured on its own workload
(Qwen3-14B-shaped 17408 x 5120, 64 x 64 tiles, M = 2048): hybrid, the same
kernel all-dense, and the vendor BLAS dense product, with the matrix-core
roofline (JSON key "prefill"); the same three on a short, deep matrix
(70B-shaped 8192 x 28672, 128 x 128 tiles in a checkerboard, M = 256, JSON
key "tall").

Prints one JSON line.  `python bench.py --sweep` also measures the other
workloads (stderr table plus --sweep-json file).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "hybrid 2:4/dense GEMV µs + achieved HBM GB/s at 8B MLP shape; speedup vs dense"
HBM_PEAK_GBS = 8000.0
# HBM bytes per hybrid decode launch at this workload, from two rocprofv3
# --pmc passes (FETCH_SIZE, then WRITE_SIZE) scaled by a plain 128 MiB copy's
# readings; the summary, its command and the kernel it covers are in
# TRAFFIC_PROFILE.  Valid for the kernel as profiled; re-measure after
# changing it.
TRAFFIC_BYTES_PER_LAUNCH = 82_676_736
TRAFFIC_PROFILE = "profiles/k_gemv_llama8b_up_14336x4096_m1_hbm_traffic.md"
TRAFFIC_KERNEL = ("k_gemv_mixed<MT=1, B2=128, bf16, idx2, WAVES=4, STAGES=2, LR=false, XR=true> "
                  "(768 whole-slab and 256 half-slab workgroups)")
MFMA_PEAK_BF16_TFLOPS = 2500.0


def roofline(alg_bytes_: int, flops: int, us: float, kernel: str) -> dict:
    """Roofline of one product: the larger of bytes / 8 TB/s and flops /
    2.5 PF (dense bf16 matrix-core peak) bounds it; `frac` is that time over
    the measured time, `achieved` the rate in the bound's own unit."""
    t_hbm = alg_bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_PEAK_BF16_TFLOPS * 1e12)
    sec = us * 1e-6
    if t_hbm >= t_mfma:
        ach = alg_bytes_ / sec / 1e9
        return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(t_hbm / sec, 4), "alg_bytes": alg_bytes_, "alg_flops": flops,
                "roofline_us": round(1e6 * t_hbm, 3), "kernel": kernel}
    ach = flops / sec / 1e12
    return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(t_mfma / sec, 4), "alg_bytes": alg_bytes_, "alg_flops": flops,
            "roofline_us": round(1e6 * t_mfma, 3), "kernel": kernel}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(layout, m: int, y_bytes: int = 4) -> int:
    """Algorithmic bytes of one product: weights as stored, tile index,
    activations read once, outputs written once."""
    return (layout.dense_bytes + layout.val_bytes + layout.meta_bytes + layout.tidx_bytes
            + 2 * m * layout.k + y_bytes * m * layout.n)


def alg_flops(layout, m: int) -> int:
    """2 flops per stored (kept) weight per token."""
    tile = layout.b1 * layout.b2
    return 2 * m * (tile * layout.n_dense + tile * layout.n_sparse // 2)


class Timer:
    """Per-launch HIP event pairs on the current stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def run(self, name, fn):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))

    def ms(self, name):
        return [s.elapsed_time(e) for s, e in self.pairs.get(name, [])]


def copies_for(nbytes: int, rotate_bytes: int) -> int:
    return max(2, -(-rotate_bytes // max(nbytes, 1)))


def setup_matrix(hb, torch, mat, tmap, meta, rotate_bytes, dev):
    w_bits = mat.weight_bits()
    w = hb.bits_to_tensor(w_bits, mat.dtype, dev)
    first = hb.pack(w, tmap, mat.b1, mat.b2, meta)
    n_copies = copies_for(first.weight_bytes(), rotate_bytes)
    copies = [first] + [hb.pack(w, tmap, mat.b1, mat.b2, meta) for _ in range(n_copies - 1)]
    torch.cuda.synchronize()
    return w, w_bits, copies


def _oracle_passes(oracle, P, mat, x_bits, budget_s):
    """Median seconds of (unpack, float64 product) passes of the oracle."""
    times, unp, mm = [], [], []
    t_end = time.perf_counter() + budget_s
    while len(times) < 3 or (time.perf_counter() < t_end and len(times) < 5):
        t0 = time.perf_counter()
        wp = oracle.unpack(P["dense"], P["val"], P["meta"], P["tidx"], mat.n, mat.k, mat.b1, mat.b2, "idx2")
        t1 = time.perf_counter()
        oracle.ref_matmul(wp, x_bits, mat.dtype)
        t2 = time.perf_counter()
        times.append(t2 - t0)
        unp.append(t1 - t0)
        mm.append(t2 - t1)
        if time.perf_counter() > t_end and len(times) >= 1:
            break
    return statistics.median(times), statistics.median(unp), statistics.median(mm), len(times)


def cpu_baseline(mat, w_bits, tmap, x_bits, layout, budget_s=12.0):
    """The oracle as it stands (unpack to dense + float64 product), timed on
    this host's cores on the full workload matrix: once with the BLAS
    threads it starts with, once limited to one thread."""
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        threads = os.cpu_count() or 1
    P = oracle.pack(w_bits, tmap, mat.b1, mat.b2, "idx2")
    gb = alg_bytes(layout, x_bits.shape[0])
    med, unp, mm, runs = _oracle_passes(oracle, P, mat, x_bits, budget_s)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            med1, unp1, mm1, runs1 = _oracle_passes(oracle, P, mat, x_bits, budget_s / 2)
        one = {"value": round(gb / med1 / 1e9, 4), "unit": "GB/s", "cores": 1,
               "seconds_per_pass": round(med1, 4),
               "sample": f"median of {runs1} runs ({unp1:.3f} s unpack + {mm1:.3f} s matmul)"}
    return {
        "value": round(gb / med / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"whole {mat.n}x{mat.k} matrix, M={x_bits.shape[0]}: oracle unpack + float64 "
                   f"X.W'^T and |X|.|W'|^T, median of {runs} runs "
                   f"({unp:.3f} s unpack + {mm:.3f} s matmul)"),
        "seconds_per_pass": round(med, 4),
        "single_core": one,
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--meta", default="idx2", choices=["idx2", "mask4"])
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--gemm-m", type=int, default=64)
    ap.add_argument("--prefill-m", type=int, default=2048,
                    help="token count of the prefill GEMM measurement")
    ap.add_argument("--only", default="",
                    help="comma list of parts to run (pack,gemv,dense,unpack,gemm,grouped,lowrank,nm48,patterns,"
                         "prefill,tall,mid)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run plain 128 MiB device copies (torch copy kernel) as a counter reference")
    ap.add_argument("--sweep", action="store_true")
    ap.add_argument("--sweep-json", default="")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from matmul_pack_b1_amd import binding as hb
    from matmul_pack_b1_amd import workloads as wl
    hb.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    rotate = int(args.rotate_gib * (1 << 30))
    rows = set(args.only.split(",")) if args.only else {"pack", "gemv", "dense", "unpack", "gemm", "grouped",
                                                         "lowrank", "nm48", "patterns", "prefill", "tall", "mid"}

    if args.copy_calibration:
        # A plain copy of known size: 128 MiB read + 128 MiB written per
        # launch, rotating over 8 pairs (2 GiB) so the last-level cache holds
        # none of it; hardware byte counters of this kernel give the scale
        # factor for the counters of the kernels below.
        nb = 128 << 20
        bufs = [(torch.empty(nb, dtype=torch.uint8, device=dev), torch.empty(nb, dtype=torch.uint8, device=dev))
                for _ in range(8)]
        for i in range(16):
            src, dst = bufs[i % 8]
            dst.copy_(src)
        torch.cuda.synchronize()
        del bufs
        torch.cuda.empty_cache()
        log("[bench] copy calibration: 16 copies of 134217728 bytes")

    mat = wl.workload(2).matrices[0]
    tmap = mat.tile_map()
    dmap = np.zeros_like(tmap)
    log(f"[bench] setting up {mat.n}x{mat.k} {mat.dtype}, {int(tmap.sum())}/{tmap.size} sparse tiles")
    w, w_bits, hyb = setup_matrix(hb, torch, mat, tmap, args.meta, rotate, dev)
    _, _, dense = setup_matrix(hb, torch, mat, dmap, args.meta, rotate, dev) if "dense" in rows else (None, None, [])
    L = hyb[0].layout
    x_bits = mat.activation_bits(1)
    x = hb.bits_to_tensor(x_bits, mat.dtype, dev)
    xg = hb.bits_to_tensor(mat.activation_bits(args.gemm_m), mat.dtype, dev)
    y = torch.empty((1, mat.n), dtype=torch.float32, device=dev)
    yg = torch.empty((args.gemm_m, mat.n), dtype=torch.float32, device=dev)
    wout = torch.empty((mat.n, mat.k), dtype=w.dtype, device=dev)
    log(f"[bench] {len(hyb)} hybrid copies ({hyb[0].weight_bytes()} B each), {len(dense)} dense copies")

    nh = len(hyb)

    # One step = one batch through every row.  The rows are timed in separate
    # phases of the timed region (all GEMVs first, then the GEMMs, unpacks
    # and packs), so that no GEMV starts while the write-back of a previous
    # kernel's output is still draining to HBM.
    def phase(name, i, timer):
        if name == "gemv":
            timer.run("gemv", lambda: hb.gemv(hyb[(i * 3) % nh], x, out=y))
        elif name == "dense":
            timer.run("dense", lambda: hb.gemv(dense[(i * 3) % len(dense)], x, out=y))
        elif name == "gemm":
            timer.run("gemm", lambda: hb.gemm_mfma(hyb[(i * 3 + 1) % nh], xg, out=yg))
        elif name == "unpack":
            timer.run("unpack", lambda: hb.unpack(hyb[(i * 3 + 2) % nh], out=wout))
        elif name == "pack":
            timer.run("pack", lambda: hb.pack(w, tmap, mat.b1, mat.b2, args.meta, out=hyb[(i * 3 + 2) % nh]))

    def run_steps(first, count, timer):
        for i in range(first, first + count):
            for name in ("gemv", "dense"):
                if name in rows:
                    phase(name, i, timer)
        for name in ("gemm", "unpack", "pack"):
            if name in rows:
                for i in range(first, first + count):
                    phase(name, i, timer)

    warm = Timer(torch)
    run_steps(0, args.warmup, warm)
    torch.cuda.synchronize()
    timer = Timer(torch)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.warmup, args.steps, timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"[bench] timed {args.steps} steps in {wall:.3f} s")

    # Burst timing of the metric kernel: R hybrid GEMVs (rotating copies)
    # captured once in a HIP graph and replayed, bracketed by one event pair;
    # per-launch time = elapsed / R.  Replays leave almost no gap between
    # kernels, so this is the figure that matches per-dispatch profiler time.
    burst = {"stream_us": {}, "graph_us": {}}
    if "gemv" in rows or "dense" in rows:
        def launch_burst(lst, Rn, base=0):
            for i in range(Rn):
                hb.gemv(lst[(base + 3 * i) % len(lst)], x, out=y)
        for kind, lst in (("gemv", hyb), ("dense", dense)):
            if kind not in rows:
                continue
            Rk = 2 * len(lst)
            launch_burst(lst, Rk)
            torch.cuda.synchronize()
            s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s_.record()
            for rep in range(3):
                launch_burst(lst, Rk, rep)
            e_.record()
            torch.cuda.synchronize()
            burst["stream_us"][kind] = round(1e3 * s_.elapsed_time(e_) / (3 * Rk), 3)
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                g.capture_begin()
                launch_burst(lst, Rk)
                g.capture_end()
            torch.cuda.current_stream().wait_stream(cs)
            g.replay()
            torch.cuda.synchronize()
            times = []
            for rep in range(5):
                s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s_.record()
                g.replay()
                e_.record()
                torch.cuda.synchronize()
                times.append(s_.elapsed_time(e_) / Rk)
            burst["graph_us"][kind] = round(1e3 * statistics.median(times), 3)
            del g
        log(f"[bench] burst timing: {burst}")

    # Practical read-rate reference: the same number of bytes as one hybrid
    # product, read with the decode kernel's load pattern by a plain
    # streaming kernel, rotating over the same >1 GiB footprint.
    stream_ref = None
    if "gemv" in rows:
        nb = hyb[0].weight_bytes() // 16 * 16
        big = torch.empty(nb * nh, dtype=torch.uint8, device=dev)
        big.fill_(1)
        sink = torch.empty(2048 * 256, dtype=torch.int32, device=dev)
        best = None
        for grid in (512, 1024, 2048):
            for i in range(nh):
                hb.stream_read(big[i * nb:(i + 1) * nb], nb, sink, grid)
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream()
            cs.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(cs):
                g.capture_begin()
                for i in range(2 * nh):
                    j = (3 * i) % nh
                    hb.stream_read(big[j * nb:(j + 1) * nb], nb, sink, grid)
                g.capture_end()
            torch.cuda.current_stream().wait_stream(cs)
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for rep in range(5):
                s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s_.record()
                g.replay()
                e_.record()
                torch.cuda.synchronize()
                ts.append(1e3 * s_.elapsed_time(e_) / (2 * nh))
            us = statistics.median(ts)
            if best is None or us < best[1]:
                best = (grid, us)
            del g
        del big
        torch.cuda.empty_cache()
        stream_ref = {"bytes": nb, "grid": best[0], "us": round(best[1], 3),
                      "GBps": round(nb / (best[1] * 1e-6) / 1e9, 2)}
        log(f"[bench] streaming-read reference: {stream_ref}")

    res_rows = {}
    for name in ("pack", "gemv", "dense", "unpack", "gemm"):
        ms = timer.ms(name)
        if not ms:
            continue
        res_rows[name] = {"us_mean": round(1e3 * statistics.mean(ms), 3),
                          "us_median": round(1e3 * statistics.median(ms), 3),
                          "us_p10": round(1e3 * float(np.percentile(ms, 10)), 3),
                          "us_p90": round(1e3 * float(np.percentile(ms, 90)), 3)}
    gb = alg_bytes(L, 1)
    out = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(1e3 * wall / max(args.steps, 1), 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if "gemv" in res_rows:
        us = burst["graph_us"]["gemv"]
        out["value"] = round(gb / (us * 1e-6) / 1e9, 2)
        res_rows["gemv"].update({"alg_bytes": gb, "GBps_event_pairs": round(gb / (res_rows["gemv"]["us_median"] * 1e-6) / 1e9, 2),
                                 "us_graph_burst": us, "us_stream_burst": burst["stream_us"]["gemv"],
                                 "GBps": out["value"]})
        out["gemv_us"] = us
    else:
        out["value"] = None
    if "dense" in res_rows:
        Ld = dense[0].layout
        gbd = alg_bytes(Ld, 1)
        usd = burst["graph_us"]["dense"]
        res_rows["dense"].update({"alg_bytes": gbd, "us_graph_burst": usd, "us_stream_burst": burst["stream_us"]["dense"],
                                  "GBps_event_pairs": round(gbd / (res_rows["dense"]["us_median"] * 1e-6) / 1e9, 2),
                                  "GBps": round(gbd / (usd * 1e-6) / 1e9, 2)})
        out["dense_us"] = usd
        if "gemv" in res_rows:
            out["speedup_vs_dense"] = round(usd / out["gemv_us"], 4)
            out["speedup_vs_dense_event_pairs"] = round(res_rows["dense"]["us_median"] / res_rows["gemv"]["us_median"], 4)
            out["byte_ratio_dense_over_hybrid"] = round(gbd / gb, 4)
    if "pack" in res_rows:
        rd = mat.n * mat.k * 2 + hyb[0].weight_bytes()
        res_rows["pack"].update({"alg_bytes": rd, "GBps": round(rd / (res_rows["pack"]["us_median"] * 1e-6) / 1e9, 2)})
    if "unpack" in res_rows:
        rd = mat.n * mat.k * 2 + hyb[0].weight_bytes()
        res_rows["unpack"].update({"alg_bytes": rd, "GBps": round(rd / (res_rows["unpack"]["us_median"] * 1e-6) / 1e9, 2)})
    if "gemm" in res_rows:
        fl = alg_flops(L, args.gemm_m)
        res_rows["gemm"].update({"m": args.gemm_m, "alg_flops": fl,
                                 "TFLOPs": round(fl / (res_rows["gemm"]["us_median"] * 1e-6) / 1e12, 2),
                                 "GBps": round(alg_bytes(L, args.gemm_m) / (res_rows["gemm"]["us_median"] * 1e-6) / 1e9, 2),
                                 "roofline": roofline(alg_bytes(L, args.gemm_m), fl, res_rows["gemm"]["us_median"],
                                                      kernel_text(hb, L, args.gemm_m))})
    out["config"] = {"workload": f"Llama-3.1-8B up projection {mat.n}x{mat.k} bf16, {mat.b1}x{mat.b2} tiles, "
                                 f"{L.n_sparse}/{L.tiles_n * L.tiles_k} tiles 2:4 ({args.meta}), decode M=1",
                     "n": mat.n, "k": mat.k, "tile": [mat.b1, mat.b2], "n_sparse_tiles": L.n_sparse,
                     "n_tiles": L.tiles_n * L.tiles_k, "batch": 1, "meta": args.meta,
                     "rotating_copies": {"hybrid": len(hyb), "dense": len(dense)}}
    out["rows"] = res_rows
    if out["value"] is not None:
        out["roofline"] = {"bound": "hbm", "achieved": out["value"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(out["value"] / HBM_PEAK_GBS, 4), "traffic": TRAFFIC_BYTES_PER_LAUNCH,
                           "traffic_source": (f"stored figure from {TRAFFIC_PROFILE} (rocprofv3 --pmc FETCH_SIZE "
                                              f"and WRITE_SIZE of {TRAFFIC_KERNEL}, scaled by a 128 MiB copy)"
                                              if TRAFFIC_BYTES_PER_LAUNCH else "not measured for this kernel"),
                           "kernel": TRAFFIC_KERNEL, "alg_bytes_per_launch": gb}
    if stream_ref is not None and out.get("value"):
        stream_ref["gemv_frac_of_stream"] = round(out["value"] / stream_ref["GBps"], 4)
        out["stream_reference"] = stream_ref
    if "grouped" in rows:
        log("[bench] grouped decode launch on one decoder layer")
        out["grouped"] = grouped(hb, torch, wl, dev, args.meta)
        log(f"[bench] grouped: {out['grouped']}")
    if "nm48" in rows:
        log("[bench] 4:8 against 2:4")
        out["nm48"] = nm48(hb, torch, wl, dev)
        log(f"[bench] nm48: {out['nm48']}")
    if "patterns" in rows:
        log("[bench] one metadata code throughout against mixed codes")
        out["patterns"] = patterns(hb, torch, wl, dev, args.meta)
        log(f"[bench] patterns: {out['patterns']}")
    if "lowrank" in rows:
        log("[bench] sparse + low-rank decode")
        out["lowrank"] = lowrank(hb, torch, wl, dev, args.meta)
        log(f"[bench] lowrank: {out['lowrank']}")
    if "prefill" in rows and args.prefill_m > 0:
        log(f"[bench] prefill GEMM M={args.prefill_m}")
        out["prefill"] = prefill(hb, torch, wl, dev, args.prefill_m, args.meta)
        log(f"[bench] prefill: {out['prefill']}")
    if "tall" in rows:
        log("[bench] prefill GEMM on a short, deep matrix, M=256")
        out["tall"] = tall(hb, torch, wl, dev, 256, args.meta)
        log(f"[bench] tall: {out['tall']}")
    if "mid" in rows:
        # the memory-bound range of the matrix-core kernels (16 to a few
        # hundred tokens), against the vendor BLAS on the same shapes
        log("[bench] GEMM in the memory-bound range: Qwen3-14B gate/up at 64, 96, 128 tokens; 70B down at 64, 128")
        out["mid"] = ([prefill(hb, torch, wl, dev, m, args.meta) for m in (64, 96, 128)] +
                      [tall(hb, torch, wl, dev, m, args.meta) for m in (64, 128)])
        log(f"[bench] mid: {out['mid']}")
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(mat, w_bits, tmap, x_bits, L)
    if args.sweep:
        out["sweep_file"] = sweep(hb, torch, wl, dev, rotate, args)
    print(json.dumps(out), flush=True)


def graph_us(torch, launch, count, reps=5):
    """Per-launch time of `count` launches captured in one HIP graph and
    replayed between one event pair (median of `reps` replays)."""
    launch(count)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cs):
        g.capture_begin()
        launch(count)
        g.capture_end()
    torch.cuda.current_stream().wait_stream(cs)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        s_, e_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s_.record()
        g.replay()
        e_.record()
        torch.cuda.synchronize()
        times.append(1e3 * s_.elapsed_time(e_) / count)
    del g
    return statistics.median(times)


def prefill(hb, torch, wl, dev, m, meta):
    """Prefill product at the Qwen3-14B-shaped gate/up projection (17408 x
    5120, 64 x 64 tiles, 60% of the tiles 2:4): the hybrid matrix-core GEMM,
    the same kernel on the all-dense map, and torch's bf16 matmul (the
    vendor BLAS) on the dense weights as the library reference."""
    mat = wl.workload(5).matrices[0]
    return product_row(hb, torch, dev, mat, m, meta,
                       f"Qwen3-14B gate/up projection {mat.n}x{mat.k} bf16, {mat.b1}x{mat.b2} tiles")


def tall(hb, torch, wl, dev, m, meta):
    """The same three products on the 70B-shaped down projection (8192 x
    28672, 128 x 128 tiles in a checkerboard): only 32 blocks of 256 rows, so
    up to a few hundred tokens the launcher runs a register-fed shape (128
    rows x 48 or 64 tokens, K split over four wavefronts), with K also split
    across one workgroup per CU where its tiles would leave CUs idle."""
    mat = wl.workload(4).matrices[5]
    return product_row(hb, torch, dev, mat, m, meta,
                       f"Llama-3.1-70B-shaped down projection {mat.n}x{mat.k} bf16, {mat.b1}x{mat.b2} tiles "
                       f"(checkerboard)")


def kernel_text(hb, layout, m):
    """The kernel and workgroup shape hyb_gemm launches here (hyb_gemm_shape)."""
    sh = hb.gemm_shape(layout, m)
    if sh["kernel"] == "decode":
        return f"k_gemv ({sh['waves']} wavefronts per 16-row slab)"
    lds_split = sh["kernel"] == "split" and sh["row_groups"] == 4
    lds_parts = lds_split and sh["token_blocks"] >= 12
    # K parts after whole rounds of plain tiles: the tiles outnumber the CUs
    # (the parts alone run only where they fill at most half of them)
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = -(-layout.n // 256) * -(-m // (16 * sh["token_blocks"]))
    if lds_parts and tiles > cus:
        return (f"k_gemm_lds over whole rounds, then k_gemm_lds_parts + k_gemm_lds_parts_sum on the last row "
                f"blocks (256-row x {16 * sh['token_blocks']}-token workgroups on {sh['waves']} wavefronts, "
                f"K cut into equal parts in the parts launch)")
    split_name = ("k_gemm_lds_parts + k_gemm_lds_parts_sum" if lds_parts else
                  "k_gemm_lds_split + k_gemm_lds_split_sum" if lds_split else "k_gemm_split + k_gemm_split_sum")
    name = {"register": "k_gemm_rx", "lds": "k_gemm_lds", "split": split_name}[sh["kernel"]]
    split = {"register": ", wavefronts splitting K",
             "split": (", K cut into equal parts, one per workgroup" if lds_parts else
                       ", K split across one workgroup per CU" if lds_split
                       else ", wavefronts splitting K, K also split across one workgroup per CU"),
             "lds": ""}[sh["kernel"]]
    return (f"{name} ({64 * sh['row_groups']}-row x {16 * sh['token_blocks']}-token workgroups on "
            f"{sh['waves']} wavefronts{split})")


def product_row(hb, torch, dev, mat, m, meta, name):
    """Hybrid GEMM, the same kernel on the all-dense map, and the vendor
    BLAS's dense bf16 product, each a graph burst over two copies."""
    tmap = mat.tile_map()
    w = hb.bits_to_tensor(mat.weight_bits(), mat.dtype, dev)
    x = hb.bits_to_tensor(mat.activation_bits(m), mat.dtype, dev)
    y = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
    hyb = [hb.pack(w, tmap, mat.b1, mat.b2, meta) for _ in range(2)]
    den = [hb.pack(w, np.zeros_like(tmap), mat.b1, mat.b2, meta) for _ in range(2)]
    torch.cuda.synchronize()
    L, Ld = hyb[0].layout, den[0].layout
    n_launch = 8
    us_h = graph_us(torch, lambda c: [hb.gemm(hyb[i % 2], x, out=y) for i in range(c)], n_launch)
    us_d = graph_us(torch, lambda c: [hb.gemm(den[i % 2], x, out=y) for i in range(c)], n_launch)
    # vendor dense reference: bf16 X @ W^T with an fp32-accumulating bf16 output
    wt = [w, w.clone()]
    yb = torch.empty((m, mat.n), dtype=w.dtype, device=dev)
    us_v = graph_us(torch, lambda c: [torch.matmul(x, wt[i % 2].t(), out=yb) for i in range(c)], n_launch)
    fl = alg_flops(L, m)
    fl_dense = 2 * m * mat.n * mat.k
    tf = fl / (us_h * 1e-6) / 1e12
    ab = alg_bytes(L, m)
    out = {"workload": f"{name}, {L.n_sparse}/{L.tiles_n * L.tiles_k} tiles 2:4 ({meta}), prefill M={m}",
           "m": m, "hybrid_us": round(us_h, 2), "dense_same_kernel_us": round(us_d, 2),
           "vendor_blas_dense_us": round(us_v, 2), "alg_flops": fl, "dense_flops": fl_dense,
           "TFLOPs": round(tf, 1), "dense_same_kernel_TFLOPs": round(fl_dense / (us_d * 1e-6) / 1e12, 1),
           "vendor_blas_TFLOPs": round(fl_dense / (us_v * 1e-6) / 1e12, 1),
           "speedup_vs_dense_same_kernel": round(us_d / us_h, 4),
           "speedup_vs_vendor_blas": round(us_v / us_h, 4),
           "alg_bytes": ab, "GBps": round(ab / (us_h * 1e-6) / 1e9, 1),
           "roofline": roofline(ab, fl, us_h, kernel_text(hb, L, m)),
           "timing": f"graph burst of {n_launch} launches over 2 rotating copies, median of 5 replays"}
    del hyb, den, wt, w, x, y, yb
    torch.cuda.empty_cache()
    return out


def patterns(hb, torch, wl, dev, meta):
    """The decode product on the Llama-3.1-8B up projection (M = 1, the same
    tile map) with the seeded weights, whose 2:4 groups keep all six patterns
    in equal measure, against weights whose every group keeps positions 0
    and 1 (columns 2 and 3 of each group zeroed, so one metadata code fills
    the whole stream).  The kernel reads a fixed stride whatever the codes
    (SparseDecoding abstract), so the two times should agree."""
    mat = wl.workload(2).matrices[0]
    tmap = mat.tile_map()
    wb = mat.weight_bits()
    same = wb.copy()
    same[:, 2::4] = 0
    same[:, 3::4] = 0
    x = hb.bits_to_tensor(mat.activation_bits(1), mat.dtype, dev)
    y = torch.empty((1, mat.n), dtype=torch.float32, device=dev)
    out = {}
    for name, bits in (("mixed_patterns", wb), ("one_pattern", same)):
        w = hb.bits_to_tensor(bits, mat.dtype, dev)
        P0 = hb.pack(w, tmap, mat.b1, mat.b2, meta)
        n_copies = copies_for(P0.weight_bytes(), 1 << 30)
        Ps = [P0] + [hb.pack(w, tmap, mat.b1, mat.b2, meta) for _ in range(n_copies - 1)]
        torch.cuda.synchronize()
        if name == "one_pattern":
            codes = np.unique(P0.meta.cpu().numpy())
            out["one_pattern_codes"] = [hex(int(c)) for c in codes]
        us = graph_us(torch, lambda c: [hb.gemv(Ps[(3 * i) % n_copies], x, out=y) for i in range(c)],
                      2 * n_copies)
        out[name] = {"us": round(us, 3), "GBps": round(alg_bytes(P0.layout, 1) / (us * 1e-6) / 1e9, 1)}
        del Ps, P0, w
        torch.cuda.empty_cache()
    out["one_over_mixed"] = round(out["one_pattern"]["us"] / out["mixed_patterns"]["us"], 4)
    return out


def nm48(hb, torch, wl, dev):
    """4:8 sparse tiles (metadata kind mask8) against 2:4 (idx2) on the same
    tile maps: the decode product on the Llama-3.1-8B up projection at M = 1
    and 16 (rotating cold copies; both kinds store the same bytes), and the
    prefill product on the Qwen3-14B gate/up projection at M = 2048 (4:8
    tiles expand to dense matrix-core work, so the all-dense map of the same
    kernel is the comparison there)."""
    out = {}
    mat = wl.workload(2).matrices[0]
    w = hb.bits_to_tensor(mat.weight_bits(), mat.dtype, dev)
    tmap = mat.tile_map()
    for m in (1, 16):
        x = hb.bits_to_tensor(mat.activation_bits(m), mat.dtype, dev)
        y = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
        row = {}
        for meta in ("idx2", "mask8"):
            P0 = hb.pack(w, tmap, mat.b1, mat.b2, meta)
            n_copies = copies_for(P0.weight_bytes(), 1 << 30)
            Ps = [P0] + [hb.pack(w, tmap, mat.b1, mat.b2, meta) for _ in range(n_copies - 1)]
            torch.cuda.synchronize()
            us = graph_us(torch, lambda c: [hb.gemv(Ps[(3 * i) % n_copies], x, out=y) for i in range(c)],
                          2 * n_copies)
            row[meta] = {"us": round(us, 3), "GBps": round(alg_bytes(P0.layout, m) / (us * 1e-6) / 1e9, 1)}
            del Ps, P0
            torch.cuda.empty_cache()
        row["mask8_over_idx2"] = round(row["mask8"]["us"] / row["idx2"]["us"], 4)
        out[f"gemv_m{m}"] = row
    del w
    mat = wl.workload(5).matrices[0]
    tmap = mat.tile_map()
    w = hb.bits_to_tensor(mat.weight_bits(), mat.dtype, dev)
    m = 2048
    x = hb.bits_to_tensor(mat.activation_bits(m), mat.dtype, dev)
    y = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
    row = {}
    for name, meta, tm in (("idx2", "idx2", tmap), ("mask8", "mask8", tmap),
                           ("all_dense", "idx2", np.zeros_like(tmap))):
        Ps = [hb.pack(w, tm, mat.b1, mat.b2, meta) for _ in range(2)]
        torch.cuda.synchronize()
        us = graph_us(torch, lambda c: [hb.gemm(Ps[i % 2], x, out=y) for i in range(c)], 8)
        row[name] = {"us": round(us, 2), "dense_flops_TFLOPs": round(2 * m * mat.n * mat.k / (us * 1e-6) / 1e12, 1)}
        del Ps
        torch.cuda.empty_cache()
    out["gemm_m2048"] = row
    out["workloads"] = {"gemv": "Llama-3.1-8B up projection 14336x4096 bf16, 128x128 tiles, 2509/3584 sparse",
                        "gemm": "Qwen3-14B gate/up projection 17408x5120 bf16, 64x64 tiles, 13056/21760 sparse"}
    del w, x, y
    torch.cuda.empty_cache()
    return out


def grouped(hb, torch, wl, dev, meta):
    """Grouped decode launch (hyb_gemv_grouped) against separate launches on
    one Llama-3.1-8B decoder layer at M = 1: q, k, v (one x) and gate, up
    (another), each matrix with its own tile map and fraction.  Weights
    rotate over enough copies to leave the last-level cache cold."""
    W = wl.workload(3)
    groups = [[mt for mt in W.matrices if mt.name in names] for names in (("q", "k", "v"), ("gate", "up"))]
    mats = [mt for g in groups for mt in g]
    per_copy = 0
    packed = {}
    for mt in mats:
        w = hb.bits_to_tensor(mt.weight_bits(), mt.dtype, dev)
        packed[mt.name] = [hb.pack(w, mt.tile_map(), mt.b1, mt.b2, meta)]
        per_copy += packed[mt.name][0].weight_bytes()
        del w
    n_copies = copies_for(per_copy, 1 << 30)
    for mt in mats:
        w = hb.bits_to_tensor(mt.weight_bits(), mt.dtype, dev)
        packed[mt.name] += [hb.pack(w, mt.tile_map(), mt.b1, mt.b2, meta) for _ in range(n_copies - 1)]
        del w
    torch.cuda.synchronize()
    x = hb.bits_to_tensor(mats[0].activation_bits(1), "bf16", dev)
    outs = {mt.name: torch.empty((1, mt.n), dtype=torch.float32, device=dev) for mt in mats}

    def separate(count):
        for i in range(count):
            c = (3 * i) % n_copies
            for mt in mats:
                hb.gemv(packed[mt.name][c], x, out=outs[mt.name])

    def together(count):
        for i in range(count):
            c = (3 * i) % n_copies
            for g in groups:
                hb.gemv_grouped([packed[mt.name][c] for mt in g], x, outs=[outs[mt.name] for mt in g])

    reps = 2 * n_copies
    us_sep = graph_us(torch, separate, reps)
    us_grp = graph_us(torch, together, reps)
    alg = sum(alg_bytes(packed[mt.name][0].layout, 1) for mt in mats)
    out = {"workload": "Llama-3.1-8B decoder layer q, k, v (one x) and gate, up (another), "
                       "per-matrix tile fractions, M=1",
           "matrices": {mt.name: [mt.n, mt.k, int(packed[mt.name][0].layout.n_sparse)] for mt in mats},
           "launches": {"separate": len(mats), "grouped": len(groups)},
           "separate_us": round(us_sep, 3), "grouped_us": round(us_grp, 3),
           "speedup": round(us_sep / us_grp, 4), "alg_bytes": alg,
           "GBps_separate": round(alg / (us_sep * 1e-6) / 1e9, 1),
           "GBps_grouped": round(alg / (us_grp * 1e-6) / 1e9, 1),
           "timing": f"graph burst of {reps} layer passes over {n_copies} rotating copies, median of 5 replays"}
    del packed, outs
    torch.cuda.empty_cache()
    return out


def lowrank(hb, torch, wl, dev, meta, rank=64):
    """Sparse + low-rank decode (3BASiL, 2:4 sparse + rank 64) on the
    Llama-3.1-8B up projection at M = 1: the plain hybrid product of S
    against T = X V
    followed by the hybrid product with T U^T added in the same kernel.
    T comes from the projection kernel (V held transposed, 64 x 4096).
    S, V and U rotate over enough copies to leave the last-level cache cold;
    V and U are seeded normal draws scaled by 0.02."""
    mat = wl.workload(2).matrices[0]
    w = hb.bits_to_tensor(mat.weight_bits(), mat.dtype, dev)
    tmap = mat.tile_map()
    P0 = hb.pack(w, tmap, mat.b1, mat.b2, meta)
    gen = torch.Generator(device=dev)
    gen.manual_seed(64)
    def factors():
        v = (torch.randn((rank, mat.k), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        u = (torch.randn((mat.n, rank), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
        return v, u

    V0, U0 = factors()
    per_copy = P0.weight_bytes() + V0.numel() * 2 + U0.numel() * 2
    n_copies = copies_for(per_copy, 1 << 30)
    Ps, Vs, Us = [P0], [V0], [U0]
    for _ in range(n_copies - 1):
        Ps.append(hb.pack(w, tmap, mat.b1, mat.b2, meta))
        v_, u_ = factors()
        Vs.append(v_)
        Us.append(u_)
    del w
    torch.cuda.synchronize()
    x = hb.bits_to_tensor(mat.activation_bits(1), mat.dtype, dev)
    t = torch.empty((1, rank), dtype=torch.float32, device=dev)
    y = torch.empty((1, mat.n), dtype=torch.float32, device=dev)

    def plain(count):
        for i in range(count):
            hb.gemv(Ps[(3 * i) % n_copies], x, out=y)

    def two_launch(count):
        for i in range(count):
            c = (3 * i) % n_copies
            hb.lowrank_project(Vs[c], x, out=t)
            hb.gemv_lowrank(Ps[c], x, t, Us[c], out=y)

    def fused_only(count):
        for i in range(count):
            c = (3 * i) % n_copies
            hb.gemv_lowrank(Ps[c], x, t, Us[c], out=y)

    reps = 2 * n_copies
    us_plain = graph_us(torch, plain, reps)
    us_two = graph_us(torch, two_launch, reps)
    us_fused = graph_us(torch, fused_only, reps)
    b_plain = alg_bytes(P0.layout, 1)
    # projection: V + x read, T written; product: as plain plus U and T read
    b_lr = b_plain + V0.numel() * 2 + 2 * mat.k + 4 * rank + U0.numel() * 2 + 4 * rank
    out = {"workload": f"Llama-3.1-8B up projection {mat.n}x{mat.k} bf16 hybrid S ({P0.layout.n_sparse}/"
                       f"{P0.layout.tiles_n * P0.layout.tiles_k} tiles 2:4) + rank {rank} U V^T, M=1",
           "rank": rank, "plain_us": round(us_plain, 3), "sparse_lowrank_us": round(us_two, 3),
           "lowrank_kernel_us": round(us_fused, 3), "t_kernel_us_by_difference": round(us_two - us_fused, 3),
           "overhead_vs_plain": round(us_two / us_plain, 4),
           "alg_bytes": {"plain": b_plain, "sparse_lowrank": b_lr},
           "GBps_plain": round(b_plain / (us_plain * 1e-6) / 1e9, 1),
           "GBps_sparse_lowrank": round(b_lr / (us_two * 1e-6) / 1e9, 1),
           "timing": f"graph burst of {reps} products over {n_copies} rotating copies, median of 5 replays"}
    del Ps, Vs, Us
    torch.cuda.empty_cache()
    # prefill: the Qwen3-14B gate/up projection at M = 2048 with rank 64
    mat = wl.workload(5).matrices[0]
    m = 2048
    w = hb.bits_to_tensor(mat.weight_bits(), mat.dtype, dev)
    Ps = [hb.pack(w, mat.tile_map(), mat.b1, mat.b2, meta) for _ in range(2)]
    del w
    Vs, Us = [], []
    for _ in range(2):
        Vs.append((torch.randn((rank, mat.k), generator=gen, device=dev) * 0.02).to(torch.bfloat16))
        Us.append((torch.randn((mat.n, rank), generator=gen, device=dev) * 0.02).to(torch.bfloat16))
    x = hb.bits_to_tensor(mat.activation_bits(m), mat.dtype, dev)
    t = torch.empty((m, rank), dtype=torch.float32, device=dev)
    y = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    n_launch = 8
    us_g = graph_us(torch, lambda c: [hb.gemm(Ps[i % 2], x, out=y) for i in range(c)], n_launch)
    us_p = graph_us(torch, lambda c: [hb.lowrank_project(Vs[i % 2], x, out=t) for i in range(c)], n_launch)
    us_l = graph_us(torch, lambda c: [hb.gemm_lowrank(Ps[i % 2], x, t, Us[i % 2], out=y) for i in range(c)], n_launch)
    out["prefill"] = {"workload": f"Qwen3-14B gate/up projection {mat.n}x{mat.k} bf16 hybrid + rank {rank}, M={m}",
                      "gemm_us": round(us_g, 2), "project_us": round(us_p, 2), "gemm_lowrank_us": round(us_l, 2),
                      "update_us_by_difference": round(us_l - us_g, 2),
                      "sparse_lowrank_total_us": round(us_p + us_l, 2),
                      "overhead_vs_gemm": round((us_p + us_l) / us_g, 4),
                      "timing": f"graph burst of {n_launch} launches over 2 copies, median of 5 replays"}
    del Ps, Vs, Us, x, t, y
    torch.cuda.empty_cache()
    return out


def sweep(hb, torch, wl, dev, rotate, args):
    """All workloads: GEMV / GEMM time against the same kernel all-dense
    (graph bursts over rotating copies, as the main measurement)."""
    results = []

    def timed(fn, copies):
        # graph burst of 2C launches over the C rotating copies
        n = len(copies)
        return graph_us(torch, lambda c: [fn(copies[(3 * i) % n]) for i in range(c)], 2 * n)

    for cfg in (1, 2, 3, 4, 5):
        W = wl.workload(cfg)
        for mat in W.matrices:
            tmap = mat.tile_map()
            for kind, mp in (("hybrid", tmap), ("dense", np.zeros_like(tmap))):
                if cfg == 4 and kind == "dense":
                    continue  # the 0%-sparse case is the dense baseline
                log(f"[sweep] config {cfg} {mat.name} {kind}")
                w_, _, copies = setup_matrix(hb, torch, mat, mp, "idx2", rotate, dev)
                del w_
                L = copies[0].layout
                for m in W.batches:
                    x = hb.bits_to_tensor(mat.activation_bits(m), mat.dtype, dev)
                    y = torch.empty((m, mat.n), dtype=torch.float32, device=dev)
                    # hyb_gemm through the binding: a route that splits K takes its
                    # workspace from torch's allocator, which the captured graph
                    # keeps (the library-held workspace of hyb_gemm_mfma is not
                    # allocated under capture, so its split routes would run
                    # unsplit here)
                    fns = [("gemm", lambda P: hb.gemm(P, x, out=y))]
                    for fname, fn in fns:
                        us = timed(fn, copies)
                        results.append({"config": cfg, "matrix": mat.name, "kind": kind, "m": m, "fn": fname,
                                        "us": round(us, 3), "alg_bytes": alg_bytes(L, m),
                                        "GBps": round(alg_bytes(L, m) / us / 1e3, 1),
                                        "alg_flops": alg_flops(L, m),
                                        "TFLOPs": round(alg_flops(L, m) / us / 1e6, 2),
                                        "n_sparse": L.n_sparse, "tiles": L.tiles_n * L.tiles_k})
                        log(f"  m={m:5d} {fname:9s} {kind:6s} {us:9.2f} us  {results[-1]['GBps']:8.1f} GB/s  "
                            f"{results[-1]['TFLOPs']:7.2f} TF/s")
                del copies
                torch.cuda.empty_cache()
    path = args.sweep_json or os.path.join(HERE, "gpurun_out", "sweep.json")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(results, f, indent=1)
    return path


if __name__ == "__main__":
    main()
