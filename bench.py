#!/usr/bin/env python3
"""Benchmark: Lloyd iterations/s of exact batched K-Means on one MI355X.

One step = one Lloyd iteration over the whole batch: centroid norms,
FlashAssign, sort-inverse update (histogram, scan, inverse permutation,
segment reduction, finalize). The timed region is one fk_lloyd call running
exactly --steps iterations (tol = 0) on inputs already resident in HBM,
bracketed by device synchronisations. Per-phase GPU times come from HIP
events the library records on the same stream during that call.

Default workload: B=32, N=75600, d=128, K=1000, fp16 (the API example shape),
i.i.d. N(0,1) points, K random points per problem as initial centroids.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_F16 = 2500.0       # TFLOP/s, dense fp16/bf16
PEAK_HBM = 8000.0            # GB/s
PEAK_MFMA_F32 = 157.3        # TFLOP/s, dense fp32 MFMA
METRIC = "Lloyd iter/s + assign/update ms at B32 N75600 K1000 d128 fp16; % MFMA/HBM peak"
WORKLOADS = ("api_example", "io_breakdown", "large_k_zipf", "split_d", "tiny_f32")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def assign_flop(B, N, d, K) -> float:
    return 2.0 * B * N * K * d


def assign_bytes(B, N, d, K, s) -> float:
    # reads X and the centroid copy once, writes ids once (+ norms)
    return B * (N * d * s + K * d * s + 4 * N + 4 * K)


def update_bytes(B, N, d, K, s) -> float:
    # x gathered once; ids read twice, perm written and read; sums written and
    # read, old centroids read, new written; counts/offsets
    return B * N * d * s + 16.0 * B * N + 16.0 * B * K * d + 16.0 * B * K


def measured_traffic(workload: str, phase: str):
    """HBM bytes per launch of one phase from the committed rocprofv3 counter
    table, if it was taken on the current kernel source; else None."""
    from exact_means_clustering_flashassign_amd.profiling import source_digest

    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = (t.get(workload) or {}).get(phase)
    if not e or e.get("kernel_source_digest") != source_digest(phase):
        return None
    return e.get("hbm_bytes_per_launch")


# Oracle sample per workload: (problems, rows per problem); None = all rows.
CPU_SAMPLE = {"tiny_f32": (1, None), "api_example": (32, None), "io_breakdown": (32, None),
              "large_k_zipf": (1, 1 << 17), "split_d": (8, None)}


def cpu_baseline(w, name: str, min_seconds: float = 10.0):
    """The oracle, untuned, on a bounded sample of the workload: one Lloyd
    iteration over the first problems and rows of CPU_SAMPLE, repeated until
    about min_seconds of CPU time have passed, scaled to the whole batch."""
    import numpy as np
    import oracle
    import synthdata

    # every host core the process may run on, with the BLAS pool set to that
    # many threads
    cores = len(os.sched_getaffinity(0))
    blas = "unknown"
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            cores = max(p.get("num_threads", cores) for p in info)
    except Exception:  # pragma: no cover
        pass
    nb, rows = CPU_SAMPLE[name]
    nb, rows = min(nb, w.B), min(rows or w.N, w.N)
    x64 = synthdata.to_f64(np.ascontiguousarray(w.x[:nb, :rows]), w.dtype)
    c0 = w.init64()[:nb]
    total, reps = 0.0, 0
    while reps == 0 or (total < min_seconds and reps < 50):
        t0 = time.perf_counter()
        oracle.lloyd(x64, c0, 1, 0.0, w.dtype, want_near=False)
        total += time.perf_counter() - t0
        reps += 1
    if limiter is not None:
        limiter.restore_original_limits()
    per_iter_full = total / reps * (w.B / nb) * (w.N / rows)
    part = f"{nb} of the {w.B} problems" + ("" if rows == w.N else f", first {rows} of {w.N} rows")
    return {"value": 1.0 / per_iter_full, "unit": "iter/s", "cores": int(cores),
            "kind": "oracle", "blas": blas,
            "sample": f"1 Lloyd iteration on {part} (full K, d), fp64 NumPy on the host, "
                      f"{reps} run(s) in {total:.1f} s, scaled by problems and rows to the whole batch"}


def gpu_baselines(fk, torch, x, ids, centers, ws, dtype: str, reps: int = 3):
    """The standard formulations the method replaces, timed on the same inputs.

    Materialised-distance assign (rocBLAS GEMM into a (B,N,K) fp32 matrix,
    then an argmin pass) against fk_assign, and the scatter-atomic update
    against fk_update, each called on its own (HIP events on torch's current
    stream, where both libraries enqueue). Skipped when the distance matrix
    would take more than 48 GiB."""
    B, N, d = x.shape
    K = centers.shape[1]
    if B * N * K * 4 > 48 * 2**30:
        return {"skipped": f"the (B,N,K) fp32 distance matrix would take "
                           f"{B * N * K * 4 / 2**30:.0f} GiB"}
    fk.load_baseline()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    c_lp, cn = fk.fk_norms(centers, x.dtype)
    dist = torch.empty((B, N, K), dtype=torch.float32, device=x.device)
    ids_b = torch.empty_like(ids)
    mat_ms = timed(lambda: fk.fkb_assign_materialized(x, c_lp, cn, dist=dist, ids=ids_b))
    flash_ms = timed(lambda: fk.fk_assign(x, c_lp, cn, ids=ids_b))
    del dist
    torch.cuda.empty_cache()
    c_tmp = centers.clone()
    counts = torch.empty((B, K), dtype=torch.int32, device=x.device)
    sums = torch.empty((B, K, d), dtype=torch.float32, device=x.device)
    shift = torch.empty((B,), dtype=torch.float32, device=x.device)
    atomic_ms = timed(lambda: fk.fkb_update_atomic(x, ids, c_tmp, counts=counts, sums=sums))
    sort_ms = timed(lambda: fk.fk_update(x, ids, c_tmp, counts=counts, shift=shift, ws=ws))
    x_bytes = B * N * d * elem_bytes(dtype)
    return {"assign_materialized_ms": mat_ms, "assign_flash_ms": flash_ms,
            "assign_speedup": mat_ms / flash_ms,
            "update_scatter_atomic_ms": atomic_ms, "update_sort_inverse_ms": sort_ms,
            "update_speedup": atomic_ms / sort_ms,
            "scatter_atomic_effective_GBps": x_bytes / (atomic_ms * 1e-3) / 1e9,
            "note": "each call on its own, same inputs; fk_update here also computes the shift"}


PEAK_PCIE = 64.0   # GB/s, PCIe 5.0 x16, one direction


def host_stream(fk, torch, synthdata, w, args):
    """fk_lloyd_host on the workload with x in page-locked host memory: every
    iteration streams all of x over PCIe, so the bound is the host link."""
    dev = torch.device("cuda:0")
    xh = synthdata.to_torch(w.x, w.dtype).contiguous().pin_memory()
    init = synthdata.to_torch(w.init, w.dtype).to(dev)
    B, N, d, K = w.B, w.N, w.d, w.K
    ids = torch.empty((B, N), dtype=torch.int32, device=dev)
    centers = torch.empty((B, K, d), dtype=torch.float32, device=dev)
    n = fk.fk_workspace_size_host(xh.dtype, B, args.host_stream, d, K)
    raw = torch.empty(n + 256, dtype=torch.uint8, device=dev)
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + n]
    if args.warmup > 0:
        fk.fk_lloyd_host(xh, init, args.warmup, 0.0, args.host_stream, ids, centers, ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, _, n_iter = fk.fk_lloyd_host(xh, init, args.steps, 0.0, args.host_stream, ids, centers, ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    assert n_iter == args.steps
    x_bytes = B * N * d * elem_bytes(w.dtype)
    gbps = x_bytes * args.steps / elapsed / 1e9
    out = {
        "metric": METRIC, "value": args.steps / elapsed, "unit": "iter/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload} host-streamed: B={B} N={N} d={d} K={K} "
                               f"{w.dtype}, x in page-locked host memory, {args.host_stream} "
                               f"points per problem per copy, {args.steps} Lloyd iterations, "
                               "tol=0",
                   "B": B, "N": N, "d": d, "K": K, "chunk": args.host_stream},
        "roofline": {"bound": "pcie", "achieved": gbps, "peak": PEAK_PCIE, "unit": "GB/s",
                     "frac": gbps / PEAK_PCIE, "traffic": None,
                     "kernel": "host-to-device copies of x (the Lloyd kernels overlap them)"},
        "cpu_baseline": None,
    }
    print(json.dumps(out))


def host_sweep(fk, torch, synthdata, args):
    """The large-tensor sweep's shapes: one problem of fp32 points, d = 128,
    N = 2^e and K = sqrt(N), the points i.i.d. standard normal in page-locked
    host memory ("flash-kmeans and the return of exact K-Means on the GPU",
    section "The benchmark compares against four other implementations, on one
    GPU", the large-tensor paragraph). For each size: the Lloyd loop with x streamed over
    PCIe every iteration (fk_lloyd_host), and the device-resident loop on the
    same inputs (fk_lloyd) with its assign and update times. One JSON line per
    size."""
    dev = torch.device("cuda:0")
    for e in [int(v) for v in args.host_sweep.split(",")]:
        if e % 2 or not 10 <= e <= 28:
            raise SystemExit(f"--host-sweep: exponents are even, 10..28 (got {e})")
        B, N, d, K = 1, 1 << e, 128, 1 << (e // 2)
        # drawn straight into page-locked memory, or into ordinary memory
        # where the driver cannot lock that much (2^28 points are 137 GB)
        try:
            xh = torch.empty((B, N, d), dtype=torch.float32, pin_memory=True)
            host_mem = "page-locked"
        except RuntimeError:
            xh = torch.empty((B, N, d), dtype=torch.float32)
            host_mem = "pageable"
        _, init, _ = synthdata.make_mixture(B, N, d, K, "f32", n_comp=0, mean_std=0.0,
                                            seed=3000 + e, iid=True, out=xh.numpy())
        print(f"# N=2^{e}: points ready", file=sys.stderr, flush=True)
        init_d = torch.from_numpy(init).to(dev)
        ids = torch.empty((B, N), dtype=torch.int32, device=dev)
        centers = torch.empty((B, K, d), dtype=torch.float32, device=dev)
        # at least four chunks, so copies overlap the kernels at every size
        chunk = args.host_stream if args.host_stream > 0 else min(1 << 20, max(N // 4, 1))
        chunk = min(N, chunk)
        n = fk.fk_workspace_size_host(xh.dtype, B, chunk, d, K)
        raw = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        off = (-raw.data_ptr()) % 256
        hws = raw[off:off + n]
        if args.warmup > 0:
            fk.fk_lloyd_host(xh, init_d, args.warmup, 0.0, chunk, ids, centers, hws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, _, n_iter = fk.fk_lloyd_host(xh, init_d, args.steps, 0.0, chunk, ids, centers, hws)
        torch.cuda.synchronize()
        t_host = time.perf_counter() - t0
        assert n_iter == args.steps
        print(f"# N=2^{e}: host-streamed loop done", file=sys.stderr, flush=True)
        del raw, hws
        xd = xh.to(dev)
        ws = fk.workspace(xd.dtype, B, N, d, K, dev)
        if args.warmup > 0:
            fk.fk_lloyd(xd, init_d, args.warmup, 0.0, ids=ids, centers=centers, ws=ws)
        torch.cuda.synchronize()
        fk.fk_trace_begin(args.steps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fk.fk_lloyd(xd, init_d, args.steps, 0.0, ids=ids, centers=centers, ws=ws)
        torch.cuda.synchronize()
        t_dev = time.perf_counter() - t0
        tr = fk.fk_trace_end()
        a_ms = tr["assign_ms"] / tr["iterations"]
        u_ms = tr["update_ms"] / tr["iterations"]
        gbps = B * N * d * 4 * args.steps / t_host / 1e9
        achieved = assign_flop(B, N, d, K) / (a_ms * 1e-3) / 1e12
        print(json.dumps({
            "metric": METRIC, "value": args.steps / t_host, "unit": "iter/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * t_host / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "data": "synthetic",
            "config": {"workload": f"large-tensor sweep: B=1 N=2^{e} d=128 K={K} f32 i.i.d. "
                                   f"normal, x in {host_mem} host memory, {chunk} points per "
                                   f"copy, {args.steps} Lloyd iterations, tol=0",
                       "B": B, "N": N, "d": d, "K": K, "chunk": chunk, "host_memory": host_mem},
            "pcie": {"achieved": gbps, "peak": PEAK_PCIE, "unit": "GB/s",
                     "frac": gbps / PEAK_PCIE},
            "device_resident": {"iter_s": args.steps / t_dev, "assign_ms": a_ms,
                                "update_ms": u_ms,
                                "assign_roofline": {"bound": "mfma", "achieved": achieved,
                                                    "peak": PEAK_MFMA_F32, "unit": "TFLOP/s",
                                                    "frac": achieved / PEAK_MFMA_F32}},
        }), flush=True)
        del xh, xd, ws, ids, centers, init_d
        torch.cuda.empty_cache()


def mfma_peak(fk, torch, args):
    """The MFMA peak probe: v_mfma_f32_32x32x16_f16 back to back on every SIMD
    (two waves per SIMD, random operands), the instruction and occupancy of
    the small-D assign. Reports the achieved TFLOP/s against the nominal dense
    fp16 peak and the shader clock the loop ran at (from the in-kernel clock
    counters). One JSON line."""
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus                      # 2 blocks of 4 waves per CU: 2 waves per SIMD
    iters = args.peak_iters
    fk.load_baseline()
    out, stamps = fk.fkb_mfma_peak(blocks, iters, 12345, device=dev)   # warm-up
    torch.cuda.synchronize()
    reps = max(args.steps, 1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for r in range(reps):
        fk.fkb_mfma_peak(blocks, iters, 1000 + r, out=out, stamps=stamps)
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flop = blocks * 4.0 * iters * 32 * 32768
    tflops = flop / (ms * 1e-3) / 1e12
    st = stamps.cpu().numpy().astype("float64")
    khz = fk.fkb_wall_clock_khz()
    ticks = st[:, 1] - st[:, 0]
    real = st[:, 3] - st[:, 2]
    clock_mhz = float((ticks / real).mean() * khz / 1e3) if khz > 0 and (real > 0).all() else None
    print(json.dumps({
        "metric": "MFMA peak probe (v_mfma_f32_32x32x16_f16, random operands)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"mfma peak probe: {blocks} blocks x 4 waves, {iters} x 32 MFMAs "
                               "per wave, 8 accumulator chains", "blocks": blocks,
                   "iters": iters, "cus": cus},
        "frac_of_nominal": tflops / PEAK_MFMA_F16,
        "shader_clock_mhz": clock_mhz,
        "wall_clock_khz": khz,
        "frac_of_peak_at_measured_clock": (tflops / (PEAK_MFMA_F16 * clock_mhz / 2400.0)
                                           if clock_mhz else None),
    }), flush=True)


def contention(fk, torch, synthdata, args):
    """The update under contention: the large-K shape (B=1, N=2^24, d=128,
    K=32768, fp16) with cluster ids drawn from Zipf(1.1) (hot clusters: the
    hottest holds about 2.4M points) against uniform ids (the control), each
    updated by the sort-inverse fk_update and by the one-atomic-per-element
    scatter update (libfkbaseline). Update-only: the same x and ids for every
    call, HIP events on torch's current stream. One JSON line."""
    dev = torch.device("cuda:0")
    w = synthdata.make_workload("large_k_zipf")
    B, N, d, K = w.B, w.N, w.d, w.K
    x = synthdata.to_torch(w.x, w.dtype).to(dev)
    fk.load_baseline()
    c0 = synthdata.to_torch(w.init, w.dtype).to(dev).float()
    ws = fk.workspace(x.dtype, B, N, d, K, dev)
    counts = torch.empty((B, K), dtype=torch.int32, device=dev)
    sums = torch.empty((B, K, d), dtype=torch.float32, device=dev)
    shift = torch.empty((B,), dtype=torch.float32, device=dev)
    reps = max(args.steps, 1)
    x_bytes = B * N * d * elem_bytes(w.dtype)
    u_bytes = update_bytes(B, N, d, K, elem_bytes(w.dtype))

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    rows = {}
    for kind, ids_np in (("zipf1.1", synthdata.zipf_ids(B, N, K, seed=7)),
                         ("uniform", synthdata.uniform_ids(B, N, K, seed=7))):
        ids = torch.from_numpy(ids_np).to(dev)
        hot = int(torch.bincount(ids.view(-1).long(), minlength=K).max().item())
        c = c0.clone()
        sort_ms = timed(lambda: fk.fk_update(x, ids, c, counts=counts, shift=shift, ws=ws))
        atomic_ms = timed(lambda: fk.fkb_update_atomic(x, ids, c, counts=counts, sums=sums))
        rows[kind] = {"hottest_cluster_points": hot,
                      "sort_inverse_ms": sort_ms, "scatter_atomic_ms": atomic_ms,
                      "speedup": atomic_ms / sort_ms,
                      "sort_inverse_frac_of_hbm": u_bytes / (sort_ms * 1e-3) / 1e9 / PEAK_HBM,
                      "scatter_atomic_effective_GBps": x_bytes / (atomic_ms * 1e-3) / 1e9}
        del ids
    z = rows["zipf1.1"]
    print(json.dumps({
        "metric": "update under contention: sort-inverse vs scatter-atomic, ms per update",
        "value": z["sort_inverse_ms"], "unit": "ms", "n_gpus": 1, "steps": reps,
        "warmup": max(args.warmup, 1), "ms_per_step": z["sort_inverse_ms"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"large-K update: B={B} N={N} d={d} K={K} {w.dtype}, "
                               "Zipf(1.1) ids vs uniform ids", "B": B, "N": N, "d": d, "K": K},
        "variants": rows,
        "algorithmic_bytes_per_update": u_bytes,
    }), flush=True)


SMALL_TILES = ("8w128", "4w128", "4w64")
SPLIT_TILES = ("lds8", "lds4", "reg8", "reg4")


def tile_sweep(fk, torch, args):
    """Every assign tile candidate (FK_TILE) timed on a grid of shapes: the
    small-D tiles over d in {32, 64, 128} (fp16), the split-D tiles over d in
    {768, 1024} (bf16), K and the number of points. One JSON line per shape
    with each candidate's ms and the fastest; the dispatch table comes from
    these lines. Points and centroids are seeded N(0,1) draws (timing only)."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    grids = []
    for d in (32, 64, 128):
        for K in (64, 256, 1024, 4096):
            for B, N in ((1, 16384), (1, 65536), (4, 65536), (32, 75600)):
                grids.append(("f16", B, N, d, K, SMALL_TILES))
    for d in (768, 1024):
        for K in (64, 256, 1000):
            for B, N in ((1, 16384), (8, 32768)):
                grids.append(("bf16", B, N, d, K, SPLIT_TILES))
    reps = max(args.steps, 1)
    old = os.environ.get("FK_TILE")
    for dt, B, N, d, K, tiles in grids:
        tdt = torch.float16 if dt == "f16" else torch.bfloat16
        x = torch.randn((B, N, d), generator=gen, device=dev).to(tdt)
        c = torch.randn((B, K, d), generator=gen, device=dev)
        c_lp, cn = fk.fk_norms(c, tdt)
        ids = torch.empty((B, N), dtype=torch.int32, device=dev)
        row = {}
        for t in tiles:
            os.environ["FK_TILE"] = t
            fk.fk_assign(x, c_lp, cn, ids=ids)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fk.fk_assign(x, c_lp, cn, ids=ids)
            e1.record()
            e1.synchronize()
            row[t] = e0.elapsed_time(e1) / reps
        best = min(row, key=row.get)
        print(json.dumps({"dtype": dt, "B": B, "N": N, "d": d, "K": K, "ms": row, "best": best,
                          "tflops_best": assign_flop(B, N, d, K) / (row[best] * 1e-3) / 1e12}),
              flush=True)
        del x, c, c_lp, cn, ids
    if old is None:
        os.environ.pop("FK_TILE", None)
    else:
        os.environ["FK_TILE"] = old


def shard_step(fk, torch, synthdata, args):
    """One GPU's part of a data-parallel iteration at the workload's shape:
    N / shards rows of every problem (the recipe at the shard's size: a
    contiguous block, as each GPU would hold), full K: norms, assign, and the shard-local update that
    adds per-cluster sums and counts undivided (fk_update_partial), the
    input of one all-reduce of K*d + K values per problem. One JSON line."""
    dev = torch.device("cuda:0")
    N0 = synthdata.SHAPES[args.workload][1]
    w = synthdata.make_workload(args.workload, scale_n=N0 // args.shard)   # the shard's rows
    B, N, d, K = w.B, w.N, w.d, w.K
    x = synthdata.to_torch(w.x, w.dtype).to(dev)
    c = synthdata.to_torch(w.init, w.dtype).to(dev).float()
    ids = torch.empty((B, N), dtype=torch.int32, device=dev)
    sums = torch.empty((B, K, d), dtype=torch.float32, device=dev)
    counts = torch.empty((B, K), dtype=torch.int32, device=dev)
    ws = fk.workspace(x.dtype, B, N, d, K, dev)
    reps = max(args.steps, 1)

    def step():
        c_lp, cn = fk.fk_norms(c, x.dtype)
        fk.fk_assign(x, c_lp, cn, ids=ids)
        sums.zero_()
        counts.zero_()
        fk.fk_update_partial(x, ids, sums, counts, ws=ws)

    def timed(fn):
        for _ in range(max(args.warmup, 1)):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps

    c_lp, cn = fk.fk_norms(c, x.dtype)
    a_ms = timed(lambda: fk.fk_assign(x, c_lp, cn, ids=ids))
    u_ms = timed(lambda: fk.fk_update_partial(x, ids, sums, counts, ws=ws))
    s_ms = timed(step)
    s_el = elem_bytes(w.dtype)
    flop = assign_flop(B, N, d, K)
    print(json.dumps({
        "metric": "one shard's step: norms + assign + partial-sum update, ms",
        "value": s_ms, "unit": "ms", "n_gpus": 1, "steps": reps, "warmup": max(args.warmup, 1),
        "ms_per_step": s_ms, "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}, shard 1 of {args.shard}: B={B} N={N} d={d} "
                               f"K={K} {w.dtype}", "B": B, "N": N, "d": d, "K": K,
                   "shards": args.shard},
        "assign_ms": a_ms, "assign_tflops": flop / (a_ms * 1e-3) / 1e12,
        "assign_frac_of_mfma_peak": flop / (a_ms * 1e-3) / 1e12 / PEAK_MFMA_F16,
        "partial_update_ms": u_ms,
        "partial_update_frac_of_hbm": update_bytes(B, N, d, K, s_el) / (u_ms * 1e-3) / 1e9 /
        PEAK_HBM,
        "allreduce_payload_bytes": B * (K * d + K) * 4,
    }), flush=True)


def copy_calibration(mib: int, dev):
    """A plain elementwise kernel over a buffer of known size, for scaling
    the HBM byte counters (reads and writes mib MiB each)."""
    import torch

    src = torch.empty(mib * 2**18, dtype=torch.float32, device=dev).uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="api_example", choices=WORKLOADS)
    ap.add_argument("--cpu-batches", type=int, default=1,
                    help="1 = time the oracle on its bounded sample, 0 = skip")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MiB",
                    help="after the timed region, run a copy kernel of this size (counter scaling)")
    ap.add_argument("--host-stream", type=int, default=0, metavar="CHUNK",
                    help="keep x in page-locked host memory and run fk_lloyd_host, streaming "
                         "CHUNK points per problem per copy (0 = the device-resident loop)")
    ap.add_argument("--host-sweep", default="", metavar="E,E,...",
                    help="instead: the large-tensor sweep (fp32, d=128, N=2^E, K=2^(E/2)), "
                         "host-streamed and device-resident, one line per size; CHUNK from "
                         "--host-stream (default min(2^20, N/4))")
    ap.add_argument("--tol-run", type=int, default=1,
                    help="1 = after the timed region, time the workload's own tol-stopped run "
                         "(workloads whose recipe has tol > 0), 0 = skip")
    ap.add_argument("--baselines", type=int, default=1,
                    help="1 = after the timed region, time the materialised-distance assign and "
                         "the scatter-atomic update on the same inputs, 0 = skip")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="instead: the MFMA peak probe (--steps timed launches)")
    ap.add_argument("--peak-iters", type=int, default=20000,
                    help="loop iterations (32 MFMAs each) per wave of the MFMA peak probe")
    ap.add_argument("--shard", type=int, default=0, metavar="S",
                    help="instead: one shard's step (N/S rows per problem, full K) of the workload: "
                         "norms, assign and the partial-sum update")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="instead: every assign tile candidate timed over a grid of shapes "
                         "(one JSON line per shape)")
    ap.add_argument("--contention", action="store_true",
                    help="instead: the update under contention at the large-K shape (Zipf(1.1) "
                         "ids against uniform ids, sort-inverse against scatter-atomic)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every box here has one GPU).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthdata
    import exact_means_clustering_flashassign_amd as fk

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    fk.load()
    dev = torch.device("cuda:0")
    if args.mfma_peak:
        mfma_peak(fk, torch, args)
        return
    if args.host_sweep:
        host_sweep(fk, torch, synthdata, args)
        return
    if args.contention:
        contention(fk, torch, synthdata, args)
        return
    if args.tile_sweep:
        tile_sweep(fk, torch, args)
        return
    if args.shard > 0:
        shard_step(fk, torch, synthdata, args)
        return
    w = synthdata.make_workload(args.workload)
    if args.host_stream > 0:
        host_stream(fk, torch, synthdata, w, args)
        return
    x = synthdata.to_torch(w.x, w.dtype).to(dev)
    init = synthdata.to_torch(w.init, w.dtype).to(dev)
    B, N, d, K = w.B, w.N, w.d, w.K
    ids = torch.empty((B, N), dtype=torch.int32, device=dev)
    centers = torch.empty((B, K, d), dtype=torch.float32, device=dev)
    ws = fk.workspace(x.dtype, B, N, d, K, dev)

    if args.warmup > 0:
        fk.fk_lloyd(x, init, args.warmup, 0.0, ids=ids, centers=centers, ws=ws)
    torch.cuda.synchronize()
    fk.fk_trace_begin(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    _, _, n_iter = fk.fk_lloyd(x, init, args.steps, 0.0, ids=ids, centers=centers, ws=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    tr = fk.fk_trace_end()
    assert n_iter == args.steps and tr["iterations"] == args.steps

    elapsed = t1 - t0
    ms_step = 1e3 * elapsed / args.steps
    s = elem_bytes(w.dtype)
    a_ms = tr["assign_ms"] / tr["iterations"]
    u_ms = tr["update_ms"] / tr["iterations"]
    n_ms = tr["norms_ms"] / tr["iterations"]
    flop = assign_flop(B, N, d, K)
    a_bytes = assign_bytes(B, N, d, K, s)
    u_bytes = update_bytes(B, N, d, K, s)
    if w.dtype == "f32":     # fp32 MFMA; compute-bound unless K is tiny
        bound, peak, unit = "mfma", PEAK_MFMA_F32, "TFLOP/s"
        achieved = flop / (a_ms * 1e-3) / 1e12
    elif flop / a_bytes > PEAK_MFMA_F16 * 1e12 / (PEAK_HBM * 1e9):
        bound, peak, unit = "mfma", PEAK_MFMA_F16, "TFLOP/s"
        achieved = flop / (a_ms * 1e-3) / 1e12
    else:
        bound, peak, unit = "hbm", PEAK_HBM, "GB/s"
        achieved = a_bytes / (a_ms * 1e-3) / 1e9
    traffic = measured_traffic(args.workload, "assign")
    u_traffic = measured_traffic(args.workload, "update")
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration, dev)
    out = {
        "metric": METRIC,
        "value": args.steps / elapsed,
        "unit": "iter/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={B} N={N} d={d} K={K} {w.dtype}, "
                               f"{args.steps} Lloyd iterations, tol=0",
                   "B": B, "N": N, "d": d, "K": K},
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": "assign (FlashAssign)"},
        "phases_ms": {"norms": n_ms, "assign": a_ms, "update": u_ms},
        "update_roofline": {"bound": "hbm", "achieved": u_bytes / (u_ms * 1e-3) / 1e9,
                            "peak": PEAK_HBM, "unit": "GB/s",
                            "frac": u_bytes / (u_ms * 1e-3) / 1e9 / PEAK_HBM,
                            "traffic": u_traffic},
    }
    if args.tol_run > 0 and getattr(w, "tol", 0.0) > 0:
        # the recipe's own stop rule (up to 100 iterations): time to solution
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        _, _, n_tol = fk.fk_lloyd(x, init, 100, float(w.tol), ids=ids, centers=centers, ws=ws)
        torch.cuda.synchronize()
        t_tol = time.perf_counter() - t2
        out["tol_run"] = {"tol": float(w.tol), "max_iter": 100, "n_iter": n_tol,
                          "ms": 1e3 * t_tol, "ms_per_iter": 1e3 * t_tol / max(n_tol, 1)}
    out["gpu_baselines"] = (gpu_baselines(fk, torch, x, ids, centers, ws, w.dtype)
                            if args.baselines > 0 else None)
    out["cpu_baseline"] = cpu_baseline(w, args.workload) if args.cpu_batches > 0 else None
    print(json.dumps(out))


if __name__ == "__main__":
    main()
