#!/usr/bin/env python3
"""Throughput of the k-means assignment step on one MI355X.

One step = the whole hot path on one seeded input set: the centroid-norm
pre-pass (``kmeans_centroid_norms``) followed by ``kmeans_assign``, with the
three seeded sets (17, 29, 43) resident in HBM and rotated between steps
(flashlib PR #22, nightly-comparison section, "Benchmark methodology":
rotating seeded bf16 sets, warmup calls, then timed calls).

Before the warmup steps the step runs untimed for ``--settle-ms`` (250 ms):
the first milliseconds after idle run at lower clocks.  Prints one JSON line.
``value`` = points assigned per second over the timed steps (GPU-event time,
inputs already on the device).  ``roofline`` reports
the assign kernel against the bf16 dense MFMA peak, with its average launch
duration measured by HIP events on the launch stream.  ``mfma_ceiling`` is
the rate of the same MFMA issued back to back on this workload's operand
values (no memory, no epilogue): what the matrix pipe sustains on this data,
against which ``roofline.achieved`` is also read.  ``cpu_baseline`` times the
CPU oracle on a bounded sample of the same workload; the same leg checks the
outputs of the timed calls against the oracle (``parity``: the last timed
call on each seeded set, on the points that oracle run covered for the first
set and the first 2048 points of the others) and exits non-zero, after
printing the line, if any point fails the acceptance rule.
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

from means_nearest_centroid_amd import workloads as W  # noqa: E402

METRIC = "points assigned/sec + % bf16 MFMA peak at N=262144,D=128,K=4096 (1 GPU)"
BF16_DENSE_PEAK_TFLOPS = 2516.6     # MI355X: 256 CU x 4096 flop/clk x 2.4 GHz
KERNEL_SOURCES = ("means_nearest_centroid_amd/csrc/kmeans_kernels.hip",
                  "means_nearest_centroid_amd/csrc/kmeans_internal.h",
                  "means_nearest_centroid_amd/csrc/kmeans_api.hip")
# The update's kernels are built from these alone (kmeans_kernels.hip and
# the host-side kmeans_api.hip play no part in them).
UPDATE_SOURCES = ("means_nearest_centroid_amd/csrc/kmeans_update.hip",
                  "means_nearest_centroid_amd/csrc/kmeans_update_internal.h",
                  "means_nearest_centroid_amd/csrc/kmeans_internal.h")
HBM_PEAK_GBS = 8000.0               # MI355X HBM3E


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic_path(config: int, kind: str) -> str:
    return os.path.join(ROOT, "profiles", f"hbm_traffic_{kind}_workload{config}.json")


def traffic_record(config: int, kind: str = "assign"):
    """HBM bytes per assign launch (or per update call) from the committed
    counter summary, if it was taken on the current kernel sources; else None."""
    path = _traffic_path(config, kind)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sources = UPDATE_SOURCES if kind == "update" else KERNEL_SOURCES
    if rec.get("kernel_source_hash") != kernel_source_hash(sources):
        return None
    return rec


# Record kind of the assign launch's traffic: the automatic dispatch's, or a
# forced path's ("assign_persistent" for the queue kernel).
ASSIGN_PATH_NAMES = {0: "automatic", 1: "direct", 2: "split", 3: "persistent"}


def assign_traffic_kind(assign_path: int) -> str:
    return "assign" if assign_path == 0 else f"assign_{ASSIGN_PATH_NAMES[assign_path]}"


def _kernel_kind(name: str):
    if "assign_kernel" in name or "assign_queue_kernel" in name:
        return "assign"
    if "merge_kernel" in name:
        return "merge"
    if "neg_kernel" in name:
        return "copy"
    if "upd_" in name:
        return "update"
    return None


def _counter_per_dispatch(csv_path: str, counter: str):
    """Per kernel kind (assign, merge, calibration copy, and the update's
    kernels together), the counter's total over all dispatches and the number
    of dispatches, from a rocprofv3 --pmc counter_collection.csv; for the
    update, the dispatches of its last kernel (one per call: the finish kernel
    of the sort path or either bucket kernel)."""
    import csv
    import collections
    tot = collections.defaultdict(float)
    disp = collections.defaultdict(set)
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            name = row["Kernel_Name"]
            kind = _kernel_kind(name)
            if kind is None:
                continue
            tot[kind] += float(row["Counter_Value"])
            if kind != "update" or any(k in name for k in ("upd_finish_kernel", "upd_bucket_kernel",
                                                            "upd_bucket_runs_kernel")):
                disp[kind].add(row["Dispatch_Id"])
    return {k: tot[k] / len(disp[k]) for k in tot}


def record_traffic(config: int, fetch_csv: str, write_csv: str, copy_mib: int, command: str,
                   kind: str = "assign"):
    """Write the HBM-traffic record bench.py reports: counter KiB per assign
    launch (or per update call, all its kernels), scaled by what the same
    counter reads for a plain copy of known size (copy_mib MiB read and
    written)."""
    fetch = _counter_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _counter_per_dispatch(write_csv, "WRITE_SIZE")
    known = copy_mib * 1024.0                       # KiB read, and written, by the copy
    f_scale = known / fetch["copy"]
    w_scale = known / write["copy"]
    if kind == "update":
        kib_assign = fetch["update"]
        kib_assign_w = write["update"]
    else:
        kib_assign = fetch["assign"] + fetch.get("merge", 0.0)
        kib_assign_w = write["assign"] + write.get("merge", 0.0)
    rec = dict(
        workload=config,
        step=kind,
        kernel_source_hash=kernel_source_hash(UPDATE_SOURCES if kind == "update"
                                              else KERNEL_SOURCES),
        fetch_kib_per_launch=kib_assign,
        write_kib_per_launch=kib_assign_w,
        copy_fetch_kib=fetch["copy"], copy_write_kib=write["copy"], copy_kib=known,
        fetch_scale=f_scale, write_scale=w_scale,
        hbm_bytes_per_launch=int(round((kib_assign * f_scale + kib_assign_w * w_scale) * 1024)),
        command=command,
    )
    path = _traffic_path(config, kind)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


# B200 latencies (ms) of the pages' PR path for the 13 sweep shapes
# (flashlib PR #22, nightly comparison, "Benchmark results" table): another
# GPU's numbers, printed beside ours as context only.
PAGES_B200_PR_MS = {
    (65536, 64, 512): 0.0441, (65536, 64, 4096): 0.1022, (65536, 64, 16384): 0.2963,
    (65536, 128, 512): 0.0453, (65536, 128, 4096): 0.1059,
    (262144, 128, 4096): 0.2844, (262144, 128, 16384): 1.0047, (1048576, 128, 4096): 1.0148,
    (65536, 256, 512): 0.0587, (65536, 256, 4096): 0.1661,
    (262144, 256, 4096): 0.4631, (262144, 256, 16384): 1.8615, (1048576, 256, 4096): 1.9458,
}


def run_sweep(args):
    """The pages' 13-shape benchmark: per shape, three seeded sets resident
    and rotated, ``args.settle_ms`` of untimed calls, ``args.warmup``
    untimed calls, then three rounds of ``args.steps`` back-to-back
    ``kmeans_assign`` calls, each round bracketed by HIP events on the launch
    stream (no event between calls: one costs 3-4 us of stream time); the
    median of the rounds' per-call times; one JSON line per shape, then a
    geometric-mean line."""
    import torch
    import means_nearest_centroid_amd as km
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    km.load_library()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    lat_ms, ref_ms = [], []
    for (N, D, K) in W.SWEEP_SHAPES:
        print(f"[sweep] N={N} D={D} K={K}: generating", file=sys.stderr, flush=True)
        sets = []
        for seed in W.SEEDS:
            X, C, _ = W.gaussian_mixture(N, D, K, seed)
            Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev)
            Cd = torch.from_numpy(C.view(np.int16)).view(torch.bfloat16).to(dev)
            sets.append((Xd, Cd, km.kmeans_centroid_norms(Cd, stream=stream)))
            del X, C
        labels = torch.empty(N, dtype=torch.int32, device=dev)
        min_dist = torch.empty(N, dtype=torch.float32, device=dev)

        def call(i):
            X, C, n = sets[i % 3]
            km.kmeans_assign(X, C, n, labels, min_dist, stream=stream)

        settle(call, args.settle_ms)
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        rounds = []
        for _ in range(3):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.steps):
                call(i)
            e1.record(stream)
            torch.cuda.synchronize()
            rounds.append(e0.elapsed_time(e1) / args.steps)
        ms = np.array(rounds)
        med = float(np.median(ms))
        plan = km.kmeans_plan(N, D, K, cus)
        tflops = 2.0 * N * D * K / (med / 1e3) / 1e12
        ref = PAGES_B200_PR_MS[(N, D, K)]
        lat_ms.append(med)
        ref_ms.append(ref)
        print(json.dumps({
            "sweep_shape": {"N": N, "D": D, "K": K},
            "path": "split" if plan["path"] == km.PATH_SPLIT else "direct",
            "splits": plan["splits"],
            "ms": round(med, 4), "rounds_ms": [round(float(v), 4) for v in ms],
            "points_per_s": N / (med / 1e3),
            "tflops": round(tflops, 1),
            "frac_bf16_peak": round(tflops / BF16_DENSE_PEAK_TFLOPS, 4),
            "pages_b200_pr_ms": ref,
        }), flush=True)
        del sets, labels, min_dist
        torch.cuda.empty_cache()
    geo = float(np.exp(np.mean(np.log(lat_ms))))
    geo_ref = float(np.exp(np.mean(np.log(ref_ms))))
    print(json.dumps({"sweep_geomean_ms": round(geo, 4), "shapes": len(lat_ms),
                      "pages_b200_pr_geomean_ms": round(geo_ref, 4),
                      "note": "B200 numbers are another GPU's, context only"}), flush=True)


def settle(step, ms: float):
    """Run ``step(i)`` untimed until ``ms`` of wall time have passed: a GPU
    coming out of idle runs its first milliseconds of dense MFMA work at
    lower clocks (10 warmup steps of the headline workload are ~3 ms and
    measured ~15% slower than steady state).  Returns the steps run."""
    import torch
    if ms <= 0:
        return 0
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step(n)
            n += 1
        torch.cuda.synchronize()
    return n


def mfma_ceiling(X, C, dev, cus: int, tiles: int = 401, launches: int = 30,
                 settle_ms: float = 250.0):
    """Rate of the MFMA-only probe (libkmeans_mfma_stream.so) on operand rows
    made of this workload's values (points scaled by -2, as the assign kernel
    holds them, and centroids), and on zero operands: the matrix pipe's
    ceiling for this data on this GPU.  Measured the way the assign kernel
    is: ``settle_ms`` of untimed launches first (the clock a GPU holds under
    dense MFMA is reached only after some milliseconds), then ``launches``
    back-to-back launches of about the assign kernel's duration between two
    events."""
    import ctypes
    import torch
    from means_nearest_centroid_amd import build as kbuild
    lib = ctypes.CDLL(kbuild.PROBE_LIBRARY)
    lib.kmeans_mfma_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p]
    lib.kmeans_mfma_stream.restype = ctypes.c_int32
    threads = lib.kmeans_mfma_stream_threads()
    rows = int(min(8192, X.size // 128, C.size // 128))

    def operand(bits, scale):
        v = torch.from_numpy(bits.reshape(-1)[:rows * 128].view(np.int16)).view(torch.bfloat16)
        return (v.to(dev).float() * scale).to(torch.bfloat16).reshape(rows, 128).contiguous()

    wgs = 2 * cus
    sink = torch.empty(wgs * threads, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    flop = 2.0 * 32 * 32 * 16 * 16 * tiles * wgs * (threads // 64)

    def rate(a, b):
        def launch(_i=0):
            st = lib.kmeans_mfma_stream(a.data_ptr(), b.data_ptr(), rows, tiles, wgs,
                                        sink.data_ptr(), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"kmeans_mfma_stream failed ({st})")
        settle(launch, settle_ms)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            launch()
        e1.record(stream)
        e1.synchronize()
        return flop * launches / (e0.elapsed_time(e1) / 1e3) / 1e12

    data = rate(operand(C, 1.0), operand(X, -2.0))
    z = torch.zeros((rows, 128), dtype=torch.bfloat16, device=dev)
    zero = rate(z, z)
    return dict(probe="kmeans_mfma_stream: the assign kernel's MFMA back to back, no LDS, "
                      "no epilogue; operands = this workload's rows (x scaled by -2, centroids)",
                timing=f"{settle_ms:g} ms untimed, then {launches} back-to-back launches "
                       f"of {tiles} tiles between two events",
                tflops=round(data, 1), frac_of_peak=round(data / BF16_DENSE_PEAK_TFLOPS, 4),
                zero_operand_tflops=round(zero, 1))


def measure_sclk(step, n_steps: int, step_ms: float, dev):
    """Shader clock while ``step`` runs, untimed: one sleeping wave per XCD
    (kmeans_clock_sampler, on a side stream of default priority) reads the
    shader-clock counter against the 100 MHz counter over most of
    ``n_steps`` back-to-back steps.  The sampler needs a few registers and
    no LDS, so it sits beside the assign workgroups without displacing
    them.  Returns the clock per XCD in MHz."""
    import ctypes
    import torch
    from means_nearest_centroid_amd import build as kbuild
    lib = ctypes.CDLL(kbuild.PROBE_LIBRARY)
    lib.kmeans_clock_sampler.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_void_p]
    lib.kmeans_clock_sampler.restype = ctypes.c_int32
    wgs = 8
    out = torch.zeros(4 * wgs, dtype=torch.int64, device=dev)
    side = torch.cuda.Stream(device=dev)
    main = torch.cuda.current_stream()
    duration_us = max(1, int(0.8 * n_steps * step_ms * 1e3))
    torch.cuda.synchronize()
    st = lib.kmeans_clock_sampler(out.data_ptr(), wgs, duration_us, side.cuda_stream)
    if st != 0:
        raise RuntimeError(f"kmeans_clock_sampler failed ({st})")
    for i in range(n_steps):
        step(i)
    torch.cuda.synchronize()
    o = out.view(wgs, 4).cpu().numpy()
    by_xcd = {}
    for real, shader, xcd, _ in o:
        if real > 0:
            by_xcd.setdefault(int(xcd), []).append(100.0 * float(shader) / float(real))
    del main
    return {x: float(np.mean(v)) for x, v in sorted(by_xcd.items())}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(X, C, target_s: float):
    """Time the oracle on the first points of the workload, growing the
    sample until one run takes about ``target_s`` seconds.  Returns the
    baseline record and the oracle's result for the sample (the parity check
    of the timed outputs reuses it)."""
    import oracle
    n = 64
    while True:
        t0 = time.perf_counter()
        ref = oracle.assign(X[:n], C)
        dt = time.perf_counter() - t0
        if dt >= target_s or n >= X.shape[0]:
            break
        grow = max(2.0, min(16.0, 1.2 * target_s / max(dt, 1e-3)))
        n = min(X.shape[0], int(n * grow))
    rec = dict(value=n / dt, unit="points/s", cores=oracle.num_threads(), kind="oracle",
               sample=f"first {n} points of seed {W.SEEDS[0]}, all {C.shape[0]} "
                      f"centroids, fp64, {dt:.2f} s wall",
               cpu_model=cpu_model(),
               build="gcc " + " ".join(oracle.BUILD_FLAGS) + " (generic x86-64)")
    return rec, ref


def timed_output_parity(host_sets, outputs, ref0, head: int = 2048):
    """The acceptance rule on outputs of the timed calls: the last timed call
    on each seeded set, checked on the first points of every set (the pages'
    nightly comparison checks the first 2048 assignments of each seeded set,
    "Benchmark methodology"); for the first set on every point the CPU
    baseline's oracle run covered (``ref0``), else on the first ``head``."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    import parity
    per_seed = {}
    total_bad = 0
    reports = []
    for s, ((X, C), (lab, md)) in enumerate(zip(host_sets, outputs)):
        if s == 0 and ref0 is not None:
            n = len(ref0["labels"])
            ref = ref0
        else:
            n = min(head, X.shape[0])
            ref = oracle.assign(X[:n], C)
        stats, report = parity.evaluate(X, C, lab, md, idx=np.arange(n), ref=ref)
        per_seed[str(W.SEEDS[s])] = dict(points=n, bad=stats["bad"],
                                         strict=stats.get("strict"), near=stats.get("near"))
        total_bad += stats["bad"]
        if report:
            reports.append(f"seed {W.SEEDS[s]}: {report}")
    return dict(rule="labels exact where the oracle's top-two gap >= 1e-3(|best|+1), "
                     "else in the near-tie set; min_dist within 2e-3(|d|+1)",
                checked="the last timed call on each seeded set",
                points=sum(v["points"] for v in per_seed.values()), bad=total_bad,
                per_seed=per_seed), reports


UPDATE_METRIC = "centroid update (Lloyd step after assignment): points/sec at N={N},D={D},K={K} (1 GPU)"


def update_bytes(N: int, D: int, K: int) -> int:
    """Algorithmic HBM bytes of one update call without the fp32 means: every
    point row and label read once, every new row, norm and count written once
    (old rows are read only for empty clusters, none here)."""
    return N * (2 * D + 4) + K * (2 * D + 8)


def run_update(args):
    """Time kmeans_update (the Lloyd step after assignment) on one workload:
    three seeded sets resident and rotated, labels = each point's generating
    centre, outputs preallocated, no fp32 means.  One JSON line."""
    import torch
    import means_nearest_centroid_amd as km

    cfg = W.CONFIGS[args.config]
    N, D, K = cfg["N"], cfg["D"], cfg["K"]
    print(f"[bench] update: generating workload {args.config} ({cfg['name']})",
          file=sys.stderr, flush=True)
    host = []
    for s in W.SEEDS:
        X, C, meta = W.make_config(args.config, s)
        host.append((X, C, np.ascontiguousarray(meta["generating_centre"], dtype=np.int32)))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    km.load_library()

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    sets = [(to_dev(X), torch.from_numpy(lab).to(dev), to_dev(C)) for X, C, lab in host]
    # Outputs per set, so the last timed call on each set can be checked.
    outs = [(torch.empty((K, D), dtype=torch.bfloat16, device=dev),
             torch.empty(K, dtype=torch.float32, device=dev),
             torch.empty(K, dtype=torch.int32, device=dev)) for _ in sets]
    stream = torch.cuda.current_stream()

    def step(i):
        X, lab, C = sets[i % len(sets)]
        C_new, norms, counts = outs[i % len(sets)]
        km.kmeans_update(X, lab, C, C_new, norms, counts, stream=stream, path=args.update_path)

    settled = settle(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: K calls back to back, bracketed by synchronisation and
    # by GPU events on the launch stream, nothing else enqueued between the
    # calls (a timing event between two launches costs 3-4 us of stream time
    # here); a call's time is the region's over K.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(i)
    end.record(stream)
    enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    print(f"[bench] update: {ms_per_step * 1e3:.1f} us per call on the GPU, "
          f"{enqueue / args.steps * 1e6:.1f} us per call to enqueue on the host",
          file=sys.stderr, flush=True)

    if args.copy_calibration_mib:
        nbytes = args.copy_calibration_mib << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()

    timed = [(o[0].view(torch.int16).cpu().numpy().view(np.uint16), o[1].cpu().numpy(),
              o[2].cpu().numpy()) for o in outs]
    nbytes = update_bytes(N, D, K)
    avg_s = ms_per_step / 1e3
    achieved = nbytes / avg_s / 1e9
    traffic = traffic_record(args.config, "update")
    cpu = None
    timed_parity, bad_sets = None, []
    if args.cpu_seconds > 0:
        import oracle
        # The whole workload takes the oracle well under a second: repeat it
        # over the three sets until a second has passed.
        reps, t0 = 0, time.perf_counter()
        while True:
            X0, C0, l0 = host[reps % len(host)]
            oracle.update(X0, l0, C0)
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 1.0:
                break
        cpu = dict(value=reps * N / dt, unit="points/s", cores=1, kind="oracle",
                   sample=f"the whole workload, {reps} calls over the three seeded sets, "
                          f"fp64, one thread, {dt:.2f} s wall",
                   cpu_model=cpu_model(),
                   build="gcc " + " ".join(oracle.BUILD_FLAGS) + " (generic x86-64)")
        # The acceptance rule on the last timed call of every seeded set.
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import parity
        per_seed, bad_sets = {}, []
        for si, ((X0, C0, l0), (cn, nr, ct)) in enumerate(zip(host, timed)):
            try:
                st = parity.check_update(X0, l0, C0, cn, nr, ct)
                per_seed[str(W.SEEDS[si])] = dict(clusters=st["clusters"], ok=True)
            except AssertionError as e:
                per_seed[str(W.SEEDS[si])] = dict(ok=False)
                bad_sets.append(f"seed {W.SEEDS[si]}: {e}")
        timed_parity = dict(rule="counts exact, empty rows unchanged, bf16 rows within the "
                                 "fp32 summation bound of the oracle's mean, norms of the rows",
                            checked="the last timed call on each seeded set, every cluster",
                            bad_sets=len(bad_sets), per_seed=per_seed)
    out = {
        "metric": UPDATE_METRIC.format(N=N, D=D, K=K),
        "value": N / (ms_per_step / 1e3),
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"centroid update, {cfg['name']}, bf16 Gaussian mixture, labels "
                               f"= generating centres, seeds {list(W.SEEDS)} rotated",
                   "N": N, "D": D, "K": K, "settle_ms": args.settle_ms,
                   "settle_steps": settled,
                   "path": {0: "automatic", 1: "sort", 2: "buckets"}[args.update_path]},
        "roofline": dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                         unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                         traffic=(traffic["hbm_bytes_per_launch"] if traffic else None),
                         kernel="kmeans_update (all its kernels, one call)",
                         avg_launch_us=round(avg_s * 1e6, 2), bytes_per_launch=nbytes),
        "cpu_baseline": cpu,
        "parity": timed_parity,
    }
    print(json.dumps(out), flush=True)
    if bad_sets:
        print("[bench] update parity FAILED on the timed outputs:\n" + "\n".join(bad_sets),
              file=sys.stderr, flush=True)
        sys.exit(1)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=sorted(W.CONFIGS))
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="untimed steps for this long before the warmup steps, so the "
                         "timed steps run at steady-state clocks (0 disables)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle sample (0 disables)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one plain device copy of this size (counter scale)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the HBM-traffic record from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                         "run made with --copy-calibration-mib; no GPU work")
    ap.add_argument("--record-command", default="", help="command stored with the record")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the MFMA-only probe (mfma_ceiling: null)")
    ap.add_argument("--assign-path", type=int, default=0, choices=(0, 1, 2, 3),
                    help="0 the automatic dispatch (the headline figure); 1 direct, 2 split, "
                         "3 persistent (the work-queue kernel), forced through "
                         "kmeans_assign_path")
    ap.add_argument("--assign-count", type=int, default=0,
                    help="with --assign-path: its count argument (0 automatic)")
    ap.add_argument("--update-path", type=int, default=0, choices=(0, 1, 2),
                    help="with --update: 0 automatic, 1 the radix-sort path, 2 the bucket path")
    ap.add_argument("--update", action="store_true",
                    help="time kmeans_update (the Lloyd step after assignment) on the "
                         "workload instead (one JSON line)")
    ap.add_argument("--sweep", action="store_true",
                    help="time kmeans_assign on the pages' 13 shapes instead (one JSON "
                         "line per shape)")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.config, args.record_traffic[0], args.record_traffic[1],
                       args.copy_calibration_mib or 256, args.record_command,
                       kind="update" if args.update else assign_traffic_kind(args.assign_path))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the assignment library has no "
              "multi-GPU mode (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        run_sweep(args)
        return
    if args.update:
        run_update(args)
        return

    import torch
    import means_nearest_centroid_amd as km

    cfg = W.CONFIGS[args.config]
    N, D, K = cfg["N"], cfg["D"], cfg["K"]
    print(f"[bench] generating workload {args.config} ({cfg['name']})", file=sys.stderr,
          flush=True)
    host_sets = [W.make_config(args.config, s)[:2] for s in W.SEEDS]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    km.load_library()

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    sets = [(to_dev(X), to_dev(C)) for X, C in host_sets]
    norms = [torch.empty(K, dtype=torch.float32, device=dev) for _ in sets]
    # One pair of output buffers per seeded set, so that after the timed
    # region each holds the last timed call on its set (checked below).
    labels = [torch.empty(N, dtype=torch.int32, device=dev) for _ in sets]
    min_dist = [torch.empty(N, dtype=torch.float32, device=dev) for _ in sets]
    stream = torch.cuda.current_stream()
    plan = km.kmeans_plan(N, D, K, torch.cuda.get_device_properties(dev).multi_processor_count)

    def norms_only(i):
        j = i % len(sets)
        km.kmeans_centroid_norms(sets[j][1], norms[j], stream=stream)

    def assign_only(i):
        j = i % len(sets)
        X, C = sets[j]
        if args.assign_path == 0:
            km.kmeans_assign(X, C, norms[j], labels[j], min_dist[j], stream=stream)
        else:
            km.kmeans_assign_path(X, C, norms[j], args.assign_path, args.assign_count,
                                  labels[j], min_dist[j], stream=stream)

    def step(i):
        norms_only(i)
        assign_only(i)

    def region_ms(fn):
        # Per-call time of args.steps calls back to back, bracketed by
        # synchronisation and by GPU events on the launch stream, nothing
        # else enqueued between the calls (a timing event between two
        # launches costs 3-4 us of stream time here).
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    settled = settle(step, args.settle_ms)
    print(f"[bench] settled clocks with {settled} untimed steps; warmup {args.warmup} steps",
          file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps (norms + assign) back to back, bracketed by
    # synchronisation and by GPU events on the launch stream.
    t0 = time.perf_counter()
    ms_per_step = region_ms(step)
    wall = time.perf_counter() - t0
    total_ms = ms_per_step * args.steps
    print(f"[bench] {args.steps} steps: {total_ms:.3f} ms GPU, {wall * 1e3:.3f} ms wall",
          file=sys.stderr, flush=True)
    # Outputs of the timed calls, before any later launch overwrites them.
    timed_outputs = [(lab.cpu().numpy(), md.cpu().numpy()) for lab, md in zip(labels, min_dist)]
    # Each kernel's average launch time, right after the timed steps: K
    # back-to-back launches of it alone on the same rotating sets, timed the
    # same way (every set's norms written first).
    for j in range(len(sets)):
        norms_only(j)
    assign_ms = region_ms(assign_only)
    norms_ms = region_ms(norms_only)
    print(f"[bench] per launch: assign {assign_ms * 1e3:.2f} us, norms {norms_ms * 1e3:.2f} us",
          file=sys.stderr, flush=True)

    if args.copy_calibration_mib:
        # A plain streaming kernel of known traffic (read n bytes, write n
        # bytes) for scaling the HBM byte counters.
        nbytes = args.copy_calibration_mib << 20
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {nbytes} bytes read, {nbytes} bytes written",
              file=sys.stderr, flush=True)

    flops = 2.0 * N * D * K
    avg_assign_s = assign_ms / 1e3
    achieved = flops / avg_assign_s / 1e12
    traffic = traffic_record(args.config, assign_traffic_kind(args.assign_path))
    if args.assign_path == 0:
        kernel = ("kmeans_assign (assign_kernel"
                  + (" + merge_kernel" if plan["path"] == km.PATH_SPLIT else "") + ")")
        path_name = "split" if plan["path"] == km.PATH_SPLIT else "direct"
    else:
        kernel = (f"kmeans_assign_path, {ASSIGN_PATH_NAMES[args.assign_path]} forced ("
                  + {1: "assign_kernel", 2: "assign_kernel + merge_kernel",
                     3: "assign_queue_kernel"}[args.assign_path] + ")")
        path_name = f"{ASSIGN_PATH_NAMES[args.assign_path]} (forced, count {args.assign_count})"
    roofline = dict(bound="mfma", achieved=round(achieved, 2), peak=BF16_DENSE_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / BF16_DENSE_PEAK_TFLOPS, 4),
                    traffic=(traffic["hbm_bytes_per_launch"] if traffic else None),
                    kernel=kernel,
                    avg_launch_us=round(avg_assign_s * 1e6, 2),
                    flop_per_launch=flops)

    sclk = None
    if not args.no_ceiling:
        print("[bench] shader clock beside 30 untimed steps", file=sys.stderr, flush=True)
        by_xcd = measure_sclk(step, 30, ms_per_step, dev)
        if by_xcd:
            mhz = float(np.mean(list(by_xcd.values())))
            sclk = dict(method="one sleeping wave per XCD reads s_memtime against the 100 MHz "
                               "s_memrealtime beside 30 untimed steps",
                        mhz_mean=round(mhz, 0),
                        mhz_by_xcd={str(k): round(v, 0) for k, v in by_xcd.items()},
                        frac_at_sclk=round(achieved / (BF16_DENSE_PEAK_TFLOPS * mhz / 2400.0), 4))

    ceiling = None
    if not args.no_ceiling:
        print("[bench] MFMA-only probe on this workload's operands", file=sys.stderr, flush=True)
        X0, C0 = host_sets[0]
        ceiling = mfma_ceiling(X0, C0, dev, torch.cuda.get_device_properties(dev).multi_processor_count,
                               settle_ms=args.settle_ms)
        ceiling["assign_frac_of_ceiling"] = round(achieved / ceiling["tflops"], 4)

    cpu = None
    timed_parity = None
    parity_reports = []
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        X0, C0 = host_sets[0]
        cpu, ref0 = cpu_baseline(X0, C0, args.cpu_seconds)
        print("[bench] checking the timed outputs against the oracle", file=sys.stderr,
              flush=True)
        timed_parity, parity_reports = timed_output_parity(host_sets, timed_outputs, ref0)

    value = N / (ms_per_step / 1e3)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"kmeans assignment, {cfg['name']}, bf16 Gaussian mixture, "
                        f"seeds {list(W.SEEDS)} rotated",
            "N": N, "D": D, "K": K, "path": path_name,
            "splits": plan["splits"], "settle_ms": args.settle_ms, "settle_steps": settled,
        },
        "roofline": roofline,
        "mfma_ceiling": ceiling,
        "sclk": sclk,
        "cpu_baseline": cpu,
        "parity": timed_parity,
        "breakdown_us": {
            "step_mean": round(ms_per_step * 1e3, 2),
            "assign_launch_mean": round(assign_ms * 1e3, 2),
            "norms_launch_mean": round(norms_ms * 1e3, 2),
        },
        "assign_only_points_per_s": N / (assign_ms / 1e3),
    }
    print(json.dumps(out), flush=True)
    if parity_reports:
        print("[bench] timed outputs FAIL the acceptance rule:\n" + "\n".join(parity_reports),
              file=sys.stderr, flush=True)
        sys.exit(1)


if __name__ == "__main__":
    main()
