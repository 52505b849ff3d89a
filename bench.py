#!/usr/bin/env python3
"""Benchmark of exact resident top-K on one MI355X.

Default workload: the 1,000,000 x 1024 fp32 resident corpus (rows iid N(0,1),
L2-normalised), sequential single queries at K = 8, 32 and 100 -- the
configuration whose queries/s and p50 latency are the headline metric.  One
step = one query at each of the three K values (three search_resident calls,
each synchronised before the next, as an agent issues them).  Queries are
already resident in HBM when timing starts; the PCIe-inclusive interval
(query H->D, search, 2K results D->H) is measured separately and reported as
context, never as `value`.

The dominant kernel (the fused streaming scorer + per-wave top-K) is timed with
HIP events recorded by the library on the search stream inside the timed
region; its algorithmic bytes (N*D*4 corpus + D*4 query) over its average
duration give `roofline.achieved`.

cpu_baseline: the CPU oracle (fp64 dots + full sort) timed on this host's cores
on a bounded sample of the same queries; the same sample's GPU answers are
checked against it (R1-R4) before the line is printed.

filtered_exact: the same queries through search_resident_filtered (a reduced-
precision copy scanned first -- fp8 codes for this corpus size, bf16 for small
ones -- and fp32 rows re-scored only where certified bounds reach the
threshold); its answers are checked to equal the plain scan's bit for bit
before it is timed.  Reported beside `value`, which stays the plain fp32 scan.

The other four configurations run in the same default invocation and appear
under `workloads` in the same line, each with its own protocol (1,000
sequential queries per K at 10k x 384 and 50k/100k x 768, at least 100 calls per
K for the 1e8 int32 top-K, 100 batches per K for the 32-query batch at 500k x
768), its roofline fraction, the oracle timed on a bounded sample with the GPU
answers checked against it, and for the batch the matrix-core utilisation.
`--workload NAME` runs one configuration alone; `--n/--d/--k/--queries/--batch/
--seed` run a free-form synthetic corpus of the same recipe.
"""
import argparse
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "queries/s + p50 latency at N=1M,D=1024,K∈{8,32,100}; % of HBM peak"


def profile_record(name):
    """A committed PMC summary (profiles/<name>.json), if it was taken on the
    current kernel sources (their sha256 matches), else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", name + ".json")
    try:
        with open(path) as f:
            data = json.load(f)
        h = hashlib.sha256()
        for src in data["kernel_sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != data["kernel_sources_sha256"]:
            return None
        return data
    except (OSError, KeyError, ValueError):
        return None


def measured_traffic(name="gemv_topk_1m_x_1024_traffic", key="mean over K=8,32,100"):
    """HBM bytes per launch of a kernel from its committed PMC summary (FETCH_SIZE
    x the copy calibration + WRITE_SIZE), if taken on the current sources."""
    data = profile_record(name)
    try:
        return float(data["traffic_bytes_per_launch"][key]) if data else None
    except (KeyError, TypeError, ValueError):
        return None


# Committed PMC summaries (profiles/<name>.json) of each workload's dominant
# kernel: HBM bytes per launch and, for the batch, matrix-core busy cycles.
TRAFFIC_PROFILES = {
    "c1_10k_384": ("gemv_topk_10k_x_384_traffic", "mean"),
    "c2_50k_768": ("gemv_topk_50k_x_768_traffic", "mean"),
    "c2_100k_768": ("gemv_topk_100k_x_768_traffic", "mean"),
    "c3_1m_1024": ("gemv_topk_1m_x_1024_traffic", "mean over K=8,32,100"),
    "c4_1e8_int32": ("select_topk_1e8_int32_traffic", "mean"),
    "c5_q32_500k_768": ("mfma_scores_32x500k_x_768_traffic", "mean"),
}
FP32_MFMA_PEAK_TFLOPS = 157.3

# The other configurations of the default run, each with its own protocol.
SUITE = (
    ("c1_10k_384", dict(steps=1000, warmup=20, cpu_budget=3.0, cpu_queries=1, filtered_leg=False)),
    ("c2_50k_768", dict(steps=1000, warmup=20, cpu_budget=4.0, cpu_queries=40, filtered_leg=True)),
    ("c2_100k_768", dict(steps=1000, warmup=20, cpu_budget=4.0, cpu_queries=40, filtered_leg=True)),
    ("c4_1e8_int32", dict(steps=100, warmup=5)),
    ("c5_q32_500k_768", dict(steps=100, warmup=5, filtered_leg=True)),
)


def workload_traffic(name, metric="dot", filtered=False):
    if metric != "dot" or filtered or name not in TRAFFIC_PROFILES:
        return None
    return measured_traffic(*TRAFFIC_PROFILES[name])


def environment(torch, workloads):
    """Versions, device and seeds of this run (inputs are synthetic and seeded)."""
    def read(path):
        try:
            return open(path).read().strip()
        except OSError:
            return None
    props = torch.cuda.get_device_properties(0)
    return {
        "rocm": read("/opt/rocm/.info/version"), "hip_runtime": torch.version.hip, "torch": torch.__version__,
        "numpy": np.__version__, "python": sys.version.split()[0],
        "gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", None), "compute_units": props.multi_processor_count,
        "gpu_memory_gib": round(props.total_memory / 2 ** 30, 1),
        "clocks_locked": False,
        "seeds": {"generator": "numpy PCG64, SeedSequence([base_seed, config_id, stream, chunk])",
                  "base_seed": workloads.BASE_SEED,
                  "config_ids": {k: v["config_id"] for k, v in workloads.WORKLOADS.items()},
                  "streams": {"corpus": workloads.STREAM_CORPUS, "queries": workloads.STREAM_QUERIES,
                              "plant_positions": workloads.STREAM_PLANT_POS, "plant_noise": workloads.STREAM_PLANT_NOISE,
                              "duplicates": workloads.STREAM_DUP}},
        "host_cores": host_cores(), "cpu_model": cpu_model(),
    }


def pct(a, p):
    return float(np.percentile(np.asarray(a), p))


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PROFILE_EVERY = 10  # timed steps per step whose device times are read (HIP events)


def time_search(eng, torch, qdev, ks, steps, warmup, profile=True, metric="dot", filtered=False):
    """Sequential single queries; returns per-K lists of host latency (us),
    whole-call device time and streaming-kernel time (ms) (with `filtered`: the
    first pass's time in place of the streaming-kernel time).  The device times
    come from every PROFILE_EVERY-th step of the timed loop: recording and
    reading the events costs a few microseconds per call, which would otherwise
    be counted in the queries/s of the small corpora."""
    def search(q, k, oi, os_, stream):
        if filtered:
            return eng.search_resident_filtered(q, k, oi, os_, stream=stream, metric=metric)
        return eng.search_resident(q, k, oi, os_, stream=stream, metric=metric)

    n_q = qdev.shape[0]
    outs = {k: (torch.empty((1, k), dtype=torch.int32, device="cuda"),
                torch.empty((1, k), dtype=torch.float32, device="cuda")) for k in ks}
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        for k in ks:
            search(qdev[i % n_q:i % n_q + 1], k, *outs[k], stream)
    torch.cuda.synchronize()
    lat = {k: [] for k in ks}
    part = {k: [] for k in ks}
    merge = {k: [] for k in ks}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        q = qdev[i % n_q:i % n_q + 1]
        sampled = profile and i % PROFILE_EVERY == 0
        if sampled:
            eng.profile(True)
        for k in ks:
            s = time.perf_counter_ns()
            search(q, k, *outs[k], stream)
            stream.synchronize()
            lat[k].append((time.perf_counter_ns() - s) / 1e3)
            if sampled:
                total, first, kern = eng.profile_read()
                part[k].append(first if filtered and first > 0 else kern)  # no first pass: plain route
                merge[k].append(total)
        if sampled:
            eng.profile(False)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, lat, part, merge


def time_end_to_end(eng, torch, qhost, ks, reps, metric="dot", filtered=False):
    """Pages-style interval: pinned query H->D, search, K idx + K scores D->H."""
    d = qhost.shape[1]
    pin_q = torch.empty((1, d), dtype=torch.float32).pin_memory()
    qdev = torch.empty((1, d), dtype=torch.float32, device="cuda")
    res = {}
    stream = torch.cuda.current_stream()
    for k in ks:
        oi = torch.empty((1, k), dtype=torch.int32, device="cuda")
        os_ = torch.empty((1, k), dtype=torch.float32, device="cuda")
        hi = torch.empty((1, k), dtype=torch.int32).pin_memory()
        hs = torch.empty((1, k), dtype=torch.float32).pin_memory()
        ts = []
        for r in range(reps):
            pin_q.copy_(torch.from_numpy(qhost[r % qhost.shape[0]:r % qhost.shape[0] + 1]))
            s = time.perf_counter_ns()
            qdev.copy_(pin_q, non_blocking=True)
            if filtered:
                eng.search_resident_filtered(qdev, k, oi, os_, stream=stream, metric=metric)
            else:
                eng.search_resident(qdev, k, oi, os_, stream=stream, metric=metric)
            hi.copy_(oi, non_blocking=True)
            hs.copy_(os_, non_blocking=True)
            stream.synchronize()
            ts.append((time.perf_counter_ns() - s) / 1e3)
        res[k] = {"p50_us": pct(ts, 50), "p99_us": pct(ts, 99)}
    return res


def cpu_baseline_retrieval(corpus, qhost, kmax, gpu_results, budget_s, max_queries, metric="dot"):
    """Time the oracle on a bounded sample and check the GPU answers of the same
    queries against it."""
    import oracle
    from tests.gpu_util import check_retrieval  # noqa: E402  (test helpers: acceptance rules)
    times = []
    t_start = time.perf_counter()
    nq = 0
    for qi in range(min(max_queries, qhost.shape[0])):
        s = time.perf_counter()
        o_idx, o_sc = oracle.search(corpus, qhost[qi:qi + 1], kmax, metric=1 if metric == "cosine" else 0)
        times.append(time.perf_counter() - s)
        for k, (g_idx, g_sc) in gpu_results.items():
            check_retrieval(g_idx[qi], g_sc[qi], o_idx[0, :k], o_sc[0, :k], corpus, qhost[qi], oracle,
                            metric=metric)
        nq += 1
        if time.perf_counter() - t_start > budget_s:
            break
    return {"value": nq / sum(times), "unit": "queries/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {nq} queries of the workload at K={kmax} (smaller K are prefixes), fp64 "
                      f"{'cosines' if metric == 'cosine' else 'dots'} + full sort; "
                      f"GPU answers of the same queries checked against it (R1-R4)",
            "host_cores": host_cores(), "cpu_model": cpu_model(), "parity": "ok"}


def batcher_leg(args, torch, eng, qhost, ks):
    """Many concurrent single-query clients (host threads, each issuing blocking
    searches back to back, K cycling through the workload's K values) served
    by one rt_batcher in exact mode: their queries run as batched filtered
    searches.  Reports total queries/s, per-request latency (submit to answer,
    host clock) and the batch sizes reached; a sample of answers is checked to
    equal the single-query scan's bit for bit first."""
    from concurrent.futures import ThreadPoolExecutor
    from top_search_resident_amd import Batcher
    clients, reps = args.batcher_clients, args.batcher_requests
    be = eng.shared(max_k=max(ks), max_q=32)
    be.enable_filtered()
    nq = qhost.shape[0]
    with Batcher(be, max_batch=32, max_wait_us=args.batcher_wait_us, exact=True) as b:
        # parity first: a few answers against the plain single-query scan
        for qi in range(min(8, nq)):
            k = ks[qi % len(ks)]
            bi, bs = b.search(qhost[qi], k)
            si, ss = eng.search_resident(torch.from_numpy(qhost[qi:qi + 1]).cuda(), k)
            torch.cuda.synchronize()
            if not (np.array_equal(bi, si.cpu().numpy()[0]) and
                    np.array_equal(bs.view(np.uint32), ss.cpu().numpy()[0].view(np.uint32))):
                raise SystemExit("dynamic batching: answer differs from the single-query scan")

        def client(c, count):
            lat = []
            for r in range(count):
                i = (c * count + r) % nq
                t0 = time.perf_counter()
                b.search(qhost[i], ks[(c + r) % len(ks)])
                lat.append((time.perf_counter() - t0) * 1e6)
            return lat

        with ThreadPoolExecutor(clients) as ex:  # warm-up
            list(ex.map(lambda c: client(c, 2), range(clients)))
        s0 = b.stats()
        t0 = time.perf_counter()
        with ThreadPoolExecutor(clients) as ex:
            lats = list(ex.map(lambda c: client(c, reps), range(clients)))
        wall = time.perf_counter() - t0
        s1 = b.stats()
    be.close()
    lat = np.concatenate([np.asarray(x) for x in lats])
    batches = s1["batches"] - s0["batches"]
    return {"queries_per_s": lat.size / wall, "clients": clients, "requests": int(lat.size),
            "ks": list(ks), "p50_us": pct(lat, 50), "p99_us": pct(lat, 99),
            "batches": batches, "mean_batch": lat.size / max(batches, 1), "largest_batch": s1["largest_batch"],
            "max_wait_us": args.batcher_wait_us, "mode": "exact (batched filtered search)",
            "parity": "8 answers bit-identical to the single-query scan",
            "note": "host threads in Python: each request also pays the binding's per-call cost"}


def run_retrieval(args, torch, ResidentTopK, workloads):
    name = args.workload
    w = workloads.WORKLOADS[name]
    t = time.perf_counter()
    corpus, qhost = workloads.retrieval_inputs(name, queries=min(w["queries"], args.num_queries))
    gen_s = time.perf_counter() - t
    n, d = corpus.shape
    ks = tuple(w["ks"])
    batch = w.get("batch", 1)
    eng = ResidentTopK(max_n=n, max_d=d, max_k=max(ks), max_q=max(batch, 1))
    eng.upload_corpus_rowmajor(corpus)
    qdev = torch.from_numpy(qhost).cuda()
    torch.cuda.synchronize()

    if batch > 1:
        return run_batched(args, torch, eng, corpus, qhost, qdev, ks, name, gen_s)
    if args.streams > 1:
        return run_concurrent(args, torch, eng, corpus, qhost, qdev, ks, name, gen_s)

    if args.filtered:
        eng.enable_filtered()
        eng.set_filter_storage(args.filter_storage)
    wall, lat, part, merge = time_search(eng, torch, qdev, ks, args.steps, args.warmup, metric=args.metric,
                                         filtered=args.filtered)
    path = eng.filter_path_used() if args.filtered else None
    nq = args.steps * len(ks)
    qps = nq / wall
    # algorithmic bytes per launch of the dominant kernel: the corpus and the
    # query, plus the rows' norms for the cosine metric; for the filtered search
    # its first pass: the bf16 rows and the rows' norms (or the fp8 codes and a
    # {scale, bound part} pair per row) and the 16-bit upper bounds it writes
    if args.filtered and path == "fp8":
        corpus_bytes = n * d + d * 4 + n * 8 + n * 2 + (n * 4 if args.metric == "cosine" else 0)
    elif args.filtered and path != "plain":
        corpus_bytes = n * d * 2 + d * 4 + n * 4 + n * 2
    else:
        corpus_bytes = n * d * 4 + d * 4 + (n * 4 if args.metric == "cosine" else 0)
    per_k = {}
    all_part = []
    for k in ks:
        dev = np.asarray(merge[k])
        per_k[str(k)] = {
            "queries_per_s": len(lat[k]) / (np.sum(lat[k]) / 1e6),
            "p50_us": pct(lat[k], 50), "p99_us": pct(lat[k], 99),
            "device_p50_us": pct(dev * 1e3, 50), "device_p99_us": pct(dev * 1e3, 99),
            "scan_kernel_avg_us": float(np.mean(part[k]) * 1e3),
            "scan_kernel_gbs": corpus_bytes / (np.mean(part[k]) * 1e-3) / 1e9,
            "device_p50_hbm_frac": corpus_bytes / (pct(dev, 50) * 1e-3) / 1e9 / HBM_PEAK_GBS,
        }
        all_part += part[k]
    avg_ms = float(np.mean(all_part))
    achieved = corpus_bytes / (avg_ms * 1e-3) / 1e9
    line = {
        "metric": (METRIC if (name, args.metric, args.filtered) == ("c3_1m_1024", "dot", False)
                   else f"queries/s + p50 latency ({name}, {f'{path}-filtered exact ' if args.filtered else ''}"
                        f"{args.metric})"),
        "value": qps, "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{name}: resident {n} x {d} fp32 corpus (Gaussian, L2-normalised rows), "
                               f"sequential single queries, K in {list(ks)}; one step = one query per K"
                               + ("; cosine metric" if args.metric == "cosine" else "")
                               + (f"; {path}-filtered exact search (answers identical to the fp32 scan)"
                                  if args.filtered else ""),
                   "n": n, "d": d, "ks": list(ks), "queries_per_step": len(ks), "metric": args.metric,
                   "filtered": bool(args.filtered)},
        "per_k": per_k,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": workload_traffic(name, args.metric, args.filtered),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, profiles/)",
                     "kernel": ((("gemv_bound8_kernel" if path == "fp8" else "gemv_bound_kernel")
                                 + f" ({path} first pass of the filtered search)")
                                if args.filtered and path != "plain" else
                                "gemv_topk_kernel (fused scoring, per-wave top-K lists and merge tree)"
                                + ("; the filtered search ran the plain scan" if args.filtered else "")),
                     "bytes_per_launch": corpus_bytes, "avg_launch_us": avg_ms * 1e3},
        "input_gen_s": gen_s,
    }
    if getattr(args, "latency_queries", 0) and args.steps < args.latency_queries:
        # the configuration's protocol: this many sequential queries per K, for
        # the latency distribution (the timed steps above may be fewer)
        _, llat, _, lmerge = time_search(eng, torch, qdev, ks, args.latency_queries, 0, metric=args.metric,
                                         filtered=args.filtered)
        line["latency_distribution"] = {
            "queries_per_k": args.latency_queries,
            "per_k": {str(k): {"p50_us": pct(llat[k], 50), "p99_us": pct(llat[k], 99),
                               "device_p50_us": pct(np.asarray(lmerge[k]) * 1e3, 50),
                               "device_p99_us": pct(np.asarray(lmerge[k]) * 1e3, 99)} for k in ks}}
    if args.e2e_reps:
        line["end_to_end_pcie"] = time_end_to_end(eng, torch, qhost, ks, args.e2e_reps, metric=args.metric,
                                                  filtered=args.filtered)
    if not args.filtered:
        line["hbm_read_ceiling"] = read_ceiling(eng, n * d * 4, avg_ms)
    line["gpu_clocks"] = gpu_clocks()
    if not args.filtered and not args.no_filtered_leg and d % 8 == 0:
        line["filtered_exact"] = filtered_leg(args, torch, eng, qdev, ks, n, d)
    if not args.filtered and args.batcher_clients > 0 and d % 8 == 0 and args.metric == "dot":
        line["dynamic_batching"] = batcher_leg(args, torch, eng, qhost, ks)
    if not args.no_cpu_baseline:
        sample = min(args.cpu_queries, qhost.shape[0])
        gpu_res = {}
        for k in ks:
            gi = np.empty((sample, k), np.int32)
            gs = np.empty((sample, k), np.float32)
            for qi in range(sample):
                if args.filtered:
                    a, b = eng.search_resident_filtered(qdev[qi:qi + 1], k, metric=args.metric)
                else:
                    a, b = eng.search_resident(qdev[qi:qi + 1], k, metric=args.metric)
                torch.cuda.synchronize()
                gi[qi], gs[qi] = a.cpu().numpy()[0], b.cpu().numpy()[0]
            gpu_res[k] = (gi, gs)
        line["cpu_baseline"] = cpu_baseline_retrieval(corpus, qhost, max(ks), gpu_res, args.cpu_budget, sample,
                                                      metric=args.metric)
    eng.close()
    return line


def read_ceiling(eng, corpus_bytes, scan_ms, reps=20):
    """The same run's plain streaming read of the resident corpus
    (rt_read_probe): the achievable read bandwidth that the scan's is compared
    with."""
    eng.read_probe(reps=3)  # warm-up
    ms = eng.read_probe(reps=reps)
    gbs = corpus_bytes / (ms * 1e-3) / 1e9
    return {"kernel": "read_probe_kernel (a contiguous chunk per wave, non-temporal 16-byte loads, no other work)",
            "bytes": corpus_bytes,
            "avg_launch_us": ms * 1e3, "gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "scan_frac_of_ceiling": ms / scan_ms}


def gpu_clocks():
    """GPU clock levels as the amdgpu driver lists them in sysfs, read after the
    timed work (the level in use then is marked '*'; clocks are not locked);
    None when the files are not readable.  A plain file read: no other program
    is started."""
    out = {}
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        vals = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            try:
                with open(os.path.join(dev, name)) as f:
                    levels = [ln.strip() for ln in f if ln.strip()]
            except OSError:
                continue
            vals[name[7:]] = levels
        if vals:
            out[os.path.basename(os.path.dirname(dev))] = vals
    return out or None


def filtered_leg(args, torch, eng, qdev, ks, n, d):
    """The same queries through search_resident_filtered (a reduced-precision
    first pass -- bf16, or fp8 for a large corpus, as the engine chooses unless
    --filter-storage says otherwise -- then the exact fp32 re-rank of the rows
    whose bounds reach the threshold): its answers are first checked to be
    identical, bit for bit, to the plain scan's on a sample, then timed like the
    plain scan."""
    eng.enable_filtered()
    eng.set_filter_storage(args.filter_storage)
    for qi in range(min(5, qdev.shape[0])):
        for k in ks:
            a = eng.search_resident(qdev[qi:qi + 1], k, metric=args.metric)
            b = eng.search_resident_filtered(qdev[qi:qi + 1], k, metric=args.metric)
            torch.cuda.synchronize()
            if not (torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))):
                raise SystemExit(f"filtered search differs from the plain scan (query {qi}, k {k})")
    path = eng.filter_path_used()
    steps = min(args.steps, 300)
    wall, lat, part, merge = time_search(eng, torch, qdev, ks, steps, args.warmup, metric=args.metric,
                                         filtered=True)
    if path == "plain":  # a small corpus under --filter-storage auto: the engine runs the plain scan
        return {"value": steps * len(ks) / wall, "unit": "queries/s", "steps": steps, "metric": args.metric,
                "identical_to_fp32_scan": True, "first_pass_storage": path,
                "note": "below the corpus size where the two passes pay off the engine runs the plain scan",
                "per_k": {str(k): {"p50_us": pct(lat[k], 50), "p99_us": pct(lat[k], 99),
                                   "device_p50_us": pct(np.asarray(merge[k]) * 1e3, 50)} for k in ks}}
    if path == "fp8":  # codes, query, per-row {scale, bound part} (+ row norm for the cosine), 16-bit bounds written
        pass1_bytes = n * d + d * 4 + n * 8 + n * 2 + (n * 4 if args.metric == "cosine" else 0)
        kernel = "gemv_bound8_kernel"
    else:  # bf16 rows, query, row norms, 16-bit upper bounds written
        pass1_bytes, kernel = n * d * 2 + d * 4 + n * 4 + n * 2, "gemv_bound_kernel"
    p1 = float(np.mean(np.concatenate([np.asarray(part[k]) for k in ks])))
    return {"value": steps * len(ks) / wall, "unit": "queries/s", "steps": steps, "metric": args.metric,
            "identical_to_fp32_scan": True, "first_pass_storage": path,
            "per_k": {str(k): {"p50_us": pct(lat[k], 50), "p99_us": pct(lat[k], 99),
                               "device_p50_us": pct(np.asarray(merge[k]) * 1e3, 50),
                               "first_pass_avg_us": float(np.mean(part[k]) * 1e3)} for k in ks},
            "first_pass": {"kernel": kernel, "bytes_per_launch": pass1_bytes,
                           "avg_launch_us": p1 * 1e3, "achieved_gbs": pass1_bytes / (p1 * 1e-3) / 1e9,
                           "frac_of_hbm_peak": pass1_bytes / (p1 * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def run_concurrent(args, torch, eng, corpus, qhost, qdev, ks, name, gen_s):
    """S engines sharing the resident corpus, one stream each (several agents
    querying one corpus): every step issues, on each stream, one query per K,
    and then waits for all streams."""
    n, d = corpus.shape
    S = args.streams
    engines = [eng] + [eng.shared() for _ in range(S - 1)]
    streams = [torch.cuda.Stream() for _ in range(S)]
    outs = [{k: (torch.empty((1, k), dtype=torch.int32, device="cuda"),
                 torch.empty((1, k), dtype=torch.float32, device="cuda")) for k in ks} for _ in range(S)]
    n_q = qdev.shape[0]

    def step(i):
        for e in range(S):
            q = qdev[(i * S + e) % n_q:(i * S + e) % n_q + 1]
            for k in ks:
                engines[e].search_resident(q, k, *outs[e][k], stream=streams[e], metric=args.metric)

    torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    lat = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        s0 = time.perf_counter_ns()
        step(i)
        for st in streams:
            st.synchronize()
        lat.append((time.perf_counter_ns() - s0) / 1e3)
    wall = time.perf_counter() - t0
    nq = args.steps * S * len(ks)
    line = {"metric": f"queries/s with {S} concurrent streams ({name}, {args.metric})", "value": nq / wall,
            "unit": "queries/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"{name}: {S} engines sharing one resident {n} x {d} fp32 corpus, one stream "
                                   f"each; a step = one query per K on every stream, then wait for all",
                       "n": n, "d": d, "ks": list(ks), "streams": S, "metric": args.metric},
            "step_p50_us": pct(lat, 50), "step_p99_us": pct(lat, 99), "input_gen_s": gen_s}
    for e in engines[1:]:
        e.close()
    eng.close()
    return line


def batched_filtered_leg(args, torch, eng, qdev, ks, n, d):
    """The same batches through search_resident_filtered (one bf16 matrix-core
    bound pass for all queries, per-query thresholds, fp32 re-rank), after
    checking that every query's indices and score bits equal the plain
    single-query scan's."""
    q = qdev.shape[0]
    stream = torch.cuda.current_stream()
    eng.enable_filtered()
    for k in ks:
        fi, fs = eng.search_resident_filtered(qdev, k)
        plain = [eng.search_resident(qdev[i:i + 1], k) for i in range(q)]
        torch.cuda.synchronize()
        pi = torch.cat([p[0] for p in plain]).cpu().numpy()
        ps = torch.cat([p[1] for p in plain]).cpu().numpy()
        if not (np.array_equal(pi, fi.cpu().numpy()) and np.array_equal(ps.view(np.uint32), fs.cpu().numpy().view(np.uint32))):
            raise SystemExit(f"filtered batch differs from the plain single-query scan at k={k}")
    outs = {k: (torch.empty((q, k), dtype=torch.int32, device="cuda"),
                torch.empty((q, k), dtype=torch.float32, device="cuda")) for k in ks}
    for _ in range(max(args.warmup, 3)):
        for k in ks:
            eng.search_resident_filtered(qdev, k, *outs[k], stream=stream)
    torch.cuda.synchronize()
    eng.profile(True)
    lat = {k: [] for k in ks}
    p1 = {k: [] for k in ks}
    rest = {k: [] for k in ks}
    steps = max(1, min(args.steps, 200))
    t0 = time.perf_counter()
    for _ in range(steps):
        for k in ks:
            s = time.perf_counter_ns()
            eng.search_resident_filtered(qdev, k, *outs[k], stream=stream)
            stream.synchronize()
            lat[k].append((time.perf_counter_ns() - s) / 1e3)
            total, first, other = eng.profile_read()
            p1[k].append(first)
            rest[k].append(other)
    wall = time.perf_counter() - t0
    eng.profile(False)
    tiles = (n + 31) // 32
    # bf16 rows, queries, two norms per row, the upper bounds written (16-bit
    # from the direct-to-LDS kernel, else fp32) and the tile maxima
    dma = n >= 32 and d in (256, 384, 512, 768)
    pass1_bytes = n * d * 2 + q * d * 4 + n * 8 + q * n * (2 if dma else 4) + q * tiles * 4
    all_p1 = float(np.mean(np.concatenate([np.asarray(p1[k]) for k in ks])))
    traffic = measured_traffic("mfma_bound_32x500k_x_768_traffic", "mean") if (n, d, q) == (500_000, 768, 32) else None
    return {"value": q * steps * len(ks) / wall, "unit": "queries/s", "steps": steps,
            "identical_to_single_query_scan": True,
            "per_k": {str(k): {"p50_us": pct(lat[k], 50), "p99_us": pct(lat[k], 99),
                               "bound_pass_avg_us": float(np.mean(p1[k])) * 1e3,
                               "threshold_and_rerank_avg_us": float(np.mean(rest[k])) * 1e3} for k in ks},
            "bound_pass": {"kernel": ("mfma_bound_dma_kernel (direct global-to-LDS loads, 16-bit upper bounds)"
                                      if dma else "mfma_bound_kernel"),
                           "bytes_per_launch": pass1_bytes, "traffic": traffic,
                           "avg_launch_us": all_p1 * 1e3,
                           "achieved_gbs": pass1_bytes / (all_p1 * 1e-3) / 1e9,
                           "frac_of_hbm_peak": pass1_bytes / (all_p1 * 1e-3) / 1e9 / HBM_PEAK_GBS}}


def mfma_kernel_name(n, d, metric):
    if metric == "dot" and n >= 32 and d in (256, 384, 512, 768):
        return "mfma_scores_dma_kernel (direct global-to-LDS loads, query block in registers)"
    return "mfma_scores_fixed_kernel" if d in (256, 384, 512, 768, 1024) else "mfma_scores_kernel"


def mfma_utilisation(name, flops, avg_ms, metric):
    """The batch scorer's fp32 matrix-core rate against the dense fp32 MFMA
    peak, and (from the committed PMC summary, when it matches the sources)
    the fraction of SIMD cycles the matrix cores were busy."""
    achieved = flops / (avg_ms * 1e-3) / 1e12
    out = {"achieved_tflops": achieved, "peak_tflops": FP32_MFMA_PEAK_TFLOPS,
           "frac_of_peak": achieved / FP32_MFMA_PEAK_TFLOPS, "flops_per_launch": flops, "busy_frac": None}
    rec = profile_record(TRAFFIC_PROFILES[name][0]) if (metric == "dot" and name in TRAFFIC_PROFILES) else None
    if rec and "mfma_busy_frac" in rec:
        out["busy_frac"] = rec["mfma_busy_frac"]
        out["busy_source"] = "profiles/" + TRAFFIC_PROFILES[name][0] + ".json (SQ_VALU_MFMA_BUSY_CYCLES)"
    return out


def run_batched(args, torch, eng, corpus, qhost, qdev, ks, name, gen_s):
    n, d = corpus.shape
    q = qdev.shape[0]
    stream = torch.cuda.current_stream()
    outs = {k: (torch.empty((q, k), dtype=torch.int32, device="cuda"),
                torch.empty((q, k), dtype=torch.float32, device="cuda")) for k in ks}
    for _ in range(args.warmup):
        for k in ks:
            eng.search_resident(qdev, k, *outs[k], stream=stream, metric=args.metric)
    torch.cuda.synchronize()
    eng.profile(True)
    lat = {k: [] for k in ks}
    mf = {k: [] for k in ks}
    part = {k: [] for k in ks}
    merge = {k: [] for k in ks}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for k in ks:
            s = time.perf_counter_ns()
            eng.search_resident(qdev, k, *outs[k], stream=stream, metric=args.metric)
            stream.synchronize()
            lat[k].append((time.perf_counter_ns() - s) / 1e3)
            total, mfma, sel = eng.profile_read()
            part[k].append(sel)
            merge[k].append(total)
            mf[k].append(mfma)
    wall = time.perf_counter() - t0
    eng.profile(False)
    corpus_bytes = n * d * 4 + q * d * 4 + (n * 4 if args.metric == "cosine" else 0)
    flops = 2.0 * n * d * q
    per_k = {}
    for k in ks:
        mfma_ms = float(np.mean(mf[k]))
        per_k[str(k)] = {"batches_per_s": len(lat[k]) / (np.sum(lat[k]) / 1e6),
                         "queries_per_s": q * len(lat[k]) / (np.sum(lat[k]) / 1e6),
                         "p50_us": pct(lat[k], 50), "p99_us": pct(lat[k], 99),
                         "device_p50_us": pct(np.asarray(merge[k]) * 1e3, 50),
                         "device_p99_us": pct(np.asarray(merge[k]) * 1e3, 99),
                         "mfma_kernel_avg_us": mfma_ms * 1e3,
                         "select_kernel_avg_us": float(np.mean(part[k])) * 1e3,
                         "device_avg_us": float(np.mean(merge[k])) * 1e3,
                         "mfma_kernel_gbs": corpus_bytes / (mfma_ms * 1e-3) / 1e9,
                         "mfma_kernel_tflops": flops / (mfma_ms * 1e-3) / 1e12}
    all_mf = np.concatenate([np.asarray(mf[k]) for k in ks])
    achieved = corpus_bytes / (float(np.mean(all_mf)) * 1e-3) / 1e9
    line = {"metric": f"queries/s ({name}{', cosine' if args.metric == 'cosine' else ''})", "value": q * args.steps * len(ks) / wall, "unit": "queries/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": f"{name}: batch of {q} queries vs resident {n} x {d} fp32, K in {list(ks)}",
                       "n": n, "d": d, "q": q, "ks": list(ks), "metric": args.metric},
            "per_k": per_k,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": workload_traffic(name, args.metric),
                         "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, profiles/)",
                         "kernel": mfma_kernel_name(n, d, args.metric), "bytes_per_launch": corpus_bytes,
                         "avg_launch_us": float(np.mean(all_mf)) * 1e3},
            "mfma": mfma_utilisation(name, flops, float(np.mean(all_mf)), args.metric),
            "input_gen_s": gen_s}
    if args.metric == "dot" and not args.no_filtered_leg:
        line["filtered_exact"] = batched_filtered_leg(args, torch, eng, qdev, ks, n, d)
    if not args.no_cpu_baseline:
        import oracle
        from tests.gpu_util import check_retrieval
        kmax = max(ks)
        gi, gs = eng.search_resident(qdev, kmax, metric=args.metric)
        torch.cuda.synchronize()
        gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
        s = time.perf_counter()
        o_idx, o_sc = oracle.search(corpus, qhost, kmax, metric=1 if args.metric == "cosine" else 0)
        el = time.perf_counter() - s
        for qi in range(q):
            check_retrieval(gi[qi], gs[qi], o_idx[qi], o_sc[qi], corpus, qhost[qi], oracle, metric=args.metric)
        line["cpu_baseline"] = {"value": q / el, "unit": "queries/s", "cores": oracle.num_threads(),
                                "kind": "oracle", "sample": f"the full batch of {q} queries at K={kmax}",
                                "host_cores": host_cores(), "cpu_model": cpu_model(), "parity": "ok"}
    eng.close()
    return line


def run_int32(args, torch, ResidentTopK, workloads):
    name = args.workload
    w = workloads.WORKLOADS[name]
    t = time.perf_counter()
    v = workloads.int32_values(n=w["n"], dup_fraction=w["dup_fraction"], config_id=w["config_id"])
    gen_s = time.perf_counter() - t
    n = v.shape[0]
    ks = tuple(w["ks"])
    vdev = torch.from_numpy(v).cuda()
    eng = ResidentTopK(max_n=1, max_d=1, max_k=max(ks), max_q=1)
    stream = torch.cuda.current_stream()
    outs = {k: (torch.empty(k, dtype=torch.int32, device="cuda"), torch.empty(k, dtype=torch.int32, device="cuda"))
            for k in ks}
    for _ in range(args.warmup):
        for k in ks:
            eng.topk_select(vdev, k, *outs[k], stream=stream)
    torch.cuda.synchronize()
    eng.profile(True)
    lat = {k: [] for k in ks}
    part = {k: [] for k in ks}
    merge = {k: [] for k in ks}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for k in ks:
            s = time.perf_counter_ns()
            eng.topk_select(vdev, k, *outs[k], stream=stream)
            stream.synchronize()
            lat[k].append((time.perf_counter_ns() - s) / 1e3)
            total, _, kern = eng.profile_read()
            part[k].append(kern)
            merge[k].append(total)
    wall = time.perf_counter() - t0
    eng.profile(False)
    nbytes = n * 4
    per_k = {str(k): {"calls_per_s": len(lat[k]) / (np.sum(lat[k]) / 1e6), "p50_us": pct(lat[k], 50),
                      "p99_us": pct(lat[k], 99), "device_p50_us": pct(np.asarray(merge[k]) * 1e3, 50),
                      "device_p99_us": pct(np.asarray(merge[k]) * 1e3, 99),
                      "scan_kernel_avg_us": float(np.mean(part[k])) * 1e3,
                      "scan_kernel_gbs": nbytes / (float(np.mean(part[k])) * 1e-3) / 1e9} for k in ks}
    all_part = np.concatenate([np.asarray(part[k]) for k in ks])
    achieved = nbytes / (float(np.mean(all_part)) * 1e-3) / 1e9
    line = {"metric": f"top-K calls/s ({name})", "value": args.steps * len(ks) / wall, "unit": "calls/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int32",
            "data": "synthetic",
            "config": {"workload": f"{name}: raw top-K over {n} int32 (uniform, {w['dup_fraction']:.0%} duplicated), "
                                   f"K in {list(ks)}",
                       "n": n, "ks": list(ks)},
            "per_k": per_k,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": workload_traffic(name),
                         "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE, profiles/)",
                         "kernel": "select_topk_kernel",
                         "bytes_per_launch": nbytes, "avg_launch_us": float(np.mean(all_part)) * 1e3},
            "input_gen_s": gen_s}
    if not args.no_cpu_baseline:
        import oracle
        from tests.gpu_util import check_exact_topk_property
        m = min(n, 10_000_000)
        s = time.perf_counter()
        o_idx, o_val = oracle.topk(v[:m], max(ks))
        el = time.perf_counter() - s
        for k in ks:
            gi, gv = eng.topk_select(vdev, k)
            torch.cuda.synchronize()
            check_exact_topk_property(gi.cpu().numpy(), gv.cpu().numpy(), v)
        line["cpu_baseline"] = {"value": (m / n) / el, "unit": "calls/s", "cores": oracle.num_threads(),
                                "kind": "oracle",
                                "sample": f"the first {m} of {n} values at K={max(ks)}, scaled to a full call; "
                                          "GPU answers checked exactly by rank counting over all values",
                                "host_cores": host_cores(), "cpu_model": cpu_model(), "parity": "ok"}
    eng.close()
    return line


def copy_calibration(torch, nbytes, reps):
    """A plain device copy of known size, for scaling FETCH_SIZE / WRITE_SIZE."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}))


def run_one(args, torch, ResidentTopK, workloads):
    if workloads.WORKLOADS[args.workload]["kind"] == "int32":
        return run_int32(args, torch, ResidentTopK, workloads)
    return run_retrieval(args, torch, ResidentTopK, workloads)


def run_suite(args, torch, ResidentTopK, workloads):
    """The other configurations, one after the other, each with its own
    protocol; every one checks its GPU answers against the oracle."""
    import copy
    out = {}
    for name, proto in SUITE:
        sub = copy.copy(args)
        sub.workload = name
        sub.steps = proto["steps"]
        sub.warmup = proto["warmup"]
        sub.num_queries = 1000
        sub.latency_queries = 0
        sub.streams = 1
        sub.filtered = False
        sub.metric = "dot"
        sub.no_filtered_leg = not proto.get("filtered_leg", False)
        sub.cpu_budget = proto.get("cpu_budget", args.cpu_budget)
        sub.cpu_queries = proto.get("cpu_queries", args.cpu_queries)
        t0 = time.perf_counter()
        print(f"[bench] {name}: start", file=sys.stderr, flush=True)
        line = run_one(sub, torch, ResidentTopK, workloads)
        line["wall_s"] = time.perf_counter() - t0
        print(f"[bench] {name}: done in {line['wall_s']:.1f} s", file=sys.stderr, flush=True)
        out[name] = line
        torch.cuda.empty_cache()
    return out


def register_custom(args, workloads):
    """A free-form synthetic workload of the same recipe (--n given)."""
    ks = tuple(int(k) for k in str(args.k).split(","))
    if args.dtype == "int32":
        workloads.WORKLOADS["custom"] = dict(config_id=args.seed, n=args.n, ks=ks, kind="int32",
                                             dup_fraction=args.dup_fraction)
    else:
        if args.d is None:
            raise SystemExit("--d is required for a retrieval workload")
        workloads.WORKLOADS["custom"] = dict(config_id=args.seed, n=args.n, d=args.d, ks=ks,
                                             queries=args.queries, kind="retrieval", batch=args.batch)
    return "custom"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="run one configuration alone (default: c3_1m_1024 as the headline, then the others)")
    ap.add_argument("--headline-only", action="store_true", help="skip the other configurations")
    ap.add_argument("--metric", default="dot", choices=("dot", "cosine"),
                    help="similarity for the retrieval workloads (the headline line is the inner product)")
    ap.add_argument("--filtered", action="store_true",
                    help="single-query workloads: search_resident_filtered (bf16 pass + exact fp32 re-rank)")
    ap.add_argument("--filter-storage", choices=["auto", "bf16", "fp8"], default="auto",
                    help="first pass of the single-query filtered search (auto: fp8 for a large corpus)")
    ap.add_argument("--no-filtered-leg", action="store_true",
                    help="skip the extra timing of search_resident_filtered on single-query workloads")
    ap.add_argument("--streams", type=int, default=1,
                    help="single-query workloads: engines sharing the corpus, one stream each, searching concurrently")
    ap.add_argument("--num-queries", type=int, default=1000)
    ap.add_argument("--latency-queries", type=int, default=1000,
                    help="headline: sequential queries per K for the latency distribution")
    ap.add_argument("--batcher-clients", type=int, default=64,
                    help="concurrent single-query clients of the dynamic-batching leg (0: skip it)")
    ap.add_argument("--batcher-requests", type=int, default=40, help="blocking searches per client")
    ap.add_argument("--batcher-wait-us", type=int, default=300, help="batcher's longest wait for a batch to fill")
    ap.add_argument("--cpu-queries", type=int, default=40)
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time in cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--e2e-reps", type=int, default=200)
    ap.add_argument("--copy-calibration", type=int, default=0, help="bytes; run only a plain copy kernel")
    ap.add_argument("--n", type=int, default=None, help="free-form workload: rows (or int32 values)")
    ap.add_argument("--d", type=int, default=None, help="free-form workload: depth")
    ap.add_argument("--k", default="8,32,100", help="free-form workload: K values, comma-separated")
    ap.add_argument("--queries", type=int, default=100, help="free-form workload: queries")
    ap.add_argument("--batch", type=int, default=1, help="free-form workload: queries per batch (<= 32)")
    ap.add_argument("--seed", type=int, default=1000, help="free-form workload: config id of the seed sequence")
    ap.add_argument("--dtype", choices=("f32", "int32"), default="f32", help="free-form workload: data type")
    ap.add_argument("--dup-fraction", type=float, default=0.01, help="free-form int32 workload: duplicated fraction")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the row-sharded multi-GPU design is "
                                   "documented but not implemented", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration, max(1, args.steps))
        return
    import workloads
    from top_search_resident_amd import ResidentTopK
    suite = args.workload is None and args.n is None and not args.headline_only
    if args.n is not None:
        args.workload = register_custom(args, workloads)
    elif args.workload is None:
        args.workload = "c3_1m_1024"
    if args.workload != "c3_1m_1024" or args.filtered or args.metric != "dot":
        args.latency_queries = 0
    print(f"[bench] {args.workload}: start", file=sys.stderr, flush=True)
    line = run_one(args, torch, ResidentTopK, workloads)
    if suite and args.streams == 1:
        line["workloads"] = run_suite(args, torch, ResidentTopK, workloads)
    line["environment"] = environment(torch, workloads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
