"""Decode-step benchmark of the BasisKV hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one layer's whole decode path over one batch: one call of
basiskv_decode_step (the step's new token compressed into the cache, query
projection, page scoring, top-k selection, sparse attention, reconstruction).
Inputs are seeded synthetic arrays already resident in device memory when
the timed region starts; K steps run back to back on one stream and are
bracketed by torch.cuda.synchronize().  A second pass runs the same step as
its separate library calls, each call K times back to back between two HIP
events recorded on that stream, which gives every launch's average duration.
Then 100 steps are timed one by one with L2 and the memory-side cache flushed
before each ("cold_step"); for the prefill + decode workload, the prompts'
compression and the 128 decode steps of growing context are timed as well
("prefill", "decode_sequence").

The default workload is the Llama-3.1-8B-shaped layer at 32K context
(batch 8, 32 query / 8 KV heads, head dim 128, latent width 64, residual
rank 32, 32-token pages, 128 pages kept per KV head).  One JSON line goes to
stdout: value = algorithmic HBM bytes of the step / step time (GB/s), with
the step time itself as ms_per_step and us_per_layer; "roofline" covers the
dominant kernel (page scoring, route_scan_kernel); "cpu_baseline" times the
float64 oracle on a bounded sample of the same workload on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode µs/layer + achieved HBM GB/s vs peak, 8B-shaped GQA at 32K ctx, 1 GPU"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# sources the route_scan and attend_split kernels are compiled from: counter
# figures taken with other sources are not reported
KERNEL_SOURCES = ("sparse_decode_attention_latent_amd/csrc/route.hip",
                  "sparse_decode_attention_latent_amd/csrc/attend.hip",
                  "sparse_decode_attention_latent_amd/csrc/common.hpp",
                  "sparse_decode_attention_latent_amd/csrc/topk.hpp",
                  "sparse_decode_attention_latent_amd/csrc/decode_bodies.hpp")
PMC_KERNELS = ("route_scan_kernel", "attend_split_kernel")


def pmc_summary_path(workload_name):
    return os.path.join(ROOT, "profiles", f"hbm_counters_{workload_name.replace('-', '_')}.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # a step is ~0.1 ms: a few hundred steps give a timed region of tens of
    # milliseconds, long enough for clocks and caches to settle (a 50-step
    # run after 5 warm-up steps reads about 4% slower)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama8b-ctx32k")
    ap.add_argument("--context-sweep", action="store_true",
                    help="instead of the bench line: the method's step against dense decode "
                         "attention over 24K-96K contexts at batch 1 and 8 (JSON lines)")
    ap.add_argument("--cold-steps", type=int, default=100,
                    help="steps timed one by one after a 512 MiB cache flush (0 = skip)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time of the oracle sample (0 = skip)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run a 64 MiB read + 64 MiB write elementwise kernel (torch.neg) "
                         "five times, the reference for HBM counter scaling")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="summarise a rocprofv3 --kernel-trace --stats run of this script "
                         "(markdown to stdout): per-kernel durations, and the library's "
                         "kernels split by pass in dispatch order")
    ap.add_argument("--mfma-summary", nargs="+", metavar="COUNTER_DIR",
                    help="summarise rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 runs of this script, "
                         "one directory per workload named mfma_<workload> (markdown to stdout)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE; --calibration-copy) into "
                         "profiles/hbm_counters_<workload>.json")
    return ap.parse_args()


CALIB_BYTES = 64 << 20
FLUSH_BYTES = 512 << 20  # > L2 (4 MB per XCD) + the 256 MB memory-side cache


def calibration_copy():
    import torch
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def pmc_summary(fetch_dir, write_dir, workload_name):
    """Per-dispatch HBM bytes of route_scan_kernel and attend_split_kernel from
    two counter runs, scaled by what the same counters read for the
    calibration kernel; written to profiles/hbm_counters_<workload>.json."""
    import csv
    import glob

    def per_kernel(d):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            sys.exit(f"no counter_collection.csv under {d}")
        vals = {k: [] for k in PMC_KERNELS + ("calib",)}
        for f in files:
            for row in csv.DictReader(open(f)):
                name = row["Kernel_Name"]
                for k in PMC_KERNELS:
                    if k in name:
                        vals[k].append(float(row["Counter_Value"]))
                if "neg_kernel" in name:
                    vals["calib"].append(float(row["Counter_Value"]))
        if any(not v for v in vals.values()):
            sys.exit(f"{d}: a kernel or the calibration dispatches are missing")
        return {k: sum(v) / len(v) for k, v in vals.items()}

    fetch, write = per_kernel(fetch_dir), per_kernel(write_dir)
    ref_kib = CALIB_BYTES / 1024
    fetch_scale = ref_kib / fetch["calib"]
    write_scale = ref_kib / write["calib"]
    kernels = {}
    for k in PMC_KERNELS:
        kernels[k] = {"fetch_size_kib_per_dispatch": round(fetch[k], 1),
                      "write_size_kib_per_dispatch": round(write[k], 1),
                      "hbm_bytes_per_launch": round((fetch[k] * fetch_scale
                                                     + write[k] * write_scale) * 1024)}
    out = {"workload": workload_name, "source_sha256": kernel_source_sha(),
           "kernels": kernels,
           "calibration": {"kernel": "torch.neg over 64 MiB float32 (64 MiB read, 64 MiB written)",
                           "fetch_size_kib": round(fetch["calib"], 1),
                           "write_size_kib": round(write["calib"], 1),
                           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4)},
           "commands": [f"cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {c} --output-format csv -d "
                        f"$REPO/{os.path.relpath(d, ROOT)} -o run -- python3 $REPO/bench.py "
                        f"--workload {workload_name} --steps 5 --warmup 2 --cold-steps 0 "
                        f"--cpu-seconds 0 --calibration-copy"
                        for c, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir))],
           "summary_command": f"python3 bench.py --workload {workload_name} --pmc-summary "
                              f"{os.path.relpath(fetch_dir, ROOT)} {os.path.relpath(write_dir, ROOT)}"}
    path = pmc_summary_path(workload_name)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))


def _csv_rows(d, suffix):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        sys.exit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _kernel_name(name):
    """A kernel's demangled name without its return type and parameter list."""
    name = name.strip()
    if name.startswith("void "):
        name = name[len("void "):]
    if name.endswith(")"):
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                return name[:i]
    return name


def trace_summary(trace_dir):
    """Markdown summary of one rocprofv3 kernel trace of this script: rocprofv3's
    own per-kernel statistics, then the library's kernels (bkv::) split by pass
    in dispatch order.  Passes: the one-call steps (up to the first separate
    compression call, append_kernel, which only the stage pass launches), the
    stage pass (separate calls), and what follows it (cold steps after each
    cache-flushing read, whose reduction kernel opens that pass; the prefill and
    the decode sequence of the prefill + decode workload)."""
    lines = []
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    total = sum(float(r["TotalDurationNs"]) for r in stats)
    lines += ["| kernel | calls | avg µs | min µs | max µs | share % |", "|---|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = _kernel_name(r["Name"])
        name = name if len(name) <= 110 else name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{100 * float(r['TotalDurationNs']) / total:.1f} |")
    trace = _csv_rows(trace_dir, "kernel_trace.csv")
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = [_kernel_name(r["Kernel_Name"]) for r in trace]
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace]
    s1 = next((i for i, n in enumerate(names) if "append_kernel" in n), len(names))
    s2 = next((i for i in range(s1, len(names)) if "reduce_kernel" in names[i]
               or "compress_kernel" in names[i]), len(names))
    lines += ["", "The library's kernels split by pass (dispatch order in the trace):", "",
              "| kernel | pass | calls | avg µs |", "|---|---|---|---|"]
    for label, lo, hi in (("one-call steps", 0, s1), ("stage pass", s1, s2),
                          ("after the stage pass", s2, len(names))):
        acc = {}
        for n, d in zip(names[lo:hi], durs[lo:hi]):
            if n.startswith("bkv::"):
                acc.setdefault(n, []).append(d)
        for n, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| `{n}` | {label} | {len(v)} | {sum(v) / len(v):.2f} |")
    print("\n".join(lines))


def mfma_summary(dirs):
    """Markdown table of MfmaUtil and MfmaFlopsBF16 per dispatch of every
    matrix-issuing kernel, one counter directory per workload."""
    lines = ["| workload | kernel | dispatches | MfmaUtil % | MFMA GFLOP per dispatch |",
             "|---|---|---|---|---|"]
    for d in dirs:
        wl = os.path.basename(os.path.normpath(d))
        wl = wl[len("mfma_"):] if wl.startswith("mfma_") else wl
        acc = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            k = (_kernel_name(r["Kernel_Name"]), r["Counter_Name"])
            acc.setdefault(k, []).append(float(r["Counter_Value"]))
        kernels = sorted({k for k, c in acc if k.startswith("bkv::")})
        rows = []
        for k in kernels:
            util = acc.get((k, "MfmaUtil"), [0.0])
            flops = acc.get((k, "MfmaFlopsBF16"), [0.0])
            if max(flops) <= 0:
                continue
            rows.append((sum(util) / len(util), k, len(util), sum(flops) / len(flops) / 1e9))
        for u, k, n, g in sorted(rows, reverse=True):
            lines.append(f"| {wl} | `{k}` | {n} | {u:.2f} | {g:.3f} |")
    print("\n".join(lines))


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload_name, kernel="route_scan_kernel"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary, or None when there is none for this workload or the kernels'
    sources changed since the counters were taken."""
    path = pmc_summary_path(workload_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        s = json.load(f)
    if s.get("workload") != workload_name or s.get("source_sha256") != kernel_source_sha():
        return None
    return float(s["kernels"][kernel]["hbm_bytes_per_launch"])


def cpu_baseline(wl, inp, target_seconds):
    """The float64 oracle, as it stands, on whole sequences of the workload,
    cycling over the batch until about target_seconds have passed (at least
    one sequence).  BLAS runs with one thread per core this process may use
    (its CPU affinity set); the CPU model is recorded beside the figure."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import basiskv_ref as ref
    from sparse_decode_attention_latent_amd import traffic

    st = inp["storage"]
    cst = inp.get("cache_storage", st)
    f = {k: ref.storage_to_f64(inp[k], st) for k in ("A", "Bf", "P", "Q", "E", "W_O")}
    B = inp["q"].shape[0]
    one = _shape(wl, 1, inp)
    seqs = []
    for b in range(B):
        x = {k: ref.storage_to_f64(inp[k][b:b + 1], cst if k in ("z", "r", "kc") else st)
             for k in ("q", "z", "r", "kc", "k_new", "v_new")}
        x["L"] = inp["seq_lens"][b:b + 1]
        seqs.append(x)
    n_cores = len(os.sched_getaffinity(0))
    limiter = threadpool_limits(limits=n_cores, user_api="blas")
    done, elapsed, nbytes = 0, 0.0, 0
    while elapsed < target_seconds or done == 0:
        x = seqs[done % B]
        t0 = time.perf_counter()
        ref.decode_step(x["q"], x["z"], x["r"], x["kc"], x["L"], f["A"], f["Bf"], f["P"], f["Q"],
                        f["E"], f["W_O"], rb=wl.r_b, page_size=wl.page_size, top_k=wl.top_k,
                        n_pages_out=-(-x["z"].shape[2] // wl.page_size), storage=st,
                        k_new=x["k_new"], v_new=x["v_new"], recent_tokens=wl.recent_tokens,
                        cache_storage=cst, rope_inv_freq=inp.get("rope_inv_freq"))
        elapsed += time.perf_counter() - t0
        nbytes += traffic.step_bytes(one, x["L"])["total"]
        done += 1
    threads = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    limiter.unregister()
    return {"value": round(nbytes / elapsed / 1e9, 4), "unit": "GB/s",
            "cores": max(threads) if threads else 1, "affinity_cores": n_cores,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} single-sequence decode steps (append, route, select, attend, "
                      f"reconstruct) cycling over the {B} sequences of the same workload, "
                      f"float64 numpy oracle, {elapsed:.1f} s",
            "us_per_layer_equiv": round(elapsed / done * B * 1e6, 1)}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or the platform's processor string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cold_steps(prob, n, flush_bytes=FLUSH_BYTES):
    """Step times with L2 and the memory-side cache flushed before every step:
    a 512 MiB read between steps, outside the timed pair of events (a read,
    so that the caches are left holding clean lines; a fill would leave dirty
    lines whose write-back the step would pay for)."""
    import torch
    flush = torch.zeros(flush_bytes // 4, dtype=torch.float32, device="cuda")
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t = []
    for _ in range(n):
        flush.sum()
        e0.record()
        prob.decode_step()
        e1.record()
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1) * 1e3)
    del flush
    return _dist(t)


def _dist(t):
    t = sorted(t)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"n": len(t), "median_us": round(q(0.5), 3), "p10_us": round(q(0.1), 3),
            "p90_us": round(q(0.9), 3), "min_us": round(t[0], 3), "max_us": round(t[-1], 3)}


def prefill_and_sequence(wl, prob, inp, steps):
    """The prefill + decode workload's two other parts: compression of the
    prompts (prefill_batch x prefill_tokens, back to back between two HIP
    events), and its decode_steps one-call steps with the context growing by
    one token per step up to wl.ctx, each step timed by its own events."""
    import torch

    from sparse_decode_attention_latent_amd import synth, traffic
    from sparse_decode_attention_latent_amd.runner import PrefillProblem, to_device

    # -- prefill ---------------------------------------------------------------
    B, T = wl.prefill_batch, wl.prefill_tokens
    k, v = synth.kv_activations(wl, batch=B, tokens=T, stream=0)
    pre = PrefillProblem(wl, k, v, synth.factors(wl), storage=wl.storage)
    for _ in range(3):
        pre.run()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        pre.run()
    e1.record()
    torch.cuda.synchronize()
    pre_us = e0.elapsed_time(e1) / reps * 1e3
    e = 2 if wl.storage == "bf16" else 4
    pre_bytes = traffic.prefill_bytes(B, T, wl.n_kv_heads, wl.head_dim, wl.r_v, wl.r_b, wl.r_q, e)
    del pre

    # -- decode steps with a growing context ----------------------------------
    Bd = inp["q"].shape[0]
    qs = [to_device(synth.step_queries(wl, batch=Bd, step=i), wl.storage) for i in range(steps)]
    L_last = int(inp["seq_lens"].max())
    shape = _shape(wl, Bd, inp)
    t, gbs = [], []
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    for i in range(steps):
        L = L_last - (steps - 1) + i
        prob.seq_lens.fill_(L)
        prob.start_pos.fill_(L - 1)
        prob.q.copy_(qs[i])
        e0.record()
        prob.decode_step()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        t.append(us)
        gbs.append(traffic.step_bytes(shape, [L] * Bd)["total"] / (us * 1e-6) / 1e9)
    # back to the full-context state the other passes use
    prob.seq_lens.copy_(torch.from_numpy(prob.seq_lens_host).to(prob.seq_lens.device))
    prob.start_pos.copy_(prob.seq_lens - 1)
    prob.q.copy_(to_device(inp["q"], wl.storage))
    torch.cuda.synchronize()
    d = _dist(t)
    d.update({"ctx_first": L_last - (steps - 1), "ctx_last": L_last, "batch": Bd,
              "gbs_median": round(sorted(gbs)[len(gbs) // 2], 1)})
    return ({"batch": B, "tokens": T, "us": round(pre_us, 3),
             "algorithmic_bytes": pre_bytes, "gbs": round(pre_bytes / (pre_us * 1e-6) / 1e9, 1)},
            d)


SWEEP_CTX = (24576, 32768, 49152, 65536, 98304)
SWEEP_BATCH = (1, 8)
SWEEP_WORKLOADS = ("llama8b-ctx32k", "llama8b-ctx32k-b16r16-page4", "llama8b-ctx32k-fp8",
                   "llama8b-ctx32k-b16r16-page4-fp8")


def _time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def context_sweep(steps, warmup):
    """The MI355X analogue of the pages' sparse-decoding latency table: one
    decode step of the method against dense decode attention plus the output
    projection, over 24K-96K contexts at batch 1 and 8.  Timing-only state:
    pools and queries are seeded N(0, 1) draws made on the device (values do
    not change the work of either path).  One JSON line per point."""
    import torch

    from sparse_decode_attention_latent_amd import synth, traffic
    from sparse_decode_attention_latent_amd.configs import workload
    from sparse_decode_attention_latent_amd.runner import DecodeProblem, DenseProblem

    for B in SWEEP_BATCH:
        for T in SWEEP_CTX:
            row = {"batch": B, "ctx": T}
            dense_us = None
            for name in SWEEP_WORKLOADS:
                wl = workload(name).with_(batch=B, ctx=T)
                fac = dict(synth.factors(wl), storage=wl.storage)
                prob = DecodeProblem(wl, fac, device_random=(B, T, 7))
                us = _time_calls(prob.decode_step, steps, warmup)
                shape = traffic.StepShape(batch=B, n_q_heads=wl.n_q_heads,
                                          n_kv_heads=wl.n_kv_heads, head_dim=wl.head_dim,
                                          hidden=wl.hidden, r_v=wl.r_v, r_b=wl.r_b, r_q=wl.r_q,
                                          page_size=wl.page_size, max_pages=prob.max_pages,
                                          top_k=wl.top_k, elem=2,
                                          recent_tokens=wl.recent_tokens,
                                          cache_elem=1 if wl.cache == "fp8" else 0)
                gbs = traffic.step_bytes(shape, [T] * B)["total"] / (us * 1e-6) / 1e9
                row[name] = {"us": round(us, 2), "gbs": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
                if dense_us is None:  # dense baseline on the first workload's pools
                    dense = DenseProblem(prob, seed=11)
                    dense_us = _time_calls(dense.step, steps, warmup)
                    dbytes = (B * wl.n_kv_heads * T * 2 * wl.head_dim * 2
                              + wl.hidden * wl.n_q_heads * wl.head_dim * 2)
                    dgbs = dbytes / (dense_us * 1e-6) / 1e9
                    row["dense"] = {"us": round(dense_us, 2), "gbs": round(dgbs, 1),
                                    "hbm_frac": round(dgbs / HBM_PEAK_GBS, 4)}
                    del dense
                row[name]["speedup_vs_dense"] = round(dense_us / us, 3)
                del prob
                torch.cuda.empty_cache()
            print(json.dumps(row), flush=True)


def _shape(wl, B, inp):
    from sparse_decode_attention_latent_amd import traffic
    T = inp["z"].shape[2]
    return traffic.StepShape(batch=B, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads,
                             head_dim=wl.head_dim, hidden=wl.hidden, r_v=wl.r_v, r_b=wl.r_b,
                             r_q=wl.r_q, page_size=wl.page_size, max_pages=-(-T // wl.page_size),
                             top_k=wl.top_k, elem=2 if inp["storage"] == "bf16" else 4,
                             recent_tokens=wl.recent_tokens,
                             cache_elem=1 if inp.get("cache_storage") == "fp8" else 0)


def main():
    args = parse()
    if args.context_sweep:
        import torch
        from sparse_decode_attention_latent_amd import api
        if not torch.cuda.is_available():
            sys.exit("bench.py needs a GPU")
        api.lib()
        context_sweep(args.steps, args.warmup)
        return
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload)
        return
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the decode path is built and measured on one GPU's share of the work; the "
              "multi-GPU sharding is a design, not a run.", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_decode_attention_latent_amd import api, synth, traffic
    from sparse_decode_attention_latent_amd.configs import workload
    from sparse_decode_attention_latent_amd.runner import DecodeProblem

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    api.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    if args.calibration_copy:
        calibration_copy()

    wl = workload(int(args.workload) if args.workload.isdigit() else args.workload)
    # for the prefill + decode workload the step measured is the last decode
    # step (context 131072)
    wl_step = wl
    log(f"[bench] generating inputs for {wl.name} ...")
    t0 = time.perf_counter()
    inp = synth.decode_inputs(wl_step)
    prob = DecodeProblem(wl_step, inp)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident ({time.perf_counter() - t0:.1f} s)")

    # the step as one library call (five launches: compression + projection,
    # scoring, selection, attention, reconstruction)
    for _ in range(args.warmup):
        prob.decode_step()
    torch.cuda.synchronize()

    K = args.steps
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    e_start.record()
    for _ in range(K):
        prob.decode_step()
    e_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    gpu_step_us = e_start.elapsed_time(e_end) / K * 1e3
    ms_per_step = wall / K * 1e3
    log(f"[bench] timed {K} steps in {wall * 1e3:.2f} ms")

    # per-launch durations: each stage's library call K times back to back
    # on the same stream, bracketed by one pair of HIP events (average per
    # launch, including the gap between consecutive launches); a stage whose
    # host-side call takes about as long as its launch is marked host-bound
    stages = ("append", "project", "score", "select", "attend", "reconstruct")
    calls = [prob.append, prob.project, prob.score, prob.select, prob.attend, prob.reconstruct]
    if prob.rope_inv_freq is not None:  # RoPE: scoring reads the raw queries, no projection
        stages, calls = stages[:1] + stages[2:], calls[:1] + calls[2:]
    for _ in range(2):
        prob.step_unfused()
    torch.cuda.synchronize()
    per_stage, host_bound = {}, {}
    for s_name, call in zip(stages, calls):
        call()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        h0 = time.perf_counter()
        e0.record()
        for _ in range(K):
            call()
        e1.record()
        host_us = (time.perf_counter() - h0) / K * 1e6
        torch.cuda.synchronize()
        per_stage[s_name] = e0.elapsed_time(e1) / K * 1e3
        host_bound[s_name] = host_us >= 0.9 * per_stage[s_name]
    prob.step_unfused()  # leave the cache and outputs as one step leaves them
    torch.cuda.synchronize()

    # cold-cache steps (flushed before each), and for the prefill + decode
    # workload its prefill and its sequence of decode steps
    cold = cold_steps(prob, args.cold_steps) if args.cold_steps > 0 else None
    prefill = sequence = None
    if wl.decode_steps > 0:
        log(f"[bench] prefill and {wl.decode_steps} decode steps ...")
        prefill, sequence = prefill_and_sequence(wl, prob, inp, wl.decode_steps)

    shape = _shape(wl_step, inp["q"].shape[0], inp)
    sb = traffic.step_bytes(shape, inp["seq_lens"])
    value = sb["total"] / (ms_per_step * 1e-3) / 1e9
    score_gbs = sb["score"] / (per_stage["score"] * 1e-6) / 1e9
    traffic_bytes = measured_traffic(wl.name)
    attend_traffic = measured_traffic(wl.name, "attend_split_kernel")

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the float64 oracle on the host ...")
        cpu = cpu_baseline(wl_step, inp, args.cpu_seconds)

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "us_per_layer": round(ms_per_step * 1e3, 3), "gpu_us_per_step": round(gpu_step_us, 3),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.storage if wl.cache == wl.storage else f"{wl.storage} (E4M3 cache pages)",
        "data": "synthetic (seeded generator; no weights or datasets)",
        "config": {"workload": wl.name, "batch": shape.batch, "ctx": int(inp["z"].shape[2]),
                   "n_q_heads": wl.n_q_heads, "n_kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "hidden": wl.hidden, "page_size": wl.page_size,
                   "r_v": wl.r_v, "r_b": wl.r_b, "r_q": wl.r_q, "top_k": wl.top_k,
                   "recent_tokens": wl.recent_tokens, "cache": wl.cache},
        "algorithmic_bytes_per_step": sb["total"],
        "stages_us": {k: round(v, 3) for k, v in per_stage.items()},
        "stages_host_bound": [k for k in stages if host_bound[k]],
        "stages_gbs": {k: round(sb[k] / (per_stage[k] * 1e-6) / 1e9, 1) for k in stages},
        "stages_hbm_bytes_measured": {"score": traffic_bytes, "attend": attend_traffic},
        "roofline": {"kernel": ("route_rope_kernel (page scoring with rotated predicted Keys)"
                                if prob.rope_inv_freq is not None
                                else "route_scan_kernel (page scoring)"), "bound": "hbm",
                     "achieved": round(score_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": sb["score"],
                     "launch_us": round(per_stage["score"], 3),
                     "traffic": traffic_bytes},
        "cold_step": cold,
        "cpu_baseline": cpu,
    }
    if prefill is not None:
        out["prefill"] = prefill
        out["decode_sequence"] = sequence
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
