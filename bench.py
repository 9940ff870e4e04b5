"""Throughput of the speculative-decoding verification sampler on one MI355X.

One step = one call of specverify_run over the whole batch of the
benchmarked workload (B = 64 sequences, gamma = 4 drafts, V = 128256, bf16
logits): every target and draft row is read, p and q are formed by
temperature softmax, the drafts are tested, the residual or bonus token is
sampled, and accepted lengths, tokens and diagnostics are written.  A step
is one kernel launch, made through a prepared run (SpecVerify.prepare: the
tensors are checked once per set of buffers, as a serving loop that keeps
its buffers would); the line also reports the host cost of a prepared call
and of a call of SpecVerify.run, which checks them every time.

Timing: the inputs are resident in HBM before the timed region; the steps
rotate over enough copies of the batch (> 2x the 256 MB Infinity Cache) that
no step reads logits the previous steps left in the cache.  Before the timed
region the bench checks one step's outputs, times every launch with HIP
events (the kernel's average duration for the roofline) and keeps the GPU
busy for a fraction of a second so that its clocks have settled; then W
untimed warm-up steps, then exactly K steps between two events on the launch
stream.  Prints one JSON line.

The same line carries: the per-step distribution (median, p10, p90), a
warm-cache figure (no rotation), the device's streaming-read ceiling for the
same bytes (the library's read probe), token-only drafts, the on-device
commit, microseconds per call of every other workload and of draft trees
(60-node trees, B = 16), and the float64
oracle timed on the host (one core, and a pool of worker processes).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                  [--no-cpu-baseline] [--no-other-workloads] [--copy-probe]
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --out FILE --command-fetch CMD
                  --command-write CMD      (writes the traffic summary from two
                                            rocprofv3 --pmc output folders)
  python bench.py --summarize-trace DIR --bench-json FILE --out FILE --command-fetch CMD
                                           (writes the kernel-trace summary of a
                                            rocprofv3 --kernel-trace --stats run of
                                            bench.py --no-other-workloads)
  python bench.py --summarize-sq DIR [DIR ...] --out FILE --command-fetch "CMD ;; CMD"
                                           (SQ counters of rocprofv3 --pmc runs)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rows/s + logits GB/s (frac of HBM peak), B=64 γ=4 V=128256 bf16"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published peak
MALL_BYTES = 256 << 20          # Infinity Cache
KERNEL = "verify_kernel"
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verifier_specverify_amd", "csrc", "specverify.hip")
PROFILES = os.path.join(ROOT, "profiles")
CPU_WORKERS_MAX = 16            # the host share of one GPU
SETTLE_S = 0.2                  # untimed GPU work before the warm-up, for the clocks


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"{KERNEL}_{workload}_hbm_traffic.txt")


def trace_file(workload: str) -> str:
    return os.path.join(PROFILES, f"{KERNEL}_{workload}_kernel_trace.txt")


def code_text(src: str) -> str:
    """The kernel source without its // comments, trailing blanks and empty
    lines: what the compiler sees (the source holds no "//" in strings)."""
    out = []
    for line in src.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            out.append(code)
    return "\n".join(out) + "\n"


def source_hash() -> str:
    """SHA-256 of the kernel source's code (comments and blank lines
    excluded), recorded in every profile summary: a summary whose hash
    differs was taken from other code."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b64_g4_v128256_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run plain device copies of the logits' size (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--summarize-sq", nargs="+", metavar="PMC_DIR")
    ap.add_argument("--out")
    ap.add_argument("--bench-json", help="the profiled bench's output (for --summarize-trace)")
    ap.add_argument("--command-fetch", default="")
    ap.add_argument("--command-write", default="")
    return ap.parse_args()


# ---------------------------------------------------------------- rocprofv3 summaries

def _pmc_rows(folder: str, counter: str):
    """(dispatch id, kernel name, value) of one counter from a rocprofv3 --pmc csv output."""
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {folder}")
    out = []
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return sorted(out)


PROBE_COPIES = 5   # plain copies of the logits' size that --copy-probe dispatches last


def _kernel_args(name: str):
    """Template arguments of a verification kernel launch (dtype, vector
    loads, chunks per lane, draft logits, tree), or None."""
    if f"{KERNEL}<" not in name:
        return None
    return name.split(f"{KERNEL}<", 1)[1].split(">", 1)[0].replace(" ", "").split(",")


def _with_draft(name: str) -> bool:
    """A launch of the verification kernel with draft logits (not a tree launch)."""
    a = _kernel_args(name)
    return a is not None and a[3] == "true" and (len(a) < 5 or a[4] == "false")


def summarize_trace(args):
    """The kernel-trace summary of a rocprofv3 --kernel-trace --stats run of
    this bench (with --no-other-workloads, its JSON line in --bench-json):
    the durations of the verification kernel's launches with draft logits
    inside the bench's timed region (launch indices from the JSON line, in
    start-time order), every such launch of the run, every kernel's
    statistics, and the kernel source's hash."""
    files = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_trace.csv"), recursive=True)
    stats = glob.glob(os.path.join(args.summarize_trace, "**", "*kernel_stats.csv"), recursive=True)
    if not files or not stats:
        raise SystemExit(f"no kernel_trace.csv / kernel_stats.csv under {args.summarize_trace}")
    if not args.bench_json:
        raise SystemExit("--summarize-trace needs --bench-json (the profiled bench's JSON line)")
    with open(args.bench_json) as f:
        line = json.loads([l for l in f if l.startswith("{")][-1])
    rl = line["roofline"]
    a, b = rl["timed_launches"]
    launches = []
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if _with_draft(r["Kernel_Name"]):
                launches.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    launches.sort()
    if len(launches) != rl["headline_launches"]:
        raise SystemExit(f"{len(launches)} launches with draft logits in the trace, the bench made "
                         f"{rl['headline_launches']}: profile a run with --no-other-workloads")
    d_all = np.array([e - s for s, e in launches], dtype=np.float64)
    d = d_all[a:b]
    span = (launches[b - 1][1] - launches[a][0]) / (b - a)
    lines = [f"# rocprofv3 kernel trace, workload {line['config']['workload']}",
             f"command: {args.command_fetch}",
             f"source_sha256: {source_hash()}",
             f"# {KERNEL} launches with draft logits inside the bench's timed region",
             f"timed_launches: {b - a}",
             f"verify_kernel_avg_ns: {d.mean():.1f}",
             f"verify_kernel_median_ns: {np.median(d):.1f}",
             f"verify_kernel_p10_ns: {np.percentile(d, 10):.1f}",
             f"verify_kernel_p90_ns: {np.percentile(d, 90):.1f}",
             f"timed_span_per_launch_ns: {span:.1f}",
             f"bench_ms_per_step_same_run: {line['ms_per_step']:.6f}",
             f"# every launch with draft logits of the run (checks, warm-up, settle, warm-cache)",
             f"all_launches: {len(d_all)}",
             f"all_avg_ns: {d_all.mean():.1f}",
             "# run_kernel_stats.csv (all kernels of the run):"]
    with open(stats[0]) as f:
        lines += [l.rstrip("\n") for l in f]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(args):
    """HBM traffic per launch of the verification kernel: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) averaged over its dispatches, each scaled by
    bytes / counter of the copy probe (the plain copies dispatched after the
    last verifier launch, of exactly the logits' size)."""
    from rejection_sampling_verifier_specverify_amd.workloads import WORKLOADS
    w = WORKLOADS[args.workload]
    copy_bytes = logit_bytes_of(w)
    res = {}
    for name, folder in (("FETCH_SIZE", args.summarize_pmc[0]), ("WRITE_SIZE", args.summarize_pmc[1])):
        rows = _pmc_rows(folder, name)
        ker = [(d, v) for d, k, v in rows if _with_draft(k)]
        if not ker:
            raise SystemExit(f"{name}: no {KERNEL} dispatch with draft logits in {folder}")
        last = max(d for d, _ in ker)
        # the probe's copies are the run's last ones
        cp = [v for d, k, v in rows if d > last and "copy" in k.lower()][-PROBE_COPIES:]
        if not cp:
            raise SystemExit(f"{name}: no copy-probe dispatch after the last {KERNEL} in {folder}")
        kv = float(np.mean([v for _, v in ker]))
        cv = float(np.mean(cp))
        res[name] = dict(kernel_kib=kv, copy_kib=cv, factor=copy_bytes / (cv * 1024.0),
                         n_kernel=len(ker), n_copy=len(cp))
    fetch = res["FETCH_SIZE"]["kernel_kib"] * 1024.0 * res["FETCH_SIZE"]["factor"]
    write = res["WRITE_SIZE"]["kernel_kib"] * 1024.0 * res["WRITE_SIZE"]["factor"]
    lines = [
        f"# HBM traffic of {KERNEL} (launches with draft logits), workload {w.name}",
        "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by",
        "# copy_bytes / (1024 * what the counter reads for a plain copy of copy_bytes).",
        f"command_fetch: {args.command_fetch}",
        f"command_write: {args.command_write}",
        f"source_sha256: {source_hash()}",
        f"copy_bytes: {copy_bytes}",
    ]
    for name, r in res.items():
        lines += [f"{name.lower()}_kernel_kib_per_dispatch: {r['kernel_kib']:.1f}",
                  f"{name.lower()}_kernel_dispatches: {r['n_kernel']}",
                  f"{name.lower()}_copy_kib_per_dispatch: {r['copy_kib']:.1f}",
                  f"{name.lower()}_copy_dispatches: {r['n_copy']}",
                  f"{name.lower()}_factor: {r['factor']:.5f}"]
    lines += [f"fetch_bytes_per_launch: {fetch:.0f}",
              f"write_bytes_per_launch: {write:.0f}",
              f"traffic_bytes_per_launch: {fetch + write:.0f}",
              f"algorithmic_logit_bytes_per_launch: {logit_bytes_of(w)}"]
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_sq(args):
    """SQ counters per dispatch of the verification kernel, with draft logits
    and token-only, averaged over the dispatches of one or more rocprofv3
    --pmc runs of this bench (one pass of counters per folder)."""
    rows = {}
    cmds = args.command_fetch.split(" ;; ")
    for folder in args.summarize_sq:
        files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {folder}")
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                a = _kernel_args(name)
                if a is None:
                    continue
                cls = "with_draft" if _with_draft(name) else "tree" if len(a) > 4 and a[4] == "true" else "token_only"
                rows.setdefault(r["Counter_Name"], {}).setdefault(cls, {}).setdefault(
                    int(r["Dispatch_Id"]), 0.0)
                rows[r["Counter_Name"]][cls][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    lines = [f"# SQ counters per dispatch of {KERNEL}, workload {args.workload}: launches with draft",
             "# logits and token-only launches, averaged over their dispatches",
             "# commands (from /tmp, TMPDIR=/tmp), one pass each:"]
    lines += [f"#   {c}" for c in cmds if c]
    lines += [f"source_sha256: {source_hash()}", "counter,with_draft,token_only"]
    for cnt in sorted(rows):
        v = [np.mean(list(rows[cnt][c].values())) if c in rows[cnt] else float("nan")
             for c in ("with_draft", "token_only")]
        lines.append(f"{cnt},{v[0]:.3f},{v[1]:.3f}")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def logit_bytes_of(w) -> int:
    """Every logit of the workload once: sum over sequences of (2 gamma + 1) rows of V."""
    from rejection_sampling_verifier_specverify_amd.workloads import make_inputs
    return int(make_inputs(w, seed=0).logit_bytes)


def _kv(fn: str):
    kv = {}
    with open(fn) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    return kv


def read_traffic(workload: str):
    """Traffic bytes per launch from the committed summary, or None when there
    is none or it was taken from another version of the kernel source."""
    fn = traffic_file(workload)
    if not os.path.exists(fn):
        return None
    kv = _kv(fn)
    if kv.get("source_sha256") != source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def read_profile_ns(workload: str):
    """Average duration (ns) of the verification kernel's launches with draft
    logits in the committed rocprofv3 kernel-trace summary, or None when it
    was taken from another version of the kernel source."""
    fn = trace_file(workload)
    if not os.path.exists(fn):
        return None
    kv = _kv(fn)
    if kv.get("source_sha256") != source_hash() or "verify_kernel_avg_ns" not in kv:
        return None
    return float(kv["verify_kernel_avg_ns"])


# ---------------------------------------------------------------- the oracle on the host

_POOL_INP = None


def _pool_work(args):
    from oracle import verify_batch
    seqs, = args
    inp = _POOL_INP
    verify_batch(inp.target, inp.draft, inp.draft_tokens, inp.uniforms, inp.temperatures, inp.cu_draft,
                 inp.workload.dtype, sequences=seqs)
    return sum(int(inp.gammas[b]) + 1 for b in seqs)


def cpu_baseline(inp, budget_s: float):
    """The float64 oracle on the host, cycling over the sequences of the
    benchmarked batch: one process and one thread for budget_s, then a pool of
    forked worker processes (one per core of the host's share, at most
    CPU_WORKERS_MAX) for budget_s.  Runs before any GPU work of this process."""
    import multiprocessing as mp
    from oracle import verify_batch
    B = inp.batch
    rows = seqs = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = seqs % B
        verify_batch(inp.target, inp.draft, inp.draft_tokens, inp.uniforms, inp.temperatures,
                     inp.cu_draft, inp.workload.dtype, sequences=[b])
        rows += int(inp.gammas[b]) + 1
        seqs += 1
    one = rows / (time.perf_counter() - t0)
    cores = max(1, min(len(os.sched_getaffinity(0)), CPU_WORKERS_MAX))
    global _POOL_INP
    _POOL_INP = inp
    chunks = [([b],) for b in range(B)]
    prows = 0
    with mp.get_context("fork").Pool(cores) as pool:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            prows += sum(pool.map(_pool_work, chunks, chunksize=max(1, B // (4 * cores))))
        dt = time.perf_counter() - t0
    pooled = prows / dt
    return dict(value=pooled, unit="rows/s", cores=cores, kind="oracle", single_core=one,
                sample=(f"float64 numpy oracle cycling over the {B} sequences of the benchmarked batch: "
                        f"{rows} target rows on one core in {budget_s:.0f} s, then {prows} rows on a pool of "
                        f"{cores} worker processes in {dt:.1f} s (value: the pool)"))


def cpu_commit_us(acc, toks, cu_draft, B, cap) -> float:
    """The commit oracle on one host thread: microseconds per call (about 1 s of calls)."""
    from oracle import commit_reference
    rows = np.zeros((B, cap), dtype=np.int32)
    lens = np.zeros(B, dtype=np.int32)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        commit_reference(acc, toks, cu_draft, rows, lens, cap)
        n += 1
    return (time.perf_counter() - t0) / n * 1e6


# ---------------------------------------------------------------- GPU measurement

def _prepare(w, seed, dev, token_only=False, inp=None):
    """Device copies of a workload's batch (enough to exceed 2x the Infinity
    Cache), a handle and output buffers."""
    import torch
    from rejection_sampling_verifier_specverify_amd.binding import SpecVerify
    from rejection_sampling_verifier_specverify_amd.workloads import make_inputs
    if inp is None:
        inp = make_inputs(w, seed=seed)
    B = inp.batch
    R_d = int(inp.cu_draft[-1])
    R_t = R_d + B

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    logit_bytes = inp.target.nbytes + (0 if token_only else inp.draft.nbytes)
    ncopy = max(1, int(np.ceil(2 * MALL_BYTES / logit_bytes)) + 1) if logit_bytes < 2 * MALL_BYTES else 1
    t0, d0 = up(inp.target), None if token_only else up(inp.draft)
    copies = [(t0, d0)] + [(t0.clone(), None if d0 is None else d0.clone()) for _ in range(ncopy - 1)]
    small = dict(draft_tokens=up(inp.draft_tokens), uniforms=up(inp.uniforms), temperatures=up(inp.temperatures))
    cu = up(inp.cu_draft)
    ragged = inp.uniform_gamma is None
    sv = SpecVerify(max_batch=B, max_gamma=max(int(inp.gammas.max()), 1), vocab=inp.workload.vocab,
                    dtype=inp.workload.dtype)
    out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
               out_tokens=torch.empty(R_t, dtype=torch.int32, device=dev),
               p_draft=torch.empty(max(R_d, 1), device=dev), q_draft=torch.empty(max(R_d, 1), device=dev),
               beta=torch.empty(max(R_d, 1), device=dev), resid_mass=torch.empty(max(R_d, 1), device=dev))
    gamma_kw = dict(cu_draft=cu, num_draft_rows=R_d) if ragged else dict(gamma=inp.uniform_gamma)

    launches = [0]   # launches of this batch so far, in stream order
    # one prepared run per copy: the arguments are checked once, and a step
    # is the launch itself (SpecVerify.run checks them on every call)
    prepared = [sv.prepare(t, d, small["draft_tokens"], small["uniforms"], small["temperatures"], **out, **gamma_kw)
                for (t, d) in copies]

    def step(k, copy=None):
        launches[0] += 1
        prepared[(k if copy is None else copy) % ncopy]()

    def step_checked(k):
        t, d = copies[k % ncopy]
        launches[0] += 1
        sv.run(t, d, small["draft_tokens"], small["uniforms"], small["temperatures"], **out, **gamma_kw)

    return dict(inp=inp, sv=sv, out=out, step=step, step_checked=step_checked, launches=launches, ncopy=ncopy,
                copies=copies, logit_bytes=logit_bytes,
                R_t=R_t, R_d=R_d, B=B, gamma_kw=gamma_kw, ragged=ragged)


def _check_outputs(ctx):
    """Every sequence of the step just run has a valid result: 0 <= n <= gamma_b,
    n + 1 tokens in [0, V), -1 after them."""
    acc = ctx["out"]["accepted_len"].cpu().numpy()
    toks = ctx["out"]["out_tokens"].cpu().numpy()
    inp = ctx["inp"]
    g = inp.gammas
    cu_t = inp.cu_t
    V = inp.workload.vocab
    for b in range(inp.batch):
        n = int(acc[b])
        assert 0 <= n <= g[b], f"sequence {b}: accepted_len {n}"
        t = toks[cu_t[b]:cu_t[b] + g[b] + 1]
        assert np.all((t[:n + 1] >= 0) & (t[:n + 1] < V)) and np.all(t[n + 1:] == -1), f"sequence {b}: tokens {t}"
    return acc, toks


def _events_time(step, k0, n, stream):
    """ms per step of n back-to-back steps between two events on `stream`."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(k0, k0 + n):
        step(k)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _per_step(step, n, stream):
    """Per-step durations (us) with an event between consecutive steps."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record(stream)
    for k in range(n):
        step(k)
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(n)])


def _kernel_us(ctx, n):
    """The verification kernel's mean launch duration (us): HIP events that the
    library records on the launch stream around each launch."""
    sv = ctx["sv"]
    sv.set_timing(True)
    for k in range(n):
        ctx["step"](k)
    runs, launch_ms, tail_ms = sv.timing_totals()
    sv.set_timing(False)
    return launch_ms / runs * 1e3


def _settle(step, stream, seconds):
    import torch
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            step(k)
            k += 1
        torch.cuda.synchronize()


def _probe_gbps(ctx, dev, stream, reps=200):
    """The library's streaming-read probe over the same logits, timed like the
    steps: back-to-back launches rotating over the copies, after a settle;
    GB/s of the logits."""
    import torch
    from rejection_sampling_verifier_specverify_amd.binding import specverify_probe_read
    sink = torch.zeros(1, dtype=torch.int32, device=dev)

    def probe(k):
        t, d = ctx["copies"][k % ctx["ncopy"]]
        specverify_probe_read(t, d, sink, stream.cuda_stream)

    _settle(probe, stream, 0.05)
    ms = _events_time(probe, 0, reps, stream)
    return ctx["logit_bytes"] / (ms * 1e-3) / 1e9


def _workload_line(w, seed, dev, stream, steps):
    """Microseconds per call and logits GB/s of one workload (µs per call from
    back-to-back steps after a settle; the kernel's own duration from events)."""
    ctx = _prepare(w, seed, dev)
    ctx["step"](0)
    import torch
    torch.cuda.synchronize()
    _check_outputs(ctx)
    kus = _kernel_us(ctx, min(steps, 100))
    _settle(ctx["step"], stream, 0.05)
    ms = _events_time(ctx["step"], 0, steps, stream)
    res = dict(us_per_call=ms * 1e3, kernel_us_events_each=kus, rows_per_s=ctx["R_t"] / (ms * 1e-3),
               logits_GBps=ctx["logit_bytes"] / (ms * 1e-3) / 1e9,
               frac=ctx["logit_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               batch=ctx["B"], rows_target=ctx["R_t"], rows_draft=ctx["R_d"], logit_bytes=ctx["logit_bytes"],
               rotating_copies=ctx["ncopy"])
    ctx["sv"].close()
    return res


def _tree_line(name, seed, dev, stream, steps):
    """Draft trees (specverify_run_tree): microseconds per call over rotating
    copies, after a settle; outputs checked for shape."""
    import torch
    from rejection_sampling_verifier_specverify_amd.binding import SpecVerify
    from rejection_sampling_verifier_specverify_amd.workloads import make_tree_inputs
    inp = make_tree_inputs(name, seed)
    B, N = inp.batch, int(inp.cu_nodes[-1])
    R_t = N + B
    w = inp.workload

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    logit_bytes = inp.target.nbytes
    ncopy = max(1, int(np.ceil(2 * MALL_BYTES / logit_bytes)) + 1) if logit_bytes < 2 * MALL_BYTES else 1
    t0 = up(inp.target)
    copies = [t0] + [t0.clone() for _ in range(ncopy - 1)]
    small = {k: up(getattr(inp, k)) for k in ("parents", "tokens", "uniforms", "temperatures", "cu_nodes")}
    gmax = int(np.max(np.diff(inp.cu_nodes)))
    sv = SpecVerify(max_batch=B, max_gamma=max(gmax, 1), vocab=w.vocab, dtype=w.dtype)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty(R_t, dtype=torch.int32, device=dev)
    nodes = torch.empty(R_t, dtype=torch.int32, device=dev)

    def step(k):
        sv.run_tree(copies[k % ncopy], small["cu_nodes"], N, small["parents"], small["tokens"], small["uniforms"],
                    small["temperatures"], acc, toks, out_nodes=nodes)

    step(0)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    assert np.all((a >= 0) & (a <= np.diff(inp.cu_nodes))), a
    _settle(step, stream, 0.05)
    ms = _events_time(step, 0, steps, stream)
    sv.close()
    return dict(us_per_call=ms * 1e3, rows_per_s=R_t / (ms * 1e-3), logits_GBps=logit_bytes / (ms * 1e-3) / 1e9,
                frac=logit_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, batch=B, nodes=N, rows_target=R_t,
                vocab=w.vocab, logits=w.dtype, logit_bytes=logit_bytes, rotating_copies=ncopy,
                mean_accepted_depth=float(np.mean(a)))


def main():
    args = parse()
    if args.summarize_pmc or args.summarize_trace or args.summarize_sq:
        if not args.out:
            raise SystemExit("--summarize-pmc / --summarize-trace / --summarize-sq need --out")
        if args.summarize_pmc:
            summarize_pmc(args)
        elif args.summarize_trace:
            summarize_trace(args)
        else:
            summarize_sq(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the verifier "
              "shards over sequences with no communication, so N GPUs run N independent copies "
              "of this measurement.", file=sys.stderr)
        sys.exit(2)
    from rejection_sampling_verifier_specverify_amd.workloads import WORKLOADS, make_inputs, token_only
    w = WORKLOADS[args.workload]
    inp = make_inputs(w, seed=args.seed)
    # the oracle on the host runs first, before this process touches the GPU
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)
        cpu_tok = cpu_baseline(token_only(inp), min(args.cpu_seconds, 5.0))

    import torch
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    ctx = _prepare(w, args.seed, dev, inp=inp)
    step = ctx["step"]
    R_t, B = ctx["R_t"], ctx["B"]
    logit_bytes = ctx["logit_bytes"]

    # untimed: one checked step, the launch durations, the clock settle, the warm-up
    step(0)
    torch.cuda.synchronize()
    _check_outputs(ctx)
    kernel_us = _kernel_us(ctx, args.steps)
    per_step = _per_step(step, args.steps, stream)
    _settle(step, stream, SETTLE_S)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # timed: exactly K steps between two events on the launch stream
    first_timed = ctx["launches"][0]
    ms = _events_time(step, 0, args.steps, stream)
    acc, toks = _check_outputs(ctx)          # the timed steps' last outputs are valid
    warm_ms = _events_time(lambda k: step(k, copy=0), 0, args.steps, stream)   # no rotation: cache-warm
    probe = _probe_gbps(ctx, dev, stream)
    # host cost of one call, K enqueues timed on the host while the GPU runs
    # behind: a prepared run (the steps above) and SpecVerify.run, which
    # checks every tensor on every call
    host_us = {}
    for key, fn in (("prepared_run", step), ("run", ctx["step_checked"])):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            fn(k)
        host_us[key] = (time.perf_counter() - t0) / args.steps * 1e6
    torch.cuda.synchronize()
    headline_launches = ctx["launches"][0]   # every launch of the headline batch, in stream order

    # token-only drafts (draft logits NULL, q_i = delta_{x_i}) on the same batch
    tctx = _prepare(w, args.seed, dev, token_only=True, inp=token_only(inp))
    tctx["step"](0)
    torch.cuda.synchronize()
    _check_outputs(tctx)
    tok_kus = _kernel_us(tctx, args.steps)
    _settle(tctx["step"], stream, 0.05)
    tok_ms = _events_time(tctx["step"], 0, args.steps, stream)
    tok_bytes = tctx["logit_bytes"]
    tctx["sv"].close()

    # the on-device commit of a step: K commits of the last step's outputs into
    # token rows with room for all of them
    sv, out = ctx["sv"], ctx["out"]
    cap = args.steps * (int(inp.gammas.max()) + 1) + 1
    seq_tokens = torch.zeros((B, cap), dtype=torch.int32, device=dev)
    seq_lens = torch.zeros(B, dtype=torch.int32, device=dev)
    appended = torch.empty(B, dtype=torch.int32, device=dev)
    next_token = torch.empty(B, dtype=torch.int32, device=dev)

    def commit(_k=0):
        sv.commit(out["accepted_len"], out["out_tokens"], seq_tokens, seq_lens, appended=appended,
                  next_token=next_token, **ctx["gamma_kw"])

    for _ in range(5):
        commit()
    seq_lens.zero_()
    torch.cuda.synchronize()
    commit_us = _events_time(commit, 0, args.steps, stream) * 1e3
    assert int(seq_lens.min()) >= args.steps   # every call appended to every sequence

    if args.copy_probe:   # plain copies of the logits' size, for FETCH/WRITE_SIZE calibration
        src = torch.empty(logit_bytes // 2, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(PROBE_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()
    sv.close()

    others = {}
    if not args.no_other_workloads:
        for name, ow in WORKLOADS.items():
            if name != w.name:
                others[name] = _workload_line(ow, args.seed, dev, stream, 100)
                torch.cuda.empty_cache()
        others["tree_b16_tree60_v128256_bf16"] = _tree_line("b16_tree60_v128256_bf16", args.seed, dev, stream, 100)
        torch.cuda.empty_cache()

    # one launch per step: the launches' average duration is the timed
    # region's elapsed time over K (back-to-back launches on one stream)
    launch_us = ms * 1e3
    achieved = logit_bytes / (launch_us * 1e-6) / 1e9
    prof_ns = read_profile_ns(w.name)
    res = {
        "metric": METRIC,
        "value": R_t / (ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "gamma": inp.uniform_gamma if not ctx["ragged"] else "ragged",
                   "vocab": w.vocab, "logits": w.dtype, "rows_target": R_t, "rows_draft": ctx["R_d"],
                   "rotating_copies": ctx["ncopy"], "seed": args.seed},
        "logits_GBps": logit_bytes / (ms * 1e-3) / 1e9,
        "sequences_per_s": B / (ms * 1e-3),
        "step_us": {"mean": ms * 1e3, "median": float(np.median(per_step)), "p10": float(np.percentile(per_step, 10)),
                    "p90": float(np.percentile(per_step, 90)),
                    "note": "median/p10/p90 from an event between consecutive steps (a separate pass)"},
        "step_frac": logit_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "warm_cache": {"ms_per_step": warm_ms, "logits_GBps": logit_bytes / (warm_ms * 1e-3) / 1e9,
                       "note": "every step reads the same copy, so part of it comes from the Infinity Cache"},
        "launch": {"step": "a prepared run (SpecVerify.prepare: the tensors checked once per set of buffers)",
                   "host_us_per_call": host_us},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": read_traffic(w.name), "kernel": KERNEL,
                     "alg_bytes_per_launch": logit_bytes, "kernel_us": launch_us,
                     "duration_source": ("HIP events on the launch stream around the K timed launches "
                                         "(one launch per step), elapsed / K"),
                     "timed_launches": [first_timed, first_timed + args.steps],
                     "headline_launches": headline_launches,
                     "kernel_us_events_each": kernel_us,
                     "events_each_note": ("the library's events around every launch: an event between "
                                          "launches adds the dispatch gap to each"),
                     "frac_profile": (logit_bytes / prof_ns / HBM_PEAK_GBPS) if prof_ns else None,
                     "profile_kernel_us": prof_ns / 1e3 if prof_ns else None,
                     "probe_GBps": probe, "frac_of_probe": achieved / probe},
        "token_only": {"ms_per_step": tok_ms, "value": R_t / (tok_ms * 1e-3), "unit": "rows/s",
                       "logits_GBps": tok_bytes / (tok_ms * 1e-3) / 1e9, "kernel_us_events_each": tok_kus,
                       "roofline": {"bound": "hbm", "achieved": tok_bytes / (tok_ms * 1e-3) / 1e9,
                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": tok_bytes / (tok_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                    "alg_bytes_per_launch": tok_bytes}},
        "commit": {"kernel": "commit_kernel", "us_per_call": commit_us, "sequences": B,
                   # reads accepted_len, out_tokens, seq_lens; writes at most R_t tokens
                   # and seq_lens, appended, next_token
                   "bytes_per_call_max": 4 * (2 * R_t + 5 * B), "bound": "latency"},
        "workloads": others,
    }
    if cpu is not None:
        res["cpu_baseline"] = cpu
        res["token_only"]["cpu_baseline"] = cpu_tok
        res["commit"]["cpu_oracle_us_per_call"] = cpu_commit_us(acc, toks, inp.cu_draft, B, cap)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
