"""Throughput of the speculative-decoding verification sampler on one MI355X.

One step = one call of specverify_run over the whole batch of the
benchmarked workload (B = 64 sequences, gamma = 4 drafts, V = 128256, bf16
logits): every target and draft row is read, p and q are formed by
temperature softmax, the drafts are tested, the residual or bonus token is
sampled, and accepted lengths, tokens and diagnostics are written.

Timing: the inputs are resident in HBM before the timed region; the step
rotates over enough copies of the batch (> 2x the 256 MB Infinity Cache)
that no step reads logits the previous steps left in the cache.  HIP events
on the launch stream bracket the K timed steps.  Prints one JSON line.

Kernel durations come from HIP events that the library records on the same
stream around each of its two launches, over a repeat of the K steps (kept
out of the timed region because events between kernels add gaps); the HBM bytes
the streaming kernel actually moves come from a rocprofv3 counter summary
(FETCH_SIZE and WRITE_SIZE, scaled by what the same counters read for a plain
copy of known size), reported only while the kernel source still hashes to
the one that summary was taken from.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                  [--no-cpu-baseline] [--copy-probe]
  python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --out FILE --command-fetch CMD
                  --command-write CMD      (writes the traffic summary from two
                                            rocprofv3 --pmc output folders)
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
KERNEL_SRC = os.path.join(ROOT, "rejection_sampling_verifier_specverify_amd", "csrc", "specverify.hip")
PROFILES = os.path.join(ROOT, "profiles")


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"stream_kernel_{workload}_hbm_traffic.txt")


def source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="b64_g4_v128256_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of the logits' size (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--out")
    ap.add_argument("--command-fetch", default="")
    ap.add_argument("--command-write", default="")
    return ap.parse_args()


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


def summarize_pmc(args):
    """HBM traffic per launch of stream_kernel: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch) averaged over its dispatches, each scaled by bytes / counter
    of the copy probe (the plain copies dispatched after the last verifier
    launch, of exactly the logits' size)."""
    from rejection_sampling_verifier_specverify_amd.workloads import WORKLOADS, make_inputs
    w = WORKLOADS[args.workload]
    copy_bytes = logit_bytes_of(w)
    res = {}
    for name, folder in (("FETCH_SIZE", args.summarize_pmc[0]), ("WRITE_SIZE", args.summarize_pmc[1])):
        rows = _pmc_rows(folder, name)
        ker = [(d, v) for d, k, v in rows if "stream_kernel" in k]
        if not ker:
            raise SystemExit(f"{name}: no stream_kernel dispatch in {folder}")
        last = max(d for d, _ in ker)
        # the probe's copies are the run's last ones (a small copy, such as a
        # device-to-host read, may come between the kernel and the probe)
        cp = [v for d, k, v in rows if d > last and "copy" in k.lower()][-PROBE_COPIES:]
        if not cp:
            raise SystemExit(f"{name}: no copy-probe dispatch after the last stream_kernel in {folder}")
        kv = float(np.mean([v for _, v in ker]))
        cv = float(np.mean(cp))
        res[name] = dict(kernel_kib=kv, copy_kib=cv, factor=copy_bytes / (cv * 1024.0),
                         n_kernel=len(ker), n_copy=len(cp))
    fetch = res["FETCH_SIZE"]["kernel_kib"] * 1024.0 * res["FETCH_SIZE"]["factor"]
    write = res["WRITE_SIZE"]["kernel_kib"] * 1024.0 * res["WRITE_SIZE"]["factor"]
    lines = [
        f"# HBM traffic of stream_kernel, workload {w.name}",
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


def logit_bytes_of(w) -> int:
    """Every logit of the workload once: sum over sequences of (2 gamma + 1) rows of V."""
    from rejection_sampling_verifier_specverify_amd.workloads import make_inputs
    return int(make_inputs(w, seed=0).logit_bytes)


def read_traffic(workload: str):
    """Traffic bytes per launch from the committed summary, or None when there
    is none or it was taken from another version of the kernel source."""
    fn = traffic_file(workload)
    if not os.path.exists(fn):
        return None
    kv = {}
    with open(fn) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_hash():
        return None
    return float(kv["traffic_bytes_per_launch"])


def cpu_baseline(inp, budget_s: float):
    """Time the float64 oracle on the host, one sequence per call, cycling over
    the benchmarked batch until the budget is spent; one process, one thread."""
    from oracle import verify_batch
    B = inp.batch
    rows = 0
    seqs = 0
    t0 = time.perf_counter()
    while True:
        b = seqs % B
        verify_batch(inp.target, inp.draft, inp.draft_tokens, inp.uniforms, inp.temperatures,
                     inp.cu_draft, inp.workload.dtype, sequences=[b])
        rows += int(inp.gammas[b]) + 1
        seqs += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="rows/s", cores=1, kind="oracle",
                sample=f"{seqs} sequence verifications cycling over the {B} sequences of the "
                       f"benchmarked batch ({rows} target rows, {dt:.1f} s), float64 numpy, "
                       f"one process, one thread")


def cpu_commit_baseline(inp, out, cap) -> float:
    """The commit oracle on the host, one thread, over the same run outputs:
    microseconds per call (about 1 s of calls)."""
    from oracle import commit_reference
    acc = out["accepted_len"].cpu().numpy()
    toks = out["out_tokens"].cpu().numpy()
    rows = np.zeros((inp.batch, cap), dtype=np.int32)
    lens = np.zeros(inp.batch, dtype=np.int32)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < 1.0:
        commit_reference(acc, toks, inp.cu_draft, rows, lens, cap)
        n += 1
    return (time.perf_counter() - t0) / n * 1e6


def main():
    args = parse()
    if args.summarize_pmc:
        if not args.out:
            raise SystemExit("--summarize-pmc needs --out")
        summarize_pmc(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the verifier "
              "shards over sequences with no communication, so N GPUs run N independent copies "
              "of this measurement.", file=sys.stderr)
        sys.exit(2)
    import torch
    from rejection_sampling_verifier_specverify_amd.binding import SpecVerify
    from rejection_sampling_verifier_specverify_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w, seed=args.seed)
    B = inp.batch
    R_d = int(inp.cu_draft[-1])
    R_t = R_d + B
    dev = torch.device("cuda:0")
    logit_bytes = inp.logit_bytes
    ncopy = max(2, int(np.ceil(2 * MALL_BYTES / logit_bytes)) + 1)

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    target0, draft0 = up(inp.target), up(inp.draft)
    copies = [(target0, draft0)] + [(target0.clone(), draft0.clone()) for _ in range(ncopy - 1)]
    tokens = torch.from_numpy(inp.draft_tokens).to(dev)
    uniforms = torch.from_numpy(inp.uniforms).to(dev)
    temps = torch.from_numpy(inp.temperatures).to(dev)
    cu = torch.from_numpy(inp.cu_draft).to(dev)
    ragged = inp.uniform_gamma is None
    sv = SpecVerify(max_batch=B, max_gamma=int(inp.gammas.max()), vocab=w.vocab, dtype=w.dtype)
    out = dict(accepted_len=torch.empty(B, dtype=torch.int32, device=dev),
               out_tokens=torch.empty(R_t, dtype=torch.int32, device=dev),
               p_draft=torch.empty(max(R_d, 1), device=dev), q_draft=torch.empty(max(R_d, 1), device=dev),
               beta=torch.empty(max(R_d, 1), device=dev), resid_mass=torch.empty(max(R_d, 1), device=dev))
    gamma_kw = dict(cu_draft=cu, num_draft_rows=R_d) if ragged else dict(gamma=inp.uniform_gamma)

    def step(k):
        t, d = copies[k % ncopy]
        sv.run(t, d, tokens, uniforms, temps, **out, **gamma_kw)

    stream = torch.cuda.current_stream(dev)
    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    # Timed region: K steps between two events on torch's current stream, which
    # is the launch stream; nothing else is recorded in between.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(args.steps):
        step(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps

    # Kernel durations: the same K steps again, with the library recording HIP
    # events around each of its two launches on the launch stream.  The events
    # between the kernels add dispatch gaps, so this pass is kept out of the
    # timed region above.
    sv.set_timing(True)
    for k in range(args.steps):
        step(k)
    nrec, ks, kf = sv.timing_totals()
    sv.set_timing(False)
    stream_ms = ks / nrec
    finish_ms = kf / nrec

    # Token-only drafts (draft logits NULL, q_i = delta_{x_i}) on the same batch:
    # only the target rows are read.
    def step_tok(k):
        t, _ = copies[k % ncopy]
        sv.run(t, None, tokens, uniforms, temps, **out, **gamma_kw)

    for k in range(args.warmup):
        step_tok(k)
    torch.cuda.synchronize()
    ev0.record(stream)
    for k in range(args.steps):
        step_tok(k)
    ev1.record(stream)
    torch.cuda.synchronize()
    tok_ms = ev0.elapsed_time(ev1) / args.steps
    sv.set_timing(True)
    for k in range(args.steps):
        step_tok(k)
    tn, tks, tkf = sv.timing_totals()
    sv.set_timing(False)
    tok_bytes = int(inp.target.nbytes)
    tok_stream_ms = tks / tn

    # The on-device commit of a step (specverify_commit): K commits of the last
    # step's outputs into token rows with room for all of them, between two
    # events on the launch stream.
    cap = args.steps * (int(inp.gammas.max()) + 1) + 1
    seq_tokens = torch.zeros((B, cap), dtype=torch.int32, device=dev)
    seq_lens = torch.zeros(B, dtype=torch.int32, device=dev)
    appended = torch.empty(B, dtype=torch.int32, device=dev)
    next_token = torch.empty(B, dtype=torch.int32, device=dev)

    def commit():
        sv.commit(out["accepted_len"], out["out_tokens"], seq_tokens, seq_lens, appended=appended,
                  next_token=next_token, **gamma_kw)

    for _ in range(5):
        commit()
    seq_lens.zero_()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.steps):
        commit()
    ev1.record(stream)
    torch.cuda.synchronize()
    commit_us = ev0.elapsed_time(ev1) / args.steps * 1e3
    assert int(seq_lens.min()) >= args.steps   # every call appended to every sequence

    if args.copy_probe:   # plain copy of the logits' size, for FETCH/WRITE_SIZE calibration
        src = torch.empty(logit_bytes // 2, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(PROBE_COPIES):
            dst.copy_(src)
        torch.cuda.synchronize()

    # algorithmic bytes of one launch: every logit once, plus the small inputs and outputs
    small_in = 4 * R_d + 4 * R_t + 4 * B + (4 * (B + 1) if ragged else 0)
    small_out = 4 * B + 4 * R_t + 16 * R_d
    alg_bytes = logit_bytes + small_in + small_out
    gbps = logit_bytes / (stream_ms * 1e-3) / 1e9
    traffic = read_traffic(w.name)
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
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "gamma": inp.uniform_gamma if not ragged else "ragged",
                   "vocab": w.vocab, "logits": w.dtype, "rows_target": R_t, "rows_draft": R_d,
                   "rotating_copies": ncopy, "seed": args.seed},
        "logits_GBps": logit_bytes / (ms * 1e-3) / 1e9,
        "sequences_per_s": B / (ms * 1e-3),
        "kernel_ms": {"stream": stream_ms, "finish": finish_ms},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": traffic, "kernel": "stream_kernel",
                     "alg_bytes_per_launch": logit_bytes, "kernel_launches_timed": nrec},
        "step_GBps": alg_bytes / (ms * 1e-3) / 1e9,
        "token_only": {"ms_per_step": tok_ms, "value": R_t / (tok_ms * 1e-3), "unit": "rows/s",
                       "logits_GBps": tok_bytes / (tok_ms * 1e-3) / 1e9,
                       "kernel_ms": {"stream": tok_stream_ms, "finish": tkf / tn},
                       "roofline": {"bound": "hbm", "achieved": tok_bytes / (tok_stream_ms * 1e-3) / 1e9,
                                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": tok_bytes / (tok_stream_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                                    "alg_bytes_per_launch": tok_bytes}},
        "commit": {"kernel": "commit_kernel", "us_per_call": commit_us, "sequences": B,
                   # reads accepted_len, out_tokens, seq_lens; writes at most R_t tokens
                   # and seq_lens, appended, next_token
                   "bytes_per_call_max": 4 * (2 * R_t + 5 * B),
                   "bound": "latency"},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
        res["commit"]["cpu_oracle_us_per_call"] = cpu_commit_baseline(inp, out, cap)
        from rejection_sampling_verifier_specverify_amd.workloads import token_only
        res["token_only"]["cpu_baseline"] = cpu_baseline(token_only(inp), min(args.cpu_seconds, 5.0))
    sv.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
