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

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                  [--no-cpu-baseline] [--copy-probe]
"""
from __future__ import annotations

import argparse
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
    return ap.parse_args()


def cpu_baseline(inp, budget_s: float):
    """Time the float64 oracle on the host over whole sequences until the budget
    is spent (at least one sequence); one process."""
    from oracle import verify_batch
    B = inp.batch
    rows = 0
    t0 = time.perf_counter()
    done = 0
    for b in range(B):
        verify_batch(inp.target, inp.draft, inp.draft_tokens, inp.uniforms, inp.temperatures,
                     inp.cu_draft, inp.workload.dtype, sequences=[b])
        rows += int(inp.gammas[b]) + 1
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="rows/s", cores=1, kind="oracle",
                sample=f"first {done} of {B} sequences of the benchmarked batch ({rows} target rows), "
                       f"float64 numpy, one process, {dt:.1f} s")


def main():
    args = parse()
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
    # per-step events give the spread; the outer pair gives the mean
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for k in range(args.steps):
        step(k)
        evs[k + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    per = np.array([evs[k].elapsed_time(evs[k + 1]) for k in range(args.steps)])
    ms = total_ms / args.steps

    # per-kernel durations (HIP events around each of the two kernels)
    sv.set_timing(True)
    ks, kf = [], []
    for k in range(min(args.steps, 100)):
        step(k)
        a, f = sv.last_timing()
        ks.append(a)
        kf.append(f)
    sv.set_timing(False)
    stream_ms = float(np.mean(ks))
    finish_ms = float(np.mean(kf))

    if args.copy_probe:   # plain copy of the logits' size, for FETCH/WRITE_SIZE calibration
        src = torch.empty(logit_bytes // 2, dtype=torch.int16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()

    # algorithmic bytes of one launch: every logit once, plus the small inputs and outputs
    small_in = 4 * R_d + 4 * R_t + 4 * B + (4 * (B + 1) if ragged else 0)
    small_out = 4 * B + 4 * R_t + 16 * R_d
    alg_bytes = logit_bytes + small_in + small_out
    gbps = logit_bytes / (stream_ms * 1e-3) / 1e9
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
        "step_us_p10_p50_p90": [float(np.percentile(per, q) * 1e3) for q in (10, 50, 90)],
        "kernel_ms": {"stream": stream_ms, "finish": finish_ms},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None, "kernel": "stream_kernel",
                     "alg_bytes_per_launch": logit_bytes},
        "step_GBps": alg_bytes / (ms * 1e-3) / 1e9,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    sv.close()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
