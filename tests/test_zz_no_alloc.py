"""The allocation-free entry point, specverify_run_static, against the
handle-based specverify_run through the C ABI.

Both launch the same kernels with the same launch shape on the same inputs,
so accepted lengths, tokens and diagnostics must agree bit for bit; the
static run's outputs must also pass the oracle comparison.  Consecutive
calls share the device's static scratch: a batch, a smaller one, then the
larger one again with new inputs (what the smaller run left in the scratch
must not leak into the larger one).  A run that needs more than the scratch
is refused before any launch and leaves its outputs untouched.
"""
import numpy as np
import pytest

from rejection_sampling_verifier_specverify_amd.binding import (ERR_TOO_LARGE, SpecVerify, SpecVerifyError,
                                                                 SpecVerifyStatic)
from rejection_sampling_verifier_specverify_amd.workloads import make_inputs, token_only

from parity import alloc_outputs, compare, fetch, gpu_run, to_device

pytestmark = pytest.mark.gpu


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8)


def _static_vs_handle(inp, label, max_batch, max_gamma):
    print(f"[no-alloc] {label}: B={inp.batch} V={inp.workload.vocab} gammas<={int(np.max(inp.gammas))}", flush=True)
    kw = dict(max_batch=max_batch, max_gamma=max_gamma, vocab=inp.workload.vocab, dtype=inp.workload.dtype)
    dev = to_device(inp)
    ref_out, got_out = alloc_outputs(inp), alloc_outputs(inp)
    sv = SpecVerify(**kw)
    gpu_run(sv, dev, ref_out, inp)
    gpu_run(SpecVerifyStatic(**kw), dev, got_out, inp)
    ref, got = fetch(ref_out), fetch(got_out)
    sv.close()
    for k in ref:
        assert np.array_equal(_bits(ref[k]), _bits(got[k])), (label, k)
    rep = compare(inp, got)
    print(f"[no-alloc] {label}: {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()


def test_static_run_matches_handle_run_on_consecutive_calls():
    w = "b64_g4_v128256_bf16"
    _static_vs_handle(make_inputs(w, seed=21), "headline B=64", 64, 4)
    _static_vs_handle(make_inputs(w, seed=22, batch=16), "smaller B=16", 64, 4)
    _static_vs_handle(make_inputs(w, seed=23), "headline again B=64", 64, 4)


def test_static_run_ragged_and_token_only():
    w = "b512_gragged1to7_v152064_bf16"
    big = make_inputs(w, seed=31, batch=96)
    _static_vs_handle(big, "ragged B=96", 96, 7)
    _static_vs_handle(make_inputs(w, seed=32, batch=8), "ragged B=8", 96, 7)
    _static_vs_handle(token_only(make_inputs("b64_g4_v128256_bf16", seed=33, batch=24)), "token-only B=24", 64, 4)


def test_static_run_beyond_the_scratch_is_refused():
    """2800 target rows of V = 262144 (128 chunks) need 48 * 2800 * 128 bytes
    of exchange records, more than the 16 MiB scratch: TOO_LARGE, and the
    outputs keep their fill values (the inputs are real, sized tensors)."""
    import torch
    print("[no-alloc] beyond the scratch: B=2800 gamma=0 V=262144", flush=True)
    B, V = 2800, 262144
    tgt = torch.empty((B, V), dtype=torch.bfloat16, device="cuda:0")
    u = torch.full((B,), 0.5, dtype=torch.float32, device="cuda:0")
    T = torch.ones(B, dtype=torch.float32, device="cuda:0")
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    toks = torch.full((B,), -7, dtype=torch.int32, device="cuda:0")
    sv = SpecVerifyStatic(max_batch=B, max_gamma=0, vocab=V, dtype="bf16")
    with pytest.raises(SpecVerifyError) as e:
        sv.run(tgt, None, None, u, T, acc, toks, gamma=0)
    assert e.value.status == ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert int((acc != -7).sum()) == 0 and int((toks != -7).sum()) == 0
    del tgt
    torch.cuda.empty_cache()
