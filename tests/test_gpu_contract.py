"""GPU tests of the data contract and of the output law.

* Uniforms outside [0, 1), or NaN, are invalid data (accepted_len -1), for
  sampled, greedy and token-only sequences alike.
* Low temperatures (T = 0.05 .. 0.25) on headline-shaped logits: p(x), q(x),
  beta within 1e-5 relative of the float64 oracle.
* Logits whose last row ends flush with the end of a device allocation: no
  load leaves the rows.
* The output law on the GPU (velog "6-1편. Speculative Decoding", section
  2-3: the acceptance rate is beta = sum min(p, q), item 1; the emitted token
  has law p, item 3): one launch over 10^5 copies of a V = 8 row, with seeded
  drafts and uniforms; the acceptance rate within 4.5 sigma of beta, and a
  chi-square test of the first emitted token against p_0 and of the bonus
  token against p_1.  This covers the decisions next to switching points
  that the element-wise parity tests set aside.
"""
import dataclasses

import numpy as np
import pytest
from scipy import stats

from oracle import sequence_distributions
from rejection_sampling_verifier_specverify_amd.binding import SpecVerify
from rejection_sampling_verifier_specverify_amd.workloads import make_custom, make_inputs, token_only

from parity import alloc_outputs, compare, fetch, gpu_run, to_device

pytestmark = pytest.mark.gpu


def _run(inp, ragged=None, label=""):
    print(f"[contract] {label} B={inp.batch} V={inp.workload.vocab}", flush=True)
    g = int(np.max(inp.gammas))
    sv = SpecVerify(max_batch=inp.batch, max_gamma=max(g, 1), vocab=inp.workload.vocab, dtype=inp.workload.dtype)
    out = alloc_outputs(inp)
    gpu_run(sv, to_device(inp), out, inp, ragged=ragged)
    got = fetch(out)
    sv.close()
    return got


@pytest.mark.parametrize("tok", [False, True])
def test_uniforms_outside_unit_interval_are_invalid(tok):
    rng = np.random.default_rng(31)
    V, gam = 5000, [2, 2, 2, 2, 2, 2, 2, 2]
    R_t = 24
    tgt = rng.normal(size=(R_t, V)) * 2
    pair = [r for b in range(8) for r in range(3 * b, 3 * b + 2)]
    drf = tgt[pair] + rng.normal(size=(16, V))
    toks = rng.integers(0, V, 16).astype(np.int32)
    u = rng.random(R_t).astype(np.float32)
    T = [1.0, 1.0, 0.0, 1.0, 0.7, 0.0, 1.0, 1.0]
    bad = {1: (3 + 0, 1.0), 2: (6 + 2, np.nan), 3: (9 + 2, 1.5), 5: (15 + 1, -1e-7), 6: (18 + 0, np.inf)}
    for b, (r, v) in bad.items():
        u[r] = np.float32(v)
    u[21 + 2] = np.nextafter(np.float32(1.0), np.float32(0.0))   # seq 7: largest float below 1 is valid
    u[0] = 0.0                                                    # seq 0: 0 is valid
    inp = make_custom(tgt, drf, toks, u, T, gam, dtype="f32")
    if tok:
        inp = token_only(inp)
    got = _run(inp, label=f"uniform contract token_only={tok}")
    rep = compare(inp, got)
    print(f"[contract] {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()
    for b in range(8):
        if b in bad:
            assert got["accepted_len"][b] == -1 and np.all(got["out_tokens"][3 * b:3 * b + 3] == -1), b
        else:
            assert got["accepted_len"][b] >= 0, b


@pytest.mark.parametrize("T", [0.05, 0.1, 0.25])
def test_low_temperature_parity(T):
    """Headline-shaped logits (V = 128256, N(0, 3^2), draft 0.8 t + N(0, 1.5^2))
    at low temperatures: |l s| reaches a few hundred, where the rounding of
    the exponent offset matters most."""
    base = make_inputs("b64_g4_v128256_bf16", seed=5, batch=8)
    inp = dataclasses.replace(base, temperatures=np.full(8, T, dtype=np.float32))
    got = _run(inp, label=f"T={T}")
    rep = compare(inp, got)
    print(f"[contract] T={T}: {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()


def test_rows_ending_at_the_end_of_an_allocation():
    """The last target row ends exactly where its device allocation ends (a
    20 MiB tensor: torch gives allocations of 10 MiB or more a segment of
    their own, rounded to 2 MiB), and so does the last draft row: every load
    of the last chunk stays inside the rows."""
    import torch
    V = 129280                      # 63.1 chunks of 2048: the last chunk is partial
    n = 20 * (1 << 20) // 2         # bf16 elements in 20 MiB
    rng = np.random.default_rng(41)
    gam = [1] * 8
    inp = make_custom(rng.normal(size=(16, V)) * 2, rng.normal(size=(8, V)) * 2,
                      rng.integers(0, V, 8), rng.random(16), [1.0] * 8, gam, dtype="bf16")
    torch.cuda.synchronize()
    torch.cuda.empty_cache()        # no cached block to split: each tensor gets its own allocation
    tbuf = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    dbuf = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    tflat = torch.from_numpy(inp.target.view(np.int16).reshape(-1)).to("cuda:0")
    dflat = torch.from_numpy(inp.draft.view(np.int16).reshape(-1)).to("cuda:0")
    tbuf[n - tflat.numel():] = tflat
    dbuf[n - dflat.numel():] = dflat
    dev = to_device(inp)
    dev["target"] = tbuf[n - tflat.numel():].view(torch.bfloat16).view(16, V)
    dev["draft"] = dbuf[n - dflat.numel():].view(torch.bfloat16).view(8, V)
    assert dev["target"].data_ptr() + 16 * V * 2 == tbuf.data_ptr() + 2 * n
    sv = SpecVerify(max_batch=8, max_gamma=1, vocab=V, dtype="bf16")
    out = alloc_outputs(inp)
    gpu_run(sv, dev, out, inp)
    rep = compare(inp, fetch(out))
    print(f"[contract] flush rows: {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("tok", [False, True])
def test_output_law_over_many_sequences(tok):
    V, B = 8, 100_000
    rng = np.random.default_rng(2024)
    lt = rng.normal(size=(2, V)) * 1.2
    ld = lt[0] + rng.normal(size=V) * 0.9
    T = 0.9
    p, q = sequence_distributions(lt, None if tok else ld[None, :], [0], T)
    p0, p1, q0 = p[0], p[1], q[0]
    if tok:   # a token-only drafter proposes x from some law r of its own
        q0 = np.array([0.3, 0.05, 0.05, 0.2, 0.1, 0.1, 0.15, 0.05])
    x = rng.choice(V, size=B, p=q0 / q0.sum()).astype(np.int32)
    u = rng.random(2 * B).astype(np.float32)
    tgt = np.tile(lt, (B, 1))
    drf = np.tile(ld, (B, 1))
    inp = make_custom(tgt, drf, x, u, [T] * B, [1] * B, dtype="f32")
    if tok:
        inp = token_only(inp)
    got = _run(inp, label=f"law token_only={tok}")
    acc = got["accepted_len"]
    assert np.all((acc == 0) | (acc == 1))
    # acceptance rate: beta = sum min(p, q) (token-only: sum_x r(x) p(x))
    beta = float(np.sum(q0 * p0)) if tok else float(np.sum(np.minimum(p0, q0)))
    rate = float(np.mean(acc == 1))
    sig = np.sqrt(beta * (1 - beta) / B)
    print(f"[contract] law: acceptance {rate:.5f} beta {beta:.5f} sigma {sig:.2e}", flush=True)
    assert abs(rate - beta) < 4.5 * sig
    first = got["out_tokens"][0::2]
    bonus = got["out_tokens"][1::2][acc == 1]
    for counts, law, name in ((np.bincount(first, minlength=V), p0, "first"),
                              (np.bincount(bonus, minlength=V), p1, "bonus")):
        n = counts.sum()
        chi2 = float(((counts - n * law) ** 2 / (n * law)).sum())
        pv = float(stats.chi2.sf(chi2, V - 1))
        print(f"[contract] law {name}: n={n} chi2={chi2:.2f} p={pv:.3g}", flush=True)
        assert pv > 1e-4, (name, counts, law)


@pytest.mark.parametrize("name,ragged,tok", [("b64_g4_v128256_bf16", False, False),
                                             ("b512_gragged1to7_v152064_bf16", True, False),
                                             ("b64_g4_v128256_bf16", False, True)])
def test_prepared_run_matches_run(name, ragged, tok):
    """SpecVerify.prepare checks the tensors once; its launches give the same
    bits as SpecVerify.run on the same tensors, call after call."""
    import torch
    inp = make_inputs(name, seed=5)
    if tok:
        inp = token_only(inp)
    print(f"[contract] prepared {name} ragged={ragged} token_only={tok}", flush=True)
    g = int(np.max(inp.gammas))
    sv = SpecVerify(max_batch=inp.batch, max_gamma=max(g, 1), vocab=inp.workload.vocab, dtype=inp.workload.dtype)
    dev = to_device(inp)
    out = alloc_outputs(inp)
    gpu_run(sv, dev, out, inp, ragged=ragged)
    want = fetch(out)
    kw = dict(cu_draft=dev["cu_draft"], num_draft_rows=int(inp.cu_draft[-1])) if ragged else dict(gamma=inp.uniform_gamma)
    prepared = sv.prepare(dev["target"], dev["draft"], dev["draft_tokens"], dev["uniforms"], dev["temperatures"],
                          **out, **kw)
    for call in range(2):
        for v in out.values():
            v.fill_(-9)
        prepared()
        got = fetch(out)
        for k in want:
            assert np.array_equal(got[k], want[k], equal_nan=True), (call, k)
    assert (want["accepted_len"] >= 0).all()
    sv.close()
    with pytest.raises(RuntimeError):
        prepared()
    torch.cuda.synchronize()
