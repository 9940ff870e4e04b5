"""GPU parity: the HIP verifier against the float64 oracle on seeded inputs.

Every test calls the C ABI through the ctypes binding on cuda:0 and compares
element by element with the oracle (rules in tests/parity.py).
"""
import numpy as np
import pytest

from rejection_sampling_verifier_specverify_amd.binding import (
    ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, SpecVerify, SpecVerifyError)
from rejection_sampling_verifier_specverify_amd.workloads import (
    WORKLOADS, Workload, make_custom, make_inputs, token_only)

from parity import alloc_outputs, compare, fetch, gpu_run, to_device

pytestmark = pytest.mark.gpu


def _handle(inp, **kw):
    g = int(np.max(inp.gammas)) if inp.batch else 0
    return SpecVerify(max_batch=max(inp.batch, 1), max_gamma=max(g, 1), vocab=inp.workload.vocab,
                      dtype=inp.workload.dtype, **kw)


def _check(inp, sequences=None, ragged=None, label=""):
    print(f"[parity] {label} B={inp.batch} V={inp.workload.vocab} dtype={inp.workload.dtype} "
          f"rows={inp.target.shape[0]}+{inp.draft.shape[0] if inp.draft is not None else 'tokens'}", flush=True)
    sv = _handle(inp)
    dev = to_device(inp)
    out = alloc_outputs(inp)
    gpu_run(sv, dev, out, inp, ragged=ragged)
    got = fetch(out)
    rep = compare(inp, got, sequences)
    print(f"[parity] {label}: {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()
    return rep, got


@pytest.mark.parametrize("name,batch", [
    ("b1_g4_v32000_f32", 1),
    ("b64_g4_v128256_bf16", 6),
    ("b256_g8_v128256_bf16_mixedT", 12),
    ("b32_g1_v129280_bf16_mtp", 10),
    ("b512_gragged1to7_v152064_bf16", 12),
])
def test_small_batches_every_sequence(name, batch):
    inp = make_inputs(name, seed=0, batch=batch)
    rep, _ = _check(inp, label=f"{name}[:{batch}]")
    assert rep.checked == batch


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_seeds_small(seed):
    for name, batch in (("b1_g4_v32000_f32", 1), ("b32_g1_v129280_bf16_mtp", 8)):
        _check(make_inputs(name, seed=seed, batch=batch), label=f"{name} seed={seed}")


def test_headline_full_size_every_sequence():
    """B=64, gamma=4, V=128256, bf16: the benchmarked configuration, all 64 sequences."""
    inp = make_inputs("b64_g4_v128256_bf16", seed=0)
    rep, got = _check(inp, label="headline full")
    assert rep.checked == 64
    assert rep.exact >= 60


def test_mtp_full_size_every_sequence():
    _check(make_inputs("b32_g1_v129280_bf16_mtp", seed=0), label="mtp full")


@pytest.mark.parametrize("name", ["b256_g8_v128256_bf16_mixedT", "b512_gragged1to7_v152064_bf16"])
def test_large_full_size_sampled_sequences(name):
    """Full batch on the GPU; the oracle checks a spread of sequences one by one."""
    inp = make_inputs(name, seed=0)
    B = inp.batch
    seqs = sorted(set(np.linspace(0, B - 1, 20).astype(int).tolist()) | {0, B - 1})
    _check(inp, sequences=seqs, label=f"{name} full (sampled {len(seqs)})")


# ------------------------------------------------------------------ edge cases

def _rand_custom(V, gammas, T, seed, dtype="bf16", draft_noise=0.5, scale=2.0):
    rng = np.random.default_rng(seed)
    R_d = int(np.sum(gammas))
    R_t = R_d + len(gammas)
    tgt = rng.normal(size=(R_t, V)) * scale
    pair = np.concatenate([np.arange(int(np.sum(gammas[:b])), int(np.sum(gammas[:b + 1]))) + b
                           for b in range(len(gammas))]).astype(int) if R_d else np.zeros(0, int)
    drf = tgt[pair] + rng.normal(size=(R_d, V)) * draft_noise if R_d else np.zeros((0, V))
    toks = np.array([int(np.argmax(drf[k] / max(T[0], 1e-3) + rng.gumbel(size=V))) for k in range(R_d)],
                    dtype=np.int32)
    u = rng.random(R_t).astype(np.float32)
    return make_custom(tgt, drf, toks, u, T, gammas, dtype=dtype)


@pytest.mark.parametrize("V", [1, 5, 63, 1000, 1023, 1024, 1025, 2047, 2048, 2049, 8192, 8193, 20007, 131072,
                               131080])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_vocab_sizes_and_tails(V, dtype):
    gam = [3, 0, 2, 4]
    inp = _rand_custom(V, gam, [0.9] * 4, seed=V, dtype=dtype)
    _check(inp, label=f"V={V} {dtype}")


@pytest.mark.parametrize("V,dtype", [(262144, "bf16"), (262144, "f32")])
def test_max_vocab(V, dtype):
    inp = _rand_custom(V, [2, 1], [1.0, 0.5], seed=9, dtype=dtype)
    _check(inp, label=f"V={V} {dtype}")


def test_ragged_with_zero_drafts_and_uniform_form_agree():
    gam = [0, 3, 7, 1, 0, 5, 2, 6]
    inp = _rand_custom(30000, gam, [1.0] * 8, seed=4)
    _check(inp, label="ragged with zeros")
    uni = _rand_custom(30000, [3] * 5, [0.8] * 5, seed=5)
    _, a = _check(uni, ragged=False, label="uniform form")
    _, b = _check(uni, ragged=True, label="ragged form of a uniform batch")
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k


@pytest.mark.parametrize("case", ["decreasing", "first_not_zero", "last_not_rd", "gamma_too_big"])
def test_invalid_layout_flags_whole_batch(case):
    """A cu_draft that is not a layout makes every sequence and every token invalid;
    the next run with a valid layout on the same handle is exact again."""
    import torch
    gam = [2, 3, 1, 2]
    inp = _rand_custom(5000, gam, [1.0] * 4, seed=11)
    sv = _handle(inp)
    dev = to_device(inp)
    cu = inp.cu_draft.astype(np.int32).copy()
    if case == "decreasing":
        cu[2] = cu[1] - 1
    elif case == "first_not_zero":
        cu[0] = 1
    elif case == "last_not_rd":
        cu[-1] -= 1
    else:
        cu[1:] += 3          # sequence 0 claims more drafts than the handle allows
        cu[-1] = inp.cu_draft[-1]
    bad = dict(dev, cu_draft=torch.from_numpy(cu).to("cuda:0"))
    out = alloc_outputs(inp)
    gpu_run(sv, bad, out, inp, ragged=True)
    got = fetch(out)
    assert np.all(got["accepted_len"] == -1), got["accepted_len"]
    assert np.all(got["out_tokens"] == -1), got["out_tokens"]
    out2 = alloc_outputs(inp)
    gpu_run(sv, dev, out2, inp, ragged=True)
    assert compare(inp, fetch(out2)).ok()


def test_gamma_zero_plain_sampling():
    inp = _rand_custom(50000, [0] * 16, [0.7] * 16, seed=6)
    rep, _ = _check(inp, label="gamma=0")
    assert rep.checked == 16


def test_equal_distributions_accept_everything():
    rng = np.random.default_rng(12)
    V, gam = 20000, [4, 4, 4]
    tgt = rng.normal(size=(15, V)) * 2
    pair = [0, 1, 2, 3, 5, 6, 7, 8, 10, 11, 12, 13]
    toks = rng.integers(0, V, size=12)
    u = rng.random(15).astype(np.float32)
    u[[0, 1, 2, 3]] = np.float32(0.99999994)
    inp = make_custom(tgt, tgt[pair], toks, u, [1.0, 0.6, 2.0], gam)
    rep, got = _check(inp, label="p == q")
    assert np.all(got["accepted_len"] == 4)
    np.testing.assert_allclose(got["beta"], 1.0, atol=1e-5)
    np.testing.assert_allclose(got["resid_mass"], 0.0, atol=1e-6)


def test_disjoint_support_rejects_at_zero():
    rng = np.random.default_rng(13)
    V = 12000
    tgt = rng.normal(size=(3, V))
    drf = rng.normal(size=(2, V))
    tgt[0, V // 2:] = -np.inf
    drf[0, : V // 2] = -np.inf
    toks = [V // 2 + 17, 3]
    for u0 in (0.0, 0.5):
        inp = make_custom(tgt, drf, toks, [u0, 0.1, 0.37], [1.0], [2])
        rep, got = _check(inp, label=f"disjoint u0={u0}")
        assert got["accepted_len"][0] == 0 and got["out_tokens"][0] < V // 2
        assert got["beta"][0] == 0.0 and got["p_draft"][0] == 0.0


def test_greedy_ties_and_mixed_temperatures():
    rng = np.random.default_rng(14)
    V, gam = 9000, [5, 5, 5, 5, 5, 5]
    R_t = 36
    tgt = np.round(rng.normal(size=(R_t, V)) * 2, 0)      # many exact ties at the max
    pair = [r for b in range(6) for r in range(b * 6, b * 6 + 5)]
    drf = np.round(tgt[pair] + rng.normal(size=(30, V)) * 0.3, 0)
    am = np.argmax(tgt[pair], axis=1)
    toks = np.where(rng.random(30) < 0.8, am, rng.integers(0, V, 30)).astype(np.int32)
    inp = make_custom(tgt, drf, toks, rng.random(R_t), [0.0, 0.0, 0.6, 0.0, 1.0, 0.0], gam)
    rep, _ = _check(inp, label="greedy ties")
    assert rep.greedy == 4


def test_one_hot_rows_zero_residual_fallback():
    V, gam = 40000, [3, 3]
    tgt = np.full((8, V), -400.0)
    drf = np.full((6, V), -300.0)
    for rr in range(8):
        tgt[rr, 1000 * rr + 7] = 0.0
    pair = [0, 1, 2, 4, 5, 6]
    for k, rr in enumerate(pair):
        drf[k, 1000 * rr + 7] = 0.0
    toks = [1000 * rr + 7 for rr in pair]
    toks[1] = 5          # q(5) = e^-300 > p(5) = e^-400: rejected, residual mass 0 -> sample p
    inp = make_custom(tgt, drf, toks, [0.3] * 8, [1.0, 1.0], gam, dtype="f32")
    rep, got = _check(inp, label="one-hot fallback")
    assert got["accepted_len"][0] == 1 and got["out_tokens"][1] == 1007
    assert got["accepted_len"][1] == 3


@pytest.mark.parametrize("case", ["nan", "posinf", "all_neginf", "token", "neg_T", "nan_T", "tiny_T",
                                  "nan_greedy", "partial_neginf"])
def test_invalid_data_flagged_per_sequence(case):
    rng = np.random.default_rng(15)
    V, gam = 10000, [2, 2, 2]
    tgt = rng.normal(size=(9, V))
    drf = rng.normal(size=(6, V))
    toks = rng.integers(0, V, 6).astype(np.int32)
    T = [1.0, 1.0, 0.0]
    if case == "nan":
        tgt[5, 9999] = np.nan          # bonus row of sequence 1
    elif case == "posinf":
        drf[2, 10] = np.inf
    elif case == "all_neginf":
        tgt[4, :] = -np.inf
    elif case == "token":
        toks[3] = V
    elif case == "neg_T":
        T[1] = -1.0
    elif case == "nan_T":
        T[1] = float("nan")
    elif case == "tiny_T":
        T[1] = 1e-39
    elif case == "nan_greedy":
        drf[5, 123] = np.nan
    elif case == "partial_neginf":
        tgt[3:6, : V // 2] = -np.inf  # valid: only half the row
    inp = make_custom(tgt, drf, toks, rng.random(9), T, gam, dtype="f32")
    rep, got = _check(inp, label=f"invalid {case}")
    if case == "partial_neginf":
        assert np.all(got["accepted_len"] >= 0)
    else:
        assert rep.invalid == 1
        bad = 2 if case == "nan_greedy" else 1
        assert got["accepted_len"][bad] == -1
        assert np.all(got["out_tokens"][bad * 3: bad * 3 + 3] == -1)


def test_repeated_runs_bitwise_identical():
    """Fixed reduction order: 100 launches on the same buffers give the same bits."""
    import torch
    inp = make_inputs("b64_g4_v128256_bf16", seed=3, batch=16)
    sv = _handle(inp)
    dev = to_device(inp)
    ref = None
    for k in range(100):
        out = alloc_outputs(inp)
        gpu_run(sv, dev, out, inp)
        got = fetch(out)
        if ref is None:
            ref = got
        for name in ref:
            assert np.array_equal(got[name].view(np.uint32), ref[name].view(np.uint32)), (k, name)


def test_back_to_back_runs_on_one_stream_do_not_interfere():
    """Different batches launched back to back on one handle (epoch-tagged slots)."""
    a = make_inputs("b32_g1_v129280_bf16_mtp", seed=0, batch=12)
    b = make_inputs("b32_g1_v129280_bf16_mtp", seed=7, batch=5)
    sv = _handle(a)
    da, db = to_device(a), to_device(b)
    oa, ob = alloc_outputs(a), alloc_outputs(b)
    for _ in range(3):
        gpu_run(sv, da, oa, a)
        gpu_run(sv, db, ob, b)
    ga, gb = fetch(oa), fetch(ob)
    assert compare(a, ga).ok() and compare(b, gb).ok()


@pytest.mark.parametrize("V,dtype,gam", [(128256, "bf16", [4] * 24), (262144, "bf16", [3, 0, 2, 4]),
                                         (131080, "f32", [3, 0, 2, 4]), (262144, "f32", [2, 1])])
def test_one_poll_budget_helps_and_stays_bit_exact(V, dtype, gam):
    """With a one-poll budget a waiting wave computes the missing chunk statistics of its
    row itself (forced from the host): every output, diagnostics included, is bit-identical
    to a run with the default budget, and the tokens match the oracle."""
    inp = _rand_custom(V, gam, [0.9] * len(gam), seed=V + len(gam), dtype=dtype)
    dev = to_device(inp)
    sv = _handle(inp, spin_limit=1)
    out = alloc_outputs(inp)
    gpu_run(sv, dev, out, inp)
    got = fetch(out)
    ref_h = _handle(inp)
    out2 = alloc_outputs(inp)
    gpu_run(ref_h, dev, out2, inp)
    ref = fetch(out2)
    for k in got:
        assert np.array_equal(got[k], ref[k], equal_nan=True), k
    rep = compare(inp, got)
    assert rep.ok(), rep.summary()


def test_host_validation_errors():
    import torch
    inp = make_inputs("b1_g4_v32000_f32", seed=0)
    sv = SpecVerify(max_batch=2, max_gamma=4, vocab=32000, dtype="f32")
    dev = to_device(inp)
    out = alloc_outputs(inp)
    lib = __import__("rejection_sampling_verifier_specverify_amd.binding", fromlist=["x"])
    with pytest.raises(ValueError):                # the binding: 5 drafts per sequence need 5 tokens
        sv.run(dev["target"], dev["draft"], dev["draft_tokens"], dev["uniforms"], dev["temperatures"],
               gamma=5, **out)
    with pytest.raises(SpecVerifyError) as e:      # the library: gamma beyond the handle's limit
        inp_c = lib.Inputs(1, 5, None, 5, dev["target"].data_ptr(), 32000, dev["draft"].data_ptr(), 32000,
                           dev["draft_tokens"].data_ptr(), dev["uniforms"].data_ptr(),
                           dev["temperatures"].data_ptr())
        out_c = lib.Outputs(out["accepted_len"].data_ptr(), out["out_tokens"].data_ptr(), None, None, None, None)
        lib.specverify_run(sv.handle, inp_c, out_c, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == ERR_INVALID_ARGUMENT
    with pytest.raises(SpecVerifyError) as e:      # logits not aligned to their element size
        raw = torch.zeros(5 * 32000 * 4 + 4, dtype=torch.uint8, device="cuda:0")
        inp_c = lib.Inputs(1, 4, None, 4, raw.data_ptr() + 1, 32000, dev["draft"].data_ptr(), 32000,
                           dev["draft_tokens"].data_ptr(), dev["uniforms"].data_ptr(),
                           dev["temperatures"].data_ptr())
        out_c = lib.Outputs(out["accepted_len"].data_ptr(), out["out_tokens"].data_ptr(), None, None, None, None)
        lib.specverify_run(sv.handle, inp_c, out_c, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == ERR_UNSUPPORTED
    # a row stride that breaks 16-byte alignment is accepted (element-wise loads)
    padded = torch.zeros(5, 32003, device="cuda:0")
    padded[:, :32000] = dev["target"]
    dpad = torch.zeros(4, 32001, device="cuda:0")
    dpad[:, :32000] = dev["draft"]
    out2 = alloc_outputs(inp)
    sv.run(padded[:, :32000], dpad[:, :32000], dev["draft_tokens"], dev["uniforms"], dev["temperatures"],
           gamma=4, **out2)
    out3 = alloc_outputs(inp)
    sv.run(dev["target"], dev["draft"], dev["draft_tokens"], dev["uniforms"], dev["temperatures"],
           gamma=4, **out3)
    a, b = fetch(out2), fetch(out3)
    for k in a:
        assert np.array_equal(a[k], b[k], equal_nan=True), k
    with pytest.raises(SpecVerifyError):
        SpecVerify(max_batch=0, max_gamma=4, vocab=32000, dtype="f32")
    with pytest.raises(SpecVerifyError) as e:
        SpecVerify(max_batch=1, max_gamma=1, vocab=524289, dtype="f32")
    assert e.value.status == ERR_UNSUPPORTED


# ---------------------------------------------------------------- token-only drafts (q = delta_x)


@pytest.mark.parametrize("name,batch", [("b64_g4_v128256_bf16", 16), ("b256_g8_v128256_bf16_mixedT", 24),
                                        ("b32_g1_v129280_bf16_mtp", 32), ("b1_g4_v32000_f32", None),
                                        ("b512_gragged1to7_v152064_bf16", 40)])
def test_token_only_workloads(name, batch):
    inp = token_only(make_inputs(name, seed=3, batch=batch))
    _check(inp, label=f"token-only {name}")


@pytest.mark.parametrize("V,dtype", [(1, "bf16"), (63, "bf16"), (2049, "bf16"), (20007, "bf16"),
                                     (131080, "f32"), (262144, "bf16")])
def test_token_only_vocab_shapes(V, dtype):
    inp = token_only(_rand_custom(V, [3, 0, 2, 4], [0.9, 1.0, 0.0, 0.7], seed=V + 1, dtype=dtype))
    _check(inp, label=f"token-only V={V} {dtype}")


def test_token_only_point_mass_edges():
    """x the only finite logit of its chunk (its chunk's residual is empty), and
    p(x) ~ 1 (Z ~ 0)."""
    V = 6000                              # fp32: chunks of 1024 logits
    rng = np.random.default_rng(21)
    tgt = rng.normal(size=(5, V)) * 2.0
    tgt[0, 2048:4096] = -np.inf           # chunks 2 and 3 of row 0: only x = 3000 is finite
    tgt[0, 3000] = 1.0
    tgt[1, :] = -30.0                     # row 1: x = 5999 carries almost all of p
    tgt[1, 5999] = 30.0
    drf = tgt[[0, 1, 3]] + rng.normal(size=(3, V))
    toks = np.array([3000, 5999, 17], dtype=np.int32)
    u = np.array([0.99, 0.5, 0.3, 0.999, 0.4], dtype=np.float32)
    base = make_custom(tgt, drf, toks, u, [1.0, 1.0], [2, 1])
    _check(token_only(base), label="token-only edges")


def test_token_only_one_poll_budget_bit_exact():
    inp = token_only(_rand_custom(128256, [4] * 12, [0.9] * 12, seed=77))
    dev = to_device(inp)
    a = _handle(inp, spin_limit=1)
    b = _handle(inp)
    oa, ob = alloc_outputs(inp), alloc_outputs(inp)
    gpu_run(a, dev, oa, inp)
    gpu_run(b, dev, ob, inp)
    ga, gb = fetch(oa), fetch(ob)
    for k in ga:
        assert np.array_equal(ga[k], gb[k], equal_nan=True), k
    rep = compare(inp, ga)
    assert rep.ok(), rep.summary()


@pytest.mark.parametrize("case", ["nan", "all_neginf", "token", "neg_T", "nan_T", "tiny_T", "nan_greedy",
                                  "partial_neginf"])
def test_token_only_invalid_data_flagged_per_sequence(case):
    """The phase-1-only launch (no draft logits) flags the same invalid data."""
    rng = np.random.default_rng(16)
    V, gam = 10000, [2, 2, 2]
    tgt = rng.normal(size=(9, V))
    toks = rng.integers(0, V, 6).astype(np.int32)
    T = [1.0, 1.0, 0.0]
    bad = 1
    if case == "nan":
        tgt[5, 9999] = np.nan          # bonus row of sequence 1
    elif case == "all_neginf":
        tgt[4, :] = -np.inf
    elif case == "token":
        toks[3] = V
    elif case == "neg_T":
        T[1] = -1.0
    elif case == "nan_T":
        T[1] = float("nan")
    elif case == "tiny_T":
        T[1] = 1e-39
    elif case == "nan_greedy":
        tgt[7, 123] = np.nan           # sequence 2 is greedy
        bad = 2
    elif case == "partial_neginf":
        tgt[3:6, : V // 2] = -np.inf   # valid: only half the row
    drf = rng.normal(size=(6, V))
    inp = token_only(make_custom(tgt, drf, toks, rng.random(9), T, gam, dtype="f32"))
    rep, got = _check(inp, label=f"token-only invalid {case}")
    if case == "partial_neginf":
        assert np.all(got["accepted_len"] >= 0)
    else:
        assert rep.invalid == 1
        assert got["accepted_len"][bad] == -1
        assert np.all(got["out_tokens"][bad * 3: bad * 3 + 3] == -1)


def test_token_only_invalid_layout_flags_whole_batch():
    import torch
    inp = token_only(_rand_custom(5000, [2, 3, 1, 2], [1.0] * 4, seed=12))
    sv = _handle(inp)
    dev = to_device(inp)
    cu = inp.cu_draft.astype(np.int32).copy()
    cu[2] = cu[1] - 1
    out = alloc_outputs(inp)
    gpu_run(sv, dict(dev, cu_draft=torch.from_numpy(cu).to("cuda:0")), out, inp, ragged=True)
    got = fetch(out)
    assert np.all(got["accepted_len"] == -1) and np.all(got["out_tokens"] == -1)
    out2 = alloc_outputs(inp)
    gpu_run(sv, dev, out2, inp, ragged=True)
    assert compare(inp, fetch(out2)).ok()


def test_ragged_all_gamma_zero_runs_phase_one_only():
    """A ragged batch with no drafts at all (R_d = 0): plain sampling of every row."""
    inp = _rand_custom(40000, [0] * 9, [0.7, 1.0, 0.0, 0.5, 1.3, 0.0, 0.9, 1.0, 0.2], seed=13)
    rep, _ = _check(inp, ragged=True, label="ragged gamma=0")
    assert rep.checked == 9


def test_token_only_headline_full_size_every_sequence():
    """The benchmarked batch with token-only drafts (the bench line's token_only run), all 64 sequences."""
    inp = token_only(make_inputs("b64_g4_v128256_bf16", seed=0))
    rep, _ = _check(inp, label="token-only headline full")
    assert rep.checked == 64


@pytest.mark.parametrize("name", ["b256_g8_v128256_bf16_mixedT", "b512_gragged1to7_v152064_bf16"])
def test_token_only_large_full_size_sampled_sequences(name):
    inp = token_only(make_inputs(name, seed=0))
    B = inp.batch
    seqs = sorted(set(np.linspace(0, B - 1, 20).astype(int).tolist()) | {0, B - 1})
    _check(inp, sequences=seqs, label=f"token-only {name} full (sampled {len(seqs)})")


def _as_f64(logits, dtype):
    a = np.asarray(logits)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@pytest.mark.parametrize("tok", [False, True])
@pytest.mark.parametrize("ug", [0.0, float(np.nextafter(np.float32(1.0), np.float32(0.0)))])
def test_final_uniform_extremes_emit_tokens_with_weight(ug, tok):
    """u_gamma = 0 (the first token with weight) and the largest float below 1
    (the last one; the scan's rounding fallback): every sequence's final token
    lies in the support of the distribution it is drawn from."""
    import dataclasses
    gam = [4, 4, 0, 2, 3, 1]
    inp = _rand_custom(20007, gam, [0.8, 1.0, 0.9, 0.7, 1.1, 0.6], seed=21)
    if tok:
        inp = token_only(inp)
    u = inp.uniforms.copy()
    cu_t, g = inp.cu_t, inp.gammas
    for b in range(inp.batch):
        u[cu_t[b] + g[b]] = np.float32(ug)
    inp = dataclasses.replace(inp, uniforms=u)
    _, got = _check(inp, label=f"u_gamma={ug} token-only={tok}")
    dt = inp.workload.dtype
    for b in range(inp.batch):
        n = int(got["accepted_len"][b])
        assert 0 <= n <= g[b]
        t = int(got["out_tokens"][cu_t[b] + n])
        T = float(inp.temperatures[b])
        lt = _as_f64(inp.target[cu_t[b] + n], dt) / T
        p = np.exp(lt - lt.max())
        p /= p.sum()
        assert p[t] > 0.0, (b, n, t)
        if n < g[b]:   # a rejected draft: the residual max(0, p - q) must not vanish at t
            x = int(inp.draft_tokens[inp.cu_draft[b] + n])
            if inp.draft is None:
                q = np.zeros_like(p)
                q[x] = 1.0
            else:
                ld = _as_f64(inp.draft[inp.cu_draft[b] + n], dt) / T
                q = np.exp(ld - ld.max())
                q /= q.sum()
            if np.maximum(p - q, 0.0).sum() > 1e-6:
                assert p[t] - q[t] > -1e-6 * max(p[t], q[t]), (b, n, t, p[t], q[t])


def _random_case(k):
    """Case k of a seeded sweep over shapes: vocabularies at and around the
    chunk edges (and V = 1), both dtypes, uniform and ragged gamma (0
    included), flat, peaked and heavy-tailed targets, close and far drafts,
    low, mixed and greedy temperatures, and token-only drafts."""
    import random
    rng = random.Random(7919 * (k + 1))
    V = rng.choice([1, 2, 7, 64, 1000, 2047, 2048, 2049, 4097, 32000, 50257, 128256, 152064,
                    rng.randint(1, 70000), rng.randint(70000, 200000)])
    dtype = rng.choice(["f32", "bf16"])
    B = rng.randint(1, 16)
    ragged = rng.random() < 0.4
    gamma = (rng.randint(0, 3), rng.randint(3, 8)) if ragged else rng.randint(0, 8)
    tgt = rng.choice([("normal", rng.uniform(0.5, 8.0)), ("gumbel", rng.uniform(0.5, 4.0)),
                      ("student_t", rng.choice([2.0, 3.0, 5.0]), rng.uniform(0.5, 3.0))])
    temps = rng.choice([("const", rng.choice([1.0, 0.7, 0.3, 0.1, 2.0])), ("choice", (0.0, 0.05, 0.5, 1.0, 1.5))])
    w = Workload(f"sweep{k}", 60 + k, B, gamma, V, dtype, tgt, rng.uniform(0.0, 1.2), rng.uniform(0.0, 2.0), temps)
    inp = make_inputs(w, seed=k)
    tok = int(inp.cu_draft[-1]) > 0 and rng.random() < 0.3
    return (token_only(inp) if tok else inp), ragged, tok


@pytest.mark.parametrize("k", range(200))
def test_random_shapes_sweep(k):
    """A seeded sweep of odd shapes, each checked sequence by sequence against the oracle."""
    inp, ragged, tok = _random_case(k)
    _check(inp, ragged=True if ragged else None,
           label=f"sweep {k} gamma={inp.workload.gamma} temps={inp.workload.temps} token_only={tok}")
