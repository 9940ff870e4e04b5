"""GPU tests of verification over draft trees (specverify_run_tree) through
the C ABI, against the float64 tree oracle (tests/tree_parity.py rules).

* Seeded EAGLE-like trees (f32 and bf16, sampled, greedy and mixed
  temperatures), a full-size 60-node batch at V = 128256.
* A seeded sweep of random tree shapes (vocabulary, dtype, branching per
  depth, node budget, temperatures).
* Shapes: empty trees (N = 0), chains, a root with 100 children (more than
  one wave of candidates), a 255-node chain (the largest tree), duplicate
  candidates, vocabularies with a partial last chunk.
* Invalid data: a parent that is not an earlier node, a token outside
  [0, V), a NaN logit, a uniform of 1.
* A chain through run_tree equals the linear token-only run.
* The output law over 10^5 copies of a small tree: the first emitted token
  has law p_root (chi-square), the acceptance rate of the first candidate
  is p_root(c) (velog "6-1편. Speculative Decoding", section 2-3 item 3).
* Determinism over repeated runs; host-side errors.
"""
import ctypes

import numpy as np
import pytest
from scipy import stats

from oracle import softmax_t
from rejection_sampling_verifier_specverify_amd import binding
from rejection_sampling_verifier_specverify_amd.binding import SpecVerify
from rejection_sampling_verifier_specverify_amd.workloads import (TreeInputs, TreeWorkload, f32_to_bf16_bits,
                                                                  make_inputs, make_tree_inputs, token_only)

from parity import alloc_outputs, compare, fetch, gpu_run, to_device
from tree_parity import compare_tree

pytestmark = pytest.mark.gpu


def _dev(inp, device="cuda:0"):
    import torch

    def up(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(target=up(inp.target), parents=up(inp.parents), tokens=up(inp.tokens), uniforms=up(inp.uniforms),
                temperatures=up(inp.temperatures), cu_nodes=up(inp.cu_nodes))


def _outs(inp, device="cuda:0"):
    import torch
    B, N = inp.batch, int(inp.cu_nodes[-1])
    R_t = N + B
    return dict(accepted_len=torch.full((B,), -7, dtype=torch.int32, device=device),
                out_tokens=torch.full((R_t,), -7, dtype=torch.int32, device=device),
                out_nodes=torch.full((R_t,), -7, dtype=torch.int32, device=device),
                p_cand=torch.full((max(N, 1),), float("nan"), dtype=torch.float32, device=device))


def _run(inp, label, max_gamma=None, sv=None):
    N = int(inp.cu_nodes[-1])
    gmax = int(np.max(np.diff(inp.cu_nodes))) if inp.batch else 0
    print(f"[tree] {label}: B={inp.batch} N={N} V={inp.workload.vocab} {inp.workload.dtype}", flush=True)
    own = sv is None
    if own:
        sv = SpecVerify(max_batch=max(inp.batch, 1), max_gamma=max(gmax, 1) if max_gamma is None else max_gamma,
                        vocab=inp.workload.vocab, dtype=inp.workload.dtype)
    d, o = _dev(inp), _outs(inp)
    sv.run_tree(d["target"], d["cu_nodes"], N, d["parents"], d["tokens"], d["uniforms"], d["temperatures"],
                o["accepted_len"], o["out_tokens"], out_nodes=o["out_nodes"], p_cand=o["p_cand"])
    got = fetch(o)
    got["p_cand"] = got["p_cand"][:N]
    if own:
        sv.close()
    return got


def _check(inp, label, **kw):
    got = _run(inp, label, **kw)
    rep = compare_tree(inp, got)
    print(f"[tree] {label}: {rep.summary()}", flush=True)
    assert rep.ok(), rep.summary()
    return got, rep


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_seeded_trees_f32(seed):
    _check(make_tree_inputs("b8_tree12_v32000_f32", seed, batch=32), f"b8_tree12 f32 seed={seed}")


def test_seeded_trees_bf16_full_size():
    inp = make_tree_inputs("b16_tree60_v128256_bf16", 3)
    _check(inp, "b16_tree60 bf16")


def test_seeded_trees_bf16_peaked_and_greedy():
    w = TreeWorkload("peaked", 12, 12, 40, (5, 3, 2, 1), 50000, "bf16", ("normal", 6.0), 0.5,
                     ("choice", (0.0, 0.7, 1.3)))
    _check(make_tree_inputs(w, 4), "peaked bf16 mixed T")


def _random_tree_case(k):
    """Case k of a seeded sweep over tree shapes: vocabularies around the
    chunk edges, both dtypes, node budgets from 0 to 200, random branching
    per depth (wide roots, chains), close and far drafters, sampled, greedy
    and mixed temperatures."""
    import random
    rng = random.Random(104729 * (k + 1))
    V = rng.choice([1, 2, 7, 2047, 2048, 2049, 32000, 128256, rng.randint(1, 70000), rng.randint(70000, 160000)])
    depth = rng.randint(1, 8)
    branching = tuple(rng.choice([1, 1, 2, 3, 4, 8, 16, 64]) for _ in range(depth))
    w = TreeWorkload(f"tree_sweep{k}", 200 + k, rng.randint(1, 12), rng.choice([0, 1, 5, 12, 60, 200]), branching, V,
                     rng.choice(["f32", "bf16"]),
                     rng.choice([("normal", rng.uniform(0.5, 8.0)), ("gumbel", rng.uniform(0.5, 4.0))]),
                     rng.uniform(0.0, 3.0),
                     rng.choice([("const", rng.choice([1.0, 0.5, 0.1, 0.0, 2.0])), ("choice", (0.0, 0.3, 1.0, 1.5))]))
    return make_tree_inputs(w, k)


@pytest.mark.parametrize("k", range(60))
def test_random_tree_shapes_sweep(k):
    """A seeded sweep of tree shapes, each tree checked against the oracle."""
    inp = _random_tree_case(k)
    _check(inp, f"tree sweep {k} branching={inp.workload.branching} nodes={inp.workload.nodes}")


def _custom(target, parents_per_seq, tokens_per_seq, u, T, dtype="f32"):
    counts = [len(p) for p in parents_per_seq]
    cu = np.zeros(len(counts) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(counts)
    V = target.shape[1]
    w = TreeWorkload("custom", 96, len(counts), max(counts + [0]), (1,), V, dtype, ("normal", 1.0), 0.0,
                     ("const", 1.0))
    tg = target.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(target.astype(np.float32))
    return TreeInputs(w, 0, tg, np.concatenate([np.asarray(p, np.int32) for p in parents_per_seq] + [np.zeros(0, np.int32)]),
                      np.concatenate([np.asarray(t, np.int32) for t in tokens_per_seq] + [np.zeros(0, np.int32)]),
                      np.asarray(u, np.float32), np.asarray(T, np.float32), cu)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [7, 2049, 33000])
def test_shapes(dtype, V):
    rng = np.random.default_rng(V)
    shapes = [
        [],                                        # N = 0: the bonus from the root
        [0, 1, 2, 3],                              # a chain
        [0] * 100,                                 # a root with 100 candidates
        [0, 0, 1, 1, 2, 2, 3, 4],                  # a small tree
        [0, 0, 0],                                 # duplicate candidates (below)
    ]
    par, tok, rows = [], [], []
    for si, sh in enumerate(shapes):
        n = len(sh)
        lg = rng.normal(size=(n + 1, V)) * 5.0
        t = []
        for k, pa in enumerate(sh, start=1):
            order = np.argsort(-(lg[pa] + rng.normal(size=V)))
            sib = sum(1 for x in sh[:k - 1] if x == pa)
            t.append(int(order[sib % V]))
        if si == 4:
            t = [t[0], t[0], t[1]]                 # the first candidate twice
        par.append(sh)
        tok.append(t)
        rows.append(lg)
    target = np.concatenate(rows)
    u = rng.random(target.shape[0])
    T = [1.0, 0.7, 1.0, 0.0, 1.0]
    inp = _custom(target, par, tok, u, T, dtype)
    _check(inp, f"shapes V={V} {dtype}")


def test_largest_tree_is_a_255_node_chain():
    rng = np.random.default_rng(255)
    V, N = 300, 255
    lg = rng.normal(size=(N + 1, V)) * 8.0
    tok = [int(np.argmax(lg[k - 1])) for k in range(1, N + 1)]   # likely candidates: a deep walk
    inp = _custom(lg, [list(range(N))], [tok], rng.random(N + 1) * 0.5, [1.0])
    got, _ = _check(inp, "255-node chain", max_gamma=255)
    assert got["accepted_len"][0] > 10


@pytest.mark.parametrize("case", ["parent", "token", "nan", "u_one"])
def test_invalid_trees(case):
    rng = np.random.default_rng(9)
    V = 500
    par = [[0, 0, 1], [0, 1, 2]]
    tok = [[1, 2, 3], [4, 5, 6]]
    target = rng.normal(size=(8, V))
    u = rng.random(8)
    if case == "parent":
        par[0][1] = 2                              # node 2's parent must be 0 or 1
    elif case == "token":
        tok[0][2] = V
    elif case == "nan":
        target[2, 7] = np.nan
    elif case == "u_one":
        u[3] = 1.0
    got, rep = _check(_custom(target, par, tok, u, [1.0, 1.0]), f"invalid {case}")
    assert got["accepted_len"][0] == -1 and got["accepted_len"][1] >= 0
    assert rep.invalid == 1


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_chain_tree_equals_linear_token_only_run(T):
    base = token_only(make_inputs("b64_g4_v128256_bf16", seed=8, batch=16))
    base.temperatures[:] = T
    import torch
    from rejection_sampling_verifier_specverify_amd.workloads import TreeInputs as TI
    B = base.batch
    g = 4
    tw = TreeWorkload("chain", 95, B, g, (1,), base.workload.vocab, "bf16", ("normal", 1.0), 0.0, ("const", T))
    tree = TI(tw, 0, base.target, np.tile(np.arange(g, dtype=np.int32), B), base.draft_tokens.copy(),
              base.uniforms, base.temperatures, base.cu_draft.copy())
    got_t = _run(tree, f"chain as tree T={T}")
    sv = SpecVerify(max_batch=B, max_gamma=g, vocab=base.workload.vocab, dtype="bf16")
    out = alloc_outputs(base)
    gpu_run(sv, to_device(base), out, base)
    got_l = fetch(out)
    sv.close()
    rep_l = compare(base, got_l)
    rep_t = compare_tree(tree, got_t)
    print(f"[tree] chain T={T}: linear {rep_l.summary()} | tree {rep_t.summary()}", flush=True)
    assert rep_l.ok() and rep_t.ok()
    same = (got_t["accepted_len"] == got_l["accepted_len"]) & np.array(
        [np.array_equal(got_t["out_tokens"][b * 5:b * 5 + 5], got_l["out_tokens"][b * 5:b * 5 + 5]) for b in range(B)])
    assert same.sum() >= B - rep_l.boundary, (same, rep_l.summary())


def test_output_law_over_many_trees():
    """10^5 copies of one tree (V = 8): root candidates A (token 0) and B
    (token 1), A's candidate C (token 2).  The first emitted token has law
    p_root; A is accepted with probability p_root(0); given A, the next
    token has law p_A."""
    V, B = 8, 100_000
    rng = np.random.default_rng(77)
    lg = rng.normal(size=(4, V)) * 1.1
    T = 0.9
    par, tok = [0, 0, 1], [0, 1, 2]
    target = np.tile(lg, (B, 1))
    u = rng.random(4 * B)
    inp = _custom(target, [par] * B, [tok] * B, u, [T] * B)
    got = _run(inp, "law")
    acc = got["accepted_len"]
    toks = got["out_tokens"].reshape(B, 4)
    nodes = got["out_nodes"].reshape(B, 4)
    assert np.all(acc >= 0)
    p0 = softmax_t(lg[0], T)
    pA = softmax_t(lg[1], T)
    first = np.bincount(toks[:, 0], minlength=V)
    chi = float(((first - B * p0) ** 2 / (B * p0)).sum())
    pv = float(stats.chi2.sf(chi, V - 1))
    rate = float(np.mean(nodes[:, 0] == 1))
    sig = np.sqrt(p0[0] * (1 - p0[0]) / B)
    print(f"[tree] law: first-token chi2={chi:.2f} p={pv:.3g}; P(accept A)={rate:.5f} vs {p0[0]:.5f}", flush=True)
    assert pv > 1e-4
    assert abs(rate - p0[0]) < 4.5 * sig
    viaA = nodes[:, 0] == 1
    second = np.bincount(toks[viaA, 1], minlength=V)
    n = int(viaA.sum())
    chi2 = float(((second - n * pA) ** 2 / (n * pA)).sum())
    assert float(stats.chi2.sf(chi2, V - 1)) > 1e-4


def test_repeated_runs_are_identical():
    inp = make_tree_inputs("b8_tree12_v32000_f32", 5, batch=16)
    sv = SpecVerify(max_batch=16, max_gamma=12, vocab=32000, dtype="f32")
    first = _run(inp, "determinism 0", sv=sv)
    for k in range(20):
        again = _run(inp, f"determinism {k + 1}", sv=sv) if k == 0 else _run(inp, "", sv=sv)
        for key in first:
            assert np.array_equal(first[key].view(np.uint8), again[key].view(np.uint8)), key
    sv.close()


def test_host_errors():
    import torch
    sv = SpecVerify(max_batch=4, max_gamma=4, vocab=1000, dtype="f32")
    lib = binding.load_library()
    acc = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    toks = torch.zeros(8, dtype=torch.int32, device="cuda:0")
    tgt = torch.zeros(8, 1000, device="cuda:0")
    u = torch.zeros(8, device="cuda:0")
    T = torch.ones(2, device="cuda:0")
    cu = torch.tensor([0, 3, 6], dtype=torch.int32, device="cuda:0")
    tk = torch.zeros(6, dtype=torch.int32, device="cuda:0")
    inp = binding.TreeInputs(2, cu.data_ptr(), 6, None, tk.data_ptr(), tgt.data_ptr(), 1000, u.data_ptr(),
                             T.data_ptr())
    out = binding.TreeOutputs(acc.data_ptr(), toks.data_ptr(), None, None)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.specverify_run_tree(sv.handle, ctypes.byref(inp), ctypes.byref(out), s) == binding.ERR_INVALID_ARGUMENT
    inp.parents = tk.data_ptr()
    inp.num_nodes = 30                               # R_t = 32 > 4 * 5 rows of the handle
    assert lib.specverify_run_tree(sv.handle, ctypes.byref(inp), ctypes.byref(out), s) == binding.ERR_INVALID_ARGUMENT
    with pytest.raises(ValueError):
        sv.run_tree(tgt, cu, 6, tk[:5], tk, u, T, acc, toks)
    sv.close()
