"""Pins of the tree oracle (oracle/tree_oracle.py), on the CPU.

* A chain is the linear token-only case: the tree oracle and the chain
  oracle agree on every output (sampled and greedy).
* The law of the emitted tokens, by exact enumeration: with dyadic target
  probabilities every ratio and CDF edge is a multiple of 1/8, so running
  the oracle at the midpoints of an 8-point grid per uniform counts each
  outcome with its exact probability.  Every emitted token must have the
  target law of its node (velog "6-1편. Speculative Decoding", section 2-3
  item 3: the emitted token has law p), also when several candidates of a
  node are tried in turn.
* A hand-worked packed batch (tests/golden/tree_worked_example.json).
* Invalid data, duplicate candidates, forced decisions.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import (decode_logits, softmax_t, tree_children, verify_sequence, verify_tree, verify_tree_batch)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tree_worked_example.json")


@pytest.mark.parametrize("T", [1.0, 0.6, 0.0])
@pytest.mark.parametrize("seed", range(6))
def test_chain_is_the_linear_token_only_case(T, seed):
    rng = np.random.default_rng(100 + seed)
    V, N = int(rng.integers(3, 40)), int(rng.integers(0, 6))
    target = rng.normal(size=(N + 1, V)) * 2.0
    tokens = rng.integers(0, V, N)
    if T == 0.0:   # make some drafts the argmax so that chains get accepted
        for i in range(N):
            if rng.random() < 0.6:
                tokens[i] = int(np.argmax(target[i]))
    u = rng.random(N + 1)
    tree = verify_tree(target, np.arange(N), tokens, u, T)
    lin = verify_sequence(target, None, tokens, u, T)
    assert tree.n == lin.n
    assert tree.tokens == lin.tokens
    assert tree.path == list(range(1, tree.n + 1))
    if T > 0:
        np.testing.assert_allclose(tree.p_cand, lin.p_x, rtol=0, atol=0)


# Root p over 4 tokens; nodes: 1 = A (parent 0, token 0), 2 = B (parent 0,
# token 1), 3 = A1 (parent 1, token 3), 4 = A2 (parent 1, token 2).
LAW_P = {0: [1 / 2, 1 / 4, 1 / 8, 1 / 8],   # root: A tested at 1/2, B at (1/4)/(1/2)
         1: [1 / 8, 1 / 8, 1 / 4, 1 / 2],   # A: A1 (token 3) at 1/2, A2 (token 2) at (1/4)/(1/2)
         2: [1 / 4, 1 / 4, 1 / 4, 1 / 4],   # B: a leaf
         3: [1 / 2, 1 / 8, 1 / 8, 1 / 4],   # A1: a leaf
         4: [1 / 8, 3 / 8, 1 / 4, 1 / 4]}   # A2: a leaf
LAW_PARENTS = [0, 0, 1, 1]
LAW_TOKENS = [0, 1, 3, 2]


def _law_outcomes(verify=verify_tree):
    target = np.log(np.array([LAW_P[v] for v in range(5)]))
    M = 8
    grid = (np.arange(M) + 0.5) / M
    outcomes = {}
    for us in itertools.product(grid, repeat=5):
        res = verify(target, LAW_PARENTS, LAW_TOKENS, np.array(us), 1.0)
        key = (tuple(res.path), tuple(res.tokens))
        outcomes[key] = outcomes.get(key, 0) + 1
    total = M ** 5
    return {k: v / total for k, v in outcomes.items()}


def _first_token_law(law):
    first = np.zeros(4)
    for (path, toks), pr in law.items():
        first[toks[0]] += pr
    return first


def test_emitted_tokens_have_the_target_law_by_enumeration():
    law = _law_outcomes()
    assert abs(sum(law.values()) - 1.0) < 1e-12
    # the first token has law p_root
    np.testing.assert_allclose(_first_token_law(law), LAW_P[0], rtol=0, atol=1e-12)
    # after an accepted candidate c, the next token has law p_c
    for node in (1, 2):
        nxt = np.zeros(4)
        mass = 0.0
        for (path, toks), pr in law.items():
            if len(path) >= 1 and path[0] == node:
                nxt[toks[1]] += pr
                mass += pr
        np.testing.assert_allclose(nxt / mass, LAW_P[node], rtol=0, atol=1e-12)
        assert abs(mass - LAW_P[0][LAW_TOKENS[node - 1]]) < 1e-12   # P(first token = c's token via c)
    for node in (3, 4):
        nxt = np.zeros(4)
        mass = 0.0
        for (path, toks), pr in law.items():
            if len(path) == 2 and path[1] == node:
                nxt[toks[2]] += pr
                mass += pr
        np.testing.assert_allclose(nxt / mass, LAW_P[node], rtol=0, atol=1e-12)


def test_a_planted_mistake_breaks_the_law():
    """A copy of the oracle with a mistake planted in it (rejected candidates
    are not removed from the residual, so later candidates are tested against
    p itself) fails the enumeration: the first token no longer has law p."""
    import oracle.tree_oracle as mod
    src = open(mod.__file__).read()
    assert src.count("w[x] = 0.0") == 1
    import sys
    import types
    mut = types.ModuleType("oracle.tree_oracle_mutant")
    mut.__package__ = "oracle"
    sys.modules[mut.__name__] = mut   # dataclasses look their module up
    try:
        exec(compile(src.replace("w[x] = 0.0", "pass"), "tree_oracle_mutant", "exec"), mut.__dict__)
    finally:
        del sys.modules[mut.__name__]
    bad = _first_token_law(_law_outcomes(mut.verify_tree))
    assert np.abs(bad - np.array(LAW_P[0])).max() > 0.05
    good = _first_token_law(_law_outcomes())
    np.testing.assert_allclose(good, LAW_P[0], rtol=0, atol=1e-12)


def test_worked_example():
    g = json.load(open(GOLDEN))
    tgt = np.array([[float(x) for x in row] for row in g["target"]], dtype=np.float32)
    acc, out, nodes, p_cand, _ = verify_tree_batch(
        tgt, np.array(g["parents"]), np.array(g["tokens"]), np.array(g["uniforms"], dtype=np.float32),
        np.array(g["temperatures"], dtype=np.float32), np.array(g["cu_nodes"]), "f32")
    assert acc.tolist() == g["expected_accepted_len"]
    assert out.tolist() == g["expected_out_tokens"]
    assert nodes.tolist() == g["expected_out_nodes"]
    exp = np.array([np.nan if v is None else v for v in g["expected_p_cand"]])
    np.testing.assert_allclose(p_cand, exp, rtol=1e-15, atol=0)


def test_children_in_node_order():
    assert tree_children([0, 0, 1, 0, 3], 0) == [1, 2, 4]
    assert tree_children([0, 0, 1, 0, 3], 3) == [5]
    assert tree_children([0, 0, 1, 0, 3], 5) == []


@pytest.mark.parametrize("case", ["parent_self", "parent_ahead", "parent_negative", "token", "u_one", "u_nan",
                                  "nan_logit", "neginf_row", "neg_T"])
def test_invalid_trees(case):
    rng = np.random.default_rng(7)
    V, N = 6, 3
    target = rng.normal(size=(N + 1, V))
    parents = np.array([0, 1, 1])
    tokens = np.array([1, 2, 3])
    u = np.array([0.1, 0.2, 0.3, 0.4])
    T = 1.0
    if case == "parent_self":
        parents[1] = 2
    elif case == "parent_ahead":
        parents[0] = 3
    elif case == "parent_negative":
        parents[2] = -1
    elif case == "token":
        tokens[2] = V
    elif case == "u_one":
        u[3] = 1.0
    elif case == "u_nan":
        u[0] = np.nan
    elif case == "nan_logit":
        target[3, 2] = np.nan
    elif case == "neginf_row":
        target[2] = -np.inf
    elif case == "neg_T":
        T = -1.0
    res = verify_tree(target, parents, tokens, u, T)
    assert res.n == -1 and res.tokens == [] and np.isnan(res.p_cand).all()


def test_duplicate_candidate_is_rejected_after_the_first():
    target = np.log(np.array([[0.25, 0.25, 0.5], [1 / 3] * 3, [1 / 3] * 3]))
    # both children propose token 2 (p = 1/2); the first is rejected (u = 0.9),
    # the second then has residual probability 0 and is rejected for any u
    for u1 in (0.0, 0.3, 0.999):
        res = verify_tree(target, [0, 0], [2, 2], [0.9, u1, 0.5], 1.0)
        assert res.n == 0 and res.removed == [1, 2]
        assert res.tokens[0] in (0, 1)


def test_forced_decisions_follow_the_other_branch():
    rng = np.random.default_rng(3)
    target = rng.normal(size=(4, 5))
    parents, tokens = [0, 1, 0], [1, 2, 3]
    u = np.array([0.999, 0.5, 0.5, 0.5])
    base = verify_tree(target, parents, tokens, u, 1.0)
    assert base.path[:1] != [1]
    forced = verify_tree(target, parents, tokens, u, 1.0, force={1: True})
    assert forced.path[:1] == [1] and forced.tokens[0] == 1
