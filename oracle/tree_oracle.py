"""Float64 CPU oracle of verification over a draft tree.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; it shares no code with the HIP path.

The draft is a tree instead of a chain (Perplexity "Accelerating Sonar
through speculation", section "추측적 디코딩", stage 2 "초안 생성": the
drafter may explore a tree up to a given depth, as EAGLE and Medusa do; and
section "EAGLE": at every node the drafter keeps its Top-K candidates rather
than only the best token).  The pages give no rule for verifying several
candidates of one node.  Reading (also in the design notes): the candidates
are the drafter's tokens without a distribution, so each is the point mass
q = delta_c (the token-only draft of the chain case), and the pages' rule is
applied node by node, one candidate at a time:

* at node v the target distribution is p_v = softmax(target row of v / T);
  its children c_1, c_2, ... (in node order) are tested in turn against the
  current residual r (r = p_v at first): accept c_i when
  u_{c_i} < min(1, r(c_i) / q(c_i)) = r(c_i)  -- velog "6-1편. Speculative
  Decoding", section 2-1 (the min(1, p/q) rule) with q = delta_c;
* a rejected candidate turns r into norm(max(0, r - delta_c)), i.e. r with
  c removed and renormalised -- the same page, section 2-2 (the residual);
* an accepted candidate is emitted and the walk continues at its node;
* when every child of the current node is rejected, or it has none (a leaf:
  every node on the path was accepted), the final token is sampled from r by
  inverse CDF in token order with the one final uniform (the chain case's
  residual or bonus sample);
* T = 0 (greedy, "How to Scale Your Model -- All About Transformer
  Inference", Appendix D): a candidate is accepted when it equals the argmax
  of its node's target logits; the first such child in node order is
  followed; otherwise the argmax is emitted.

A chain (node k's parent is k - 1) is exactly the token-only linear case,
and every emitted token has the target law of its node (the pins check
both).

Layout of one sequence: N drafted nodes 1..N, node 0 the root; parents[k-1]
is node k's parent, in [0, k - 1]; tokens[k-1] is node k's candidate;
target row k is the target distribution after node k (row 0: after the
committed prefix); uniform u[k-1] tests node k, u[N] is the final sample.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from .specverify_oracle import FLT_MIN, argmax_first, decode_logits, inverse_cdf, softmax_t

__all__ = ["TreeResult", "tree_children", "verify_tree", "verify_tree_batch", "tree_rows"]


@dataclasses.dataclass
class TreeResult:
    n: int                        # accepted depth; -1 = invalid sequence
    path: List[int]               # the accepted nodes, root excluded (n of them)
    tokens: List[int]             # n path tokens and the final token
    stop: int                     # the node whose children were all rejected, or the leaf reached
    removed: List[int]            # the rejected children of `stop`, in test order
    p_cand: np.ndarray            # [N] p_parent(c): each candidate under its parent's target distribution
    tests: List[tuple]            # (node, ratio, u) of every test taken, in order
    sample_margin: float          # u-distance of the final uniform to its CDF interval edge
    sample_mass: float            # mass of the final distribution, relative to p of `stop` (1 - removed mass)
    fallback: bool                # the residual lost all its mass: sampled before the last removal
    greedy: bool


def tree_children(parents: Sequence[int], v: int) -> List[int]:
    """Children of node v in node order (nodes are 1-based, 0 is the root)."""
    return [k + 1 for k, par in enumerate(parents) if int(par) == v]


def _tree_valid(target: np.ndarray, parents: np.ndarray, tokens: np.ndarray, u: np.ndarray, T: float,
                V: int) -> bool:
    """The chain case's invalid-data rules, plus parents in [0, k - 1] for node k."""
    if not np.isfinite(T) or T < 0.0 or (0.0 < T < FLT_MIN):
        return False
    if np.isnan(target).any() or np.isposinf(target).any():
        return False
    if np.any(np.all(np.isneginf(target), axis=1)):
        return False
    if np.any((tokens < 0) | (tokens >= V)):
        return False
    N = parents.shape[0]
    if np.any((parents < 0) | (parents > np.arange(N))):
        return False
    if not np.all((u >= 0.0) & (u < 1.0)):
        return False
    return True


def verify_tree(target: np.ndarray, parents: Sequence[int], tokens: Sequence[int], u: Sequence[float], T: float,
                force: Optional[Dict[int, bool]] = None) -> TreeResult:
    """Verify one sequence whose drafts form a tree (see the module text).

    target: [N+1, V] float64 logits; parents, tokens: [N]; u: [N+1].
    ``force`` overrides the decision of the named nodes' tests (node ->
    accepted): the walk a float32 implementation may take when a uniform
    lies next to its ratio.
    """
    target = np.asarray(target, dtype=np.float64)
    parents = np.asarray(parents, dtype=np.int64).reshape(-1)
    tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    N, V = tokens.shape[0], target.shape[1]
    assert parents.shape[0] == N and target.shape[0] == N + 1 and u.shape[0] == N + 1
    force = force or {}
    if not _tree_valid(target, parents, tokens, u, float(T), V):
        return TreeResult(-1, [], [], -1, [], np.full(N, np.nan), [], np.inf, np.nan, False, T == 0.0)

    if T == 0.0:
        at = [argmax_first(target[v]) for v in range(N + 1)]
        p_cand = np.array([1.0 if tokens[k] == at[parents[k]] else 0.0 for k in range(N)])
        v, path, tests, removed = 0, [], [], []
        while True:
            nxt = None
            removed = []
            for c in tree_children(parents, v):
                ok = bool(tokens[c - 1] == at[v])
                ok = force.get(c, ok)
                tests.append((c, 1.0 if ok else 0.0, float(u[c - 1])))
                if ok:
                    nxt = c
                    break
                removed.append(c)
            if nxt is None:
                break
            path.append(nxt)
            v = nxt
        out = [int(tokens[c - 1]) for c in path] + [at[v]]
        return TreeResult(len(path), path, out, v, removed, p_cand, tests, np.inf, 1.0, False, True)

    p = [softmax_t(target[v], T) for v in range(N + 1)]
    p_cand = np.array([p[parents[k]][tokens[k]] for k in range(N)])
    v, path, tests = 0, [], []
    while True:
        w = p[v].copy()           # the residual at v, unnormalised
        nxt, removed, fallback, w_before = None, [], False, None
        for c in tree_children(parents, v):
            x = int(tokens[c - 1])
            r = w[x] / np.sum(w)  # the candidate's probability under the residual; q(c) = 1
            ok = bool(u[c - 1] < min(1.0, r))
            ok = force.get(c, ok)
            tests.append((c, float(r), float(u[c - 1])))
            if ok:
                nxt = c
                break
            removed.append(c)
            w_before = w.copy()
            w[x] = 0.0            # max(0, r - delta_c), up to the normaliser
        if nxt is None:
            break
        path.append(nxt)
        v = nxt
    if np.sum(w) == 0.0:          # cannot happen with u < 1 (r = 1 accepts); mirrors the chain's Z = 0 rule
        w, fallback = w_before, True
    t, margin = inverse_cdf(w, float(u[N]))
    out = [int(tokens[c - 1]) for c in path] + [t]
    return TreeResult(len(path), path, out, v, removed, p_cand, tests, margin, float(np.sum(w)), fallback,
                      False)


def tree_rows(target: np.ndarray, parents: np.ndarray, tokens: np.ndarray, uniforms: np.ndarray,
              cu_nodes: np.ndarray, dtype: str, b: int):
    """The rows of sequence b in the packed layout: nodes cu_nodes[b] ..
    cu_nodes[b+1] - 1 and target rows / uniforms cu_t[b] .. cu_t[b] + N_b with
    cu_t[b] = cu_nodes[b] + b.  Returns (target [N+1, V] decoded, parents [N],
    tokens [N], u [N+1])."""
    n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
    t0 = n0 + b
    N = n1 - n0
    return (decode_logits(target[t0:t0 + N + 1], dtype), np.asarray(parents[n0:n1]),
            np.asarray(tokens[n0:n1]), np.asarray(uniforms[t0:t0 + N + 1]))


def verify_tree_batch(target: np.ndarray, parents: np.ndarray, tokens: np.ndarray, uniforms: np.ndarray,
                      temperatures: np.ndarray, cu_nodes: np.ndarray, dtype: str,
                      sequences: Optional[Sequence[int]] = None):
    """Verify a packed batch of trees.  Returns (accepted_len [B],
    out_tokens [R_t], out_nodes [R_t], p_cand [N_total], results): sequence
    b's n_b + 1 emitted tokens and its n_b accepted nodes (1-based, in path
    order) start at cu_t[b]; other entries are -1 (p_cand NaN).  Sequences
    outside ``sequences`` keep accepted_len -2."""
    cu_nodes = np.asarray(cu_nodes, dtype=np.int64)
    B = cu_nodes.shape[0] - 1
    N_tot = int(cu_nodes[-1])
    R_t = N_tot + B
    acc = np.full(B, -2, dtype=np.int64)
    out_tokens = np.full(R_t, -1, dtype=np.int64)
    out_nodes = np.full(R_t, -1, dtype=np.int64)
    p_cand = np.full(N_tot, np.nan)
    results = {}
    for b in (range(B) if sequences is None else sequences):
        n0, n1 = int(cu_nodes[b]), int(cu_nodes[b + 1])
        t0 = n0 + b
        tg, par, tk, u = tree_rows(target, parents, tokens, uniforms, cu_nodes, dtype, b)
        res = verify_tree(tg, par, tk, u, float(temperatures[b]))
        results[b] = res
        acc[b] = res.n
        if res.n >= 0:
            out_tokens[t0:t0 + res.n + 1] = res.tokens
            out_nodes[t0:t0 + res.n] = res.path
        p_cand[n0:n1] = res.p_cand
    return acc, out_tokens, out_nodes, p_cand, results
