"""GPU-vs-oracle comparison for draft trees (the tree analogue of parity.py).

A sequence's GPU output must equal the float64 oracle's, or differ only
where float32 may legitimately differ:
  * a candidate test whose uniform lies within 1e-5 of its ratio r: the
    GPU may take the other branch; the oracle is re-run with that decision
    forced, and the GPU output must equal that walk (one flip at a time);
  * the final sample: the GPU token must have positive weight under the stop
    node's residual and its CDF interval must come within the band of the
    final uniform (the band is parity.sample_band of the residual's mass).
Invalid and greedy sequences must match exactly.  p_cand within 1e-5
relative of the oracle (1e-6 absolute floor, as Z in parity.py: a
candidate probability is an e times a scale, both rounded).
"""
import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

from oracle import decode_logits, softmax_t, tree_rows, verify_tree, verify_tree_batch

from parity import sample_band

ACC_BAND = 1e-5


@dataclasses.dataclass
class TreeReport:
    checked: int = 0
    exact: int = 0
    flips: int = 0          # sequences explained by one forced decision
    sample_edge: int = 0    # sequences whose final token is the neighbour across a CDF edge
    invalid: int = 0
    greedy: int = 0
    mismatches: List[str] = dataclasses.field(default_factory=list)
    max_rel_p: float = 0.0

    def ok(self) -> bool:
        return not self.mismatches

    def summary(self) -> str:
        return (f"checked={self.checked} exact={self.exact} flips={self.flips} sample_edge={self.sample_edge} "
                f"invalid={self.invalid} greedy={self.greedy} p_cand_max_rel={self.max_rel_p:.2e} "
                f"mismatches={self.mismatches[:5]}")


def _sample_ok(tg, par, tk, res, T, u_final, tok) -> bool:
    w = softmax_t(tg[res.stop], T).copy()
    for c in res.removed:
        w[int(tk[c - 1])] = 0.0
    if np.sum(w) == 0.0:
        return False
    if tok < 0 or tok >= w.shape[0] or w[tok] <= 0.0:
        return False
    C = np.cumsum(w) / np.sum(w)
    lo = C[tok - 1] if tok > 0 else 0.0
    hi = C[tok]
    band = sample_band(float(res.sample_mass))
    return lo - band <= u_final < hi + band


def _walk_matches(res, n, toks, nodes) -> bool:
    return (res.n == n and list(res.tokens) == list(toks[:n + 1]) and list(res.path) == list(nodes[:n]))


def compare_tree(inp, got: Dict[str, np.ndarray], sequences: Optional[Sequence[int]] = None) -> TreeReport:
    rep = TreeReport()
    B = inp.batch
    dtype = inp.workload.dtype
    seqs = range(B) if sequences is None else sequences
    acc_o, out_o, nodes_o, pc_o, results = verify_tree_batch(
        inp.target, inp.parents, inp.tokens, inp.uniforms, inp.temperatures, inp.cu_nodes, dtype, sequences=seqs)
    for b in seqs:
        rep.checked += 1
        res = results[b]
        n0, n1 = int(inp.cu_nodes[b]), int(inp.cu_nodes[b + 1])
        N = n1 - n0
        t0 = n0 + b
        gn = int(got["accepted_len"][b])
        gt = got["out_tokens"][t0:t0 + N + 1]
        gnodes = got["out_nodes"][t0:t0 + N + 1] if "out_nodes" in got else None
        T = float(inp.temperatures[b])
        if res.n < 0:
            rep.invalid += 1
            if gn != -1 or np.any(gt != -1) or (gnodes is not None and np.any(gnodes != -1)):
                rep.mismatches.append(f"seq {b}: invalid in the oracle, GPU n={gn}")
            continue
        if gn < 0 or gn > N or np.any(gt[gn + 1:] != -1) or (gnodes is not None and np.any(gnodes[gn:] != -1)):
            rep.mismatches.append(f"seq {b}: malformed GPU output n={gn}")
            continue
        if gnodes is None:
            gnodes_l = list(res.path)
        else:
            gnodes_l = [int(x) for x in gnodes[:gn]]
        if res.greedy:
            rep.greedy += 1
        if _walk_matches(res, gn, gt.tolist(), gnodes_l):
            rep.exact += 1
        else:
            tg, par, tk, u = tree_rows(inp.target, inp.parents, inp.tokens, inp.uniforms, inp.cu_nodes, dtype, b)
            explained = False
            if not res.greedy:
                # the same walk with a final token across a near CDF edge
                if (res.n == gn and list(res.path) == gnodes_l and list(res.tokens[:gn]) == gt[:gn].tolist()
                        and _sample_ok(tg, par, tk, res, T, float(u[N]), int(gt[gn]))):
                    rep.sample_edge += 1
                    explained = True
                # one test next to its ratio taken the other way
                for (c, r, uc) in res.tests:
                    if explained or not np.isfinite(r) or abs(uc - r) > ACC_BAND:
                        continue
                    alt = verify_tree(tg, par, tk, u, T, force={c: not (uc < min(1.0, r))})
                    if alt.n == gn and list(alt.path) == gnodes_l and list(alt.tokens[:gn]) == gt[:gn].tolist():
                        if alt.tokens[gn] == int(gt[gn]) or _sample_ok(tg, par, tk, alt, T, float(u[N]), int(gt[gn])):
                            rep.flips += 1
                            explained = True
            if not explained:
                rep.mismatches.append(f"seq {b}: GPU n={gn} tokens={gt[:gn + 1].tolist()} nodes={gnodes_l}, "
                                      f"oracle n={res.n} tokens={res.tokens} nodes={res.path}")
        if "p_cand" in got and not res.greedy:
            g = got["p_cand"][n0:n1].astype(np.float64)
            o = res.p_cand
            err = np.abs(g - o)
            tol = np.maximum(1e-5 * np.abs(o), 1e-6)
            rep.max_rel_p = max(rep.max_rel_p, float(np.where(np.abs(o) > 1e-6, err / np.maximum(np.abs(o), 1e-30), 0).max()) if N else 0.0)
            if np.any(~(err <= tol)):
                k = int(np.argmax(err - tol))
                rep.mismatches.append(f"seq {b}: p_cand[{k}] GPU {g[k]:.9g} oracle {o[k]:.9g}")
        elif "p_cand" in got and res.greedy:
            g = got["p_cand"][n0:n1]
            if np.any(g != res.p_cand):
                rep.mismatches.append(f"seq {b}: greedy p_cand {g.tolist()} vs {res.p_cand.tolist()}")
    return rep
