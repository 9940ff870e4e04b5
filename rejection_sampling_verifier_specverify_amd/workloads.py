"""Seeded synthetic inputs for the speculative-decoding verification sampler.

This module draws the random data that both the HIP path and the CPU oracle
consume: target and draft logits, the drafter's tokens, the verifier's
uniforms, the per-sequence temperatures and the ragged draft lengths.  It
holds none of the verifier's arithmetic (no softmax, no acceptance test, no
residual, no inverse CDF).  The drafter's own sampling -- "Mq proposes gamma
tokens" (velog "6-1편. Speculative Decoding", section 2 "알고리즘 4단계",
step 1) -- is simulated with the Gumbel-max trick, argmax(l_d / T + G), which
draws exactly from softmax(l_d / T) without computing it; a greedy drafter
(T = 0) proposes argmax(l_d).

Recipe (every stream is numpy ``Generator(Philox(SeedSequence(key)))``):
  * key (seed, cfg_id, 0): per-sequence metadata, drawn in this order --
    ragged draft lengths (if the workload is ragged), then temperatures (if
    they are drawn from a set).
  * key (seed, cfg_id, 1, r): float64 values of target row r.
  * key (seed, cfg_id, 2, d): draft row d: first the additive noise, then
    the V Gumbel(0, 1) draws of the drafter (T > 0 only).
  * key (seed, cfg_id, 3): the verifier uniforms, one float32 in [0, 1) per
    target row, in packed row order.
Logits are drawn in float64, then rounded to float32 and, for bf16
workloads, from float32 to bf16 with round-to-nearest-even.  Draft rows are
built from the float64 (unrounded) target row of the same position.

Layout (the layout the C ABI takes): sequence b owns draft rows
cu_draft[b] .. cu_draft[b+1]-1 and target rows cu_t[b] .. cu_t[b]+gamma_b,
where cu_t[b] = cu_draft[b] + b.  uniforms[cu_t[b] + i] for i < gamma_b is
the acceptance uniform of position i, uniforms[cu_t[b] + gamma_b] feeds the
final (residual or bonus) sample.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional, Sequence, Tuple, Union

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "HEADLINE", "Inputs", "make_inputs", "token_only",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
    "TreeWorkload", "TREE_WORKLOADS", "TreeInputs", "make_tree_inputs", "tree_shape",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """A synthetic verification batch: shapes and value distributions."""
    name: str
    cfg_id: int
    batch: int
    gamma: Union[int, Tuple[int, int]]   # fixed draft length, or (lo, hi) uniform ragged
    vocab: int
    dtype: str                           # "f32" or "bf16"
    target: Tuple                        # ("normal", sigma) | ("gumbel", scale) | ("student_t", nu, scale)
    draft_scale: float                   # draft = draft_scale * target + N(0, draft_sigma^2)
    draft_sigma: float
    temps: Tuple                         # ("const", T) | ("choice", (T0, T1, ...))

    @property
    def ragged(self) -> bool:
        return not isinstance(self.gamma, int)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("b1_g4_v32000_f32", 0, 1, 4, 32000, "f32",
                 ("normal", 2.0), 1.0, 0.5, ("const", 1.0)),
        Workload("b64_g4_v128256_bf16", 1, 64, 4, 128256, "bf16",
                 ("normal", 3.0), 0.8, 1.5, ("const", 0.7)),
        Workload("b256_g8_v128256_bf16_mixedT", 2, 256, 8, 128256, "bf16",
                 ("gumbel", 2.0), 1.0, 1.0, ("choice", (0.0, 0.6, 1.0))),
        Workload("b32_g1_v129280_bf16_mtp", 3, 32, 1, 129280, "bf16",
                 ("normal", 2.5), 1.0, 0.3, ("const", 1.0)),
        Workload("b512_gragged1to7_v152064_bf16", 4, 512, (1, 7), 152064, "bf16",
                 ("student_t", 3.0, 2.0), 0.7, 2.0, ("const", 0.8)),
    ]
}
HEADLINE = "b64_g4_v128256_bf16"


@dataclasses.dataclass
class Inputs:
    """One batch in the packed layout.  Logits are float32 arrays (f32) or
    uint16 arrays holding bf16 bit patterns (bf16)."""
    workload: Workload
    seed: int
    target: np.ndarray        # [R_t, V]
    draft: Optional[np.ndarray]   # [R_d, V]; None: token-only drafts
    draft_tokens: np.ndarray  # [R_d] int32
    uniforms: np.ndarray      # [R_t] float32
    temperatures: np.ndarray  # [B] float32
    cu_draft: np.ndarray      # [B+1] int32

    @property
    def batch(self) -> int:
        return int(self.cu_draft.shape[0] - 1)

    @property
    def gammas(self) -> np.ndarray:
        return np.diff(self.cu_draft).astype(np.int64)

    @property
    def cu_t(self) -> np.ndarray:
        return (self.cu_draft + np.arange(self.batch + 1)).astype(np.int64)

    @property
    def uniform_gamma(self) -> Optional[int]:
        g = self.gammas
        if g.size and np.all(g == g[0]):
            return int(g[0])
        return None

    @property
    def logit_bytes(self) -> int:
        return int(self.target.nbytes + (self.draft.nbytes if self.draft is not None else 0))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    rounded = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = (((b[nan] >> 16) | 0x40) & 0xFFFF).astype(np.uint16)
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _stream(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence(list(key))))


def _draw_target(w: Workload, rng: np.random.Generator) -> np.ndarray:
    kind = w.target[0]
    if kind == "normal":
        return rng.standard_normal(w.vocab) * w.target[1]
    if kind == "gumbel":
        return rng.gumbel(0.0, w.target[1], size=w.vocab)
    if kind == "student_t":
        return rng.standard_t(w.target[1], size=w.vocab) * w.target[2]
    raise ValueError(f"unknown target distribution {kind!r}")


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def _as_f64(row: np.ndarray, dtype: str) -> np.ndarray:
    return (row if dtype == "f32" else bf16_bits_to_f32(row)).astype(np.float64)


def drafter_token(draft_logits: np.ndarray, T: float, rng: np.random.Generator) -> int:
    """The simulated drafter: a draw from softmax(l_d / T) by the Gumbel-max
    trick (T > 0), or argmax l_d for a greedy drafter (T = 0)."""
    if T > 0.0:
        return int(np.argmax(draft_logits / T + rng.gumbel(size=draft_logits.shape[0])))
    return int(np.argmax(draft_logits))


def make_inputs(w: Union[Workload, str], seed: int = 0, *, batch: Optional[int] = None,
                threads: Optional[int] = None) -> Inputs:
    """Draw one batch of workload ``w`` (optionally with a smaller batch)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if batch is not None:
        w = w.replace(batch=batch)
    B, V = w.batch, w.vocab
    meta = _stream(seed, w.cfg_id, 0)
    if w.ragged:
        lo, hi = w.gamma
        gammas = meta.integers(lo, hi + 1, size=B)
    else:
        gammas = np.full(B, w.gamma, dtype=np.int64)
    if w.temps[0] == "const":
        temps = np.full(B, w.temps[1], dtype=np.float32)
    else:
        choices = np.asarray(w.temps[1], dtype=np.float32)
        temps = choices[meta.integers(0, len(choices), size=B)]
    cu_draft = np.zeros(B + 1, dtype=np.int32)
    cu_draft[1:] = np.cumsum(gammas)
    R_d = int(cu_draft[-1])
    R_t = R_d + B
    store = np.float32 if w.dtype == "f32" else np.uint16
    target = np.empty((R_t, V), dtype=store)
    draft = np.empty((R_d, V), dtype=store)
    tokens = np.empty(R_d, dtype=np.int32)

    def one_sequence(b: int) -> None:
        g = int(gammas[b])
        t0 = int(cu_draft[b]) + b
        d0 = int(cu_draft[b])
        T = float(temps[b])
        for i in range(g + 1):
            t64 = _draw_target(w, _stream(seed, w.cfg_id, 1, t0 + i))
            target[t0 + i] = _round(t64, w.dtype)
            if i == g:
                break
            rng = _stream(seed, w.cfg_id, 2, d0 + i)
            d64 = w.draft_scale * t64 + rng.standard_normal(V) * w.draft_sigma
            draft[d0 + i] = _round(d64, w.dtype)
            tokens[d0 + i] = drafter_token(_as_f64(draft[d0 + i], w.dtype), T, rng)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if B > 1 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one_sequence, range(B)))
    else:
        for b in range(B):
            one_sequence(b)
    uniforms = _stream(seed, w.cfg_id, 3).random(R_t, dtype=np.float32)
    return Inputs(w, seed, target, draft, tokens, uniforms, temps, cu_draft)


def make_custom(target: np.ndarray, draft: np.ndarray, tokens: Sequence[int],
                uniforms: Sequence[float], temperatures: Sequence[float],
                gammas: Sequence[int], dtype: str = "f32") -> Inputs:
    """Pack hand-built rows (float64/float32 logits) into the batch layout."""
    gam = np.asarray(gammas, dtype=np.int64)
    cu = np.zeros(len(gam) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(gam)
    tgt = np.asarray(target, dtype=np.float64)
    drf = np.asarray(draft, dtype=np.float64).reshape(-1, tgt.shape[1])
    w = Workload("custom", 99, len(gam), int(gam[0]) if len(set(gam.tolist())) == 1 else (int(gam.min()), int(gam.max())),
                 tgt.shape[1], dtype, ("normal", 1.0), 1.0, 0.0, ("const", 1.0))
    return Inputs(w, 0, _round(tgt, dtype), _round(drf, dtype),
                  np.asarray(tokens, dtype=np.int32).reshape(-1),
                  np.asarray(uniforms, dtype=np.float32).reshape(-1),
                  np.asarray(temperatures, dtype=np.float32).reshape(-1), cu)


def token_only(inp: Inputs) -> Inputs:
    """The same batch with token-only drafts: the drafted tokens stay (they
    were drawn from the draft distribution, one possible drafter's law) and
    the draft logits are dropped, so q_i = delta_{x_i}."""
    return dataclasses.replace(inp, draft=None)


# ---------------------------------------------------------------- draft trees

@dataclasses.dataclass(frozen=True)
class TreeWorkload:
    """A batch whose drafts form trees (EAGLE / Medusa style: the drafter's
    Top-K candidates at every node, Perplexity "Accelerating Sonar through
    speculation", section "EAGLE").  ``branching[d]`` children per node at
    depth d, nodes numbered breadth-first, at most ``nodes`` per tree."""
    name: str
    cfg_id: int
    batch: int
    nodes: int
    branching: Tuple[int, ...]
    vocab: int
    dtype: str
    target: Tuple                  # as Workload.target
    draft_sigma: float             # the drafter's scores: target row + N(0, draft_sigma^2)
    temps: Tuple                   # ("const", T) | ("choice", (T0, T1, ...))

    def replace(self, **kw) -> "TreeWorkload":
        return dataclasses.replace(self, **kw)


TREE_WORKLOADS = {
    w.name: w for w in [
        # an EAGLE-2 sized tree: 60 candidates, depth 4
        TreeWorkload("b16_tree60_v128256_bf16", 10, 16, 60, (4, 3, 2, 2, 1, 1), 128256, "bf16",
                     ("normal", 3.0), 1.5, ("const", 0.7)),
        # peaked rows, so that walks go deep (parity cases)
        TreeWorkload("b8_tree12_v32000_f32", 11, 8, 12, (3, 2, 1, 1), 32000, "f32",
                     ("normal", 6.0), 0.5, ("choice", (0.0, 0.8, 1.0))),
    ]
}


@dataclasses.dataclass
class TreeInputs:
    """One batch of draft trees in the packed layout of the C ABI: sequence
    b's nodes are cu_nodes[b] .. cu_nodes[b+1] - 1 (parents as local node
    numbers, 0 = root), its target rows and uniforms start at
    cu_t[b] = cu_nodes[b] + b."""
    workload: TreeWorkload
    seed: int
    target: np.ndarray        # [R_t, V] float32 or bf16 bits
    parents: np.ndarray       # [N] int32
    tokens: np.ndarray        # [N] int32
    uniforms: np.ndarray      # [R_t] float32
    temperatures: np.ndarray  # [B] float32
    cu_nodes: np.ndarray      # [B+1] int32

    @property
    def batch(self) -> int:
        return int(self.cu_nodes.shape[0] - 1)

    @property
    def cu_t(self) -> np.ndarray:
        return (self.cu_nodes + np.arange(self.batch + 1)).astype(np.int64)

    @property
    def logit_bytes(self) -> int:
        return int(self.target.nbytes)


def tree_shape(nodes: int, branching: Sequence[int]) -> np.ndarray:
    """Parents of a breadth-first tree with branching[d] children per node at
    depth d (the last entry repeats), cut at ``nodes`` nodes."""
    parents = []
    level = [0]
    d = 0
    while len(parents) < nodes and level:
        k = branching[min(d, len(branching) - 1)]
        nxt = []
        for v in level:
            for _ in range(k):
                if len(parents) == nodes:
                    break
                parents.append(v)
                nxt.append(len(parents))
        level = nxt
        d += 1
    return np.asarray(parents, dtype=np.int32)


def make_tree_inputs(w: Union[TreeWorkload, str], seed: int = 0, *, batch: Optional[int] = None,
                     nodes: Optional[Sequence[int]] = None) -> TreeInputs:
    """Draw one batch of tree workload ``w``.  ``nodes`` gives each sequence's
    node count (default: the workload's).  The candidates of node v are the
    drafter's top-k tokens at v: the k largest scores target_v + noise
    (distinct tokens, best first).

    Streams: key (seed, cfg_id, 0): temperatures; (seed, cfg_id, 1, r):
    target row r; (seed, cfg_id, 2, r): the drafter's noise at row r;
    (seed, cfg_id, 3): the uniforms."""
    if isinstance(w, str):
        w = TREE_WORKLOADS[w]
    if batch is not None:
        w = w.replace(batch=batch)
    B, V = w.batch, w.vocab
    counts = np.full(B, w.nodes, dtype=np.int64) if nodes is None else np.asarray(nodes, dtype=np.int64)
    meta = _stream(seed, w.cfg_id, 0)
    if w.temps[0] == "const":
        temps = np.full(B, w.temps[1], dtype=np.float32)
    else:
        choices = np.asarray(w.temps[1], dtype=np.float32)
        temps = choices[meta.integers(0, len(choices), size=B)]
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(counts)
    N = int(cu[-1])
    R_t = N + B
    store = np.float32 if w.dtype == "f32" else np.uint16
    target = np.empty((R_t, V), dtype=store)
    parents = np.empty(N, dtype=np.int32)
    tokens = np.empty(N, dtype=np.int32)
    proxy = Workload("tree-rows", w.cfg_id, B, 0, V, w.dtype, w.target, 1.0, 0.0, ("const", 1.0))

    def one_sequence(b: int) -> None:
        n = int(counts[b])
        n0, t0 = int(cu[b]), int(cu[b]) + b
        par = tree_shape(n, w.branching)
        parents[n0:n0 + n] = par
        kids = {}
        for k, pa in enumerate(par, start=1):
            kids.setdefault(int(pa), []).append(k)
        for v in range(n + 1):
            t64 = _draw_target(proxy, _stream(seed, w.cfg_id, 1, t0 + v))
            target[t0 + v] = _round(t64, w.dtype)
            if v in kids:
                score = t64 + _stream(seed, w.cfg_id, 2, t0 + v).standard_normal(V) * w.draft_sigma
                top = np.argsort(-score, kind="stable")[:len(kids[v])]
                for k, tok in zip(kids[v], top):
                    tokens[n0 + k - 1] = int(tok)

    nthreads = min(16, os.cpu_count() or 1)
    if B > 1 and nthreads > 1:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(one_sequence, range(B)))
    else:
        for b in range(B):
            one_sequence(b)
    uniforms = _stream(seed, w.cfg_id, 3).random(R_t, dtype=np.float32)
    return TreeInputs(w, seed, target, parents, tokens, uniforms, temps, cu)
