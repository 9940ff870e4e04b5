"""Float64 CPU oracle of the speculative-decoding verification sampler.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The product
path (the HIP library and its Python binding) never calls it, and it shares
no code with that path: it decodes its own inputs and computes every step
with plain numpy in float64.

What it computes, per sequence, with the pages' notation (p = target
distribution, q = draft distribution, x = drafted token, gamma = number of
drafts):

1. p and q by temperature softmax of the target and draft logits of each
   position, with the sequence's temperature T applied to both (a reading:
   the pages never mention a temperature; see ``softmax_t``).
2. For positions i = 0 .. gamma-1 in order, accept x_i when
   u_i < min(1, p_i(x_i) / q_i(x_i)) -- velog "6-1편. Speculative Decoding",
   section 2-1 "추측 수락/거부 규칙" (the min(1, p/q) rule); the same page,
   section 2 "알고리즘 4단계", step 3.
3. At the first rejection n, sample from the residual
   p'(x) = norm(max(0, p(x) - q(x))) -- same page, section 2-2 "보정 분포
   p'(x)" and step 4 of "알고리즘 4단계".  If every draft is accepted,
   sample a bonus token from p_gamma (step 4; also "How to Scale Your
   Model -- All About Transformer Inference", Appendix D "Speculative
   Sampling", and Perplexity "Accelerating Sonar through speculation",
   section "추측적 디코딩": n drafts emit up to n + 1 tokens).
4. Sampling is proportional to the weights (velog page, box "샘플링이란"),
   done as inverse CDF in token order with one uniform u_gamma.
5. Greedy decoding (T = 0): accept while the draft equals the target
   argmax, replace the first wrong token by the target argmax, and if all
   are right take one more argmax from the last logits (scaling-book
   Appendix D, the three greedy steps).

Diagnostics per draft row: p(x), q(x), beta = sum_x min(p, q) (velog page,
section 2-3, item 1) and the residual mass Z = sum_x max(0, p - q) (section
2-3, item 2: the normaliser of p').

Readings where the pages are silent (each also listed in the design notes):
  * temperature: one T per sequence divides both target and draft logits;
  * u_0 .. u_{gamma-1} drive the acceptance tests, u_gamma the one final
    sample (residual or bonus);
  * q(x) = 0: ratio is +inf if p(x) > 0 (accept), 0/0 rejects;
  * Z = 0 (p <= q everywhere): the residual is undefined (the page divides
    by 1 - beta); sample from p instead;
  * CDF in ascending token id, strict ``C_k > u * Z``; if rounding leaves no
    such k, the last token of positive weight;
  * greedy ties: the lowest token id wins;
  * invalid data (any NaN or +inf logit, a row of only -inf, a token outside
    [0, V), a temperature that is negative, non-finite or in (0, FLT_MIN), a
    uniform outside [0, 1) or NaN) makes the whole sequence invalid: accepted
    length -1, tokens -1.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests
(worked examples from the pages, closed forms, invariants, exact u-grid
measures, brute force on tiny inputs, the greedy limit, a hand-worked packed
batch and a table of bf16 bit patterns).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np

FLT_MIN = float(np.finfo(np.float32).tiny)

__all__ = [
    "decode_logits", "softmax_t", "argmax_first", "inverse_cdf",
    "SequenceResult", "verify_sequence", "verify_batch", "FLT_MIN",
    "final_weights", "cdf_interval", "sequence_distributions", "sequence_rows",
]


def decode_logits(rows: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits -> float64.  bf16 is the top half of a float32."""
    if dtype == "f32":
        return np.asarray(rows, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        wide = np.asarray(rows, dtype=np.uint16).astype(np.uint32) << 16
        return wide.view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def softmax_t(logits: np.ndarray, T: float) -> np.ndarray:
    """Temperature softmax exp(l/T) / sum exp(l/T), T > 0, in float64.

    Shifting by the row maximum L leaves the ratio unchanged and keeps
    every exponent <= 0; exp(-inf) = 0.
    """
    L = np.max(logits)
    e = np.exp((logits - L) / T)
    return e / np.sum(e)


def argmax_first(logits: np.ndarray) -> int:
    """Index of the largest logit; the lowest index wins ties."""
    return int(np.argmax(logits))


def inverse_cdf(weights: np.ndarray, u: float):
    """Sample proportional to non-negative ``weights`` with uniform u.

    Returns (token, margin): token = min{k : C_k > u * C_{V-1}} with
    C = cumsum(weights) in token order; margin is the distance in u-units
    from u to the nearer edge of the chosen token's CDF interval.
    """
    C = np.cumsum(weights)
    Z = C[-1]
    thr = u * Z
    hits = np.nonzero(C > thr)[0]
    if hits.size:
        t = int(hits[0])
    else:  # u * Z rounded up to the total: take the last token with weight
        t = int(np.nonzero(weights > 0)[0][-1])
    lo = C[t - 1] if t > 0 else 0.0
    margin = min(abs(u - lo / Z), abs(u - C[t] / Z))
    return t, float(margin)


@dataclasses.dataclass
class SequenceResult:
    n: int                      # accepted drafts; -1 = invalid sequence
    tokens: List[int]           # n + 1 emitted tokens (empty if invalid)
    p_x: np.ndarray             # [gamma] p_i(x_i)
    q_x: np.ndarray             # [gamma] q_i(x_i)
    beta: np.ndarray            # [gamma] sum min(p_i, q_i)
    resid: np.ndarray           # [gamma] sum max(0, p_i - q_i)
    acc_margin: List[float]     # |u_i - r_i| of each evaluated test, i <= n (inf if r_i = inf)
    sample_margin: float        # u-distance of u_gamma to the chosen CDF interval edge
    sample_mass: float          # total weight of the sampled distribution (Z, or 1 for p)
    fallback: bool              # residual mass was 0, sampled from p
    greedy: bool
    # Every position, also those after the first rejection (for the parity
    # accounting of decisions that lie near a switching point):
    accept: np.ndarray = None       # [gamma] bool: u_i < min(1, r_i) (greedy: x_i == argmax)
    ratio: np.ndarray = None        # [gamma] r_i = p_i(x_i) / q_i(x_i) (rules of the q = 0 case)
    acc_margin_all: np.ndarray = None   # [gamma] |u_i - r_i| (inf if r_i = inf; greedy: inf)
    alt_tokens: List[int] = None    # [gamma+1] final token if the first rejection were at j
                                    # (j = gamma: the bonus token)
    alt_margin: np.ndarray = None   # [gamma+1] margins of those samples
    alt_mass: np.ndarray = None     # [gamma+1] their total weights
    alt_fallback: np.ndarray = None # [gamma+1] bool: Z = 0 fallback to p at j


def _sequence_valid(target: np.ndarray, draft: np.ndarray, tokens: np.ndarray,
                    u: np.ndarray, T: float, V: int) -> bool:
    if not np.isfinite(T) or T < 0.0 or (0.0 < T < FLT_MIN):
        return False
    for rows in (target, draft):
        if rows.size == 0:
            continue
        if np.isnan(rows).any() or np.isposinf(rows).any():
            return False
        if np.any(np.all(np.isneginf(rows), axis=1)):
            return False
    if np.any((tokens < 0) | (tokens >= V)):
        return False
    # the uniforms are draws from [0, 1) (velog page, section 2 step 3: a
    # rejection "with probability 1 - p/q" needs u uniform on the unit
    # interval); anything else, NaN included, is invalid data
    if not np.all((u >= 0.0) & (u < 1.0)):
        return False
    return True


def final_weights(p_j: np.ndarray, q_j: Optional[np.ndarray]):
    """Weights of the final sample at position j, unnormalised, and whether
    the Z = 0 fallback applied.

    q_j None: j is the bonus position (all drafts accepted) and the sample
    is drawn from p_j itself (velog page, section 2 step 4).  Otherwise j is
    the first rejection and the sample is drawn from max(0, p_j - q_j)
    (section 2-2); if that is zero everywhere, from p_j (the page divides
    by 1 - beta = 0 there; reading R5).
    """
    if q_j is None:
        return p_j, False
    w = np.maximum(0.0, p_j - q_j)
    if np.sum(w) == 0.0:
        return p_j, True
    return w, False


def cdf_interval(weights: np.ndarray, t: int):
    """The u-interval [C_{t-1} / Z, C_t / Z) that inverse_cdf maps to token
    t, with C = cumsum(weights) in token order and Z = C_{V-1}."""
    C = np.cumsum(weights)
    Z = C[-1]
    lo = C[t - 1] if t > 0 else 0.0
    return float(lo / Z), float(C[t] / Z)


def sequence_distributions(target: np.ndarray, draft: Optional[np.ndarray], tokens: Sequence[int], T: float):
    """p_i (i <= gamma) and q_i (i < gamma) of a sampled sequence, T > 0:
    temperature softmax of the target and draft logits; a token-only draft
    is the point mass delta_{x_i}."""
    target = np.asarray(target, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
    gamma, V = tokens.shape[0], target.shape[1]
    p = [softmax_t(target[i], T) for i in range(gamma + 1)]
    if draft is None:
        q = [np.eye(1, V, int(tokens[i]))[0] for i in range(gamma)]
    else:
        draft = np.asarray(draft, dtype=np.float64).reshape(-1, V)
        q = [softmax_t(draft[i], T) for i in range(gamma)]
    return p, q


def verify_sequence(target: np.ndarray, draft: Optional[np.ndarray], tokens: Sequence[int],
                    u: Sequence[float], T: float) -> SequenceResult:
    """Verify one sequence.

    target: [gamma+1, V] float64 logits; draft: [gamma, V]; tokens: [gamma]
    drafted ids; u: [gamma+1] uniforms in [0, 1); T: temperature (0 = greedy).

    draft None: token-only drafts.  An n-gram or token-matching drafter gives
    no distribution (velog "6-1편. Speculative Decoding", section 4 "그 이후
    등장한 아이디어들: Mq 모델", N-gram; "How to Scale Your Model -- All About
    Transformer Inference", Appendix D, the drafter options).  The draft
    distribution is then the point mass q_i = delta_{x_i}, and every step below
    applies unchanged: accept with probability min(1, p(x) / 1) = p(x); the
    residual max(0, p - delta_x) is p with x removed; beta = p(x); the draft's
    argmax (greedy) is x.

    Besides the emitted tokens, the result holds the decision of every
    position (as if each were reached) and the final sample for every
    possible first rejection: they are what a float32 implementation may
    legitimately reach instead when a uniform lies next to a switching point.
    """
    target = np.asarray(target, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64).reshape(-1)
    u = np.asarray(u, dtype=np.float64).reshape(-1)
    token_only = draft is None
    gamma, V = tokens.shape[0], target.shape[1]
    draft_chk = np.zeros((0, V)) if token_only else np.asarray(draft, dtype=np.float64).reshape(-1, V)
    assert target.shape[0] == gamma + 1 and u.shape[0] == gamma + 1
    assert token_only or draft_chk.shape[0] == gamma
    nan = np.full(gamma, np.nan)
    if not _sequence_valid(target, draft_chk, tokens, u, float(T), V):
        return SequenceResult(-1, [], nan, nan.copy(), nan.copy(), nan.copy(), [], np.inf, np.nan, False, T == 0.0,
                              np.zeros(0, bool), np.zeros(0), np.zeros(0), [], np.zeros(0), np.zeros(0),
                              np.zeros(0, bool))

    if T == 0.0:
        # Greedy verification: the distributions are one-hot at the argmax.
        at = [argmax_first(target[i]) for i in range(gamma + 1)]
        ad = [int(tokens[i]) if token_only else argmax_first(draft_chk[i]) for i in range(gamma)]
        accept = np.array([tokens[i] == at[i] for i in range(gamma)], dtype=bool)
        p_x = accept.astype(np.float64)
        q_x = np.array([1.0 if tokens[i] == ad[i] else 0.0 for i in range(gamma)])
        beta = np.array([1.0 if at[i] == ad[i] else 0.0 for i in range(gamma)])
        n = gamma
        for i in range(gamma):
            if not accept[i]:
                n = i
                break
        out = [int(t) for t in tokens[:n]] + [at[n]]
        inf_g = np.full(gamma, np.inf)
        return SequenceResult(n, out, p_x, q_x, beta, 1.0 - beta, [], np.inf, 1.0, False, True,
                              accept, p_x / np.maximum(q_x, 1e-300), inf_g, list(at),
                              np.full(gamma + 1, np.inf), np.ones(gamma + 1), np.zeros(gamma + 1, bool))

    p, q = sequence_distributions(target, draft, tokens, T)
    p_x = np.array([p[i][tokens[i]] for i in range(gamma)])
    q_x = np.array([q[i][tokens[i]] for i in range(gamma)])
    beta = np.array([np.sum(np.minimum(p[i], q[i])) for i in range(gamma)])
    resid = np.array([np.sum(np.maximum(0.0, p[i] - q[i])) for i in range(gamma)])

    # the test of every position: u_i < min(1, r_i) (velog page, section 2-1)
    ratio = np.empty(gamma)
    accept = np.zeros(gamma, dtype=bool)
    margin_all = np.empty(gamma)
    for i in range(gamma):
        if q_x[i] > 0.0:
            r = p_x[i] / q_x[i]
        else:
            r = np.inf if p_x[i] > 0.0 else 0.0
        ratio[i] = r
        accept[i] = u[i] < min(1.0, r)
        margin_all[i] = abs(u[i] - r) if np.isfinite(r) else np.inf
    n = gamma
    for i in range(gamma):
        if not accept[i]:
            n = i
            break

    # the final sample for every possible first rejection j, and the bonus
    # sample (j = gamma), all with the one uniform u_gamma (reading R2)
    alt_tokens, alt_margin, alt_mass, alt_fb = [], np.empty(gamma + 1), np.empty(gamma + 1), np.zeros(gamma + 1, bool)
    for j in range(gamma + 1):
        w, fb = final_weights(p[j], q[j] if j < gamma else None)
        t, m = inverse_cdf(w, float(u[gamma]))
        alt_tokens.append(t)
        alt_margin[j] = m
        alt_mass[j] = float(np.sum(w))
        alt_fb[j] = fb

    out = [int(x) for x in tokens[:n]] + [alt_tokens[n]]
    acc_margin = [float(margin_all[i]) for i in range(min(n + 1, gamma))]
    return SequenceResult(n, out, p_x, q_x, beta, resid, acc_margin, float(alt_margin[n]),
                          float(alt_mass[n]), bool(alt_fb[n]), False,
                          accept, ratio, margin_all, alt_tokens, alt_margin, alt_mass, alt_fb)


def sequence_rows(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
                  uniforms: np.ndarray, cu_draft: np.ndarray, dtype: str, b: int):
    """The rows of sequence b in the packed layout of the C ABI, decoded.

    Sequence b owns draft rows cu_draft[b] .. cu_draft[b+1] - 1 and target
    rows cu_t[b] .. cu_t[b] + gamma_b with cu_t[b] = cu_draft[b] + b (one
    more target row than draft rows per sequence); its uniforms sit at the
    target rows' positions.  Returns (target [gamma+1, V], draft [gamma, V] or
    None, tokens [gamma], u [gamma+1]).
    """
    d0, d1 = int(cu_draft[b]), int(cu_draft[b + 1])
    t0 = d0 + b
    g = d1 - d0
    return (decode_logits(target[t0:t0 + g + 1], dtype),
            None if draft is None else decode_logits(draft[d0:d1], dtype),
            np.asarray(draft_tokens[d0:d1]), np.asarray(uniforms[t0:t0 + g + 1]))


def verify_batch(target: np.ndarray, draft: Optional[np.ndarray], draft_tokens: np.ndarray,
                 uniforms: np.ndarray, temperatures: np.ndarray, cu_draft: np.ndarray,
                 dtype: str, sequences: Optional[Sequence[int]] = None):
    """Verify a packed batch (the layout of the C ABI).  ``draft`` None:
    token-only drafts (see ``verify_sequence``).

    Returns (accepted_len [B], out_tokens [R_t], p_x, q_x, beta, resid
    [R_d] each, per-sequence results).  out_tokens of sequence b holds its
    n_b + 1 emitted tokens from cu_t[b] on and -1 in its other rows.
    ``sequences`` restricts the work to a subset; the other entries stay at
    their fill values (accepted_len -2, tokens -1, diagnostics NaN).
    """
    cu_draft = np.asarray(cu_draft, dtype=np.int64)
    B = cu_draft.shape[0] - 1
    R_d = int(cu_draft[-1])
    R_t = R_d + B
    acc_len = np.full(B, -2, dtype=np.int64)
    out = np.full(R_t, -1, dtype=np.int64)
    diag = {k: np.full(R_d, np.nan) for k in ("p_x", "q_x", "beta", "resid")}
    results = {}
    for b in (range(B) if sequences is None else sequences):
        d0, d1 = int(cu_draft[b]), int(cu_draft[b + 1])
        t0 = d0 + b
        tg, dr, tk, u = sequence_rows(target, draft, draft_tokens, uniforms, cu_draft, dtype, b)
        res = verify_sequence(tg, dr, tk, u, float(temperatures[b]))
        results[b] = res
        acc_len[b] = res.n
        if res.n >= 0:
            out[t0:t0 + res.n + 1] = res.tokens
        diag["p_x"][d0:d1] = res.p_x
        diag["q_x"][d0:d1] = res.q_x
        diag["beta"][d0:d1] = res.beta
        diag["resid"][d0:d1] = res.resid
    return acc_len, out, diag["p_x"], diag["q_x"], diag["beta"], diag["resid"], results
