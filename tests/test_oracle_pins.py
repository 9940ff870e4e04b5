"""Pins of the float64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages (tests/golden), a closed form, an identity that
the oracle does not compute the same way, an exact measure over a fine grid
of uniforms, brute force on tiny inputs, a statistical law with an explicit
sigma bound, or a special case that reduces to a library routine.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats

from oracle import argmax_first, inverse_cdf, softmax_t, verify_sequence

GRID = 200_000  # u-grid points for exact-measure pins (step 5e-6)


def _ugrid(n=GRID):
    return (np.arange(n) + 0.5) / n


def _measure_tokens(weights, n=GRID):
    """Fraction of a midpoint grid of u that inverse_cdf maps to each token."""
    V = len(weights)
    counts = np.zeros(V)
    for u in _ugrid(n)[:: max(1, n // 20000)]:
        t, _ = inverse_cdf(np.asarray(weights, dtype=np.float64), float(u))
        counts[t] += 1
    return counts / counts.sum()


# ---------------------------------------------------------------- worked examples

def test_sampling_worked_example(golden_dir):
    """velog page, box '샘플링이란': probabilities 0.6/0.3/0.1 are drawn 60/30/10%."""
    g = json.load(open(os.path.join(golden_dir, "sampling_three_tokens.json")))
    p = np.array(g["probabilities"])
    freq = _measure_tokens(p)
    np.testing.assert_allclose(freq, g["selection_frequencies"], atol=1e-4)
    # Interval edges in token order: [0, .6) -> 0, [.6, .9) -> 1, [.9, 1) -> 2.
    assert inverse_cdf(p, 0.59)[0] == 0 and inverse_cdf(p, 0.61)[0] == 1
    assert inverse_cdf(p, 0.89)[0] == 1 and inverse_cdf(p, 0.91)[0] == 2
    t, margin = inverse_cdf(p, 0.65)
    assert t == 1 and margin == pytest.approx(0.05, abs=1e-12)


def test_inverse_cdf_strict_and_zero_weight():
    """The CDF test is strict, C_k > u Z, so a token of zero weight is never drawn:
    at u = 0 the first token of positive weight, and at an exact interval edge
    the next token of positive weight (reading of the '샘플링이란' box: a token
    of probability 0 has no chance)."""
    assert inverse_cdf(np.array([0.0, 0.6, 0.0, 0.4]), 0.0)[0] == 1
    assert inverse_cdf(np.array([0.5, 0.0, 0.5]), 0.5)[0] == 2
    assert inverse_cdf(np.array([0.25, 0.25, 0.0, 0.5]), 0.5)[0] == 3


def test_bonus_path_through_softmax(golden_dir):
    """gamma = 0: the emitted token is a sample of p = softmax(log p0) (T = 1)."""
    g = json.load(open(os.path.join(golden_dir, "sampling_three_tokens.json")))
    p0 = np.array(g["probabilities"])
    logits = np.log(p0)[None, :] + 5.0           # shift: softmax is shift invariant
    counts = np.zeros(3)
    for u in _ugrid(20000):
        r = verify_sequence(logits, np.zeros((0, 3)), [], [u], 1.0)
        assert r.n == 0
        counts[r.tokens[0]] += 1
    np.testing.assert_allclose(counts / counts.sum(), g["selection_frequencies"], atol=1e-4)


def test_expected_tokens_worked_example(golden_dir):
    """velog page, section 3-1 and table '예시로 한눈에 보기': alpha=0.8, gamma=4.

    Positions whose beta is exactly 0.8: p uniform over 8 tokens, q puts
    0.55/6 on tokens 0..5 and 0.225 on 6, 7, so sum min(p, q) = 6*0.55/6 + 2/8
    = 0.8.  Drafts are drawn from q with numpy's own sampler.
    """
    g = json.load(open(os.path.join(golden_dir, "expected_tokens_worked_example.json")))
    alpha, gamma = g["alpha"], g["gamma"]
    assert (1 - alpha ** (gamma + 1)) == pytest.approx(g["numerator_printed"], abs=5e-5)
    assert (1 - alpha) == pytest.approx(g["denominator_printed"])
    EN = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert EN == pytest.approx(g["expected_tokens_printed"], abs=0.005)

    p = np.full(8, 1 / 8)
    q = np.array([0.55 / 6] * 6 + [0.225, 0.225])
    assert np.minimum(p, q).sum() == pytest.approx(alpha, abs=1e-15)
    lt, ld = np.log(p), np.log(q)
    rng = np.random.default_rng(1234)
    trials = 20000
    emitted = np.empty(trials)
    for k in range(trials):
        x = rng.choice(8, size=gamma, p=q)
        u = rng.random(gamma + 1)
        r = verify_sequence(np.tile(lt, (gamma + 1, 1)), np.tile(ld, (gamma, 1)), x, u, 1.0)
        emitted[k] = r.n + 1
    # P(N >= k) = alpha^(k-1): check each tail and the mean, 4.5 sigma.
    for kk in range(1, gamma + 2):
        pk = alpha ** (kk - 1)
        sig = np.sqrt(pk * (1 - pk) / trials) + 1e-12
        assert abs(np.mean(emitted >= kk) - pk) < 4.5 * sig + 1e-12, kk
    var = sum(k * k * (alpha ** (k - 1) * (1 - alpha) if k <= gamma else alpha ** gamma)
              for k in range(1, gamma + 2)) - EN ** 2
    assert abs(emitted.mean() - EN) < 4.5 * np.sqrt(var / trials)


def test_hand_worked_residual():
    """p = (.5, .3, .2), q = (.2, .3, .5), by hand from the velog page 2-1..2-3:
    beta = .2 + .3 + .2 = .7; max(0, p - q) = (.3, 0, 0) so Z = .3 and p' = (1, 0, 0);
    x = 0 (q <= p) is always accepted; x = 2 is accepted iff u < .2/.5 = .4 and
    otherwise replaced by token 0; x = 1 (p = q) is always accepted."""
    lt = np.log([0.5, 0.3, 0.2])[None, :].repeat(2, 0)
    ld = np.log([0.2, 0.3, 0.5])[None, :]
    r = verify_sequence(lt, ld, [2], [0.39, 0.7], 1.0)
    assert r.n == 1 and r.tokens[0] == 2
    r = verify_sequence(lt, ld, [2], [0.41, 0.7], 1.0)
    assert r.n == 0 and r.tokens == [0]
    assert r.beta[0] == pytest.approx(0.7, abs=1e-12)
    assert r.resid[0] == pytest.approx(0.3, abs=1e-12)
    assert r.p_x[0] == pytest.approx(0.2) and r.q_x[0] == pytest.approx(0.5)
    assert r.acc_margin == [pytest.approx(0.01, abs=1e-12)]
    for u0 in (0.0, 0.5, 0.999999):
        assert verify_sequence(lt, ld, [0], [u0, 0.5], 1.0).n == 1
        assert verify_sequence(lt, ld, [1], [u0, 0.5], 1.0).n == 1
    # rejected x = 2 for any u_gamma -> token 0 (p' is one-hot)
    for ug in (0.0, 0.5, 0.999999):
        assert verify_sequence(lt, ld, [2], [0.9, ug], 1.0).tokens == [0]


# ---------------------------------------------------------------- exact u-grid measures

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_acceptance_measure_is_min_one_ratio(seed):
    """The set of u_i that accepts x has measure min(1, p(x)/q(x)) (velog 2-1)."""
    rng = np.random.default_rng(seed)
    V = 6
    lt, ld = rng.normal(size=(2, V)), rng.normal(size=(1, V))
    p, q = np.exp(lt[0]) / np.exp(lt[0]).sum(), np.exp(ld[0]) / np.exp(ld[0]).sum()
    us = _ugrid(4000)
    for x in range(V):
        acc = np.mean([verify_sequence(lt, ld, [x], [u, 0.5], 1.0).n == 1 for u in us])
        assert acc == pytest.approx(min(1.0, p[x] / q[x]), abs=2.5e-4)


@pytest.mark.parametrize("seed", [3, 4])
def test_residual_measure_is_normalised_excess(seed):
    """Given rejection, u_gamma maps to token t with measure max(0,p-q)_t / Z (velog 2-2)."""
    rng = np.random.default_rng(seed)
    V = 5
    lt, ld = rng.normal(size=(2, V)) * 1.5, rng.normal(size=(1, V)) * 1.5
    p, q = np.exp(lt[0]) / np.exp(lt[0]).sum(), np.exp(ld[0]) / np.exp(ld[0]).sum()
    x = int(np.argmax(q - p))              # a token with q > p, so u_0 = 0.999999 rejects
    w = np.maximum(0, p - q)
    counts = np.zeros(V)
    for u in _ugrid(10000):
        r = verify_sequence(lt, ld, [x], [0.999999, u], 1.0)
        assert r.n == 0
        counts[r.tokens[0]] += 1
    np.testing.assert_allclose(counts / counts.sum(), w / w.sum(), atol=1e-4)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("T", [1.0, 0.6])
def test_brute_force_output_law(T):
    """Exact law of the emitted tokens on V = 3, gamma = 1, by enumeration.

    Every draft x0 is enumerated with weight q0(x0); the decision at position
    0 depends on u0 alone and the final sample on u1 alone, so the law is the
    product of 1-D measures taken on midpoint grids of the oracle's own
    decisions.  The first emitted token must have law p0 and the bonus token
    (all accepted) law p1 (velog 2-3, item 3: P(x = x') = p(x'))."""
    rng = np.random.default_rng(7)
    V = 3
    lt, ld = rng.normal(size=(2, V)), rng.normal(size=(1, V))
    P = np.array([np.exp(r / T) / np.exp(r / T).sum() for r in lt])
    q = np.exp(ld[0] / T) / np.exp(ld[0] / T).sum()
    us = _ugrid(5000)
    first = np.zeros(V)
    bonus = np.zeros(V)
    for x0 in range(V):
        acc = np.mean([verify_sequence(lt, ld, [x0], [u, 0.5], T).n == 1 for u in us])
        rej_law = np.zeros(V)
        if acc < 1.0:
            for u in us:
                r = verify_sequence(lt, ld, [x0], [1.0 - 1e-9, u], T)
                assert r.n == 0
                rej_law[r.tokens[0]] += 1.0 / len(us)
        first[x0] += q[x0] * acc
        first += q[x0] * (1.0 - acc) * rej_law
        if acc > 0.0:
            law = np.zeros(V)
            for u in us:
                r = verify_sequence(lt, ld, [x0], [0.0, u], T)
                law[r.tokens[1]] += 1.0 / len(us)
            bonus += q[x0] * acc * law
    np.testing.assert_allclose(first, P[0], atol=1e-3)
    np.testing.assert_allclose(bonus / bonus.sum(), P[1], atol=1e-3)


# ---------------------------------------------------------------- statistical laws

def test_acceptance_rate_matches_beta_1e5():
    """Empirical acceptance over 10^5 trials with x ~ q equals beta = sum min(p, q)
    (velog 2-3, item 1) within 4.5 sigma."""
    rng = np.random.default_rng(11)
    V = 8
    lt, ld = rng.normal(size=(2, V)) * 1.2, rng.normal(size=(1, V)) * 1.2
    p = np.exp(lt[0]) / np.exp(lt[0]).sum()
    q = np.exp(ld[0]) / np.exp(ld[0]).sum()
    beta = np.minimum(p, q).sum()
    trials = 100_000
    xs = rng.choice(V, size=trials, p=q)
    us = rng.random(trials)
    acc = 0
    for k in range(trials):
        acc += verify_sequence(lt, ld, [xs[k]], [us[k], 0.5], 1.0).n == 1
    sig = np.sqrt(beta * (1 - beta) / trials)
    assert abs(acc / trials - beta) < 4.5 * sig


def test_output_law_chi_square():
    """The first emitted token is distributed as p0, and the bonus token (all
    accepted) as p_gamma: chi-square, V = 8, df = 7, p-value > 1e-4
    (velog 2-3, item 3; scaling-book Appendix D: the sampling distribution is
    unchanged)."""
    rng = np.random.default_rng(5)
    V, gamma = 8, 1
    lt, ld = rng.normal(size=(2, V)), rng.normal(size=(1, V)) + rng.normal(size=V) * 0.7
    P = np.array([np.exp(r) / np.exp(r).sum() for r in lt])
    q = np.exp(ld[0]) / np.exp(ld[0]).sum()
    trials = 40_000
    xs = rng.choice(V, size=trials, p=q)
    U = rng.random((trials, 2))
    first = np.zeros(V)
    bonus = np.zeros(V)
    for k in range(trials):
        r = verify_sequence(lt, ld, [xs[k]], U[k], 1.0)
        first[r.tokens[0]] += 1
        if r.n == gamma:
            bonus[r.tokens[-1]] += 1
    for counts, law in ((first, P[0]), (bonus, P[1])):
        chi2 = ((counts - counts.sum() * law) ** 2 / (counts.sum() * law)).sum()
        assert stats.chi2.sf(chi2, V - 1) > 1e-4, (counts, law)


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("T", [1.0, 0.7, 2.5])
def test_equal_distributions_always_accept(T):
    """p = q bitwise => min(1, p/q) = 1 for every drafted token (velog 2-1, case
    q <= p); the bonus token is searchsorted(cumsum p_gamma, u * sum p_gamma)."""
    rng = np.random.default_rng(21)
    gamma, V = 4, 50
    lt = rng.normal(size=(gamma + 1, V)) * 3
    for trial in range(40):
        x = rng.integers(0, V, size=gamma)
        u = rng.random(gamma + 1)
        u[: gamma] = np.maximum(u[: gamma], 0.999999 if trial % 2 else 0.0)
        r = verify_sequence(lt, lt[:gamma], x, u, T)
        assert r.n == gamma and r.tokens[:gamma] == list(x)
        pg = np.exp((lt[gamma] - lt[gamma].max()) / T)
        c = np.cumsum(pg)
        assert r.tokens[gamma] == int(np.searchsorted(c, u[gamma] * c[-1], side="right"))
        np.testing.assert_allclose(r.beta, 1.0, atol=1e-12)
        np.testing.assert_allclose(r.resid, 0.0, atol=1e-12)


def test_disjoint_support_always_rejects():
    """q puts all its mass where p is 0 => every draft is rejected at position 0
    (velog 2-1, case q > p with p(x) = 0) and the residual is p itself (2-2)."""
    rng = np.random.default_rng(31)
    V = 10
    lt = rng.normal(size=(3, V))
    ld = rng.normal(size=(2, V))
    lt[0, 5:] = -np.inf          # p_0 lives on 0..4
    ld[0, :5] = -np.inf          # q_0 lives on 5..9
    p0 = np.exp(lt[0, :5]) / np.exp(lt[0, :5]).sum()
    counts = np.zeros(V)
    for u in _ugrid(10000):
        x0 = 5 + int(u * 5) % 5
        r = verify_sequence(lt, ld, [x0, 1], [0.0, 0.0, u], 1.0)
        assert r.n == 0
        counts[r.tokens[0]] += 1
    assert counts[5:].sum() == 0
    np.testing.assert_allclose(counts[:5] / counts.sum(), p0, atol=1e-4)
    r = verify_sequence(lt, ld, [7, 1], [0.0, 0.0, 0.3], 1.0)
    assert r.beta[0] == 0.0 and r.resid[0] == pytest.approx(1.0, abs=1e-12)


def test_greedy_is_argmax_comparison():
    """T = 0 reduces to the textbook greedy rule with numpy.argmax
    (scaling-book Appendix D, greedy steps 1-3)."""
    rng = np.random.default_rng(41)
    gamma, V = 6, 40
    for trial in range(300):
        lt = np.round(rng.normal(size=(gamma + 1, V)) * 2, 1)   # rounding creates ties
        ld = np.round(rng.normal(size=(gamma, V)) * 2, 1)
        am = np.argmax(lt, axis=1)
        x = np.where(rng.random(gamma) < 0.7, am[:gamma], rng.integers(0, V, size=gamma))
        r = verify_sequence(lt, ld, x, rng.random(gamma + 1), 0.0)
        expect = []
        for i in range(gamma):
            if x[i] == am[i]:
                expect.append(int(x[i]))
            else:
                expect.append(int(am[i]))
                break
        else:
            expect.append(int(am[gamma]))
        assert r.tokens == expect and r.n == len(expect) - 1


def test_greedy_is_zero_temperature_limit():
    """The sampled rule at T -> 0 (well separated logits) gives the greedy result,
    whatever the uniforms: two branches of the oracle agree in the limit."""
    rng = np.random.default_rng(51)
    gamma, V = 5, 30
    for trial in range(200):
        lt = rng.permutation(V)[None, :].repeat(gamma + 1, 0).astype(np.float64)
        for i in range(gamma + 1):
            lt[i] = rng.permutation(V)
        ld = np.array([rng.permutation(V) for _ in range(gamma)], dtype=np.float64)
        x = np.where(rng.random(gamma) < 0.6, np.argmax(lt[:gamma], 1), rng.integers(0, V, gamma))
        u = rng.random(gamma + 1)
        g = verify_sequence(lt, ld, x, u, 0.0)
        s = verify_sequence(lt, ld, x, u, 1e-3)
        assert g.tokens == s.tokens and g.n == s.n


def test_zero_residual_mass_falls_back_to_p():
    """A rejection with max(0, p - q) == 0 in float64 (both distributions one-hot
    at the same token after rounding): the residual is undefined (velog 2-2
    divides by 1 - beta = 0); the oracle samples from p instead."""
    V = 16
    lt = np.full((2, V), -400.0)
    ld = np.full((1, V), -300.0)
    lt[:, 3] = 0.0
    ld[0, 3] = 0.0
    # p(3) = q(3) = 1.0 exactly; p(x) = e^-400 < q(x) = e^-300 elsewhere.
    r = verify_sequence(lt, ld, [9], [0.5, 0.25], 1.0)
    assert r.n == 0 and r.fallback and r.tokens == [3]
    assert r.resid[0] == 0.0


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("seed", range(4))
def test_invariants(seed):
    """beta + Z = 1 and beta = 1 - |p - q|_1 / 2 (velog 2-3, item 2); emitted
    prefix = drafts; a residual token has p > q; n + 1 in [1, gamma + 1]."""
    rng = np.random.default_rng(100 + seed)
    gamma, V = 5, 300
    T = [0.5, 1.0, 1.7, 0.9][seed]
    lt = rng.normal(size=(gamma + 1, V)) * 2
    ld = 0.8 * lt[:gamma] + rng.normal(size=(gamma, V))
    for trial in range(30):
        x = rng.integers(0, V, size=gamma)
        u = rng.random(gamma + 1)
        r = verify_sequence(lt, ld, x, u, T)
        assert 0 <= r.n <= gamma and len(r.tokens) == r.n + 1
        assert r.tokens[: r.n] == list(x[: r.n])
        for i in range(gamma):
            p = np.exp((lt[i] - lt[i].max()) / T); p /= p.sum()
            q = np.exp((ld[i] - ld[i].max()) / T); q /= q.sum()
            assert r.beta[i] + r.resid[i] == pytest.approx(1.0, abs=1e-12)
            assert r.beta[i] == pytest.approx(1 - 0.5 * np.abs(p - q).sum(), abs=1e-12)
        if r.n < gamma and not r.fallback:
            t = r.tokens[-1]
            p = np.exp((lt[r.n] - lt[r.n].max()) / T); p /= p.sum()
            q = np.exp((ld[r.n] - ld[r.n].max()) / T); q /= q.sum()
            assert p[t] > q[t] and t != x[r.n]


def test_softmax_and_argmax_helpers():
    l = np.array([1.0, 3.0, 3.0, -np.inf, 2.0])
    assert argmax_first(l) == 1
    p = softmax_t(l, 1.0)
    assert p[3] == 0.0 and p.sum() == pytest.approx(1.0, abs=1e-15)
    assert p[1] / p[4] == pytest.approx(np.e, rel=1e-14)
    assert softmax_t(l, 0.5)[1] / softmax_t(l, 0.5)[4] == pytest.approx(np.e ** 2, rel=1e-14)


# ---------------------------------------------------------------- invalid data

@pytest.mark.parametrize("case", ["nan_target", "posinf_draft", "all_neginf", "token_high",
                                  "token_neg", "neg_T", "nan_T", "tiny_T", "nan_greedy"])
def test_invalid_sequences(case):
    rng = np.random.default_rng(61)
    gamma, V = 3, 20
    lt = rng.normal(size=(gamma + 1, V))
    ld = rng.normal(size=(gamma, V))
    x = np.array([1, 2, 3])
    T = 1.0
    if case == "nan_target":
        lt[3, 7] = np.nan                      # in the bonus row: still invalid
    elif case == "posinf_draft":
        ld[2, 0] = np.inf
    elif case == "all_neginf":
        lt[1, :] = -np.inf
    elif case == "token_high":
        x[1] = V
    elif case == "token_neg":
        x[0] = -1
    elif case == "neg_T":
        T = -0.5
    elif case == "nan_T":
        T = float("nan")
    elif case == "tiny_T":
        T = 1e-39
    elif case == "nan_greedy":
        T = 0.0
        ld[0, 5] = np.nan
    r = verify_sequence(lt, ld, x, rng.random(gamma + 1), T)
    assert r.n == -1 and r.tokens == []


def test_partial_neginf_rows_are_valid():
    rng = np.random.default_rng(71)
    lt = rng.normal(size=(2, 12))
    ld = rng.normal(size=(1, 12))
    lt[:, :6] = -np.inf
    r = verify_sequence(lt, ld, [2], [0.3, 0.6], 1.0)   # p(2) = 0 -> reject
    assert r.n == 0 and r.tokens[0] >= 6 and r.p_x[0] == 0.0


# ---------------------------------------------------------------- token-only drafts (q = delta_x)

def _p(logits, T=1.0):
    z = np.asarray(logits, dtype=np.float64) / T
    e = np.exp(z - z.max())
    return e / e.sum()


@pytest.mark.parametrize("seed", [10, 11])
def test_token_only_acceptance_measure_is_p_of_x(seed):
    """With q = delta_x, min(1, p(x)/q(x)) = p(x): the accepting u_0 have measure p(x)."""
    rng = np.random.default_rng(seed)
    V = 6
    lt = rng.normal(size=(2, V)) * 1.5
    p = _p(lt[0])
    us = _ugrid(4000)
    for x in range(V):
        acc = np.mean([verify_sequence(lt, None, [x], [u, 0.5], 1.0).n == 1 for u in us])
        assert acc == pytest.approx(p[x], abs=2.5e-4)


def test_token_only_residual_is_p_without_x():
    """After a rejection the sample is p with x removed, renormalised: max(0, p - delta_x)."""
    rng = np.random.default_rng(12)
    V = 5
    lt = rng.normal(size=(2, V)) * 1.5
    p = _p(lt[0])
    x = int(np.argmax(p))
    want = p.copy()
    want[x] = 0.0
    want /= want.sum()
    counts = np.zeros(V)
    for u in _ugrid(10000):
        r = verify_sequence(lt, None, [x], [0.999999, u], 1.0)
        if r.n == 0:
            counts[r.tokens[0]] += 1
    assert counts.sum() == 10000            # u_0 = 0.999999 >= p(x): always rejected
    np.testing.assert_allclose(counts / counts.sum(), want, atol=1e-4)


def test_token_only_diagnostics_closed_form():
    """q(x) = 1, beta = sum min(p, delta_x) = p(x), Z = sum max(0, p - delta_x) = 1 - p(x)."""
    rng = np.random.default_rng(13)
    lt = rng.normal(size=(4, 40)) * 2.0
    toks = [3, 17, 39]
    r = verify_sequence(lt, None, toks, [0.3, 0.2, 0.9, 0.5], 0.8)
    p = [_p(lt[i], 0.8) for i in range(3)]
    for i, x in enumerate(toks):
        assert r.q_x[i] == 1.0
        assert r.p_x[i] == pytest.approx(p[i][x], rel=1e-12)
        assert r.beta[i] == pytest.approx(p[i][x], rel=1e-12)
        assert r.resid[i] == pytest.approx(1.0 - p[i][x], rel=1e-12)


@pytest.mark.parametrize("T", [1.0, 0.0])
def test_token_only_equals_point_mass_draft_logits(T):
    """A token-only draft is the draft whose logits are 0 at x and -inf elsewhere
    (its softmax is exactly delta_x): the two give identical results."""
    rng = np.random.default_rng(14)
    V, g = 30, 4
    for _ in range(40):
        lt = rng.normal(size=(g + 1, V)) * 2.0
        toks = rng.integers(0, V, size=g)
        ld = np.full((g, V), -np.inf)
        ld[np.arange(g), toks] = 0.0
        u = rng.random(g + 1)
        a = verify_sequence(lt, None, toks, u, T)
        b = verify_sequence(lt, ld, toks, u, T)
        assert (a.n, a.tokens) == (b.n, b.tokens)
        for k in ("p_x", "q_x", "beta", "resid"):
            np.testing.assert_allclose(getattr(a, k), getattr(b, k), rtol=1e-12, atol=1e-15)


def test_token_only_output_law_is_p():
    """Whatever token-only drafter proposes x_0 (law r), the first emitted token
    has law p_0: enumeration of x_0, with the acceptance measured on a u_0 grid
    and the residual law on a u_1 grid (velog 2-3, item 3: P(x = x') = p(x'))."""
    rng = np.random.default_rng(15)
    V = 4
    lt = rng.normal(size=(2, V))
    P0 = _p(lt[0])
    r = np.array([0.5, 0.1, 0.3, 0.1])     # any drafter's law over x_0
    us = _ugrid(4000)
    first = np.zeros(V)
    for x0 in range(V):
        acc = np.mean([verify_sequence(lt, None, [x0], [u, 0.5], 1.0).n == 1 for u in us])
        law = np.zeros(V)
        for u in us:
            res = verify_sequence(lt, None, [x0], [0.999999, u], 1.0)
            assert res.n == 0
            law[res.tokens[0]] += 1.0 / len(us)
        first[x0] += r[x0] * acc
        first += r[x0] * (1.0 - acc) * law
    np.testing.assert_allclose(first, P0, atol=1e-3)


def test_token_only_greedy_is_argmax_comparison():
    lt = np.array([[0.0, 3.0, 1.0], [2.0, 0.0, 0.0], [0.0, 0.0, 5.0]])
    r = verify_sequence(lt, None, [1, 2], [0.5, 0.5, 0.5], 0.0)
    assert r.n == 1 and r.tokens == [1, 0]                 # argmax of row 1 is 0, not 2
    assert r.q_x.tolist() == [1.0, 1.0]
    assert r.beta.tolist() == [1.0, 0.0] and r.resid.tolist() == [0.0, 1.0]
