"""The seeded input generator: reproducibility, layout, rounding, drafter law."""
import numpy as np
import pytest
from scipy import stats

from rejection_sampling_verifier_specverify_amd.workloads import (
    WORKLOADS, HEADLINE, bf16_bits_to_f32, drafter_token, f32_to_bf16_bits, make_inputs)


def test_bf16_round_to_nearest_even_table():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)            # bf16 spacing at 1.0
    cases = {
        float(one): 0x3F80,
        float(one + ulp / 2): 0x3F80,            # tie -> even (down)
        float(one + ulp + ulp / 2): 0x3F82,      # tie -> even (up)
        float(one + ulp / 2 + 2.0 ** -20): 0x3F81,
        float(-one - ulp / 4): 0xBF80,
        float("inf"): 0x7F80,
        float("-inf"): 0xFF80,
        0.0: 0x0000,
    }
    got = f32_to_bf16_bits(np.array(list(cases), dtype=np.float32))
    assert [int(v) for v in got] == list(cases.values())
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]
    x = np.random.default_rng(0).normal(size=10000).astype(np.float32) * 100
    back = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_layout_and_reproducibility(name):
    w = WORKLOADS[name]
    a = make_inputs(w, seed=0, batch=3)
    b = make_inputs(w, seed=0, batch=3)
    c = make_inputs(w, seed=1, batch=3)
    B = 3
    assert a.cu_draft.shape == (B + 1,) and a.cu_draft[0] == 0
    g = np.diff(a.cu_draft)
    if w.ragged:
        assert g.min() >= w.gamma[0] and g.max() <= w.gamma[1]
    else:
        assert np.all(g == w.gamma)
    R_d = int(a.cu_draft[-1])
    assert a.target.shape == (R_d + B, w.vocab) and a.draft.shape == (R_d, w.vocab)
    assert a.target.dtype == (np.float32 if w.dtype == "f32" else np.uint16)
    assert a.draft_tokens.shape == (R_d,) and a.uniforms.shape == (R_d + B,)
    assert np.all((a.draft_tokens >= 0) & (a.draft_tokens < w.vocab))
    assert np.all((a.uniforms >= 0) & (a.uniforms < 1)) and a.uniforms.dtype == np.float32
    for k in ("target", "draft", "draft_tokens", "uniforms", "temperatures", "cu_draft"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert not np.array_equal(a.target, c.target)
    # the first batch rows do not depend on the batch size (per-row streams)
    if not w.ragged:
        d = make_inputs(w, seed=0, batch=2)
        assert np.array_equal(d.target, a.target[: d.target.shape[0]])


def test_target_value_distribution_headline():
    a = make_inputs(HEADLINE, seed=0, batch=2)
    t = bf16_bits_to_f32(a.target).astype(np.float64)
    assert abs(t.std() - 3.0) < 0.02 and abs(t.mean()) < 0.02
    d = bf16_bits_to_f32(a.draft).astype(np.float64)
    pair = np.concatenate([np.arange(a.cu_draft[b], a.cu_draft[b + 1]) + b for b in range(a.batch)])
    resid = d - 0.8 * t[pair]
    assert abs(resid.std() - 1.5) < 0.02
    assert np.all(a.temperatures == np.float32(0.7))


def test_mixed_temperatures_and_ragged():
    a = make_inputs("b256_g8_v128256_bf16_mixedT", seed=0, batch=24)
    assert set(np.unique(a.temperatures).tolist()) <= {0.0, np.float32(0.6), 1.0}
    assert (a.temperatures == 0).any()
    r = make_inputs("b512_gragged1to7_v152064_bf16", seed=0, batch=40)
    g = np.diff(r.cu_draft)
    assert len(set(g.tolist())) > 3


def test_drafter_token_law():
    """Gumbel-max draws follow softmax(l/T): chi-square on 8 tokens."""
    rng = np.random.default_rng(3)
    l = rng.normal(size=8)
    T = 0.7
    p = np.exp(l / T) / np.exp(l / T).sum()
    g = np.random.Generator(np.random.Philox(5))
    counts = np.bincount([drafter_token(l, T, g) for _ in range(20000)], minlength=8)
    chi2 = ((counts - 20000 * p) ** 2 / (20000 * p)).sum()
    assert stats.chi2.sf(chi2, 7) > 1e-4
    assert drafter_token(l, 0.0, g) == int(np.argmax(l))
