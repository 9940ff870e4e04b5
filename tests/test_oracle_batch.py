"""Pins of the oracle's packed-batch layer, its bf16 decoding, its uniform
contract and its per-position alternatives.

The packed layout (verify_batch, sequence_rows) is pinned by a batch worked
by hand (tests/golden/packed_batch_worked_example.json), whose uniforms and
rows are chosen so that an off-by-one in the uniform index or in the output
position changes the result.  decode_logits is pinned by bf16 bit patterns
whose values follow from the format's definition (sign, 8-bit exponent with
bias 127, 7-bit fraction: the upper half of an IEEE binary32).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (cdf_interval, decode_logits, final_weights, inverse_cdf, sequence_rows,
                    verify_batch, verify_sequence)


def _golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "packed_batch_worked_example.json")))


def _rows(rows):
    return np.array([[-np.inf if v == "-inf" else float(v) for v in r] for r in rows])


def _bf16(rows, table):
    key = lambda v: "-inf" if v == "-inf" else str(int(v))
    return np.array([[int(table[key(v)], 16) for v in r] for r in rows], dtype=np.uint16)


def _expect(g, name):
    return np.array([np.nan if v is None else v for v in g[name]], dtype=np.float64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_packed_batch_worked_example(golden_dir, dtype):
    g = _golden(golden_dir)
    if dtype == "f32":
        tgt = _rows(g["target"]).astype(np.float32)
        drf = _rows(g["draft"]).astype(np.float32)
    else:
        tgt = _bf16(g["target"], g["bf16_bits"])
        drf = _bf16(g["draft"], g["bf16_bits"])
    acc, out, p_x, q_x, beta, resid, res = verify_batch(
        tgt, drf, np.array(g["draft_tokens"], np.int32), np.array(g["uniforms"], np.float32),
        np.array(g["temperatures"], np.float32), np.array(g["cu_draft"], np.int32), dtype)
    assert acc.tolist() == g["expect_accepted_len"]
    assert out.tolist() == g["expect_out_tokens"]
    for name, got in (("expect_p_x", p_x), ("expect_q_x", q_x), ("expect_beta", beta),
                      ("expect_resid", resid)):
        np.testing.assert_allclose(got, _expect(g, name), rtol=0, atol=1e-15, equal_nan=True, err_msg=name)


def test_packed_batch_subset_keeps_fill_values(golden_dir):
    g = _golden(golden_dir)
    acc, out, p_x, q_x, beta, resid, res = verify_batch(
        _rows(g["target"]).astype(np.float32), _rows(g["draft"]).astype(np.float32),
        np.array(g["draft_tokens"], np.int32), np.array(g["uniforms"], np.float32),
        np.array(g["temperatures"], np.float32), np.array(g["cu_draft"], np.int32), "f32",
        sequences=g["subset"])
    assert acc.tolist() == g["expect_subset_accepted_len"]
    assert out.tolist() == g["expect_subset_out_tokens"]
    assert sorted(res) == g["subset"]
    # only the draft row of sequence 3 (row 3) was verified
    assert np.isnan(p_x[[0, 1, 2, 4]]).all() and p_x[3] == 1.0 and resid[3] == 1.0


def test_sequence_rows_of_the_worked_batch(golden_dir):
    """Sequence 2 of the golden batch: target rows 4-5, draft row 2, uniforms 4-5."""
    g = _golden(golden_dir)
    tgt = _rows(g["target"]).astype(np.float32)
    drf = _rows(g["draft"]).astype(np.float32)
    t, d, x, u = sequence_rows(tgt, drf, np.array(g["draft_tokens"]), np.array(g["uniforms"], np.float32),
                               np.array(g["cu_draft"]), "f32", 2)
    assert np.array_equal(t, _rows(g["target"])[4:6]) and np.array_equal(d, _rows(g["draft"])[2:3])
    assert x.tolist() == [0] and u.tolist() == [np.float32(0.2), np.float32(0.75)]
    t, d, x, u = sequence_rows(tgt, drf, np.array(g["draft_tokens"]), np.array(g["uniforms"], np.float32),
                               np.array(g["cu_draft"]), "f32", 1)
    assert t.shape == (1, 4) and d.shape == (0, 4) and x.size == 0 and u.tolist() == [np.float32(0.2)]


def _bf16_value(bits: int) -> float:
    """The value a bf16 bit pattern stands for, from the format's fields."""
    s = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return s * math.inf if m == 0 else math.nan
    if e == 0:
        return s * math.ldexp(m / 128.0, -126)
    return s * math.ldexp(1.0 + m / 128.0, e - 127)


def test_decode_logits_bf16_table():
    table = {0x3F80: 1.0, 0xC000: -2.0, 0x7F80: math.inf, 0xFF80: -math.inf, 0x0000: 0.0,
             0x4049: 3.140625, 0x3F81: 1.0078125, 0xBF80: -1.0, 0x4040: 3.0,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126, 0x7F7F: 3.3895313892515355e38}
    bits = np.array(list(table), dtype=np.uint16)
    got = decode_logits(bits, "bf16")
    assert got.dtype == np.float64
    for b, v, g in zip(table, table.values(), got):
        assert g == v, hex(b)
        assert g == _bf16_value(b), hex(b)
    nan = decode_logits(np.array([0x7FC0, 0xFFC1], np.uint16), "bf16")
    assert np.isnan(nan).all()
    negz = decode_logits(np.array([0x8000], np.uint16), "bf16")[0]
    assert negz == 0.0 and math.copysign(1.0, negz) == -1.0
    # every finite pattern of one exponent, from the format's fields
    sweep = np.arange(0x3F00, 0x4100, dtype=np.uint32).astype(np.uint16)
    assert [float(v) for v in decode_logits(sweep, "bf16")] == [_bf16_value(int(b)) for b in sweep]
    # 2-D rows keep their shape; float32 rows are widened exactly
    assert decode_logits(bits.reshape(3, 4), "bf16").shape == (3, 4)
    f = np.array([[1.5, -0.1, np.float32(1e-40)]], np.float32)
    assert decode_logits(f, "f32").tolist() == [[1.5, float(np.float32(-0.1)), float(np.float32(1e-40))]]


@pytest.mark.parametrize("bad", [1.0, 1.5, -1e-7, float("nan"), float("inf")])
@pytest.mark.parametrize("where", [0, 2])
def test_uniform_outside_unit_interval_is_invalid(bad, where):
    """Uniforms are draws from [0, 1) (velog page, section 2 step 3: rejection
    with probability 1 - p/q needs u uniform on the unit interval); a value
    outside, or NaN, makes the sequence invalid data, also for greedy rows."""
    rng = np.random.default_rng(3)
    lt, ld = rng.normal(size=(3, 7)), rng.normal(size=(2, 7))
    u = [0.3, 0.4, 0.5]
    u[where] = bad
    for T in (1.0, 0.0):
        r = verify_sequence(lt, ld, [1, 2], u, T)
        assert r.n == -1 and r.tokens == []
    for edge in (0.0, float(np.nextafter(np.float32(1.0), np.float32(0.0)))):
        u[where] = edge
        assert verify_sequence(lt, ld, [1, 2], u, 1.0).n >= 0


def test_cdf_interval_three_tokens(golden_dir):
    """The '샘플링이란' example: intervals [0, .6), [.6, .9), [.9, 1) in token order."""
    g = json.load(open(os.path.join(golden_dir, "sampling_three_tokens.json")))
    p = np.array(g["probabilities"])
    ivs = [cdf_interval(p, t) for t in range(3)]
    np.testing.assert_allclose(ivs, [(0.0, 0.6), (0.6, 0.9), (0.9, 1.0)], atol=1e-15)
    for t, (lo, hi) in enumerate(ivs):
        assert inverse_cdf(p, (lo + hi) / 2)[0] == t


def test_final_weights_cases():
    p = np.array([0.5, 0.3, 0.2])
    q = np.array([0.2, 0.3, 0.5])
    w, fb = final_weights(p, None)                 # bonus: p itself
    assert w is p and not fb
    w, fb = final_weights(p, q)                    # residual: (0.3, 0, 0)
    np.testing.assert_allclose(w, [0.3, 0.0, 0.0], atol=1e-15)
    assert not fb
    w, fb = final_weights(p, p.copy())             # Z = 0: fall back to p
    assert fb and w is p


@pytest.mark.parametrize("seed", range(6))
def test_alternatives_are_the_paths_forced_by_the_uniforms(seed):
    """alt_tokens[j] is the final token the oracle emits when the first
    rejection is at j, and accept[i] is the decision at i when i is reached:
    both checked by forcing the path with the uniforms (u = 0 accepts any
    positive ratio; the largest float below 1 rejects any ratio below 1)."""
    rng = np.random.default_rng(200 + seed)
    gamma, V = 4, 60
    T = [0.7, 1.0, 1.4][seed % 3]
    lt = rng.normal(size=(gamma + 1, V)) * 1.5
    ld = lt[:gamma] + rng.normal(size=(gamma, V))
    tok_only = seed >= 4
    x = rng.integers(0, V, size=gamma)
    u = rng.random(gamma + 1)
    base = verify_sequence(lt, None if tok_only else ld, x, u, T)
    assert base.alt_tokens[base.n] == base.tokens[-1]
    below1 = float(np.nextafter(1.0, 0.0))
    for j in range(gamma + 1):
        if j < gamma and base.ratio[j] >= 1.0:
            continue
        uf = u.copy()
        uf[:j] = 0.0
        if j < gamma:
            uf[j] = below1
        r = verify_sequence(lt, None if tok_only else ld, x, uf, T)
        assert r.n == j and r.tokens[-1] == base.alt_tokens[j], j
        assert r.alt_tokens == base.alt_tokens
        if j < gamma and base.ratio[j] > 0.0:
            # reaching j with the original u_j decides exactly as accept[j]
            uf2 = u.copy()
            uf2[:j] = 0.0
            reached = verify_sequence(lt, None if tok_only else ld, x, uf2, T)
            assert (reached.n > j) == bool(base.accept[j]), j


def test_acceptance_margin_counts_ratios_at_or_above_one():
    """A ratio just above 1 with u just below 1 is a decision next to its
    switching point: its margin |u - r| is reported (no infinite margin for
    r >= 1)."""
    p = np.array([0.5, 0.5])
    q = np.array([0.5 - 1e-7, 0.5 + 1e-7])
    lt, ld = np.log(p)[None].repeat(2, 0), np.log(q)[None]
    r = verify_sequence(lt, ld, [0], [0.999999, 0.5], 1.0)
    assert r.n == 1 and r.ratio[0] > 1.0
    assert r.acc_margin_all[0] == pytest.approx(r.ratio[0] - 0.999999, abs=1e-12)
    assert r.acc_margin[0] < 1e-5
