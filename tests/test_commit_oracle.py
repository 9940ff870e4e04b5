"""Pins of the commit oracle (oracle/commit_oracle.py) against a worked
example written out by hand and against the invariants of an append."""
import json
import os

import numpy as np

from oracle import commit_reference


def test_commit_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "commit_worked_example.json")))
    toks, lens, app, nxt = commit_reference(np.array(g["accepted_len"]), np.array(g["out_tokens"]),
                                            np.array(g["cu_draft"]), np.array(g["seq_tokens"]),
                                            np.array(g["seq_lens"]), g["capacity"])
    assert toks.tolist() == g["expect_seq_tokens"]
    assert lens.tolist() == g["expect_seq_lens"]
    assert app.tolist() == g["expect_appended"]
    assert nxt.tolist() == g["expect_next_token"]


def _random_case(rng, B, cap):
    gam = rng.integers(0, 6, size=B)
    cu = np.concatenate([[0], np.cumsum(gam)]).astype(np.int64)
    R_t = int(cu[-1]) + B
    acc = np.array([rng.integers(-1, g + 1) for g in gam], dtype=np.int64)
    out = np.full(R_t, -1, dtype=np.int64)
    for b in range(B):
        t0 = int(cu[b]) + b
        if acc[b] >= 0:
            out[t0:t0 + acc[b] + 1] = rng.integers(0, 50000, size=acc[b] + 1)
    toks = rng.integers(0, 50000, size=(B, cap)).astype(np.int32)
    lens = rng.integers(0, cap + 1, size=B).astype(np.int32)
    return gam, cu, acc, out, toks, lens


def test_commit_invariants_random():
    rng = np.random.default_rng(7)
    cap = 12
    for _ in range(50):
        B = int(rng.integers(1, 9))
        gam, cu, acc, out, toks, lens = _random_case(rng, B, cap)
        t2, l2, app, nxt = commit_reference(acc, out, cu, toks, lens, cap)
        assert toks.shape == t2.shape
        for b in range(B):
            t0 = int(cu[b]) + b
            if acc[b] < 0:
                assert app[b] == 0 and nxt[b] == -1 and l2[b] == lens[b]
                assert np.array_equal(t2[b], toks[b])
            elif lens[b] + acc[b] + 1 > cap:
                assert app[b] == -1 and nxt[b] == -1 and l2[b] == lens[b]
                assert np.array_equal(t2[b], toks[b])
            else:
                k = acc[b] + 1
                L = lens[b]
                assert app[b] == k and l2[b] == L + k
                assert np.array_equal(t2[b, :L], toks[b, :L])            # prefix kept
                assert np.array_equal(t2[b, L:L + k], out[t0:t0 + k])     # the emitted tokens, in order
                assert np.array_equal(t2[b, L + k:], toks[b, L + k:])     # tail kept
                assert nxt[b] == out[t0 + acc[b]]                         # the target's token
        # inputs are not modified
        assert t2 is not toks and l2 is not lens


def test_commit_rejects_length_beyond_gamma_and_negative_length():
    cu = np.array([0, 2])
    out = np.array([5, 6, 7])
    toks = np.zeros((1, 8), dtype=np.int32)
    # n = 3 > gamma = 2: not a verification result of this layout
    t2, l2, app, nxt = commit_reference(np.array([3]), out, cu, toks, np.array([0]), 8)
    assert app.tolist() == [0] and nxt.tolist() == [-1] and l2.tolist() == [0] and not t2.any()
    # a negative committed length never fits
    t2, l2, app, nxt = commit_reference(np.array([1]), out, cu, toks, np.array([-1]), 8)
    assert app.tolist() == [-1] and l2.tolist() == [-1] and not t2.any()
    # exactly full: fits
    t2, l2, app, nxt = commit_reference(np.array([2]), out, cu, toks, np.array([5]), 8)
    assert app.tolist() == [3] and l2.tolist() == [8] and t2[0, 5:].tolist() == [5, 6, 7] and nxt.tolist() == [7]
