"""The parity harness itself, on the CPU: fabricated GPU outputs are accepted
or rejected by compare() exactly as its rules say.

The batch (V = 4, float32 logits 0 and -inf, so every probability is an
exact fraction) has one sequence whose final uniform sits 3e-8 below a CDF
edge and one whose acceptance uniform sits 2e-7 above its ratio r = 1/2.
"""
import dataclasses

import numpy as np

from rejection_sampling_verifier_specverify_amd.workloads import make_custom

from parity import compare

NINF = -np.inf


def _batch():
    # seq 0 (gamma 1): p0 = (1/4,1/4,1/4,1/4), q0 = (1,0,0,0), x0 = 0: r = 1/4,
    #   u0 = 0.1 accepts far from r; bonus p1 = (1/4,...): u1 just below the
    #   edge 1/2 between tokens 1 and 2 -> token 1 (neighbour across: 2).
    # seq 1 (gamma 2): p0 uniform, q0 = (1/2,1/2,0,0), x0 = 0: r = 1/2,
    #   u0 = 0.5 + 2e-7 rejects next to r; residual max(0, p0 - q0) =
    #   (0,0,1/4,1/4), u2 = 0.3 -> token 2 (far from its edges).  Had x0
    #   been accepted: p1 uniform, q1 = (0,0,0,1), x1 = 3, r = 1/4, u1 =
    #   0.9 rejects; residual (1/4,1/4,1/4,0) with u2 = 0.3 -> token 0.
    # seq 2 (gamma 1): q0 = (1,0,0,0), x0 = 0, r = 1/4 with u0 = 0.7: a
    #   rejection far from its switching point; residual (0,1/4,1/4,1/4),
    #   u1 = 0.6 -> token 2.
    z, n = 0.0, NINF
    tgt = [[z, z, z, z], [z, z, z, z],
           [z, z, z, z], [z, z, z, z], [z, z, z, z],
           [z, z, z, z], [z, z, z, z]]
    drf = [[z, n, n, n],
           [z, z, n, n], [n, n, n, z],
           [z, n, n, n]]
    u = np.array([0.1, 0.5, 0.5, 0.9, 0.3, 0.7, 0.6], dtype=np.float32)
    u[1] = np.nextafter(np.float32(0.5), np.float32(0.0))   # 3e-8 below the edge 1/2
    u[2] = np.float32(0.5) + np.float32(2 ** -22)           # 2.4e-7 above r = 1/2
    return make_custom(np.array(tgt), np.array(drf), [0, 0, 3, 0], u, [1.0, 1.0, 1.0], [1, 2, 1])


def _got(acc, toks):
    return {"accepted_len": np.array(acc, np.int32), "out_tokens": np.array(toks, np.int32)}


# the oracle's outputs of _batch(): seq 0 [0, 1]; seq 1 n = 0, [2, -1, -1]; seq 2 n = 0, [2, -1]
RIGHT = ([1, 0, 0], [0, 1, 2, -1, -1, 2, -1])


def test_exact_outputs_pass_and_boundaries_are_counted():
    rep = compare(_batch(), _got(*RIGHT), check_diag=False)
    assert rep.ok(), rep.summary()
    assert rep.checked == 3 and rep.exact == 3
    assert rep.boundary == 2 and rep.boundary_mismatch == 0


def test_neighbour_across_the_near_edge_is_accepted():
    acc, toks = RIGHT
    toks = list(toks)
    toks[1] = 2                                  # seq 0's bonus: the token across the edge 1/2
    rep = compare(_batch(), _got(acc, toks), check_diag=False)
    assert rep.ok(), rep.summary()
    assert rep.boundary_mismatch == 1 and rep.exact == 2


def test_far_token_at_a_boundary_is_rejected():
    acc, toks = RIGHT
    toks = list(toks)
    toks[1] = 3                                  # two intervals away from u
    rep = compare(_batch(), _got(acc, toks), check_diag=False)
    assert not rep.ok() and "final token 3" in rep.mismatches[0]


def test_wrong_prefix_is_rejected():
    acc, toks = RIGHT
    toks = list(toks)
    toks[0] = 1                                  # seq 0 accepted x0 = 0, not 1
    rep = compare(_batch(), _got(acc, toks), check_diag=False)
    assert not rep.ok() and "prefix" in rep.mismatches[0]


def test_flip_next_to_the_ratio_is_accepted_with_its_own_final_token():
    acc, toks = RIGHT
    acc, toks = list(acc), list(toks)
    # seq 1 accepts x0 (u0 is 2.4e-7 above r): it then rejects x1 and samples
    # the residual of position 1 with u2 = 0.3 -> token 0
    acc[1] = 1
    toks[2:5] = [0, 0, -1]
    rep = compare(_batch(), _got(acc, toks), check_diag=False)
    assert rep.ok(), rep.summary()
    assert rep.acc_flips == 1 and rep.boundary_mismatch == 1
    toks[3] = 1                                  # the residual of position 1 gives 0, not 1
    rep = compare(_batch(), _got(acc, toks), check_diag=False)
    assert not rep.ok() and "final token 1" in rep.mismatches[0]


def test_flip_far_from_the_ratio_is_rejected():
    acc, toks = RIGHT
    acc, toks = list(acc), list(toks)
    acc[2] = 1                                   # seq 2 rejected with u0 = 0.7, r = 1/4
    toks[5:7] = [0, 1]
    rep = compare(_batch(), _got(acc, toks), check_diag=False)
    assert not rep.ok() and "decision at 0 differs" in rep.mismatches[0]


def test_malformed_outputs_are_rejected():
    for acc, toks in (([1, 3, 0], RIGHT[1]),                       # n beyond gamma
                      (RIGHT[0], [0, 1, 2, 7, -1, 2, -1]),         # a token after n
                      (RIGHT[0], [0, 1, 2, -1, -1, 4, -1])):       # token outside [0, V)
        rep = compare(_batch(), _got(acc, toks), check_diag=False)
        assert not rep.ok(), (acc, toks)


def test_invalid_and_greedy_sequences_must_match_exactly():
    inp = _batch()
    bad = dataclasses.replace(inp, uniforms=inp.uniforms.copy())
    bad.uniforms[5] = np.float32(1.0)            # seq 2's uniform outside [0, 1): invalid data
    rep = compare(bad, _got([1, 0, -1], [0, 1, 2, -1, -1, -1, -1]), check_diag=False)
    assert rep.ok() and rep.invalid == 1, rep.summary()
    rep = compare(bad, _got(*RIGHT), check_diag=False)
    assert not rep.ok()
    greedy = dataclasses.replace(inp, temperatures=np.zeros(3, np.float32))
    # T = 0: argmax ties go to the lowest id, 0 in every row: x0 = 0 is
    # accepted everywhere, seq 1's x1 = 3 is replaced by 0
    rep = compare(greedy, _got([1, 1, 1], [0, 0, 0, 0, -1, 0, 0]), check_diag=False)
    assert rep.ok() and rep.greedy == 3, rep.summary()
    rep = compare(greedy, _got([1, 1, 1], [0, 1, 0, 0, -1, 0, 0]), check_diag=False)
    assert not rep.ok()
