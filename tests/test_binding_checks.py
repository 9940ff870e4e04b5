"""The binding's argument checks, on the CPU (CPU tensors stand in for device
ones: the checks compare each tensor's device with the handle's).  The C
library reads raw memory, so a wrong dtype, a short tensor or a strided one
must be refused before any pointer is passed on."""
import pytest
import torch

from rejection_sampling_verifier_specverify_amd.binding import check_commit_args, check_run_args

DEV = torch.device("cpu")
V = 100


def _args(B=3, **over):
    gamma = 2   # shapes below; a ragged call passes gamma=None with cu_draft
    R_d, R_t = B * gamma, B * (gamma + 1)
    a = dict(vocab=V, logits_dtype=torch.bfloat16, device=DEV,
             target=torch.zeros(R_t, V, dtype=torch.bfloat16), draft=torch.zeros(R_d, V, dtype=torch.bfloat16),
             draft_tokens=torch.zeros(R_d, dtype=torch.int32), uniforms=torch.zeros(R_t),
             temperatures=torch.ones(B), accepted_len=torch.zeros(B, dtype=torch.int32),
             out_tokens=torch.zeros(R_t, dtype=torch.int32), gamma=gamma,
             diagnostics=(("beta", torch.zeros(R_d)), ("p_draft", None)))
    a.update(over)
    return a


def test_good_arguments_pass():
    assert check_run_args(**_args()) == (3, 6, 9)
    # token-only drafts: no draft logits
    assert check_run_args(**_args(draft=None)) == (3, 6, 9)
    # ragged: cu_draft int32 [B+1] and the host copy of cu_draft[B]
    assert check_run_args(**_args(gamma=None, cu_draft=torch.tensor([0, 2, 4, 6], dtype=torch.int32),
                                  num_draft_rows=6)) == (3, 6, 9)
    # padded rows (stride > V) and extra rows are fine
    pad = torch.zeros(9, V + 28, dtype=torch.bfloat16)[:, :V]
    assert check_run_args(**_args(target=pad)) == (3, 6, 9)


@pytest.mark.parametrize("field,bad,exc", [
    ("draft_tokens", torch.zeros(6, dtype=torch.int64), TypeError),       # torch's default integer type
    ("temperatures", torch.ones(3, dtype=torch.float64), TypeError),
    ("uniforms", torch.zeros(9, dtype=torch.float16), TypeError),
    ("accepted_len", torch.zeros(3), TypeError),
    ("out_tokens", torch.zeros(8, dtype=torch.int32), ValueError),          # one short
    ("uniforms", torch.zeros(18)[::2], ValueError),                         # strided
    ("target", torch.zeros(8, V, dtype=torch.bfloat16), ValueError),        # too few rows
    ("draft", torch.zeros(6, V - 1, dtype=torch.bfloat16), ValueError),     # rows shorter than V
    ("target", torch.zeros(9, V, dtype=torch.float32), TypeError),          # wrong logits dtype
    ("target", torch.zeros(V, 9, dtype=torch.bfloat16).t(), ValueError),   # column-major
    ("diagnostics", (("beta", torch.zeros(5)),), ValueError),
    ("diagnostics", (("q_draft", torch.zeros(6, dtype=torch.float64)),), TypeError),
])
def test_bad_arguments_are_refused(field, bad, exc):
    with pytest.raises(exc):
        check_run_args(**_args(**{field: bad}))


def test_ragged_needs_its_row_count_and_int32_offsets():
    with pytest.raises(ValueError):
        check_run_args(**_args(gamma=None, cu_draft=torch.tensor([0, 2, 4, 6], dtype=torch.int32)))
    with pytest.raises(TypeError):
        check_run_args(**_args(gamma=None, cu_draft=torch.tensor([0, 2, 4, 6]), num_draft_rows=6))
    with pytest.raises(ValueError):
        check_run_args(**_args(gamma=None, cu_draft=torch.tensor([0, 2, 4], dtype=torch.int32), num_draft_rows=6))


def test_wrong_device_is_refused():
    meta = torch.zeros(6, dtype=torch.int32, device="meta")
    with pytest.raises(ValueError, match="must be on"):
        check_run_args(**_args(draft_tokens=meta))


def test_commit_checks():
    i32 = lambda *s: torch.zeros(*s, dtype=torch.int32)
    ok = dict(device=DEV, accepted_len=i32(3), out_tokens=i32(9), seq_tokens=i32(3, 20), seq_lens=i32(3), gamma=2)
    assert check_commit_args(**ok) == (3, 9)
    for field, bad in (("out_tokens", i32(8)), ("seq_lens", torch.zeros(3, dtype=torch.int64)),
                       ("seq_tokens", i32(2, 20)), ("seq_tokens", i32(20, 3).t()), ("appended", i32(2))):
        with pytest.raises((TypeError, ValueError)):
            check_commit_args(**dict(ok, **{field: bad}))


def _tree_args(**over):
    from rejection_sampling_verifier_specverify_amd.binding import check_tree_args  # noqa: F401
    B, N = 2, 5
    R_t = N + B
    a = dict(vocab=V, logits_dtype=torch.float32, device=DEV, target=torch.zeros(R_t, V),
             cu_nodes=torch.tensor([0, 3, 5], dtype=torch.int32), num_nodes=N,
             parents=torch.zeros(N, dtype=torch.int32), tokens=torch.zeros(N, dtype=torch.int32),
             uniforms=torch.zeros(R_t), temperatures=torch.ones(B), accepted_len=torch.zeros(B, dtype=torch.int32),
             out_tokens=torch.zeros(R_t, dtype=torch.int32), out_nodes=torch.zeros(R_t, dtype=torch.int32),
             p_cand=None)
    a.update(over)
    return a


def test_tree_arguments():
    from rejection_sampling_verifier_specverify_amd.binding import check_tree_args
    assert check_tree_args(**_tree_args()) == (2, 5, 7)
    assert check_tree_args(**_tree_args(out_nodes=None, p_cand=torch.zeros(5))) == (2, 5, 7)
    bad = [dict(parents=torch.zeros(4, dtype=torch.int32)),          # short
           dict(tokens=torch.zeros(5, dtype=torch.int64)),           # wrong dtype
           dict(cu_nodes=None),                                      # missing
           dict(target=torch.zeros(6, V)),                           # too few rows
           dict(target=torch.zeros(7, V, dtype=torch.bfloat16)),     # wrong logits dtype
           dict(out_nodes=torch.zeros(6, dtype=torch.int32)),        # short optional output
           dict(p_cand=torch.zeros(5, dtype=torch.float64)),
           dict(num_nodes=-1)]
    for over in bad:
        with pytest.raises((TypeError, ValueError)):
            check_tree_args(**_tree_args(**over))
