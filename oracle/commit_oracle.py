"""Oracle of the on-device commit that follows a verification run.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the HIP path.

What it computes.  Perplexity "Accelerating Sonar through speculation",
section "단일 토큰에 대한 MTP 스케줄링": after the drafts are verified, a small
amount of extra GPU work avoids a GPU-to-CPU synchronisation.  The target's
input tokens are shifted, and a kernel inserts the next target token at the
position that follows them.  Section "추측적 디코딩을 통한 추론" of the same page
names the reason: the number of accepted tokens fixes the next run's
sequence lengths, which otherwise forces that synchronisation.

Reading (the page gives no layout, so the plainest one is taken).  Each
sequence b keeps its committed tokens in row b of a device buffer,
``seq_tokens[b, 0:seq_lens[b]]``.  A verification emits n_b + 1 tokens:
x_0 .. x_{n_b - 1}, then the target's token t_b (the residual or bonus
sample).  The commit
  * appends those n_b + 1 tokens at ``seq_lens[b]``;
  * advances ``seq_lens[b]`` by n_b + 1;
  * reports ``next_token[b] = t_b``, the token that starts sequence b's next
    step;
  * reports ``appended[b]`` = n_b + 1.
A sequence is left untouched, with ``appended[b] = 0`` and
``next_token[b] = -1``, when its verification reported it invalid
(n_b < 0) or the layout does not allow n_b (n_b > gamma_b).  A sequence
whose tokens would not fit in its row (``seq_lens[b] + n_b + 1 >
capacity``, or a negative length) is also left untouched, with
``appended[b] = -1`` and ``next_token[b] = -1``.

Parity pins (``tests/test_commit_oracle.py``): a worked example written out
by hand (``tests/golden/commit_worked_example.json``), the invariants of an
append (prefix and tail of each row unchanged, appended tokens equal to the
run's emitted tokens in order), and each refusal case.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

__all__ = ["commit_reference"]


def commit_reference(accepted_len: np.ndarray, out_tokens: np.ndarray, cu_draft: np.ndarray,
                     seq_tokens: np.ndarray, seq_lens: np.ndarray,
                     capacity: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Commit one verification step.

    ``accepted_len`` [B] and ``out_tokens`` [R_t] are a verification run's
    outputs.  ``cu_draft`` [B+1] holds the draft-row offsets, so the target
    rows of sequence b start at ``cu_draft[b] + b``.  ``seq_tokens`` [B, >=
    capacity] and ``seq_lens`` [B] are the committed tokens and lengths
    before the step.

    Returns new copies ``(seq_tokens, seq_lens, appended, next_token)``.
    """
    acc = np.asarray(accepted_len, dtype=np.int64)
    out = np.asarray(out_tokens, dtype=np.int64)
    cu = np.asarray(cu_draft, dtype=np.int64)
    toks = np.array(seq_tokens, dtype=np.int32, copy=True)
    lens = np.array(seq_lens, dtype=np.int32, copy=True)
    B = acc.shape[0]
    appended = np.zeros(B, dtype=np.int32)
    next_token = np.full(B, -1, dtype=np.int32)
    for b in range(B):
        n = int(acc[b])
        gamma = int(cu[b + 1] - cu[b])
        if n < 0 or n > gamma:
            continue                       # invalid sequence: nothing is committed
        k = n + 1                          # x_0 .. x_{n-1}, then the target's token
        start = int(lens[b])
        if start < 0 or start + k > capacity:
            appended[b] = -1               # does not fit: nothing is committed
            continue
        t0 = int(cu[b]) + b                # first target row of sequence b
        for j in range(k):
            toks[b, start + j] = out[t0 + j]
        lens[b] = start + k
        appended[b] = k
        next_token[b] = out[t0 + n]
    return toks, lens, appended, next_token
