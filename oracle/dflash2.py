"""Plain CPU oracle of the DFlash-2 additions to the drafting step (test
infrastructure only, like the rest of this package).

Source: [guide] "DFlash：块扩散加速的 LLM 推测解码技术" (txtmix.com DFlash guide),
section 7 "DFlash 2：并行起草的新一代", bullet on the path selector: instead of
the single most likely candidate per position, DFlash 2 keeps the top-16
candidates of every block position, scores candidate pairs of adjacent
positions with a low-rank bilinear form, and walks one path along those
scores (greedily, or by sampling with rejection sampling keeping the
target's distribution); the selector costs about 2.0 M parameters.

The page gives no formula.  Readings taken here (plain ones, stated once):

* A candidate token t is represented by its row of the shared embedding
  E[t]; the low-rank bilinear form is s(a, b) = (W_u E[a]) . (W_v E[b]) with
  W_u, W_v of shape [r, d] (torch Linear layout).  r = 256 at d = 4096 gives
  2 * 4096 * 256 = 2.1 M parameters, the page's 2.0 M.
* The score of stepping from the chosen candidate a at position i to
  candidate b at position i+1 is the draft's own logit of b plus s(a, b), so
  that with s = 0 the path is the argmax chain of the draft.
* Position 0 takes its top-1 candidate (no predecessor inside the block).
* Ties go to the lower candidate index (the candidate with the higher logit,
  then the lower id, as the top-16 lists are ordered).
* Verification along the path is the greedy prefix acceptance of
  ``verify_accept`` with the path in place of the argmax drafts.

Arithmetic is float64 throughout; the inputs are the stored weights (bf16
values held as float32) and the draft's top-16 lists.
"""
from __future__ import annotations

import numpy as np


def selector_vectors(tokens, embed, wu, wv):
    """(u, v) = (W_u E[t], W_v E[t]) for every token of ``tokens`` (any shape),
    float64, shape tokens.shape + (r,)."""
    t = np.asarray(tokens, dtype=np.int64)
    e = np.asarray(embed, dtype=np.float64)[t.reshape(-1)]
    u = e @ np.asarray(wu, dtype=np.float64).T
    v = e @ np.asarray(wv, dtype=np.float64).T
    r = u.shape[-1]
    return u.reshape(t.shape + (r,)), v.reshape(t.shape + (r,))


def pair_scores(ids, embed, wu, wv):
    """s[i, a, b] = u(ids[i, a]) . v(ids[i+1, b]) for adjacent positions
    i = 0 .. B-2 of one request's candidate lists ids [B, K]; float64 [B-1, K, K]."""
    u, v = selector_vectors(ids, embed, wu, wv)
    B = u.shape[0]
    s = np.empty((max(B - 1, 0), u.shape[1], v.shape[1]), dtype=np.float64)
    for i in range(B - 1):
        s[i] = u[i] @ v[i + 1].T
    return s


def select_path(ids, logits, embed, wu, wv):
    """Greedy path through one request's top-K candidates.

    ids [B, K] candidate tokens per block position (top-K of the draft,
    ordered by logit descending then id ascending), logits [B, K] their
    logits.  Step 0 takes candidate 0; step i+1 takes the candidate b that
    maximises logits[i+1, b] + s[i, k_i, b] (ties to the lower index).

    Returns (path tokens [B], chosen candidate indices [B], step scores [B],
    margins [B]): the step score of position 0 is its logit, a margin is the
    best step score minus the second best at that step.
    """
    ids = np.asarray(ids, dtype=np.int64)
    lg = np.asarray(logits, dtype=np.float64)
    B, K = ids.shape
    s = pair_scores(ids, embed, wu, wv)
    k = np.zeros(B, dtype=np.int64)
    score = np.zeros(B, dtype=np.float64)
    margin = np.zeros(B, dtype=np.float64)
    score[0] = lg[0, 0]
    margin[0] = lg[0, 0] - lg[0, 1] if K > 1 else np.inf
    for i in range(B - 1):
        step = lg[i + 1] + s[i, k[i]]
        k[i + 1] = int(np.argmax(step))
        score[i + 1] = step[k[i + 1]]
        rest = np.delete(step, k[i + 1])
        margin[i + 1] = score[i + 1] - rest.max() if K > 1 else np.inf
    path = ids[np.arange(B), k]
    return path, k, score, margin
