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


# ---------------------------------------------------------------------------
# sampled drafting and lossless verification
#
# Sources: [guide] section 7 (the DFlash-2 path is walked greedily or by
# sampling, with rejection sampling keeping the output distribution exactly
# the target's) and section 3.3 (the target verifies every drafted token in
# parallel; rejected positions are resampled); the guide's CLI examples
# sample at temperature 1 with top-p 0.95 and top-k 64 or 20.
#
# Readings (the pages give no algorithm; this is the standard rejection
# sampling of speculative decoding written out):
# * Sampling settings warp a row of logits in this order: divide by the
#   temperature, keep the top-k (k = 0: all; ties at the boundary to the lower
#   id), softmax, keep the smallest prefix (probability descending, then id)
#   whose cumulative probability reaches top-p, renormalise.
# * The DFlash-2 draft keeps only its top-16 candidates per position, so its
#   distribution q at a position is the warp of those 16 logits (top-k capped
#   at 16); each block position is drafted independently from its q with one
#   uniform number.
# * Position i's draft x is accepted when u < p(x) / q(x) (p the target's
#   warped distribution at that position, u a uniform number in [0, 1)); at
#   the first rejection the target token is drawn from max(0, p - q)
#   renormalised, and after B acceptances from the target's p at position B.
#   The cycle commits the accepted drafts and that token, as in the greedy
#   case.
# * A draw with uniform v from probabilities w walks the support in a fixed
#   order and takes the first entry whose running sum exceeds v * sum(w): the
#   draft's list order; for the target, its kept top-k list (probability
#   descending, then id), or token ids ascending when top-k is 0.
# * top-p below 1 with top-k 0 (a nucleus over the whole vocabulary) is not
#   covered.
# All arithmetic is float64.  Random numbers are inputs.


def warp_sorted(logits, temperature, top_k, top_p):
    """Warped probabilities of logits already ordered by logit descending
    (then id ascending): temperature, top-k, softmax, top-p; zeros where cut."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    n = len(z) if not top_k else min(int(top_k), len(z))
    p = np.zeros(len(z), dtype=np.float64)
    e = np.exp(z[:n] - z[:n].max())
    p[:n] = e / e.sum()
    if top_p < 1.0:
        c = np.cumsum(p[:n])
        keep = int(np.searchsorted(c, top_p, side="left")) + 1  # first index whose sum reaches top_p
        keep = min(keep, n)
        p[keep:] = 0.0
        p /= p.sum()
    return p


def draft_distribution(ids, logits, temperature, top_k, top_p):
    """q of one block position from its top-16 list: {token: probability}."""
    k = min(int(top_k), len(ids)) if top_k else len(ids)
    q = warp_sorted(logits, temperature, k, top_p)
    return {int(t): float(w) for t, w in zip(ids, q) if w > 0.0}, q


def draw(weights, v):
    """Index of the first entry whose running sum exceeds v * sum(weights)
    (the last positive entry if rounding leaves none)."""
    w = np.asarray(weights, dtype=np.float64)
    c = np.cumsum(w)
    hit = np.nonzero(c > v * c[-1])[0]
    if len(hit):
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def draft_sample(ids, logits, temperature, top_k, top_p, v):
    """One drafted token per block position: ids, logits [B, 16] (top-16
    lists), v [B] uniform numbers.  Returns tokens [B]."""
    out = []
    for i in range(len(ids)):
        _, q = draft_distribution(ids[i], logits[i], temperature, top_k, top_p)
        out.append(int(ids[i][draw(q, v[i])]))
    return np.asarray(out, dtype=np.int64)


def target_distribution(logits_row, temperature, top_k, top_p):
    """The target's warped distribution over the vocabulary at one position:
    (p [V], walk order of its support)."""
    lg = np.asarray(logits_row, dtype=np.float64)
    V = len(lg)
    if not top_k:
        if top_p < 1.0:
            raise ValueError("top-p below 1 needs top-k >= 1")
        z = lg / float(temperature)
        e = np.exp(z - z.max())
        return e / e.sum(), np.arange(V)
    order = np.argsort(-lg, kind="stable")[:int(top_k)]
    p = np.zeros(V, dtype=np.float64)
    p[order] = warp_sorted(lg[order], temperature, top_k, top_p)
    return p, order


def spec_verify_sample(draft, draft_ids, draft_logits, target_logits, temperature, top_k, top_p, u,
                       return_draw=False):
    """Rejection-sampling verification of one request's block.

    draft [B] drafted tokens; draft_ids, draft_logits [B, 16] the draft's
    top-16 lists; target_logits [B+1, V] the target's logits at positions
    n .. n+B; u [B+1, 2] uniform numbers (u[i, 0] for the accept test at
    position i, u[i, 1] for the draw at the position where the cycle ends).

    Returns (a, committed list, next pending token, margins): a accepted
    drafts, committed = draft[:a] + [drawn token]; margins[i] = |u[i,0] -
    p(x)/q(x)| for the tested positions and, last, the distance of the final
    draw's threshold to the nearest running-sum boundary (relative to the
    total), which tells how close a decision came to flipping.  With
    return_draw, also (walk order, weights, threshold) of the final draw.
    """
    B = len(draft)
    margins = []
    a = B
    for i in range(B):
        qd, _ = draft_distribution(draft_ids[i], draft_logits[i], temperature, top_k, top_p)
        p, _ = target_distribution(target_logits[i], temperature, top_k, top_p)
        x = int(draft[i])
        qx, px = qd.get(x, 0.0), p[x]
        ratio = px / qx if qx > 0 else -1.0
        margins.append(abs(u[i][0] - ratio) if qx > 0 else np.inf)
        if not (qx > 0 and u[i][0] < ratio):
            a = i
            break
    p, order = target_distribution(target_logits[a], temperature, top_k, top_p)
    r = p[order].copy()
    if a < B:
        qd, _ = draft_distribution(draft_ids[a], draft_logits[a], temperature, top_k, top_p)
        for j, t in enumerate(order):
            r[j] = max(0.0, r[j] - qd.get(int(t), 0.0))
    if r.sum() <= 0.0:  # p == q on the support: fall back to the target's most likely token
        r = p[order].copy()
    j = draw(r, u[a][1])
    c = np.cumsum(r)
    thr = u[a][1] * c[-1]
    margins.append(float(np.min(np.abs(c - thr)) / c[-1]))
    tok = int(order[j])
    committed = [int(t) for t in draft[:a]] + [tok]
    if return_draw:
        return a, committed, tok, np.asarray(margins), (order, r, thr)
    return a, committed, tok, np.asarray(margins)
