"""Pins of the DFlash-2 path selector oracle (CPU only).

The selector ([guide] section 7, path selector bullet) is only sketched by the
page, so its pins are the reductions the reading implies and a case worked
out by hand:

* with a zero bilinear form the path is the draft's argmax chain (top-1
  candidate at every position);
* a 3-position case with unit-vector embeddings, W_u = I and W_v a cyclic
  shift, where the pair scores (1 and 3) override the logits at positions 1
  and 2 and the direction of the form matters (u of the earlier position,
  v of the later one);
* adding a constant to one position's logits leaves the path unchanged;
* a block of one position takes its top-1 candidate.
"""
import numpy as np
import pytest

from oracle.dflash2 import pair_scores, select_path


def _random_lists(rng, B, K, V):
    ids = np.stack([rng.choice(V, size=K, replace=False) for _ in range(B)])
    lg = -np.sort(-rng.standard_normal((B, K)), axis=1)
    return ids, lg


def test_zero_form_gives_argmax_chain():
    rng = np.random.default_rng(0)
    V, d, r, B, K = 50, 16, 8, 7, 5
    E = rng.standard_normal((V, d))
    ids, lg = _random_lists(rng, B, K, V)
    for wu, wv in ((np.zeros((r, d)), rng.standard_normal((r, d))),
                   (rng.standard_normal((r, d)), np.zeros((r, d)))):
        path, k, score, _ = select_path(ids, lg, E, wu, wv)
        assert np.array_equal(k, np.zeros(B, dtype=np.int64))
        assert np.array_equal(path, ids[:, 0])
        np.testing.assert_array_equal(score, lg[:, 0])


def test_hand_worked_path():
    # embeddings: 32 tokens, d = 4; W_u = I, W_v = cyclic shift (W_v x)_j = x_{(j+1) mod 4}
    E = np.zeros((32, 4))
    E[10] = [1, 0, 0, 0]
    E[11] = [0, 0, 0, 1]
    E[21] = [0, 1, 0, 0]   # v(21) = (1,0,0,0): u(10).v(21) = 1, u(21).v(10) = 0
    E[31] = [0, 0, 3, 0]   # v(31) = (0,3,0,0): u(21).v(31) = 3
    wu = np.eye(4)
    wv = np.zeros((4, 4))
    for j in range(4):
        wv[j, (j + 1) % 4] = 1.0
    ids = np.array([[10, 11], [20, 21], [30, 31]])
    lg = np.array([[1.0, 0.5], [1.0, 0.9], [2.0, 0.0]])
    s = pair_scores(ids, E, wu, wv)
    np.testing.assert_array_equal(s[0], [[0.0, 1.0], [0.0, 0.0]])
    np.testing.assert_array_equal(s[1], [[0.0, 0.0], [0.0, 3.0]])
    path, k, score, margin = select_path(ids, lg, E, wu, wv)
    # step 1 from token 10: 20 scores 1.0 + 0, 21 scores 0.9 + 1 = 1.9 -> 21
    # step 2 from token 21: 30 scores 2.0 + 0, 31 scores 0.0 + 3 = 3.0 -> 31
    assert path.tolist() == [10, 21, 31] and k.tolist() == [0, 1, 1]
    np.testing.assert_allclose(score, [1.0, 1.9, 3.0], rtol=0, atol=1e-15)
    np.testing.assert_allclose(margin, [0.5, 0.9, 1.0], rtol=0, atol=1e-15)
    # the same lists with the form's direction reversed (u and v swapped) keep the argmax chain
    path_rev, _, _, _ = select_path(ids, lg, E, wv, wu)
    assert path_rev.tolist() == [10, 20, 30]


def test_logit_shift_per_position_keeps_path():
    rng = np.random.default_rng(1)
    V, d, r, B, K = 80, 12, 6, 9, 16
    E = rng.standard_normal((V, d))
    wu, wv = rng.standard_normal((r, d)), rng.standard_normal((r, d))
    ids, lg = _random_lists(rng, B, K, V)
    p0, k0, _, _ = select_path(ids, lg, E, wu, wv)
    shifted = lg + rng.standard_normal((B, 1)) * 5
    p1, k1, _, _ = select_path(ids, shifted, E, wu, wv)
    assert np.array_equal(p0, p1) and np.array_equal(k0, k1)


@pytest.mark.parametrize("K", [1, 16])
def test_single_position_block(K):
    rng = np.random.default_rng(2)
    E = rng.standard_normal((40, 8))
    ids, lg = _random_lists(rng, 1, K, 40)
    path, k, score, _ = select_path(ids, lg, E, rng.standard_normal((4, 8)), rng.standard_normal((4, 8)))
    assert path.tolist() == [ids[0, 0]] and k.tolist() == [0] and score[0] == lg[0, 0]


# --- sampled drafting and rejection-sampling verification --------------------

from oracle import verify_accept  # noqa: E402
from oracle.dflash2 import draft_distribution, draft_sample, spec_verify_sample, target_distribution, warp_sorted  # noqa: E402


def test_warp_by_hand():
    lg = np.log([0.5, 0.3, 0.15, 0.05])
    np.testing.assert_allclose(warp_sorted(lg, 1.0, 0, 1.0), [0.5, 0.3, 0.15, 0.05], atol=1e-15)
    # top-p 0.75: 0.5 < 0.75 <= 0.8, so two are kept and renormalised
    np.testing.assert_allclose(warp_sorted(lg, 1.0, 0, 0.75), [0.625, 0.375, 0, 0], atol=1e-15)
    # top-k 3 drops the last and renormalises over 0.95
    np.testing.assert_allclose(warp_sorted(lg, 1.0, 3, 1.0), [0.5 / 0.95, 0.3 / 0.95, 0.15 / 0.95, 0], atol=1e-15)
    # temperature 2 takes square roots of the probabilities before renormalising
    s = np.sqrt([0.5, 0.3, 0.15, 0.05])
    np.testing.assert_allclose(warp_sorted(lg, 2.0, 0, 1.0), s / s.sum(), atol=1e-15)
    # the target's top-k keeps the k largest logits, ties to the lower id
    p, order = target_distribution(np.array([1.0, 3.0, 3.0, 0.0, 2.0]), 1.0, 2, 1.0)
    assert order.tolist() == [1, 2] and p[0] == p[3] == p[4] == 0.0


def _random_case(seed, V=7, B=3, K=5, sharp=1.5):
    rng = np.random.default_rng(seed)
    tl = rng.standard_normal((B + 1, V)) * sharp
    dl = rng.standard_normal((B, V)) * sharp + 0.5 * tl[:B]  # a draft that partly agrees
    ids = np.argsort(-dl, axis=1, kind="stable")[:, :K]
    lg = np.take_along_axis(dl, ids, axis=1)
    return tl, ids, lg


@pytest.mark.parametrize("T,top_k,top_p", [(1.0, 0, 1.0), (0.7, 4, 0.9), (1.3, 3, 1.0)])
def test_rejection_sampling_keeps_the_target_distribution(T, top_k, top_p):
    """Monte Carlo over the uniform numbers: the first committed token follows
    the target's warped distribution at that position, and the first draft is
    accepted with probability sum_x min(p(x), q(x)) (both within 5 sigma)."""
    tl, ids, lg = _random_case(3)
    B, V = ids.shape[0], tl.shape[1]
    p0, _ = target_distribution(tl[0], T, top_k, top_p)
    qd0, _ = draft_distribution(ids[0], lg[0], T, top_k, top_p)
    acc_prob = sum(min(p0[t], w) for t, w in qd0.items())
    rng = np.random.default_rng(11)
    N = 60000
    counts = np.zeros(V)
    accepted = 0
    for _ in range(N):
        d = draft_sample(ids, lg, T, top_k, top_p, rng.random(B))
        a, com, nxt, _ = spec_verify_sample(d, ids, lg, tl, T, top_k, top_p, rng.random((B + 1, 2)))
        counts[com[0]] += 1
        accepted += a >= 1
        assert nxt == com[-1] and len(com) == a + 1
    freq = counts / N
    sig = np.sqrt(p0 * (1 - p0) / N) + 1e-12
    assert np.all(np.abs(freq - p0) <= 5 * sig + 1e-9), (freq, p0)
    s = np.sqrt(acc_prob * (1 - acc_prob) / N)
    assert abs(accepted / N - acc_prob) <= 5 * s


def test_draft_equal_to_target_accepts_everything():
    rng = np.random.default_rng(4)
    B, V = 4, 9
    tl = rng.standard_normal((B + 1, V))
    ids = np.argsort(-tl[:B], axis=1, kind="stable")  # the full vocabulary as the list
    lg = np.take_along_axis(tl[:B], ids, axis=1)
    for _ in range(200):
        d = draft_sample(ids, lg, 1.0, 0, 1.0, rng.random(B))
        a, com, _, _ = spec_verify_sample(d, ids, lg, tl, 1.0, 0, 1.0, rng.random((B + 1, 2)))
        assert a == B and com[:B] == d.tolist()


def test_near_zero_temperature_is_greedy_verification():
    """Both distributions collapse onto their argmax: the sampled path and
    the rejection test reduce to greedy drafting and greedy prefix
    acceptance, whatever the uniform numbers."""
    rng = np.random.default_rng(5)
    B, V = 6, 40
    for trial in range(30):
        tl = rng.standard_normal((B + 1, V))
        dl = tl[:B] + rng.standard_normal((B, V)) * 0.8
        ids = np.argsort(-dl, axis=1, kind="stable")[:, :16]
        lg = np.take_along_axis(dl, ids, axis=1)
        d = draft_sample(ids, lg, 1e-4, 0, 1.0, rng.random(B))
        assert d.tolist() == ids[:, 0].tolist()
        a, com, nxt, _ = spec_verify_sample(d, ids, lg, tl, 1e-4, 0, 1.0, rng.random((B + 1, 2)))
        ga, gcom, gnxt = verify_accept(d, np.argmax(tl, axis=1))
        assert (a, com, nxt) == (ga, gcom, gnxt)
