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
