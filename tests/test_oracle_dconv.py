"""Pins of the dynamic conv taps (CPU only).

* A case worked by hand: two channels, rank 1, a two-row block.
* Identity static taps with a zero form give the draft without conv, bit
  for bit (the conv then passes the stored rows through).
* A row's taps come from that row's source only: changing one source row
  moves the conv output of that row and of the next one, no other.
* The reading's parameter count (rank 64, hidden 4096, four convs in each
  of five layers) against the page's 16.5 M.
"""
import numpy as np

import synth
from oracle import DraftOracle, dynamic_conv, dynamic_taps, to_bf16


def test_hand_worked_case():
    x = np.array([[1.0, 2.0], [3.0, 4.0]])
    prev0 = np.array([0.5, -1.0])
    D = np.array([[1.0, 1.0]])
    U = np.array([[0.1], [0.2], [0.3], [0.4]])
    w = np.array([[1.0, 1.0], [0.0, 0.0]])
    a, b = dynamic_taps(x, D, U, w)
    # row 0: t = 3, taps a = (1.3, 1.6), b = (0.9, 1.2); row 1: t = 7, a = (1.7, 2.4), b = (2.1, 2.8)
    np.testing.assert_allclose(a, [[1.3, 1.6], [1.7, 2.4]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b, [[0.9, 1.2], [2.1, 2.8]], rtol=0, atol=1e-12)
    y = dynamic_conv(x, a, b, prev0)
    np.testing.assert_allclose(y, [[1.75, 2.0], [7.2, 15.2]], rtol=0, atol=1e-12)


def test_identity_taps_and_zero_form_equal_no_conv():
    shape = synth.config("small_dconv", n_layers=2, window=0, batch=1)
    w = synth.make_weights(shape, norm_std=0.1)
    for lw in w["layers"]:
        lw["conv"] = np.zeros_like(lw["conv"])
        lw["conv"][:, 0, :] = 1.0
        lw["dconv_u"] = np.zeros_like(lw["dconv_u"])
    plain = dict(shape, conv2=0, conv_rank=0)
    rng = np.random.default_rng(0)
    hidden = [to_bf16(rng.standard_normal((30, shape["hidden"])).astype(np.float32)) for _ in range(shape["n_feat"])]
    outs = []
    for cfg in (shape, plain):
        o = DraftOracle(cfg, w)
        st = o.new_request()
        o.inject(st, hidden)
        outs.append(o.draft_block(st, 7) if cfg["conv2"] else o.draft_block(st))
    assert np.array_equal(outs[0], outs[1])


def test_taps_are_local_to_the_row():
    rng = np.random.default_rng(1)
    B, d, K, r = 6, 8, 12, 3
    src = rng.standard_normal((B, K))
    x = rng.standard_normal((B, d))
    D, U = rng.standard_normal((r, K)), rng.standard_normal((2 * d, r))
    w = rng.standard_normal((2, d))
    prev0 = rng.standard_normal(d)
    y0 = dynamic_conv(x, *dynamic_taps(src, D, U, w), prev0)
    for j in range(B):
        s2 = src.copy()
        s2[j] += 1.0
        y1 = dynamic_conv(x, *dynamic_taps(s2, D, U, w), prev0)
        changed = np.nonzero(np.any(y1 != y0, axis=1))[0].tolist()
        assert changed == [j]  # the taps move only row j (row j+1 reads row j's input, not its taps)
        x2 = x.copy()
        x2[j] += 1.0
        y2 = dynamic_conv(x2, *dynamic_taps(src, D, U, w), prev0)
        assert np.nonzero(np.any(y2 != y0, axis=1))[0].tolist() == [j, j + 1][: 2 if j + 1 < B else 1]


def test_parameter_count_of_the_reading():
    d, r, layers = 4096, 64, 5
    params = layers * 4 * (r * d + 2 * d * r)  # D [r, d] and U [2d, r] per conv, four convs per layer
    assert params == 15_728_640 and abs(params / 16.5e6 - 1) < 0.05
