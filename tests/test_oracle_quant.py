"""Pins of the 4-bit draft-weight oracle (CPU only).

* Weights already on a 4-bit grid (each group = b0 + s0 * q0 with a
  power-of-two step, codes 0 and 15 present) come back exactly: the codes,
  the scales and biases, and the dequantised values equal the weights.
* A constant group has scale 0, codes 0 and dequantises to itself.
* On random bf16 weights every dequantised value is within half a step of
  the weight (plus the gap the bf16 scale leaves at the top of the group),
  codes stay in 0..15 and each group's smallest weight is reproduced.
* A draft whose quantised matrices lie on the grid drafts exactly (float64,
  bit for bit) as the unquantised draft, and the matrices the 4-bit draft
  does not own (embedding, LM head, gains) are left as they are.
"""
import numpy as np

import synth
from oracle import DraftOracle, to_bf16
from oracle.quant import GROUP, dequantize_q4, q4_draft_weights, quantize_q4


def _grid(rng, N, K):
    """bf16-exact weights on a 4-bit grid per group of 64."""
    G = K // GROUP
    e = rng.integers(4, 12, size=(N, G))          # step 2^-e
    m = rng.integers(-100, 100, size=(N, G))      # bias m * 2^-e (|m + q| < 128: exact in bf16)
    q = rng.integers(0, 16, size=(N, G, GROUP))
    q[..., 0] = 0
    q[..., 1] = 15
    q = np.take_along_axis(q, rng.permuted(np.tile(np.arange(GROUP), (N, G, 1)), axis=-1), axis=-1)
    step = np.ldexp(1.0, -e)
    w = (m[..., None] + q) * step[..., None]
    w = w.reshape(N, K).astype(np.float32)
    assert np.array_equal(to_bf16(w), w)
    return w, q.reshape(N, K).astype(np.uint8), step.astype(np.float32), (m * step).astype(np.float32)


def test_grid_weights_come_back_exactly():
    rng = np.random.default_rng(0)
    w, q0, s0, b0 = _grid(rng, 48, 256)
    q, s, b = quantize_q4(w)
    assert np.array_equal(q, q0) and np.array_equal(s, s0) and np.array_equal(b, b0)
    assert np.array_equal(dequantize_q4(q, s, b), w.astype(np.float64))


def test_constant_group():
    w = np.full((2, 128), 0.375, dtype=np.float32)
    w[1, 64:] = -1.5
    q, s, b = quantize_q4(w)
    assert np.all(q == 0) and np.all(s == 0)
    assert np.array_equal(dequantize_q4(q, s, b), w.astype(np.float64))


def test_half_step_error_bound_on_random_weights():
    rng = np.random.default_rng(1)
    w = to_bf16(rng.standard_normal((64, 1024)).astype(np.float32) * 0.02)
    q, s, b = quantize_q4(w)
    assert q.max() <= 15
    wh = dequantize_q4(q, s, b)
    wg = w.reshape(64, -1, GROUP).astype(np.float64)
    lo, hi = wg.min(-1), wg.max(-1)
    s64 = s.astype(np.float64)
    gap = np.abs((hi - lo) - 15 * s64)  # what the bf16 rounding of the scale leaves uncovered
    bound = np.repeat(s64 / 2 + gap, GROUP, axis=1) * (1 + 1e-6) + 1e-12
    assert np.all(np.abs(wh - w) <= bound)
    # the smallest weight of every group is reproduced
    assert np.array_equal(wh.reshape(64, -1, GROUP).min(-1), lo)
    # and the error is a real quantisation error, not zero
    assert np.mean(np.abs(wh - w)) > 1e-5


def test_grid_draft_drafts_like_the_unquantised_draft():
    shape = synth.config("small_bf16", n_layers=2)
    w = synth.make_weights(shape, norm_std=0.1)
    rng = np.random.default_rng(2)
    w["fc"] = _grid(rng, *w["fc"].shape)[0]
    for lw in w["layers"]:
        for name in ("wqkv", "wo", "wgateup", "wdown"):
            lw[name] = _grid(rng, *lw[name].shape)[0] * np.float32(1.0 / 64)
    wq = q4_draft_weights(w)
    for key in ("embed", "lm_head", "final_norm", "fc_norm"):
        assert wq[key] is w[key]
    assert wq["layers"][0]["attn_norm"] is w["layers"][0]["attn_norm"]
    hidden = [to_bf16(rng.standard_normal((40, shape["hidden"])).astype(np.float32)) for _ in range(shape["n_feat"])]
    outs = []
    for ww in (w, wq):
        o = DraftOracle(shape, ww)
        st = o.new_request()
        o.inject(st, hidden)
        outs.append(o.draft_block(st))
    assert np.array_equal(outs[0], outs[1])
