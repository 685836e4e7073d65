"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks one oracle function against something other than itself:
a worked example printed on the pages, a closed form, a library routine, or
brute force on tiny inputs.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

from conftest import GOLDEN
from oracle import (attention, feature_layers, per_token_cost, rmsnorm, rope,
                    select, swiglu, to_bf16, verify_accept)
from oracle.dflash_oracle import softmax, two_tap_conv


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- verify / accept ---------------------------------------------------------


def test_accept_printed_example():
    """8 drafted, first 6 agree, 7th differs -> accept 6, continue at the 7th."""
    g = _golden("accept_example.json")
    B = g["drafted"]
    rng = np.random.default_rng(0)
    d = rng.integers(0, 1000, size=B)
    G = np.concatenate([d.copy(), [7]])
    k = g["first_mismatch_1based"] - 1
    G[k] = (d[k] + 1) % 1000
    a, committed, nxt = verify_accept(d, G)
    assert a == g["accepted"]
    # generation continues from the 7th position with the target's own token
    assert len(committed) == g["continue_from_1based"]
    assert committed[:a] == [int(x) for x in d[:a]]
    assert committed[a] == int(G[k]) == nxt


def _accept_brute(d, G):
    # longest k such that the first k drafts are a prefix of the target's tokens
    best = 0
    for k in range(len(d) + 1):
        if tuple(d[:k]) == tuple(G[:k]):
            best = k
    return best


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_accept_brute_force(B):
    V = 3
    for d in itertools.product(range(V), repeat=B):
        for G in itertools.product(range(V), repeat=B + 1):
            a, committed, nxt = verify_accept(d, G)
            assert a == _accept_brute(d, G)
            assert len(committed) == a + 1
            assert list(committed[:a]) == list(d[:a])
            assert committed[-1] == G[a] == nxt


def test_accept_special_cases():
    d = [5, 6, 7, 8]
    a, c, n = verify_accept(d, [1, 6, 7, 8, 9])
    assert (a, c, n) == (0, [1], 1)
    a, c, n = verify_accept(d, [5, 6, 7, 8, 9])
    assert (a, c, n) == (4, [5, 6, 7, 8, 9], 9)
    with pytest.raises(ValueError):
        verify_accept(d, [5, 6, 7, 8])


# --- per-token cost ----------------------------------------------------------


def test_cost_closed_form():
    g = _golden("cost_example.json")
    for case in g["cases"]:
        c = per_token_cost(g["t_draft_ms"], g["t_verify_ms"], case["accepted"])
        assert round(c, case["printed_decimals"]) == case["printed_per_token_ms"]
    c6 = per_token_cost(g["t_draft_ms"], g["t_verify_ms"], 6)
    assert c6 == pytest.approx(23.0 / 6.0)
    assert round(g["baseline_per_token_ms"] / c6) == g["printed_speedup_approx"]


# --- feature layers ------------------------------------------------------------


def test_feature_layers_rule():
    for case in _golden("feature_layers.json")["cases"]:
        got = feature_layers(case["n_target_layers"], case["k"])
        assert got == case["layers"]
        # layer 2 (1-based) first, third-from-last last, evenly spaced
        L = case["n_target_layers"]
        assert got[0] + 1 == 2 and got[-1] + 1 == L - 2
        assert len(set(np.diff(got))) == 1


# --- bf16 rounding -------------------------------------------------------------


def test_bf16_matches_torch_random_bits():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    ours = to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_edge_cases():
    vals = np.array([0.0, -0.0, 1.0, np.inf, -np.inf, np.nan,
                     1.0 + 2.0**-8,           # halfway, even below -> down
                     1.0 + 3 * 2.0**-8,       # halfway, odd below -> up
                     1.0 + 2.0**-8 + 2.0**-20,  # just above halfway -> up
                     3.3895313892515355e38,   # max bf16 finite
                     3.4e38,                  # rounds to inf
                     1e-40, -1e-42, 2.0**-133],  # subnormals
                    dtype=np.float32)
    ours = to_bf16(vals)
    ref = torch.from_numpy(vals.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert ours[6] == 1.0 and ours[7] == 1.0 + 4 * 2.0**-8 and ours[8] == 1.0 + 2.0**-7


# --- RMSNorm -------------------------------------------------------------------


def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 96)) * 3
    g = rng.standard_normal(96)
    for eps in (1e-6, 1e-5):
        ref = Fn.rms_norm(torch.from_numpy(x), (96,), torch.from_numpy(g), eps).numpy()
        np.testing.assert_allclose(rmsnorm(x, g, eps), ref, rtol=1e-13, atol=1e-13)


# --- RoPE ----------------------------------------------------------------------


def test_rope_is_complex_rotation():
    rng = np.random.default_rng(3)
    rows, heads, dh = 6, 3, 64
    x = rng.standard_normal((rows, heads, dh))
    pos = np.array([0, 1, 7, 100, 4096, 32775])
    theta = 1.0e6
    half = dh // 2
    z = x[..., :half] + 1j * x[..., half:]
    freq = np.array([theta ** (-(2.0 * j) / dh) for j in range(half)])
    rot = np.exp(1j * np.outer(pos, freq))[:, None, :]
    w = z * rot
    ref = np.concatenate([w.real, w.imag], axis=-1)
    np.testing.assert_allclose(rope(x, pos, theta), ref, rtol=1e-12, atol=1e-12)
    # position 0 is the identity; norms are preserved
    np.testing.assert_array_equal(rope(x[:1], np.array([0]), theta), x[:1])
    np.testing.assert_allclose(np.linalg.norm(rope(x, pos, theta), axis=-1),
                               np.linalg.norm(x, axis=-1), rtol=1e-12)


def test_rope_frequency_schedule_by_hand():
    """The frequency of pair j is theta^(-2j/dh), checked on angles worked out
    by hand, with textbook values of cos(1) and sin(1):

    * dh 4, theta 1e4: pair 1 turns at 1e4^(-2/4) = 1/100 rad per position, so
      position 100 turns it by 1 rad; pair 0 turns at 1 rad per position.
    * dh 128, theta 1e6 (the Qwen3-8B-shaped draft): pair 32 turns at
      1e6^(-64/128) = 1e-3 rad per position, so position 1000 turns it by 1 rad.

    A slip in the exponent (theta^(-j/dh), theta^(-2j/(dh-2)), or pairs of
    adjacent channels instead of halves) moves these off the unit circle
    points below."""
    cos1, sin1 = 0.5403023058681398, 0.8414709848078965  # cos(1), sin(1)
    # dh 4: x = e_1 (real part of pair 1) at position 100 -> (cos 1, sin 1) on channels 1, 3
    x = np.zeros((1, 1, 4))
    x[0, 0, 1] = 1.0
    y = rope(x, np.array([100]), 1.0e4)[0, 0]
    np.testing.assert_allclose(y, [0.0, cos1, 0.0, sin1], rtol=0, atol=1e-13)
    # the imaginary part turns the other way round: e_3 -> (-sin 1, cos 1) on channels 1, 3
    x = np.zeros((1, 1, 4))
    x[0, 0, 3] = 1.0
    y = rope(x, np.array([100]), 1.0e4)[0, 0]
    np.testing.assert_allclose(y, [0.0, -sin1, 0.0, cos1], rtol=0, atol=1e-13)
    # pair 0 at position 1 turns by 1 rad as well
    x = np.zeros((1, 1, 4))
    x[0, 0, 0] = 1.0
    y = rope(x, np.array([1]), 1.0e4)[0, 0]
    np.testing.assert_allclose(y, [cos1, 0.0, sin1, 0.0], rtol=0, atol=1e-13)
    # dh 128, theta 1e6: pair 32 (channels 32 and 96) at position 1000
    x = np.zeros((1, 1, 128))
    x[0, 0, 32] = 1.0
    y = rope(x, np.array([1000]), 1.0e6)[0, 0]
    expect = np.zeros(128)
    expect[32], expect[96] = cos1, sin1
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-12)


def test_rope_relative_position():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 128))
    k = rng.standard_normal((1, 1, 128))
    th = 5.0e5

    def score(pq, pk):
        return float(np.sum(rope(q, np.array([pq]), th) * rope(k, np.array([pk]), th)))

    assert score(10, 3) == pytest.approx(score(1010, 1003), rel=1e-9, abs=1e-9)
    assert score(5, 5) == pytest.approx(float(np.sum(q * k)), rel=1e-12)


# --- attention -----------------------------------------------------------------


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (32, 8)])
def test_attention_matches_sdpa(hq, hkv):
    rng = np.random.default_rng(5)
    rows, keys, dh = 16, 53, 64
    q = rng.standard_normal((rows, hq, dh))
    k = rng.standard_normal((keys, hkv, dh))
    v = rng.standard_normal((keys, hkv, dh))
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    mask = torch.ones(rows, keys, dtype=torch.bool)
    ref = Fn.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


def test_attention_single_key_and_gqa_to_mha():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((5, 8, 32))
    k = rng.standard_normal((1, 2, 32))
    v = rng.standard_normal((1, 2, 32))
    out = attention(q, k, v)
    for j in range(8):
        np.testing.assert_allclose(out[:, j, :], np.broadcast_to(v[0, j // 4], (5, 32)))
    k = rng.standard_normal((9, 2, 32))
    v = rng.standard_normal((9, 2, 32))
    mha = attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1))
    np.testing.assert_allclose(attention(q, k, v), mha, rtol=1e-14, atol=1e-14)


def test_softmax_shift_invariance_and_sum():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((3, 40)) * 30
    p = softmax(s)
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(softmax(s + 1234.5), p, rtol=1e-12)
    ref = torch.softmax(torch.from_numpy(s), dim=-1).numpy()
    np.testing.assert_allclose(p, ref, rtol=1e-12, atol=1e-15)


# --- SwiGLU --------------------------------------------------------------------


def test_swiglu_matches_torch():
    rng = np.random.default_rng(8)
    g = rng.standard_normal((4, 50)) * 6
    u = rng.standard_normal((4, 50))
    ref = (Fn.silu(torch.from_numpy(g)) * torch.from_numpy(u)).numpy()
    np.testing.assert_allclose(swiglu(g, u), ref, rtol=1e-13, atol=1e-13)


# --- select --------------------------------------------------------------------


def test_select_ties_lowest_id_and_topk_order():
    logits = np.array([[0.5, 2.0, 2.0, -1.0, 2.0, 0.5],
                       [3.0, 1.0, 3.0, 3.0, 0.0, 1.0]])
    d, margin, tk = select(logits, topk=4)
    assert list(d) == [1, 0]
    assert list(margin) == [0.0, 0.0]
    ids, vals = tk
    for r in range(2):
        brute = sorted(range(6), key=lambda i: (-logits[r, i], i))[:4]
        assert list(ids[r]) == brute
        np.testing.assert_array_equal(vals[r], logits[r, brute])


def test_select_random_against_brute_force():
    rng = np.random.default_rng(9)
    logits = np.round(rng.standard_normal((8, 300)) * 4, 1)  # many ties
    d, margin, tk = select(logits, topk=16)
    for r in range(8):
        row = list(logits[r])
        best = max(row)
        assert d[r] == row.index(best)
        s = sorted(row, reverse=True)
        assert margin[r] == s[0] - s[1]
        assert list(tk[0][r]) == sorted(range(300), key=lambda i: (-row[i], i))[:16]


# --- two-tap conv --------------------------------------------------------------


def test_two_tap_conv_identity_and_shift():
    rng = np.random.default_rng(10)
    x = rng.standard_normal((16, 24))
    prev = rng.standard_normal(24)
    ident = np.stack([np.ones(24), np.zeros(24)])
    np.testing.assert_array_equal(two_tap_conv(x, ident, prev), x)
    shift = np.stack([np.zeros(24), np.ones(24)])
    y = two_tap_conv(x, shift, prev)
    np.testing.assert_array_equal(y[0], prev)
    np.testing.assert_array_equal(y[1:], x[:-1])
    # linear in the taps: a per-channel combination of the two shifts
    w = rng.standard_normal((2, 24))
    np.testing.assert_allclose(two_tap_conv(x, w, prev),
                               w[0] * x + w[1] * np.concatenate([prev[None], x[:-1]]),
                               rtol=1e-14)
