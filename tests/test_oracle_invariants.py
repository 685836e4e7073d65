"""Invariants of the composed oracle: lossless decoding and exact reductions."""
import numpy as np
import pytest

import synth
from oracle import (DraftOracle, OracleDrafter, TinyTarget, greedy_ar, rmsnorm,
                    select, spec_generate, to_bf16)


@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    tw = synth.tiny_target_weights(cfg)
    dw = synth.make_weights(cfg, shared=tw)
    target = TinyTarget(cfg, tw, cfg["feat_layers"])
    prm = synth.prompt(cfg)
    ref = greedy_ar(target, prm, cfg["new_tokens"])
    return cfg, tw, dw, target, prm, ref


def test_tiny_spec_equals_greedy(tiny):
    cfg, tw, dw, target, prm, ref = tiny
    log = []
    out = spec_generate(target, OracleDrafter(DraftOracle(cfg, dw)), prm,
                        cfg["new_tokens"], cfg["block_size"], log=log)
    assert out == ref
    assert len(out) == cfg["new_tokens"]
    assert all(0 <= e["a"] <= cfg["block_size"] for e in log)


class _ScriptedDrafter:
    """Drafts taken from the known greedy continuation (perfect) or shifted by one (adversarial)."""

    def __init__(self, ref, n_prompt, B, V, shift):
        self.ref, self.n0, self.B, self.V, self.shift = ref, n_prompt, B, V, shift
        self.n = n_prompt + 1
        self.accepts = []

    def inject(self, feats):
        pass

    def draft(self, last_token):
        i0 = self.n - self.n0  # index into ref of the token at position n
        seq = [self.ref[i] if i < len(self.ref) else 0 for i in range(i0, i0 + self.B)]
        return [(t + self.shift) % self.V for t in seq]

    def verify(self, d, G):
        from oracle import verify_accept
        a, c, nxt = verify_accept(d, G)
        self.accepts.append(a)
        self.n += a + 1
        return a, c, nxt


@pytest.mark.parametrize("shift", [0, 1])
def test_tiny_spec_lossless_perfect_and_adversarial(tiny, shift):
    cfg, tw, dw, target, prm, ref = tiny
    dr = _ScriptedDrafter(ref, len(prm), cfg["block_size"], cfg["vocab"], shift)
    out = spec_generate(target, dr, prm, cfg["new_tokens"], cfg["block_size"])
    assert out == ref
    if shift == 0:
        assert all(a == cfg["block_size"] for a in dr.accepts[:-1])
    else:
        assert all(a == 0 for a in dr.accepts)


def _small(name="small_bf16", **over):
    cfg = synth.config(name, **over)
    return cfg, synth.make_weights(cfg, norm_std=0.1)


def _run(cfg, w, ctx, last_token=None, chunks=None, start=0):
    o = DraftOracle(cfg, w)
    st = o.new_request(start)
    H = synth.hidden_rows(cfg, 0, start, ctx - start)
    edges = chunks or [0, ctx - start]
    for a, b in zip(edges[:-1], edges[1:]):
        o.inject(st, [h[a:b] for h in H])
    return o, st, o.draft_block(st, last_token, trace=True)


def test_inject_chunking_invariance():
    cfg, w = _small(n_layers=1)
    o1, st1, _ = _run(cfg, w, 37)
    o2, st2, _ = _run(cfg, w, 37, chunks=[0, 5, 6, 20, 37])
    for l in range(cfg["n_layers"]):
        np.testing.assert_allclose(st1.K[l], st2.K[l], rtol=0, atol=np.abs(st1.K[l]).max() * 2**-7)
        assert np.mean(st1.K[l] == st2.K[l]) > 0.999
        assert np.mean(st1.V[l] == st2.V[l]) > 0.999


def test_feature_projection_is_linear_in_the_layers():
    """concat(H) @ W_fc^T equals the sum of per-layer partial products."""
    cfg, w = _small(n_layers=1)
    o = DraftOracle(cfg, w)
    H = synth.hidden_rows(cfg, 0, 0, 9)
    f, u = o.context_feature(H)
    d = cfg["hidden"]
    parts = sum(np.asarray(H[k], np.float64) @ np.asarray(w["fc"][:, k * d:(k + 1) * d], np.float64).T
                for k in range(cfg["n_feat"]))
    np.testing.assert_allclose(u, parts, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(f, to_bf16(rmsnorm(parts, w["fc_norm"], cfg["rms_eps"])))


def test_window_at_least_context_equals_no_window():
    cfg, w = _small(n_layers=1)
    _, _, (l0, h0) = _run(cfg, w, 300)
    cfgw = dict(cfg, window=512)
    _, _, (l1, h1) = _run(cfgw, w, 300)
    np.testing.assert_array_equal(l0, l1)


def test_window_drops_old_positions():
    """With window W, the block sees exactly the last W positions."""
    cfg, w = _small(n_layers=1)
    cfgw = dict(cfg, window=64)
    _, _, (lw_, _) = _run(cfgw, w, 300)
    # same result as a request that only ever injected the last 64 positions
    _, _, (ls, _) = _run(cfgw, w, 300, start=236)
    np.testing.assert_array_equal(lw_, ls)
    _, _, (l0, _) = _run(cfg, w, 300)
    assert not np.array_equal(lw_, l0)


def test_conv_identity_taps_reproduce_plain_forward():
    cfg, w = _small(n_layers=2)
    _, _, (l0, h0) = _run(cfg, w, 50)
    cfgc = dict(cfg, conv2=1)
    wc = dict(w)
    wc["layers"] = []
    for lw in w["layers"]:
        lw = dict(lw)
        c = np.zeros((4, 2, cfg["hidden"]), np.float32)
        c[:, 0, :] = 1.0
        lw["conv"] = c
        wc["layers"].append(lw)
    _, _, (l1, h1) = _run(cfgc, wc, 50, last_token=17)
    np.testing.assert_array_equal(l0, l1)
    # a non-identity tap changes the result and makes it depend on the last token
    wc["layers"][0]["conv"] = wc["layers"][0]["conv"].copy()
    wc["layers"][0]["conv"][0, 1, :] = 0.5
    _, _, (l2, _) = _run(cfgc, wc, 50, last_token=17)
    _, _, (l3, _) = _run(cfgc, wc, 50, last_token=18)
    assert not np.array_equal(l1, l2) and not np.array_equal(l2, l3)


def test_gqa_equals_mha_with_repeated_kv_weights():
    cfg, w = _small(n_layers=1)
    group = cfg["n_q_heads"] // cfg["n_kv_heads"]
    dh, hq, hkv = cfg["head_dim"], cfg["n_q_heads"], cfg["n_kv_heads"]
    wm = dict(w)
    wm["layers"] = []
    for lw in w["layers"]:
        q = lw["wqkv"][: hq * dh]
        k = lw["wqkv"][hq * dh:(hq + hkv) * dh].reshape(hkv, dh, -1)
        v = lw["wqkv"][(hq + hkv) * dh:].reshape(hkv, dh, -1)
        k = np.repeat(k, group, axis=0).reshape(hq * dh, -1)
        v = np.repeat(v, group, axis=0).reshape(hq * dh, -1)
        wm["layers"].append(dict(lw, wqkv=np.concatenate([q, k, v], 0)))
    cfgm = dict(cfg, n_kv_heads=hq)
    _, _, (l0, _) = _run(cfg, w, 40)
    _, _, (l1, _) = _run(cfgm, wm, 40)
    np.testing.assert_allclose(l0, l1, rtol=1e-12, atol=1e-12)


def test_zero_output_projections_leave_the_mask_embedding():
    """With W_o = W_down = 0 the residual stays E[mask]: every row gets the same logits."""
    cfg, w = _small(n_layers=2)
    wz = dict(w)
    wz["layers"] = [dict(lw, wo=np.zeros_like(lw["wo"]), wdown=np.zeros_like(lw["wdown"]))
                    for lw in w["layers"]]
    _, _, (lg, hs) = _run(cfg, wz, 20)
    for h in hs:
        np.testing.assert_array_equal(h, np.repeat(w["embed"][cfg["mask_id"]][None].astype(np.float64), cfg["block_size"], 0))
    assert np.all(lg == lg[0])
    d, _, _ = select(lg)
    assert len(set(d.tolist())) == 1


def test_block_rows_depend_on_position_only_through_rope():
    """All block rows start from the same mask embedding and differ only through
    the RoPE positions of q and k: with W_q = W_k = 0 every row is identical."""
    cfg, w = _small(n_layers=1)
    hq, hkv, dh = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    wz = dict(w)
    wz["layers"] = []
    for lw in w["layers"]:
        wqkv = lw["wqkv"].copy()
        wqkv[: (hq + hkv) * dh] = 0
        wz["layers"].append(dict(lw, wqkv=wqkv))
    _, _, (lg, _) = _run(cfg, wz, 33)
    assert np.all(lg == lg[0])
