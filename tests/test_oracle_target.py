"""Pins of the target verify-forward oracle (CPU only).

* With fp32 storage and multi-head attention it is the tiny target of the
  end-to-end workload, whose row-by-row forward is pinned by speculative
  decoding equalling greedy decoding: logits and feature layers agree to
  fp32 rounding, for the prompt in one block and in chunks.
* Causality: a row's logits do not depend on later tokens.
* Grouped-query attention equals multi-head attention with each K/V head's
  weights repeated over its query heads.
* A block processed in chunks equals the block in one call.
"""
import numpy as np

import synth
from oracle import TinyTarget, feature_layers
from oracle.target import TargetOracle


def _tiny():
    cfg = synth.config("tiny")
    tw = synth.tiny_target_weights(cfg)
    tcfg = dict(cfg, n_layers=cfg["target_layers"], n_kv_heads=cfg["n_q_heads"])
    layers = [dict(wqkv=np.concatenate([lw["wq"], lw["wk"], lw["wv"]]), wo=lw["wo"],
                   wgateup=np.concatenate([lw["wgate"], lw["wup"]]), wdown=lw["wdown"],
                   attn_norm=lw["attn_norm"], mlp_norm=lw["mlp_norm"]) for lw in tw["layers"]]
    w = dict(embed=tw["embed"], lm_head=tw["lm_head"], final_norm=tw["final_norm"], layers=layers)
    return cfg, tw, tcfg, w


def test_equals_tiny_target_row_by_row():
    cfg, tw, tcfg, w = _tiny()
    feats = cfg["feat_layers"]
    tiny = TinyTarget(cfg, tw, feats)
    o = TargetOracle(tcfg, w)
    rng = np.random.default_rng(0)
    prompt = rng.integers(0, cfg["vocab"], size=23)
    tc = tiny.new_cache()
    ref_lg, ref_f = [], []
    for p, t in enumerate(prompt):
        lg, f = tiny.forward_row(tc, int(t), p)
        ref_lg.append(lg)
        ref_f.append(f)
    for chunks in ([23], [5, 1, 17]):
        cache = o.new_cache()
        lgs, fs = [], {l: [] for l in feats}
        off = 0
        for c in chunks:
            lg, f = o.forward(cache, prompt[off:off + c], feats)
            lgs.append(lg)
            for l in feats:
                fs[l].append(f[l])
            off += c
        lg = np.concatenate(lgs)
        np.testing.assert_allclose(lg, np.stack(ref_lg), rtol=2e-5, atol=2e-5)
        for k, l in enumerate(feats):
            np.testing.assert_allclose(np.concatenate(fs[l]), np.stack([f[k] for f in ref_f]), rtol=2e-5, atol=2e-5)


def test_causal_and_chunked():
    shape = synth.config("small_bf16", n_layers=2)
    w = synth.make_weights(shape, norm_std=0.1)
    o = TargetOracle(shape, w)
    rng = np.random.default_rng(1)
    toks = rng.integers(0, shape["vocab"], size=20)
    c1 = o.new_cache()
    full, _ = o.forward(c1, toks)
    c2 = o.new_cache()
    a, _ = o.forward(c2, toks[:12])
    b, _ = o.forward(c2, toks[12:])
    np.testing.assert_allclose(np.concatenate([a, b]), full, rtol=1e-12, atol=1e-12)
    toks2 = toks.copy()
    toks2[15:] = (toks2[15:] + 7) % shape["vocab"]
    c3 = o.new_cache()
    alt, _ = o.forward(c3, toks2)
    np.testing.assert_allclose(alt[:15], full[:15], rtol=1e-12, atol=1e-12)
    assert not np.allclose(alt[15:], full[15:])


def test_gqa_equals_mha_with_repeated_heads():
    shape = synth.config("small_bf16", n_layers=2, dtype="f32")
    w = synth.make_weights(shape)
    hq, hkv, dh = shape["n_q_heads"], shape["n_kv_heads"], shape["head_dim"]
    G = hq // hkv
    mha = dict(shape, n_kv_heads=hq)
    w2 = dict(w, layers=[])
    for lw in w["layers"]:
        q = lw["wqkv"][: hq * dh]
        k = lw["wqkv"][hq * dh: (hq + hkv) * dh].reshape(hkv, dh, -1)
        v = lw["wqkv"][(hq + hkv) * dh:].reshape(hkv, dh, -1)
        kr = np.repeat(k, G, axis=0).reshape(hq * dh, -1)
        vr = np.repeat(v, G, axis=0).reshape(hq * dh, -1)
        w2["layers"].append(dict(lw, wqkv=np.concatenate([q, kr, vr])))
    toks = np.random.default_rng(2).integers(0, shape["vocab"], size=9)
    a, _ = TargetOracle(shape, w).forward(TargetOracle(shape, w).new_cache(), toks)
    b, _ = TargetOracle(mha, w2).forward(TargetOracle(mha, w2).new_cache(), toks)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)
    # the draft's feature rule for a 36-layer target
    assert feature_layers(36) == [1, 9, 17, 25, 33]
