"""Plain CPU oracle of the target-side verify forward (test infrastructure only).

Sources: [guide] "DFlash：块扩散加速的 LLM 推测解码技术", section 4 (the target
runs once over the original context plus the drafted block and checks every
drafted token in parallel; its hidden states of the feature layers feed the
draft's next context) and section 3.2 (five feature layers from layer 2 to
the third-from-last); [news] "DFlash 2 发布", section "速度之外" (a cycle costs
one draft plus one target verification, 3 ms + 20 ms in its example).

The target is a pre-norm causal decoder shaped like the draft's layers
(RMSNorm, RoPE rotate-half, grouped-query attention, SwiGLU, final RMSNorm,
untied embedding and LM head), with its own paged KV cache in the GPU path.
A forward over R new tokens at positions ctx .. ctx+R-1 of one request
appends their K/V to the cache; row i attends causally to every cached
position and to new rows 0..i.  Readings: the pages do not describe the
target's layers (any decoder of this family is a target); the draft's
storage points are used for it as well (bf16 rounding of the GEMM inputs
a, m, o, z, of q/k/v after RoPE and of the cached K/V; float64 elsewhere);
a feature handed to the draft is the residual stream after the feature
layer, rounded to the storage dtype.
"""
from __future__ import annotations

import numpy as np

from .dflash_oracle import _store, rmsnorm, rope, softmax, swiglu


class TargetOracle:
    """Causal decoder with a KV cache per request.

    cfg: hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, n_layers,
    dtype, rope_theta, rms_eps.  w: embed [V, d], lm_head [V, d], final_norm
    [d], layers[l] = {wqkv [(Hq+2Hkv) dh, d], wo [d, Hq dh], wgateup [2F, d],
    wdown [d, F], attn_norm [d], mlp_norm [d]} (torch Linear layout).
    """

    def __init__(self, cfg: dict, w: dict):
        self.cfg = cfg
        self.w = w
        self.store = _store(cfg["dtype"])
        self.d, self.hq, self.hkv, self.dh = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        self.F, self.V, self.L = cfg["ffn"], cfg["vocab"], cfg["n_layers"]
        self.eps, self.theta = cfg["rms_eps"], cfg["rope_theta"]
        self._f64 = {}

    def _mat(self, key, a):
        """float64 copy of a weight matrix, converted once."""
        if key not in self._f64:
            self._f64[key] = np.asarray(a, dtype=np.float64)
        return self._f64[key]

    def new_cache(self):
        """Per layer K, V lists of [Hkv, dh] rows, one per cached position."""
        return [dict(k=[], v=[]) for _ in range(self.L)]

    @staticmethod
    def truncate(cache, n_pos: int):
        for c in cache:
            del c["k"][n_pos:]
            del c["v"][n_pos:]

    def forward(self, cache, tokens, feat_layers=()):
        """R new tokens at positions len(cache) .. len(cache)+R-1.

        Returns (logits [R, V] float64, features {layer: [R, d] stored dtype}).
        """
        st = self.store
        tokens = np.asarray(tokens, dtype=np.int64)
        R = len(tokens)
        p0 = len(cache[0]["k"])
        pos = p0 + np.arange(R)
        h = np.asarray(np.asarray(self.w["embed"])[tokens], dtype=np.float64)
        G = self.hq // self.hkv
        feats = {}
        for l in range(self.L):
            lw = self.w["layers"][l]
            wqkv = self._mat(("wqkv", l), lw["wqkv"])
            wq = wqkv[: self.hq * self.dh]
            wk = wqkv[self.hq * self.dh: (self.hq + self.hkv) * self.dh]
            wv = wqkv[(self.hq + self.hkv) * self.dh:]
            a = st(rmsnorm(h, lw["attn_norm"], self.eps))
            q = st(rope((a @ wq.T).reshape(R, self.hq, self.dh), pos, self.theta))
            k = st(rope((a @ wk.T).reshape(R, self.hkv, self.dh), pos, self.theta))
            v = st((a @ wv.T).reshape(R, self.hkv, self.dh))
            for i in range(R):
                cache[l]["k"].append(k[i])
                cache[l]["v"].append(v[i])
            K = np.asarray(np.stack(cache[l]["k"]), dtype=np.float64)  # [p0+R, Hkv, dh]
            Vv = np.asarray(np.stack(cache[l]["v"]), dtype=np.float64)
            o = np.empty((R, self.hq, self.dh))
            for j in range(self.hq):
                g = j // G
                s = (np.asarray(q[:, j], dtype=np.float64) @ K[:, g].T) / np.sqrt(self.dh)  # [R, p0+R]
                mask = np.arange(p0 + R)[None, :] <= pos[:, None]  # causal
                s = np.where(mask, s, -np.inf)
                o[:, j] = softmax(s) @ Vv[:, g]
            o = st(o.reshape(R, -1))
            h = h + o @ self._mat(("wo", l), lw["wo"]).T
            m = st(rmsnorm(h, lw["mlp_norm"], self.eps))
            gu = m @ self._mat(("wgateup", l), lw["wgateup"]).T
            z = st(swiglu(gu[:, : self.F], gu[:, self.F:]))
            h = h + z @ self._mat(("wdown", l), lw["wdown"]).T
            if l in feat_layers:
                feats[l] = st(h)
        hn = st(rmsnorm(h, self.w["final_norm"], self.eps))
        logits = hn @ self._mat("lm_head", self.w["lm_head"]).T
        return logits, feats
