"""Tiny target decoder and the speculative loop (test infrastructure only).

The target is a random-init pre-norm causal decoder (RMSNorm, RoPE, MHA,
SwiGLU, final RMSNorm, untied embedding and LM head).  It computes every
position row by row with the same operations whatever the number of rows in
the call, so its verify-mode logits equal its one-token-at-a-time logits bit
for bit.  That makes the lossless property checkable exactly: speculative
output must equal plain greedy decoding of the same target ([news]
"一次写一块"; [guide] sections 3.3 and 4).

The speculative loop follows [guide] section 4: the target's features of the
context feed the draft, the draft proposes a block in one forward, the target
checks the block together with the pending token, the matching prefix plus
the target's own next token is committed, and the features of the committed
positions are injected before the next block.
"""
from __future__ import annotations

import numpy as np

from .dflash_oracle import rmsnorm, rope, swiglu, softmax, verify_accept


class TinyTarget:
    """Row-independent float64 decoder.  ``feat_layers`` outputs are exposed."""

    def __init__(self, cfg: dict, w: dict, feat_layers):
        self.cfg = cfg
        self.w = {k: v for k, v in w.items() if k != "layers"}
        self.layers = [{k: np.asarray(v, np.float64) for k, v in lw.items()} for lw in w["layers"]]
        self.E = np.asarray(w["embed"], np.float64)
        self.E_lm = np.asarray(w["lm_head"], np.float64)
        self.gf = np.asarray(w["final_norm"], np.float64)
        self.h = cfg["n_q_heads"]
        self.dh = cfg["head_dim"]
        self.eps = cfg["rms_eps"]
        self.theta = cfg["rope_theta"]
        self.feat_layers = list(feat_layers)

    def new_cache(self):
        return [dict(k=[], v=[]) for _ in self.layers]

    @staticmethod
    def truncate(cache, n_pos: int):
        for c in cache:
            del c["k"][n_pos:]
            del c["v"][n_pos:]

    def forward_row(self, cache, token: int, pos: int):
        """Process one token at ``pos``; returns (logits [V], features [K, d] fp32)."""
        assert len(cache[0]["k"]) == pos, "rows must arrive in position order"
        h = self.E[int(token)].copy()
        feats = []
        p = np.array([pos])
        for i, lw in enumerate(self.layers):
            a = rmsnorm(h[None, :], lw["attn_norm"], self.eps)[0]
            q = rope((lw["wq"] @ a).reshape(1, self.h, self.dh), p, self.theta)[0]
            k = rope((lw["wk"] @ a).reshape(1, self.h, self.dh), p, self.theta)[0]
            v = (lw["wv"] @ a).reshape(self.h, self.dh)
            cache[i]["k"].append(k)
            cache[i]["v"].append(v)
            K = np.stack(cache[i]["k"], 0)
            Vv = np.stack(cache[i]["v"], 0)
            o = np.empty((self.h, self.dh))
            for j in range(self.h):
                s = (K[:, j, :] @ q[j]) / np.sqrt(self.dh)
                o[j] = softmax(s[None, :])[0] @ Vv[:, j, :]
            h = h + lw["wo"] @ o.reshape(-1)
            m = rmsnorm(h[None, :], lw["mlp_norm"], self.eps)[0]
            h = h + lw["wdown"] @ swiglu(lw["wgate"] @ m, lw["wup"] @ m)
            if i in self.feat_layers:
                feats.append(h.astype(np.float32))
        logits = self.E_lm @ rmsnorm(h[None, :], self.gf, self.eps)[0]
        return logits, feats


def greedy_ar(target: TinyTarget, prompt, new_tokens: int):
    """Plain greedy decoding, one token per target step."""
    cache = target.new_cache()
    logits = None
    for p, t in enumerate(prompt):
        logits, _ = target.forward_row(cache, int(t), p)
    out = [int(np.argmax(logits))]
    pos = len(prompt)
    while len(out) < new_tokens:
        logits, _ = target.forward_row(cache, out[-1], pos)
        pos += 1
        out.append(int(np.argmax(logits)))
    return out


def spec_generate(target: TinyTarget, drafter, prompt, new_tokens: int, block: int,
                  log: list | None = None):
    """Speculative decoding with a block drafter; returns the committed tokens.

    ``drafter`` provides ``inject(features_per_layer)`` (arrays [rows, d] for
    the next positions), ``draft(last_token) -> B ids``, and
    ``verify(draft, greedy) -> (a, committed, next_pending)``.  Reading of the
    block: the B drafts sit at positions n .. n+B-1 after the pending token
    at n-1; the target checks [pending, d_0 .. d_{B-1}] and yields B+1 greedy
    tokens.  The loop stops at exactly ``new_tokens`` committed tokens,
    counting the token produced by the prefill.
    """
    cache = target.new_cache()
    feats = []
    logits = None
    for p, t in enumerate(prompt):
        logits, f = target.forward_row(cache, int(t), p)
        feats.append(f)
    c = int(np.argmax(logits))
    out = [c]
    n = len(prompt) + 1
    drafter.inject([np.stack([f[k] for f in feats], 0) for k in range(len(feats[0]))])
    while len(out) < new_tokens:
        d = [int(x) for x in drafter.draft(c)]
        assert len(d) == block
        G, vfeats = [], []
        for i, tok in enumerate([c] + d):
            lg, f = target.forward_row(cache, tok, n - 1 + i)
            G.append(int(np.argmax(lg)))
            vfeats.append(f)
        a, committed, c_next = drafter.verify(d, G)
        ref = verify_accept(d, G)
        assert (a, list(committed), c_next) == (ref[0], ref[1], ref[2])
        if log is not None:
            log.append(dict(n=n, draft=d, greedy=G, a=a))
        out.extend(committed)
        drafter.inject([np.stack([f[k] for f in vfeats[: a + 1]], 0) for k in range(len(vfeats[0]))])
        target.truncate(cache, n + a)
        n += a + 1
        c = c_next
    return out[:new_tokens]


class OracleDrafter:
    """Adapter that drives a ``DraftOracle`` through the speculative loop."""

    def __init__(self, oracle, start: int = 0):
        self.o = oracle
        self.st = oracle.new_request(start)

    def inject(self, feats):
        self.o.inject(self.st, feats)

    def draft(self, last_token):
        from .dflash_oracle import select

        logits = self.o.draft_block(self.st, last_token)
        return select(logits)[0]

    def verify(self, d, G):
        return verify_accept(d, G)
