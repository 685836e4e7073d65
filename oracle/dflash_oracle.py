"""Plain CPU oracle of the DFlash drafting step (test infrastructure only).

Sources (web pages about DFlash; cited by page and section):

* [guide] "DFlash：块扩散加速的 LLM 推测解码技术" (txtmix.com DFlash guide),
  section 3.1 (one forward drafts a whole block; block 16, 10 for LLaMA-3.1;
  draft reuses the target's embedding and LM head; 5 layers, 8 for the coder
  draft), section 3.2 (five target layers evenly spaced from layer 2 to the
  third-from-last, concatenated, projected, RMSNormed, written into every
  draft layer's K/V projection and KV cache), section 3.3 and section 4
  (target verifies the block; the matching prefix is kept), section 7
  (DFlash 2: top-16 candidates per position; a two-tap depthwise conv around
  attention and MLP whose block start reads the last verified token).
* [news] "DFlash 2 发布" (openai-hub.com), section "DFlash 2 的核心：一次写一块"
  (8 drafted, first 6 match the target's greedy choice, 7th differs: accept
  6) and section "速度之外" (per-token cost example: 3 ms draft + 20 ms
  verify).
* [repo] llmapis.com post, "数据和技术细节" (draft sliding window bounding draft
  KV growth).

Where the pages leave a step open, the plain reading is taken; each such
reading is named in the docstring of the function that applies it.

Precision: every matmul, norm and softmax runs in float64.  Values are
rounded to the storage dtype (bf16 by round-to-nearest-even on the float32
bit pattern, or float32 for fp32 workloads) only at these storage points:
weights and input hidden states (already stored), the context feature f, the
K/V cache, block q/k/v after RoPE, and the GEMM inputs a, m, o, z and the
final normed hidden.  The residual stream and logits stay float64.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


# ---------------------------------------------------------------------------
# rounding


def to_bf16(x) -> np.ndarray:
    """Round to bfloat16 (nearest-even on the float32 bit pattern), as float32.

    NaN maps to the canonical quiet NaN 0x7FC0; overflow rounds to +-inf.
    """
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    r = np.where(np.isnan(x32), np.uint32(0x7FC00000), r)
    return r.view(np.float32)


def to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float32)


def _store(dtype: str):
    return to_bf16 if dtype == "bf16" else to_f32


# ---------------------------------------------------------------------------
# building blocks


def feature_layers(n_target_layers: int, k: int = 5) -> list[int]:
    """0-based target layers whose outputs feed the draft ([guide] section 3.2).

    Reading: "from layer 2 to the third-from-last" in 1-based numbering is the
    0-based span [1, L-3]; k layers are spaced evenly over it with integer
    floor (exact for L = 32 and 36, where the span divides by 4).
    """
    if k < 2 or n_target_layers < 4:
        raise ValueError("need k >= 2 and at least 4 target layers")
    first, last = 1, n_target_layers - 3
    return [first + (i * (last - first)) // (k - 1) for i in range(k)]


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * gamma over the last axis, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding by rotate-half pairs (j, j + dh/2).

    x: [rows, heads, dh]; pos: [rows] absolute positions.  Pair j turns by the
    angle pos * theta^(-2j/dh).  Reading: the pages name no RoPE variant; the
    rotate-half form of the Qwen and LLaMA families is used, without scaling.
    """
    x = np.asarray(x, dtype=np.float64)
    dh = x.shape[-1]
    half = dh // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / dh)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def softmax(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.float64)
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Grouped-query attention with no mask among the given keys.

    q: [rows, Hq, dh]; k, v: [keys, Hkv, dh].  Query head j reads KV head
    j // (Hq / Hkv); scores are scaled by 1/sqrt(dh).  Every query row sees
    every key given to it: the block is bidirectional and sees all visible
    context positions.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows, hq, dh = q.shape
    hkv = k.shape[1]
    group = hq // hkv
    out = np.empty((rows, hq, dh), dtype=np.float64)
    for j in range(hq):
        g = j // group
        s = (q[:, j, :] @ k[:, g, :].T) / np.sqrt(dh)
        out[:, j, :] = softmax(s) @ v[:, g, :]
    return out


def silu(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def swiglu(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    return silu(gate) * np.asarray(up, dtype=np.float64)


def two_tap_conv(x: np.ndarray, w: np.ndarray, x_prev0: np.ndarray) -> np.ndarray:
    """Depthwise two-tap conv along the block ([guide] section 7).

    y[i] = w0 * x[i] + w1 * x[i-1]; row 0 reads ``x_prev0`` in place of
    x[-1].  Reading: the pages call the taps "dynamic" without giving their
    form; static per-channel taps are used, and the block start reads the
    shared embedding of the last verified token.
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    prev = np.concatenate([np.asarray(x_prev0, dtype=np.float64)[None, :], x[:-1]], axis=0)
    return w[0][None, :] * x + w[1][None, :] * prev


def dynamic_taps(src, D, U, w_static):
    """Dynamic two-tap conv taps of every row ([guide] section 7: the conv
    is "dynamic"; the page gives no form and puts the cost at 16.5 M
    parameters).

    Reading: the taps of a row are a rank-r linear function of that row of
    the conv's own input, added to the static taps: t = D src (D [r, d]),
    then [a; b] = w_static + U t (U [2d, r]: rows 0..d-1 give a, rows
    d..2d-1 give b).  The input is the stored normed rows for the convs
    before attention and the MLP, and the projection's output (W_o o,
    W_down z) for the convs after them.  With r = 64 and d = 4096 the four
    convs of one layer hold 4 * 3 * 4096 * 64 = 3.1 M parameters, 15.7 M
    over five layers, the page's 16.5 M within 5 %.

    src [rows, d]; w_static [2, d].  Returns (a, b), each [rows, d], float64.
    """
    t = np.asarray(src, dtype=np.float64) @ np.asarray(D, dtype=np.float64).T
    delta = t @ np.asarray(U, dtype=np.float64).T
    d = delta.shape[1] // 2
    w = np.asarray(w_static, dtype=np.float64)
    return w[0][None, :] + delta[:, :d], w[1][None, :] + delta[:, d:]


def dynamic_conv(x, a, b, x_prev0):
    """y[i] = a[i] * x[i] + b[i] * x[i-1] with per-row taps; row 0 reads
    ``x_prev0`` in place of x[-1]."""
    x = np.asarray(x, dtype=np.float64)
    prev = np.concatenate([np.asarray(x_prev0, dtype=np.float64)[None, :], x[:-1]], axis=0)
    return a * x + b * prev


def select(logits: np.ndarray, topk: int = 0):
    """Greedy choice per position from float logits [rows, V].

    Returns (argmax ids with ties to the lowest id, top-1 minus top-2 margin,
    top-k ids and values ordered by logit descending then id ascending, or
    None when topk == 0).
    """
    logits = np.asarray(logits, dtype=np.float64)
    d = np.argmax(logits, axis=-1).astype(np.int64)
    part = -np.partition(-logits, 1, axis=-1)[:, :2]
    margin = part[:, 0] - part[:, 1]
    tk = None
    if topk:
        order = np.argsort(-logits, axis=-1, kind="stable")[:, :topk]
        tk = (order.astype(np.int64), np.take_along_axis(logits, order, axis=-1))
    return d, margin, tk


def verify_accept(draft, greedy):
    """Keep the longest prefix of ``draft`` that matches the target's greedy tokens.

    draft d[0..B) are the drafted tokens for positions n..n+B-1; greedy
    G[0..B] are the target's greedy tokens for positions n..n+B ([news]
    "一次写一块": with 8 drafted and the first 6 matching, 6 are accepted and
    generation continues at the 7th).  a = number of leading i with
    d[i] == G[i]; the cycle commits d[0..a) followed by the target's own token
    G[a], which becomes the next pending token.
    Returns (a, committed list, new pending token).
    """
    d = [int(t) for t in draft]
    g = [int(t) for t in greedy]
    if len(g) != len(d) + 1:
        raise ValueError("greedy must hold one more token than draft")
    a = 0
    while a < len(d) and d[a] == g[a]:
        a += 1
    committed = d[:a] + [g[a]]
    return a, committed, g[a]


def per_token_cost(t_draft: float, t_verify: float, accepted: float) -> float:
    """Cost per output token of one draft+verify round ([news] "速度之外")."""
    return (t_draft + t_verify) / accepted


# ---------------------------------------------------------------------------
# draft model


@dataclass
class RequestState:
    """One request's drafting state.

    ``ctx_len`` positions [0, ctx_len) are committed and known to the target
    (the pending token sits at position ctx_len).  ``kv_begin`` is the first
    injected position.  K/V hold per-layer arrays [positions, Hkv, dh] for
    positions [kv_pos0, ctx_len).
    """

    kv_begin: int = 0
    ctx_len: int = 0
    kv_pos0: int = 0
    K: list = field(default_factory=list)
    V: list = field(default_factory=list)


class DraftOracle:
    """Block-diffusion draft forward with target-feature KV injection.

    cfg: shape dictionary (hidden, n_q_heads, n_kv_heads, head_dim, ffn,
    vocab, n_layers, block_size, n_feat, dtype, rope_theta, rms_eps, window,
    conv2, topk, mask_id).  w: weights in [out, in] layout (see
    ``synth.make_weights``).
    """

    def __init__(self, cfg: dict, w: dict):
        self.cfg = cfg
        self.w = w
        self.store = _store(cfg["dtype"])
        self.d = cfg["hidden"]
        self.hq = cfg["n_q_heads"]
        self.hkv = cfg["n_kv_heads"]
        self.dh = cfg["head_dim"]
        self.F = cfg["ffn"]
        self.L = cfg["n_layers"]
        self.B = cfg["block_size"]
        self.eps = cfg["rms_eps"]
        self.theta = cfg["rope_theta"]
        self.window = int(cfg.get("window") or 0)

    # -- helpers -----------------------------------------------------------
    def _w64(self, a):
        return np.asarray(a, dtype=np.float64)

    def _kv_rows(self, layer: int):
        """Row ranges of W_k and W_v inside the fused [q; k; v] weight."""
        q = self.hq * self.dh
        kv = self.hkv * self.dh
        wqkv = self.w["layers"][layer]["wqkv"]
        return wqkv[:q], wqkv[q:q + kv], wqkv[q + kv:q + 2 * kv]

    def new_request(self, start: int = 0) -> RequestState:
        st = RequestState(kv_begin=start, ctx_len=start, kv_pos0=start)
        for _ in range(self.L):
            st.K.append(np.zeros((0, self.hkv, self.dh), dtype=np.float32))
            st.V.append(np.zeros((0, self.hkv, self.dh), dtype=np.float32))
        return st

    # -- step 1: concat + projection + RMSNorm --------------------------------
    def context_feature(self, hidden: list) -> np.ndarray:
        """f = RMSNorm(concat_k(H_k) @ W_fc^T; gamma_fc), stored ([guide] 3.2).

        Reading: a single bias-free linear [K*d -> d]; concatenation in
        ascending target-layer order along channels.
        """
        X = np.concatenate([self._w64(h) for h in hidden], axis=1)
        u = X @ self._w64(self.w["fc"]).T
        return self.store(rmsnorm(u, self.w["fc_norm"], self.eps)), u

    # -- step 2: KV injection ---------------------------------------------------
    def inject(self, st: RequestState, hidden: list) -> dict:
        """Write the feature of new positions into every layer's K/V ([guide] 3.2).

        hidden: n_feat arrays [rows, d] for positions ctx_len .. ctx_len+rows-1.
        Reading: K = RoPE(f W_k^l, p) and V = f W_v^l with the same W_k^l, W_v^l
        the layer applies to its block rows; no bias and no extra norm.  With
        a window W, only the last W positions are kept ([repo]).
        """
        rows = hidden[0].shape[0]
        pos = np.arange(st.ctx_len, st.ctx_len + rows)
        f, u = self.context_feature(hidden)
        f64 = self._w64(f)
        ks, vs = [], []
        for l in range(self.L):
            _, wk, wv = self._kv_rows(l)
            k = (f64 @ self._w64(wk).T).reshape(rows, self.hkv, self.dh)
            v = (f64 @ self._w64(wv).T).reshape(rows, self.hkv, self.dh)
            k = self.store(rope(k, pos, self.theta))
            v = self.store(v)
            st.K[l] = np.concatenate([st.K[l], k], axis=0)
            st.V[l] = np.concatenate([st.V[l], v], axis=0)
            ks.append(k)
            vs.append(v)
        st.ctx_len += rows
        if self.window:
            lo = max(st.kv_pos0, st.ctx_len - self.window)
            cut = lo - st.kv_pos0
            if cut > 0:
                for l in range(self.L):
                    st.K[l] = st.K[l][cut:]
                    st.V[l] = st.V[l][cut:]
                st.kv_pos0 = lo
        return dict(f=f, u=u, k=ks, v=vs, pos=pos)

    def visible(self, st: RequestState, layer: int):
        """Context K/V visible to the block: [max(kv_begin, ctx_len - W), ctx_len)."""
        lo = st.kv_begin if not self.window else max(st.kv_begin, st.ctx_len - self.window)
        cut = lo - st.kv_pos0
        return st.K[layer][cut:], st.V[layer][cut:]

    # -- steps 3-4: draft forward ----------------------------------------------
    def draft_block(self, st: RequestState, last_token: int | None = None, trace: bool = False):
        """Single-step block-diffusion draft of B positions ([guide] 3.1, 3.2, 7).

        Reading: the block is B mask-token rows at positions n .. n+B-1 with
        n = ctx_len + 1 (the pending token at ctx_len is not a draft row);
        pre-norm layers; attention of each block row over the visible context
        K/V and all B block rows; SwiGLU MLP; a draft-owned final RMSNorm
        before the shared LM head.  Returns float64 logits [B, V] and, with
        ``trace``, the residual stream before each layer and after the last.
        """
        cfg = self.cfg
        B, d, hq, hkv, dh = self.B, self.d, self.hq, self.hkv, self.dh
        n = st.ctx_len + 1
        qpos = np.arange(n, n + B)
        st_ = self.store
        conv = bool(cfg.get("conv2"))
        dyn = conv and int(cfg.get("conv_rank") or 0) > 0
        e_prev = None
        if conv:
            if last_token is None:
                raise ValueError("the conv variant needs the last verified token")
            e_prev = self._w64(self.w["embed"][int(last_token)])

        h = np.repeat(self._w64(self.w["embed"][cfg["mask_id"]])[None, :], B, axis=0)
        hs = [h.copy()] if trace else None
        for l in range(self.L):
            lw = self.w["layers"][l]
            wq, wk, wv = self._kv_rows(l)
            x = rmsnorm(h, lw["attn_norm"], self.eps)
            if dyn:  # the stored normed rows are the taps' source and the conv's input
                xs = self._w64(st_(x))
                ta, tb = dynamic_taps(xs, lw["dconv_d"][0], lw["dconv_u"][0], lw["conv"][0])
                x = dynamic_conv(xs, ta, tb, e_prev)
            elif conv:
                x = two_tap_conv(x, lw["conv"][0], e_prev)
            a = self._w64(st_(x))
            q = st_(rope((a @ self._w64(wq).T).reshape(B, hq, dh), qpos, self.theta))
            kb = st_(rope((a @ self._w64(wk).T).reshape(B, hkv, dh), qpos, self.theta))
            vb = st_((a @ self._w64(wv).T).reshape(B, hkv, dh))
            kc, vc = self.visible(st, l)
            o = attention(q, np.concatenate([kc, kb], 0), np.concatenate([vc, vb], 0))
            o = self._w64(st_(o.reshape(B, hq * dh)))
            y = o @ self._w64(lw["wo"]).T
            if dyn:
                ta, tb = dynamic_taps(y, lw["dconv_d"][1], lw["dconv_u"][1], lw["conv"][1])
                y = dynamic_conv(y, ta, tb, e_prev)
            elif conv:
                y = two_tap_conv(y, lw["conv"][1], e_prev)
            h = h + y
            x = rmsnorm(h, lw["mlp_norm"], self.eps)
            if dyn:
                xs = self._w64(st_(x))
                ta, tb = dynamic_taps(xs, lw["dconv_d"][2], lw["dconv_u"][2], lw["conv"][2])
                x = dynamic_conv(xs, ta, tb, e_prev)
            elif conv:
                x = two_tap_conv(x, lw["conv"][2], e_prev)
            m = self._w64(st_(x))
            wg = self._w64(lw["wgateup"][: self.F])
            wu = self._w64(lw["wgateup"][self.F:])
            z = self._w64(st_(swiglu(m @ wg.T, m @ wu.T)))
            y = z @ self._w64(lw["wdown"]).T
            if dyn:
                ta, tb = dynamic_taps(y, lw["dconv_d"][3], lw["dconv_u"][3], lw["conv"][3])
                y = dynamic_conv(y, ta, tb, e_prev)
            elif conv:
                y = two_tap_conv(y, lw["conv"][3], e_prev)
            h = h + y
            if trace:
                hs.append(h.copy())
        hn = self._w64(st_(rmsnorm(h, self.w["final_norm"], self.eps)))
        logits = self.lm_head(hn)
        return (logits, hs) if trace else logits

    def lm_head(self, hn: np.ndarray, chunk: int = 16384) -> np.ndarray:
        """Shared LM head hn @ E_lm^T in float64, one vocabulary chunk at a time."""
        V = self.w["lm_head"].shape[0]
        out = np.empty((hn.shape[0], V), dtype=np.float64)
        for c0 in range(0, V, chunk):
            out[:, c0:c0 + chunk] = hn @ self._w64(self.w["lm_head"][c0:c0 + chunk]).T
        return out
