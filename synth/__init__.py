"""Seeded synthetic inputs for the DFlash drafting hot path.

This module only draws random numbers and names workload shapes.  It holds
none of the drafting arithmetic, so both the CPU oracle and the GPU path can
be fed from it without sharing any of the method.

Every stream is ``numpy.random.default_rng([seed, stream, *keys])``.  Values
meant to be stored in bfloat16 are rounded with torch's CPU conversion (a
library routine) and handed out as float32 arrays that hold bf16 values
exactly.

Workload shapes follow the DFlash guide (txtmix.com, section 3.1: block 16,
10 for LLaMA-3.1; 5 draft layers, 8 for the coder draft; shared embedding and
LM head) and the five workloads this project measures:

* ``tiny``          fp32, 2-layer draft over a 4-layer random decoder target.
* ``qwen3_8b``      Qwen3-8B-shaped draft, bf16, batch 1, ctx 4096, block 16.
* ``llama31_8b``    LLaMA-3.1-8B-shaped draft, bf16, batch 1, ctx 8192, block 10.
* ``coder_b64``     8-layer Qwen3-8B-shaped draft, 64 ragged requests.
* ``dflash2_long``  qwen3_8b + two-tap conv + top-16, ctx 32768, window 4096.
* ``dflash2_dyn``   dflash2_long with dynamic conv taps of rank 64.

The ``small_*`` shapes are parity cases: small enough for the oracle to finish
in seconds, ragged enough (vocab, context, block) to leave partial tiles.
"""
from __future__ import annotations

import copy
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream ids
S_WEIGHTS = 0
S_HIDDEN = 1
S_ACCEPT = 2
S_CTXLEN = 3
S_PAGES = 4
S_PROMPT = 5
S_TARGET = 6

_BASE = dict(
    hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
    vocab=151936, n_layers=5, block_size=16, n_feat=5, dtype="bf16",
    rope_theta=1.0e6, rms_eps=1.0e-6, window=0, conv2=0, topk=0, selector_rank=0,
    batch=1, ctx=4096, ctx_range=None, target_layers=36, page_size=16,
    seed=2, weight_bits=16, conv_rank=0,
)

CONFIGS = {
    "tiny": dict(
        hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=1024,
        vocab=1024, n_layers=2, block_size=8, n_feat=2, dtype="f32",
        rope_theta=1.0e4, rms_eps=1.0e-6, ctx=64, target_layers=4,
        feat_layers=[1, 2], new_tokens=64, seed=1,
    ),
    "qwen3_8b": dict(seed=2),
    "llama31_8b": dict(
        ffn=14336, vocab=128256, block_size=10, rope_theta=5.0e5,
        rms_eps=1.0e-5, ctx=8192, target_layers=32, seed=3,
    ),
    "coder_b64": dict(
        n_layers=8, batch=64, ctx=None, ctx_range=(512, 8192), seed=4,
    ),
    "qwen3_8b_q4": dict(weight_bits=4, seed=2),
    "dflash2_dyn": dict(
        conv2=1, conv_rank=64, topk=16, ctx=32768, window=4096, batch=4, seed=6, selector_rank=256,
    ),
    "dflash2_long": dict(
        conv2=1, topk=16, ctx=32768, window=4096, batch=4, seed=5, selector_rank=256,
    ),
    # parity cases
    "small_bf16": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=2, ctx=300, target_layers=36, seed=11,
    ),
    "small_block10": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=2053, n_layers=2, block_size=10, ctx=271, rope_theta=5.0e5,
        rms_eps=1.0e-5, target_layers=32, seed=12,
    ),
    "small_batch": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=2, batch=5, ctx=None, ctx_range=(17, 700),
        seed=13,
    ),
    "small_dh64": dict(
        hidden=768, n_q_heads=12, n_kv_heads=4, head_dim=64, ffn=2048,
        vocab=1500, n_layers=2, ctx=129, seed=14,
    ),
    "small_window": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=2, window=128, batch=2, ctx=None,
        ctx_range=(150, 420), seed=16,
    ),
    "small_target": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=6, block_size=17, target=1, seed=17,
    ),
    "small_dconv": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=2, conv2=1, conv_rank=32, topk=16, window=128, batch=2,
        ctx=500, seed=19,
    ),
    "small_q4": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=2, batch=3, ctx=None, ctx_range=(40, 400), weight_bits=4,
        seed=18,
    ),
    "small_conv": dict(
        hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1536,
        vocab=3001, n_layers=2, conv2=1, topk=16, window=128, batch=2,
        ctx=500, seed=15, selector_rank=64, sel_std=0.3,
    ),
}


def config(name: str, **over) -> dict:
    """Return the full shape dictionary of a named workload."""
    cfg = copy.deepcopy(_BASE)
    cfg.update(copy.deepcopy(CONFIGS[name]))
    cfg.update(over)
    cfg["name"] = name
    if "feat_layers" not in cfg:
        cfg["feat_layers"] = None
    cfg["mask_id"] = cfg.get("mask_id", cfg["vocab"] - 1)
    return cfg


def rng(seed: int, stream: int, *keys: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)] + [int(k) for k in keys])


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype with torch's CPU conversion."""
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    t = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)
    return t.numpy()


_CHUNK = 1 << 24


def _normal(seed, stream, keys, shape, std, mean=0.0):
    """N(mean, std) float32 of ``shape`` drawn in fixed 16M-value chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    chunks = [(i, min(_CHUNK, n - i * _CHUNK)) for i in range((n + _CHUNK - 1) // _CHUNK)]

    def fill(arg):
        ci, cnt = arg
        g = rng(seed, stream, *keys, ci)
        seg = out[ci * _CHUNK: ci * _CHUNK + cnt]
        g.standard_normal(cnt, dtype=np.float32, out=seg)
        seg *= np.float32(std)
        if mean:
            seg += np.float32(mean)

    if len(chunks) > 1:
        with ThreadPoolExecutor(16) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out.reshape(shape)


# tensor ids for weight streams
_TID = dict(embed=0, lm_head=1, fc=2, fc_norm=3, final_norm=4, wqkv=10,
            wo=11, wgateup=12, wdown=13, attn_norm=14, mlp_norm=15, conv=16, sel_u=20, sel_v=21,
            dconv_d=22, dconv_u=23)


def make_weights(cfg: dict, seed: int | None = None, norm_std: float = 0.0,
                 shared: dict | None = None) -> dict:
    """Random-init draft weights in torch Linear layout ([out, in], row-major).

    ``shared`` (a target's weights) supplies ``embed`` and ``lm_head`` when
    the draft shares them with a concrete target, as in the tiny workload.

    Every matrix is N(0, 0.02).  RMSNorm gains are 1 (``norm_std`` > 0 draws
    them as 1 + N(0, norm_std) instead, to make the gain visible in tests).
    Conv taps (when ``conv2``) are w0 = 1 + N(0, 0.02), w1 = N(0, 0.02);
    with ``conv_rank`` r the dynamic taps' forms D ([4, r, d]) and U
    ([4, 2d, r]) are N(0, 0.02).
    The path selector's forms (when ``selector_rank``) are [r, d] matrices of
    N(0, cfg["sel_std"]) (0.02 unless the shape says otherwise).
    """
    seed = cfg["seed"] if seed is None else seed
    d, hq, hkv, dh = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    F, V, L, K = cfg["ffn"], cfg["vocab"], cfg["n_layers"], cfg["n_feat"]
    dt = cfg["dtype"]

    def mat(name, shape, layer=0):
        return to_storage(_normal(seed, S_WEIGHTS, (_TID[name], layer), shape, 0.02), dt)

    def gain(name, layer=0):
        if norm_std > 0:
            return to_storage(_normal(seed, S_WEIGHTS, (_TID[name], layer), (d,), norm_std, 1.0), dt)
        return np.ones(d, dtype=np.float32)

    w = dict(
        embed=shared["embed"] if shared else mat("embed", (V, d)),
        lm_head=shared["lm_head"] if shared else mat("lm_head", (V, d)),
        fc=mat("fc", (d, K * d)),
        fc_norm=gain("fc_norm"),
        final_norm=gain("final_norm"),
        layers=[],
    )
    for l in range(L):
        lw = dict(
            wqkv=mat("wqkv", ((hq + 2 * hkv) * dh, d), l),
            wo=mat("wo", (d, hq * dh), l),
            wgateup=mat("wgateup", (2 * F, d), l),
            wdown=mat("wdown", (d, F), l),
            attn_norm=gain("attn_norm", l),
            mlp_norm=gain("mlp_norm", l),
        )
        if cfg.get("conv2"):
            c = _normal(seed, S_WEIGHTS, (_TID["conv"], l), (4, 2, d), 0.02)
            c[:, 0, :] += 1.0
            lw["conv"] = to_storage(c, dt)
            r = int(cfg.get("conv_rank") or 0)
            if r:  # dynamic taps: D [4, r, d], U [4, 2d, r]
                lw["dconv_d"] = to_storage(_normal(seed, S_WEIGHTS, (_TID["dconv_d"], l), (4, r, d), 0.02), dt)
                lw["dconv_u"] = to_storage(_normal(seed, S_WEIGHTS, (_TID["dconv_u"], l), (4, 2 * d, r), 0.02), dt)
        w["layers"].append(lw)
    r = int(cfg.get("selector_rank") or 0)
    if r:
        sd = float(cfg.get("sel_std", 0.02))
        w["sel_u"] = to_storage(_normal(seed, S_WEIGHTS, (_TID["sel_u"], 0), (r, d), sd), dt)
        w["sel_v"] = to_storage(_normal(seed, S_WEIGHTS, (_TID["sel_v"], 0), (r, d), sd), dt)
    return w


def context_kv(cfg: dict, req: int, layer: int, count: int):
    """Synthetic cached K and V of a target's first ``count`` positions for
    one request and layer: two arrays [count, Hkv, dh] of N(0, 1) values in
    the storage dtype (stands in for a prefill that is not recomputed)."""
    g = rng(cfg["seed"], S_TARGET, 61, req, layer)
    shp = (count, cfg["n_kv_heads"], cfg["head_dim"])
    k = g.standard_normal(shp, dtype=np.float32)
    v = g.standard_normal(shp, dtype=np.float32)
    return to_storage(k, cfg["dtype"]), to_storage(v, cfg["dtype"])


def target_weights_device(cfg: dict, n_layers: int, device) -> dict:
    """Random-init target decoder of the shape's dimensions and ``n_layers``
    layers, drawn by torch's generator on ``device`` (a 36-layer 8B-shaped
    target is ~8.2 G values, too many to draw on the host): every matrix
    N(0, 0.02) in the storage dtype, all gains 1, untied embedding and LM
    head.  Same (seed, n_layers) always gives the same weights."""
    import torch

    d, hq, hkv, dh = cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    F, V = cfg["ffn"], cfg["vocab"]
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    g = torch.Generator(device=device)

    def mat(tid, shape, layer=0):
        g.manual_seed(int(rng(cfg["seed"], S_TARGET, 71, tid, layer).integers(1 << 62)))
        t = torch.empty(shape, dtype=dt, device=device)
        rows = max(1, (1 << 26) // shape[1])
        for r0 in range(0, shape[0], rows):  # fp32 draws in slices of <= 64 M values
            blk = t[r0:r0 + rows]
            blk.copy_(torch.randn(blk.shape, generator=g, device=device, dtype=torch.float32) * 0.02)
        return t

    def ones():
        return torch.ones(d, dtype=dt, device=device)

    w = dict(embed=mat(0, (V, d)), lm_head=mat(1, (V, d)), final_norm=ones(), layers=[])
    for l in range(n_layers):
        w["layers"].append(dict(
            wqkv=mat(10, ((hq + 2 * hkv) * dh, d), l), wo=mat(11, (d, hq * dh), l),
            wgateup=mat(12, (2 * F, d), l), wdown=mat(13, (d, F), l),
            attn_norm=ones(), mlp_norm=ones()))
    return w


def uniforms(cfg: dict, shape, key: int = 0) -> np.ndarray:
    """Uniform numbers in [0, 1) (float32) for the sampled draws."""
    g = rng(cfg["seed"], S_TARGET, 41, key)
    return g.random(shape, dtype=np.float32)


def target_logits_near(cfg: dict, ids: np.ndarray, lg: np.ndarray, key: int = 0, scale: float = 2.0,
                       agree: float = 1.0) -> np.ndarray:
    """Synthetic target logits [n, B+1, V] (float32) for sampled
    verification: N(0, scale) everywhere, plus ``agree`` times the draft's
    own logits at its top-16 candidates of positions 0..B-1, so the target
    and the draft partly agree and acceptance is neither certain nor rare."""
    n, B, K = ids.shape
    g = rng(cfg["seed"], S_TARGET, 51, key)
    t = g.standard_normal((n, B + 1, cfg["vocab"]), dtype=np.float32) * np.float32(scale)
    for r in range(n):
        for i in range(B):
            t[r, i, ids[r, i]] += np.float32(agree) * lg[r, i]
    return t


def candidate_lists(cfg: dict, n_req: int, key: int = 0):
    """Synthetic top-16 lists for the path selector: per request and block
    position 16 distinct token ids and logits sorted descending, N(0, 2)."""
    g = rng(cfg["seed"], S_TARGET, 31, key)
    B, V = cfg["block_size"], cfg["vocab"]
    ids = np.stack([np.stack([g.choice(V, size=16, replace=False) for _ in range(B)]) for _ in range(n_req)])
    lg = -np.sort(-g.standard_normal((n_req, B, 16)) * 2.0, axis=-1)
    return ids.astype(np.int32), lg.astype(np.float32)


def context_lengths(cfg: dict) -> list[int]:
    """Per-request context length (number of injected positions)."""
    if cfg.get("ctx_range"):
        lo, hi = cfg["ctx_range"]
        g = rng(cfg["seed"], S_CTXLEN)
        return [int(x) for x in g.integers(lo, hi + 1, size=cfg["batch"])]
    return [int(cfg["ctx"])] * cfg["batch"]


def hidden_rows(cfg: dict, req: int, start: int, count: int) -> list[np.ndarray]:
    """Synthetic target hidden states for positions [start, start+count).

    Returns ``n_feat`` arrays [count, d] of N(0,1) values in the storage
    dtype.  Rows are keyed by (request, position block of 256) so a position
    always gets the same values however the rows are chunked.
    """
    d, K = cfg["hidden"], cfg["n_feat"]
    out = [np.empty((count, d), dtype=np.float32) for _ in range(K)]
    p = start
    while p < start + count:
        blk = p // 256
        lo = blk * 256
        take = min(start + count, lo + 256) - p
        for k in range(K):
            g = rng(cfg["seed"], S_HIDDEN, req, k, blk)
            full = g.standard_normal((256, d), dtype=np.float32)
            out[k][p - start: p - start + take] = full[p - lo: p - lo + take]
        p += take
    return [to_storage(o, cfg["dtype"]) for o in out]


def hidden_rows_device(cfg: dict, req: int, start: int, count: int, device) -> list:
    """The distribution of ``hidden_rows`` (N(0,1) in the storage dtype) drawn
    by torch's generator on ``device``, for batched workloads too large to
    draw on the host (64 requests x ~4.5K positions x 5 features x 4096).

    Values differ from ``hidden_rows``; the same (seed, req, start, count)
    always gives the same rows.  Returns ``n_feat`` device tensors [count, d].
    """
    import torch

    seed = int(rng(cfg["seed"], S_HIDDEN, req, start, count).integers(1 << 62))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    dt = torch.bfloat16 if cfg["dtype"] == "bf16" else torch.float32
    return [torch.randn((count, cfg["hidden"]), generator=g, device=device, dtype=torch.float32).to(dt)
            for _ in range(cfg["n_feat"])]


def page_permutation(cfg: dict, n_pages_total: int) -> np.ndarray:
    """A seeded random permutation of the physical KV page pool."""
    return rng(cfg["seed"], S_PAGES).permutation(n_pages_total).astype(np.int32)


def accept_schedule(cfg: dict, n_cycles: int, req: int = 0) -> np.ndarray:
    """Prescribed accept length a* ~ U{1..B} per cycle."""
    B = cfg["block_size"]
    return rng(cfg["seed"], S_ACCEPT, req, 0).integers(1, B + 1, size=n_cycles)


def synthetic_greedy(draft: np.ndarray, a_star: int, vocab: int, g: np.random.Generator) -> np.ndarray:
    """Target greedy tokens G[0..B] that agree with ``draft`` on exactly a* leading positions.

    G[i] = draft[i] for i < a*; G[a*] differs from draft[a*] (when a* < B);
    every later entry is uniform over the vocabulary.
    """
    B = len(draft)
    G = g.integers(0, vocab, size=B + 1).astype(np.int64)
    G[:a_star] = draft[:a_star]
    if a_star < B:
        r = int(g.integers(0, vocab - 1))
        G[a_star] = (int(draft[a_star]) + 1 + r) % vocab
    return G.astype(np.int32)


def prompt(cfg: dict) -> np.ndarray:
    """Uniform-random prompt ids for the tiny end-to-end workload."""
    return rng(cfg["seed"], S_PROMPT).integers(0, cfg["vocab"], size=cfg["ctx"]).astype(np.int64)


def tiny_target_weights(cfg: dict) -> dict:
    """Random-init 4-layer decoder used as the target of the tiny workload.

    d 256, 4 heads (MHA), head_dim 64, SwiGLU 1024, vocab 1024, untied
    embedding / LM head, every matrix N(0, 0.02), all gains 1.  The draft
    shares ``embed`` and ``lm_head`` with it.
    """
    seed = cfg["seed"]
    d, h, dh, F, V = cfg["hidden"], cfg["n_q_heads"], cfg["head_dim"], cfg["ffn"], cfg["vocab"]

    def mat(tid, shape, layer=0):
        return _normal(seed, S_TARGET, (tid, layer), shape, 0.02)

    w = dict(embed=mat(0, (V, d)), lm_head=mat(1, (V, d)),
             final_norm=np.ones(d, np.float32), layers=[])
    for l in range(cfg["target_layers"]):
        w["layers"].append(dict(
            wq=mat(10, (h * dh, d), l), wk=mat(11, (h * dh, d), l),
            wv=mat(12, (h * dh, d), l), wo=mat(13, (d, h * dh), l),
            wgate=mat(14, (F, d), l), wup=mat(15, (F, d), l),
            wdown=mat(16, (d, F), l),
            attn_norm=np.ones(d, np.float32), mlp_norm=np.ones(d, np.float32),
        ))
    return w
