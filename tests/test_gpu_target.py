"""Target verify forward on the GPU against the oracle (needs an MI355X).

[guide] section 4: the target runs once over the context plus the drafted
block and checks every drafted token; its feature layers feed the draft.

* Parity (small GQA target, 6 layers, bf16): prompts prefilled in chunks of
  up to 17 rows, then a 17-row verify call; per call the logits (row bar),
  the feature layers, the greedy tokens (exact outside near ties) and the K/V
  appended to the pages match the oracle.  Before every call the oracle's K/V
  are written into the pages (teacher forcing), so each call is compared on
  identical inputs.  A rollback of the context length makes the next call
  overwrite the rolled-back positions.
* End to end (the tiny fp32 workload): the whole speculative loop on the GPU
  - target prefill, feature injection, draft, target verify of
  [pending, drafts], acceptance, injection of the accepted rows' features,
  target rollback - commits exactly the oracle target's greedy decoding.
"""
import numpy as np
import pytest
import torch

import synth
from helpers import assert_rows_close, assert_tokens_match, unpack_kv, write_kv
from oracle import greedy_ar, TinyTarget, verify_accept
from oracle.target import TargetOracle

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda")


def _target(shape, w, n_req, max_ctx):
    from block_diffusion_drafter_proj_amd.drafter import Target

    ppr = (max_ctx + 15) // 16 + 1
    t = Target(shape, w, max_batch=n_req, max_pages=n_req * ppr + 3, max_pages_per_req=ppr,
               max_position=max_ctx + 8, poison_kv=True)
    perm = synth.page_permutation(shape, n_req * ppr + 3)
    pages = [[int(x) for x in perm[r * ppr:(r + 1) * ppr]] for r in range(n_req)]
    for r in range(n_req):
        t.bind(r, pages[r])
    return t, pages


def _force_kv(t, shape, pages, caches, n_req):
    view = t.kv_view()
    for r in range(n_req):
        n = len(caches[r][0]["k"])
        if n == 0:
            continue
        for l in range(shape["n_layers"]):
            write_kv(view, l, pages[r], list(range(n)), np.stack(caches[r][l]["k"]), np.stack(caches[r][l]["v"]))
    torch.cuda.synchronize()


@pytest.mark.parametrize("n_req", [1, 3])
def test_target_forward_parity(n_req):
    dev = _dev()
    shape = synth.config("small_target")
    w = synth.make_weights(shape, norm_std=0.1)
    V, d, L = shape["vocab"], shape["hidden"], shape["n_layers"]
    feats = [1, 3]
    t, pages = _target(shape, w, n_req, 128)
    o = TargetOracle(shape, w)
    caches = [o.new_cache() for _ in range(n_req)]
    rng = np.random.default_rng(20 + n_req)
    exempt = 0
    for call, R in enumerate([17, 17, 17, 12, 1, 17]):
        toks = rng.integers(0, V, size=(n_req, R)).astype(np.int32)
        _force_kv(t, shape, pages, caches, n_req)
        lg = torch.empty((n_req * R, V), dtype=torch.float32, device=dev)
        greedy, gf = t.forward(list(range(n_req)), R, torch.from_numpy(toks.reshape(-1)).to(dev), feats, logits=lg)
        torch.cuda.synchronize()
        g_lg = lg.cpu().numpy().reshape(n_req, R, V)
        g_greedy = greedy.cpu().numpy().reshape(n_req, R)
        view = t.kv_view()
        for r in range(n_req):
            p0 = len(caches[r][0]["k"])
            ref_lg, ref_f = o.forward(caches[r], toks[r], feats)
            assert_rows_close(g_lg[r], ref_lg, what=f"call {call} req {r} logits")
            exempt += assert_tokens_match(g_greedy[r], ref_lg, what=f"call {call} req {r} greedy")
            for l in feats:
                assert_rows_close(gf[l].float().cpu().numpy().reshape(n_req, R, d)[r], ref_f[l],
                                  what=f"call {call} req {r} feature {l}")
            for l in range(L):
                kg, vg = unpack_kv(view, l, pages[r], list(range(p0, p0 + R)))
                kr = np.stack(caches[r][l]["k"][p0:p0 + R])
                vr = np.stack(caches[r][l]["v"][p0:p0 + R])
                assert_rows_close(kg, kr, what=f"call {call} req {r} K layer {l}")
                assert_rows_close(vg, vr, what=f"call {call} req {r} V layer {l}")
            assert t.context_length(r) == p0 + R
        if call == 2:  # roll every request back by 5 positions: the next call overwrites them
            for r in range(n_req):
                n = len(caches[r][0]["k"]) - 5
                t.set_context_length(r, n)
                TargetOracle.truncate(caches[r], n)
    t.check()
    print(f"[target n_req={n_req}] near-tie greedy positions exempt: {exempt}", flush=True)


def test_speculative_loop_on_gpu_equals_greedy():
    """The tiny workload with every step on the GPU: the committed tokens
    equal the oracle target's plain greedy decoding."""
    dev = _dev()
    from block_diffusion_drafter_proj_amd.drafter import Drafter, Target

    cfg = synth.config("tiny")
    tw = synth.tiny_target_weights(cfg)
    feats = cfg["feat_layers"]
    B, V = cfg["block_size"], cfg["vocab"]
    tshape = dict(cfg, n_layers=cfg["target_layers"], n_kv_heads=cfg["n_q_heads"], target=1, block_size=64)
    twl = dict(embed=tw["embed"], lm_head=tw["lm_head"], final_norm=tw["final_norm"], layers=[
        dict(wqkv=np.concatenate([lw["wq"], lw["wk"], lw["wv"]]), wo=lw["wo"],
             wgateup=np.concatenate([lw["wgate"], lw["wup"]]), wdown=lw["wdown"],
             attn_norm=lw["attn_norm"], mlp_norm=lw["mlp_norm"]) for lw in tw["layers"]])
    tgt = Target(tshape, twl, max_batch=1, max_pages=20, max_position=300)
    tgt.bind(0, list(range(20)))
    w = synth.make_weights(cfg, shared=tw)
    dr = Drafter(cfg, w, max_batch=1, max_pages=12, max_position=300)
    dr.bind(0, list(range(12)))
    prompt = synth.prompt(cfg).astype(np.int32)
    new = cfg["new_tokens"]
    ref = greedy_ar(TinyTarget(cfg, tw, feats), prompt, new)

    g, f = tgt.forward([0], len(prompt), torch.from_numpy(prompt).to(dev), feats)
    c = int(g[-1].item())
    out = [c]
    dr.inject([0], [len(prompt)], [f[l] for l in feats])
    n = len(prompt) + 1
    cycles = 0
    while len(out) < new:
        d = dr.draft([0])  # [1, B]
        toks = torch.cat([torch.tensor([c], dtype=torch.int32, device=dev), d[0]])
        G, vf = tgt.forward([0], B + 1, toks, feats)
        acc, com, last = dr.verify(d, G[None])
        a = int(acc.item())
        ref_a, ref_com, ref_next = verify_accept(d[0].cpu().numpy(), G.cpu().numpy())
        assert a == ref_a
        out.extend(com[0, :a + 1].cpu().numpy().tolist())
        dr.inject([0], [a + 1], [vf[l][:a + 1].contiguous() for l in feats])
        tgt.set_context_length(0, n + a)
        n += a + 1
        c = int(last.item())
        cycles += 1
    out = out[:new]
    tgt.check()
    dr.check()
    mism = [i for i in range(new) if out[i] != ref[i]]
    assert not mism, f"first mismatch at {mism[0]}: gpu {out[mism[0]]} greedy {ref[mism[0]]}"
    print(f"[gpu speculative loop] {new} tokens in {cycles} cycles (mean accepted {new / cycles - 1:.2f}) "
          f"= greedy AR of the target", flush=True)


@pytest.mark.parametrize("ctxs", [[4096], [0, 77, 2049]])
def test_target_full_size(ctxs):
    """Qwen3-8B-shaped layers (hidden 4096, 32/8 heads x 128, ffn 12288,
    vocab 151936; 2 of the 36 layers, each layer's launches being the same),
    a cached context of synthetic K/V written into the pages and into the
    oracle's cache, then a 17-row verify call and a 1-row call (the
    autoregressive step): logits, greedy, both layers' features and the
    appended K/V match the oracle."""
    dev = _dev()
    from block_diffusion_drafter_proj_amd.drafter import Target

    shape = synth.config("qwen3_8b", n_layers=2, target=1, block_size=17)
    w = synth.make_weights(shape)
    V, d, L = shape["vocab"], shape["hidden"], shape["n_layers"]
    n = len(ctxs)
    ppr = (max(ctxs) + 40) // 16 + 1
    t = Target(shape, w, max_batch=n, max_pages=n * ppr, max_pages_per_req=ppr,
               max_position=max(ctxs) + 64, poison_kv=True)
    perm = synth.page_permutation(shape, n * ppr)
    pages = [[int(x) for x in perm[r * ppr:(r + 1) * ppr]] for r in range(n)]
    o = TargetOracle(shape, w)
    caches = [o.new_cache() for _ in range(n)]
    view = t.kv_view()
    for r, c in enumerate(ctxs):
        t.bind(r, pages[r])
        for l in range(L):
            K, Vv = synth.context_kv(shape, r, l, c)
            caches[r][l]["k"].extend(list(K))
            caches[r][l]["v"].extend(list(Vv))
            if c:
                write_kv(view, l, pages[r], list(range(c)), K, Vv)
        t.set_context_length(r, c)
    torch.cuda.synchronize()
    rng = np.random.default_rng(31 + n)
    exempt = 0
    for call, R in enumerate([17, 1]):
        toks = rng.integers(0, V, size=(n, R)).astype(np.int32)
        lg = torch.empty((n * R, V), dtype=torch.float32, device=dev)
        greedy, gf = t.forward(list(range(n)), R, torch.from_numpy(toks.reshape(-1)).to(dev), [0, 1], logits=lg)
        torch.cuda.synchronize()
        print(f"[target full size ctxs={ctxs}] call {call} ({R} rows) done on the GPU", flush=True)
        g_lg = lg.cpu().numpy().reshape(n, R, V)
        g_greedy = greedy.cpu().numpy().reshape(n, R)
        for r in range(n):
            p0 = len(caches[r][0]["k"])
            ref_lg, ref_f = o.forward(caches[r], toks[r], [0, 1])
            assert_rows_close(g_lg[r], ref_lg, what=f"call {call} req {r} logits")
            exempt += assert_tokens_match(g_greedy[r], ref_lg, what=f"call {call} req {r} greedy")
            for l in (0, 1):
                assert_rows_close(gf[l].float().cpu().numpy().reshape(n, R, d)[r], ref_f[l],
                                  what=f"call {call} req {r} feature {l}")
            for l in range(L):
                kg, vg = unpack_kv(view, l, pages[r], list(range(p0, p0 + R)))
                assert_rows_close(kg, np.stack(caches[r][l]["k"][p0:p0 + R]), what=f"call {call} req {r} K {l}")
                assert_rows_close(vg, np.stack(caches[r][l]["v"][p0:p0 + R]), what=f"call {call} req {r} V {l}")
    t.check()
    print(f"[target full size ctxs={ctxs}] near-tie greedy positions exempt: {exempt}", flush=True)
