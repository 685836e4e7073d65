#!/usr/bin/env python
"""Throughput of the DFlash drafting hot path on one MI355X.

One step is one speculative cycle of the whole path on a batch of synthetic
input: the draft forward over a block of mask positions (steps 3-4), prefix
acceptance against synthetic target tokens (step 5), and injection of the
accepted rows' target features into the draft KV cache (steps 1-2).

Workload (default ``qwen3_8b``): Qwen3-8B-shaped 5-layer draft, bf16, hidden
4096, 32 q / 8 kv heads, head_dim 128, SwiGLU 12288, vocab 151936 shared LM
head, 5 target feature layers projected 20480 -> 4096, block 16, batch 1,
context 4096 injected positions.  Weights N(0, 0.02), target hidden states
N(0, 1), accept length per block drawn from U{1..16}.  Every input is seeded
and resident in HBM before the timed region.

Target tokens must agree with the GPU's own drafts on a prescribed prefix, so
the cycle sequence is run once untimed to record the drafts and build the
target tokens, the state is rebuilt from the same context, and the same
cycles are then timed back to back with no host synchronisation inside.

Output: one JSON line.  ``value`` is draft blocks/s of the full cycle;
accepted tok/s, the draft-only rate at fixed context, the per-kernel time
breakdown, the roofline of the dominant kernel (the LM-head GEMM, timed with
HIP events on the call's stream during the timed region) and the CPU oracle
timed on the host are reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/s + accepted tok/s, ctx4K block16 bf16; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
PROFILE_FILE = os.path.join(ROOT, "profiles", "lm_head_gemm_qwen3_8b_ctx4096.md")
GEMM_SRC = os.path.join(ROOT, "block_diffusion_drafter_proj_amd", "csrc", "gemm.hip")


def elt(shape):
    return 2 if shape["dtype"] == "bf16" else 4


def draft_bytes(shape, ctx):
    """Algorithmic HBM bytes of one draft forward of one request at context ``ctx``:
    every weight the forward multiplies once, the visible context K/V once."""
    e = elt(shape)
    d, hq, hkv, dh, F, V, L = (shape[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim",
                                                   "ffn", "vocab", "n_layers"))
    layer = (hq + 2 * hkv) * dh * d + d * hq * dh + 2 * F * d + d * F
    kv = L * ctx * 2 * hkv * dh
    return e * (L * layer + V * d + kv)


def inject_bytes(shape, rows):
    """Algorithmic bytes of injecting ``rows`` positions: W_fc and every layer's
    K/V projection once, the hidden rows in, the K/V rows out."""
    e = elt(shape)
    d, hkv, dh, L, K = (shape[k] for k in ("hidden", "n_kv_heads", "head_dim", "n_layers", "n_feat"))
    return e * (K * d * d + L * 2 * hkv * dh * d + rows * (K * d + L * 2 * hkv * dh))


def lm_head_bytes(shape, rows):
    e = elt(shape)
    return e * (shape["vocab"] * shape["hidden"] + rows * shape["hidden"])


def file_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(shape):
    """HBM bytes per LM-head launch from the committed counter summary, or None
    when it is missing or was taken from a different GEMM source."""
    if not os.path.exists(PROFILE_FILE):
        return None
    txt = open(PROFILE_FILE).read()
    m = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    s = re.search(r"gemm_source_sha256_16:\s*([0-9a-f]+)", txt)
    if not m or not s or s.group(1) != file_sha(GEMM_SRC):
        return None
    return float(m.group(1))


def cpu_baseline(shape, weights, a_mean):
    """The oracle on the host: one cycle (inject of a_mean+1 rows, one draft
    forward at the workload's context, the accept step)."""
    import synth
    from oracle import DraftOracle, select, verify_accept

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    o = DraftOracle(shape, weights)
    st = o.new_request()
    ctx = shape["ctx"]
    # the context K/V of the sample: random bf16 values of the workload's shape
    g = np.random.default_rng(7)
    for l in range(shape["n_layers"]):
        st.K[l] = synth.to_storage(g.standard_normal((ctx, shape["n_kv_heads"], shape["head_dim"]), np.float32), shape["dtype"])
        st.V[l] = synth.to_storage(g.standard_normal((ctx, shape["n_kv_heads"], shape["head_dim"]), np.float32), shape["dtype"])
    st.ctx_len = ctx
    rows = int(round(a_mean)) + 1
    H = synth.hidden_rows(shape, 0, ctx, rows)
    t0 = time.perf_counter()
    logits = o.draft_block(st)
    d, _, _ = select(logits)
    G = np.concatenate([d, [0]])
    verify_accept(d, G)
    t1 = time.perf_counter()
    o.inject(st, H)
    t2 = time.perf_counter()
    cycle = t2 - t0
    return dict(value=1.0 / cycle, unit="draft blocks/s", cores=int(threads), kind="oracle",
                sample=f"1 cycle at ctx {ctx}: draft forward {t1 - t0:.2f} s + inject of {rows} rows "
                       f"{t2 - t1:.2f} s (float64 numpy; context K/V filled with random bf16 values)",
                draft_s=t1 - t0, inject_s=t2 - t1, accepted_tok_per_s=a_mean / cycle)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="qwen3_8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the drafting path runs per request on a single "
              f"MI355X and has no multi-GPU mode (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": 1 << 30, "bytes_written": 1 << 30}))
        return

    import synth
    from block_diffusion_drafter_proj_amd import binding as Bnd
    from block_diffusion_drafter_proj_amd.drafter import Drafter

    shape = synth.config(args.config)
    assert shape["batch"] == 1 and not shape.get("ctx_range"), "bench.py runs the batch-1 workloads"
    dev = torch.device("cuda")
    t_setup = time.perf_counter()
    weights = synth.make_weights(shape)
    ctx, B, V, d = shape["ctx"], shape["block_size"], shape["vocab"], shape["hidden"]
    n_cycles = args.warmup + args.steps
    sched = synth.accept_schedule(shape, n_cycles).astype(int)
    extra = int(sched.sum()) + n_cycles
    max_pos = ctx + extra + 2 * B + 16
    pages = (max_pos + 15) // 16 + 1
    dr = Drafter(shape, weights, max_batch=1, max_pages=pages, max_pages_per_req=pages,
                 max_position=max_pos, max_inject_rows=1024)
    tdt = dr.tdt
    # all target hidden states the run needs, resident on the device
    Hall = [torch.from_numpy(h).to(tdt).to(dev) for h in synth.hidden_rows(shape, 0, 0, ctx + extra)]
    page_ids = list(range(pages))

    def reset():
        dr.bind(0, page_ids)
        dr.inject([0], [ctx], [h[:ctx] for h in Hall])

    reset()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    # ---- draft-only rate at fixed context (state is unchanged by a draft) ----
    out = torch.empty((1, B), dtype=torch.int32, device=dev)
    for _ in range(args.warmup):
        dr.draft([0], out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        dr.draft([0], out=out)
    e1.record()
    torch.cuda.synchronize()
    draft_ms = e0.elapsed_time(e1) / args.steps

    # per-kernel breakdown of the draft forward (separate pass, every class timed)
    Bnd.dflash_profile_begin(dr.h, (1 << len(Bnd.KERNELS)) - 1)
    for _ in range(5):
        dr.draft([0], out=out)
    breakdown = Bnd.dflash_profile_end(dr.h)
    breakdown = {k: round(ms / 5, 4) for k, (ms, n) in breakdown.items()}

    # ---- record pass: drafts -> target tokens with the prescribed accept lengths ----
    gen = synth.rng(shape["seed"], synth.S_ACCEPT, 1)
    Gs, starts = [], []
    pos = ctx
    for i in range(n_cycles):
        dd = dr.draft([0], out=out).cpu().numpy()[0]
        G = synth.synthetic_greedy(dd, int(sched[i]), V, gen)
        Gs.append(torch.from_numpy(G[None]).to(dev))
        a = int(sched[i])
        starts.append(pos)
        dr.inject([0], [a + 1], [h[pos:pos + a + 1] for h in Hall])
        pos += a + 1
    torch.cuda.synchronize()

    # ---- timed cycles ----
    reset()
    acc = torch.empty((n_cycles, 1), dtype=torch.int32, device=dev)
    com = torch.empty((n_cycles, 1, B + 1), dtype=torch.int32, device=dev)
    last = torch.empty((n_cycles, 1), dtype=torch.int32, device=dev)

    def cycle(i):
        dr.draft([0], out=out)
        dr.verify(out, Gs[i], acc[i], com[i], last[i])
        a = int(sched[i])
        p0 = starts[i]
        dr.inject([0], [a + 1], [h[p0:p0 + a + 1] for h in Hall])

    for i in range(args.warmup):
        cycle(i)
    torch.cuda.synchronize()
    Bnd.dflash_profile_begin(dr.h, 1 << Bnd.KERNELS.index("lm_head"))
    t0 = time.perf_counter()
    e0.record()
    for i in range(args.warmup, n_cycles):
        cycle(i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lm = Bnd.dflash_profile_end(dr.h)["lm_head"]
    dr.check()
    got = acc.cpu().numpy()[:, 0]
    assert np.array_equal(got, sched), "accept lengths differ from the schedule"
    cycle_ms = e0.elapsed_time(e1) / args.steps
    wall_ms = (t1 - t0) * 1e3 / args.steps
    acc_timed = int(sched[args.warmup:].sum())

    # ---- roofline of the dominant kernel ----
    lm_ms = lm[0] / lm[1]
    lm_bytes = lm_head_bytes(shape, B)
    achieved = lm_bytes / (lm_ms * 1e-3) / 1e9
    traffic = measured_traffic(shape)
    roofline = dict(bound="hbm", kernel="lm_head (k_gemm bf16 argmax epilogue)", achieved=round(achieved, 1),
                    peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                    traffic=traffic, algorithmic_bytes=lm_bytes, avg_ms=round(lm_ms, 4))
    db = draft_bytes(shape, ctx)
    a_mean = float(sched[args.warmup:].mean())
    cyc_bytes = draft_bytes(shape, ctx + extra // 2) + inject_bytes(shape, a_mean + 1)

    result = {
        "metric": METRIC,
        "value": round(1e3 / cycle_ms, 2),
        "unit": "draft blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {shape['n_layers']}-layer draft, hidden {d}, "
                               f"{shape['n_q_heads']}/{shape['n_kv_heads']} heads x {shape['head_dim']}, "
                               f"ffn {shape['ffn']}, vocab {V}, block {B}, ctx {ctx}, batch 1",
                   "global_batch": 1, "block": B, "ctx": ctx, "parallelism": "none (1 GPU)"},
        "accepted_tok_per_s": round(acc_timed / (cycle_ms * 1e-3 * args.steps), 1),
        "committed_tok_per_s": round((acc_timed + args.steps) / (cycle_ms * 1e-3 * args.steps), 1),
        "mean_accept": round(a_mean, 3),
        "cycle_ms_events": round(cycle_ms, 4),
        "draft_only_blocks_per_s": round(1e3 / draft_ms, 2),
        "draft_ms": round(draft_ms, 4),
        "draft_algorithmic_bytes": db,
        "draft_roofline_frac": round(db / (draft_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "cycle_roofline_frac": round(cyc_bytes / (cycle_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_ms_per_draft": breakdown,
        "roofline": roofline,
        "setup_s": round(setup_s, 1),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(shape, weights, a_mean)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
