"""Shared test helpers: comparison rules and GPU-side set-up from a shape dict.

Comparison rules for floating point (GPU vs the float64 oracle): per row the
relative L2 error is at most ``tol`` = 2e-2, and no element is an outlier:
|gpu - ref| <= elem_tol * (|ref| + rms(ref row)).  elem_tol is ELEM_TOL = 3e-2
for one-step and teacher-forced comparisons (f, K/V, each layer's output on
the oracle's input, logits in lock step) and FREE_ELEM_TOL = 6e-2 for whole
free-running forwards at full size, where one-ulp bf16 re-roundings cascade
through 5-8 layers.  Measured worst ratios on an MI355X: 2.2e-2 for lock-step
logits at the small shapes, 6.1e-3 for the full-size K/V and forced checks,
4.4e-2 for the full-size free-running forwards (coder_b64, 8 layers); the
conftest prints them per test.  A single wrong column or a dropped term
still shows up there when the row norm hides it.  Free-running forwards with
dynamic conv taps take FREE_ELEM_TOL_DYN = 9e-2: their taps are formed from
the conv inputs themselves (t sums d perturbed inputs), so each layer's
rounding differences also move the next taps, and the free-running divergence
at full size grows about twice as fast (worst row error 1.5e-2 against 7.9e-3
with static taps; worst element ratio 6.2e-2).  Integer outputs are
compared exactly; a draft position is exempt when the oracle's top-1 / top-2
logit margin is below 1e-2 (a near tie that fp32 rounding may flip).
"""
from __future__ import annotations

import math

import numpy as np

TOL = 2e-2
ELEM_TOL = 3e-2
FREE_ELEM_TOL = 6e-2
FREE_ELEM_TOL_DYN = 9e-2
MARGIN = 1e-2

# Worst ratios seen by assert_rows_close in the running test (conftest prints
# them per test): the row rel-L2 error and max |gpu - ref| / (|ref| + rms).
WORST = {"row": 0.0, "elem": 0.0, "elem_free": 0.0, "what": ""}


def assert_rows_close(gpu, ref, tol=TOL, what="", elem_tol=ELEM_TOL):
    g = np.asarray(gpu, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    g = g.reshape(-1, r.shape[-1])
    r = r.reshape(-1, r.shape[-1])
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    d = g - r
    rn = np.linalg.norm(d, axis=-1) / np.maximum(np.linalg.norm(r, axis=-1), 1e-30)
    rms = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    ratio = np.abs(d) / np.maximum(np.abs(r) + rms, 1e-300)
    WORST["row"] = max(WORST["row"], float(rn.max()))
    key = "elem_free" if "free" in what else "elem"
    if float(ratio.max()) > WORST[key]:
        WORST[key] = float(ratio.max())
        if key == "elem":
            WORST["what"] = what
    assert rn.max() <= tol, f"{what}: row rel-L2 error {rn.max():.3e} > {tol}"
    bad = ratio > elem_tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} elements out of tolerance, worst "
                           f"{np.max(np.abs(d) / (np.abs(r) + rms)):.3e}")


def assert_tokens_match(gpu_ids, ref_logits, what=""):
    """Exact equality of argmax ids except at near ties; returns #exempt positions."""
    from oracle import select

    ref_logits = np.asarray(ref_logits, dtype=np.float64).reshape(-1, ref_logits.shape[-1])
    d, margin, _ = select(ref_logits)
    g = np.asarray(gpu_ids).reshape(-1)
    keep = margin >= MARGIN
    mism = np.nonzero((g != d) & keep)[0]
    assert len(mism) == 0, f"{what}: token mismatch at {mism.tolist()} gpu={g[mism].tolist()} ref={d[mism].tolist()}"
    return int((~keep).sum())


def pages_needed(ctx_max: int, extra: int, window: int = 0) -> int:
    if window:
        return window // 16 + 1
    return math.ceil((ctx_max + extra) / 16) + 1


def unpack_kv(kv_view, layer: int, pages, positions, window: int = 0):
    """Gather K, V [len(positions), Hkv, dh] of one request from the paged pool.

    kv_view: [L, max_pages, 2, Hkv, 16*dh] (torch, any device).  K rows are
    stored [16][dh] per head, V transposed [dh][16].
    """
    import torch

    L, P, _, hkv, s = kv_view.shape
    dh = s // 16
    out_k, out_v = [], []
    npg = len(pages)
    for p in positions:
        lp = p // 16
        idx = lp % npg if window else lp
        pg = int(pages[idx])
        blk = kv_view[layer, pg].float().cpu()
        k = blk[0].reshape(hkv, 16, dh)[:, p % 16, :]
        v = blk[1].reshape(hkv, dh, 16)[:, :, p % 16]
        out_k.append(k.numpy())
        out_v.append(v.numpy())
    return np.stack(out_k), np.stack(out_v)


def write_kv(kv_view, layer: int, pages, positions, K, V, window: int = 0):
    """Store K, V [len(positions), Hkv, dh] of one request into the paged pool
    (teacher forcing: the GPU then drafts from exactly the oracle's cache)."""
    import torch

    L, P, _, hkv, s = kv_view.shape
    dh = s // 16
    npg = len(pages)
    by_page = {}
    for i, p in enumerate(positions):
        lp = p // 16
        idx = lp % npg if window else lp
        by_page.setdefault(int(pages[idx]), []).append((p % 16, i))
    Kt = torch.from_numpy(np.ascontiguousarray(K, np.float32))
    Vt = torch.from_numpy(np.ascontiguousarray(V, np.float32))
    for pg, items in by_page.items():
        blk = kv_view[layer, pg].float().cpu()
        kk = blk[0].reshape(hkv, 16, dh)
        vv = blk[1].reshape(hkv, dh, 16)
        for slot, i in items:
            kk[:, slot, :] = Kt[i]
            vv[:, :, slot] = Vt[i]
        kv_view[layer, pg, 0] = kk.reshape(hkv, s).to(kv_view.dtype).to(kv_view.device)
        kv_view[layer, pg, 1] = vv.reshape(hkv, s).to(kv_view.dtype).to(kv_view.device)
