"""dflash_draft_block_static (the draft entry point that allocates nothing:
its scratch lives in the library's static device array) against
dflash_draft_block (scratch in the handle's workspace), through the C ABI.

Both run the same kernels on the same rows, so drafts, top-16 lists and
debug logits must agree bit for bit.  Two calls in a row per handle, the
second with fewer requests than the first, so the second call runs on the
array that the first left behind.
"""
import numpy as np
import pytest
import torch

import synth
from block_diffusion_drafter_proj_amd import binding as B
from helpers import pages_needed

pytestmark = pytest.mark.gpu


def _handle(name, **over):
    from block_diffusion_drafter_proj_amd.drafter import Drafter

    shape = synth.config(name, **over)
    w = synth.make_weights(shape, norm_std=0.1)
    n = shape["batch"]
    ctxs = synth.context_lengths(shape)
    B_ = shape["block_size"]
    win = shape.get("window") or 0
    ppr = pages_needed(max(ctxs), 2 * B_ + 2, win)
    dr = Drafter(shape, w, max_batch=n, max_pages=n * ppr, max_pages_per_req=ppr,
                 max_position=max(ctxs) + 4 * B_ + 8, max_inject_rows=512, poison_kv=True)
    for r in range(n):
        dr.bind(r, list(range(r * ppr, (r + 1) * ppr)))
    dev = torch.device("cuda")
    H = [synth.hidden_rows(shape, r, 0, c) for r, c in enumerate(ctxs)]
    hidden = [torch.from_numpy(np.concatenate([H[r][k] for r in range(n)], 0)).to(dr.tdt).to(dev)
              for k in range(shape["n_feat"])]
    dr.inject(list(range(n)), ctxs, hidden)
    return shape, dr


def _run(dr, shape, slots, static):
    dev = torch.device("cuda")
    n, Bk, V = len(slots), shape["block_size"], shape["vocab"]
    out = torch.full((n, Bk), -7, dtype=torch.int32, device=dev)
    lg = torch.full((n, Bk, V), float("nan"), dtype=torch.float32, device=dev)
    tk_ids = tk_val = None
    if shape.get("topk"):
        tk_ids = torch.full((n, Bk, 16), -7, dtype=torch.int32, device=dev)
        tk_val = torch.full((n, Bk, 16), float("nan"), dtype=torch.float32, device=dev)
    last = None
    if shape.get("conv2"):
        last = torch.tensor([(37 * s + 5) % V for s in slots], dtype=torch.int32, device=dev)
    fn = B.dflash_draft_block_static if static else B.dflash_draft_block
    ptr = lambda t: t.data_ptr() if t is not None else 0  # noqa: E731
    fn(dr.h, dr.stream, list(slots), ptr(last), out.data_ptr(), ptr(tk_ids), ptr(tk_val),
       debug_logits=lg.data_ptr())
    torch.cuda.synchronize()
    res = [out.cpu().numpy(), lg.cpu().numpy()]
    if tk_ids is not None:
        res += [tk_ids.cpu().numpy(), tk_val.cpu().numpy()]
    return res


@pytest.mark.parametrize("name,over,calls", [
    # 80 rows (tiled GEMMs, attention split merge), then 32 rows (64-row skinny block)
    ("small_batch", {}, [[0, 1, 2, 3, 4], [3, 1]]),
    # DFlash-2 form: conv taps and top-16; 48 rows then 16 rows
    ("small_conv", {"batch": 3, "ctx": None, "ctx_range": (60, 300)}, [[0, 1, 2], [2]]),
    # batch 1 at a larger width (one 16-row block, RoPE epilogue, argmax epilogue), twice
    ("small_dh64", {}, [[0], [0]]),
], ids=["rows80_then_32", "conv_rows48_then_16", "rows16_twice"])
def test_static_scratch_equals_workspace(name, over, calls):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    shape, dr = _handle(name, **over)
    print(f"[no-alloc {name}] calls {calls}", flush=True)
    for slots in calls:
        assert 0 < B.dflash_draft_static_bytes(dr.cfg, len(slots)) <= B.DFLASH_STATIC_SCRATCH_BYTES
        ref = _run(dr, shape, slots, static=False)
        got = _run(dr, shape, slots, static=True)
        for a, b in zip(ref, got):
            np.testing.assert_array_equal(a, b)
        assert np.all(ref[0] >= 0)
    dr.check()


def test_static_scratch_rejects_oversized_calls():
    """A call whose scratch exceeds the static array is refused with
    DFLASH_E_CAPACITY before anything is enqueued; smaller calls on the same
    handle still run and equal the workspace path."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # 256 requests of a draft with a wide MLP: the SwiGLU output alone is
    # 4096 rows x 8192 x 2 bytes = 64 MiB
    shape, dr = _handle("small_bf16", batch=256, ffn=8192, ctx=None, ctx_range=(1, 8), vocab=1031)
    assert B.dflash_draft_static_bytes(dr.cfg, 256) > B.DFLASH_STATIC_SCRATCH_BYTES
    assert B.dflash_draft_static_bytes(dr.cfg, 4) <= B.DFLASH_STATIC_SCRATCH_BYTES
    out = torch.full((256, shape["block_size"]), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(B.DFlashError) as ei:
        B.dflash_draft_block_static(dr.h, dr.stream, list(range(256)), 0, out.data_ptr())
    assert ei.value.status == B.E_CAPACITY and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert torch.all(out == -7)  # nothing ran
    ref = _run(dr, shape, [5, 200, 17, 3], static=False)
    got = _run(dr, shape, [5, 200, 17, 3], static=True)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)
    dr.check()
