"""Tiny fp32 end-to-end: speculative decoding with the GPU draft equals plain
greedy decoding of the same target (the lossless property), and every block
the GPU drafts agrees with the oracle's (lock step)."""
import numpy as np
import pytest
import torch

import synth
from helpers import assert_rows_close, assert_tokens_match
from oracle import DraftOracle, OracleDrafter, TinyTarget, greedy_ar, spec_generate, verify_accept

pytestmark = pytest.mark.gpu


class GpuDrafter:
    def __init__(self, dr):
        self.dr = dr
        self.dev = dr.dev
        self.dr.bind(0, list(range(dr.cfg.max_pages_per_req)))

    def inject(self, feats):
        hidden = [torch.from_numpy(np.ascontiguousarray(f, np.float32)).to(self.dev) for f in feats]
        self.dr.inject([0], [feats[0].shape[0]], hidden)

    def draft(self, last_token, debug_logits=None):
        d = self.dr.draft([0], debug_logits=debug_logits)
        return d.cpu().numpy()[0]

    def verify(self, d, G):
        dt = torch.tensor([list(d)], dtype=torch.int32, device=self.dev)
        gt = torch.tensor([list(G)], dtype=torch.int32, device=self.dev)
        acc, com, last = self.dr.verify(dt, gt)
        a = int(acc.cpu()[0])
        return a, [int(x) for x in com.cpu().numpy()[0, :a + 1]], int(last.cpu()[0])


class Lockstep:
    """Drives the GPU and the oracle drafter together; continues with the oracle's block."""

    def __init__(self, gpu, ref):
        self.gpu, self.ref = gpu, ref
        self.blocks = 0
        self.exempt = 0

    def inject(self, feats):
        self.gpu.inject(feats)
        self.ref.inject(feats)

    def draft(self, last_token):
        V = self.ref.o.cfg["vocab"]
        B = self.ref.o.cfg["block_size"]
        lg = torch.empty((1, B, V), dtype=torch.float32, device=self.gpu.dev)
        g = self.gpu.draft(last_token, debug_logits=lg)
        ref_logits = self.ref.o.draft_block(self.ref.st, last_token)
        assert_rows_close(lg.cpu().numpy()[0], ref_logits, what=f"logits block {self.blocks}")
        self.exempt += assert_tokens_match(g, ref_logits, what=f"block {self.blocks}")
        self.blocks += 1
        return np.argmax(ref_logits, axis=-1)

    def verify(self, d, G):
        got = self.gpu.verify(d, G)
        assert got == verify_accept(d, G)
        return got


@pytest.fixture(scope="module")
def tiny():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.config("tiny")
    tw = synth.tiny_target_weights(cfg)
    dw = synth.make_weights(cfg, shared=tw)
    target = TinyTarget(cfg, tw, cfg["feat_layers"])
    prm = synth.prompt(cfg)
    ref = greedy_ar(target, prm, cfg["new_tokens"])
    return cfg, dw, target, prm, ref


def _gpu(cfg, dw):
    from block_diffusion_drafter_proj_amd.drafter import Drafter
    return Drafter(cfg, dw, max_batch=1, max_pages=16, max_position=256, max_inject_rows=64)


def test_tiny_speculative_equals_greedy(tiny):
    cfg, dw, target, prm, ref = tiny
    out = spec_generate(target, GpuDrafter(_gpu(cfg, dw)), prm, cfg["new_tokens"], cfg["block_size"])
    assert out == ref


def test_tiny_lockstep_with_oracle(tiny):
    cfg, dw, target, prm, ref = tiny
    ls = Lockstep(GpuDrafter(_gpu(cfg, dw)), OracleDrafter(DraftOracle(cfg, dw)))
    out = spec_generate(target, ls, prm, cfg["new_tokens"], cfg["block_size"])
    assert out == ref
    assert ls.blocks > 0
    print(f"tiny: {ls.blocks} blocks, {ls.exempt} near-tie positions", flush=True)
