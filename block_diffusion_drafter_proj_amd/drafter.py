"""Torch-facing wrapper of the C ABI: owns the device buffers of one handle.

PyTorch only supplies device memory and streams here.  Every step of the
drafting path runs in libdflash.so; this class marshals tensors into the
binding calls and keeps the buffers alive.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def _dtype_code(name: str) -> int:
    return B.BF16 if name == "bf16" else B.F32


def torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def make_config(shape: dict, *, max_batch: int, max_pages: int, max_pages_per_req: int,
                max_position: int, max_inject_rows: int = 1024) -> B.DFlashConfig:
    """C config from a shape dictionary (the keys of ``synth.config``)."""
    c = B.DFlashConfig()
    c.hidden = shape["hidden"]
    c.n_q_heads = shape["n_q_heads"]
    c.n_kv_heads = shape["n_kv_heads"]
    c.head_dim = shape["head_dim"]
    c.ffn = shape["ffn"]
    c.vocab = shape["vocab"]
    c.n_layers = shape["n_layers"]
    c.block_size = shape["block_size"]
    c.n_feat = shape["n_feat"]
    c.dtype = _dtype_code(shape["dtype"])
    c.mask_token_id = shape.get("mask_id", shape["vocab"] - 1)
    c.page_size = B.PAGE
    c.window = int(shape.get("window") or 0)
    c.conv2 = int(shape.get("conv2") or 0)
    c.topk = int(shape.get("topk") or 0)
    c.max_batch = max_batch
    c.max_pages = max_pages
    c.max_pages_per_req = max_pages_per_req
    c.max_position = max_position
    c.max_inject_rows = max_inject_rows
    c.rms_eps = shape["rms_eps"]
    c.rope_theta = shape["rope_theta"]
    c.selector_rank = int(shape.get("selector_rank") or 0)
    c.target = int(shape.get("target") or 0)
    c.weight_bits = int(shape.get("weight_bits") or 16)
    c.conv_rank = int(shape.get("conv_rank") or 0) if c.conv2 else 0
    return c


class Drafter:
    """One dflash handle with its weights, KV pool and workspace on ``device``."""

    def __init__(self, shape: dict, weights: dict, *, max_batch: int = 1, max_pages: int,
                 max_pages_per_req: int | None = None, max_position: int,
                 max_inject_rows: int = 1024, device: str = "cuda", poison_kv: bool = False):
        self.shape = shape
        self.dev = torch.device(device)
        self.tdt = torch_dtype(shape["dtype"])
        self.cfg = make_config(shape, max_batch=max_batch, max_pages=max_pages,
                               max_pages_per_req=max_pages_per_req or max_pages,
                               max_position=max_position, max_inject_rows=max_inject_rows)
        B.dflash_validate_config(self.cfg)
        self._keep = []

        def up(a):
            if isinstance(a, torch.Tensor):
                t = a.to(self.dev, self.tdt).contiguous()
            else:
                t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.tdt).to(self.dev)
            self._keep.append(t)
            return t.data_ptr()

        w = B.DFlashWeights()
        w.embed = up(weights["embed"])
        w.lm_head = up(weights["lm_head"])
        if not shape.get("target"):
            w.fc = up(weights["fc"])
            w.fc_norm = up(weights["fc_norm"])
        w.final_norm = up(weights["final_norm"])
        for l, lw in enumerate(weights["layers"]):
            L = w.layers[l]
            L.wqkv = up(lw["wqkv"])
            L.wo = up(lw["wo"])
            L.wgateup = up(lw["wgateup"])
            L.wdown = up(lw["wdown"])
            L.attn_norm = up(lw["attn_norm"])
            L.mlp_norm = up(lw["mlp_norm"])
            L.conv = up(lw["conv"]) if "conv" in lw else None
            L.dconv_d = up(lw["dconv_d"]) if "dconv_d" in lw else None
            L.dconv_u = up(lw["dconv_u"]) if "dconv_u" in lw else None
        if self.cfg.selector_rank:
            w.sel_u = up(weights["sel_u"])
            w.sel_v = up(weights["sel_v"])
        self.w = w
        kvb = B.dflash_kv_pool_bytes(self.cfg)
        wsb = B.dflash_workspace_bytes(self.cfg)
        self.kv_pool = torch.empty(kvb, dtype=torch.uint8, device=self.dev)
        if poison_kv:
            self.kv_pool.fill_(0xFF)  # NaN in bf16 and fp32
        self.workspace = torch.empty(wsb, dtype=torch.uint8, device=self.dev)
        self.packed = torch.empty(B.dflash_packed_weights_bytes(self.cfg), dtype=torch.uint8, device=self.dev)
        self.h = B.dflash_create(self.cfg, self.w, self.kv_pool.data_ptr(), self.workspace.data_ptr(),
                                 self.packed.data_ptr())

    # -- helpers ------------------------------------------------------------
    @property
    def stream(self) -> int:
        return torch.cuda.current_stream(self.dev).cuda_stream

    def kv_view(self) -> torch.Tensor:
        """KV pool as [L, max_pages, 2, Hkv, 16*dh] of the storage dtype."""
        c = self.cfg
        return self.kv_pool.view(self.tdt).view(c.n_layers, c.max_pages, 2, c.n_kv_heads, 16 * c.head_dim)

    def close(self):
        if getattr(self, "h", None):
            B.dflash_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- the C entry points --------------------------------------------------
    def bind(self, slot: int, page_ids, start_pos: int = 0):
        B.dflash_bind_request(self.h, slot, list(page_ids), start_pos)

    def context_length(self, slot: int) -> int:
        return B.dflash_context_length(self.h, slot)

    def inject(self, slots, n_new, hidden, debug_f: torch.Tensor | None = None):
        """hidden: n_feat device tensors [sum(n_new), d] of the storage dtype."""
        for t in hidden:
            assert t.is_contiguous() and t.dtype == self.tdt and t.device.type == "cuda"
        B.dflash_inject_context(self.h, self.stream, list(slots), list(n_new),
                                [t.data_ptr() for t in hidden],
                                debug_f.data_ptr() if debug_f is not None else 0)

    def draft(self, slots, last_token: torch.Tensor | None = None, *, out: torch.Tensor | None = None,
              topk_ids=None, topk_logits=None, debug_logits=None, debug_hidden=None,
              hidden_in=None) -> torch.Tensor:
        n = len(slots)
        Bk = self.cfg.block_size
        if out is None:
            out = torch.empty((n, Bk), dtype=torch.int32, device=self.dev)
        ptr = lambda t: t.data_ptr() if t is not None else 0  # noqa: E731
        B.dflash_draft_block(self.h, self.stream, list(slots), ptr(last_token), out.data_ptr(),
                             ptr(topk_ids), ptr(topk_logits), ptr(debug_logits), ptr(debug_hidden),
                             ptr(hidden_in))
        return out

    def select_path(self, topk_ids: torch.Tensor, topk_logits: torch.Tensor, path=None, step_scores=None):
        """DFlash-2 path through the top-16 lists [n, B, 16] -> path [n, B]."""
        n = topk_ids.shape[0]
        path = path if path is not None else torch.empty((n, self.cfg.block_size), dtype=torch.int32,
                                                          device=self.dev)
        B.dflash_select_path(self.h, self.stream, n, topk_ids.data_ptr(), topk_logits.data_ptr(), path.data_ptr(),
                             step_scores.data_ptr() if step_scores is not None else 0)
        return path

    def draft_sample(self, sampling, topk_ids, topk_logits, uniforms, out=None):
        """Sampled drafting: one token per position from the top-16 lists."""
        n = topk_ids.shape[0]
        out = out if out is not None else torch.empty((n, self.cfg.block_size), dtype=torch.int32, device=self.dev)
        B.dflash_draft_sample(self.h, self.stream, n, sampling, topk_ids.data_ptr(), topk_logits.data_ptr(),
                              uniforms.data_ptr(), out.data_ptr())
        return out

    def verify_sample(self, sampling, draft, topk_ids, topk_logits, target_logits, uniforms):
        """Rejection-sampling verification -> (accept [n], committed [n, B+1], last [n])."""
        n = draft.shape[0]
        Bk = self.cfg.block_size
        accept = torch.empty(n, dtype=torch.int32, device=self.dev)
        committed = torch.empty((n, Bk + 1), dtype=torch.int32, device=self.dev)
        last = torch.empty(n, dtype=torch.int32, device=self.dev)
        B.dflash_verify_sample(self.h, self.stream, n, sampling, draft.data_ptr(), topk_ids.data_ptr(),
                               topk_logits.data_ptr(), target_logits.data_ptr(), uniforms.data_ptr(),
                               accept.data_ptr(), committed.data_ptr(), last.data_ptr())
        return accept, committed, last

    def verify(self, draft: torch.Tensor, greedy: torch.Tensor, accept=None, committed=None, last=None):
        n = draft.shape[0]
        Bk = self.cfg.block_size
        accept = accept if accept is not None else torch.empty(n, dtype=torch.int32, device=self.dev)
        committed = committed if committed is not None else torch.empty((n, Bk + 1), dtype=torch.int32, device=self.dev)
        last = last if last is not None else torch.empty(n, dtype=torch.int32, device=self.dev)
        B.dflash_verify_accept(self.h, self.stream, n, draft.data_ptr(), greedy.data_ptr(),
                               accept.data_ptr(), committed.data_ptr(), last.data_ptr())
        return accept, committed, last

    def check(self):
        B.dflash_check(self.h, self.stream)


class Target(Drafter):
    """A target-model handle (config ``target`` = 1): causal verify forwards
    over its own paged KV cache.  ``block_size`` of the shape is the largest
    number of rows per request of one call."""

    def forward(self, slots, n_rows: int, tokens: torch.Tensor, feat_layers=(), logits=None, greedy=None,
                feats=None):
        """tokens [len(slots) * n_rows] int32 (device) -> (greedy [rows], features {layer: [rows, d]}).
        ``greedy`` and ``feats`` may be given preallocated (at least rows long)."""
        rows = len(slots) * n_rows
        if greedy is None:
            greedy = torch.empty(rows, dtype=torch.int32, device=self.dev)
        if feats is None:
            feats = {l: torch.empty((rows, self.cfg.hidden), dtype=self.tdt, device=self.dev) for l in feat_layers}
        B.dflash_target_forward(self.h, self.stream, list(slots), n_rows, tokens.data_ptr(), greedy.data_ptr(),
                                logits.data_ptr() if logits is not None else 0, list(feat_layers),
                                [feats[l].data_ptr() for l in feat_layers])
        return greedy, feats

    def set_context_length(self, slot: int, ctx_len: int):
        B.dflash_set_context_length(self.h, self.stream, slot, ctx_len)
