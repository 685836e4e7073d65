"""Plain CPU oracle of the 4-bit draft weights (test infrastructure only).

Source: [guide] "DFlash：块扩散加速的 LLM 推测解码技术", section 8 (getting
started, the local MLX example): the MLX backend runs a DFlash-2 draft
quantised to 4 bits (``--draft-bits 4``), and the guide advises a block
size of at most 5 when the target or the draft is quantised, because the
quantised matmul kernels lose efficiency at wider verify widths.  The pages
give no format.

Reading taken here (the plain group-wise affine 4-bit scheme):

* Every matrix the draft owns (the context projection W_fc and, per layer,
  W_qkv, W_o, W_gate/up, W_down) is quantised along its input dimension in
  groups of 64 consecutive weights of one output row.  The shared embedding
  and LM head (the target's), the norm gains, conv taps and selector forms
  stay in the storage dtype.
* A group with smallest value lo and largest value hi keeps a scale
  s = bf16((hi - lo) / 15) and a bias b = lo (a bf16 value already); each
  weight w keeps q = clamp(round_half_even((w - b) / s), 0, 15), or q = 0
  when s = 0.  These steps run in float32 (one rounding per operation), so
  that the integer codes are a decision both sides take in the same
  precision.
* The draft computes with the dequantised weight s * q + b, exactly (no
  rounding of the weight itself): its forward is the ordinary forward with
  every quantised matrix replaced by these values.
"""
from __future__ import annotations

import numpy as np

from .dflash_oracle import to_bf16

GROUP = 64
QUANTISED = ("wqkv", "wo", "wgateup", "wdown")  # per layer, besides the top-level "fc"


def quantize_q4(w):
    """w [N, K] storage-dtype values (float32 array of bf16 values), K a
    multiple of 64 -> (q uint8 [N, K], s float32 [N, K/64], b float32 [N, K/64])."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % GROUP:
        raise ValueError("the input dimension must be a multiple of 64")
    wg = w.reshape(N, K // GROUP, GROUP)
    lo = wg.min(axis=-1)
    hi = wg.max(axis=-1)
    s = to_bf16((hi - lo) / np.float32(15.0))
    b = to_bf16(lo)
    d = wg - b[..., None]  # float32
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s[..., None] > 0, d / s[..., None], np.float32(0.0)).astype(np.float32)
    q = np.clip(np.rint(qf), 0, 15).astype(np.uint8)
    return q.reshape(N, K), s.astype(np.float32), b.astype(np.float32)


def dequantize_q4(q, s, b):
    """s * q + b per group, float64 [N, K]."""
    q = np.asarray(q, dtype=np.float64)
    N, K = q.shape
    s64 = np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=1)
    b64 = np.repeat(np.asarray(b, dtype=np.float64), GROUP, axis=1)
    return s64 * q + b64


def q4_draft_weights(w: dict) -> dict:
    """The draft's weights as the 4-bit draft computes with them: a copy of
    ``w`` whose quantised matrices are replaced by their dequantised values
    (float64); every other entry is the same object."""
    out = dict(w)
    out["fc"] = dequantize_q4(*quantize_q4(w["fc"]))
    out["layers"] = []
    for lw in w["layers"]:
        nl = dict(lw)
        for name in QUANTISED:
            nl[name] = dequantize_q4(*quantize_q4(lw[name]))
        out["layers"].append(nl)
    return out
