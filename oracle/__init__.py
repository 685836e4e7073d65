"""Plain CPU oracle for the DFlash drafting hot path (test infrastructure).

This package is the independent reference that the GPU path is checked
against.  It is slow on purpose: numpy only, float64 arithmetic, one step
per line of the method, no blocking or fusion.  It shares no code with the
HIP library and imports nothing from it.

Only the test suite, the package smoke check and the CPU-baseline leg of the
benchmark may import it.  The product path never routes through it.

Parity status per function (what pins it, see ``tests/test_oracle_*.py``):

* ``to_bf16``          pinned: equals torch's CPU bfloat16 conversion.
* ``feature_layers``   pinned: the layer rule's arithmetic for 32/36 layers.
* ``rmsnorm``          pinned: torch ``F.rms_norm`` in float64.
* ``rope``             pinned: complex multiplication by exp(i*theta*p);
                       relative-position property.
* ``attention``        pinned: torch ``scaled_dot_product_attention``
                       (float64, explicit mask, repeated KV heads).
* ``swiglu``           pinned: torch ``F.silu``.
* ``select``           pinned: ``np.argsort(kind="stable")`` / brute force.
* ``verify_accept``    pinned: the 8-drafted / 6-matched example; brute force
                       over all tiny (d, G).
* ``per_token_cost``   pinned: (3+20)/6 and (3+20)/2 from the cost example.
* ``DraftOracle``      composition of the above; the whole draft forward's
                       values are "parity unpinned" by the pages (they print
                       no activation or token for any weights) and are pinned
                       through the decomposition and invariants: batch /
                       window / conv-identity / GQA-to-MHA reductions.
* ``spec_generate``    pinned: equals ``greedy_ar`` exactly (lossless).
* ``dflash2.select_path`` (DFlash-2 path selector) pinned: zero bilinear form
                       gives the argmax chain; a hand-worked 3-position case
                       with an asymmetric form; per-position logit shifts.
* ``dflash2.warp_sorted``, ``draft_sample``, ``spec_verify_sample`` (sampled
                       drafting, rejection-sampling verification) pinned:
                       hand-worked temperature / top-k / top-p warps; Monte
                       Carlo: the first committed token follows the target's
                       distribution and the first draft is accepted with
                       probability sum min(p, q); a draft equal to the target
                       is always accepted; near-zero temperature reduces to
                       greedy verification.
* ``target.TargetOracle`` (target verify forward) pinned: equals the tiny
                       target row by row (fp32, MHA); causal; chunked equals
                       one block; GQA equals MHA with repeated K/V heads.
* ``dynamic_taps``, ``dynamic_conv`` (the DFlash-2 conv's dynamic taps)
                       pinned: a small case worked by hand; identity static
                       taps with a zero form equal the draft without conv;
                       a row's source moves only its own and the next row's
                       output; the reading's parameter count against the
                       page's 16.5 M.
* ``quant.quantize_q4``, ``dequantize_q4``, ``q4_draft_weights`` (4-bit draft
                       weights) pinned: weights already on a 4-bit grid come
                       back exactly (codes, scales, biases and values); a
                       constant group; the error bound of a half step on
                       random weights; a draft whose weights lie on the grid
                       drafts exactly as the unquantised draft.
"""
from .dflash_oracle import (  # noqa: F401
    DraftOracle,
    RequestState,
    attention,
    dynamic_conv,
    dynamic_taps,
    feature_layers,
    per_token_cost,
    rmsnorm,
    rope,
    select,
    swiglu,
    to_bf16,
    to_f32,
    verify_accept,
)
from .dflash2 import (  # noqa: F401
    draft_sample,
    pair_scores,
    select_path,
    selector_vectors,
    spec_verify_sample,
    target_distribution,
    warp_sorted,
)
from .quant import dequantize_q4, q4_draft_weights, quantize_q4  # noqa: F401
from .target import TargetOracle  # noqa: F401
from .tiny_target import OracleDrafter, TinyTarget, greedy_ar, spec_generate  # noqa: F401
