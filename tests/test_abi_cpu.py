"""The C ABI without a GPU: exports, configuration checks, argument validation.

Argument validation runs on the host before any HIP call, so every error
path below is reachable here.  Handle creation does not touch the device,
which is initialised by the first call that needs it.
"""
import ctypes
import json
import os

import pytest

import synth
from block_diffusion_drafter_proj_amd import binding as B
from block_diffusion_drafter_proj_amd.drafter import make_config
from conftest import GOLDEN
from oracle import feature_layers


def _cfg(name="small_bf16", **kw):
    shape = synth.config(name)
    args = dict(max_batch=4, max_pages=64, max_pages_per_req=32, max_position=4096, max_inject_rows=256)
    args.update(kw)
    return make_config(shape, **args)


def _fake_weights(n_layers, conv=False):
    w = B.DFlashWeights()
    p = 1 << 20
    for name in ("embed", "lm_head", "fc", "fc_norm", "final_norm"):
        setattr(w, name, p)
        p += 1 << 20
    for l in range(n_layers):
        for name in ("wqkv", "wo", "wgateup", "wdown", "attn_norm", "mlp_norm"):
            setattr(w.layers[l], name, p)
            p += 1 << 20
        if conv:
            w.layers[l].conv = p
            p += 1 << 20
    return w


def test_library_exports_every_declared_function():
    L = B.lib()
    names = B.declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/dflash.h but not exported"
    assert B.dflash_abi_version() == 4


def test_feature_layers_entry_point_matches_rule():
    with open(os.path.join(GOLDEN, "feature_layers.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert B.dflash_feature_layers(c["n_target_layers"], c["k"]) == c["layers"]
    for L in range(4, 97):
        for k in (2, 3, 5):
            assert B.dflash_feature_layers(L, k) == feature_layers(L, k)
    with pytest.raises(B.DFlashError) as e:
        B.dflash_feature_layers(3, 5)
    assert e.value.status == B.E_INVALID


@pytest.mark.parametrize("name", sorted(synth.CONFIGS))
def test_every_workload_config_is_valid(name):
    shape = synth.config(name)
    cfg = make_config(shape, max_batch=shape["batch"], max_pages=1024,
                      max_pages_per_req=max(300, (shape.get("window") or 0) // 16 + 1),
                      max_position=40000)
    B.dflash_validate_config(cfg)
    assert B.dflash_workspace_bytes(cfg) > 0
    kv = B.dflash_kv_pool_bytes(cfg)
    e = 2 if shape["dtype"] == "bf16" else 4
    assert kv == shape["n_layers"] * 1024 * 2 * shape["n_kv_heads"] * 16 * shape["head_dim"] * e


@pytest.mark.parametrize("field,value", [
    ("hidden", 300), ("head_dim", 96), ("n_kv_heads", 3), ("ffn", 1000), ("n_layers", 0),
    ("n_layers", 65), ("block_size", 0), ("block_size", 17), ("target", 2), ("n_feat", 0), ("n_feat", 9),
    ("dtype", 7), ("mask_token_id", 3001), ("page_size", 32), ("window", 100), ("topk", 8),
    ("max_batch", 0), ("max_batch", 257), ("max_pages", 0), ("max_position", 3),
    ("max_inject_rows", 0), ("conv2", 2), ("weight_bits", 8), ("weight_bits", 0),
    ("conv_rank", 16), ("conv_rank", 8),
])
def test_invalid_configs_are_rejected(field, value):
    cfg = _cfg()
    setattr(cfg, field, value)
    with pytest.raises(B.DFlashError) as e:
        B.dflash_validate_config(cfg)
    assert e.value.status == B.E_INVALID
    assert B.dflash_workspace_bytes(cfg) == 0
    assert B.dflash_last_error()


def test_create_rejects_null_and_misaligned_buffers():
    cfg = _cfg()
    w = _fake_weights(cfg.n_layers)
    with pytest.raises(B.DFlashError):
        B.dflash_create(cfg, w, 0, 1 << 30, 1 << 32)
    with pytest.raises(B.DFlashError):
        B.dflash_create(cfg, w, 1 << 30, 1 << 31, 0)
    with pytest.raises(B.DFlashError):
        B.dflash_create(cfg, w, (1 << 30) + 8, 1 << 31, 1 << 32)
    w.layers[1].wo = None
    with pytest.raises(B.DFlashError) as e:
        B.dflash_create(cfg, w, 1 << 30, 1 << 31, 1 << 32)
    assert "layer 1" in str(e.value)
    cfgc = _cfg("small_conv")
    with pytest.raises(B.DFlashError):
        B.dflash_create(cfgc, _fake_weights(cfgc.n_layers, conv=False), 1 << 30, 1 << 31, 1 << 32)


def test_packed_weights_bytes():
    shape = synth.config("qwen3_8b")
    cfg = make_config(shape, max_batch=1, max_pages=300, max_pages_per_req=300, max_position=8192)
    d, F, V, L = 4096, 12288, 151936, 5
    qkv = (32 + 16) * 128
    expect = 2 * (V * d + d * 5 * d + L * (qkv * d + d * 4096 + 2 * F * d + d * F))
    assert B.dflash_packed_weights_bytes(cfg) == expect
    big = make_config(synth.config("small_bf16", hidden=8192), max_batch=1, max_pages=8,
                      max_pages_per_req=8, max_position=512)
    with pytest.raises(B.DFlashError) as e:
        B.dflash_validate_config(big)
    assert e.value.status == B.E_UNSUPPORTED


def test_q4_packed_bytes_and_rules():
    """A 4-bit draft packs its own matrices as 4-bit codes plus a (scale,
    bias) pair of bf16 per 64 inputs (0.5625 bytes per weight); the LM head
    stays bf16.  4-bit weights need a bf16 draft handle."""
    shape = synth.config("qwen3_8b_q4")
    cfg = make_config(shape, max_batch=1, max_pages=300, max_pages_per_req=300, max_position=8192)
    d, F, V, L = 4096, 12288, 151936, 5
    qkv = (32 + 16) * 128

    def q4(N, K):
        return N * K // 2 + N * (K // 64) * 4

    expect = 2 * V * d + q4(d, 5 * d) + L * (q4(qkv, d) + q4(d, 4096) + q4(2 * F, d) + q4(d, F))
    assert B.dflash_packed_weights_bytes(cfg) == expect
    for field, val in (("dtype", 1), ("target", 1)):
        c2 = make_config(shape, max_batch=1, max_pages=300, max_pages_per_req=300, max_position=8192)
        setattr(c2, field, val)
        with pytest.raises(B.DFlashError) as e:
            B.dflash_validate_config(c2)
        assert e.value.status == B.E_INVALID


@pytest.fixture()
def handle():
    cfg = _cfg()
    h = B.dflash_create(cfg, _fake_weights(cfg.n_layers), 1 << 30, 1 << 31, 1 << 32)
    yield h, cfg
    B.dflash_destroy(h)


def test_bind_validation(handle):
    h, cfg = handle
    for slot, pages, start in [(-1, [0], 0), (4, [0], 0), (0, [], 0), (0, [64], 0),
                               (0, [-1], 0), (0, list(range(33)), 0), (0, [0], -1), (0, [0], 17)]:
        with pytest.raises(B.DFlashError) as e:
            B.dflash_bind_request(h, slot, pages, start)
        assert e.value.status == B.E_INVALID
    assert B.dflash_context_length(h, 0) == -1


def test_compute_calls_validate_before_touching_the_device(handle):
    h, cfg = handle
    vp = 1 << 32
    # unbound slots, duplicate slots, bad counts
    for slots in ([0], [0, 0], [5], []):
        with pytest.raises(B.DFlashError) as e:
            B.dflash_inject_context(h, 0, slots, [1] * len(slots), [vp] * cfg.n_feat)
        assert e.value.status == B.E_INVALID
        with pytest.raises(B.DFlashError) as e:
            B.dflash_draft_block(h, 0, slots, 0, vp)
        assert e.value.status == B.E_INVALID
    with pytest.raises(B.DFlashError) as e:
        B.dflash_verify_accept(h, 0, 0, vp, vp, vp, vp, vp)
    assert e.value.status == B.E_INVALID
    with pytest.raises(B.DFlashError) as e:
        B.dflash_verify_accept(h, 0, 1, vp, 0, vp, vp, vp)
    assert e.value.status == B.E_INVALID
    with pytest.raises(B.DFlashError) as e:
        B.dflash_verify_accept(h, 0, 5, vp, vp, vp, vp, vp)
    assert e.value.status == B.E_INVALID
    # a NULL hidden pointer
    with pytest.raises(B.DFlashError):
        B.dflash_inject_context(h, 0, [0], [1], [vp] * (cfg.n_feat - 1) + [0])


def test_null_handle_is_rejected():
    lib = B.lib()
    assert lib.dflash_bind_request(None, 0, None, 0, 0) == B.E_INVALID
    assert lib.dflash_inject_context(None, None, 1, None, None, None, None) == B.E_INVALID
    assert lib.dflash_draft_block(None, None, 1, None, None, None, None, None, None) == B.E_INVALID
    assert lib.dflash_verify_accept(None, None, 1, None, None, None, None, None) == B.E_INVALID
    assert lib.dflash_check(None, None) == B.E_INVALID
    assert lib.dflash_context_length(None, 0) == -1
    out = ctypes.c_void_p()
    assert lib.dflash_create(None, None, None, None, None, ctypes.byref(out)) == B.E_INVALID


def test_profiling_calls_without_launches(handle):
    """The timing calls validate their handle and, with no launch bracketed
    in between, report no class (nothing to synchronise on)."""
    h, _ = handle
    lib = B.lib()
    assert lib.dflash_profile_begin(None, 1) == B.E_INVALID
    assert lib.dflash_profile_mask(None, 1) == B.E_INVALID
    assert lib.dflash_profile_end(None, None, None) == B.E_INVALID
    B.dflash_profile_begin(h, 1 << B.KERNELS.index("lm_head"))
    B.dflash_profile_mask(h, 0)
    B.dflash_profile_mask(h, 0xFFFFFFFF)  # bits of unknown classes are ignored
    assert B.dflash_profile_end(h) == {}


def test_selector_config_rules_and_entry_validation():
    """The path selector needs topk 16 and a rank that is a multiple of 64 up
    to 512; its entry point refuses a handle without one before any device
    work (DFLASH_E_UNSUPPORTED)."""
    for r, topk, ok in ((64, 16, True), (256, 16, True), (512, 16, True), (32, 16, False), (576, 16, False),
                        (-64, 16, False), (64, 0, False)):
        c = _cfg("small_conv", max_batch=2)
        c.selector_rank = r
        c.topk = topk
        if ok:
            B.dflash_validate_config(c)
        else:
            with pytest.raises(B.DFlashError) as e:
                B.dflash_validate_config(c)
            assert e.value.status == B.E_INVALID
    # packed bytes grow by the two fp32 [V, r] tables
    c0 = _cfg("small_conv", max_batch=2)
    c0.selector_rank = 0
    c1 = _cfg("small_conv", max_batch=2)
    c1.selector_rank = 64
    grow = B.dflash_packed_weights_bytes(c1) - B.dflash_packed_weights_bytes(c0)
    assert 2 * 3001 * 64 * 4 <= grow < 2 * 3001 * 64 * 4 + 512
    # a handle without a selector: refused on the host
    h = B.dflash_create(c0, _fake_weights(c0.n_layers, conv=True), 1 << 30, 2 << 30, 3 << 30)
    try:
        with pytest.raises(B.DFlashError) as e:
            B.dflash_select_path(h, 0, 1, 1 << 20, 1 << 20, 1 << 20)
        assert e.value.status == B.E_UNSUPPORTED
    finally:
        B.dflash_destroy(h)
    # a selector handle needs both forms
    w = _fake_weights(c1.n_layers, conv=True)
    with pytest.raises(B.DFlashError) as e:
        B.dflash_create(c1, w, 1 << 30, 2 << 30, 3 << 30)
    assert e.value.status == B.E_INVALID


def test_target_handle_rules():
    """A target handle takes up to 64 rows per request and none of the draft's
    extras; draft entry points refuse it and the target forward refuses a
    draft handle, before any device work."""
    c = _cfg("small_target", max_batch=2)
    B.dflash_validate_config(c)
    for field, val in (("block_size", 65), ("window", 16), ("conv2", 1), ("topk", 16)):
        c2 = _cfg("small_target", max_batch=2)
        setattr(c2, field, val)
        with pytest.raises(B.DFlashError):
            B.dflash_validate_config(c2)
    w = _fake_weights(c.n_layers)
    w.fc = w.fc_norm = None  # a target has no context projection
    h = B.dflash_create(c, w, 1 << 30, 2 << 30, 3 << 30)
    try:
        with pytest.raises(B.DFlashError) as e:
            B.dflash_draft_block(h, 0, [0], 0, 1 << 20)
        assert e.value.status == B.E_INVALID and "target" in str(e.value)
        with pytest.raises(B.DFlashError) as e:  # the slot is not bound
            B.dflash_target_forward(h, 0, [0], 17, 1 << 20, 1 << 20)
        assert e.value.status == B.E_INVALID
        with pytest.raises(B.DFlashError) as e:  # nor can its length be set
            B.dflash_set_context_length(h, 0, 0, 5)
        assert e.value.status == B.E_INVALID and "not bound" in str(e.value)
    finally:
        B.dflash_destroy(h)
    d = _cfg("small_bf16", max_batch=2)
    hd = B.dflash_create(d, _fake_weights(d.n_layers), 1 << 30, 2 << 30, 3 << 30)
    try:
        with pytest.raises(B.DFlashError) as e:
            B.dflash_target_forward(hd, 0, [0], 1, 1 << 20, 1 << 20)
        assert e.value.status == B.E_INVALID and "target" in str(e.value)
    finally:
        B.dflash_destroy(hd)
