"""The bench's algorithmic work counts (what every roofline fraction divides
by), checked against the workload shapes on the CPU.

For the Qwen3-8B-shaped draft (hidden 4096, 32 q / 8 kv heads x 128, SwiGLU
12288, vocab 151936, 5 layers, bf16): QKV weights 50.3 MB, O 33.6 MB, gate/up
201.3 MB, down 100.7 MB per layer, the shared LM head 1.245 GB, and 83.9 MB
of context K/V at 4096 visible positions over the 5 layers."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

MB = 1e6


def test_qwen3_8b_draft_bytes():
    shape = synth.config("qwen3_8b")
    per_layer = {"qkv": 48 * 128 * 4096 * 2, "o": 4096 * 4096 * 2, "gateup": 2 * 12288 * 4096 * 2,
                 "down": 4096 * 12288 * 2}
    assert round(per_layer["qkv"] / MB, 1) == 50.3
    assert round(per_layer["o"] / MB, 1) == 33.6
    assert round(per_layer["gateup"] / MB, 1) == 201.3
    assert round(per_layer["down"] / MB, 1) == 100.7
    lm = 151936 * 4096 * 2
    kv = 5 * 4096 * 2 * 8 * 128 * 2
    assert round(lm / 1e9, 3) == 1.245 and round(kv / MB, 1) == 83.9
    assert bench.draft_bytes(shape, [4096]) == 5 * sum(per_layer.values()) + lm + kv == 3_257_925_632


def test_class_work_lm_head_and_gemm_rows():
    shape = synth.config("qwen3_8b")
    flops, nbytes = bench.class_work(shape, "lm_head", 16, [4096])
    assert flops == 2 * 16 * 151936 * 4096
    assert nbytes == 2 * (151936 * 4096 + 16 * 4096)  # weights and the 16 normed rows in
    flops, nbytes = bench.class_work(shape, "gateup_gemm", 1024, [4096] * 64)
    assert flops == 2 * 1024 * (2 * 12288) * 4096
    assert nbytes == 2 * (2 * 12288 * 4096 + 1024 * 4096 + 1024 * 12288)  # SwiGLU writes F columns


def test_class_work_attention_counts_visible_kv_once():
    shape = synth.config("qwen3_8b")
    vis = [100, 5000]
    flops, nbytes = bench.class_work(shape, "attn", 32, vis)
    kv = sum(vis) * 2 * 8 * 128 * 2
    qkv_in = 32 * (32 + 16) * 128 * 2
    o_out = 32 * 32 * 128 * 2
    assert nbytes == kv + qkv_in + o_out
    # QK^T and PV over the visible keys plus the 16 block keys of each request
    assert flops == 4.0 * 32 * 128 * 16 * sum(v + 16 for v in vis)
