"""The algorithmic byte counts bench.py divides by, pinned on the CPU.

Delta-KV: 2,488 B per 32-token group and stream at D = 128 (a 256-byte fp16
keyframe and 31 Q4_0 rows of 72 bytes).  Strided references: 74 B per token
and stream at D = 128 plus every reference row once, which is exactly the
library's plane sizes when no plane needs alignment padding.
"""
import os
import types

import numpy as np

import bench
import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import dkv as binding


def test_delta_kv_bytes_70b_layer():
    assert bench.algorithmic_bytes(16, 8, 64, 128, 32768, 32) == 2 * 16 * 8 * 1024 * 2488
    # a partial last group: 2 groups of which the second holds 8 tokens
    assert bench.algorithmic_bytes(1, 1, 1, 128, 40, 32) == 2 * (2 * 256 + 38 * 72)


def test_strided_bytes_match_the_library_planes():
    w = types.SimpleNamespace(D=128, Hkv=8)
    lens = np.full(16, 32768)
    got = bench.strided_bytes(w, 32, lens)
    assert got == 2 * 8 * 16 * (32768 * 74 + 1024 * 256)
    if not os.path.exists(binding.LIB_PATH):
        from quantized_decode_attention_delta_amd import build
        build.build()
    cfg = dkv.Config(batch=16, n_q_heads=64, n_kv_heads=8, head_dim=128, kf=32, max_tokens=32768)
    assert got == dkv.dkv_strided_cache_bytes(cfg)


def test_strided_bytes_ragged_and_empty():
    w = types.SimpleNamespace(D=64, Hkv=2)
    lens = np.array([0, 1, 33])
    per_tok = 64 // 2 + 2 * 2 + 2
    want = 2 * 2 * ((1 * per_tok + 1 * 128) + (33 * per_tok + 2 * 128))
    assert bench.strided_bytes(w, 32, lens) == want
