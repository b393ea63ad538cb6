"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import dkv as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dkv.h")


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        from quantized_decode_attention_delta_amd import build
        build.build()
    return dkv.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dkv_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = _lib()
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding._SIGS), set(names) ^ set(binding._SIGS)


def _cfg(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, kf=32, max_tokens=1000)
    base.update(kw)
    return dkv.Config(**base)


@pytest.mark.parametrize("kw,want", [
    (dict(), binding.DKV_OK),
    (dict(batch=0), binding.DKV_ERR_ARG),
    (dict(n_q_heads=7), binding.DKV_ERR_ARG),
    (dict(head_dim=48), binding.DKV_ERR_ARG),
    (dict(head_dim=96), binding.DKV_ERR_UNSUPPORTED),
    (dict(head_dim=256), binding.DKV_ERR_UNSUPPORTED),
    (dict(kf=0), binding.DKV_ERR_ARG),
    (dict(kf=2048), binding.DKV_ERR_UNSUPPORTED),
    (dict(max_tokens=0), binding.DKV_ERR_ARG),
    (dict(page_tokens=256, kf=512, n_pages=4, max_pages_per_seq=2), binding.DKV_ERR_ARG),
    (dict(page_tokens=256, n_pages=0, max_pages_per_seq=2), binding.DKV_ERR_ARG),
    (dict(page_tokens=256, n_pages=4, max_pages_per_seq=2), binding.DKV_OK),
    (dict(n_q_heads=64, n_kv_heads=2), binding.DKV_ERR_UNSUPPORTED),
])
def test_check_config(kw, want):
    _lib()
    assert dkv.dkv_check_config(_cfg(**kw)) == want


def test_sizes():
    _lib()
    c = _cfg(batch=16, n_q_heads=64, n_kv_heads=8, max_tokens=32768)
    rec = dkv.dkv_group_record_bytes(c)
    # two streams of 2,488 algorithmic bytes per 32-token group, plus 64 bytes of
    # V code padding (the keyframe slot) and 8+8 bytes of scale slot 0, padded
    # to whole 128-byte lines
    assert rec == 5120 and 2 * 2488 + 64 + 16 == 5056
    assert dkv.dkv_group_record_bytes(_cfg(head_dim=64)) == 2560           # 2528 rounded up
    assert dkv.dkv_cache_bytes(c) == 16 * 8 * 1024 * rec
    assert dkv.dkv_state_bytes(c) == 16 * 8 * 2 * 128 * 4
    assert dkv.dkv_workspace_bytes(c) > 0
    # one launch (the split kernel merges its own partials) only on small
    # launches: at most 16 splits per row and 256 workgroups
    assert dkv.dkv_attn_decode_launches(c) == 2
    assert dkv.dkv_attn_decode_launches(_cfg(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, max_tokens=256)) == 1
    assert dkv.dkv_attn_decode_launches(_cfg(batch=1, n_q_heads=32, n_kv_heads=8, max_tokens=4096)) == 2
    assert dkv.dkv_attn_decode_launches(_cfg(batch=1, n_q_heads=32, n_kv_heads=8, max_tokens=512)) == 1
    assert dkv.dkv_attn_decode_launches(_cfg(head_dim=96)) == 0
    # split plan: 2048-token runs for full caches, 1024 in paged mode
    assert dkv.dkv_attn_decode_plan(c) == (16, 2048)
    assert dkv.dkv_attn_decode_plan(_cfg(batch=64, n_q_heads=32, n_kv_heads=8, page_tokens=256, n_pages=8400,
                                         max_pages_per_seq=257)) == (65, 1024)
    # runs of at least 128 tokens while 256 or more workgroups remain: the
    # 8B layer (8 pairs of 4096 tokens) in 32 runs of 4 groups; a single
    # 256-token sequence keeps its 8 runs of one group; kf = 512 runs stay one
    # group (512 tokens) each
    assert dkv.dkv_attn_decode_plan(_cfg(batch=1, n_q_heads=32, n_kv_heads=8, max_tokens=4096)) == (32, 128)
    assert dkv.dkv_attn_decode_plan(_cfg(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=64, max_tokens=256)) == (8, 32)
    assert dkv.dkv_attn_decode_plan(_cfg(batch=8, n_q_heads=32, n_kv_heads=8, kf=512, max_tokens=16384)) == (32, 512)
    assert dkv.dkv_attn_decode_plan(_cfg(batch=8, n_q_heads=32, n_kv_heads=8, max_tokens=16384)) == (32, 512)
    for B, Hkv, S in ((1, 8, 4096), (2, 4, 1000), (3, 1, 70000), (64, 8, 65536), (1, 1, 64)):
        ns, tk = dkv.dkv_attn_decode_plan(_cfg(batch=B, n_q_heads=Hkv, n_kv_heads=Hkv, max_tokens=S))
        assert ns * tk >= S and (ns - 1) * tk < S                    # the runs tile the capacity
        assert tk <= 2048 and (tk >= 128 or ns * B * Hkv >= 256 or ns * tk < 128 * 2)
    assert dkv.dkv_q4_0_cache_bytes(c) == 16 * 8 * 2 * 32768 * 128 // 32 * 18
    # paged comparison caches: a page of 256 tokens holds 8 tiles per kv-head
    cpg = _cfg(page_tokens=256, n_pages=5, max_pages_per_seq=3)
    assert dkv.dkv_q4_0_cache_bytes(cpg) == 5 * 2 * 8 * 36 * 128
    assert dkv.f16_cache_shape(cpg) == (5, 2, 256, 128) and dkv.f16_cache_shape(c) == (16, 8, 32768, 128)
    assert dkv.dkv_cache_bytes(_cfg(head_dim=96)) == 0
    # strided references: per stream 1024 fp16 reference rows, 32768 tokens of
    # 64 code bytes, 8 scale bytes and a 2-byte index, planes 256-byte aligned
    lay = dkv.dkv_strided_layout(c)
    assert lay == dict(refs=0, codes=1024 * 256, scales=1024 * 256 + 32768 * 64,
                       idx=1024 * 256 + 32768 * 72, stream_bytes=1024 * 256 + 32768 * 74, nref=1024)
    assert dkv.dkv_strided_cache_bytes(c) == 16 * 8 * 2 * lay["stream_bytes"]
    assert dkv.dkv_strided_cache_bytes(_cfg(page_tokens=256, n_pages=8, max_pages_per_seq=4)) == 0
    assert dkv.dkv_strided_cache_bytes(_cfg(kf=1, max_tokens=70000)) == 0      # 70000 references > 65536


def test_argument_errors_return_before_launch():
    lib = _lib()
    c = _cfg()
    cp = ctypes.byref(c.c())
    fake = ctypes.c_void_p(0x1000)
    null = None
    # null pointers
    assert lib.dkv_encode_prefill(cp, null, fake, null, fake, fake, fake, 10, null) == binding.DKV_ERR_ARG
    assert lib.dkv_append(cp, fake, fake, null, fake, null, fake, null) == binding.DKV_ERR_ARG
    assert lib.dkv_attn_decode(cp, fake, null, null, fake, 0.0, fake, fake, 1 << 30, null) == binding.DKV_ERR_ARG
    # missing / short workspace
    assert lib.dkv_attn_decode(cp, fake, null, fake, fake, 0.0, fake, null, 0, null) == binding.DKV_ERR_WORKSPACE
    assert lib.dkv_attn_decode(cp, fake, null, fake, fake, 0.0, fake, fake, 16, null) == binding.DKV_ERR_WORKSPACE
    assert lib.dkv_attn_decode_ref(cp, fake, null, fake, fake, 0.0, fake, fake, 16, null) == binding.DKV_ERR_WORKSPACE
    # paged mode needs a block table
    cpg = ctypes.byref(_cfg(page_tokens=256, n_pages=8, max_pages_per_seq=4).c())
    assert lib.dkv_encode_prefill(cpg, fake, fake, null, fake, fake, fake, 10, null) == binding.DKV_ERR_ARG
    # unsupported config propagates
    cbad = ctypes.byref(_cfg(head_dim=96).c())
    assert lib.dkv_append(cbad, fake, fake, null, fake, fake, fake, null) == binding.DKV_ERR_UNSUPPORTED
    # comparison caches: paged mode needs a block table and 32-token-aligned pages
    assert lib.dkv_q4_0_encode(cpg, fake, null, fake, fake, fake, 10, null) == binding.DKV_ERR_ARG
    assert lib.dkv_attn_decode_f16(cpg, fake, fake, null, fake, fake, 0.0, fake, fake, 1 << 30,
                                   null) == binding.DKV_ERR_ARG
    cp16 = ctypes.byref(_cfg(kf=16, page_tokens=48, n_pages=8, max_pages_per_seq=4).c())
    assert lib.dkv_attn_decode_q4_0(cp16, fake, fake, fake, fake, 0.0, fake, fake, 1 << 30,
                                    null) == binding.DKV_ERR_UNSUPPORTED
    assert dkv.dkv_q4_0_cache_bytes(_cfg(kf=16, page_tokens=48, n_pages=8, max_pages_per_seq=4)) == 0
    assert lib.dkv_attn_decode_f16(cp, fake, fake, null, fake, fake, 0.0, fake, fake, 16, null) == binding.DKV_ERR_WORKSPACE
    # one serving step: null state / new rows, short workspace
    assert lib.dkv_append_attn_decode(cp, fake, null, null, fake, fake, fake, fake, fake, 0.0, fake, fake,
                                      1 << 30, null) == binding.DKV_ERR_ARG
    assert lib.dkv_append_attn_decode(cp, fake, fake, null, fake, fake, fake, fake, fake, 0.0, fake, fake,
                                      16, null) == binding.DKV_ERR_WORKSPACE
    # attention distortion: null pointers, empty s_max, unsupported head_dim
    d = [fake] * 4
    assert lib.dkv_attn_distortion(cp, *d, 10, fake, fake, 0.0, fake, fake, null, null) == binding.DKV_ERR_ARG
    assert lib.dkv_attn_distortion(cp, *d, 0, fake, fake, 0.0, fake, fake, fake, null) == binding.DKV_ERR_ARG
    assert lib.dkv_attn_distortion(cbad, *d, 10, fake, fake, 0.0, fake, fake, fake, null) == binding.DKV_ERR_UNSUPPORTED
    # strided references: contiguous only, null pointers, negative window, short workspace
    assert lib.dkv_strided_encode_prefill(cpg, fake, fake, fake, fake, 10, 0, null) == binding.DKV_ERR_UNSUPPORTED
    assert lib.dkv_strided_encode_prefill(cp, fake, null, fake, fake, 10, 0, null) == binding.DKV_ERR_ARG
    assert lib.dkv_strided_encode_prefill(cp, fake, fake, fake, fake, 10, -1, null) == binding.DKV_ERR_ARG
    assert lib.dkv_strided_attn_decode(cp, fake, null, fake, 0.0, fake, fake, 1 << 30, null) == binding.DKV_ERR_ARG
    assert lib.dkv_strided_attn_decode(cp, fake, fake, fake, 0.0, fake, fake, 16, null) == binding.DKV_ERR_WORKSPACE
    assert lib.dkv_strided_layout(cp, null) == binding.DKV_ERR_ARG
    assert lib.dkv_strided_append(cp, fake, fake, fake, null, 0, null) == binding.DKV_ERR_ARG
    assert lib.dkv_strided_append_attn_decode(cp, fake, fake, fake, fake, 0, fake, fake, 0.0, fake, fake, 16,
                                              null) == binding.DKV_ERR_WORKSPACE
    assert lib.dkv_strided_append_attn_decode(cp, fake, fake, fake, null, 0, fake, fake, 0.0, fake, fake, 1 << 30,
                                              null) == binding.DKV_ERR_ARG
    assert lib.dkv_strided_append(cpg, fake, fake, fake, fake, 0, null) == binding.DKV_ERR_UNSUPPORTED
    # Q4-keyframe variant: groups in whole tiles (kf divides 32 or is a multiple
    # of 32); attention at kf 1 and 32 only; null pointers
    c48 = ctypes.byref(_cfg(kf=48).c())
    assert lib.dkv_q4k_encode_prefill(c48, fake, fake, null, fake, fake, fake, 10, null) == binding.DKV_ERR_UNSUPPORTED
    assert lib.dkv_q4k_append(c48, fake, fake, null, fake, fake, fake, null) == binding.DKV_ERR_UNSUPPORTED
    c8 = ctypes.byref(_cfg(kf=8).c())
    assert lib.dkv_attn_decode_q4k(c8, fake, null, fake, fake, 0.0, fake, fake, 1 << 30,
                                   null) == binding.DKV_ERR_UNSUPPORTED
    assert lib.dkv_q4k_encode_prefill(c8, fake, null, null, fake, fake, fake, 10, null) == binding.DKV_ERR_ARG
    assert lib.dkv_q4k_reconstruct(cp, fake, null, fake, 10, fake, null, null) == binding.DKV_ERR_ARG
    assert lib.dkv_attn_decode_q4k(cp, fake, null, fake, fake, 0.0, fake, fake, 16, null) == binding.DKV_ERR_WORKSPACE
    assert lib.dkv_attn_decode_q4k(cpg, fake, null, fake, fake, 0.0, fake, fake, 1 << 30, null) == binding.DKV_ERR_ARG
    assert lib.dkv_check_config(None) == binding.DKV_ERR_ARG
    assert dkv.status_str(binding.DKV_ERR_WORKSPACE) == "workspace missing or too small"


def test_binding_refuses_cpu_tensors():
    import torch
    _lib()
    c = _cfg()
    t = torch.zeros(10)
    with pytest.raises((ValueError, TypeError)):
        dkv.dkv_encode_prefill(c, t, t, None, t, t, t, 10)


def test_binding_rejects_undersized_caches():
    """Every call that reads or writes a cache checks its size against the
    library's size query before anything else reaches the C ABI (a short
    buffer would otherwise be read or written past its end on the GPU)."""
    import torch
    _lib()
    c = _cfg()
    short = torch.zeros(dkv.dkv_cache_bytes(c) - 1, dtype=torch.uint8)
    q = torch.zeros(c.batch * c.n_q_heads * c.head_dim)
    lens = torch.zeros(c.batch, dtype=torch.int32)
    ws = torch.zeros(dkv.dkv_workspace_bytes(c), dtype=torch.uint8)
    calls = [
        lambda: dkv.dkv_attn_decode(c, short, None, q, lens, q, ws),
        lambda: dkv.dkv_attn_decode_ref(c, short, None, q, lens, q, ws),
        lambda: dkv.dkv_attn_decode_partial(c, short, None, q, lens, ws),
        lambda: dkv.dkv_reconstruct(c, short, None, lens, 4, q, q),
        lambda: dkv.dkv_export(c, short, None, lens, 4, q, q, q),
        lambda: dkv.dkv_q4_0_export(c, torch.zeros(dkv.dkv_q4_0_cache_bytes(c) - 1, dtype=torch.uint8), None, lens,
                                    4, short, short),
    ]
    for i, f in enumerate(calls):
        with pytest.raises(ValueError, match="elements, needs"):
            f()


def test_noalloc_decode_rejects_before_touching_the_gpu():
    """dkv_attn_decode_noalloc checks its arguments and that the split-K
    partials fit its fixed 160 MiB scratch before anything reaches the GPU."""
    lib = _lib()
    fake = ctypes.c_void_p(0x1000)
    ok = ctypes.byref(_cfg().c())
    assert lib.dkv_attn_decode_noalloc(ok, fake, None, None, fake, 0.0, fake, None) == binding.DKV_ERR_ARG
    cpg = ctypes.byref(_cfg(page_tokens=256, n_pages=8, max_pages_per_seq=4).c())
    assert lib.dkv_attn_decode_noalloc(cpg, fake, None, fake, fake, 0.0, fake, None) == binding.DKV_ERR_ARG
    # 64 sequences x 256 query heads x 32 splits x 132 floats = 277 MB of partials
    big = _cfg(batch=64, n_q_heads=256, n_kv_heads=16, max_tokens=65536)
    assert dkv.dkv_workspace_bytes(big) > 160 << 20
    assert lib.dkv_attn_decode_noalloc(ctypes.byref(big.c()), fake, None, fake, fake, 0.0, fake,
                                       None) == binding.DKV_ERR_SCRATCH
    assert "scratch" in dkv.status_str(binding.DKV_ERR_SCRATCH)
