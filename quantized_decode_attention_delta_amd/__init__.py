"""Delta-KV compressed KV cache and fused decode attention for MI355X (gfx950).

The compute path lives in the HIP library ``libdkv.so`` (C ABI in
``include/dkv.h``); :mod:`.dkv` is its thin ctypes binding over torch tensors
and :mod:`.synth` draws the seeded synthetic workloads.
"""
from .dkv import (  # noqa: F401
    Config, DkvError, load, status_str,
    dkv_check_config, dkv_group_record_bytes, dkv_attn_decode_noalloc, dkv_cache_bytes, dkv_state_bytes, dkv_workspace_bytes,
    dkv_attn_decode_launches, dkv_attn_decode_plan,
    dkv_q4_0_cache_bytes, dkv_encode_prefill, dkv_append, dkv_attn_decode, dkv_append_attn_decode,
    dkv_attn_decode_ref, dkv_attn_decode_partial,
    dkv_reconstruct, dkv_export, export_shapes, dkv_q4_0_encode, dkv_q4_0_export, dkv_attn_decode_q4_0,
    dkv_attn_decode_f16, f16_cache_shape, dkv_stream_read_sink_words, dkv_stream_read, dkv_attn_distortion,
    dkv_q8_0_encode, dkv_strided_cache_bytes, dkv_strided_layout, dkv_strided_encode_prefill,
    dkv_strided_attn_decode, dkv_strided_append, dkv_strided_append_attn_decode,
    dkv_q4k_encode_prefill, dkv_q4k_append, dkv_q4k_reconstruct, dkv_attn_decode_q4k,
)
