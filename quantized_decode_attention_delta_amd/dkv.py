"""Thin Python binding of libdkv.so (the C ABI declared in include/dkv.h).

Argument marshalling only: every step of the Delta-KV path runs in the HIP
library.  Functions take torch tensors on the GPU, check dtype, device and
contiguity, and pass raw pointers plus torch's current HIP stream.  If the
library is missing the binding raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdkv.so")

DKV_OK, DKV_ERR_ARG, DKV_ERR_UNSUPPORTED, DKV_ERR_WORKSPACE, DKV_ERR_HIP, DKV_ERR_SCRATCH = range(6)


class DkvError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "n_q_heads", "n_kv_heads", "head_dim", "kf", "max_tokens",
        "page_tokens", "n_pages", "max_pages_per_seq")]


@dataclasses.dataclass
class Config:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kf: int
    max_tokens: int = 0
    page_tokens: int = 0
    n_pages: int = 0
    max_pages_per_seq: int = 0

    def c(self) -> _Config:
        return _Config(*(int(getattr(self, f[0])) for f in _Config._fields_))

    @property
    def G(self):
        return self.n_q_heads // self.n_kv_heads


_lib = None

_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32
_F = ctypes.c_float
_CFG = ctypes.POINTER(_Config)

_SIGS = {
    "dkv_status_str": ([_I32], ctypes.c_char_p),
    "dkv_check_config": ([_CFG], _I32),
    "dkv_group_record_bytes": ([_CFG], _SZ),
    "dkv_cache_bytes": ([_CFG], _SZ),
    "dkv_state_bytes": ([_CFG], _SZ),
    "dkv_workspace_bytes": ([_CFG], _SZ),
    "dkv_attn_decode_launches": ([_CFG], _I32),
    "dkv_attn_decode_plan": ([_CFG, _P, _P], _I32),
    "dkv_encode_prefill": ([_CFG, _P, _P, _P, _P, _P, _P, _I32, _P], _I32),
    "dkv_append": ([_CFG, _P, _P, _P, _P, _P, _P, _P], _I32),
    "dkv_attn_decode": ([_CFG, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_attn_decode_noalloc": ([_CFG, _P, _P, _P, _P, _F, _P, _P], _I32),
    "dkv_append_attn_decode": ([_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_attn_decode_ref": ([_CFG, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_attn_decode_partial": ([_CFG, _P, _P, _P, _P, _F, _P, _SZ, _P], _I32),
    "dkv_reconstruct": ([_CFG, _P, _P, _P, _I32, _P, _P, _P], _I32),
    "dkv_export": ([_CFG, _P, _P, _P, _I32, _P, _P, _P, _P], _I32),
    "dkv_q4_0_cache_bytes": ([_CFG], _SZ),
    "dkv_q4_0_encode": ([_CFG, _P, _P, _P, _P, _P, _I32, _P], _I32),
    "dkv_q4_0_export": ([_CFG, _P, _P, _P, _I32, _P, _P, _P], _I32),
    "dkv_attn_decode_q4_0": ([_CFG, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_attn_decode_f16": ([_CFG, _P, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_q4k_encode_prefill": ([_CFG, _P, _P, _P, _P, _P, _P, _I32, _P], _I32),
    "dkv_q4k_append": ([_CFG, _P, _P, _P, _P, _P, _P, _P], _I32),
    "dkv_q4k_reconstruct": ([_CFG, _P, _P, _P, _I32, _P, _P, _P], _I32),
    "dkv_attn_decode_q4k": ([_CFG, _P, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_q8_0_encode": ([_CFG, _P, _P, _P, _I32, _P, _P, _P], _I32),
    "dkv_attn_distortion": ([_CFG, _P, _P, _P, _P, _I32, _P, _P, _F, _P, _P, _P, _P], _I32),
    "dkv_stream_read_sink_words": ([], _SZ),
    "dkv_stream_read": ([_P, _SZ, _P, _SZ, _P], _I32),
    "dkv_strided_cache_bytes": ([_CFG], _SZ),
    "dkv_strided_layout": ([_CFG, _P], _I32),
    "dkv_strided_encode_prefill": ([_CFG, _P, _P, _P, _P, _I32, _I32, _P], _I32),
    "dkv_strided_attn_decode": ([_CFG, _P, _P, _P, _F, _P, _P, _SZ, _P], _I32),
    "dkv_strided_append": ([_CFG, _P, _P, _P, _P, _I32, _P], _I32),
    "dkv_strided_append_attn_decode": ([_CFG, _P, _P, _P, _P, _I32, _P, _P, _F, _P, _P, _SZ, _P], _I32),
}


def load(path: str = LIB_PATH):
    """Load libdkv.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python __graft_entry__.py build)")
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_str(s: int) -> str:
    return load().dkv_status_str(s).decode()


def _check(fn, st):
    if st != DKV_OK:
        raise DkvError(fn, st, status_str(st))


# ------------------------------------------------------------------ size queries
def dkv_check_config(cfg: Config) -> int:
    return load().dkv_check_config(ctypes.byref(cfg.c()))


def dkv_group_record_bytes(cfg: Config) -> int:
    return load().dkv_group_record_bytes(ctypes.byref(cfg.c()))


def dkv_cache_bytes(cfg: Config) -> int:
    return load().dkv_cache_bytes(ctypes.byref(cfg.c()))


def dkv_state_bytes(cfg: Config) -> int:
    return load().dkv_state_bytes(ctypes.byref(cfg.c()))


def dkv_workspace_bytes(cfg: Config) -> int:
    return load().dkv_workspace_bytes(ctypes.byref(cfg.c()))


def dkv_attn_decode_launches(cfg: Config) -> int:
    return load().dkv_attn_decode_launches(ctypes.byref(cfg.c()))


def dkv_attn_decode_plan(cfg: Config) -> tuple:
    """(nsplit, split_tokens) of dkv_attn_decode's split plan for cfg."""
    ns, tk = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("dkv_attn_decode_plan", load().dkv_attn_decode_plan(ctypes.byref(cfg.c()), ctypes.byref(ns),
                                                               ctypes.byref(tk)))
    return ns.value, tk.value


def dkv_q4_0_cache_bytes(cfg: Config) -> int:
    return load().dkv_q4_0_cache_bytes(ctypes.byref(cfg.c()))


# ------------------------------------------------------------------ tensor helpers
def _ptr(t, dtype=None, name="tensor", numel=None):
    import torch
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    return ctypes.c_void_p(t.data_ptr())


def _bt_numel(cfg: Config) -> int:
    """Entries of a block table [batch][max_pages_per_seq] (paged mode only)."""
    return cfg.batch * cfg.max_pages_per_seq if cfg.page_tokens > 0 else 0


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _f16(t, name, numel=None):
    import torch
    return _ptr(t, (torch.float16, torch.int16, torch.uint16), name, numel)


# ------------------------------------------------------------------ entry points
def dkv_encode_prefill(cfg: Config, cache, state, block_table, k, v, seq_lens, s_max: int, stream=None):
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    st = load().dkv_encode_prefill(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(state, torch.float32, "state", B * H * 2 * D),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _f16(k, "k", B * H * s_max * D), _f16(v, "v", B * H * s_max * D),
        _ptr(seq_lens, torch.int32, "seq_lens", B), int(s_max), _stream(stream))
    _check("dkv_encode_prefill", st)


def dkv_append(cfg: Config, cache, state, block_table, k_new, v_new, positions, stream=None):
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    st = load().dkv_append(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(state, torch.float32, "state", B * H * 2 * D),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _f16(k_new, "k_new", B * H * D), _f16(v_new, "v_new", B * H * D),
        _ptr(positions, torch.int32, "positions", B), _stream(stream))
    _check("dkv_append", st)


def _attn(fn, cfg, cache, block_table, q, seq_lens, out, workspace, softmax_scale, stream):
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    st = getattr(load(), fn)(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(q, torch.float32, "q", B * Hq * D), _ptr(seq_lens, torch.int32, "seq_lens", B),
        float(softmax_scale), _ptr(out, torch.float32, "out", B * Hq * D),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check(fn, st)


def dkv_attn_decode(cfg: Config, cache, block_table, q, seq_lens, out, workspace, softmax_scale=0.0,
                    stream=None):
    _attn("dkv_attn_decode", cfg, cache, block_table, q, seq_lens, out, workspace, softmax_scale, stream)


def dkv_attn_decode_noalloc(cfg: Config, cache, block_table, q, seq_lens, out, softmax_scale=0.0, stream=None):
    """dkv_attn_decode with its split-K partials in the library's fixed scratch array (no workspace)."""
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_attn_decode_noalloc(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(q, torch.float32, "q", B * Hq * D), _ptr(seq_lens, torch.int32, "seq_lens", B),
        float(softmax_scale), _ptr(out, torch.float32, "out", B * Hq * D), _stream(stream))
    _check("dkv_attn_decode_noalloc", st)


def dkv_append_attn_decode(cfg: Config, cache, state, block_table, k_new, v_new, positions, q, seq_lens, out,
                           workspace, softmax_scale=0.0, stream=None):
    """dkv_append then dkv_attn_decode in one call (the append fused into the split launch)."""
    import torch
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_append_attn_decode(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(state, torch.float32, "state", B * H * 2 * D),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _f16(k_new, "k_new", B * H * D), _f16(v_new, "v_new", B * H * D),
        _ptr(positions, torch.int32, "positions", B), _ptr(q, torch.float32, "q", B * Hq * D),
        _ptr(seq_lens, torch.int32, "seq_lens", B), float(softmax_scale), _ptr(out, torch.float32, "out", B * Hq * D),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check("dkv_append_attn_decode", st)


def dkv_attn_decode_ref(cfg: Config, cache, block_table, q, seq_lens, out, workspace, softmax_scale=0.0,
                        stream=None):
    _attn("dkv_attn_decode_ref", cfg, cache, block_table, q, seq_lens, out, workspace, softmax_scale, stream)


def dkv_attn_decode_partial(cfg: Config, cache, block_table, q, seq_lens, workspace, softmax_scale=0.0,
                            stream=None):
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_attn_decode_partial(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(q, torch.float32, "q", B * Hq * D), _ptr(seq_lens, torch.int32, "seq_lens", B),
        float(softmax_scale), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("dkv_attn_decode_partial", st)


def dkv_reconstruct(cfg: Config, cache, block_table, seq_lens, s_max: int, k_out, v_out, stream=None):
    import torch
    n = cfg.batch * cfg.n_kv_heads * s_max * cfg.head_dim
    st = load().dkv_reconstruct(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(seq_lens, torch.int32, "seq_lens", cfg.batch), int(s_max),
        _ptr(k_out, torch.float32, "k_out", n), _ptr(v_out, torch.float32, "v_out", n), _stream(stream))
    _check("dkv_reconstruct", st)


def dkv_q8_0_encode(cfg: Config, k, v, seq_lens, s_max: int, codes, scales, stream=None):
    """Q8_0 of the absolute K/V rows: codes int8 [B][Hkv][2][s_max][D], scales fp16 bits [B][Hkv][2][s_max][D/32]."""
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    n = B * H * s_max * D
    st = load().dkv_q8_0_encode(
        ctypes.byref(cfg.c()), _f16(k, "k", n), _f16(v, "v", n), _ptr(seq_lens, torch.int32, "seq_lens", B),
        int(s_max), _ptr(codes, torch.int8, "codes", 2 * n),
        _ptr(scales, (torch.int16, torch.float16), "scales", 2 * n // 32), _stream(stream))
    _check("dkv_q8_0_encode", st)


def dkv_attn_distortion(cfg: Config, k_hat, v_hat, k, v, s_max: int, q, seq_lens, d_k, d_v, logits,
                        softmax_scale: float = 0.0, stream=None):
    """Attention-preserving distortion d_k, d_v [B][Hq] of reconstructed K/V against fp16 originals."""
    import torch
    n = cfg.batch * cfg.n_kv_heads * s_max * cfg.head_dim
    st = load().dkv_attn_distortion(
        ctypes.byref(cfg.c()), _ptr(k_hat, torch.float32, "k_hat", n), _ptr(v_hat, torch.float32, "v_hat", n),
        _f16(k, "k", n), _f16(v, "v", n), int(s_max),
        _ptr(q, torch.float32, "q", cfg.batch * cfg.n_q_heads * cfg.head_dim),
        _ptr(seq_lens, torch.int32, "seq_lens", cfg.batch), float(softmax_scale),
        _ptr(logits, torch.float32, "logits", cfg.batch * cfg.n_q_heads * s_max),
        _ptr(d_k, torch.float32, "d_k", cfg.batch * cfg.n_q_heads),
        _ptr(d_v, torch.float32, "d_v", cfg.batch * cfg.n_q_heads), _stream(stream))
    _check("dkv_attn_distortion", st)


def export_shapes(cfg: Config, s_max: int):
    ng = -(-s_max // cfg.kf)
    nd = s_max - ng
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    return (B, H, 2, ng, D), (B, H, 2, nd, D // 2), (B, H, 2, nd, D // 32)


def dkv_export(cfg: Config, cache, block_table, seq_lens, s_max: int, kf_rows, codes, scales, stream=None):
    import torch
    skf, scd, ssc = export_shapes(cfg, s_max)
    st = load().dkv_export(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(seq_lens, torch.int32, "seq_lens", cfg.batch), int(s_max),
        _f16(kf_rows, "kf_rows", math.prod(skf)), _ptr(codes, torch.uint8, "codes", math.prod(scd)),
        _f16(scales, "scales", math.prod(ssc)), _stream(stream))
    _check("dkv_export", st)


def f16_cache_shape(cfg: Config):
    """Shape of each of the two fp16 arrays (K, V) dkv_attn_decode_f16 reads."""
    if cfg.page_tokens > 0:
        return (cfg.n_pages, cfg.n_kv_heads, cfg.page_tokens, cfg.head_dim)
    return (cfg.batch, cfg.n_kv_heads, cfg.max_tokens, cfg.head_dim)


def dkv_q4_0_encode(cfg: Config, q4_cache, block_table, k, v, seq_lens, s_max: int, stream=None):
    import torch
    n = cfg.batch * cfg.n_kv_heads * s_max * cfg.head_dim
    st = load().dkv_q4_0_encode(
        ctypes.byref(cfg.c()), _ptr(q4_cache, torch.uint8, "q4_cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _f16(k, "k", n), _f16(v, "v", n), _ptr(seq_lens, torch.int32, "seq_lens", cfg.batch), int(s_max),
        _stream(stream))
    _check("dkv_q4_0_encode", st)


def dkv_q4_0_export(cfg: Config, q4_cache, block_table, seq_lens, s_max: int, codes, scales, stream=None):
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    st = load().dkv_q4_0_export(
        ctypes.byref(cfg.c()), _ptr(q4_cache, torch.uint8, "q4_cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(seq_lens, torch.int32, "seq_lens", B), int(s_max),
        _ptr(codes, torch.uint8, "codes", B * H * 2 * s_max * D // 2),
        _f16(scales, "scales", B * H * 2 * s_max * D // 32), _stream(stream))
    _check("dkv_q4_0_export", st)


def dkv_attn_decode_q4_0(cfg: Config, q4_cache, block_table, q, seq_lens, out, workspace, softmax_scale=0.0,
                         stream=None):
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_attn_decode_q4_0(
        ctypes.byref(cfg.c()), _ptr(q4_cache, torch.uint8, "q4_cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)), _ptr(q, torch.float32, "q", B * Hq * D),
        _ptr(seq_lens, torch.int32, "seq_lens", B), float(softmax_scale),
        _ptr(out, torch.float32, "out", B * Hq * D), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("dkv_attn_decode_q4_0", st)


# ------------------------------------------------------- Q4-keyframe variant
def dkv_q4k_encode_prefill(cfg: Config, cache, state, block_table, k, v, seq_lens, s_max: int, stream=None):
    """Q4-keyframe encode into a cache of dkv_q4_0_cache_bytes(cfg) bytes."""
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    st = load().dkv_q4k_encode_prefill(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(state, torch.float32, "state", B * H * 2 * D),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _f16(k, "k", B * H * s_max * D), _f16(v, "v", B * H * s_max * D),
        _ptr(seq_lens, torch.int32, "seq_lens", B), int(s_max), _stream(stream))
    _check("dkv_q4k_encode_prefill", st)


def dkv_q4k_append(cfg: Config, cache, state, block_table, k_new, v_new, positions, stream=None):
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    st = load().dkv_q4k_append(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(state, torch.float32, "state", B * H * 2 * D),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _f16(k_new, "k_new", B * H * D), _f16(v_new, "v_new", B * H * D),
        _ptr(positions, torch.int32, "positions", B), _stream(stream))
    _check("dkv_q4k_append", st)


def dkv_q4k_reconstruct(cfg: Config, cache, block_table, seq_lens, s_max: int, k_out, v_out, stream=None):
    import torch
    n = cfg.batch * cfg.n_kv_heads * s_max * cfg.head_dim
    st = load().dkv_q4k_reconstruct(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(seq_lens, torch.int32, "seq_lens", cfg.batch), int(s_max),
        _ptr(k_out, torch.float32, "k_out", n), _ptr(v_out, torch.float32, "v_out", n), _stream(stream))
    _check("dkv_q4k_reconstruct", st)


def dkv_attn_decode_q4k(cfg: Config, cache, block_table, q, seq_lens, out, workspace, softmax_scale=0.0,
                        stream=None):
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_attn_decode_q4k(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_q4_0_cache_bytes(cfg)),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)), _ptr(q, torch.float32, "q", B * Hq * D),
        _ptr(seq_lens, torch.int32, "seq_lens", B), float(softmax_scale),
        _ptr(out, torch.float32, "out", B * Hq * D), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("dkv_attn_decode_q4k", st)


def dkv_attn_decode_f16(cfg: Config, k, v, block_table, q, seq_lens, out, workspace, softmax_scale=0.0,
                        stream=None):
    """F16 decode attention; k, v fp16 of f16_cache_shape(cfg) each."""
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    n = math.prod(f16_cache_shape(cfg))
    st = load().dkv_attn_decode_f16(
        ctypes.byref(cfg.c()), _f16(k, "k", n), _f16(v, "v", n),
        _ptr(block_table, torch.int32, "block_table", _bt_numel(cfg)),
        _ptr(q, torch.float32, "q", B * Hq * D), _ptr(seq_lens, torch.int32, "seq_lens", B),
        float(softmax_scale), _ptr(out, torch.float32, "out", B * Hq * D),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check("dkv_attn_decode_f16", st)


def dkv_stream_read_sink_words() -> int:
    return load().dkv_stream_read_sink_words()


def dkv_stream_read(buf, sink, nbytes=None, stream=None):
    """Streaming-read ceiling: read `buf` (any GPU tensor) once; sink: int32/uint32 GPU tensor."""
    import torch
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    st = load().dkv_stream_read(_ptr(buf, None, "buf"), n, _ptr(sink, (torch.int32,), "sink"), sink.numel(),
                                _stream(stream))
    _check("dkv_stream_read", st)


# ------------------------------------------------------------------ strided references
def dkv_strided_cache_bytes(cfg: Config) -> int:
    return load().dkv_strided_cache_bytes(ctypes.byref(cfg.c()))


def dkv_strided_layout(cfg: Config) -> dict:
    """Plane offsets inside one stream, the stream's bytes and the reference rows per stream."""
    import numpy as np
    out = np.zeros(6, np.int64)
    st = load().dkv_strided_layout(ctypes.byref(cfg.c()), out.ctypes.data_as(ctypes.c_void_p))
    _check("dkv_strided_layout", st)
    return dict(refs=int(out[0]), codes=int(out[1]), scales=int(out[2]), idx=int(out[3]),
                stream_bytes=int(out[4]), nref=int(out[5]))


def dkv_strided_encode_prefill(cfg: Config, cache, k, v, seq_lens, s_max: int, window: int = 0, stream=None):
    """Strided-reference residual encode of tokens [0, seq_lens[b]) (k, v fp16 [B][Hkv][s_max][D])."""
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    n = B * H * s_max * D
    st = load().dkv_strided_encode_prefill(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_strided_cache_bytes(cfg)),
        _f16(k, "k", n), _f16(v, "v", n), _ptr(seq_lens, torch.int32, "seq_lens", B), int(s_max), int(window),
        _stream(stream))
    _check("dkv_strided_encode_prefill", st)


def dkv_strided_attn_decode(cfg: Config, cache, q, seq_lens, out, workspace, softmax_scale=0.0, stream=None):
    """Decode attention over the strided-reference cache."""
    import torch
    B, Hq, D = cfg.batch, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_strided_attn_decode(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_strided_cache_bytes(cfg)),
        _ptr(q, torch.float32, "q", B * Hq * D), _ptr(seq_lens, torch.int32, "seq_lens", B), float(softmax_scale),
        _ptr(out, torch.float32, "out", B * Hq * D), _ptr(workspace, torch.uint8, "workspace"),
        workspace.numel() if workspace is not None else 0, _stream(stream))
    _check("dkv_strided_attn_decode", st)


def dkv_strided_append(cfg: Config, cache, k_new, v_new, positions, window: int = 0, stream=None):
    """Append one token per sequence (k_new, v_new fp16 [B][Hkv][D]) at positions[b] (< 0: none)."""
    import torch
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    st = load().dkv_strided_append(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_strided_cache_bytes(cfg)),
        _f16(k_new, "k_new", B * H * D), _f16(v_new, "v_new", B * H * D),
        _ptr(positions, torch.int32, "positions", B), int(window), _stream(stream))
    _check("dkv_strided_append", st)


def dkv_strided_append_attn_decode(cfg: Config, cache, k_new, v_new, positions, q, seq_lens, out, workspace,
                                   window: int = 0, softmax_scale=0.0, stream=None):
    """dkv_strided_append then dkv_strided_attn_decode in one call (the append inside the split launch)."""
    import torch
    B, H, Hq, D = cfg.batch, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    st = load().dkv_strided_append_attn_decode(
        ctypes.byref(cfg.c()), _ptr(cache, torch.uint8, "cache", dkv_strided_cache_bytes(cfg)),
        _f16(k_new, "k_new", B * H * D), _f16(v_new, "v_new", B * H * D),
        _ptr(positions, torch.int32, "positions", B), int(window), _ptr(q, torch.float32, "q", B * Hq * D),
        _ptr(seq_lens, torch.int32, "seq_lens", B), float(softmax_scale), _ptr(out, torch.float32, "out", B * Hq * D),
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel() if workspace is not None else 0,
        _stream(stream))
    _check("dkv_strided_append_attn_decode", st)
