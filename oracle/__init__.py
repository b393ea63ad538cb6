"""Delta-KV CPU oracle (TEST INFRASTRUCTURE ONLY).

ctypes wrapper around ``dkv_oracle.c``: the plain sequential C reference of the
Delta-KV codec (keyframe + closed-loop Q4_0 deltas) and float64 decode
attention.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package; the HIP library never does, and
the two share no code.

Canonical encoded layout of one stream (what every function here produces):

* ``kf_rows``  uint16 ``[ceil(S/kf), D]`` -- fp16 bits of each group's keyframe
* ``codes``    uint8  ``[n_delta, D/2]``  -- Q4_0 bytes, block-major, byte i of a
  block holds code i (low nibble) and code i+16 (high nibble)
* ``scales``   uint16 ``[n_delta, D/32]`` -- fp16 bits of each block scale

with ``n_delta = S - ceil(S/kf)``; delta token t sits at row
``(t//kf)*(kf-1) + t%kf - 1``.

``q4k_encode_stream`` is the Q4-keyframe variant: the keyframe itself is
stored as Q4_0 of its absolute values, so every token is one plain Q4_0 row
(``codes`` [S, D/2], ``scales`` [S, D/32]); with kf = 1 it is plain Q4_0.

``strided_encode_stream`` is the strided-reference variant: every token's Q4_0
residual against the nearest of the references at positions 0, stride, ...
(fp16 rows kept exactly), with the reference index stored per token.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdkv_oracle.so")
_lib = None

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    L = ctypes.c_long
    I = ctypes.c_int
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = ctypes.c_float
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_q40_block.argtypes = [P, P, P]
    lib.oracle_q40_block.restype = None
    lib.oracle_q40_pack.argtypes = [P, P]
    lib.oracle_q40_unpack.argtypes = [P, P]
    lib.oracle_delta_index.argtypes = [L, I]
    lib.oracle_delta_index.restype = L
    lib.oracle_step.argtypes = [P, L, I, I, P, P, P, P]
    lib.oracle_encode_stream.argtypes = [P, L, I, I, P, P, P, P, P]
    lib.oracle_reconstruct_stream.argtypes = [P, P, P, L, I, I, P]
    lib.oracle_q40_abs_stream.argtypes = [P, L, I, P, P]
    lib.oracle_q40_dequant_stream.argtypes = [P, P, L, I, P]
    lib.oracle_attention_f64.argtypes = [P, I, P, P, L, I, ctypes.c_float, P]
    lib.oracle_q80_block.argtypes = [P, P, P]
    lib.oracle_q80_abs_stream.argtypes = [P, L, I, P, P]
    lib.oracle_q80_dequant_stream.argtypes = [P, P, L, I, P]
    lib.oracle_sqdist_f16.argtypes = [P, P, I]
    lib.oracle_sqdist_f16.restype = ctypes.c_double
    lib.oracle_strided_encode_stream.argtypes = [P, L, I, I, I, P, P, P, P, P]
    lib.oracle_q4k_step.argtypes = [P, L, I, I, P, P, P]
    lib.oracle_q4k_encode_stream.argtypes = [P, L, I, I, P, P, P, P]
    lib.oracle_q4k_reconstruct_stream.argtypes = [P, P, L, I, I, P]
    for name in ("oracle_step", "oracle_encode_stream", "oracle_reconstruct_stream",
                 "oracle_q40_abs_stream", "oracle_q40_dequant_stream", "oracle_attention_f64",
                 "oracle_q40_pack", "oracle_q40_unpack", "oracle_q80_block", "oracle_q80_abs_stream",
                 "oracle_q80_dequant_stream", "oracle_strided_encode_stream", "oracle_q4k_step",
                 "oracle_q4k_encode_stream", "oracle_q4k_reconstruct_stream"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_f16_bits(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------- scalars
def f16_to_f32(h: int) -> float:
    return float(_load().oracle_f16_to_f32(int(h)))


def f32_to_f16(f: float) -> int:
    return int(_load().oracle_f32_to_f16(float(np.float32(f))))


def n_groups(S: int, kf: int) -> int:
    return -(-S // kf)


def n_delta(S: int, kf: int) -> int:
    return S - n_groups(S, kf)


def delta_index(t: int, kf: int) -> int:
    return int(_load().oracle_delta_index(t, kf))


# ---------------------------------------------------------------- Q4_0 block
def q40_block(v) -> tuple[int, np.ndarray]:
    """Quantise 32 fp32 values -> (fp16 scale bits, codes[32] in 0..15)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    assert v.shape == (32,)
    s = np.zeros(1, np.uint16)
    c = np.zeros(32, np.uint8)
    _load().oracle_q40_block(_p(v), _p(s), _p(c))
    return int(s[0]), c


def q40_pack(codes) -> np.ndarray:
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    out = np.zeros(16, np.uint8)
    _load().oracle_q40_pack(_p(codes), _p(out))
    return out


def q40_unpack(b) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint8))
    out = np.zeros(32, np.uint8)
    _load().oracle_q40_unpack(_p(b), _p(out))
    return out


# ---------------------------------------------------------------- streams
class EncodedStream:
    __slots__ = ("kf_rows", "codes", "scales", "recon", "state", "S", "D", "kf")

    def __init__(self, S, D, kf):
        self.S, self.D, self.kf = S, D, kf
        self.kf_rows = np.zeros((n_groups(S, kf), D), np.uint16)
        self.codes = np.zeros((n_delta(S, kf), D // 2), np.uint8)
        self.scales = np.zeros((n_delta(S, kf), D // 32), np.uint16)
        self.recon = None
        self.state = np.zeros(D, np.float32)


def encode_stream(x, kf: int, want_recon: bool = True) -> EncodedStream:
    """Encode one stream x[S][D] (fp16) with keyframe interval kf."""
    x = _as_f16_bits(x)
    S, D = x.shape
    assert D % 32 == 0 and kf >= 1
    e = EncodedStream(S, D, kf)
    if want_recon:
        e.recon = np.zeros((S, D), np.float32)
    _load().oracle_encode_stream(_p(x), S, D, kf, _p(e.kf_rows), _p(e.codes), _p(e.scales),
                                 _p(e.recon) if want_recon else None, _p(e.state))
    return e


def step(e: EncodedStream, x_row, t: int, xh: np.ndarray) -> None:
    """Append token t of a stream into the canonical arrays (in place)."""
    x_row = _as_f16_bits(x_row)
    assert xh.dtype == np.float32 and xh.flags["C_CONTIGUOUS"]
    _load().oracle_step(_p(x_row), t, e.D, e.kf, _p(e.kf_rows), _p(e.codes), _p(e.scales), _p(xh))


def reconstruct_stream(kf_rows, codes, scales, S: int, D: int, kf: int) -> np.ndarray:
    kf_rows = _as_f16_bits(kf_rows)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _as_f16_bits(scales)
    out = np.zeros((S, D), np.float32)
    _load().oracle_reconstruct_stream(_p(kf_rows), _p(codes), _p(scales), S, D, kf, _p(out))
    return out


def q40_abs_stream(x) -> tuple[np.ndarray, np.ndarray]:
    x = _as_f16_bits(x)
    S, D = x.shape
    codes = np.zeros((S, D // 2), np.uint8)
    scales = np.zeros((S, D // 32), np.uint16)
    _load().oracle_q40_abs_stream(_p(x), S, D, _p(codes), _p(scales))
    return codes, scales


def q40_dequant_stream(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _as_f16_bits(scales)
    S, D = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((S, D), np.float32)
    _load().oracle_q40_dequant_stream(_p(codes), _p(scales), S, D, _p(out))
    return out


class Q4KStream:
    """One stream of the Q4-keyframe variant: ``codes`` uint8 [S, D/2] and
    ``scales`` uint16 [S, D/32] (one plain-Q4_0 row per token), the
    reconstruction ``recon`` float32 [S, D] and the final ``state`` [D]."""
    __slots__ = ("codes", "scales", "recon", "state", "S", "D", "kf")

    def __init__(self, S, D, kf):
        self.S, self.D, self.kf = S, D, kf
        self.codes = np.zeros((S, D // 2), np.uint8)
        self.scales = np.zeros((S, D // 32), np.uint16)
        self.recon = None
        self.state = np.zeros(D, np.float32)


def q4k_encode_stream(x, kf: int, want_recon: bool = True) -> Q4KStream:
    """Q4-keyframe encode of one stream x[S][D] (fp16): the row at every
    multiple of kf is Q4_0 of its absolute values, every other row Q4_0 of
    its closed-loop delta ([DKV] "핵심 아이디어", "벤치마크")."""
    x = _as_f16_bits(x)
    S, D = x.shape
    assert D % 32 == 0 and kf >= 1
    e = Q4KStream(S, D, kf)
    if want_recon:
        e.recon = np.zeros((S, D), np.float32)
    _load().oracle_q4k_encode_stream(_p(x), S, D, kf, _p(e.codes), _p(e.scales),
                                     _p(e.recon) if want_recon else None, _p(e.state))
    return e


def q4k_step(e: Q4KStream, x_row, t: int, xh: np.ndarray) -> None:
    """Append token t of a Q4-keyframe stream into its arrays (in place)."""
    x_row = _as_f16_bits(x_row)
    assert xh.dtype == np.float32 and xh.flags["C_CONTIGUOUS"]
    _load().oracle_q4k_step(_p(x_row), t, e.D, e.kf, _p(e.codes), _p(e.scales), _p(xh))


def q4k_reconstruct_stream(codes, scales, kf: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = _as_f16_bits(scales)
    S, D = codes.shape[0], codes.shape[1] * 2
    out = np.zeros((S, D), np.float32)
    _load().oracle_q4k_reconstruct_stream(_p(codes), _p(scales), S, D, kf, _p(out))
    return out


def q4k_encode_cache(k, v, seq_lens, kf: int, want_recon: bool = True):
    """Q4-keyframe encode of every stream of fp16 K/V [B][Hkv][s_max][D]:
    a dict of Q4KStream keyed (b, h, s), s = 0 for K and 1 for V (usable with
    attention_cache)."""
    k = _as_f16_bits(k)
    v = _as_f16_bits(v)
    B, H, _, D = k.shape
    out = {}
    for b in range(B):
        S = int(seq_lens[b])
        for h in range(H):
            for s, x in ((0, k), (1, v)):
                out[(b, h, s)] = q4k_encode_stream(np.ascontiguousarray(x[b, h, :S]), kf, want_recon)
    return out


def q80_block(v) -> tuple[int, np.ndarray]:
    """Q8_0 of one 32-value block (fp32 inputs): (fp16 bits of the scale, int8 codes[32])."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    assert v.shape == (32,)
    d = np.zeros(1, np.uint16)
    c = np.zeros(32, np.int8)
    _load().oracle_q80_block(_p(v), _p(d), _p(c))
    return int(d[0]), c


def q80_abs_stream(x) -> tuple[np.ndarray, np.ndarray]:
    """Q8_0 of the absolute rows of one stream x[S][D] (fp16): codes int8 [S][D], scales uint16 [S][D/32]."""
    x = _as_f16_bits(x)
    S, D = x.shape
    codes = np.zeros((S, D), np.int8)
    scales = np.zeros((S, D // 32), np.uint16)
    _load().oracle_q80_abs_stream(_p(x), S, D, _p(codes), _p(scales))
    return codes, scales


def q80_dequant_stream(codes, scales) -> np.ndarray:
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.int8))
    scales = _as_f16_bits(scales)
    S, D = codes.shape
    out = np.zeros((S, D), np.float32)
    _load().oracle_q80_dequant_stream(_p(codes), _p(scales), S, D, _p(out))
    return out


class StridedStream:
    """One stream coded against strided references: ``refs`` uint16
    [ceil(S/stride), D] (fp16 bits of tokens 0, stride, ...), ``ref_idx`` int32
    [S], ``codes`` uint8 [S, D/2] and ``scales`` uint16 [S, D/32] (the Q4_0
    residual of every token, in the canonical byte order above), ``recon``
    float32 [S, D]."""
    __slots__ = ("refs", "ref_idx", "codes", "scales", "recon")


def sqdist_f16(a, b) -> float:
    """Squared distance of two fp16 rows, summed in double in channel order."""
    a, b = _as_f16_bits(a), _as_f16_bits(b)
    assert a.shape == b.shape and a.ndim == 1
    return float(_load().oracle_sqdist_f16(_p(a), _p(b), a.shape[0]))


def strided_encode_stream(x, stride: int, window: int = 0) -> StridedStream:
    """Strided-reference residual coding of one stream x[S][D] (fp16)."""
    x = _as_f16_bits(x)
    S, D = x.shape
    e = StridedStream()
    e.refs = np.zeros(((S + stride - 1) // stride, D), np.uint16)
    e.ref_idx = np.zeros(S, np.int32)
    e.codes = np.zeros((S, D // 2), np.uint8)
    e.scales = np.zeros((S, D // 32), np.uint16)
    e.recon = np.zeros((S, D), np.float32)
    if S:
        _load().oracle_strided_encode_stream(_p(x), S, D, stride, window, _p(e.refs), _p(e.ref_idx),
                                             _p(e.codes), _p(e.scales), _p(e.recon))
    return e


def attention_f64(q, K, V, scale: float) -> np.ndarray:
    """Float64 decode attention of G heads q[G][D] over K[S][D], V[S][D]."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    G, D = q.shape
    S = K.shape[0]
    assert K.shape == (S, D) and V.shape == (S, D)
    out = np.zeros((G, D), np.float64)
    _load().oracle_attention_f64(_p(q), G, _p(K), _p(V), S, D, float(np.float32(scale)), _p(out))
    return out


def attention_distortion_f64(q, K, V, K_hat, V_hat, scale: float):
    """Attention-preserving distortion of one decode step ("KV 캐시 벡터 양자화와
    주의 보존 변환", section 어텐션 보존 왜곡), in float64, for G query heads
    q[G][D] over one kv-head's keys/values K, V [S][D] and their
    reconstructions K_hat, V_hat:

      d_k[g] = || q_g K_hat^T - q_g K^T ||^2       the logit row, unscaled dot
                                                   products as the page prints them
      d_v[g] = || a_g V_hat - a_g V ||^2          a_g = softmax(scale * q_g K^T),
                                                   the attention weights on the
                                                   exact keys (so d_v isolates V)

    The page's expectation is the mean of these over (sequence, head) rows.
    With S = 0 both are 0.  Returns (d_k[G], d_v[G]).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    K_hat = np.asarray(K_hat, dtype=np.float64)
    V_hat = np.asarray(V_hat, dtype=np.float64)
    G = q.shape[0]
    if K.shape[0] == 0:
        return np.zeros(G), np.zeros(G)
    d_k = ((q @ K_hat.T - q @ K.T) ** 2).sum(axis=1)
    logits = float(np.float32(scale)) * (q @ K.T)                 # [G][S]
    a = np.exp(logits - logits.max(axis=1, keepdims=True))
    a /= a.sum(axis=1, keepdims=True)
    d_v = ((a @ V_hat - a @ V) ** 2).sum(axis=1)
    return d_k, d_v


# ---------------------------------------------------------------- whole caches
def encode_cache(k, v, seq_lens, kf: int, want_recon: bool = True):
    """Encode every stream of fp16 K/V [B][Hkv][s_max][D].

    Returns a dict of per-(b, h, stream) EncodedStream objects keyed
    ``(b, h, s)`` with s = 0 for K and 1 for V.
    """
    k = _as_f16_bits(k)
    v = _as_f16_bits(v)
    B, H, _, D = k.shape
    out = {}
    for b in range(B):
        S = int(seq_lens[b])
        for h in range(H):
            for s, x in ((0, k), (1, v)):
                out[(b, h, s)] = encode_stream(np.ascontiguousarray(x[b, h, :S]), kf, want_recon)
    return out


def attention_distortion_cache(enc, k, v, q, seq_lens, n_kv_heads: int, scale: float):
    """attention_distortion_f64 for every (sequence, query head) of q[B][Hq][D]
    over an encoded cache (from encode_cache) and its fp16 inputs k, v
    [B][Hkv][s_max][D].  Returns (d_k[B][Hq], d_v[B][Hq])."""
    q = np.asarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    G = Hq // n_kv_heads
    kx = _as_f16_bits(k).view(np.float16)
    vx = _as_f16_bits(v).view(np.float16)
    d_k = np.zeros((B, Hq))
    d_v = np.zeros((B, Hq))
    for b in range(B):
        S = int(seq_lens[b])
        for h in range(n_kv_heads):
            hq = slice(h * G, (h + 1) * G)
            d_k[b, hq], d_v[b, hq] = attention_distortion_f64(
                q[b, hq], kx[b, h, :S], vx[b, h, :S], enc[(b, h, 0)].recon, enc[(b, h, 1)].recon, scale)
    return d_k, d_v


def attention_cache(enc, q, seq_lens, n_kv_heads: int, scale: float, heads=None):
    """Float64 attention for q[B][Hq][D] over an encoded cache (from encode_cache).

    ``heads``: optional list of (b, hq) pairs to compute; others stay NaN.
    """
    q = np.asarray(q, dtype=np.float32)
    B, Hq, D = q.shape
    G = Hq // n_kv_heads
    out = np.full((B, Hq, D), np.nan)
    want = None if heads is None else set(heads)
    for b in range(B):
        for h in range(n_kv_heads):
            hq = [h * G + g for g in range(G)]
            if want is not None:
                hq = [x for x in hq if (b, x) in want]
                if not hq:
                    continue
            Kr = enc[(b, h, 0)].recon
            Vr = enc[(b, h, 1)].recon
            res = attention_f64(q[b, hq], Kr, Vr, scale)
            out[b, hq] = res
    return out
