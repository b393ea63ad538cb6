"""Pins of the oracle's Q4-keyframe variant (keyframes stored as Q4_0 of their
absolute values, every other row as Q4_0 of its closed-loop delta, so every
row takes the 4-bit storage of plain Q4_0: Delta-KV article, sections
"핵심 아이디어" and "벤치마크").

Each pin is a fact fixed outside the variant's own routine: plain Q4_0 (itself
pinned to hand-worked blocks), the fp16-keyframe Delta-KV oracle (pinned in
test_oracle.py), a hand-worked three-row stream, and the error decay that the
closed loop guarantees for a constant sequence.
"""
import numpy as np
import pytest

import oracle
from quantized_decode_attention_delta_amd import synth


def _walk(S, D, seed, sigma=0.01):
    rng = np.random.default_rng(seed)
    x = np.cumsum(rng.standard_normal((S, D)) * sigma, axis=0) + rng.standard_normal(D)
    return x.astype(np.float16)


@pytest.mark.parametrize("S,D", [(1, 32), (37, 64), (100, 128)])
def test_kf1_is_plain_q4_0(S, D):
    """kf = 1: every row is a keyframe, so the stream is plain Q4_0 of the
    absolute rows, byte for byte, and decodes to Q4_0's dequantised values."""
    x = _walk(S, D, S)
    e = oracle.q4k_encode_stream(x, 1)
    codes, scales = oracle.q40_abs_stream(x)
    assert np.array_equal(e.codes, codes)
    assert np.array_equal(e.scales, scales)
    assert np.array_equal(e.recon, oracle.q40_dequant_stream(codes, scales))
    assert np.array_equal(oracle.q4k_reconstruct_stream(e.codes, e.scales, 1), e.recon)


@pytest.mark.parametrize("kf", [2, 7, 32, 128])
def test_keyframe_rows_are_q4_0_of_the_row(kf):
    """At every multiple of kf the row is coded against zero, whatever came
    before: its codes and scales are plain Q4_0 of that row alone."""
    x = _walk(300, 64, kf)
    e = oracle.q4k_encode_stream(x, kf)
    keys = np.arange(0, 300, kf)
    codes, scales = oracle.q40_abs_stream(x[keys])
    assert np.array_equal(e.codes[keys], codes)
    assert np.array_equal(e.scales[keys], scales)
    assert np.array_equal(e.recon[keys], oracle.q40_dequant_stream(codes, scales))


def _representable_rows(n, D, rng):
    """Rows that Q4_0 stores exactly: a power-of-two scale s, codes 1..15 and
    one code 0 (the row's largest magnitude, -8 s) at the first channel of each
    block, so the block quantiser finds m = -8 s, s exactly, and every code."""
    rows = np.zeros((n, D), np.float32)
    for i in range(n):
        for b in range(D // 32):
            s = 2.0 ** int(rng.integers(-6, 2)) * (1 if rng.random() < 0.5 else -1)
            c = rng.integers(1, 16, 32)
            c[0] = 0
            rows[i, 32 * b:32 * b + 32] = (c - 8) * s
    return rows.astype(np.float16)


@pytest.mark.parametrize("kf", [4, 32])
def test_exact_keyframes_reduce_to_delta_kv(kf):
    """When every keyframe row is exactly representable in Q4_0, the decoder
    starts each group from the exact row, as the fp16-keyframe Delta-KV codec
    does: every delta row's codes and scales, and every reconstruction, equal
    that oracle's."""
    rng = np.random.default_rng(kf)
    S, D = 5 * kf + 3, 64
    x = _walk(S, D, 7 + kf).astype(np.float32)
    keys = np.arange(0, S, kf)
    x[keys] = _representable_rows(len(keys), D, rng).astype(np.float32)
    x = x.astype(np.float16)
    q = oracle.q4k_encode_stream(x, kf)
    d = oracle.encode_stream(x, kf)
    assert np.array_equal(q.recon[keys], x[keys].astype(np.float32))
    delta = np.array([t for t in range(S) if t % kf])
    di = [oracle.delta_index(int(t), kf) for t in delta]
    assert np.array_equal(q.codes[delta], d.codes[di])
    assert np.array_equal(q.scales[delta], d.scales[di])
    assert np.array_equal(q.recon, d.recon)


def test_constant_sequence_after_an_exact_keyframe_is_exact():
    rng = np.random.default_rng(3)
    row = _representable_rows(1, 128, rng)[0]
    x = np.tile(row, (40, 1))
    e = oracle.q4k_encode_stream(x, 16)
    assert np.array_equal(e.recon, x.astype(np.float32))
    # every delta is zero: scale +-0 (m = +0 gives m / -8 = -0), code 8
    delta = [t for t in range(40) if t % 16]
    assert not (e.scales[delta] & 0x7FFF).any()
    assert np.all(oracle.q40_unpack(e.codes[delta[0], :16]) == 8)


def test_constant_sequence_error_decays_geometrically():
    """A constant row whose keyframe is not exact: each closed-loop delta
    quantises the remaining error, so the largest error falls by at least 8
    per token (a block's error is at most its scale |m|/8, the clamp at code
    15 included), down to fp32 rounding of the reconstruction."""
    rng = np.random.default_rng(11)
    row = rng.standard_normal(128).astype(np.float16)
    x = np.tile(row, (12, 1))
    e = oracle.q4k_encode_stream(x, 64)
    err = np.abs(e.recon - x.astype(np.float32)).max(axis=1)
    assert err[0] > 0
    floor = 2.0 ** -22 * float(np.abs(row.astype(np.float32)).max())
    for t in range(1, 12):
        assert err[t] <= err[t - 1] / 8 * (1 + 2.0 ** -9) + floor, (t, err[t - 1], err[t])
    assert err[-1] <= floor


def test_hand_worked_stream():
    """D = 32, kf = 2, three rows worked by hand:
    row 0 (keyframe): channel 0 = -1, others 0.5 -> m = -1, s = 0.125,
      codes 0 and 12, reconstruction exact;
    row 1 (delta): channel 0 moves by +0.25 -> d = 0.25 at channel 0 only,
      s = -0.03125, code 0 there and 8 elsewhere, reconstruction exact;
    row 2 (keyframe again, coded against zero, not against row 1): channel 5
      = 3, others 0 -> m = 3, s = -0.375, code 0 at channel 5, 8 elsewhere."""
    x = np.zeros((3, 32), np.float32)
    x[0] = 0.5
    x[0, 0] = -1.0
    x[1] = x[0]
    x[1, 0] = -0.75
    x[2, 5] = 3.0
    x = x.astype(np.float16)
    e = oracle.q4k_encode_stream(x, 2)
    f16 = lambda v: int(np.float16(v).view(np.uint16))  # noqa: E731
    assert [int(s) for s in e.scales[:, 0]] == [f16(0.125), f16(-0.03125), f16(-0.375)]
    c0 = oracle.q40_unpack(e.codes[0])
    assert c0[0] == 0 and np.all(c0[1:] == 12)
    c1 = oracle.q40_unpack(e.codes[1])
    assert c1[0] == 0 and np.all(c1[1:] == 8)
    c2 = oracle.q40_unpack(e.codes[2])
    assert c2[5] == 0 and np.all(np.delete(c2, 5) == 8)
    assert np.array_equal(e.recon, x.astype(np.float32))


def test_append_equals_prefill_and_decoder_equals_encoder():
    x = _walk(150, 64, 5)
    full = oracle.q4k_encode_stream(x, 32)
    part = oracle.q4k_encode_stream(x[:61], 32)
    grown = oracle.Q4KStream(150, 64, 32)
    grown.codes[:61], grown.scales[:61] = part.codes, part.scales
    xh = part.state.copy()
    for t in range(61, 150):
        oracle.q4k_step(grown, x[t], t, xh)
    assert np.array_equal(grown.codes, full.codes)
    assert np.array_equal(grown.scales, full.scales)
    assert np.array_equal(xh, full.state)
    assert np.array_equal(oracle.q4k_reconstruct_stream(full.codes, full.scales, 32), full.recon)


def test_q4k_cache_attention_matches_brute_force():
    """attention_cache over a Q4-keyframe cache is float64 softmax attention
    over its reconstruction (checked against a direct numpy evaluation)."""
    w = synth.make("8b", S=90, B=2, Hq=4, Hkv=2, D=64)
    enc = oracle.q4k_encode_cache(w.k, w.v, w.seq_lens, 32)
    q = synth.queries(w)
    scale = 1 / np.sqrt(w.D)
    out = oracle.attention_cache(enc, q, w.seq_lens, w.Hkv, scale)
    for b in range(w.B):
        for hq in range(w.Hq):
            h = hq // (w.Hq // w.Hkv)
            K = enc[(b, h, 0)].recon.astype(np.float64)
            V = enc[(b, h, 1)].recon.astype(np.float64)
            lg = float(np.float32(scale)) * (K @ q[b, hq].astype(np.float64))
            p = np.exp(lg - lg.max())
            ref = (p @ V) / p.sum()
            assert np.allclose(out[b, hq], ref, rtol=1e-12, atol=1e-12)
