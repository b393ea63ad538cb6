"""Pins of the oracle's strided-reference residual coding (the gist.science
explainer of DeltaKV, section 3.A: references at a fixed stride, the residual
against the most similar reference, reconstruction as reference + residual).

Each check is independent of the oracle's own arithmetic:
* periodic data whose references cover every phase reconstructs exactly,
  choosing the lowest-index reference of the right phase (closed form);
* the chosen reference is the exact-arithmetic nearest one (fractions over
  the fp16 values; random rows have no near ties);
* the window bound, stride 1 (every token its own reference) and tokens
  before the second reference (only reference 0);
* the stored codes and scales, unpacked here from their nibbles, give the
  reconstruction, and its error stays within half a Q4_0 step (a whole one
  where the code clamps).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rows(rng, n, D, scale=1.0):
    return (rng.standard_normal((n, D)) * scale).astype(np.float16)


def _unpack(codes_row):
    """Canonical Q4_0 bytes -> codes per channel (byte i: code i low, code i+16 high)."""
    D = codes_row.size * 2
    out = np.zeros(D, np.int64)
    for b in range(D // 32):
        by = codes_row[16 * b:16 * b + 16].astype(np.int64)
        out[32 * b:32 * b + 16] = by & 15
        out[32 * b + 16:32 * b + 32] = by >> 4
    return out


def test_periodic_data_finds_exact_references():
    rng = np.random.default_rng(11)
    P, stride, D, S = 5, 3, 32, 40
    T = _rows(rng, P, D)
    x = np.stack([T[t % P] for t in range(S)])
    e = oracle.strided_encode_stream(x, stride)
    for t in range(S):
        ks = [k for k in range(t // stride + 1) if (k * stride) % P == t % P]
        if not ks:
            continue
        assert e.ref_idx[t] == ks[0], t
        assert np.array_equal(e.recon[t], x[t].astype(np.float32)), t
        assert np.all(e.codes[t] == 0x88) and np.all((e.scales[t] & 0x7FFF) == 0), t   # +-0: m = 0 over -8
    # from the fifth reference on every phase is covered
    assert all(e.ref_idx[t] * stride % P == t % P for t in range(12, S))


@pytest.mark.parametrize("window", [0, 3])
def test_choice_is_the_exact_nearest_reference(window):
    rng = np.random.default_rng(12)
    stride, D, S = 4, 32, 50
    x = _rows(rng, S, D)
    e = oracle.strided_encode_stream(x, stride, window)
    xf = [[Fraction(float(v)) for v in row] for row in x]
    for t in range(S):
        kt = t // stride
        k0 = max(0, kt - window + 1) if window > 0 else 0
        d = [sum((a - b) ** 2 for a, b in zip(xf[t], xf[k * stride])) for k in range(k0, kt + 1)]
        best = k0 + min(range(len(d)), key=lambda i: (d[i], i))
        assert e.ref_idx[t] == best, (t, e.ref_idx[t], best)
        assert k0 <= e.ref_idx[t] <= kt


def test_references_are_the_strided_rows_and_reconstruct_exactly():
    rng = np.random.default_rng(13)
    stride, D, S = 8, 64, 70
    x = _rows(rng, S, D, 3.0)
    e = oracle.strided_encode_stream(x, stride)
    assert e.refs.shape == (9, D)
    for k in range(9):
        assert np.array_equal(e.refs[k], x[k * stride].view(np.uint16))
        assert np.array_equal(e.recon[k * stride], x[k * stride].astype(np.float32))
    assert np.all(e.ref_idx[:stride] == 0)


def test_stride_one_is_lossless():
    rng = np.random.default_rng(14)
    x = _rows(rng, 20, 32)
    e = oracle.strided_encode_stream(x, 1)
    assert np.array_equal(e.recon, x.astype(np.float32))
    assert np.array_equal(e.ref_idx, np.arange(20))


@pytest.mark.parametrize("window", [0, 2])
def test_stored_residual_decodes_to_recon_within_half_a_step(window):
    rng = np.random.default_rng(15)
    stride, D, S = 4, 64, 60
    x = (np.cumsum(rng.standard_normal((S, D)) * 0.1, axis=0) + rng.standard_normal(D)).astype(np.float16)
    e = oracle.strided_encode_stream(x, stride, window)
    for t in range(S):
        r = e.refs[e.ref_idx[t]].view(np.float16).astype(np.float32)
        c = _unpack(e.codes[t])
        sf = e.scales[t].view(np.float16).astype(np.float32)
        dec = np.empty(D, np.float32)
        for b in range(D // 32):
            dec[32 * b:32 * b + 32] = r[32 * b:32 * b + 32] + (c[32 * b:32 * b + 32] - 8).astype(np.float32) * sf[b]
        assert np.array_equal(dec, e.recon[t]), t
        err = np.abs(e.recon[t].astype(np.float64) - x[t].astype(np.float64))
        # half a step, a whole one where the code clamps at 15 (a value of the
        # sign opposite to the block's largest one), plus the fp16 scale rounding
        step = np.repeat(np.abs(sf.astype(np.float64)), 32)
        bound = step * (np.where(c == 15, 1.0, 0.5) + 2.0 ** -6) + 1e-6
        assert np.all(err <= bound), t


def test_sqdist_closed_form():
    a = np.array([1.0, -2.0, 0.5, 0.0], np.float16)
    b = np.array([0.0, 1.0, 0.5, -3.0], np.float16)
    assert oracle.sqdist_f16(a, b) == 1.0 + 9.0 + 0.0 + 9.0


def test_rows_with_inf_or_nan_take_a_defined_reference():
    """Non-finite rows (outside the cache's finite-input contract) still pick
    one defined reference: a NaN distance ranks above every number, +inf
    included, and the lowest index wins among equals.  Stride 2, D = 32:
      t = 3 holds a NaN: every distance is NaN, so reference 0;
      t = 5 holds +inf: every distance is +inf (references finite), so 0;
      t = 6 is reference 3 itself, whose row holds -inf in channel 1: its
        distance to itself is NaN (-inf - -inf), to references 0..2 +inf, so
        reference 0;
      t = 9 (window 2: references 3 and 4) is finite: reference 3 (the -inf
        row) is at distance +inf, so reference 4 is chosen."""
    D = 32
    x = np.zeros((10, D), np.float16)
    x[:, 0] = np.arange(10, dtype=np.float16)
    x[3, 7] = np.float16("nan")
    x[5, 2] = np.float16("inf")
    x[6, 1] = -np.float16("inf")
    got = oracle.strided_encode_stream(x, 2, window=0).ref_idx
    assert got[3] == 0 and got[5] == 0 and got[6] == 0
    got_w = oracle.strided_encode_stream(x, 2, window=2).ref_idx
    assert got_w[9] == 4
    # a NaN distance must not stick as the running best: t = 9 with window 3
    # sees references 2, 3, 4 in that order; 2 and 4 are finite, 4 is nearer
    x2 = x.copy()
    x2[4, 3] = np.float16("nan")       # reference 2 (t = 4) now at NaN distance
    assert oracle.strided_encode_stream(x2, 2, window=3).ref_idx[9] == 4
    x2[8, 3] = np.float16("nan")       # reference 4 too: only reference 3 (+inf) is left ranked
    assert oracle.strided_encode_stream(x2, 2, window=3).ref_idx[9] == 3
