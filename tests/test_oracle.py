"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test checks the oracle against a value worked out by hand, a closed form,
an invariant of the method, a special case that reduces to a library routine
(numpy's fp16 rounding, torch's scaled-dot-product attention in float64), or
the error bound that the closed-loop design guarantees.  None of them re-types
the oracle's own formulas.
"""
import math
import os

import numpy as np
import pytest

import oracle
from quantized_decode_attention_delta_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ fp16
def test_f16_to_f32_exhaustive_vs_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(b)) for b in bits], np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_f32_to_f16_rne_vs_numpy():
    rng = np.random.default_rng(1)
    vals = [0.0, -0.0, 65504.0, 65519.99, 65520.0, -65520.0, 1e9, 2.0 ** -24, 2.0 ** -25,
            3 * 2.0 ** -26, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 0.1, -0.1, 1 / 3]
    x = np.concatenate([
        np.array(vals, np.float32),
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 5, 20000),
        # every fp16 value and every halfway point between neighbours
        (np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)),
        ((np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
          + np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)) / 2).astype(np.float32),
    ]).astype(np.float32)
    x = np.concatenate([x, -x])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(v)) for v in x], np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


# ------------------------------------------------------------------ Q4_0 block
def _golden_blocks():
    cases = []
    with open(os.path.join(GOLDEN, "q40_hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, ins, scale, codes, packed, deq = [p.strip() for p in line.split("|")]

            def kv(s, conv):
                return {int(a): conv(b) for a, b in (t.split(":") for t in s.split())} if s else {}

            cases.append((name, kv(ins, float), int(scale, 16), kv(codes, int),
                          kv(packed, lambda h: int(h, 16)), kv(deq, float)))
    return cases


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c[0])
def test_q40_hand_worked_blocks(case):
    name, ins, scale, code_over, byte_over, deq_over = case
    v = np.zeros(32, np.float32)
    for i, val in ins.items():
        v[i] = val
    s16, codes = oracle.q40_block(v)
    assert s16 == scale, hex(s16)
    want_codes = np.full(32, 8, np.uint8)
    for i, c in code_over.items():
        want_codes[i] = c
    assert np.array_equal(codes, want_codes)
    want_bytes = np.full(16, 0x88, np.uint8)
    for i, b in byte_over.items():
        want_bytes[i] = b
    assert np.array_equal(oracle.q40_pack(codes), want_bytes)
    assert np.array_equal(oracle.q40_unpack(want_bytes), want_codes)
    sf = np.array([scale], np.uint16).view(np.float16).astype(np.float32)[0]
    deq = (codes.astype(np.float32) - 8) * sf
    want_deq = np.zeros(32, np.float32)
    for i, d in deq_over.items():
        want_deq[i] = d
    assert np.array_equal(deq, want_deq)


def _rand_blocks(n, seed):
    rng = np.random.default_rng(seed)
    mags = np.float32(10.0) ** rng.uniform(-6, 4, (n, 1)).astype(np.float32)
    v = (rng.standard_normal((n, 32)).astype(np.float32) * mags).astype(np.float32)
    # sprinkle exact ties and zeros
    v[::7, 5] = -v[::7, 9]
    v[::11, :16] = 0.0
    return v


def test_q40_invariants():
    """Power-of-two scaling and negation are exact symmetries of Q4_0; the
    argmax element always maps to code 0; codes are nibbles."""
    for v in _rand_blocks(400, 3):
        s, c = oracle.q40_block(v)
        assert c.max() <= 15
        a = np.abs(v)
        if a.max() > 0:
            am = int(np.argmax(a))      # numpy argmax: first index of the max
            assert c[am] == 0
            sf = np.float16(np.array([s], np.uint16).view(np.float16)[0])
            assert np.sign(sf) == -np.sign(v[am])
        s2, c2 = oracle.q40_block(-v)
        assert np.array_equal(c2, c) and s2 == (s ^ 0x8000)
        s4, c4 = oracle.q40_block(v * np.float32(4.0))
        assert np.array_equal(c4, c)
        f = np.array([s], np.uint16).view(np.float16).astype(np.float64)[0]
        f4 = np.array([s4], np.uint16).view(np.float16).astype(np.float64)[0]
        if 2.0 ** -13 < abs(f) < 2.0 ** 13:     # normal range on both sides: exact
            assert f4 == 4 * f


def test_q40_nearest_level_vs_bruteforce():
    """Each non-clamped code selects the grid level (c-8)*s32 nearest to the
    value (ties upward), checked by brute force over all 16 levels."""
    for v in _rand_blocks(300, 5):
        s, c = oracle.q40_block(v)
        a = np.abs(v.astype(np.float64))
        if a.max() == 0:
            assert np.all(c == 8)
            continue
        m = float(v[np.argmax(a)])
        s32 = m / -8.0
        levels = (np.arange(16) - 8) * s32
        for j in range(32):
            err = np.abs(levels - float(v[j]))
            best = err.min()
            if c[j] == 15 and abs(float(v[j]) - 8 * s32) <= abs(s32) * 0.5 + 1e-6 * abs(s32):
                continue   # value beyond the top level: clamped
            assert err[c[j]] <= best + 1e-5 * abs(s32), (j, c[j], err)


# ------------------------------------------------------------------ stream codec
def _rand_walk(S, D, seed, rel=0.01):
    rng = np.random.default_rng(seed)
    x = np.zeros((S, D), np.float64)
    x[0] = rng.standard_normal(D)
    for t in range(1, S):
        x[t] = x[t - 1] + rel * rng.standard_normal(D)
    return x.astype(np.float16)


def test_kf1_reconstructs_fp16_exactly():
    """kf = 1: every token is a keyframe, so the cache is the fp16 rows."""
    x = _rand_walk(50, 64, 7)
    e = oracle.encode_stream(x, 1)
    assert e.codes.shape[0] == 0 and e.kf_rows.shape == (50, 64)
    assert np.array_equal(e.recon, x.astype(np.float32))
    assert np.array_equal(e.kf_rows, x.view(np.uint16))


def test_zero_keyframe_gives_plain_q40_of_absolute_values():
    """With an all-zero keyframe, the first delta is the token itself, so its
    block equals Q4_0 of the absolute values (the plain Q4_0 cache)."""
    rng = np.random.default_rng(9)
    x = np.zeros((2, 128), np.float16)
    x[1] = rng.standard_normal(128).astype(np.float16)
    e = oracle.encode_stream(x, 4)
    codes, scales = oracle.q40_abs_stream(x[1:2])
    assert np.array_equal(e.codes[0], codes[0]) and np.array_equal(e.scales[0], scales[0])


def test_constant_sequence_is_exact_after_keyframe():
    x = np.tile(_rand_walk(1, 128, 11), (70, 1))
    e = oracle.encode_stream(x, 32)
    assert np.array_equal(e.recon, x.astype(np.float32))
    assert np.all(e.codes == 0x88) and np.all(e.scales == 0x8000)


def test_worked_two_token_example():
    """D=32, kf=4: x0 = 1 everywhere, x1 = x0 but x1[0] = 1.5, x2 = x1.
    Delta of token 1 is 0.5 at channel 0: scale -0.0625 (0xAC00), code 0 there,
    reconstruction exact; token 2 repeats token 1, giving the all-zero block."""
    x = np.ones((3, 32), np.float16)
    x[1, 0] = 1.5
    x[2] = x[1]
    e = oracle.encode_stream(x, 4)
    assert list(e.scales[:, 0]) == [0xAC00, 0x8000]
    assert e.codes[0, 0] == 0x80 and np.all(e.codes[0, 1:] == 0x88)
    assert np.all(e.codes[1] == 0x88)
    assert np.array_equal(e.recon, x.astype(np.float32))


def _scale_f32(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("kf", [2, 32, 512])
def test_error_bound_at_every_token(kf):
    """Closed loop: at every token the reconstruction error is the current
    block's quantisation error only (it does not grow with the distance from
    the keyframe, the stability claim of the Delta-KV article)."""
    x = _rand_walk(1100, 64, 13 + kf)
    e = oracle.encode_stream(x, kf)
    xf = x.astype(np.float64)
    for t in range(x.shape[0]):
        if t % kf == 0:
            assert np.array_equal(e.recon[t], x[t].astype(np.float32))
            continue
        di = oracle.delta_index(t, kf)
        d = xf[t] - e.recon[t - 1].astype(np.float64)
        for b in range(2):
            s16 = _scale_f32(e.scales[di, b])
            blk = d[32 * b:32 * b + 32]
            m = blk[np.argmax(np.abs(blk))]
            s32 = m / -8.0
            slack = abs(s16 - s32) * 8 + 4 * np.spacing(np.float32(np.abs(xf[t, 32 * b:32 * b + 32]).max() + 1e-30))
            err = np.abs(xf[t, 32 * b:32 * b + 32] - e.recon[t, 32 * b:32 * b + 32])
            codes = oracle.q40_unpack(e.codes[di, 16 * b:16 * b + 16])
            bound = np.where(codes == 15, abs(s16), abs(s16) / 2) + slack
            assert np.all(err <= bound + 1e-12), (t, b)


def test_decoder_matches_encoder_and_state():
    x = _rand_walk(333, 128, 17)
    for kf in (1, 3, 32, 100):
        e = oracle.encode_stream(x, kf)
        r = oracle.reconstruct_stream(e.kf_rows, e.codes, e.scales, e.S, e.D, kf)
        assert np.array_equal(r, e.recon)
        assert np.array_equal(e.state, e.recon[-1])


def test_prefill_equals_token_by_token_appends():
    x = _rand_walk(97, 64, 19)
    kf = 16
    e = oracle.encode_stream(x, kf)
    a = oracle.EncodedStream(97, 64, kf)
    xh = np.zeros(64, np.float32)
    for t in range(97):
        oracle.step(a, x[t], t, xh)
    assert np.array_equal(a.codes, e.codes) and np.array_equal(a.scales, e.scales)
    assert np.array_equal(a.kf_rows, e.kf_rows) and np.array_equal(xh, e.state)


def test_open_loop_would_drift_but_closed_loop_does_not():
    """The stability claim separates closed from open loop: quantising raw
    token-to-token differences drifts like a random walk over 512 deltas,
    while the oracle's error stays at the single-step level."""
    x = _rand_walk(512, 64, 23)
    e = oracle.encode_stream(x, 512)
    err_closed = np.abs(e.recon.astype(np.float64) - x.astype(np.float64))
    # open loop, built from the plain Q4_0 of each raw difference
    xf = x.astype(np.float32)
    diffs = np.diff(xf, axis=0).astype(np.float16)   # fp16 only to reuse the abs quantiser
    codes, scales = oracle.q40_abs_stream(diffs)
    deq = oracle.q40_dequant_stream(codes, scales)
    open_rec = np.concatenate([xf[:1], xf[:1] + np.cumsum(deq, axis=0)])
    err_open = np.abs(open_rec - xf)
    assert err_closed[400:].max() < 0.5 * err_open[400:].max()
    assert err_closed[400:].max() < 3 * err_closed[1:50].max()


def test_byte_count_formula():
    """Bytes per stream: 2*D per keyframe + 18 bytes per 32 delta elements
    (e.g. 2,488 bytes per 32-token group at D=128)."""
    x = _rand_walk(64, 128, 29)
    e = oracle.encode_stream(x, 32)
    per_group = e.kf_rows[0].nbytes + 31 * (e.codes[0].nbytes + e.scales[0].nbytes)
    assert per_group == 2488
    S = 1000
    for kf in (1, 32, 128, 512):
        ng = math.ceil(S / kf)
        assert oracle.n_delta(S, kf) == S - ng


# ------------------------------------------------------------------ attention
def _sdpa_f64(q, K, V, scale):
    import torch
    qt = torch.from_numpy(q.astype(np.float64))[None, :, None, :]        # [1][G][1][D]
    kt = torch.from_numpy(K.astype(np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    vt = torch.from_numpy(V.astype(np.float64))[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(), scale=float(scale))
    return o[0, :, 0].numpy()


@pytest.mark.parametrize("G,S,D", [(1, 1, 64), (4, 37, 64), (8, 256, 64), (4, 200, 128)])
def test_attention_vs_torch_sdpa_f64(G, S, D):
    rng = np.random.default_rng(G * 1000 + S)
    q = rng.standard_normal((G, D)).astype(np.float32)
    K = (rng.standard_normal((S, D)) * 2).astype(np.float32)
    V = rng.standard_normal((S, D)).astype(np.float32)
    scale = np.float32(1 / math.sqrt(D))
    got = oracle.attention_f64(q, K, V, scale)
    ref = _sdpa_f64(q, K, V, scale)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(31)
    D = 64
    q = rng.standard_normal((3, D)).astype(np.float32)
    V = rng.standard_normal((5, D)).astype(np.float32)
    # one token: the output is that token's value row
    o = oracle.attention_f64(q, rng.standard_normal((1, D)).astype(np.float32), V[:1], 0.125)
    assert np.array_equal(o, np.repeat(V[:1].astype(np.float64), 3, 0))
    # identical keys: uniform weights, the mean of V
    K = np.repeat(rng.standard_normal((1, D)).astype(np.float32), 5, 0)
    o = oracle.attention_f64(q, K, V, 0.125)
    np.testing.assert_allclose(o, np.repeat(V.astype(np.float64).mean(0, keepdims=True), 3, 0), rtol=1e-12, atol=1e-14)
    # two tokens whose logits differ by exactly ln 3: weights 3/4 and 1/4
    q1 = np.zeros((1, D), np.float32)
    q1[0, 0] = 1.0
    K2 = np.zeros((2, D), np.float32)
    K2[0, 0] = np.float32(math.log(3.0))
    o = oracle.attention_f64(q1, K2, V[:2], 1.0)
    l = float(K2[0, 0])
    w = math.exp(l) / (math.exp(l) + 1)
    np.testing.assert_allclose(o[0], w * V[0].astype(np.float64) + (1 - w) * V[1].astype(np.float64), rtol=1e-12, atol=1e-14)
    # empty sequence: zero row
    assert np.all(oracle.attention_f64(q, np.zeros((0, D), np.float32), np.zeros((0, D), np.float32), 0.1) == 0)


def test_attention_head_permutation_equivariance():
    rng = np.random.default_rng(37)
    q = rng.standard_normal((8, 64)).astype(np.float32)
    K = rng.standard_normal((50, 64)).astype(np.float32)
    V = rng.standard_normal((50, 64)).astype(np.float32)
    perm = rng.permutation(8)
    a = oracle.attention_f64(q, K, V, 0.2)
    b = oracle.attention_f64(q[perm], K, V, 0.2)
    assert np.array_equal(a[perm], b)


def test_attention_over_cache_matches_per_stream():
    w = synth.make("8b", B=1, S=100, Hq=8, Hkv=2)
    enc = oracle.encode_cache(w.k, w.v, w.seq_lens, w.kf)
    q = synth.queries(w)
    out = oracle.attention_cache(enc, q, w.seq_lens, w.Hkv, 1 / math.sqrt(w.D))
    ref = _sdpa_f64(q[0, 4:8], enc[(0, 1, 0)].recon, enc[(0, 1, 1)].recon, np.float32(1 / math.sqrt(w.D)))
    np.testing.assert_allclose(out[0, 4:8], ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ statistics
def test_delta_mse_far_below_q40_on_slow_walks():
    """Statistical sanity, not parity: with ~1% token-to-token changes the
    delta range is ~100x smaller than the absolute range, so the squared
    error drops by orders of magnitude against plain Q4_0."""
    w = synth.make("70b", B=1, Hkv=1, Hq=1, S=2048)
    x = w.k[0, 0]
    e = oracle.encode_stream(x, 32)
    codes, scales = oracle.q40_abs_stream(x)
    deq = oracle.q40_dequant_stream(codes, scales)
    xf = x.astype(np.float64)
    mse_d = np.mean((e.recon - xf) ** 2)
    mse_q = np.mean((deq - xf) ** 2)
    assert mse_d < mse_q / 100, (mse_d, mse_q)


# ------------------------------------------------ attention-preserving distortion
# ("KV 캐시 벡터 양자화와 주의 보존 변환", 어텐션 보존 왜곡): closed forms that pin
# every part of the definition -- the squared logit error, the softmax scale,
# the weights taken on the exact keys, and the normalisation of the weights.

def _dist_inputs(S=7, D=32, G=3, seed=5):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((G, D)).astype(np.float32)
    K = rng.standard_normal((S, D)).astype(np.float16).astype(np.float64)
    V = rng.standard_normal((S, D)).astype(np.float16).astype(np.float64)
    return q, K, V


def test_distortion_zero_when_exact():
    q, K, V = _dist_inputs()
    d_k, d_v = oracle.attention_distortion_f64(q, K, V, K.copy(), V.copy(), 0.3)
    assert np.all(d_k == 0) and np.all(d_v == 0)


def test_distortion_key_offset_closed_form():
    # K_hat = K + delta * e_c for every token: d_k = S * (q_c * delta)^2 per head,
    # and d_v stays 0 (the weights use the exact keys, V_hat = V)
    q, K, V = _dist_inputs()
    S, c, delta = K.shape[0], 5, 0.125
    Kh = K.copy()
    Kh[:, c] += delta
    d_k, d_v = oracle.attention_distortion_f64(q, K, V, Kh, V, 0.3)
    np.testing.assert_allclose(d_k, S * (q[:, c].astype(np.float64) * delta) ** 2, rtol=1e-12)
    assert np.all(d_v == 0)


def test_distortion_value_offset_closed_form():
    # V_hat = V + Delta for every token: the weights sum to 1, so d_v = ||Delta||^2
    q, K, V = _dist_inputs()
    Delta = np.linspace(-0.5, 0.5, V.shape[1])
    d_k, d_v = oracle.attention_distortion_f64(q, K, V, K, V + Delta, 0.3)
    np.testing.assert_allclose(d_v, np.full(q.shape[0], (Delta ** 2).sum()), rtol=1e-12)
    assert np.all(d_k == 0)


def test_distortion_two_tokens_logistic_weight():
    # error only in V_0, channel 0, size 1: d_v = a_0^2 with a_0 the logistic of
    # scale * q.(K_0 - K_1) on the EXACT keys (K_hat is perturbed to catch a
    # definition that takes the weights from the reconstruction)
    q, K, V = _dist_inputs(S=2, D=32, G=2)
    scale = 0.7
    Vh = V.copy()
    Vh[0, 0] += 1.0
    Kh = K + 0.25
    _, d_v = oracle.attention_distortion_f64(q, K, V, Kh, Vh, scale)
    # the scale is an fp32 value, as it crosses the C ABI
    z = float(np.float32(scale)) * (q.astype(np.float64) @ (K[0] - K[1]))
    a0 = 1.0 / (1.0 + np.exp(-z))
    np.testing.assert_allclose(d_v, a0 ** 2, rtol=1e-12)


def test_distortion_single_token_and_empty():
    q, K, V = _dist_inputs(S=1)
    Kh, Vh = K + 0.01, V - 0.02
    d_k, d_v = oracle.attention_distortion_f64(q, K, V, Kh, Vh, 0.3)
    np.testing.assert_allclose(d_k, (q.astype(np.float64) @ (Kh[0] - K[0])) ** 2, rtol=1e-12)
    np.testing.assert_allclose(d_v, np.full(q.shape[0], ((Vh[0] - V[0]) ** 2).sum()), rtol=1e-12)
    e = np.zeros((0, K.shape[1]))
    d_k, d_v = oracle.attention_distortion_f64(q, e, e, e, e, 0.3)
    assert np.all(d_k == 0) and np.all(d_v == 0)


# ---------------------------------------------------------------- Q8_0 comparison
# The 8-bit reference of the Delta-KV article's "벤치마크" section, under the
# documented rule of that format: d = max|v| / 127, code = round-half-away(v/d),
# scale stored as fp16(d).  Values below are worked by hand.

def test_q80_hand_blocks():
    # single spike 1.0: d = 1/127 = 0.0078740..., fp16 RNE: 2^-7 * (1 + 8/1024) -> 0x2008
    d, c = oracle.q80_block(np.array([1.0] + [0.0] * 31, np.float32))
    assert d == 0x2008 and c[0] == 127 and not c[1:].any()
    # d = 1 exactly (max 127): ties round away from zero, both signs
    v = np.zeros(32, np.float32)
    v[:7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.49, -126.5]
    d, c = oracle.q80_block(v)
    assert d == 0x3C00
    assert list(c[:7]) == [127, 3, -3, 1, -1, 1, -127]
    # all zero: scale +0, codes 0
    d, c = oracle.q80_block(np.zeros(32, np.float32))
    assert d == 0x0000 and not c.any()


def test_q80_error_bound_and_symmetry():
    rng = np.random.default_rng(11)
    for trial in range(300):
        v = (rng.standard_normal(32) * 10.0 ** rng.uniform(-3, 3)).astype(np.float16).astype(np.float32)
        d16, c = oracle.q80_block(v)
        d = np.float64(np.float32(np.abs(v).max()) / np.float32(127.0))
        ds = np.float64(oracle.f16_to_f32(d16))
        assert np.abs(c.astype(np.int64)).max() <= 127
        err = np.abs(v.astype(np.float64) - c.astype(np.float64) * ds)
        bound = d / 2 * (1 + 1e-6) + 127 * abs(d - ds)
        assert np.all(err <= bound + 1e-12), (trial, err.max(), bound)
        d16n, cn = oracle.q80_block(-v)
        assert d16n == d16 and np.array_equal(cn, -c)


def test_q80_stream_matches_blocks():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 64)).astype(np.float16)
    codes, scales = oracle.q80_abs_stream(x)
    for t in range(5):
        for b in range(2):
            d, c = oracle.q80_block(x[t, 32 * b:32 * b + 32].astype(np.float32))
            assert scales[t, b] == d and np.array_equal(codes[t, 32 * b:32 * b + 32], c)
    deq = oracle.q80_dequant_stream(codes, scales)
    sc = np.repeat(scales.view(np.float16).astype(np.float32), 32, axis=1)
    assert np.array_equal(deq, codes.astype(np.float32) * sc)


# ------------------------------------------------ dequantisers, pinned by hand
# The dequantised value of a Q4_0 code c under stored scale s16 is
# (c - 8) * float(s16); of a Q8_0 code c it is c * float(s16).  The blocks
# below are fed to the oracle's stream dequantisers as raw bytes and fp16
# scale bits, and every output is compared with a value written out by hand.

def test_q40_dequant_stream_golden_blocks():
    """Every hand-worked block of tests/golden/q40_hand_blocks.txt, as packed
    bytes + scale bits, dequantises to its golden values.  Blocks are laid two
    per row (D = 64) in a 3-row stream, so a wrong block or row index, a
    missing scale or a wrong code offset changes some value."""
    cases = _golden_blocks()
    assert len(cases) == 6
    codes = np.full((3, 32), 0x88, np.uint8)
    scales = np.zeros((3, 2), np.uint16)
    want = np.zeros((3, 64), np.float32)
    for i, (name, ins, scale, code_over, byte_over, deq_over) in enumerate(cases):
        t, b = divmod(i, 2)
        for j, by in byte_over.items():
            codes[t, 16 * b + j] = by
        scales[t, b] = scale
        for j, d in deq_over.items():
            want[t, 32 * b + j] = d
    got = oracle.q40_dequant_stream(codes, scales)
    assert got.dtype == np.float32 and got.shape == (3, 64)
    assert np.array_equal(got, want), np.argwhere(got != want)


def test_q40_dequant_stream_every_code_literal():
    """All 16 codes under a negative and a positive scale, written out: block 0
    has byte i = i | (15 - i) << 4 (low nibbles code i, high nibbles code
    15 - i) with scale -2.0 (0xC000); block 1 repeats the bytes with scale
    0.25 (0x3400)."""
    row = np.array([i | ((15 - i) << 4) for i in range(16)], np.uint8)
    codes = np.concatenate([row, row])[None, :]
    scales = np.array([[0xC000, 0x3400]], np.uint16)
    want_b0 = [16, 14, 12, 10, 8, 6, 4, 2, 0, -2, -4, -6, -8, -10, -12, -14,
               -14, -12, -10, -8, -6, -4, -2, 0, 2, 4, 6, 8, 10, 12, 14, 16]
    want_b1 = [-2.0, -1.75, -1.5, -1.25, -1.0, -0.75, -0.5, -0.25, 0.0, 0.25, 0.5, 0.75, 1.0, 1.25, 1.5, 1.75,
               1.75, 1.5, 1.25, 1.0, 0.75, 0.5, 0.25, 0.0, -0.25, -0.5, -0.75, -1.0, -1.25, -1.5, -1.75, -2.0]
    got = oracle.q40_dequant_stream(codes, scales)
    assert np.array_equal(got[0], np.array(want_b0 + want_b1, np.float32))


def test_q80_dequant_stream_literal():
    """Q8_0 codes times their fp16 scale, written out: block 0 under 1.0
    (0x3C00), block 1 under 0x2008 = 129/16384 (127 * 129/16384 = 16383/16384),
    row 1 under -2.0 (0xC000) and +0 (0x0000)."""
    codes = np.zeros((2, 64), np.int8)
    codes[0, :7] = [127, 3, -3, 1, -1, 0, -127]
    codes[0, 32:35] = [127, -127, 2]
    codes[1, :3] = [-5, 100, -128]
    codes[1, 32:34] = [50, -50]
    scales = np.array([[0x3C00, 0x2008], [0xC000, 0x0000]], np.uint16)
    want = np.zeros((2, 64), np.float64)
    want[0, :7] = [127.0, 3.0, -3.0, 1.0, -1.0, 0.0, -127.0]
    want[0, 32:35] = [16383 / 16384, -16383 / 16384, 258 / 16384]
    want[1, :3] = [10.0, -200.0, 256.0]
    got = oracle.q80_dequant_stream(codes, scales)
    assert np.array_equal(got.astype(np.float64), want), np.argwhere(got != want)


def _gqa_workload(G, seed):
    """B = 2 sequences, Hkv = 3 kv-heads whose K/V differ by head (offsets of
    +4 * head), G query heads per kv-head."""
    rng = np.random.default_rng(seed)
    B, H, S, D = 2, 3, 40, 64
    base = rng.standard_normal((B, H, S, D))
    k = (base + 4.0 * np.arange(H)[None, :, None, None]).astype(np.float16)
    v = (rng.standard_normal((B, H, S, D)) - 3.0 * np.arange(H)[None, :, None, None]).astype(np.float16)
    q = rng.standard_normal((B, H * G, D)).astype(np.float32)
    lens = np.array([S, 23], np.int32)
    return k, v, q, lens, H


@pytest.mark.parametrize("G", [1, 4, 8])
def test_cache_helpers_map_query_head_to_kv_head(G):
    """Query head hq of a group of G reads kv-head hq // G: the cache-level
    helpers (attention_cache, attention_distortion_cache) equal the per-head
    float64 routines called on that kv-head's rows, for every (sequence,
    query head); a mapping such as hq % Hkv would pick another head's K/V."""
    k, v, q, lens, H = _gqa_workload(G, 40 + G)
    enc = oracle.encode_cache(k, v, lens, 8)
    scale = np.float32(0.125)
    att = oracle.attention_cache(enc, q, lens, H, scale)
    dk, dv = oracle.attention_distortion_cache(enc, k, v, q, lens, H, scale)
    for b in range(2):
        S = int(lens[b])
        for hq in range(H * G):
            kv = hq // G
            kr = oracle.reconstruct_stream(enc[(b, kv, 0)].kf_rows, enc[(b, kv, 0)].codes, enc[(b, kv, 0)].scales,
                                           S, 64, 8)
            vr = oracle.reconstruct_stream(enc[(b, kv, 1)].kf_rows, enc[(b, kv, 1)].codes, enc[(b, kv, 1)].scales,
                                           S, 64, 8)
            ref = _sdpa_f64(q[b, hq:hq + 1], kr, vr, scale)
            np.testing.assert_allclose(att[b, hq], ref[0], rtol=1e-12, atol=1e-12)
            e_k, e_v = oracle.attention_distortion_f64(q[b, hq:hq + 1], k[b, kv, :S].astype(np.float64),
                                                       v[b, kv, :S].astype(np.float64), kr, vr, scale)
            np.testing.assert_allclose([dk[b, hq], dv[b, hq]], [e_k[0], e_v[0]], rtol=1e-12, atol=0)
