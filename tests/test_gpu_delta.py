"""GPU parity of the Delta-KV path against the CPU oracle, through the C ABI.

Codec results (keyframes, Q4_0 codes, fp16 scale bit patterns, reconstructed
K/V, recon state) must be bit-exact; decode attention must be within 2e-3 max
relative error per output row of the float64 oracle.  Sizes span several
groups and tiles with ragged tails; every workload recipe is covered.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

pytestmark = pytest.mark.gpu

import gpu_util as U  # noqa: E402


def _case(name, **kw):
    return synth.make(name, **kw)


CODEC_CASES = [
    ("tiny", dict(), 32, 0),
    ("8b", dict(S=700, Hq=8, Hkv=2), 32, 0),
    ("8b", dict(S=700, Hq=8, Hkv=2, D=64), 32, 0),
    ("long", dict(S=1500, B=2, Hq=8, Hkv=2, kf=128), 128, 0),
    ("long", dict(S=1300, B=2, Hq=8, Hkv=2, kf=512), 512, 0),
    ("long", dict(S=700, B=2, Hq=8, Hkv=2, D=64, kf=128), 128, 0),
    ("long", dict(S=900, B=1, Hq=16, Hkv=1, kf=128), 128, 0),
    ("8b", dict(S=500, Hq=8, Hkv=2), 96, 0),
    ("mixed", dict(S=1400, B=3, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 64, 256),
    ("70b", dict(S=999, B=3, Hq=16, Hkv=2), 32, 0),
    ("mixed", dict(S=1400, B=4, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 32, 256),
    ("8b", dict(S=100, Hq=4, Hkv=1), 1, 0),
    ("8b", dict(S=97, Hq=4, Hkv=1), 7, 0),
]


@pytest.mark.parametrize("name,kw,kf,page", CODEC_CASES, ids=lambda x: str(x))
def test_prefill_codec_bit_exact(name, kw, kf, page):
    w = _case(name, **kw)
    r = U.prefill(w, kf=kf, page_tokens=page)
    enc = U.oracle_encode(w, kf, r.lens_np)
    U.assert_codec_exact(r, enc, kf)


@pytest.mark.parametrize("name,kw,kf,page", CODEC_CASES, ids=lambda x: str(x))
@pytest.mark.parametrize("fn", ["dkv_attn_decode", "dkv_attn_decode_ref"])
def test_attention_parity(name, kw, kf, page, fn):
    w = _case(name, **kw)
    r = U.prefill(w, kf=kf, page_tokens=page)
    enc = U.oracle_encode(w, kf, r.lens_np)
    q = synth.queries(w)
    got = U.attention(r, q, fn)
    ref = U.oracle_attention(enc, w, q, r.lens_np)
    err = U.rel_err(got, ref)
    assert err <= U.ATTN_TOL, err


def test_ragged_and_empty_sequences():
    w = _case("8b", S=300, B=5, Hq=8, Hkv=2)
    lens = np.array([0, 1, 31, 33, 300], np.int32)
    r = U.prefill(w, lens=lens)
    enc = U.oracle_encode(w, w.kf, lens)
    U.assert_codec_exact(r, enc, w.kf)
    q = synth.queries(w)
    for fn in ("dkv_attn_decode", "dkv_attn_decode_ref"):
        got = U.attention(r, q, fn)
        assert np.all(got[0] == 0.0)                      # empty sequence: zero rows
        ref = U.oracle_attention(enc, w, q, lens)
        ref[0] = 0.0
        assert U.rel_err(got, ref) <= U.ATTN_TOL


def test_ragged_and_empty_sequences_long_interval():
    w = _case("long", S=700, B=6, Hq=8, Hkv=2, kf=128)
    lens = np.array([0, 1, 33, 128, 129, 700], np.int32)
    r = U.prefill(w, kf=128, lens=lens)
    enc = U.oracle_encode(w, 128, lens)
    U.assert_codec_exact(r, enc, 128)
    q = synth.queries(w)
    for fn in ("dkv_attn_decode", "dkv_attn_decode_ref"):
        got = U.attention(r, q, fn)
        assert np.all(got[0] == 0.0)
        ref = U.oracle_attention(enc, w, q, lens)
        ref[0] = 0.0
        assert U.rel_err(got, ref) <= U.ATTN_TOL


def test_appends_equal_prefill_and_oracle():
    """Prefill part of each sequence, append the rest token by token: the cache
    and state match a single prefill and the oracle bit for bit."""
    w = _case("8b", S=200, B=3, Hq=8, Hkv=2)
    kf = 32
    full = U.prefill(w, kf=kf)
    start = np.array([0, 37, 64], np.int32)
    r = U.prefill(w, kf=kf, lens=start)
    k, v = full.k, full.v
    pos = torch.from_numpy(start.copy()).to(U.DEV)
    for t in range(int(start.min()), w.S):
        p = np.where(t >= start, t, -1).astype(np.int32)
        pos.copy_(torch.from_numpy(p))
        kn = k[:, :, min(t, w.S - 1)].contiguous()
        vn = v[:, :, min(t, w.S - 1)].contiguous()
        dkv.dkv_append(r.cfg, r.cache, r.state, None, kn, vn, pos)
    r.lens = full.lens
    r.lens_np = full.lens_np
    enc = U.oracle_encode(w, kf, full.lens_np)
    U.assert_codec_exact(r, enc, kf)
    assert torch.equal(r.state, full.state)


def test_append_paged_matches_oracle():
    w = _case("mixed", S=600, B=4, Hq=8, Hkv=2, min_len=64, extra_tokens=40)
    r = U.prefill(w, page_tokens=256)
    lens = r.lens_np.copy()
    for step in range(40):
        pos = torch.from_numpy(lens.astype(np.int32)).to(U.DEV)
        kn = torch.stack([r.k[b, :, int(lens[b])] for b in range(w.B)]).contiguous()
        vn = torch.stack([r.v[b, :, int(lens[b])] for b in range(w.B)]).contiguous()
        dkv.dkv_append(r.cfg, r.cache, r.state, r.bt, kn, vn, pos)
        lens += 1
    r.lens_np = lens.astype(np.int32)
    r.lens = torch.from_numpy(r.lens_np).to(U.DEV)
    enc = U.oracle_encode(w, w.kf, r.lens_np)
    U.assert_codec_exact(r, enc, w.kf)
    q = synth.queries(w, step=3)
    got = U.attention(r, q)
    ref = U.oracle_attention(enc, w, q, r.lens_np)
    assert U.rel_err(got, ref) <= U.ATTN_TOL


def test_resume_through_host_copy():
    """Cache + state copied to the host and back continue bit-exactly."""
    w = _case("8b", S=160, B=2, Hq=8, Hkv=2)
    a = U.prefill(w, lens=np.array([100, 120], np.int32))
    cache_h, state_h = a.cache.cpu(), a.state.cpu()
    b_cache, b_state = cache_h.to(U.DEV), state_h.to(U.DEV)
    for t in range(100, 160):
        p = torch.tensor([t, t if t >= 120 else -1], dtype=torch.int32, device=U.DEV)
        kn = a.k[:, :, t].contiguous()
        vn = a.v[:, :, t].contiguous()
        dkv.dkv_append(a.cfg, a.cache, a.state, None, kn, vn, p)
        dkv.dkv_append(a.cfg, b_cache, b_state, None, kn, vn, p)
    assert torch.equal(a.cache, b_cache) and torch.equal(a.state, b_state)


def test_attention_repeatable():
    w = _case("70b", S=700, B=2, Hq=16, Hkv=2)
    r = U.prefill(w)
    q = synth.queries(w)
    a = U.attention(r, q)
    b = U.attention(r, q)
    assert np.array_equal(a, b)


def test_softmax_scale_argument():
    w = _case("8b", S=200, Hq=8, Hkv=2)
    r = U.prefill(w)
    enc = U.oracle_encode(w, w.kf, r.lens_np)
    q = synth.queries(w)
    qd = torch.from_numpy(q).to(U.DEV)
    out = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    dkv.dkv_attn_decode(r.cfg, r.cache, None, qd, r.lens, out, r.ws, softmax_scale=0.25)
    scale = np.float32(0.25)
    ref = np.zeros((w.B, w.Hq, w.D))
    G = w.Hq // w.Hkv
    for h in range(w.Hkv):
        ref[0, h * G:(h + 1) * G] = oracle.attention_f64(q[0, h * G:(h + 1) * G], enc[(0, h, 0)].recon,
                                                         enc[(0, h, 1)].recon, scale)
    assert U.rel_err(out.cpu().numpy(), ref) <= U.ATTN_TOL


@pytest.mark.parametrize("qscale", [1e3, 1e-3])
@pytest.mark.parametrize("name,kw,kf", [("8b", dict(S=600, Hq=8, Hkv=2), 32),
                                        ("70b", dict(S=600, B=2, Hq=16, Hkv=2), 32),
                                        ("long", dict(S=1100, B=2, Hq=8, Hkv=2, kf=512), 512)])
def test_query_scale(name, kw, kf, qscale):
    """Queries far from unit size (a very peaked or a nearly flat softmax):
    the matrix-core kernels scale the query operands by 2^-E before the fp16
    split, so attention stays within 2e-3 of the oracle."""
    w = _case(name, **kw)
    print(f"query scale {name} {kw} kf={kf} x{qscale}", flush=True)
    r = U.prefill(w, kf=kf)
    enc = U.oracle_encode(w, kf, r.lens_np)
    q = (synth.queries(w) * np.float32(qscale)).astype(np.float32)
    got = U.attention(r, q)
    ref = U.oracle_attention(enc, w, q, r.lens_np)
    assert U.rel_err(got, ref) <= U.ATTN_TOL


@pytest.mark.parametrize("vscale", [100.0, 0.01])
@pytest.mark.parametrize("name,kw,kf", [("8b", dict(S=600, Hq=8, Hkv=2), 32),
                                        ("long", dict(S=1100, B=2, Hq=8, Hkv=2, kf=128), 128)])
def test_value_scale(name, kw, kf, vscale):
    """K and V far from unit size (the 8b data's lognormal channels times 100
    reach about 2,000): the codec stays bit-exact with the oracle, and the V
    weights' range bias (from the group's largest scale) keeps attention
    within 2e-3."""
    w = _case(name, **kw)
    print(f"value scale {name} {kw} kf={kf} x{vscale}", flush=True)
    w.k = (w.k.astype(np.float32) * np.float32(vscale)).astype(np.float16)
    w.v = (w.v.astype(np.float32) * np.float32(vscale)).astype(np.float16)
    assert np.isfinite(w.k.astype(np.float32)).all() and np.isfinite(w.v.astype(np.float32)).all()
    r = U.prefill(w, kf=kf)
    enc = U.oracle_encode(w, kf, r.lens_np)
    U.assert_codec_exact(r, enc, kf)
    q = synth.queries(w) / np.float32(vscale)
    got = U.attention(r, q)
    ref = U.oracle_attention(enc, w, q, r.lens_np)
    assert U.rel_err(got, ref) <= U.ATTN_TOL


# Runs of several whole groups per workgroup: 32 sequences x 8 kv-heads make
# the split plan cut each sequence into 8 runs (8 groups at kf = 32, 2 at
# kf = 128), and the lengths put every count of whole groups in a run, with
# and without a partial last group, through the pipelined kernels (keyframe
# batches of 4 closed early, a run of one group, the partial group after it).
# At kf > 32 with at most 4 query heads per kv-head the forward kernel takes
# the groups tile by tile (NT = kf/32 tiles, 3 at kf = 96), so a group's last
# tile, a partial last tile and a run that ends inside a group all occur.
RUN_LENS = [0, 1, 31, 32, 33, 63, 64, 65, 96, 97, 127, 128, 129, 160, 192, 224,
            255, 256, 257, 300, 511, 512, 513, 640, 1000, 1024, 1025, 1500, 2000, 2016, 2047, 2048]


@pytest.mark.parametrize("kf,Hq,D", [(32, 64, 128), (128, 64, 128), (32, 32, 128), (32, 16, 128), (32, 8, 128),
                                     (32, 32, 64), (128, 32, 128), (128, 16, 128), (128, 8, 128), (512, 32, 128),
                                     (64, 32, 64), (96, 32, 128)])
def test_runs_of_every_length(kf, Hq, D):
    print(f"runs of every length kf={kf} Hq={Hq} D={D}", flush=True)
    w = _case("70b", S=2048, B=32, Hq=Hq, D=D)
    lens = np.array(RUN_LENS, np.int32)
    r = U.prefill(w, kf=kf, lens=lens)
    pairs = {(b, h) for b in range(1, w.B) for h in (0, 5)}
    enc = U.oracle_encode(w, kf, lens, pairs=pairs)
    q = synth.queries(w)
    got = U.attention(r, q)
    assert np.all(got[0] == 0.0)                      # empty sequence: zero rows
    ref = U.oracle_attention(enc, w, q, lens, pairs=pairs)
    assert U.rel_err(got, ref) <= U.ATTN_TOL
    assert np.isfinite(got).all()


@pytest.mark.parametrize("S,parity", [(4096, "even"), (4192, "odd")])
def test_ragged_batch_every_pair(S, parity):
    """A ragged batch (8 sequences of 1..S tokens, 8 kv-heads) with an even
    split count, where each row's runs are rotated across the XCDs, and with an
    odd one, where they are not: every (sequence, kv-head) pair's decode
    attention against the oracle's float64 attention over its own encoding."""
    print(f"ragged batch every pair S={S} ({parity} split count)", flush=True)
    w = _case("8b", S=S, B=8, Hq=32, Hkv=8)
    lens = np.random.default_rng(11).integers(1, S + 1, size=w.B).astype(np.int32)
    lens[3] = S                                       # a full-length row
    r = U.prefill(w, kf=32, lens=lens)
    ns, _ = dkv.dkv_attn_decode_plan(r.cfg)
    assert (ns % 2 == 0) == (parity == "even"), ns
    enc = U.oracle_encode(w, 32, lens)
    q = synth.queries(w)
    got = U.attention(r, q)
    ref = U.oracle_attention(enc, w, q, lens)
    assert U.rel_err(got, ref) <= U.ATTN_TOL
    assert np.isfinite(got).all()


def test_stream_read_reads_every_word():
    """The streaming-read diagnostic: the XOR of its sink words is the XOR of
    every 32-bit word of the buffer (each word is read exactly once)."""
    rng = np.random.default_rng(7)
    for nbytes in (16, 1040, 3 * 1024 * 1024 + 48):
        host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).to(U.DEV)
        sink = torch.full((dkv.dkv_stream_read_sink_words(),), -1, dtype=torch.int32, device=U.DEV)
        dkv.dkv_stream_read(buf, sink)
        got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), nbytes
