"""GPU parity of the Q4-keyframe variant (keyframes stored as Q4_0 of their
absolute values, every other token as Q4_0 of its closed-loop delta; the
plain Q4_0 tile layout) against the CPU oracle, through the C ABI.

* codes and fp16 scale bit patterns (via dkv_q4_0_export), reconstructions
  (dkv_q4k_reconstruct) and the state: bit-exact with oracle.q4k_encode_stream,
  at kf 1, 8, 32 and 128, contiguous and on shuffled 256-token pages, ragged
  and empty sequences;
* kf = 1: the whole cache equals the plain Q4_0 encoder's, byte for byte;
* appends one token at a time equal a prefill of the grown sequences;
* decode attention (kf 1 and 32; 1, 2, 4, 8 query heads per kv-head; D 64 and
  128) within 2e-3 of float64 attention over the oracle's reconstruction,
  also with queries scaled by 1e3 and 1e-3 and values by 100.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

pytestmark = pytest.mark.gpu

import gpu_util as U  # noqa: E402


class _Q4K:
    pass


def _setup(name, kw, kf, lens=None, page_tokens=0, extra=0):
    """Workload, config (contiguous, or shuffled pages with one extra unmapped
    logical page per sequence), and a Q4-keyframe prefill of `lens` tokens."""
    r = _Q4K()
    r.w = w = synth.make(name, **kw)
    r.lens_np = np.asarray(w.seq_lens if lens is None else lens, np.int32)
    r.bt = None
    cap = w.k.shape[2]
    if page_tokens:
        need = [-(-(int(L) + extra) // page_tokens) for L in r.lens_np]
        maxp = max(need) + 1
        perm = np.random.default_rng(23).permutation(int(sum(need))).astype(np.int32)
        table = np.full((w.B, maxp), -1, np.int32)
        pos = 0
        for b, k in enumerate(need):
            table[b, :k] = perm[pos:pos + k]
            pos += k
        r.cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=kf,
                           page_tokens=page_tokens, n_pages=max(1, int(sum(need))), max_pages_per_seq=maxp)
        r.bt = torch.from_numpy(table).to(U.DEV)
    else:
        r.cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=kf, max_tokens=cap)
    r.lens = torch.from_numpy(r.lens_np).to(U.DEV)
    r.cache = torch.full((dkv.dkv_q4_0_cache_bytes(r.cfg),), 0xA5, dtype=torch.uint8, device=U.DEV)
    r.state = torch.zeros(w.B, w.Hkv, 2, w.D, dtype=torch.float32, device=U.DEV)
    r.ws = torch.zeros(dkv.dkv_workspace_bytes(r.cfg), dtype=torch.uint8, device=U.DEV)
    r.k = torch.from_numpy(np.ascontiguousarray(w.k)).to(U.DEV)
    r.v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    r.s_max = cap
    dkv.dkv_q4k_encode_prefill(r.cfg, r.cache, r.state, r.bt, r.k, r.v, r.lens, r.s_max)
    return r


def _oracle(r, kf, lens=None):
    w = r.w
    lens = r.lens_np if lens is None else lens
    return {(b, h, s): oracle.q4k_encode_stream(np.ascontiguousarray(x[b, h, :int(lens[b])]), kf)
            for b in range(w.B) for h in range(w.Hkv) for s, x in ((0, w.k), (1, w.v))}


def _assert_exact(r, enc):
    w, S = r.w, r.s_max
    codes = torch.zeros((w.B, w.Hkv, 2, S, w.D // 2), dtype=torch.uint8, device=U.DEV)
    scales = torch.zeros((w.B, w.Hkv, 2, S, w.D // 32), dtype=torch.int16, device=U.DEV)
    dkv.dkv_q4_0_export(r.cfg, r.cache, r.bt, r.lens, S, codes, scales)
    ko = torch.zeros(w.B, w.Hkv, S, w.D, dtype=torch.float32, device=U.DEV)
    vo = torch.zeros_like(ko)
    dkv.dkv_q4k_reconstruct(r.cfg, r.cache, r.bt, r.lens, S, ko, vo)
    codes, scales = codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16)
    rec = (ko.cpu().numpy(), vo.cpu().numpy())
    state = r.state.cpu().numpy()
    for (b, h, s), e in enc.items():
        L = e.S
        assert np.array_equal(codes[b, h, s, :L], e.codes), ("codes", b, h, s)
        assert np.array_equal(scales[b, h, s, :L], e.scales), ("scales", b, h, s)
        assert np.array_equal(rec[s][b, h, :L].view(np.uint32), e.recon.view(np.uint32)), ("recon", b, h, s)
        if L > 0:
            assert np.array_equal(state[b, h, s].view(np.uint32), e.state.view(np.uint32)), ("state", b, h, s)


CODEC = [
    # (workload, overrides, kf, lengths, page_tokens)
    ("tiny", dict(), 32, None, 0),
    ("8b", dict(S=300, B=6, Hq=8, Hkv=2), 32, [0, 1, 31, 32, 33, 300], 0),
    ("8b", dict(S=300, B=3, Hq=8, Hkv=2, D=64), 1, [300, 17, 64], 0),
    ("8b", dict(S=300, B=3, Hq=8, Hkv=2), 8, [300, 9, 0], 0),
    ("long", dict(S=700, B=2, Hq=8, Hkv=2), 128, [700, 129], 0),
    ("8b", dict(S=700, B=5, Hq=8, Hkv=2), 32, [0, 1, 255, 257, 700], 256),
    ("8b", dict(S=700, B=3, Hq=8, Hkv=2), 128, [700, 128, 300], 256),
    ("mixed", dict(B=4, S=1500, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 1, None, 256),
]


@pytest.mark.parametrize("name,kw,kf,lens,page", CODEC, ids=str)
def test_q4k_codec_bit_exact(name, kw, kf, lens, page):
    print(f"q4k codec {name} {kw} kf={kf} lens={lens} page={page}", flush=True)
    r = _setup(name, kw, kf, lens, page)
    _assert_exact(r, _oracle(r, kf))


@pytest.mark.parametrize("page", [0, 256])
def test_kf1_cache_is_plain_q4_0(page):
    """At kf = 1 the Q4-keyframe cache and the plain Q4_0 cache of the same
    rows are the same bytes (both start from the same fill)."""
    print(f"q4k kf=1 vs q4_0 page={page}", flush=True)
    r = _setup("8b", dict(S=500, B=3, Hq=8, Hkv=2), 1, [500, 33, 257], page)
    q4 = torch.full_like(r.cache, 0xA5)
    dkv.dkv_q4_0_encode(r.cfg, q4, r.bt, r.k, r.v, r.lens, r.s_max)
    assert torch.equal(q4, r.cache)


@pytest.mark.parametrize("kf,page", [(32, 0), (8, 0), (128, 256), (1, 256)])
def test_q4k_append_equals_prefill(kf, page):
    print(f"q4k append kf={kf} page={page}", flush=True)
    lens0 = np.array([40, 0, 95], np.int32)
    steps = 70
    r = _setup("8b", dict(S=300, B=3, Hq=8, Hkv=2), kf, lens0, page, extra=steps)
    for t in range(steps):
        pos = torch.from_numpy(lens0 + t).to(U.DEV)
        kn = r.k[torch.arange(3), :, pos.long()].contiguous()
        vn = r.v[torch.arange(3), :, pos.long()].contiguous()
        dkv.dkv_q4k_append(r.cfg, r.cache, r.state, r.bt, kn, vn, pos)
    r.lens_np = lens0 + steps
    r.lens = torch.from_numpy(r.lens_np).to(U.DEV)
    _assert_exact(r, _oracle(r, kf))


ATTN = [
    # (workload, overrides, kf, lengths, page_tokens)
    ("tiny", dict(), 32, None, 0),                                             # G = 1, D = 64
    ("8b", dict(S=700, B=3, Hq=4, Hkv=2), 32, [700, 0, 45], 0),                # G = 2, an empty sequence
    ("8b", dict(S=4096, B=1, Hq=32, Hkv=8), 32, None, 0),                      # G = 4
    ("70b", dict(S=1000, B=2, Hq=64, Hkv=8), 32, [1000, 333], 0),              # G = 8
    ("8b", dict(S=600, B=3, Hq=8, Hkv=2, D=64), 32, [600, 31, 33], 0),
    ("8b", dict(S=600, B=3, Hq=8, Hkv=2), 1, [600, 1, 257], 0),               # plain Q4_0
    ("8b", dict(S=700, B=4, Hq=8, Hkv=2), 32, [0, 1, 257, 700], 256),          # paged
    ("mixed", dict(B=4, S=2100, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 32, None, 256),
]


@pytest.mark.parametrize("name,kw,kf,lens,page", ATTN, ids=str)
def test_q4k_attention(name, kw, kf, lens, page):
    print(f"q4k attention {name} {kw} kf={kf} lens={lens} page={page}", flush=True)
    r = _setup(name, kw, kf, lens, page)
    enc = _oracle(r, kf)
    q_np = synth.queries(r.w)
    got = U.attention(r, q_np, fn="dkv_attn_decode_q4k")
    ref = U.oracle_attention(enc, r.w, q_np, r.lens_np)
    assert U.rel_err(got, ref) <= U.ATTN_TOL
    for b, L in enumerate(r.lens_np):
        if L == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("qs,vs", [(1e3, 1.0), (1e-3, 1.0), (1.0, 100.0)])
def test_q4k_attention_scaled(qs, vs):
    """Queries scaled by 1e3 / 1e-3 (logit range) and values by 100 (the
    weight range bias with suffix sums of up to 32 weights)."""
    print(f"q4k attention scaled q x{qs} v x{vs}", flush=True)
    w = synth.make("8b", S=500, B=2, Hq=8, Hkv=2)
    w.v = (w.v.astype(np.float32) * vs).astype(np.float16)
    lens = np.array([500, 77], np.int32)
    r = _setup("8b", dict(S=500, B=2, Hq=8, Hkv=2), 32, lens)
    r.w.v = w.v
    r.v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    dkv.dkv_q4k_encode_prefill(r.cfg, r.cache, r.state, r.bt, r.k, r.v, r.lens, r.s_max)
    enc = _oracle(r, 32)
    q_np = (synth.queries(r.w) * np.float32(qs)).astype(np.float32)
    got = U.attention(r, q_np, fn="dkv_attn_decode_q4k")
    ref = U.oracle_attention(enc, r.w, q_np, r.lens_np)
    assert U.rel_err(got, ref) <= U.ATTN_TOL
