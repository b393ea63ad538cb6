"""GPU parity of the strided-reference residual cache (the gist.science
explainer of DeltaKV, section 3.A) against the CPU oracle, through the C ABI.

Encode: every stream's reference rows, per-token reference indices, Q4_0
residual codes and fp16 scales must be bit-identical to the oracle's (the
nearest-reference choice is made in double on both sides with the same
order of operations and no fused multiply-add).  Decode attention: within
2e-3 per output row of float64 attention over the oracle's reconstruction.
Cases cover lengths 0, 1, around the stride and the 32-token tile, 1 to 16
query heads per kv-head, D = 64 and 128, windows, and runs of several tiles
per workgroup (32 sequences x 8 kv-heads).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

pytestmark = pytest.mark.gpu

import gpu_util as U  # noqa: E402

CASES = [
    # (workload, overrides, stride, window, lens, sampled (b, h) pairs or None for all)
    ("tiny", dict(), 32, 0, None, None),
    ("8b", dict(S=700, Hq=8, Hkv=2), 32, 0, None, None),
    ("8b", dict(S=700, Hq=8, Hkv=2, D=64), 32, 4, None, None),
    ("8b", dict(S=400, B=6, Hq=8, Hkv=2), 32, 0, [0, 1, 31, 32, 33, 400], None),
    ("8b", dict(S=500, Hq=8, Hkv=2), 8, 16, None, None),
    ("mixed", dict(B=4, S=1500, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 32, 0, None, None),
    ("70b", dict(S=600, B=2, Hq=16, Hkv=2), 32, 0, None, None),
    ("70b", dict(S=300, B=2, Hq=32, Hkv=2), 16, 0, None, None),
    ("70b", dict(S=2048, B=32, Hq=32, Hkv=8), 32, 0, "ragged", [(1, 0), (7, 5), (20, 3), (31, 7)]),
    ("8b", dict(S=200, Hq=8, Hkv=2), 1, 0, None, None),            # every token its own reference
    ("8b", dict(S=600, Hq=8, Hkv=2), 32, 1, None, None),           # only the latest reference
    ("70b", dict(S=300, B=2, Hq=32, Hkv=2, D=64), 32, 0, None, None),
    # runs of 8 tiles with at most 8 query heads per kv-head (the paired
    # column halves rescaled as the running max moves), G = 8 and D = 64
    ("70b", dict(S=2048, B=32, Hq=64, Hkv=8), 32, 64, "ragged", [(1, 0), (9, 6), (31, 7)]),
    ("70b", dict(S=2048, B=32, Hq=32, Hkv=8, D=64), 32, 0, "ragged", [(1, 3), (12, 1), (30, 7)]),
]


def _cfg(w, stride):
    return dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=stride,
                      max_tokens=w.S + w.extra_tokens)


@pytest.mark.parametrize("name,kw,stride,window,lens,pairs", CASES)
def test_strided_cache_matches_oracle(name, kw, stride, window, lens, pairs):
    w = synth.make(name, **kw)
    print(f"strided case {name} {kw} stride={stride} window={window} lens={lens}", flush=True)
    if lens == "ragged":
        lens = np.random.default_rng(3).integers(0, w.S + 1, w.B)
        lens[:3] = [0, w.S, 1]
    lens_np = np.asarray(w.seq_lens if lens is None else lens, np.int32)
    cfg = _cfg(w, stride)
    lay = dkv.dkv_strided_layout(cfg)
    cache = torch.full((dkv.dkv_strided_cache_bytes(cfg),), 0xA5, dtype=torch.uint8, device=U.DEV)
    k = torch.from_numpy(np.ascontiguousarray(w.k)).to(U.DEV)
    v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    lens_d = torch.from_numpy(lens_np).to(U.DEV)
    s_max = w.k.shape[2]
    dkv.dkv_strided_encode_prefill(cfg, cache, k, v, lens_d, s_max, window)
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=U.DEV)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_attn_decode(cfg, cache, q, lens_d, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    host = cache.cpu().numpy()

    D, G, sb = w.D, w.Hq // w.Hkv, lay["stream_bytes"]
    scale = np.float32(1 / math.sqrt(D))
    todo = pairs if pairs is not None else [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    ref = np.full((w.B, w.Hq, D), np.nan)
    for (b, h) in todo:
        L = int(lens_np[b])
        recon = []
        for s, x in ((0, w.k), (1, w.v)):
            e = oracle.strided_encode_stream(np.ascontiguousarray(x[b, h, :L]), stride, window)
            st = host[((b * w.Hkv + h) * 2 + s) * sb:][:sb]
            nr = -(-L // stride)
            refs = st[:nr * D * 2].view(np.uint16).reshape(nr, D)
            codes = st[lay["codes"]:lay["codes"] + L * D // 2].reshape(L, D // 2)
            scales = st[lay["scales"]:lay["scales"] + L * D // 16].view(np.uint16).reshape(L, D // 32)
            idx = st[lay["idx"]:lay["idx"] + 2 * L].view(np.uint16)
            assert np.array_equal(refs, e.refs), ("refs", b, h, s)
            assert np.array_equal(idx.astype(np.int32), e.ref_idx), ("idx", b, h, s)
            assert np.array_equal(codes, e.codes), ("codes", b, h, s)
            assert np.array_equal(scales, e.scales), ("scales", b, h, s)
            recon.append(e.recon)
        if L == 0:
            assert np.all(got[b, h * G:(h + 1) * G] == 0.0), (b, h)
            continue
        ref[b, h * G:(h + 1) * G] = oracle.attention_f64(q_np[b, h * G:(h + 1) * G], recon[0], recon[1], scale)
    assert U.rel_err(got, ref) <= U.ATTN_TOL
    assert np.isfinite(got).all()


def test_strided_periodic_sequence_reconstructs_exactly():
    """Periodic rows (period 5, stride 8): once the references cover every
    phase (token 32), each token finds an exact reference and its residual
    codes are all zero; attention matches the oracle over its reconstruction."""
    rng = np.random.default_rng(21)
    B, H, G, D, S, P, stride = 2, 2, 4, 128, 1000, 5, 8
    T = (rng.standard_normal((B, H, 2, P, D))).astype(np.float16)
    x = np.stack([T[..., t % P, :] for t in range(S)], axis=3)          # [B][H][2][S][D]
    k = np.ascontiguousarray(x[:, :, 0])
    v = np.ascontiguousarray(x[:, :, 1])
    cfg = dkv.Config(batch=B, n_q_heads=H * G, n_kv_heads=H, head_dim=D, kf=stride, max_tokens=S)
    cache = torch.zeros(dkv.dkv_strided_cache_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    lens = torch.full((B,), S, dtype=torch.int32, device=U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, cache, torch.from_numpy(k).to(U.DEV), torch.from_numpy(v).to(U.DEV), lens, S)
    q_np = rng.standard_normal((B, H * G, D)).astype(np.float32)
    out = torch.zeros(B, H * G, D, dtype=torch.float32, device=U.DEV)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_attn_decode(cfg, cache, torch.from_numpy(q_np).to(U.DEV), lens, out, ws)
    torch.cuda.synchronize()
    lay = dkv.dkv_strided_layout(cfg)
    host = cache.cpu().numpy()
    scale = np.float32(1 / math.sqrt(D))
    for b in range(B):
        for h in range(H):
            for s in range(2):
                st = host[((b * H + h) * 2 + s) * lay["stream_bytes"]:]
                codes = st[lay["codes"]:lay["codes"] + S * D // 2].reshape(S, D // 2)
                # stride 8 and period 5: references 0..4 cover every phase by token 32
                assert np.all(codes[32:] == 0x88), (b, h, s)
            # tokens before 32 carry Q4_0 residuals, so the reference is the
            # oracle's reconstruction, itself exact from token 32 on
            rk = oracle.strided_encode_stream(k[b, h], stride)
            rv = oracle.strided_encode_stream(v[b, h], stride)
            assert np.array_equal(rk.recon[32:], k[b, h, 32:].astype(np.float32))
            assert np.array_equal(rv.recon[32:], v[b, h, 32:].astype(np.float32))
            ref = oracle.attention_f64(q_np[b, h * G:(h + 1) * G], rk.recon, rv.recon, scale)
            g = out[b, h * G:(h + 1) * G].cpu().numpy()
            assert U.rel_err(g[None], ref[None]) <= U.ATTN_TOL


@pytest.mark.parametrize("kw,stride,window", [
    (dict(S=300, B=3, Hq=8, Hkv=2, extra_tokens=40), 32, 0),
    (dict(S=300, B=3, Hq=8, Hkv=2, D=64, extra_tokens=40), 8, 16),
])
def test_strided_append_matches_prefill(kw, stride, window):
    """Prefill of a prefix, then one token per step (one sequence skipping some
    steps with a negative position): the cache bytes of every encoded token
    and reference equal those of a prefill over the grown sequences, and so do
    the attention outputs."""
    w = synth.make("8b", **kw)
    print(f"strided append {kw} stride={stride} window={window}", flush=True)
    cfg = _cfg(w, stride)
    lay = dkv.dkv_strided_layout(cfg)
    s_max = w.k.shape[2]
    k = torch.from_numpy(np.ascontiguousarray(w.k)).to(U.DEV)
    v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    lens = np.array([100, 0, 257], np.int32)
    a = torch.full((dkv.dkv_strided_cache_bytes(cfg),), 0xA5, dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, a, k, v, torch.from_numpy(lens).to(U.DEV), s_max, window)
    for step in range(40):
        pos = lens.copy()
        if step % 3 == 1:
            pos[1] = -1
        kn = torch.stack([k[b, :, max(int(pos[b]), 0)] for b in range(w.B)]).contiguous()
        vn = torch.stack([v[b, :, max(int(pos[b]), 0)] for b in range(w.B)]).contiguous()
        dkv.dkv_strided_append(cfg, a, kn, vn, torch.from_numpy(pos).to(U.DEV), window)
        lens = lens + (pos >= 0)
    bcache = torch.full_like(a, 0x5A)
    lens_d = torch.from_numpy(lens.astype(np.int32)).to(U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, bcache, k, v, lens_d, s_max, window)
    torch.cuda.synchronize()
    ha, hb = a.cpu().numpy(), bcache.cpu().numpy()
    D, sb = w.D, lay["stream_bytes"]
    for b in range(w.B):
        L = int(lens[b])
        for h in range(w.Hkv):
            for s in range(2):
                o = ((b * w.Hkv + h) * 2 + s) * sb
                for lo, n in ((0, -(-L // stride) * D * 2), (lay["codes"], L * D // 2),
                              (lay["scales"], L * D // 16), (lay["idx"], 2 * L)):
                    assert np.array_equal(ha[o + lo:o + lo + n], hb[o + lo:o + lo + n]), (b, h, s, lo)
    q = torch.from_numpy(synth.queries(w)).to(U.DEV)
    oa = torch.zeros(w.B, w.Hq, D, dtype=torch.float32, device=U.DEV)
    ob = torch.zeros_like(oa)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_attn_decode(cfg, a, q, lens_d, oa, ws)
    dkv.dkv_strided_attn_decode(cfg, bcache, q, lens_d, ob, ws)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)


@pytest.mark.parametrize("kw,stride,window", [
    (dict(S=300, B=3, Hq=8, Hkv=2, extra_tokens=40), 32, 64),
    (dict(S=300, B=3, Hq=16, Hkv=2, D=64, extra_tokens=40), 8, 0),
    (dict(S=2048, B=32, Hq=32, Hkv=8, extra_tokens=8), 32, 64),     # runs of 16 tiles
])
def test_strided_fused_step_matches_append_then_decode(kw, stride, window):
    """dkv_strided_append_attn_decode leaves the same cache bytes and gives the
    same output as dkv_strided_append followed by dkv_strided_attn_decode."""
    w = synth.make("8b" if kw.get("Hkv") == 2 else "70b", **kw)
    print(f"strided fused step {kw} stride={stride} window={window}", flush=True)
    cfg = _cfg(w, stride)
    s_max = w.k.shape[2]
    k = torch.from_numpy(np.ascontiguousarray(w.k)).to(U.DEV)
    v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    lens = np.minimum(np.asarray(w.seq_lens, np.int32), w.S - 5)
    lens[0] = 0
    a = torch.zeros(dkv.dkv_strided_cache_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, a, k, v, torch.from_numpy(lens).to(U.DEV), s_max, window)
    bcache = a.clone()
    ws_a = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    ws_b = torch.zeros_like(ws_a)
    oa = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    ob = torch.zeros_like(oa)
    for step in range(8):
        pos = lens.copy()
        if step % 3 == 2:
            pos[1] = -1
        kn = torch.stack([k[b, :, max(int(pos[b]), 0)] for b in range(w.B)]).contiguous()
        vn = torch.stack([v[b, :, max(int(pos[b]), 0)] for b in range(w.B)]).contiguous()
        lens = lens + (pos >= 0)
        pd = torch.from_numpy(pos).to(U.DEV)
        ld = torch.from_numpy(lens.astype(np.int32)).to(U.DEV)
        q = torch.from_numpy(synth.queries(w, step=step)).to(U.DEV)
        dkv.dkv_strided_append(cfg, a, kn, vn, pd, window)
        dkv.dkv_strided_attn_decode(cfg, a, q, ld, oa, ws_a)
        dkv.dkv_strided_append_attn_decode(cfg, bcache, kn, vn, pd, q, ld, ob, ws_b, window=window)
        torch.cuda.synchronize()
        assert torch.equal(a, bcache), f"cache differs after step {step}"
        assert torch.equal(oa, ob), f"output differs after step {step}"


@pytest.mark.parametrize("qscale", [1e3, 1e-3])
def test_strided_query_scale(qscale):
    """Queries far from unit size (a very peaked or a nearly flat softmax): the
    logits' fp16 query operands are scaled by 2^-E first, so attention stays
    within 2e-3 of the oracle."""
    w = synth.make("8b", S=500, Hq=8, Hkv=2)
    print(f"strided query scale {qscale}", flush=True)
    cfg = _cfg(w, 32)
    lens_np = np.asarray(w.seq_lens, np.int32)
    cache = torch.zeros(dkv.dkv_strided_cache_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    lens = torch.from_numpy(lens_np).to(U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, cache, torch.from_numpy(w.k).to(U.DEV), torch.from_numpy(w.v).to(U.DEV),
                                   lens, w.k.shape[2], 0)
    q_np = (synth.queries(w) * np.float32(qscale)).astype(np.float32)
    out = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_attn_decode(cfg, cache, torch.from_numpy(q_np).to(U.DEV), lens, out, ws)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    ref = np.zeros((w.B, w.Hq, w.D))
    for b in range(w.B):
        L = int(lens_np[b])
        for h in range(w.Hkv):
            rec = [oracle.strided_encode_stream(np.ascontiguousarray(x[b, h, :L]), 32, 0).recon for x in (w.k, w.v)]
            ref[b, h * G:(h + 1) * G] = oracle.attention_f64(q_np[b, h * G:(h + 1) * G], rec[0], rec[1],
                                                             np.float32(1 / math.sqrt(w.D)))
    assert U.rel_err(out.cpu().numpy(), ref) <= U.ATTN_TOL


@pytest.mark.parametrize("window", [0, 2, 3])
def test_strided_nonfinite_rows_take_the_oracle_reference(window):
    """Rows holding NaN or infinities (outside the finite-input contract) take
    the reference the oracle's order gives them (a NaN distance ranks above
    every number, lowest index among equals), in the prefill and in the
    append; tokens whose row and reference are finite keep bit-exact codes."""
    D, S, stride = 64, 10, 2
    x = np.zeros((S, D), np.float16)
    x[:, 0] = np.arange(S, dtype=np.float16)
    x[:, 5] = np.linspace(-1, 1, S).astype(np.float16)
    x[3, 7] = np.float16("nan")
    x[4, 3] = np.float16("nan")
    x[5, 2] = np.float16("inf")
    x[6, 1] = -np.float16("inf")
    cfg = dkv.Config(batch=1, n_q_heads=1, n_kv_heads=1, head_dim=D, kf=stride, max_tokens=S)
    lay = dkv.dkv_strided_layout(cfg)
    kx = torch.from_numpy(x[None, None].copy()).to(U.DEV)
    lens = torch.full((1,), S, dtype=torch.int32, device=U.DEV)
    pre = torch.zeros(dkv.dkv_strided_cache_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, pre, kx, kx, lens, S, window)
    app = torch.zeros_like(pre)
    for t in range(S):
        row = kx[:, :, t].contiguous()
        dkv.dkv_strided_append(cfg, app, row, row, torch.full((1,), t, dtype=torch.int32, device=U.DEV), window)
    torch.cuda.synchronize()
    e = oracle.strided_encode_stream(x, stride, window)
    finite = np.isfinite(x.astype(np.float32)).all(axis=1)
    for name, c in (("prefill", pre), ("append", app)):
        st = c.cpu().numpy()[:lay["stream_bytes"]]
        idx = st[lay["idx"]:lay["idx"] + 2 * S].view(np.uint16).astype(np.int32)
        assert np.array_equal(idx, e.ref_idx), (name, idx, e.ref_idx)
        codes = st[lay["codes"]:lay["codes"] + S * D // 2].reshape(S, D // 2)
        scales = st[lay["scales"]:lay["scales"] + S * D // 16].view(np.uint16).reshape(S, D // 32)
        for t in range(S):
            if finite[t] and finite[e.ref_idx[t] * stride]:
                assert np.array_equal(codes[t], e.codes[t]) and np.array_equal(scales[t], e.scales[t]), (name, t)
