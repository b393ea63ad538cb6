"""GPU parity of the in-run comparison paths (plain Q4_0 of absolute values and
F16) against the CPU oracle, through the C ABI.

Q4_0 codes and fp16 scale bit patterns must be bit-exact with the oracle's
Q4_0 of the absolute rows; both attentions must be within 2e-3 max relative
error per output row of float64 attention over the oracle's dequantised (Q4_0)
or widened (F16) rows.
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
    ("tiny", dict(), None),
    ("8b", dict(S=700, Hq=8, Hkv=2), None),
    ("8b", dict(S=400, Hq=8, Hkv=2, D=64), None),
    ("70b", dict(S=333, B=3, Hq=16, Hkv=1), None),
    ("8b", dict(S=300, B=6, Hq=8, Hkv=2), [0, 1, 31, 32, 33, 300]),
]


def _setup(name, kw, lens):
    w = synth.make(name, **kw)
    lens_np = np.asarray(w.seq_lens if lens is None else lens, np.int32)
    cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=32, max_tokens=w.S)
    return w, lens_np, cfg


def _f16_inputs(w, lens_np, poison=True):
    """fp16 K/V on the device; rows past each sequence's length hold NaN."""
    k = np.ascontiguousarray(w.k).copy()
    v = np.ascontiguousarray(w.v).copy()
    if poison:
        for b, L in enumerate(lens_np):
            k[b, :, L:] = np.float16(np.nan)
            v[b, :, L:] = np.float16(np.nan)
    return torch.from_numpy(k).to(U.DEV), torch.from_numpy(v).to(U.DEV)


def _q40_encode(w, lens_np, cfg):
    q4 = torch.full((dkv.dkv_q4_0_cache_bytes(cfg),), 0xA5, dtype=torch.uint8, device=U.DEV)
    k, v = _f16_inputs(w, lens_np, poison=False)
    lens = torch.from_numpy(lens_np).to(U.DEV)
    dkv.dkv_q4_0_encode(cfg, q4, k, v, lens, w.S)
    return q4, lens


@pytest.mark.parametrize("name,kw,lens", CASES, ids=lambda x: str(x))
def test_q40_encode_bit_exact(name, kw, lens):
    w, lens_np, cfg = _setup(name, kw, lens)
    q4, lens_t = _q40_encode(w, lens_np, cfg)
    S, D = w.S, w.D
    codes = torch.zeros((w.B, w.Hkv, 2, S, D // 2), dtype=torch.uint8, device=U.DEV)
    scales = torch.zeros((w.B, w.Hkv, 2, S, D // 32), dtype=torch.int16, device=U.DEV)
    dkv.dkv_q4_0_export(cfg, q4, lens_t, S, codes, scales)
    codes = codes.cpu().numpy()
    scales = scales.cpu().numpy().view(np.uint16)
    for b in range(w.B):
        L = int(lens_np[b])
        for h in range(w.Hkv):
            for s, x in enumerate((w.k, w.v)):
                oc, osc = oracle.q40_abs_stream(np.ascontiguousarray(x[b, h, :L]))
                assert np.array_equal(codes[b, h, s, :L], oc), ("codes", b, h, s)
                assert np.array_equal(scales[b, h, s, :L], osc), ("scales", b, h, s)


@pytest.mark.parametrize("name,kw,lens", CASES, ids=lambda x: str(x))
def test_q40_attention_parity(name, kw, lens):
    w, lens_np, cfg = _setup(name, kw, lens)
    q4, lens_t = _q40_encode(w, lens_np, cfg)
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=U.DEV)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_attn_decode_q4_0(cfg, q4, q, lens_t, out, ws)
    got = out.cpu().numpy()
    G = w.Hq // w.Hkv
    scale = np.float32(1 / math.sqrt(w.D))
    ref = np.zeros((w.B, w.Hq, w.D))
    for b in range(w.B):
        L = int(lens_np[b])
        for h in range(w.Hkv):
            kr = oracle.q40_dequant_stream(*oracle.q40_abs_stream(np.ascontiguousarray(w.k[b, h, :L])))
            vr = oracle.q40_dequant_stream(*oracle.q40_abs_stream(np.ascontiguousarray(w.v[b, h, :L])))
            ref[b, h * G:(h + 1) * G] = oracle.attention_f64(q_np[b, h * G:(h + 1) * G], kr, vr, scale)
    for b in range(w.B):
        if lens_np[b] == 0:
            assert np.all(got[b] == 0.0)
    assert U.rel_err(got, ref) <= U.ATTN_TOL


@pytest.mark.parametrize("name,kw,lens", CASES, ids=lambda x: str(x))
def test_f16_attention_parity(name, kw, lens):
    w, lens_np, cfg = _setup(name, kw, lens)
    k, v = _f16_inputs(w, lens_np, poison=True)
    lens_t = torch.from_numpy(lens_np).to(U.DEV)
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    out = torch.full((w.B, w.Hq, w.D), float("nan"), dtype=torch.float32, device=U.DEV)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_attn_decode_f16(cfg, k, v, w.S, q, lens_t, out, ws)
    got = out.cpu().numpy()
    G = w.Hq // w.Hkv
    scale = np.float32(1 / math.sqrt(w.D))
    ref = np.zeros((w.B, w.Hq, w.D))
    for b in range(w.B):
        L = int(lens_np[b])
        for h in range(w.Hkv):
            kr = w.k[b, h, :L].astype(np.float32)
            vr = w.v[b, h, :L].astype(np.float32)
            ref[b, h * G:(h + 1) * G] = oracle.attention_f64(q_np[b, h * G:(h + 1) * G], kr, vr, scale)
    for b in range(w.B):
        if lens_np[b] == 0:
            assert np.all(got[b] == 0.0)
    assert U.rel_err(got, ref) <= U.ATTN_TOL


def test_delta_kv_closer_to_f16_than_q40():
    """On the 1 % AR(1) data the Delta-KV attention output is closer to F16
    attention than plain Q4_0 attention is (the quality claim of the Delta-KV
    article's benchmark section, measured here on attention outputs)."""
    w, lens_np, cfg = _setup("8b", dict(S=1024, Hq=8, Hkv=2), None)
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    lens_t = torch.from_numpy(lens_np).to(U.DEV)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    outs = {}
    k, v = _f16_inputs(w, lens_np, poison=False)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device=U.DEV)
    dkv.dkv_attn_decode_f16(cfg, k, v, w.S, q, lens_t, out, ws)
    outs["f16"] = out.cpu().numpy()
    q4, _ = _q40_encode(w, lens_np, cfg)
    dkv.dkv_attn_decode_q4_0(cfg, q4, q, lens_t, out, ws)
    outs["q40"] = out.cpu().numpy()
    r = U.prefill(w, kf=32)
    outs["dkv"] = U.attention(r, q_np)
    e_q = np.abs(outs["q40"] - outs["f16"]).max()
    e_d = np.abs(outs["dkv"] - outs["f16"]).max()
    assert e_d < e_q, (e_d, e_q)


@pytest.mark.parametrize("name,kw,lens", [
    ("tiny", dict(), None),
    ("8b", dict(S=700, Hq=8, Hkv=2), None),
    ("8b", dict(S=400, Hq=8, Hkv=2, D=64), None),
    ("long", dict(S=900, B=2, Hq=8, Hkv=2), None),
    ("8b", dict(S=300, B=6, Hq=8, Hkv=2), [0, 1, 31, 32, 33, 300]),
])
def test_q8_0_encode_bit_exact(name, kw, lens):
    """Q8_0 codes and fp16 scale bit patterns equal the oracle's Q8_0 of the
    absolute rows; rows past each sequence's length keep their contents."""
    w, lens_np, cfg = _setup(name, kw, lens)
    print(f"q8_0 case {name} {kw} lens={lens}", flush=True)
    B, H, S, D = w.B, w.Hkv, w.S, w.D
    k = torch.from_numpy(np.ascontiguousarray(w.k)).to(U.DEV)
    v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    codes = torch.full((B, H, 2, S, D), 0x55, dtype=torch.int8, device=U.DEV)
    scales = torch.full((B, H, 2, S, D // 32), 0x1234, dtype=torch.int16, device=U.DEV)
    dkv.dkv_q8_0_encode(cfg, k, v, torch.from_numpy(lens_np).to(U.DEV), S, codes, scales)
    torch.cuda.synchronize()
    gc = codes.cpu().numpy()
    gs = scales.cpu().numpy().view(np.uint16)
    for b in range(B):
        L = int(lens_np[b])
        for h in range(H):
            for s, x in enumerate((w.k, w.v)):
                rc, rs = oracle.q80_abs_stream(x[b, h, :L])
                assert np.array_equal(gc[b, h, s, :L], rc), (b, h, s)
                assert np.array_equal(gs[b, h, s, :L], rs), (b, h, s)
                assert np.all(gc[b, h, s, L:] == 0x55) and np.all(gs[b, h, s, L:] == 0x1234)
