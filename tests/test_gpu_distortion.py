"""GPU parity of the attention-preserving distortion report ("KV 캐시 벡터 양자화와
주의 보존 변환", 어텐션 보존 왜곡) against the CPU oracle, through the C ABI.

The HIP path encodes the cache, reconstructs K/V (dkv_reconstruct, itself
bit-exact with the oracle) and computes d_k, d_v per (sequence, query head) in
fp32 from the reconstruction-minus-input differences; the oracle does the same
in float64 on its own encoding.  Both quantities are sums of squares of small
differences, so fp32 accumulation over at most a few thousand tokens stays
within 1e-4 relative (the bar written here, per row, with an absolute floor of
1e-6 of the largest row for rows that are zero or nearly so).
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

RTOL = 1e-4

CASES = [
    ("tiny", dict(), None, 0),
    ("8b", dict(S=700, Hq=8, Hkv=2), None, 0),
    ("8b", dict(S=400, Hq=8, Hkv=2, D=64), None, 0),
    ("long", dict(S=1500, B=2, Hq=8, Hkv=2), None, 0),
    ("8b", dict(S=300, B=6, Hq=8, Hkv=2), [0, 1, 31, 32, 33, 300], 0),
    ("mixed", dict(B=3, S=2000, Hq=8, Hkv=2, min_len=100, extra_tokens=0), None, 256),
]


def _close(got, ref):
    floor = 1e-6 * max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref) / np.maximum(np.abs(ref), floor)
    return float(err.max())


def _distortion_gpu(cfg, kh, vh, k, v, s_max, q, lens, scale):
    B, Hq = cfg.batch, cfg.n_q_heads
    d_k = torch.full((B, Hq), float("nan"), device=U.DEV)
    d_v = torch.full((B, Hq), float("nan"), device=U.DEV)
    logits = torch.empty(B * Hq * s_max, dtype=torch.float32, device=U.DEV)
    dkv.dkv_attn_distortion(cfg, kh, vh, k, v, s_max, q, lens, d_k, d_v, logits, softmax_scale=scale)
    torch.cuda.synchronize()
    return d_k.cpu().numpy().astype(np.float64), d_v.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("name,kw,lens,page", CASES)
def test_delta_kv_distortion_matches_oracle(name, kw, lens, page):
    w = synth.make(name, **kw)
    print(f"distortion case {name} {kw} lens={lens} page={page}", flush=True)
    r = U.prefill(w, page_tokens=page, lens=lens)
    kh = torch.empty(w.B, w.Hkv, r.s_max, w.D, dtype=torch.float32, device=U.DEV)
    vh = torch.empty_like(kh)
    dkv.dkv_reconstruct(r.cfg, r.cache, r.bt, r.lens, r.s_max, kh, vh)
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    scale = 1.0 / math.sqrt(w.D)
    d_k, d_v = _distortion_gpu(r.cfg, kh, vh, r.k, r.v, r.s_max, q, r.lens, scale)

    enc = oracle.encode_cache(w.k, w.v, r.lens_np, w.kf)
    rk, rv = oracle.attention_distortion_cache(enc, w.k, w.v, q_np, r.lens_np, w.Hkv, scale)
    assert _close(d_k, rk) <= RTOL, (d_k, rk)
    assert _close(d_v, rv) <= RTOL, (d_v, rv)
    for b in range(w.B):
        if r.lens_np[b] == 0:
            assert np.all(d_k[b] == 0) and np.all(d_v[b] == 0)


def test_q4_0_distortion_matches_oracle():
    """The same report on the plain Q4_0 comparison (dequantised on the device
    from its own export) against the oracle's Q4_0 of the absolute rows."""
    w = synth.make("8b", S=600, Hq=8, Hkv=2)
    lens_np = np.asarray(w.seq_lens, np.int32)
    cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=32, max_tokens=w.S)
    k = torch.from_numpy(np.ascontiguousarray(w.k)).to(U.DEV)
    v = torch.from_numpy(np.ascontiguousarray(w.v)).to(U.DEV)
    lens = torch.from_numpy(lens_np).to(U.DEV)
    q4 = torch.zeros(dkv.dkv_q4_0_cache_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_q4_0_encode(cfg, q4, None, k, v, lens, w.S)
    B, H, S, D = w.B, w.Hkv, w.S, w.D
    codes = torch.zeros(B, H, 2, S, D // 2, dtype=torch.uint8, device=U.DEV)
    scales = torch.zeros(B, H, 2, S, D // 32, dtype=torch.int16, device=U.DEV)
    dkv.dkv_q4_0_export(cfg, q4, None, lens, S, codes, scales)
    deq = []
    for s in range(2):
        c = codes[:, :, s].reshape(B, H, S, D // 32, 16)
        full = torch.cat([(c & 15), (c >> 4)], dim=-1).float() - 8.0
        sc = scales[:, :, s].view(torch.float16).float()[..., None]
        deq.append((full * sc).reshape(B, H, S, D).contiguous())
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    scale = 1.0 / math.sqrt(D)
    d_k, d_v = _distortion_gpu(cfg, deq[0], deq[1], k, v, S, q, lens, scale)

    G = w.Hq // w.Hkv
    rk = np.zeros((B, w.Hq))
    rv = np.zeros((B, w.Hq))
    for b in range(B):
        L = int(lens_np[b])
        for h in range(H):
            kd = oracle.q40_dequant_stream(*oracle.q40_abs_stream(w.k[b, h, :L]))
            vd = oracle.q40_dequant_stream(*oracle.q40_abs_stream(w.v[b, h, :L]))
            kx = w.k[b, h, :L].astype(np.float64)
            vx = w.v[b, h, :L].astype(np.float64)
            rk[b, h * G:(h + 1) * G], rv[b, h * G:(h + 1) * G] = oracle.attention_distortion_f64(
                q_np[b, h * G:(h + 1) * G], kx, vx, kd, vd, scale)
    assert _close(d_k, rk) <= RTOL, (d_k, rk)
    assert _close(d_v, rv) <= RTOL, (d_v, rv)
