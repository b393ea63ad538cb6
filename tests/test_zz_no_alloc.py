"""GPU check of dkv_attn_decode_noalloc (the decode whose split-K partials live
in the library's fixed device scratch array) against dkv_attn_decode with a
caller-owned workspace, through the C ABI: two calls in a row on one GPU, the
second with a smaller input, each output bit-identical to dkv_attn_decode's
(same kernels and split plan) and within 2e-3 of the float64 oracle on
sampled rows.  The reference workspace's partial records are filled with NaN
bytes (its arrival counters with zeros), so neither path may read partial
records it has not written."""
import math

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

import gpu_util as U  # noqa: E402

pytestmark = pytest.mark.gpu


def _one_call(w, kf, page_tokens, pairs):
    r = U.prefill(w, kf=kf, page_tokens=page_tokens)
    q_np = synth.queries(w)
    q = torch.from_numpy(q_np).to(U.DEV)
    ws = torch.full((dkv.dkv_workspace_bytes(r.cfg),), 0xFF, dtype=torch.uint8, device=U.DEV)
    ws[:(r.cfg.batch * r.cfg.n_kv_heads * 4 + 255) // 256 * 256] = 0      # arrival counters start at zero
    ref = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    got = torch.full_like(ref, float("nan"))
    dkv.dkv_attn_decode(r.cfg, r.cache, r.bt, q, r.lens, ref, ws)
    dkv.dkv_attn_decode_noalloc(r.cfg, r.cache, r.bt, q, r.lens, got)
    torch.cuda.synchronize()
    assert torch.equal(got, ref), float((got - ref).abs().max())
    # and the oracle, on sampled (sequence, kv-head) pairs
    G, D = w.Hq // w.Hkv, w.D
    scale = np.float32(1 / math.sqrt(D))
    g = got.cpu().numpy()
    for b, h in pairs:
        L = int(r.lens_np[b])
        ek = oracle.encode_stream(np.ascontiguousarray(w.k[b, h, :L]), r.cfg.kf)
        ev = oracle.encode_stream(np.ascontiguousarray(w.v[b, h, :L]), r.cfg.kf)
        o = oracle.attention_f64(q_np[b, h * G:(h + 1) * G], ek.recon, ev.recon, scale)
        assert U.rel_err(g[b, h * G:(h + 1) * G][None], o[None]) <= U.ATTN_TOL, (b, h)


@pytest.mark.parametrize("kf,page_tokens", [(32, 0), (128, 0), (32, 256)])
def test_noalloc_matches_workspace_decode_twice(kf, page_tokens):
    print(f"noalloc decode kf={kf} page_tokens={page_tokens}", flush=True)
    big = synth.make("70b", B=8, S=4096, Hq=64, Hkv=8)
    _one_call(big, kf, page_tokens, [(0, 0), (5, 7)])
    small = synth.make("8b", B=2, S=700, Hq=8, Hkv=2)
    _one_call(small, kf, page_tokens, [(0, 1), (1, 0)])
