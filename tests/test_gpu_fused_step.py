"""GPU checks of dkv_append_attn_decode, one serving step in one call (the append
of each sequence's new token fused into the decode's split launch where the
kf = 32, GQA <= 8 kernel runs, the append kernel first elsewhere).

Every step must leave the cache bytes and the reconstruction state bit-identical
to dkv_append followed by dkv_attn_decode, and give bit-identical attention
outputs (the same kernels read the same bytes); after the steps the cache must
still reconstruct bit-exactly as the oracle's encoding of the grown sequences,
and attention must be within 2e-3 of the float64 oracle.
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

pytestmark = pytest.mark.gpu

import gpu_util as U  # noqa: E402

CASES = [
    # (workload, overrides, page_tokens, kf, steps); every case crosses a group boundary
    ("mixed", dict(S=600, B=4, Hq=8, Hkv=2, min_len=64, extra_tokens=40), 256, 32, 40),
    ("8b", dict(S=300, B=3, Hq=8, Hkv=2, extra_tokens=40), 0, 32, 40),
    ("70b", dict(S=200, B=2, Hq=16, Hkv=2, extra_tokens=40), 0, 32, 35),
    ("8b", dict(S=200, B=2, Hq=8, Hkv=2, D=64, extra_tokens=40), 0, 32, 35),
    ("8b", dict(S=300, B=2, Hq=8, Hkv=2, extra_tokens=70), 0, 64, 70),      # long-interval kernel: append first
    ("70b", dict(S=200, B=2, Hq=16, Hkv=1, extra_tokens=40), 0, 32, 35),    # 16 heads per kv-head: append first
]


def _clone(r):
    c = U.Run()
    c.__dict__.update(r.__dict__)
    c.cache = r.cache.clone()
    c.state = r.state.clone()
    c.ws = torch.zeros_like(r.ws)
    return c


@pytest.mark.parametrize("name,kw,page,kf,steps", CASES)
def test_fused_step_matches_append_then_decode(name, kw, page, kf, steps):
    w = synth.make(name, **kw)
    print(f"fused step case {name} {kw} page={page} kf={kf}", flush=True)
    a = U.prefill(w, kf=kf, page_tokens=page)
    b = _clone(a)
    lens = a.lens_np.copy()
    oa = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    ob = torch.zeros_like(oa)
    for step in range(steps):
        pos = torch.from_numpy(lens.astype(np.int32)).to(U.DEV)
        kn = torch.stack([a.k[i, :, int(lens[i])] for i in range(w.B)]).contiguous()
        vn = torch.stack([a.v[i, :, int(lens[i])] for i in range(w.B)]).contiguous()
        lens += 1
        ln = torch.from_numpy(lens.astype(np.int32)).to(U.DEV)
        q = torch.from_numpy(synth.queries(w, step=step)).to(U.DEV)
        dkv.dkv_append(a.cfg, a.cache, a.state, a.bt, kn, vn, pos)
        dkv.dkv_attn_decode(a.cfg, a.cache, a.bt, q, ln, oa, a.ws)
        dkv.dkv_append_attn_decode(b.cfg, b.cache, b.state, b.bt, kn, vn, pos, q, ln, ob, b.ws)
        torch.cuda.synchronize()
        assert torch.equal(a.cache, b.cache), f"cache differs after step {step}"
        assert torch.equal(a.state, b.state), f"state differs after step {step}"
        assert torch.equal(oa, ob), f"output differs after step {step}"
    b.lens_np = lens.astype(np.int32)
    b.lens = torch.from_numpy(b.lens_np).to(U.DEV)
    enc = U.oracle_encode(w, kf, b.lens_np)
    U.assert_codec_exact(b, enc, kf)
    q = synth.queries(w, step=steps - 1)
    ref = U.oracle_attention(enc, w, q, b.lens_np)
    assert U.rel_err(ob.cpu().numpy(), ref) <= U.ATTN_TOL


def test_fused_step_skips_negative_positions():
    """A negative position appends nothing for that sequence, as dkv_append."""
    w = synth.make("8b", S=200, B=3, Hq=8, Hkv=2, extra_tokens=10)
    a = U.prefill(w)
    b = _clone(a)
    lens = a.lens_np.copy()
    p = np.array([lens[0], -1, lens[2]], np.int32)
    pos = torch.from_numpy(p).to(U.DEV)
    kn = torch.stack([a.k[i, :, int(lens[i])] for i in range(w.B)]).contiguous()
    vn = torch.stack([a.v[i, :, int(lens[i])] for i in range(w.B)]).contiguous()
    ln = torch.from_numpy((lens + (p >= 0)).astype(np.int32)).to(U.DEV)
    q = torch.from_numpy(synth.queries(w)).to(U.DEV)
    oa = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    ob = torch.zeros_like(oa)
    dkv.dkv_append(a.cfg, a.cache, a.state, a.bt, kn, vn, pos)
    dkv.dkv_attn_decode(a.cfg, a.cache, a.bt, q, ln, oa, a.ws)
    dkv.dkv_append_attn_decode(b.cfg, b.cache, b.state, b.bt, kn, vn, pos, q, ln, ob, b.ws)
    torch.cuda.synchronize()
    assert torch.equal(a.cache, b.cache) and torch.equal(a.state, b.state) and torch.equal(oa, ob)
