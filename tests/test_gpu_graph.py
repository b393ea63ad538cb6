"""Decode attention captured in a HIP graph and replayed.

The decode step (split phase + combine) is captured once and replayed several
times, with eager decode work and synchronisations between the replays; every
replay must reproduce the eager output bit for bit.
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

pytestmark = pytest.mark.gpu

import gpu_util as U  # noqa: E402


@pytest.mark.parametrize("name,kw,kf", [("70b", dict(S=999, B=3, Hq=16, Hkv=2), 32),
                                        ("long", dict(S=1300, B=2, Hq=8, Hkv=2, kf=512), 512)])
def test_graph_replay_matches_eager(name, kw, kf):
    w = synth.make(name, **kw)
    r = U.prefill(w, kf=kf)
    q = torch.from_numpy(synth.queries(w)).to(U.DEV)
    q2 = torch.from_numpy(synth.queries(w, 1)).to(U.DEV)
    out = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    other = torch.zeros_like(out)
    dkv.dkv_attn_decode(r.cfg, r.cache, r.bt, q, r.lens, out, r.ws)
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dkv.dkv_attn_decode(r.cfg, r.cache, r.bt, q, r.lens, out, r.ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        # eager work on the same workspace between replays
        dkv.dkv_attn_decode(r.cfg, r.cache, r.bt, q2, r.lens, other, r.ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
    assert not torch.equal(other, eager)


def test_strided_graph_replay_matches_eager():
    """The strided-reference decode (split phase + combine) captured once and
    replayed, with eager strided decodes on the same workspace in between."""
    w = synth.make("70b", S=999, B=3, Hq=16, Hkv=2)
    print("strided graph replay", flush=True)
    cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=32, max_tokens=w.S)
    cache = torch.zeros(dkv.dkv_strided_cache_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    lens = torch.from_numpy(np.asarray(w.seq_lens, np.int32)).to(U.DEV)
    dkv.dkv_strided_encode_prefill(cfg, cache, torch.from_numpy(w.k).to(U.DEV), torch.from_numpy(w.v).to(U.DEV),
                                   lens, w.S, 64)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=U.DEV)
    q = torch.from_numpy(synth.queries(w)).to(U.DEV)
    q2 = torch.from_numpy(synth.queries(w, 1)).to(U.DEV)
    out = torch.zeros(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    other = torch.zeros_like(out)
    dkv.dkv_strided_attn_decode(cfg, cache, q, lens, out, ws)
    torch.cuda.synchronize()
    eager = out.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            dkv.dkv_strided_attn_decode(cfg, cache, q, lens, out, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        dkv.dkv_strided_attn_decode(cfg, cache, q2, lens, other, ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
    assert not torch.equal(other, eager)
