"""Helpers of the GPU parity tests: upload a synthetic workload, run the HIP
path through the C ABI, and compare it with the CPU oracle."""
import math

import numpy as np
import torch

import oracle
import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

DEV = torch.device("cuda:0")
ATTN_TOL = 2e-3   # max relative error per output row, vs the float64 oracle


class Run:
    pass


def make_cfg(w, kf=None, page_tokens=0, capacity=None):
    kf = kf or w.kf
    cap = capacity or (w.S + w.extra_tokens)
    if page_tokens:
        maxp = -(-cap // page_tokens)
        return dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=kf,
                          max_tokens=0, page_tokens=page_tokens, n_pages=0, max_pages_per_seq=maxp)
    return dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=kf, max_tokens=cap)


def shuffled_pages(w, cfg, seed=5):
    need = [-(-(int(L) + w.extra_tokens) // cfg.page_tokens) for L in w.seq_lens]
    n = int(sum(need))
    perm = np.random.default_rng(seed).permutation(n).astype(np.int32)
    table = np.full((w.B, cfg.max_pages_per_seq), -1, np.int32)
    pos = 0
    for b, k in enumerate(need):
        table[b, :k] = perm[pos:pos + k]
        pos += k
    return table, n


def prefill(w, kf=None, page_tokens=0, lens=None, capacity=None):
    r = Run()
    r.w = w
    r.cfg = make_cfg(w, kf, page_tokens, capacity)
    r.bt = None
    if page_tokens:
        table, n = shuffled_pages(w, r.cfg)
        r.cfg.n_pages = n
        r.bt = torch.from_numpy(table).to(DEV)
    r.lens_np = np.asarray(w.seq_lens if lens is None else lens, np.int32)
    r.lens = torch.from_numpy(r.lens_np).to(DEV)
    r.cache = torch.full((dkv.dkv_cache_bytes(r.cfg),), 0xA5, dtype=torch.uint8, device=DEV)
    r.state = torch.zeros(w.B, w.Hkv, 2, w.D, dtype=torch.float32, device=DEV)
    r.ws = torch.zeros(dkv.dkv_workspace_bytes(r.cfg), dtype=torch.uint8, device=DEV)
    r.k = torch.from_numpy(np.ascontiguousarray(w.k)).to(DEV)
    r.v = torch.from_numpy(np.ascontiguousarray(w.v)).to(DEV)
    r.s_max = w.k.shape[2]
    dkv.dkv_encode_prefill(r.cfg, r.cache, r.state, r.bt, r.k, r.v, r.lens, r.s_max)
    return r


def export(r, s_max=None):
    s_max = s_max or r.s_max
    skf, scd, ssc = dkv.export_shapes(r.cfg, s_max)
    kf = torch.zeros(skf, dtype=torch.int16, device=DEV)
    cd = torch.zeros(scd, dtype=torch.uint8, device=DEV)
    sc = torch.zeros(ssc, dtype=torch.int16, device=DEV)
    dkv.dkv_export(r.cfg, r.cache, r.bt, r.lens, s_max, kf, cd, sc)
    return (kf.cpu().numpy().view(np.uint16), cd.cpu().numpy(), sc.cpu().numpy().view(np.uint16))


def reconstruct(r, s_max=None):
    s_max = s_max or r.s_max
    w = r.w
    ko = torch.zeros(w.B, w.Hkv, s_max, w.D, dtype=torch.float32, device=DEV)
    vo = torch.zeros_like(ko)
    dkv.dkv_reconstruct(r.cfg, r.cache, r.bt, r.lens, s_max, ko, vo)
    return ko.cpu().numpy(), vo.cpu().numpy()


def oracle_encode(w, kf, lens, pairs=None):
    enc = {}
    for b in range(w.B):
        L = int(lens[b])
        for h in range(w.Hkv):
            if pairs is not None and (b, h) not in pairs:
                continue
            for s, x in ((0, w.k), (1, w.v)):
                enc[(b, h, s)] = oracle.encode_stream(np.ascontiguousarray(x[b, h, :L]), kf)
    return enc


def assert_codec_exact(r, enc, kf):
    """Keyframes, codes, scales (fp16 bits), reconstruction and state: bit-exact."""
    ekf, ecd, esc = export(r)
    kr, vr = reconstruct(r)
    state = r.state.cpu().numpy()
    for (b, h, s), e in enc.items():
        L = e.S
        ng, nd = oracle.n_groups(L, kf), oracle.n_delta(L, kf)
        assert np.array_equal(ekf[b, h, s, :ng], e.kf_rows), ("keyframes", b, h, s)
        assert np.array_equal(ecd[b, h, s, :nd], e.codes), ("codes", b, h, s)
        assert np.array_equal(esc[b, h, s, :nd], e.scales), ("scales", b, h, s)
        rec = (kr if s == 0 else vr)[b, h, :L]
        assert np.array_equal(rec.view(np.uint32), e.recon.view(np.uint32)), ("recon", b, h, s)
        if L > 0:
            assert np.array_equal(state[b, h, s].view(np.uint32), e.state.view(np.uint32)), ("state", b, h, s)


def attention(r, q_np, fn="dkv_attn_decode", lens=None):
    q = torch.from_numpy(np.ascontiguousarray(q_np)).to(DEV)
    out = torch.full((r.w.B, r.w.Hq, r.w.D), float("nan"), dtype=torch.float32, device=DEV)
    getattr(dkv, fn)(r.cfg, r.cache, r.bt, q, r.lens if lens is None else lens, out, r.ws)
    return out.cpu().numpy()


def oracle_attention(enc, w, q, lens, pairs=None):
    G = w.Hq // w.Hkv
    out = np.full((w.B, w.Hq, w.D), np.nan)
    scale = np.float32(1 / math.sqrt(w.D))
    for b in range(w.B):
        for h in range(w.Hkv):
            if pairs is not None and (b, h) not in pairs:
                continue
            hq = slice(h * G, (h + 1) * G)
            out[b, hq] = oracle.attention_f64(q[b, hq], enc[(b, h, 0)].recon, enc[(b, h, 1)].recon, scale)
    return out


def rel_err(got, ref):
    """Per output row: max |got - ref| / max |ref| (rows with ref == 0 use abs error)."""
    mask = ~np.isnan(ref[..., 0])
    g = got[mask].astype(np.float64)
    rr = ref[mask]
    den = np.abs(rr).max(-1)
    den = np.where(den > 0, den, 1.0)
    return (np.abs(g - rr).max(-1) / den).max() if g.size else 0.0


def make(name, **kw):
    return synth.make(name, **kw)
