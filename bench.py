#!/usr/bin/env python3
"""Delta-KV fused decode attention benchmark (one MI355X).

One step = one decode layer-step: fused decode attention (split phase +
combine) of every query head of the batch over the whole compressed cache of
one layer.  Default workload: the Llama-3-70B-shaped layer (B=16, 64 q / 8 kv
heads, D=128, S=32768, kf=32), synthetic AR(1) K/V, resident in HBM before the
timed region.  Prints ONE JSON line.

Reported:
  value        effective KV GB/s = fp16-equivalent KV bytes of the layer
               (2 * Hkv * D * S * B * 2 bytes) / step time
  roofline     dominant kernel (the fused split-phase kernel): algorithmic
               compressed bytes (+ q + partials) per launch / its average
               duration from HIP events on the launch stream, vs 8 TB/s
  cpu_baseline the CPU oracle (reconstruct + float64 attention) on a bounded
               sample of the same workload, single thread
  comparisons  the in-run F16 and plain-Q4_0 decode attentions on the same
               data (same split-K plan and combine), with their own rates
  quality      reconstruction MSE of Delta-KV and of Q4_0 against the fp16
               input, from the GPU outputs (dkv_reconstruct, dkv_q4_0_export)
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0

# HBM bytes per launch of the kf = 32, GQA<=8 split kernel on the 70b workload, from
# rocprofv3 FETCH_SIZE (x2.0) and WRITE_SIZE (x1.0) counters, each scaled by
# what the counter reads for a 1 GiB device copy.  Valid only for the kernel
# sources it was measured on (sha256 below); otherwise traffic is null.
MEASURED_TRAFFIC = {
    "workload": "70b", "kf": 32, "bytes": 692390917,
    "sources": {
        "dkv_attn_g8.hip": "0c343f056b996ccd86343ee0541bfcd9fe4e684bb2ca9085089d8036a6c4df02",
        "dkv_fused_common.h": "fdaf23f919b7f5576833b80881851acabb27f65d569c3f957be0ac5f1f8f35bd",
        "dkv_common.h": "3b302839f810f8e0f48d1491035b2d391a13053c69aed1c169162f01349d5e17",
    },
}


def spin_up(fn, ms):
    """Run fn() back to back for at least `ms` of wall time, then synchronize.

    An idle GPU starts a burst of work at reduced clocks; before the warmup
    steps the decode kernels run long enough for the clocks to settle, so the
    timed steps measure the steady state of continuous decoding.
    """
    import torch
    t_end = time.perf_counter() + ms * 1e-3
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def measured_traffic(workload, kf, kernel):
    import hashlib
    t = MEASURED_TRAFFIC
    if kernel != "fused" or workload != t["workload"] or kf != t["kf"]:
        return None
    src = os.path.join(ROOT, "quantized_decode_attention_delta_amd", "csrc")
    for name, digest in t["sources"].items():
        with open(os.path.join(src, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return t["bytes"]
METRIC = "Delta-KV decode attn: effective KV GB/s (% HBM peak) + layer-steps/s"


def algorithmic_bytes(B, Hkv, Hq, D, S, kf):
    """Compressed bytes one decode layer-step must read: per stream
    2*D*ceil(S/kf) keyframe bytes + 18*(D/32) bytes per delta token."""
    ng = -(-S // kf)
    per_stream = 2 * D * ng + 18 * (D // 32) * (S - ng)
    return 2 * B * Hkv * per_stream


def f16_equiv_bytes(B, Hkv, D, S):
    return 2 * Hkv * D * S * B * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="70b", choices=["tiny", "8b", "long", "70b", "mixed"])
    ap.add_argument("--mixed-batch", type=int, default=None, help="mixed workload: fewer sequences (default 64)")
    ap.add_argument("--mixed-max-len", type=int, default=None, help="mixed workload: shorter maximum length")
    ap.add_argument("--kf", type=int, default=None)
    ap.add_argument("--kernel", default="fused", choices=["fused", "ref"])
    ap.add_argument("--replicas", type=int, default=0, help="cache copies rotated per step (0 = auto, >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads (0 = min(16, host cores))")
    ap.add_argument("--spin-up-ms", type=float, default=300.0,
                    help="run the decode kernels this long before the warmup steps (GPU clocks settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true", help="skip the F16 / Q4_0 comparisons and the MSE report")
    ap.add_argument("--graph-layers", type=int, default=None,
                    help="decode steps of this many layers captured in one HIP graph and replayed "
                         "(default 32 for the launch-bound tiny and 8b workloads, 0 otherwise)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy a 1 GiB device buffer 3 times (a plain copy kernel of known size, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    return ap.parse_args()


def cpu_baseline(w, kf, budget_s, threads, min_s=10.0):
    """Oracle (as it stands) on a bounded sample: whole (sequence, kv-head)
    pairs, reconstruct K/V from the oracle's own encoding, float64 attention of
    the pair's G query heads.  Independent pairs run on `threads` host threads
    (the oracle's C routines release the GIL).  Encoding is untimed (it is not
    decode work); the sample grows until about `budget_s` of timed work, and
    when every pair has been decoded in less than `min_s` the pairs are
    decoded again (whole passes) until `min_s` of timed work."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    from quantized_decode_attention_delta_amd import synth
    q = synth.queries(w)
    G = w.Hq // w.Hkv
    scale = np.float32(1 / math.sqrt(w.D))
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    enc = {}

    def encode(bh):
        b, h = bh
        S = int(w.seq_lens[b])
        enc[bh] = (oracle.encode_stream(np.ascontiguousarray(w.k[b, h, :S]), kf, want_recon=False),
                   oracle.encode_stream(np.ascontiguousarray(w.v[b, h, :S]), kf, want_recon=False))

    def decode(bh):
        b, h = bh
        S = int(w.seq_lens[b])
        ek, ev = enc[bh]
        kr = oracle.reconstruct_stream(ek.kf_rows, ek.codes, ek.scales, S, w.D, kf)
        vr = oracle.reconstruct_stream(ev.kf_rows, ev.codes, ev.scales, S, w.D, kf)
        oracle.attention_f64(q[b, h * G:(h + 1) * G], kr, vr, scale)

    done = 0
    t_total = 0.0
    with cf.ThreadPoolExecutor(threads) as ex:
        while done < len(pairs) and t_total < budget_s:
            batch = pairs[done:done + threads]
            list(ex.map(encode, batch))
            t0 = time.perf_counter()
            list(ex.map(decode, batch))
            t_total += time.perf_counter() - t0
            done += len(batch)
        if done == len(pairs):
            while t_total < min(min_s, budget_s):
                t0 = time.perf_counter()
                list(ex.map(decode, pairs))
                t_total += time.perf_counter() - t0
                done += len(pairs)
    S = int(w.seq_lens[0])
    eff_bytes = done * 2 * w.D * S * 2        # fp16-equivalent K+V bytes of the sampled pairs
    return {
        "value": round(eff_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} decodes of (sequence, kv-head) pairs of the same workload ({len(pairs)} pairs"
                  f"{', whole passes repeated' if done > len(pairs) else ''}): oracle reconstruction of K and V "
                  f"+ float64 attention of {G} query heads, pairs on {threads} host threads, {t_total:.1f} s",
        "layer_steps_per_s_extrapolated": round(done / t_total / len(pairs), 6),
    }


def graph_layers(cfg, caches, q, lens, layers, stream, replays=50):
    """A decoder's view of a launch-bound layer: the decode steps of `layers`
    layers (each its own copy of the cache) captured in one HIP graph (two
    kernels per layer, no host launch in between) and replayed; the replays are
    timed with HIP events on the replay stream."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    if len(caches) < layers:
        caches = caches + [caches[0].clone() for _ in range(layers - len(caches))]
    out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=q.device)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=q.device)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):                  # warm-up outside the capture
        for l in range(layers):
            dkv.dkv_attn_decode(cfg, caches[l], None, q, lens, out, ws)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(layers):
            dkv.dkv_attn_decode(cfg, caches[l], None, q, lens, out, ws)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    rs = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(rs)
    for _ in range(replays):
        g.replay()
    e1.record(rs)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * layers)
    return {"layers": layers, "ms_per_layer_step": round(ms, 5), "layer_steps_per_s": round(1000.0 / ms, 2),
            "how": f"{layers} layers' decode steps (split + combine each, a cache copy per layer) in one "
                   f"HIP graph, {replays} replays timed with HIP events"}


def _time(fn, n, stream):
    """Mean ms per call of fn(i), i = 0..n-1, from HIP events on `stream`
    (after 100 ms of calls for the clocks to settle, and 3 warmup calls)."""
    import torch
    spin_up(lambda: fn(0), 100.0)
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def comparisons(w, cfg, k, v, q, lens, ws, steps, stream, qo):
    """In-run F16 and plain-Q4_0 decode attention on the same K/V and queries."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=k.device)
    res = {}
    f16_bytes = f16_equiv_bytes(w.B, w.Hkv, w.D, w.S)
    reps = max(1, math.ceil((1 << 30) / f16_bytes))
    ks = [k] + [k.clone() for _ in range(reps - 1)]
    vs = [v] + [v.clone() for _ in range(reps - 1)]
    ms = _time(lambda i: dkv.dkv_attn_decode_f16(cfg, ks[i % reps], vs[i % reps], None, q, lens, out, ws),
               steps, stream)
    res["f16"] = {"ms_per_step": round(ms, 5), "GBps": round((f16_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                  "hbm_frac": round((f16_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                  "bytes": f16_bytes, "replicas": reps}
    del ks, vs
    q4_bytes = 2 * w.B * w.Hkv * w.S * (w.D // 32) * 18
    q4 = torch.empty(dkv.dkv_q4_0_cache_bytes(cfg), dtype=torch.uint8, device=k.device)
    dkv.dkv_q4_0_encode(cfg, q4, None, k, v, lens, w.S)
    reps = max(1, math.ceil((1 << 30) / q4.numel()))
    q4s = [q4] + [q4.clone() for _ in range(reps - 1)]
    ms = _time(lambda i: dkv.dkv_attn_decode_q4_0(cfg, q4s[i % reps], None, q, lens, out, ws), steps, stream)
    res["q4_0"] = {"ms_per_step": round(ms, 5), "GBps": round((q4_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                   "hbm_frac": round((q4_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "bytes": q4_bytes, "replicas": reps}
    del q4s
    return res, q4


def strided_bytes(w, stride, lens_np):
    """Algorithmic bytes of one strided-reference decode launch: per stream and
    token the Q4_0 residual (D/2 code bytes, D/16 scale bytes) and a 2-byte
    reference index, plus every reference row (2*D bytes) once."""
    D = w.D
    per_tok = D // 2 + 2 * (D // 32) + 2
    total = 0
    for L in lens_np:
        L = int(L)
        total += L * per_tok + -(-L // stride) * 2 * D
    return 2 * w.Hkv * total


def strided_recon(cfg, cache, S):
    """Dequantise a strided-reference cache from its planes on the GPU:
    float [B][Hkv][2][S][D] = reference row + (code - 8) * scale."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    B, H, D = cfg.batch, cfg.n_kv_heads, cfg.head_dim
    lay = dkv.dkv_strided_layout(cfg)
    c = cache.view(B, H, 2, lay["stream_bytes"])
    nref = lay["nref"]
    refs = c[..., :nref * D * 2].contiguous().view(torch.float16).view(B, H, 2, nref, D).float()
    codes = c[..., lay["codes"]:lay["codes"] + S * D // 2].reshape(B, H, 2, S, D // 32, 16)
    full = torch.cat([codes & 15, codes >> 4], dim=-1).float() - 8.0
    sc = c[..., lay["scales"]:lay["scales"] + S * D // 16].contiguous().view(torch.float16)
    sc = sc.view(B, H, 2, S, D // 32, 1).float()
    idx = c[..., lay["idx"]:lay["idx"] + 2 * S].contiguous().view(torch.int16).view(B, H, 2, S).long() & 0xFFFF
    rr = torch.gather(refs, 3, idx.clamp(max=nref - 1)[..., None].expand(-1, -1, -1, -1, D))
    return rr + (full * sc).reshape(B, H, 2, S, D)


def strided_mixed_quality(dev, B=8, S=8192):
    """Reconstruction MSE of Delta-KV and of strided references (stride 32 with
    a window of 64 references, stride 8 with 256) on the mixed workload's two
    halves: periodic rows (period 8..64) and regime-switching rows.  Delta-KV
    via dkv_reconstruct; strided dequantised from its planes."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    from quantized_decode_attention_delta_amd import synth
    w = synth.make("mixed", B=B, S=S, extra_tokens=0)
    H, D = w.Hkv, w.D
    k = torch.from_numpy(w.k).to(dev)
    v = torch.from_numpy(w.v).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    x = torch.stack([k, v], dim=2).float()                       # [B][H][2][S][D]
    valid = (torch.arange(S, device=dev)[None, :] < lens[:, None].long())[:, None, None, :, None]
    halves = {"periodic": slice(0, B // 2), "regime": slice(B // 2, B)}

    def mse(rec):
        err = ((rec - x) ** 2) * valid
        return {n: float(err[sl].sum()) / (float(valid[sl].sum()) * H * 2 * D) for n, sl in halves.items()}

    out = {"how": f"mixed workload, {B} sequences (first half periodic, second regime-switching), "
                  f"lengths up to {S}, contiguous caches"}
    cfg = dkv.Config(batch=B, n_q_heads=w.Hq, n_kv_heads=H, head_dim=D, kf=32, max_tokens=S)
    cache = torch.empty(dkv.dkv_cache_bytes(cfg), dtype=torch.uint8, device=dev)
    state = torch.zeros(B, H, 2, D, dtype=torch.float32, device=dev)
    dkv.dkv_encode_prefill(cfg, cache, state, None, k, v, lens, S)
    kr = torch.zeros(B, H, S, D, dtype=torch.float32, device=dev)
    vr = torch.zeros_like(kr)
    dkv.dkv_reconstruct(cfg, cache, None, lens, S, kr, vr)
    out["delta_kv_kf32"] = mse(torch.stack([kr, vr], dim=2))
    del cache, kr, vr
    for stride, window in ((32, 64), (8, 256)):
        cs = dkv.Config(batch=B, n_q_heads=w.Hq, n_kv_heads=H, head_dim=D, kf=stride, max_tokens=S)
        sc = torch.zeros(dkv.dkv_strided_cache_bytes(cs), dtype=torch.uint8, device=dev)
        dkv.dkv_strided_encode_prefill(cs, sc, k, v, lens, S, window)
        out[f"strided_{stride}_w{window}"] = mse(strided_recon(cs, sc, S))
        del sc
    return out


def strided(w, k, v, q, lens, steps, stream, qo, window=64):
    """Strided-reference residual cache (references every kf tokens, nearest
    within the last `window` references) on the same K/V and queries: encode
    time, decode time against its algorithmic bytes, and the quality of its
    reconstruction, dequantised here from its own planes on the GPU."""
    import numpy as np
    import torch

    import quantized_decode_attention_delta_amd as dkv
    dev = k.device
    B, H, S, D, stride = w.B, w.Hkv, w.S, w.D, w.kf
    cfg = dkv.Config(batch=B, n_q_heads=w.Hq, n_kv_heads=H, head_dim=D, kf=stride, max_tokens=S)
    nbytes = dkv.dkv_strided_cache_bytes(cfg)
    cache = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dkv.dkv_strided_encode_prefill(cfg, cache, k, v, lens, S, window)
    torch.cuda.synchronize()
    enc_ms = (time.perf_counter() - t0) * 1e3
    reps = max(1, math.ceil((1 << 30) / nbytes))
    caches = [cache] + [cache.clone() for _ in range(reps - 1)]
    out = torch.empty(B, w.Hq, D, dtype=torch.float32, device=dev)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    ms = _time(lambda i: dkv.dkv_strided_attn_decode(cfg, caches[i % reps], q, lens, out, ws), steps, stream)
    del caches
    alg = strided_bytes(w, stride, lens.cpu().numpy())
    res = {"ms_per_step": round(ms, 5), "GBps": round((alg + qo) / (ms * 1e-3) / 1e9, 2),
           "hbm_frac": round((alg + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "bytes": alg,
           "stride": stride, "window": window, "encode_ms": round(enc_ms, 1), "replicas": reps,
           "how": "dkv_strided_attn_decode (split phase + combine)"}

    recon = strided_recon(cfg, cache, S)
    valid = (torch.arange(S, device=dev)[None, :] < lens[:, None].long())[:, None, :, None]
    nval = float(valid.sum()) * H * D
    mse = [float((((recon[:, :, s] - x.float()) ** 2) * valid).sum()) / nval for s, x in enumerate((k, v))]
    kh = recon[:, :, 0].contiguous()
    vh = recon[:, :, 1].contiguous()
    del recon
    logits = torch.empty(B * w.Hq * S, dtype=torch.float32, device=dev)
    dk = torch.empty(B, w.Hq, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    dkv.dkv_attn_distortion(cfg, kh, vh, k, v, S, q, lens, dk, dv, logits)
    qual = {"mse": sum(mse) / 2, "mse_kv": mse, "d_k": float(dk.double().mean()), "d_v": float(dv.double().mean())}
    return res, qual


def quality(w, cfg, cache, q4, k, v, lens, q):
    """Reconstruction MSE against the fp16 input, over every valid token, from
    the GPU's own outputs: Delta-KV via dkv_reconstruct, Q4_0 via its export,
    Q8_0 (the 8-bit reference, quality only) via dkv_q8_0_encode.
    Next to it the attention-preserving distortion of the same reconstructions
    (dkv_attn_distortion): the mean over (sequence, query head) of
    d_k = ||q.Khat^T - q.K^T||^2 and d_v = ||a.Vhat - a.V||^2 for this step's
    queries."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    dev = k.device
    B, H, S, D = w.B, w.Hkv, w.S, w.D
    valid = (torch.arange(S, device=dev)[None, :] < lens[:, None].long())[:, None, :, None]
    nval = float(valid.sum()) * H * D
    kr = torch.empty(B, H, S, D, dtype=torch.float32, device=dev)
    vr = torch.empty_like(kr)
    dkv.dkv_reconstruct(cfg, cache, None, lens, S, kr, vr)
    mse_d = [float((((kr - k.float()) ** 2) * valid).sum()) / nval,
             float((((vr - v.float()) ** 2) * valid).sum()) / nval]
    logits = torch.empty(B * w.Hq * S, dtype=torch.float32, device=dev)
    dk = torch.empty(B, w.Hq, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)

    def distortion(kh, vh):
        dkv.dkv_attn_distortion(cfg, kh, vh, k, v, S, q, lens, dk, dv, logits)
        return float(dk.double().mean()), float(dv.double().mean())

    dist_d = distortion(kr, vr)
    del kr, vr
    codes = torch.empty(B, H, 2, S, D // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(B, H, 2, S, D // 32, dtype=torch.int16, device=dev)
    dkv.dkv_q4_0_export(cfg, q4, None, lens, S, codes, scales)
    mse_q, deqs = [], []
    for s, x in enumerate((k, v)):
        c = codes[:, :, s].reshape(B, H, S, D // 32, 16)
        full = torch.cat([(c & 15), (c >> 4)], dim=-1).float() - 8.0
        sc = scales[:, :, s].view(torch.float16).float()[..., None]
        deq = (full * sc).reshape(B, H, S, D).contiguous()
        mse_q.append(float((((deq - x.float()) ** 2) * valid).sum()) / nval)
        deqs.append(deq)
        del c, full
    dist_q = distortion(deqs[0], deqs[1])
    del deqs, codes, scales
    # Q8_0 of the absolute rows (quality comparison only)
    c8 = torch.empty(B, H, 2, S, D, dtype=torch.int8, device=dev)
    s8 = torch.empty(B, H, 2, S, D // 32, dtype=torch.int16, device=dev)
    dkv.dkv_q8_0_encode(cfg, k, v, lens, S, c8, s8)
    mse_8, deq8 = [], []
    for s, x in enumerate((k, v)):
        sc = s8[:, :, s].view(torch.float16).float()[..., None]
        deq = (c8[:, :, s].reshape(B, H, S, D // 32, 32).float() * sc).reshape(B, H, S, D).contiguous()
        mse_8.append(float((((deq - x.float()) ** 2) * valid).sum()) / nval)
        deq8.append(deq)
    dist_8 = distortion(deq8[0], deq8[1])
    del deq8, c8, s8
    md, mq = sum(mse_d) / 2, sum(mse_q) / 2
    return {"mse_delta_kv": md, "mse_q4_0": mq, "ratio_q4_0_over_delta_kv": round(mq / md, 2) if md > 0 else None,
            "mse_delta_kv_kv": mse_d, "mse_q4_0_kv": mse_q,
            "mse_q8_0": sum(mse_8) / 2, "mse_q8_0_kv": mse_8,
            "attention_distortion": {
                "d_k_delta_kv": dist_d[0], "d_v_delta_kv": dist_d[1],
                "d_k_q4_0": dist_q[0], "d_v_q4_0": dist_q[1],
                "d_k_q8_0": dist_8[0], "d_v_q8_0": dist_8[1],
                "ratio_d_k_q4_0_over_delta_kv": round(dist_q[0] / dist_d[0], 2) if dist_d[0] > 0 else None,
                "ratio_d_v_q4_0_over_delta_kv": round(dist_q[1] / dist_d[1], 2) if dist_d[1] > 0 else None,
                "how": "mean over (sequence, query head) of ||q.Khat^T - q.K^T||^2 and ||a.Vhat - a.V||^2, "
                       "a = softmax on the exact keys, this step's queries (dkv_attn_distortion)"}}


def run_mixed(args):
    """Serving loop of the mixed workload: paged cache (256-token pages, shuffled
    physical ids), bulk prefill, then per step one appended token per sequence
    followed by decode attention over the grown cache.  A step = append + decode
    of one layer in one call (dkv_append_attn_decode: the append runs inside the
    decode's split launch); the timed steps follow the warm-up steps.  The same
    steps through separate dkv_append + dkv_attn_decode calls, on a copy of the
    prefilled cache, are timed next to it and must leave identical bytes."""
    import numpy as np
    import torch

    import quantized_decode_attention_delta_amd as dkv
    from quantized_decode_attention_delta_amd import synth

    dev = torch.device("cuda:0")
    over = {}
    if args.mixed_batch:
        over["B"] = args.mixed_batch
    if args.mixed_max_len:
        over["S"] = args.mixed_max_len
    t_gen = time.time()

    def progress(b):
        if b % 8 == 7:
            print(f"# generated {b + 1} sequences ({time.time() - t_gen:.0f} s)", file=sys.stderr, flush=True)

    w = synth.make("mixed", progress=progress, **over)
    nsteps = w.extra_tokens
    if args.warmup + args.steps > nsteps:
        sys.exit(f"bench.py: mixed workload has {nsteps} append+decode steps; warmup + steps must not exceed it")
    print(f"# workload mixed: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} L in [{int(w.seq_lens.min())}, "
          f"{int(w.seq_lens.max())}] pages {w.page_tokens} kf={w.kf} (generated in {time.time() - t_gen:.1f} s)",
          file=sys.stderr, flush=True)
    table, n_pages = synth.page_table(w)
    cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=w.kf,
                     page_tokens=w.page_tokens, n_pages=n_pages, max_pages_per_seq=table.shape[1])
    lens0 = w.seq_lens.astype(np.int32)
    # the appended tokens of every step: [step][B][Hkv][D]
    kn = np.empty((nsteps, w.B, w.Hkv, w.D), np.float16)
    vn = np.empty_like(kn)
    for b in range(w.B):
        sl = slice(int(lens0[b]), int(lens0[b]) + nsteps)
        kn[:, b] = w.k[b, :, sl].transpose(1, 0, 2)
        vn[:, b] = w.v[b, :, sl].transpose(1, 0, 2)
    cache = torch.empty(dkv.dkv_cache_bytes(cfg), dtype=torch.uint8, device=dev)
    state = torch.zeros(w.B, w.Hkv, 2, w.D, dtype=torch.float32, device=dev)
    bt = torch.from_numpy(table).to(dev)
    lens = torch.from_numpy(lens0).to(dev)
    k = torch.from_numpy(w.k).to(dev)
    v = torch.from_numpy(w.v).to(dev)
    dkv.dkv_encode_prefill(cfg, cache, state, bt, k, v, lens, w.k.shape[2])
    torch.cuda.synchronize()
    del k, v
    cache_b, state_b = cache.clone(), state.clone()
    w.k = w.v = None
    kn_t = torch.from_numpy(kn).to(dev)
    vn_t = torch.from_numpy(vn).to(dev)
    pos = torch.from_numpy(lens0[None, :] + np.arange(nsteps, dtype=np.int32)[:, None]).to(dev)   # [step][B]
    lens_after = pos + 1
    q = torch.from_numpy(np.stack([synth.queries(w, s) for s in range(nsteps)])).to(dev)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    out_b = torch.empty_like(out)

    def step(s):
        dkv.dkv_append_attn_decode(cfg, cache, state, bt, kn_t[s], vn_t[s], pos[s], q[s], lens_after[s], out, ws)

    def step_unfused(s):
        dkv.dkv_append(cfg, cache_b, state_b, bt, kn_t[s], vn_t[s], pos[s])
        dkv.dkv_attn_decode(cfg, cache_b, bt, q[s], lens_after[s], out_b, ws)

    # clocks settle on decode-only calls over the prefilled cache (appends would
    # advance the workload)
    spin_up(lambda: dkv.dkv_attn_decode(cfg, cache, bt, q[0], lens, out, ws), args.spin_up_ms)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for s in range(args.warmup, args.warmup + args.steps):
        step(s)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # the same steps as separate append and decode calls, on the copy
    for s in range(args.warmup):
        step_unfused(s)
    torch.cuda.synchronize()
    ev0.record(stream)
    for s in range(args.warmup, args.warmup + args.steps):
        step_unfused(s)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_unfused = ev0.elapsed_time(ev1) / args.steps
    same = bool(torch.equal(cache, cache_b) and torch.equal(state, state_b) and torch.equal(out, out_b))
    del cache_b, state_b

    # the decode kernel alone on the final cache (launches back to back between
    # two events on the kernel's stream: the mean launch duration), and the append alone
    last = args.warmup + args.steps - 1
    n_k = max(10, args.steps)
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(n_k):
        dkv.dkv_attn_decode_partial(cfg, cache, bt, q[last], lens_after[last], ws)
    k1.record(stream)
    torch.cuda.synchronize()
    kern_ms = k0.elapsed_time(k1) / n_k

    Lf = lens0 + last + 1                                    # lengths during the last timed decode
    Lt = [lens0 + s + 1 for s in range(args.warmup, args.warmup + args.steps)]
    comp_last = sum(algorithmic_bytes(1, w.Hkv, w.Hq, w.D, int(L), w.kf) for L in Lf)
    comp_avg = float(np.mean([sum(algorithmic_bytes(1, w.Hkv, w.Hq, w.D, int(L), w.kf) for L in x) for x in Lt]))
    eff_avg = float(np.mean([int(x.sum()) * w.Hkv * w.D * 2 * 2 for x in Lt]))
    qo = w.B * w.Hq * w.D * 4 * 2
    achieved = (comp_last + qo) / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(eff_avg / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"mixed: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} L~U[{int(w.seq_lens.min())}..] "
                        f"max {w.S}, {w.page_tokens}-token pages (shuffled), kf={w.kf}, step = append + decode",
            "kernel": "fused",
        },
        "layer_steps_per_s": round(1000.0 / ms_step, 2),
        "unfused": {"ms_per_step": round(ms_unfused, 5), "layer_steps_per_s": round(1000.0 / ms_unfused, 2),
                    "how": "dkv_append then dkv_attn_decode (3 launches per step) on a copy of the cache",
                    "identical_cache_state_output": same},
        "compressed_GBps": round((comp_avg + qo) / (ms_step * 1e-3) / 1e9, 2),
        "hbm_frac_step": round((comp_avg + qo) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": None,
            "kernel_ms": round(kern_ms, 5),
            "algorithmic_bytes": comp_last + qo,
        },
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_decode_attention_delta_amd as dkv
    from quantized_decode_attention_delta_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.workload == "mixed":
        return run_mixed(args)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    over = {} if args.kf is None else {"kf": args.kf}
    t_gen = time.time()
    w = synth.make(args.workload, **over)
    kf = w.kf
    print(f"# workload {args.workload}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.S} kf={kf} "
          f"(generated in {time.time() - t_gen:.1f} s)", file=sys.stderr, flush=True)

    cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=kf, max_tokens=w.S)
    cache_bytes = dkv.dkv_cache_bytes(cfg)
    replicas = args.replicas or max(1, math.ceil((1 << 30) / cache_bytes))
    lens = torch.from_numpy(w.seq_lens).to(dev)
    state = torch.zeros(w.B, w.Hkv, 2, w.D, dtype=torch.float32, device=dev)
    k = torch.from_numpy(w.k).to(dev)
    v = torch.from_numpy(w.v).to(dev)
    cache0 = torch.empty(cache_bytes, dtype=torch.uint8, device=dev)
    dkv.dkv_encode_prefill(cfg, cache0, state, None, k, v, lens, w.S)
    caches = [cache0] + [cache0.clone() for _ in range(replicas - 1)]
    torch.cuda.synchronize()
    q = torch.from_numpy(synth.queries(w)).to(dev)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    step_fn = dkv.dkv_attn_decode if args.kernel == "fused" else dkv.dkv_attn_decode_ref

    def step(i):
        step_fn(cfg, caches[i % replicas], None, q, lens, out, ws)

    spin_up(lambda: step(0), args.spin_up_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # dominant kernel alone: the split phase, launched back to back between two
    # events on its stream (the mean launch duration)
    n_k = max(10, args.steps)
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    h0 = time.perf_counter()
    for i in range(n_k):
        if args.kernel == "fused":
            dkv.dkv_attn_decode_partial(cfg, caches[i % replicas], None, q, lens, ws)
        else:
            dkv.dkv_attn_decode_ref(cfg, caches[i % replicas], None, q, lens, out, ws)
    host_ms = (time.perf_counter() - h0) * 1e3 / n_k      # host time to issue one launch
    k1.record(stream)
    torch.cuda.synchronize()
    kern_ms = k0.elapsed_time(k1) / n_k

    comp = algorithmic_bytes(w.B, w.Hkv, w.Hq, w.D, w.S, kf)
    qo = w.B * w.Hq * w.D * 4 * 2
    eff = f16_equiv_bytes(w.B, w.Hkv, w.D, w.S)
    achieved = (comp + qo) / (kern_ms * 1e-3) / 1e9

    # streaming-read ceiling: the library's plain read of the same cache replicas
    sink = torch.empty(dkv.dkv_stream_read_sink_words(), dtype=torch.int32, device=dev)
    sr_ms = _time(lambda i: dkv.dkv_stream_read(caches[i % replicas], sink), n_k, stream)
    sr_gbps = cache_bytes / (sr_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(eff / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.S} kf={kf}",
            "kernel": args.kernel,
            "cache_replicas": replicas,
        },
        "layer_steps_per_s": round(1000.0 / ms_step, 2),
        "compressed_GBps": round((comp + qo) / (ms_step * 1e-3) / 1e9, 2),
        "hbm_frac_step": round((comp + qo) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(args.workload, kf, args.kernel),
            "kernel_ms": round(kern_ms, 5),
            "host_issue_ms": round(host_ms, 5),
            "frac_of_stream_read": round(achieved / sr_gbps, 4),
            "algorithmic_bytes": comp + qo,
        },
        "stream_read_ceiling": {"GBps": round(sr_gbps, 1), "frac_of_peak": round(sr_gbps / HBM_PEAK_GBPS, 4),
                                "bytes": cache_bytes, "how": "dkv_stream_read over the same cache replicas"},
    }
    layers = args.graph_layers if args.graph_layers is not None else (32 if args.workload in ("tiny", "8b") else 0)
    if layers > 0:
        res["graph_layers"] = graph_layers(cfg, caches, q, lens, layers, stream)
    if not args.no_compare:
        res["comparisons"], q4 = comparisons(w, cfg, k, v, q, lens, ws, args.steps, stream, qo)
        res["comparisons"]["delta_kv"] = {"ms_per_step": res["ms_per_step"], "GBps": res["compressed_GBps"],
                                          "hbm_frac": res["hbm_frac_step"], "bytes": comp}
        res["quality"] = quality(w, cfg, cache0, q4, k, v, lens, q)
        del q4
        if w.S <= 65536 * w.kf:
            res["comparisons"]["strided"], res["quality"]["strided"] = strided(w, k, v, q, lens, args.steps, stream,
                                                                              qo)
        res["quality"]["strided_vs_delta_kv_mixed"] = strided_mixed_quality(dev)
    if not args.no_cpu_baseline:
        threads = args.cpu_threads or min(16, os.cpu_count() or 1)
        res["cpu_baseline"] = cpu_baseline(w, kf, args.cpu_seconds, threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
