#!/usr/bin/env python3
"""Delta-KV fused decode attention benchmark (one MI355X).  Prints ONE JSON line.

Default run (no flags): the mixed serving batch is the headline workload:
64 sequences of 1K..64K tokens (32 q / 8 kv heads, D = 128) in shuffled
256-token pages, kf = 32, bulk prefill, then append + decode steps; one step
is the append of every sequence's new token and decode attention of every
query head over the grown cache of one layer (one dkv_append_attn_decode
call).  The smaller configurations (tiny, the 8B-shaped layer, the long
context at kf 32 / 128 / 512, the 70B-shaped layer) follow under `configs`,
each a decode layer-step (dkv_attn_decode) with its own roofline.
Inputs are synthetic, seeded, and resident in HBM before any timed region.

Reported (headline and per configuration):
  value        effective KV GB/s = fp16-equivalent K/V bytes the step attends
               over / step time
  roofline     the dominant kernel (the decode's split-phase kernel):
               algorithmic compressed bytes + q + out per launch / its mean
               duration from HIP events on the launch stream, vs 8 TB/s;
               `traffic` = HBM bytes per launch from rocprofv3 counters
  comparisons  in-run F16 and plain-Q4_0 decode attentions on the same data
  quality      reconstruction MSE of Delta-KV, Q4_0 and Q8_0 against the
               fp16 input and the attention-preserving distortions D_K, D_V
  cpu_baseline (headline) the CPU oracle on a bounded sample of the same
               workload: encode and attention timed apart, one thread and all
               of the host's cores
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "Delta-KV decode attn: effective KV GB/s (% HBM peak) + layer-steps/s"
ATTN_TOL = 2e-3
STATIC_CONFIGS = ("tiny", "8b", "long_kf32", "long_kf128", "long_kf512", "70b")

# HBM bytes (read + written) per launch of the split-phase kernel, from
# rocprofv3 FETCH_SIZE (x2.0) and WRITE_SIZE (x1.0) counters, each scaled by
# what the counter reads for a 1 GiB device copy.  Valid only for the kernel
# and split-plan sources they were measured on (sha256 below); otherwise
# traffic is null.
MEASURED_TRAFFIC = {
    "sources": {
        "dkv_attn_g8.hip": "1ed41445bf553025e7fbd3c0875cb7f4dfd005d9fa3d61902873c88975909983",
        "dkv_fused_common.h": "c525d3bb9543ef7d48530cee671bc61a92708fc21a4bfb3bf73b9f44f9e1b74e",
        "dkv_common.h": "57ec119a4bc9a80095dbe7da0e961e0c7a888ad6910487f1210451a0fa2dcbb9",
        "dkv_append.h": "be07c04e9857cdcd9f08e6a2526b04f9ce5e0a510bffa70e7ff091ce2d00e7dc",
        "dkv_q40.h": "d4b0a8142dfd210e9daa6a9ef282fe5ccb37c516b007f54681f8c9f93af0c73c",
        "dkv_api.cpp": "1f8eb005424fc0cd5858724d486d1af0683d7a8cfbac4a05bed2ff6a7318c0f6",
    },
    "per_launch": {"mixed": 3161446633, "70b": 684889606, "long_kf512": 158607177, "long_kf128": 161538652},
}


def measured_traffic(key):
    t = MEASURED_TRAFFIC
    if key not in t["per_launch"]:
        return None
    src = os.path.join(ROOT, "quantized_decode_attention_delta_amd", "csrc")
    for name, digest in t["sources"].items():
        with open(os.path.join(src, name), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != digest:
                return None
    return t["per_launch"][key]


def algorithmic_bytes(B, Hkv, Hq, D, S, kf):
    """Compressed bytes one decode layer-step must read: per stream
    2*D*ceil(S/kf) keyframe bytes + 18*(D/32) bytes per delta token."""
    ng = -(-S // kf)
    per_stream = 2 * D * ng + 18 * (D // 32) * (S - ng)
    return 2 * B * Hkv * per_stream


def f16_equiv_bytes(B, Hkv, D, S):
    return 2 * Hkv * D * S * B * 2


def q4_0_bytes(Hkv, D, lens):
    """Plain Q4_0 cache bytes attended: 18 bytes per 32 elements, K and V."""
    return 2 * Hkv * (D // 32) * 18 * int(sum(int(L) for L in lens))


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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=120)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="all", choices=["all", "tiny", "8b", "long", "70b", "mixed"],
                    help="all (default): the mixed serving batch as the headline, the other configurations "
                         "under `configs`; otherwise that one workload alone")
    ap.add_argument("--configs", default=",".join(STATIC_CONFIGS),
                    help="with --workload all: which configurations to add under `configs`")
    ap.add_argument("--mixed-batch", type=int, default=None, help="mixed workload: fewer sequences (default 64)")
    ap.add_argument("--mixed-max-len", type=int, default=None, help="mixed workload: shorter maximum length")
    ap.add_argument("--kf", type=int, default=None, help="single static workload: keyframe interval")
    ap.add_argument("--kernel", default="fused", choices=["fused", "ref"])
    ap.add_argument("--replicas", type=int, default=0, help="cache copies rotated per step (0 = auto, >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0, help="oracle time budget (four equal parts)")
    ap.add_argument("--cpu-threads", type=int, default=0, help="oracle threads for the all-cores part "
                                                               "(0 = min(16, host cores))")
    ap.add_argument("--spin-up-ms", type=float, default=300.0,
                    help="run the decode kernels this long before the warmup steps (GPU clocks settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-compare", action="store_true", help="skip the F16 / Q4_0 comparisons and the quality report")
    ap.add_argument("--graph-layers", type=int, default=None,
                    help="decode steps of this many layers captured in one HIP graph and replayed "
                         "(default 32 for the launch-bound tiny and 8b workloads, 0 otherwise)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy a 1 GiB device buffer 3 times (a plain copy kernel of known size, "
                         "to scale the FETCH_SIZE / WRITE_SIZE counters of a profiled run)")
    return ap.parse_args()


def host_threads(args):
    return args.cpu_threads or min(16, os.cpu_count() or 1)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def log(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


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


def _time(fn, n, stream, settle_ms=100.0):
    """Mean ms per call of fn(i), i = 0..n-1, from HIP events on `stream`
    (after `settle_ms` of calls for the clocks to settle, and 3 warmup calls)."""
    import torch
    spin_up(lambda: fn(0), settle_ms)
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


def rel_err_rows(got, ref):
    """Max over output rows of max |got - ref| / max |ref| (rows of zeros: abs)."""
    import torch
    g = got.double().reshape(-1, got.shape[-1])
    r = ref.double().reshape(-1, ref.shape[-1])
    den = r.abs().amax(-1).clamp_min(1e-300)
    den = torch.where(r.abs().amax(-1) > 0, den, torch.ones_like(den))
    return float(((g - r).abs().amax(-1) / den).max()) if g.numel() else 0.0


def roofline(alg_bytes, kern_ms, traffic, kernel, sr_gbps=None):
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
         "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
         "kernel_ms": round(kern_ms, 5), "algorithmic_bytes": alg_bytes}
    if traffic is not None:
        r["traffic_over_algorithmic"] = round(traffic / alg_bytes, 4)
    if sr_gbps:
        r["frac_of_stream_read"] = round(achieved / sr_gbps, 4)
    return r


def gen_workload(name, args, **over):
    from quantized_decode_attention_delta_amd import synth
    t0 = time.time()
    progress = None
    if name == "mixed":
        def progress(n):
            if n % 16 == 0:
                log(f"generated {n} sequences ({time.time() - t0:.0f} s)")
    w = synth.make(name, progress=progress, workers=host_threads(args), **over)
    log(f"workload {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.S} (generated in {time.time() - t0:.1f} s)")
    return w


# ------------------------------------------------------------------ CPU oracle
def cpu_baseline(w, kf, lens, q, gpu_out, budget_s, threads):
    """The oracle as it stands, on the host's cores, over a bounded sample of
    whole (sequence, kv-head) pairs of the workload in a seeded order:
      encode    closed-loop encode of the pair's K and V (tokens [0, lens[b]));
      attention reconstruction of K and V from that encoding + float64
                attention of the pair's G query heads.
    Each part runs on one thread, then on `threads` threads (the oracle's C
    routines release the GIL), for about budget_s / 4 each.  The attention
    outputs are also compared with the GPU's output of the same step."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    G = w.Hq // w.Hkv
    scale = np.float32(1 / math.sqrt(w.D))
    order = np.random.default_rng(12345).permutation(w.B * w.Hkv)
    pairs = [(int(p) // w.Hkv, int(p) % w.Hkv) for p in order]
    part = budget_s / 4.0
    enc = {}
    errs = []

    def encode(bh):
        b, h = bh
        L = int(lens[b])
        enc[bh] = (oracle.encode_stream(np.ascontiguousarray(w.k[b, h, :L]), kf, want_recon=False),
                   oracle.encode_stream(np.ascontiguousarray(w.v[b, h, :L]), kf, want_recon=False))

    def attend(bh):
        b, h = bh
        L = int(lens[b])
        ek, ev = enc[bh]
        kr = oracle.reconstruct_stream(ek.kf_rows, ek.codes, ek.scales, L, w.D, kf)
        vr = oracle.reconstruct_stream(ev.kf_rows, ev.codes, ev.scales, L, w.D, kf)
        return bh, oracle.attention_f64(q[b, h * G:(h + 1) * G], kr, vr, scale)

    def check(bh, o):
        b, h = bh
        g = gpu_out[b, h * G:(h + 1) * G].astype(np.float64)
        den = np.abs(o).max(-1)
        den = np.where(den > 0, den, 1.0)
        errs.append(float((np.abs(g - o).max(-1) / den).max()))

    def eff(bh):
        return 2 * int(lens[bh[0]]) * w.D * 2

    def comp(bh):
        return algorithmic_bytes(1, 1, G, w.D, int(lens[bh[0]]), kf)

    def run_part(fn, work, nthreads, ex, repeat):
        """Run fn over `work` in chunks of nthreads until `part` seconds (cycling
        through `work` again when repeat); returns ([(item, result)], seconds)."""
        done, t, i = [], 0.0, 0
        while t < part and (repeat or i < len(work)):
            chunk = [work[(i + j) % len(work)] for j in range(nthreads)] if repeat else work[i:i + nthreads]
            t0 = time.perf_counter()
            res = list(ex.map(fn, chunk)) if ex else [fn(x) for x in chunk]
            t += time.perf_counter() - t0
            done += list(zip(chunk, res))
            i += len(chunk)
        return done, t

    out = {}
    with cf.ThreadPoolExecutor(threads) as ex:
        # encode: pairs in order (whole passes again once every pair is done)
        e1, t_e1 = run_part(encode, pairs, 1, None, True)
        mine = list(dict.fromkeys(bh for bh, _ in e1))
        rest = [bh for bh in pairs if bh not in enc]
        eT, t_eT = run_part(encode, rest or pairs, threads, ex, True)
        # attention over the encoded pairs
        a1, t_a1 = run_part(attend, mine, 1, None, True)
        aT, t_aT = run_part(attend, list(dict.fromkeys([bh for bh, _ in eT] + mine)), threads, ex, True)
    seen = set()
    for _, (bh, o) in a1 + aT:
        if bh not in seen:
            seen.add(bh)
            check(bh, o)
    total_eff = sum(2 * int(L) * w.D * 2 * w.Hkv for L in lens[:w.B])

    def rates(done, t):
        e = sum(eff(bh) for bh, _ in done)
        c = sum(comp(bh) for bh, _ in done)
        return {"GBps_effective": round(e / t / 1e9, 4), "GBps_compressed": round(c / t / 1e9, 4),
                "layer_steps_per_s": round(e / t / total_eff, 6), "pair_decodes": len(done),
                "seconds": round(t, 2)}

    def enc_rates(done, t):
        toks = sum(2 * int(lens[bh[0]]) for bh, _ in done)
        return {"tokens_per_s": round(toks / t, 1), "GBps_fp16_in": round(toks * w.D * 2 / t / 1e9, 4),
                "pairs": len(done), "seconds": round(t, 2)}

    out["attention"] = {"single_thread": rates(a1, t_a1), "all_cores": rates(aT, t_aT)}
    out["encode"] = {"single_thread": enc_rates(e1, t_e1), "all_cores": enc_rates(eT, t_eT)}
    res = {
        "value": out["attention"]["all_cores"]["GBps_effective"],
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"whole (sequence, kv-head) pairs of the same workload and step in a seeded order: encode "
                  f"(closed-loop, K and V) and attention (reconstruction + float64 attention of the {G} query "
                  f"heads) timed apart, each about {part:.0f} s on 1 thread and on {threads} threads; value = "
                  f"all-cores attention in the headline's unit (fp16-equivalent K/V bytes attended per second)",
        "host": {"nproc": os.cpu_count(), "cpu_model": cpu_model(), "threads_all_cores": threads},
        **out,
        "gpu_check": {"pairs": len(seen), "rows": len(seen) * G, "max_rel_err": max(errs) if errs else None,
                      "tol": ATTN_TOL,
                      "how": "the GPU's output of the same step against the oracle's float64 attention, "
                             "per output row max|gpu - oracle| / max|oracle|"},
    }
    return res


# ------------------------------------------------------------ quality report
def quality_sums(cfg, cache, q4, bt, k, v, lens, q, s_max, q4k=None, cfg_q4k=None):
    """Squared errors against the fp16 input over every valid token, and sums of
    the attention-preserving distortions over (sequence, query head), from the
    GPU's own outputs: Delta-KV via dkv_reconstruct, Q4_0 via dkv_q4_0_export,
    Q8_0 (the 8-bit reference, quality only) via dkv_q8_0_encode; the
    distortions d_k = ||q.Khat^T - q.K^T||^2 and d_v = ||a.Vhat - a.V||^2
    (a = softmax on the exact keys) via dkv_attn_distortion."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    dev = k.device
    B, H, D, S = cfg.batch, cfg.n_kv_heads, cfg.head_dim, s_max
    valid = (torch.arange(S, device=dev)[None, :] < lens[:, None].long())[:, None, :, None]
    res = {"n": float(valid.sum()) * H * D, "rows": B * cfg.n_q_heads}
    logits = torch.empty(B * cfg.n_q_heads * S, dtype=torch.float32, device=dev)
    dk = torch.empty(B, cfg.n_q_heads, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)

    def distortion(kh, vh):
        dkv.dkv_attn_distortion(cfg, kh, vh, k, v, S, q, lens, dk, dv, logits)
        return float(dk.double().sum()), float(dv.double().sum())

    def sse(rec, x):
        # rows past a sequence's length are not written by the exports: select, not multiply
        return float(torch.where(valid, (rec - x.float()) ** 2, 0.0).sum())

    kr = torch.empty(B, H, S, D, dtype=torch.float32, device=dev)
    vr = torch.empty_like(kr)
    dkv.dkv_reconstruct(cfg, cache, bt, lens, S, kr, vr)
    res["delta_kv"] = [sse(kr, k), sse(vr, v)]
    res["dist_delta_kv"] = distortion(kr, vr)
    del kr, vr
    codes = torch.empty(B, H, 2, S, D // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(B, H, 2, S, D // 32, dtype=torch.int16, device=dev)
    dkv.dkv_q4_0_export(cfg, q4, bt, lens, S, codes, scales)
    deqs = []
    for s in range(2):
        c = codes[:, :, s].reshape(B, H, S, D // 32, 16)
        full = torch.cat([(c & 15), (c >> 4)], dim=-1).float() - 8.0
        sc = scales[:, :, s].view(torch.float16).float()[..., None]
        deqs.append((full * sc).reshape(B, H, S, D).contiguous())
        del c, full
    del codes, scales
    res["q4_0"] = [sse(deqs[0], k), sse(deqs[1], v)]
    res["dist_q4_0"] = distortion(deqs[0], deqs[1])
    del deqs
    c8 = torch.empty(B, H, 2, S, D, dtype=torch.int8, device=dev)
    s8 = torch.empty(B, H, 2, S, D // 32, dtype=torch.int16, device=dev)
    dkv.dkv_q8_0_encode(cfg, k, v, lens, S, c8, s8)
    deq8 = []
    for s in range(2):
        sc = s8[:, :, s].view(torch.float16).float()[..., None]
        deq8.append((c8[:, :, s].reshape(B, H, S, D // 32, 32).float() * sc).reshape(B, H, S, D).contiguous())
    del c8, s8
    res["q8_0"] = [sse(deq8[0], k), sse(deq8[1], v)]
    res["dist_q8_0"] = distortion(deq8[0], deq8[1])
    del deq8
    if q4k is not None:
        kr = torch.empty(B, H, S, D, dtype=torch.float32, device=dev)
        vr = torch.empty_like(kr)
        dkv.dkv_q4k_reconstruct(cfg_q4k, q4k, bt, lens, S, kr, vr)
        res["q4k"] = [sse(kr, k), sse(vr, v)]
        res["dist_q4k"] = distortion(kr, vr)
    return res


def quality_report(parts):
    n = sum(p["n"] for p in parts)
    rows = sum(p["rows"] for p in parts)

    def mse(key):
        return [sum(p[key][s] for p in parts) / n for s in range(2)]

    def dist(key):
        return [sum(p[key][s] for p in parts) / rows for s in range(2)]

    md, mq, m8 = mse("delta_kv"), mse("q4_0"), mse("q8_0")
    dd, dq, d8 = dist("dist_delta_kv"), dist("dist_q4_0"), dist("dist_q8_0")
    a, b = sum(md) / 2, sum(mq) / 2
    extra = {}
    if all("q4k" in p for p in parts):
        mk, dk_ = mse("q4k"), dist("dist_q4k")
        extra = {"mse_q4k_kf32": sum(mk) / 2, "mse_q4k_kf32_kv": mk,
                 "d_k_q4k_kf32": dk_[0], "d_v_q4k_kf32": dk_[1],
                 "q4k_how": "Q4-keyframe variant at kf 32: keyframes as Q4_0 of their absolute values, "
                            "4.5 bits per value like Q4_0 (dkv_q4k_reconstruct)"}
    return {**extra, "mse_delta_kv": a, "mse_q4_0": b, "ratio_q4_0_over_delta_kv": round(b / a, 2) if a > 0 else None,
            "mse_delta_kv_kv": md, "mse_q4_0_kv": mq, "mse_q8_0": sum(m8) / 2, "mse_q8_0_kv": m8,
            "attention_distortion": {
                "d_k_delta_kv": dd[0], "d_v_delta_kv": dd[1], "d_k_q4_0": dq[0], "d_v_q4_0": dq[1],
                "d_k_q8_0": d8[0], "d_v_q8_0": d8[1],
                "ratio_d_k_q4_0_over_delta_kv": round(dq[0] / dd[0], 2) if dd[0] > 0 else None,
                "ratio_d_v_q4_0_over_delta_kv": round(dq[1] / dd[1], 2) if dd[1] > 0 else None,
                "how": "mean over (sequence, query head) of ||q.Khat^T - q.K^T||^2 and ||a.Vhat - a.V||^2, "
                       "a = softmax on the exact keys, this step's queries (dkv_attn_distortion)"}}


# -------------------------------------------------------- strided references
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


# ------------------------------------------------------------ static layers
def graph_layers(cfg, caches, q, lens, layers, stream, replays=50):
    """A decoder's view of a launch-bound layer: the decode steps of `layers`
    layers (each its own copy of the cache) captured in one HIP graph (no host
    launch in between) and replayed; the replays are timed with HIP events on
    the replay stream."""
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
    n = dkv.dkv_attn_decode_launches(cfg)
    return {"layers": layers, "ms_per_layer_step": round(ms, 5), "layer_steps_per_s": round(1000.0 / ms, 2),
            "how": f"{layers} layers' decode steps ({n} kernel launch{'es' if n > 1 else ''} each, a cache copy "
                   f"per layer) in one HIP graph, {replays} replays timed with HIP events"}


def static_comparisons(w, cfg, k, v, q, lens, ws, steps, stream, qo, delta_out):
    """In-run F16 and plain-Q4_0 decode attention on the same K/V and queries
    (contiguous caches, rotated over >= 1 GiB of replicas)."""
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
    res["delta_kv_vs_f16_attention_max_rel_err"] = rel_err_rows(delta_out, out)
    f16_out = out.clone()
    del ks, vs
    q4_bytes = q4_0_bytes(w.Hkv, w.D, [w.S] * w.B)
    q4 = torch.empty(dkv.dkv_q4_0_cache_bytes(cfg), dtype=torch.uint8, device=k.device)
    dkv.dkv_q4_0_encode(cfg, q4, None, k, v, lens, w.S)
    reps = max(1, math.ceil((1 << 30) / q4.numel()))
    q4s = [q4] + [q4.clone() for _ in range(reps - 1)]
    ms = _time(lambda i: dkv.dkv_attn_decode_q4_0(cfg, q4s[i % reps], None, q, lens, out, ws), steps, stream)
    res["q4_0"] = {"ms_per_step": round(ms, 5), "GBps": round((q4_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                   "hbm_frac": round((q4_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                   "bytes": q4_bytes, "replicas": reps}
    res["q4_0_vs_f16_attention_max_rel_err"] = rel_err_rows(out, f16_out)
    del q4s
    # the Q4-keyframe variant at kf 32 (same 4.5-bit storage as Q4_0)
    c32 = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=32, max_tokens=w.S)
    q4k = torch.empty(dkv.dkv_q4_0_cache_bytes(c32), dtype=torch.uint8, device=k.device)
    st = torch.zeros(w.B, w.Hkv, 2, w.D, dtype=torch.float32, device=k.device)
    dkv.dkv_q4k_encode_prefill(c32, q4k, st, None, k, v, lens, w.S)
    reps = max(1, math.ceil((1 << 30) / q4k.numel()))
    q4ks = [q4k] + [q4k.clone() for _ in range(reps - 1)]
    ms = _time(lambda i: dkv.dkv_attn_decode_q4k(c32, q4ks[i % reps], None, q, lens, out, ws), steps, stream)
    res["q4k_kf32"] = {"ms_per_step": round(ms, 5), "GBps": round((q4_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                       "hbm_frac": round((q4_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "bytes": q4_bytes, "replicas": reps,
                       "how": "dkv_attn_decode_q4k: Q4-keyframe variant at kf 32 (keyframes as Q4_0 of their "
                              "absolute values)"}
    res["q4k_kf32_vs_f16_attention_max_rel_err"] = rel_err_rows(out, f16_out)
    del q4ks
    return res, q4, (q4k, c32)


def static_config(w, kf, args, label, traffic_key, graph=0, strided_on=False, compare=True):
    """One decode layer-step (dkv_attn_decode) of a full static cache: step
    time over args.steps steps, the split-phase kernel alone, the streaming
    ceiling over the same replicas, and (compare) the in-run comparisons and
    the quality report.  Returns (result dict, tensors for the CPU baseline)."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    from quantized_decode_attention_delta_amd import synth
    dev = torch.device("cuda:0")
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
    fused = args.kernel == "fused"
    step_fn = dkv.dkv_attn_decode if fused else dkv.dkv_attn_decode_ref
    launches = dkv.dkv_attn_decode_launches(cfg) if fused else 2

    def step(i):
        step_fn(cfg, caches[i % replicas], None, q, lens, out, ws)

    stream = torch.cuda.current_stream()
    spin_up(lambda: step(0), args.spin_up_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    delta_out = out.clone()

    # dominant kernel alone: the split phase (or the one launch that also
    # merges), launched back to back between two events on its stream
    n_k = max(10, args.steps)
    if fused and launches == 2:
        G = w.Hq // w.Hkv
        name = "k_attn_g8" if kf == 32 else ("k_attn_lfwd_g8" if G <= 4 else "k_attn_long_g8")
        kernel = f"split phase ({name})"

        def kern(i):
            dkv.dkv_attn_decode_partial(cfg, caches[i % replicas], None, q, lens, ws)
    else:
        kernel = "the one launch (split phase + in-kernel merge)" if fused else "reference path (k_attn_ref + combine)"
        kern = step
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    h0 = time.perf_counter()
    for i in range(n_k):
        kern(i)
    host_ms = (time.perf_counter() - h0) * 1e3 / n_k
    k1.record(stream)
    torch.cuda.synchronize()
    kern_ms = k0.elapsed_time(k1) / n_k

    comp = algorithmic_bytes(w.B, w.Hkv, w.Hq, w.D, w.S, kf)
    qo = w.B * w.Hq * w.D * 4 * 2
    eff = f16_equiv_bytes(w.B, w.Hkv, w.D, w.S)
    sink = torch.empty(dkv.dkv_stream_read_sink_words(), dtype=torch.int32, device=dev)
    sr_ms = _time(lambda i: dkv.dkv_stream_read(caches[i % replicas], sink), n_k, stream)
    sr_gbps = cache_bytes / (sr_ms * 1e-3) / 1e9
    res = {
        "workload": label,
        "kernel_path": args.kernel,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "layer_steps_per_s": round(1000.0 / ms_step, 2),
        "launches_per_step": launches,
        "effective_GBps": round(eff / (ms_step * 1e-3) / 1e9, 2),
        "compressed_GBps": round((comp + qo) / (ms_step * 1e-3) / 1e9, 2),
        "hbm_frac_step": round((comp + qo) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "cache_replicas": replicas,
        "roofline": roofline(comp + qo, kern_ms, measured_traffic(traffic_key) if fused else None, kernel, sr_gbps),
        "host_issue_ms": round(host_ms, 5),
        "stream_read_ceiling": {"GBps": round(sr_gbps, 1), "frac_of_peak": round(sr_gbps / HBM_PEAK_GBPS, 4),
                                "bytes": cache_bytes, "how": "dkv_stream_read over the same cache replicas"},
    }
    if graph > 0 and fused:
        res["graph_layers"] = graph_layers(cfg, caches, q, lens, graph, stream)
    if compare:
        res["comparisons"], q4, (q4k, c32) = static_comparisons(w, cfg, k, v, q, lens, ws, args.steps, stream, qo,
                                                                delta_out)
        res["comparisons"]["delta_kv"] = {"ms_per_step": res["ms_per_step"], "GBps": res["compressed_GBps"],
                                          "hbm_frac": res["hbm_frac_step"], "bytes": comp}
        res["quality"] = quality_report([quality_sums(cfg, cache0, q4, None, k, v, lens, q, w.S, q4k, c32)])
        del q4, q4k
        if strided_on and w.S <= 65536 * kf:
            res["comparisons"]["strided"], res["quality"]["strided"] = strided(w, k, v, q, lens, args.steps, stream,
                                                                              qo)
    return res, (q.cpu().numpy(), delta_out.cpu().numpy())


# --------------------------------------------------------------- mixed batch
def mixed_comparisons(w, cfg, bt, k, v, lens, q, ws, cache, steps, stream, s_max):
    """The prefilled mixed batch (before any append) decoded by the paged F16
    and plain-Q4_0 comparison kernels and by Delta-KV (decode only, the same
    footing), and the quality report over every sequence, in sub-batches of 8
    sequences (the cache pools and block-table rows are shared)."""
    import torch

    import quantized_decode_attention_delta_amd as dkv
    dev = k.device
    lens_np = w.seq_lens
    qo = w.B * w.Hq * w.D * 4 * 2
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
    res = {}
    ms = _time(lambda i: dkv.dkv_attn_decode(cfg, cache, bt, q, lens, out, ws), steps, stream)
    delta_out = out.clone()
    comp = sum(algorithmic_bytes(1, w.Hkv, w.Hq, w.D, int(L), w.kf) for L in lens_np)
    res["delta_kv"] = {"ms_per_step": round(ms, 5), "GBps": round((comp + qo) / (ms * 1e-3) / 1e9, 2),
                       "hbm_frac": round((comp + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "bytes": comp,
                       "how": "dkv_attn_decode on the prefilled cache (decode only, as the comparisons)"}
    # paged F16: token rows of each page copied to its physical page
    shape = dkv.f16_cache_shape(cfg)
    kp = torch.zeros(shape, dtype=torch.float16, device=dev)
    vp = torch.zeros_like(kp)
    table = bt.cpu().numpy()
    P = cfg.page_tokens
    for b in range(w.B):
        n = -(-int(lens_np[b]) // P)
        ids = torch.from_numpy(table[b, :n].astype("int64")).to(dev)
        avail = min(n * P, k.shape[2])
        for src, dst in ((k, kp), (v, vp)):
            x = src[b, :, :avail]
            if avail < n * P:
                x = torch.nn.functional.pad(x, (0, 0, 0, n * P - avail))
            dst.index_copy_(0, ids, x.reshape(w.Hkv, n, P, w.D).transpose(0, 1))
    f16_bytes = f16_equiv_bytes(1, w.Hkv, w.D, int(lens_np.sum()))
    ms = _time(lambda i: dkv.dkv_attn_decode_f16(cfg, kp, vp, bt, q, lens, out, ws), steps, stream)
    res["f16"] = {"ms_per_step": round(ms, 5), "GBps": round((f16_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                  "hbm_frac": round((f16_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "bytes": f16_bytes}
    res["delta_kv_vs_f16_attention_max_rel_err"] = rel_err_rows(delta_out, out)
    f16_out = out.clone()
    del kp, vp
    q4 = torch.zeros(dkv.dkv_q4_0_cache_bytes(cfg), dtype=torch.uint8, device=dev)
    dkv.dkv_q4_0_encode(cfg, q4, bt, k, v, lens, s_max)
    q4_bytes = q4_0_bytes(w.Hkv, w.D, lens_np)
    ms = _time(lambda i: dkv.dkv_attn_decode_q4_0(cfg, q4, bt, q, lens, out, ws), steps, stream)
    res["q4_0"] = {"ms_per_step": round(ms, 5), "GBps": round((q4_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                   "hbm_frac": round((q4_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "bytes": q4_bytes}
    res["q4_0_vs_f16_attention_max_rel_err"] = rel_err_rows(out, f16_out)
    q4k = torch.zeros(dkv.dkv_q4_0_cache_bytes(cfg), dtype=torch.uint8, device=dev)
    st = torch.zeros(w.B, w.Hkv, 2, w.D, dtype=torch.float32, device=dev)
    dkv.dkv_q4k_encode_prefill(cfg, q4k, st, bt, k, v, lens, s_max)
    ms = _time(lambda i: dkv.dkv_attn_decode_q4k(cfg, q4k, bt, q, lens, out, ws), steps, stream)
    res["q4k_kf32"] = {"ms_per_step": round(ms, 5), "GBps": round((q4_bytes + qo) / (ms * 1e-3) / 1e9, 2),
                       "hbm_frac": round((q4_bytes + qo) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                       "bytes": q4_bytes, "how": "dkv_attn_decode_q4k: Q4-keyframe variant at kf 32"}
    res["q4k_kf32_vs_f16_attention_max_rel_err"] = rel_err_rows(out, f16_out)
    res["how"] = ("paged caches (the same shuffled 256-token pages), the prefilled batch before any append, "
                  "the first step's queries; each kernel timed back to back with HIP events")
    parts = []
    sub = 8
    for b0 in range(0, w.B, sub):
        b1 = min(w.B, b0 + sub)
        cs = dkv.Config(batch=b1 - b0, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=w.kf,
                        page_tokens=cfg.page_tokens, n_pages=cfg.n_pages, max_pages_per_seq=cfg.max_pages_per_seq)
        S = int(lens_np[b0:b1].max())
        parts.append(quality_sums(cs, cache, q4, bt[b0:b1].contiguous(), k[b0:b1, :, :S].contiguous(),
                                  v[b0:b1, :, :S].contiguous(), lens[b0:b1].contiguous(), q[b0:b1].contiguous(), S,
                                  q4k, cs))
    del q4, q4k
    qual = quality_report(parts)
    qual["how"] = "every sequence of the prefilled batch, sub-batches of 8 sequences"
    return res, qual


def run_mixed(args):
    """Serving loop of the mixed workload: paged cache (256-token pages, shuffled
    physical ids), bulk prefill, then per step one appended token per sequence
    followed by decode attention over the grown cache.  A step = append + decode
    of one layer in one call (dkv_append_attn_decode); the timed steps follow
    the warm-up steps.  The split kernel is then timed back to back on the
    final cache, and the same steps through separate dkv_append +
    dkv_attn_decode calls, on a copy of the prefilled cache, are timed and must
    leave identical bytes."""
    import numpy as np
    import torch

    import quantized_decode_attention_delta_amd as dkv
    from quantized_decode_attention_delta_amd import synth

    dev = torch.device("cuda:0")
    over = {"extra_tokens": max(128, args.warmup + args.steps)}
    if args.mixed_batch:
        over["B"] = args.mixed_batch
    if args.mixed_max_len:
        over["S"] = args.mixed_max_len
    w = gen_workload("mixed", args, **over)
    nsteps = w.extra_tokens
    table, n_pages = synth.page_table(w)
    cfg = dkv.Config(batch=w.B, n_q_heads=w.Hq, n_kv_heads=w.Hkv, head_dim=w.D, kf=w.kf,
                     page_tokens=w.page_tokens, n_pages=n_pages, max_pages_per_seq=table.shape[1])
    lens0 = w.seq_lens.astype(np.int32)
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
    s_max = w.k.shape[2]
    dkv.dkv_encode_prefill(cfg, cache, state, bt, k, v, lens, s_max)
    torch.cuda.synchronize()
    q = torch.from_numpy(np.stack([synth.queries(w, s) for s in range(nsteps)])).to(dev)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    comparisons = qual = None
    if not args.no_compare:
        log("mixed: comparisons and quality on the prefilled batch")
        comparisons, qual = mixed_comparisons(w, cfg, bt, k, v, lens, q[0], ws, cache, args.steps, stream, s_max)
    del k, v
    torch.cuda.empty_cache()
    cache_b, state_b = cache.clone(), state.clone()
    kn_t = torch.from_numpy(kn).to(dev)
    vn_t = torch.from_numpy(vn).to(dev)
    pos = torch.from_numpy(lens0[None, :] + np.arange(nsteps, dtype=np.int32)[:, None]).to(dev)   # [step][B]
    lens_after = pos + 1
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
    out_b = torch.empty_like(out)

    def step(s):
        dkv.dkv_append_attn_decode(cfg, cache, state, bt, kn_t[s], vn_t[s], pos[s], q[s], lens_after[s], out, ws)

    def step_unfused(s):
        dkv.dkv_append(cfg, cache_b, state_b, bt, kn_t[s], vn_t[s], pos[s])
        dkv.dkv_attn_decode(cfg, cache_b, bt, q[s], lens_after[s], out_b, ws)

    log("mixed: serving loop")
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
    last = args.warmup + args.steps - 1
    out_last = out.clone()

    # the split kernel alone, right after the loop, on the final cache (launches
    # back to back between two events on the kernel's stream)
    n_k = max(10, args.steps)
    k0 = torch.cuda.Event(enable_timing=True)
    k1 = torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(n_k):
        dkv.dkv_attn_decode_partial(cfg, cache, bt, q[last], lens_after[last], ws)
    k1.record(stream)
    torch.cuda.synchronize()
    kern_ms = k0.elapsed_time(k1) / n_k

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

    Lt = [lens0 + s + 1 for s in range(args.warmup, args.warmup + args.steps)]
    Lf = Lt[-1]
    comp_last = sum(algorithmic_bytes(1, w.Hkv, w.Hq, w.D, int(L), w.kf) for L in Lf)
    comp_avg = float(np.mean([sum(algorithmic_bytes(1, w.Hkv, w.Hq, w.D, int(L), w.kf) for L in x) for x in Lt]))
    eff_avg = float(np.mean([int(x.sum()) * w.Hkv * w.D * 2 * 2 for x in Lt]))
    qo = w.B * w.Hq * w.D * 4 * 2
    rf = roofline(comp_last + qo, kern_ms, measured_traffic("mixed"), "split phase (k_attn_g8), back to back on "
                  "the final cache")
    rf["kernel_ms_le_step_ms"] = bool(kern_ms <= ms_step)
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
            "workload": f"mixed serving batch: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D}, lengths uniform in "
                        f"[1024, {w.S}] (drawn {int(lens0.min())}..{int(lens0.max())}), {w.page_tokens}-token "
                        f"pages (shuffled), kf={w.kf}, half periodic templates, half regime-switching; "
                        f"step = append of one token per sequence + decode attention over the grown cache",
            "kernel": "fused",
        },
        "layer_steps_per_s": round(1000.0 / ms_step, 2),
        "launches_per_step": dkv.dkv_attn_decode_launches(cfg),
        "effective_GBps": round(eff_avg / (ms_step * 1e-3) / 1e9, 2),
        "compressed_GBps": round((comp_avg + qo) / (ms_step * 1e-3) / 1e9, 2),
        "hbm_frac_step": round((comp_avg + qo) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": rf,
        "unfused": {"ms_per_step": round(ms_unfused, 5), "layer_steps_per_s": round(1000.0 / ms_unfused, 2),
                    "how": "dkv_append then dkv_attn_decode on a copy of the prefilled cache",
                    "identical_cache_state_output": same},
    }
    if comparisons is not None:
        res["comparisons"] = comparisons
        res["quality"] = qual
        res["quality"]["strided_vs_delta_kv_mixed"] = strided_mixed_quality(dev)
    host = {"w": w, "kf": w.kf, "lens": Lf, "q": q[last].cpu().numpy(), "out": out_last.cpu().numpy()}
    return res, host


def headline_fields(d, label):
    """The contract's top-level fields for a single static workload's line."""
    return {"metric": METRIC, "value": d["effective_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": d["steps"],
            "warmup": d["warmup"], "ms_per_step": d["ms_per_step"], "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": {"workload": label, "kernel": d["kernel_path"], "cache_replicas": d["cache_replicas"]}}


def static_label(w, kf):
    names = {"tiny": "tiny", "8b": "Llama-3-8B-shaped layer", "long": "long context",
             "70b": "Llama-3-70B-shaped layer"}
    return f"{names[w.name]}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} D={w.D} S={w.S} kf={kf}"


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    import quantized_decode_attention_delta_amd as dkv
    dkv.load()
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    threads = host_threads(args)

    if args.workload in ("all", "mixed"):
        res, host = run_mixed(args)
        if not args.no_cpu_baseline:
            log("mixed: CPU oracle baseline")
            res["cpu_baseline"] = cpu_baseline(host["w"], host["kf"], host["lens"], host["q"], host["out"],
                                               args.cpu_seconds, threads)
        del host
        if args.workload == "all":
            res["configs"] = {}
            wanted = [c for c in args.configs.split(",") if c]
            long_w = None
            for name in STATIC_CONFIGS:
                if name not in wanted:
                    continue
                if name.startswith("long"):
                    long_w = long_w or gen_workload("long", args)
                    w, kf = long_w, int(name.split("kf")[1])
                else:
                    w = gen_workload(name, args)
                    kf = w.kf
                log(f"config {name}")
                graph = args.graph_layers if args.graph_layers is not None else (32 if name in ("tiny", "8b") else 0)
                d, _ = static_config(w, kf, args, static_label(w, kf), name, graph=graph,
                                     strided_on=(name == "70b"), compare=not args.no_compare)
                res["configs"][name] = d
                if not name.startswith("long"):
                    del w
                torch.cuda.empty_cache()
        print(json.dumps(res), flush=True)
        return

    over = {} if args.kf is None else {"kf": args.kf}
    w = gen_workload(args.workload, args, **over)
    kf = w.kf
    key = f"long_kf{kf}" if args.workload == "long" else args.workload
    graph = args.graph_layers if args.graph_layers is not None else (32 if args.workload in ("tiny", "8b") else 0)
    label = static_label(w, kf)
    d, (q_np, out_np) = static_config(w, kf, args, label, key, graph=graph, strided_on=(args.workload == "70b"),
                                      compare=not args.no_compare)
    res = headline_fields(d, label)
    res.update({k_: v_ for k_, v_ in d.items() if k_ not in ("workload", "steps", "warmup", "ms_per_step")})
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, kf, w.seq_lens, q_np, out_np, args.cpu_seconds, threads)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
