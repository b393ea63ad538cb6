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
    ap.add_argument("--workload", default="70b", choices=["tiny", "8b", "long", "70b"])
    ap.add_argument("--kf", type=int, default=None)
    ap.add_argument("--kernel", default="fused", choices=["fused", "ref"])
    ap.add_argument("--replicas", type=int, default=0, help="cache copies rotated per step (0 = auto, >= 1 GiB)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(w, kf, budget_s):
    """Oracle (as it stands) on a bounded sample: whole (sequence, kv-head)
    pairs, reconstruct K/V from the oracle's own encoding, float64 attention of
    the pair's G query heads.  Encoding is untimed (it is not decode work)."""
    import numpy as np

    import oracle
    from quantized_decode_attention_delta_amd import synth
    q = synth.queries(w)
    G = w.Hq // w.Hkv
    scale = np.float32(1 / math.sqrt(w.D))
    done = 0
    t_total = 0.0
    pairs = [(b, h) for b in range(w.B) for h in range(w.Hkv)]
    for (b, h) in pairs:
        S = int(w.seq_lens[b])
        ek = oracle.encode_stream(np.ascontiguousarray(w.k[b, h, :S]), kf, want_recon=False)
        ev = oracle.encode_stream(np.ascontiguousarray(w.v[b, h, :S]), kf, want_recon=False)
        t0 = time.perf_counter()
        kr = oracle.reconstruct_stream(ek.kf_rows, ek.codes, ek.scales, S, w.D, kf)
        vr = oracle.reconstruct_stream(ev.kf_rows, ev.codes, ev.scales, S, w.D, kf)
        oracle.attention_f64(q[b, h * G:(h + 1) * G], kr, vr, scale)
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= budget_s:
            break
    S = int(w.seq_lens[0])
    eff_bytes = done * 2 * w.D * S * 2        # fp16-equivalent K+V bytes of the sampled pairs
    return {
        "value": round(eff_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} of {len(pairs)} (sequence, kv-head) pairs of the same workload: oracle "
                  f"reconstruction of K and V + float64 attention of {G} query heads, one thread, "
                  f"{t_total:.1f} s",
        "layer_steps_per_s_extrapolated": round(done / t_total / len(pairs), 6),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import quantized_decode_attention_delta_amd as dkv
    from quantized_decode_attention_delta_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
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
    del k, v
    caches = [cache0] + [cache0.clone() for _ in range(replicas - 1)]
    torch.cuda.synchronize()
    q = torch.from_numpy(synth.queries(w)).to(dev)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=dev)
    ws = torch.zeros(dkv.dkv_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    step_fn = dkv.dkv_attn_decode if args.kernel == "fused" else dkv.dkv_attn_decode_ref

    def step(i):
        step_fn(cfg, caches[i % replicas], None, q, lens, out, ws)

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

    # dominant kernel alone: the split phase, timed per launch with events
    n_k = max(10, args.steps)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_k)]
    for i in range(n_k):
        evs[i][0].record(stream)
        if args.kernel == "fused":
            dkv.dkv_attn_decode_partial(cfg, caches[i % replicas], None, q, lens, ws)
        else:
            dkv.dkv_attn_decode_ref(cfg, caches[i % replicas], None, q, lens, out, ws)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))

    comp = algorithmic_bytes(w.B, w.Hkv, w.Hq, w.D, w.S, kf)
    qo = w.B * w.Hq * w.D * 4 * 2
    eff = f16_equiv_bytes(w.B, w.Hkv, w.D, w.S)
    achieved = (comp + qo) / (kern_ms * 1e-3) / 1e9
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
            "traffic": None,
            "kernel_ms": round(kern_ms, 5),
            "algorithmic_bytes": comp + qo,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, kf, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
