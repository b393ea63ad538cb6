"""Seeded synthetic KV caches and queries for the five benchmark workloads.

This module only draws random inputs (numpy, host memory); it holds none of
the Delta-KV arithmetic and is shared by the HIP-path tests, the oracle tests
and the benchmark.  Every array is a pure function of (workload, seed, sizes).

Workloads (sizes can be shrunk for tests with the same value recipe):

* ``tiny``  -- 1 q-head / 1 kv-head, D=64, S=256, B=1, kf=32.  x_0 ~ N(0,1);
  x_t = x_{t-1} + 0.01*|x_{t-1}|*eps.
* ``8b``    -- 32 q / 8 kv heads, D=128, S=4096, B=1, kf=32.  x_t[c] = sigma_c*z_t[c],
  z a stationary AR(1) walk with 1% innovations, sigma_c = exp(N(0,1)) per
  (kv-head, stream, channel) (lognormal channel outliers).
* ``long``  -- as ``8b`` with S=16384, B=8, kf=512 (sweep 32/128/512), plus a
  rare jump: with probability 0.01 per (seq, kv-head, stream, token)
  z_t += N(0, 0.5^2) on every channel.
* ``70b``   -- 64 q / 8 kv heads, D=128, S=32768, B=16, kf=32, AR(1) walk with
  unit channel scales.
* ``mixed`` -- 64 sequences, lengths uniform in [1024, 65536], 32 q / 8 kv heads,
  D=128, 256-token pages (shuffled physical ids), kf=32.  Sequences 0..31:
  periodic templates (period 8..64, template rows N(0,1)) + 0.5% noise;
  sequences 32..63: 8 regime means N(0,1), a switch to a uniformly drawn regime
  with probability 1/16 per token, + 1% noise.  Bulk prefill, then 128
  append+decode steps (the extra 128 tokens per sequence are generated here).

Values are drawn in float32/float64 and rounded to fp16 (round to nearest even)
because the cache API takes fp16 K/V.  Queries are fp32 N(0,1).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import threading

import numpy as np
from scipy.signal import lfilter

WORKLOADS = ("tiny", "8b", "long", "70b", "mixed")
_BASE_SEED = 0xD7C0


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int                 # tokens prefilled per sequence (max over the batch)
    kf: int
    seq_lens: np.ndarray   # int32 [B]
    k: np.ndarray          # fp16 [B][Hkv][S_total][D]
    v: np.ndarray          # fp16 [B][Hkv][S_total][D]
    page_tokens: int = 0
    extra_tokens: int = 0  # tokens per sequence beyond seq_lens kept for appends
    seed: int = 0

    @property
    def G(self):
        return self.Hq // self.Hkv


def default_sizes(name: str) -> dict:
    return {
        "tiny": dict(B=1, Hq=1, Hkv=1, D=64, S=256, kf=32),
        "8b": dict(B=1, Hq=32, Hkv=8, D=128, S=4096, kf=32),
        "long": dict(B=8, Hq=32, Hkv=8, D=128, S=16384, kf=512),
        "70b": dict(B=16, Hq=64, Hkv=8, D=128, S=32768, kf=32),
        "mixed": dict(B=64, Hq=32, Hkv=8, D=128, S=65536, kf=32, page_tokens=256,
                      min_len=1024, extra_tokens=128),
    }[name]


def _children(idx: int, seed: int, n: int):
    ss = np.random.SeedSequence([_BASE_SEED + idx, seed])
    return [np.random.default_rng(c) for c in ss.spawn(n)]


def _ar1_stream_block(rng, T, H, D, sigma, scales, jump_p=0.0, jump_sigma=0.0):
    """K and V of one sequence: returns float64 [2][H][T][D]."""
    phi = np.sqrt(1.0 - sigma * sigma)
    chains = 2 * H * D
    eps = rng.standard_normal((T, chains), dtype=np.float32).astype(np.float64)
    eps *= sigma
    eps[0] = rng.standard_normal(chains)
    if jump_p > 0.0:
        hit = rng.random((T, 2 * H)) < jump_p
        hit[0] = False
        n = int(hit.sum())
        if n:
            jumps = rng.standard_normal((n, D)) * jump_sigma
            view = eps.reshape(T, 2 * H, D)
            view[hit] += jumps
    z = lfilter([1.0], [1.0, -phi], eps, axis=0)          # [T][2*H*D]
    z = z.reshape(T, 2, H, D).transpose(1, 2, 0, 3)        # [2][H][T][D]
    if scales is not None:
        z = z * scales[:, :, None, :]
    return z


def make(name: str, seed: int = 0, progress=None, workers: int = 1, **over) -> Workload:
    """Build a workload.  Keyword overrides (B, S, Hq, Hkv, D, kf, ...) shrink it.
    ``progress(n)``, if given, is called with the number of sequences done after
    each sequence of the mixed workload.  ``workers`` > 1 draws the sequences on
    that many host threads; every sequence has its own generator, so the arrays
    do not depend on it."""
    p = default_sizes(name)
    p.update(over)
    B, Hq, Hkv, D, S, kf = p["B"], p["Hq"], p["Hkv"], p["D"], p["S"], p["kf"]
    assert Hq % Hkv == 0 and D % 32 == 0
    idx = WORKLOADS.index(name)
    extra = int(p.get("extra_tokens", 0))
    page_tokens = int(p.get("page_tokens", 0))
    rngs = _children(idx, seed, B + 2)
    meta_rng = rngs[B]
    if name == "mixed":
        lo = int(p.get("min_len", min(1024, S)))
        seq_lens = meta_rng.integers(lo, S + 1, size=B).astype(np.int32)
    else:
        seq_lens = np.full(B, S, np.int32)
    T = S + extra
    k = np.zeros((B, Hkv, T, D), np.float16)
    v = np.zeros((B, Hkv, T, D), np.float16)

    scales = None
    if name in ("8b", "long"):
        scales = np.exp(meta_rng.standard_normal((2, Hkv, D)))
    elif name not in ("tiny", "70b", "mixed"):
        raise ValueError(name)
    done = [0]
    lock = threading.Lock()

    def fill(b):
        rng = rngs[b]
        if name == "tiny":
            x = np.zeros((2, Hkv, T, D), np.float32)
            x[:, :, 0] = rng.standard_normal((2, Hkv, D), dtype=np.float32)
            eps = rng.standard_normal((T, 2, Hkv, D), dtype=np.float32)
            for t in range(1, T):
                prev = x[:, :, t - 1]
                x[:, :, t] = prev + np.float32(0.01) * np.abs(prev) * eps[t]
            k[b], v[b] = x[0].astype(np.float16), x[1].astype(np.float16)
        elif name in ("8b", "long", "70b"):
            jp, js = (0.01, 0.5) if name == "long" else (0.0, 0.0)
            z = _ar1_stream_block(rng, T, Hkv, D, 0.01, scales, jp, js)
            k[b] = z[0].astype(np.float16)
            v[b] = z[1].astype(np.float16)
        else:
            Tb = int(seq_lens[b]) + extra
            if b < B // 2:
                P = int(rng.integers(8, 65))
                tmpl = rng.standard_normal((2, Hkv, P, D))
                idx_t = np.arange(Tb) % P
                x = tmpl[:, :, idx_t, :]
                x = x + 0.005 * rng.standard_normal((2, Hkv, Tb, D), dtype=np.float32)
            else:
                mu = rng.standard_normal((2, Hkv, 8, D))
                switch = rng.random(Tb) < (1.0 / 16.0)
                draws = rng.integers(0, 8, size=Tb)
                reg = np.zeros(Tb, np.int64)
                cur = int(draws[0])
                for t in range(Tb):
                    if t == 0 or switch[t]:
                        cur = int(draws[t])
                    reg[t] = cur
                x = mu[:, :, reg, :]
                x = x + 0.01 * rng.standard_normal((2, Hkv, Tb, D), dtype=np.float32)
            k[b, :, :Tb] = x[0].astype(np.float16)
            v[b, :, :Tb] = x[1].astype(np.float16)
            if progress is not None:
                with lock:
                    done[0] += 1
                    progress(done[0])

    if workers > 1 and B > 1:
        with concurrent.futures.ThreadPoolExecutor(min(workers, B)) as ex:
            list(ex.map(fill, range(B)))
    else:
        for b in range(B):
            fill(b)

    return Workload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, kf=kf, seq_lens=seq_lens,
                    k=k, v=v, page_tokens=page_tokens, extra_tokens=extra, seed=seed)


def queries(w: Workload, step: int = 0) -> np.ndarray:
    """fp32 N(0,1) decode queries [B][Hq][D] for decode step ``step``."""
    rng = _children(WORKLOADS.index(w.name), w.seed * 1000003 + 7 + step, 1)[0]
    return rng.standard_normal((w.B, w.Hq, w.D), dtype=np.float32)


def page_table(w: Workload, seed_extra: int = 0):
    """Shuffled physical page ids: returns (block_table int32 [B][max_pages], n_pages)."""
    assert w.page_tokens > 0
    cap = w.S + w.extra_tokens
    max_pages = -(-cap // w.page_tokens)
    need = [-(-(int(L) + w.extra_tokens) // w.page_tokens) for L in w.seq_lens]
    n_pages = int(sum(need))
    rng = _children(WORKLOADS.index(w.name), w.seed * 7919 + 11 + seed_extra, 1)[0]
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((w.B, max_pages), -1, np.int32)
    pos = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[pos:pos + n]
        pos += n
    return table, n_pages
