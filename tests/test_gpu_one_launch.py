"""GPU checks of the decode in one launch: where the GQA <= 8 kernels run
(kf a multiple of 32 up to 512) on a small launch (at most 16 splits per
(sequence, kv-head), at most 256 workgroups), the last workgroup of each
(sequence, kv-head) to finish merges that row's split-K partial records into
the output, counting arrivals in the workspace's counters; larger launches
keep the separate combine kernel.

Checked here, through the C ABI, on both sides of that rule
(dkv_attn_decode_launches tells which side a case is on):
* the arrival counters are zero again after every call, so repeated calls on
  one workspace give bit-identical outputs;
* the output is within 2e-3 of the float64 oracle and matches the two-launch
  reference path (dkv_attn_decode_ref: LDS rebuild + separate combine);
* one-launch cases at 1, 2, 4 and 8 query heads per kv-head, paged, with an
  empty sequence, and on the long-interval kernel (kf 128 and 512);
* a workspace shared with the strided-reference and comparison decodes (whose
  partial records are larger) still gives the right result.
"""
import numpy as np
import pytest
import torch

import quantized_decode_attention_delta_amd as dkv
from quantized_decode_attention_delta_amd import synth

pytestmark = pytest.mark.gpu

import gpu_util as U  # noqa: E402


def _counter_bytes(cfg):
    return (cfg.batch * cfg.n_kv_heads * 4 + 255) // 256 * 256


CASES = [
    # (workload, overrides, kf, page_tokens, lengths, launches)
    ("tiny", dict(), 32, 0, None, 1),                                         # G = 1
    ("8b", dict(S=300, B=3, Hq=4, Hkv=2), 32, 0, [300, 0, 45], 1),            # G = 2, an empty sequence
    ("8b", dict(S=30, B=2, Hq=8, Hkv=2), 32, 0, [30, 7], 1),                  # one split per row
    ("70b", dict(S=400, B=2, Hq=64, Hkv=8), 32, 0, [400, 333], 1),            # G = 8
    ("8b", dict(S=1500, B=2, Hq=16, Hkv=4, D=64), 128, 0, [1500, 900], 1),    # long-interval kernel
    ("long", dict(S=3000, B=2, Hq=32, Hkv=8), 512, 0, [3000, 513], 1),
    ("mixed", dict(B=2, S=500, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 32, 256, None, 1),
    ("8b", dict(S=4096, B=1, Hq=32, Hkv=8), 32, 0, None, 2),                  # 128 splits per row
    ("70b", dict(S=3000, B=3, Hq=64, Hkv=8), 32, 0, [3000, 0, 1777], 2),
    ("8b", dict(S=2500, B=2, Hq=16, Hkv=4, D=64), 128, 0, [2500, 900], 2),
    ("mixed", dict(B=4, S=3000, Hq=8, Hkv=2, min_len=100, extra_tokens=0), 32, 256, None, 2),
]


@pytest.mark.parametrize("name,kw,kf,page,lens,launches", CASES)
def test_one_launch_decode(name, kw, kf, page, lens, launches):
    print(f"one-launch decode {name} {kw} kf={kf} page={page} lens={lens}", flush=True)
    w = synth.make(name, **kw)
    r = U.prefill(w, kf=kf, page_tokens=page, lens=lens)
    assert dkv.dkv_attn_decode_launches(r.cfg) == launches
    q_np = synth.queries(w)
    outs = [U.attention(r, q_np) for _ in range(3)]
    cb = _counter_bytes(r.cfg)
    assert not r.ws[:cb].any(), "arrival counters not reset"
    assert all(np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)) for o in outs[1:])
    enc = U.oracle_encode(w, kf, r.lens_np)
    ref = U.oracle_attention(enc, w, q_np, r.lens_np)
    assert U.rel_err(outs[0], ref) <= U.ATTN_TOL
    two = U.attention(r, q_np, fn="dkv_attn_decode_ref")
    assert U.rel_err(outs[0], two.astype(np.float64)) <= U.ATTN_TOL
    for b, L in enumerate(r.lens_np):
        if L == 0:
            assert np.all(outs[0][b] == 0.0)


def test_workspace_shared_with_other_decodes():
    """The strided-reference decode and the Q4_0 / F16 comparison decodes write
    more partial records than the Delta-KV decode; they sit after the arrival
    counters, so a Delta-KV decode on the same workspace is unaffected."""
    w = synth.make("8b", S=1500, B=3, Hq=8, Hkv=2)
    r = U.prefill(w, kf=32)
    q_np = synth.queries(w)
    first = U.attention(r, q_np)
    q = torch.from_numpy(q_np).to(U.DEV)
    out = torch.empty(w.B, w.Hq, w.D, dtype=torch.float32, device=U.DEV)
    sc = torch.zeros(dkv.dkv_strided_cache_bytes(r.cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_strided_encode_prefill(r.cfg, sc, r.k, r.v, r.lens, r.s_max, 0)
    dkv.dkv_strided_attn_decode(r.cfg, sc, q, r.lens, out, r.ws)
    q4 = torch.zeros(dkv.dkv_q4_0_cache_bytes(r.cfg), dtype=torch.uint8, device=U.DEV)
    dkv.dkv_q4_0_encode(r.cfg, q4, None, r.k, r.v, r.lens, r.s_max)
    dkv.dkv_attn_decode_q4_0(r.cfg, q4, None, q, r.lens, out, r.ws)
    dkv.dkv_attn_decode_f16(r.cfg, r.k, r.v, None, q, r.lens, out, r.ws)
    again = U.attention(r, q_np)
    assert np.array_equal(again.view(np.uint32), first.view(np.uint32))
    assert not r.ws[:_counter_bytes(r.cfg)].any()
