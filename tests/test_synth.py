"""Host checks of the seeded input generators: the arrays are a pure function
of (workload, seed, sizes), whatever the number of host threads drawing them,
and follow each workload's stated recipe (lengths, periodic half)."""
import numpy as np
import pytest

from quantized_decode_attention_delta_amd import synth


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("8b", dict(S=300, B=3)),
    ("long", dict(S=700, B=3)),
    ("70b", dict(S=500, B=3)),
    ("mixed", dict(B=6, S=3000)),
])
def test_workers_do_not_change_the_arrays(name, kw):
    a = synth.make(name, **kw)
    b = synth.make(name, workers=4, **kw)
    assert np.array_equal(a.seq_lens, b.seq_lens)
    assert np.array_equal(a.k.view(np.uint16), b.k.view(np.uint16))
    assert np.array_equal(a.v.view(np.uint16), b.v.view(np.uint16))


def test_mixed_recipe():
    w = synth.make("mixed", B=4, S=4096, extra_tokens=16)
    assert w.seq_lens.min() >= 1024 and w.seq_lens.max() <= 4096
    # rows past each sequence's length + appended tokens stay zero
    for b, L in enumerate(w.seq_lens):
        assert not w.k[b, :, int(L) + 16:].any()
    # the first half is a periodic template plus 0.5% noise: rows one period
    # apart differ by noise only
    x = w.k[0, 0, :int(w.seq_lens[0])].astype(np.float64)
    lags = [np.abs(x[P:] - x[:-P]).max() for P in range(8, 65)]
    assert min(lags) < 0.1 and max(lags) > 0.5
