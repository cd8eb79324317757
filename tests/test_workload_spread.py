"""The sink-free parity workloads really exercise the attention (CPU only, oracle side).

With the x40 sink at position 0 (the u/krylov_schur thread on rstation.ai: 30-50x RMS norms
for Qwen3-8B sink tokens) many decode rows of the Qwen3-8B layer put more than 0.99 of their
softmax weight on that position, and their outputs reduce to the first value row.  The
sink-free draw of the same layer, used by the sink-free GPU parity cases, must not: no row is
dominated by position 0 and the median row's largest weight stays below 0.5.
"""
import numpy as np

from oracle import nvfp4_oracle as O
from synth import kv_inputs as S
from tests import _pipeline as P


def softmax_spread(name, sink, flags=1):
    """Largest softmax weight of every (sequence, query head) decode row over the full
    sequence, and its weight on position 0, from the oracle's calibration, encoding, query
    transform and dequantisation."""
    c, k, v, kw, vw, q = P.workload(name, sink=sink)
    s, r, g = O.calibrate(S.bf16_to_f32(kw), S.bf16_to_f32(vw), True, flags)
    kc, ks = O.quantize_keys(O.key_transform(S.bf16_to_f32(k), r[None, None], flags), g[0], flags)
    grp = c["hq"] // c["hkv"]
    qp = O.query_transform(S.bf16_to_f32(q).astype(np.float64), np.repeat(s, grp, axis=0)[None], flags)
    top, first = [], []
    for b in range(c["B"]):
        kh = O.dequantize(kc[b], ks[b], g[0])
        for hq in range(c["hq"]):
            e = kh[:, hq // grp, :] @ qp[b, hq] * P.sm_scale()
            p = np.exp(e - e.max())
            p /= p.sum()
            top.append(p.max())
            first.append(p[0])
    return np.array(top), np.array(first)


def test_sink_free_layer_spreads_the_weight():
    top, first = softmax_spread("layer", sink=False)
    assert np.all(first < 0.99)
    assert np.median(top) < 0.5


def test_sink_dominates_many_rows():
    top, first = softmax_spread("layer", sink=True)
    assert np.count_nonzero(first > 0.99) > 32
