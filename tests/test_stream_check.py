"""The grouped-step decode helper of the GPU stream tests against the plain
per-step oracle decode (CPU only).

stream_check.decode_steps evaluates many decode steps per masked-attention
call; it must give, step by step, what oracle.decode_attention gives over the
simulation's keys plus the current token, and leave the simulation in the
same state as pushing the tokens one by one.
"""
import math

import numpy as np
import pytest

import oracle
from inputs import gen

from .stream_check import decode_steps


@pytest.mark.parametrize("params,seg", [((4, 6, 5, 9), 7), ((2, 3, 2, 4), 32), ((4, 0, 0, 12), 5),
                                        ((0, 8, 30, 10), 64)])
def test_grouped_steps_equal_single_steps(params, seg):
    a, s, p, w = params
    rng = np.random.default_rng(sum(params) * 31 + seg)
    T0, T1, Hq, Hkv, D = 40, 170, 8, 2, 64
    ids = np.where(rng.random(T1) < 0.3, rng.integers(0, 8, T1), rng.integers(8, 1000, T1))
    k = gen.round_storage(rng.standard_normal((Hkv, T1, D)), "bf16")
    v = gen.round_storage(rng.standard_normal((Hkv, T1, D)), "bf16")
    q = gen.round_storage(rng.standard_normal((T1, Hq, D)), "bf16")
    scale = 1.0 / math.sqrt(D)
    sep = list(range(8))

    def kv_rows(pos):
        return gen.bf16_bits_to_f64(k[:, pos]), gen.bf16_bits_to_f64(v[:, pos])

    grouped = oracle.CacheSim(a, s, p, w, sep)
    single = oracle.CacheSim(a, s, p, w, sep)
    for t in range(T0):
        grouped.push(oracle.Entry(t, int(ids[t])))
        single.push(oracle.Entry(t, int(ids[t])))
    seen = []
    o, lse, kept = decode_steps(grouped, ids, T0, T1, lambda s0, s1: q[s0:s1], kv_rows, scale, seg=seg,
                                after_push=lambda t, sim: seen.append((t, sim.positions())),
                                keep=range(T0, T1, 13))
    for t in range(T0, T1):
        keys = [e.pos for e in single.keys()] + [t]
        kk, vv = kv_rows(keys)
        o_ref, l_ref = oracle.decode_attention(gen.bf16_bits_to_f64(q[t]), kk, vv, scale)
        assert np.max(np.abs(o[t - T0] - o_ref)) < 1e-12
        assert np.max(np.abs(lse[t - T0] - l_ref)) < 1e-12
        if t in kept:
            assert kept[t].tolist() == keys
        single.push(oracle.Entry(t, int(ids[t])))
        assert seen[t - T0] == (t, single.positions())
    assert grouped.positions() == single.positions()
