"""Oracle outputs of consecutive streaming decode steps, evaluated in groups.

Decode step t attends exactly the keys the cache simulation holds before
token t is inserted, plus token t itself (P1 "Streaming-SepLLM": each token
runs the forward with the cache, then the cache is updated). For a run of
consecutive steps the keys of all of them go into one list, and step r's row
of a 0/1 mask marks its own keys. Masked attention over that list
(oracle.attention_rows, the dense masked softmax of P2 §1.2) gives, row by
row, the softmax over exactly that step's keys: a masked key contributes
exp(-inf) = 0 to both the numerator and the denominator. This is the decode
definition (oracle.decode_attention) evaluated R steps per call; the test
``test_stream_check.py`` pins the two against each other on small streams.

Only oracle functions compute here; nothing comes from the HIP path.
"""
from __future__ import annotations

import numpy as np

import oracle
from inputs import gen


def decode_steps(sim, ids, t0, t1, q_bits, kv_rows, scale, seg=32, after_push=None, keep=()):
    """Oracle decode outputs of steps t0 .. t1-1 of one sequence.

    sim      oracle.CacheSim holding exactly the tokens before t0; it is
             advanced to t1 (token t is pushed after step t's keys are taken).
    ids      token id of each absolute position (indexable by position).
    q_bits   q_bits(s0, s1) -> [s1-s0, Hq, D] bf16 bit patterns of the queries.
    kv_rows  kv_rows(positions) -> (k, v), each [Hkv, len, D] float64, the
             key/value rows of those positions.
    after_push(t, sim)  called once token t has been inserted.
    keep     steps whose ordered key list (initial, separators, recent, then
             t) is returned, for checks that depend on cache order.
    Returns (o [t1-t0, Hq, D], lse [t1-t0, Hq], {t: key positions}).
    """
    keep = set(keep)
    outs, lses, kept = [], [], {}
    for s0 in range(t0, t1, seg):
        s1 = min(t1, s0 + seg)
        keysets = []
        for t in range(s0, s1):
            I, S, R = sim.positions()
            ks = np.asarray(I + S + R + [t], np.int64)
            keysets.append(ks)
            if t in keep:
                kept[t] = ks
            sim.push(oracle.Entry(t, int(ids[t])))
            if after_push is not None:
                after_push(t, sim)
        union = np.unique(np.concatenate(keysets))
        M = np.zeros((s1 - s0, len(union)), dtype=bool)
        for r, ks in enumerate(keysets):
            M[r, np.searchsorted(union, ks)] = True
        k, v = kv_rows(union)
        q = gen.bf16_bits_to_f64(q_bits(s0, s1)).transpose(1, 0, 2)      # [Hq, R, D]
        Hq = q.shape[0]
        G = Hq // k.shape[0]
        o, lse = oracle.attention_rows(q, k, v, M, scale, [h // G for h in range(Hq)])
        outs.append(o.transpose(1, 0, 2))
        lses.append(lse.T)
    return np.concatenate(outs), np.concatenate(lses), kept
