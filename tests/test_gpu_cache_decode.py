"""GPU parity of sep_cache_update and sep_attn_decode against the oracle.

The cache must match the list-based simulation bit for bit, block by block
in logical order (initial, separator ring oldest first, recent ring oldest
first): positions, token ids and K/V bytes; every slot outside the live set
must read pos = tok = -1. A bulk update of T tokens must leave exactly the
state (pos, tok, state words, live K/V rows) of T single-token updates.
Decode outputs must match fp64 attention over the retained keys plus the
current token within the bf16 tolerance.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from inputs import configs, gen
from kv_cache_compression_sep_amd import (SEP_POLICY_DYNAMIC, SEP_POLICY_NO_ACCUM, SepCache,
                                          sep_attn_decode, sep_cache_update)

from .gpu_util import check_close, from_dev, guarded_cache, guarded_empty, slots_of, to_dev

pytestmark = pytest.mark.gpu
SEP_IDS = list(range(8))


class Stream:
    """A seeded synthetic token stream for one batch of sequences."""

    def __init__(self, seed, B, Hq, Hkv, D, T, p_sep):
        rng = np.random.default_rng(seed)
        self.ids = np.where(rng.random((B, T)) < p_sep, rng.integers(0, 8, (B, T)),
                            rng.integers(8, 1000, (B, T))).astype(np.int32)
        self.k = gen.round_storage(rng.standard_normal((B, Hkv, T, D)), "bf16")
        self.v = gen.round_storage(rng.standard_normal((B, Hkv, T, D)), "bf16")
        self.q = gen.round_storage(rng.standard_normal((B, T, Hq, D)), "bf16")
        self.B, self.Hq, self.Hkv, self.D, self.T = B, Hq, Hkv, D, T

    def push_gpu(self, cache, t0, t1, d_sep):
        sep_cache_update(cache, to_dev(np.ascontiguousarray(self.k[:, :, t0:t1]), "bf16"),
                         to_dev(np.ascontiguousarray(self.v[:, :, t0:t1]), "bf16"),
                         to_dev(np.ascontiguousarray(self.ids[:, t0:t1])), d_sep)


def live_slots(cache, b):
    return slots_of(cache, b)


def check_cache(cache, sims, stream):
    pos = cache.pos.cpu().numpy()
    tok = cache.tok.cpu().numpy()
    kc = cache.k.view(torch.int16).cpu().numpy()
    vc = cache.v.view(torch.int16).cpu().numpy()
    for b, sim in enumerate(sims):
        I, S, R = live_slots(cache, b)
        assert int(cache.state[b, 0]) == sim.t
        want = sim.positions()
        for slots, wpos, name in zip((I, S, R), want, "ISR"):
            assert pos[b, slots].tolist() == wpos, (b, name)
            assert tok[b, slots].tolist() == [int(stream.ids[b, x]) for x in wpos], (b, name)
            if wpos:
                assert np.array_equal(kc[b][:, slots], stream.k[b][:, wpos].view(np.int16)), (b, name)
                assert np.array_equal(vc[b][:, slots], stream.v[b][:, wpos].view(np.int16)), (b, name)
        dead = sorted(set(range(cache.slots)) - set(I) - set(S) - set(R))
        assert (pos[b, dead] == -1).all() and (tok[b, dead] == -1).all(), b
        assert sim.occupancy() == len(I) + len(S) + len(R)


PARAMS = [
    # a, s,  p,  w
    (4, 6, 5, 9),
    (0, 3, 1, 4),
    (2, 1, 3, 1),
    (4, 64, 64, 256),
    (3, 10, 70, 20),    # p + 1 > 64: compaction crosses a wavefront
    (1, 40, 300, 7),    # compaction across several waves
    (4, 0, 0, 12),      # StreamingLLM: initial + local only
]


# cache policies (P1 "KV Cache Manager" pseudo-code): the dynamic trigger and
# SEP_ACCUMULATION off, on the SepLLM parameter sets
POLICIES = [SEP_POLICY_DYNAMIC, SEP_POLICY_NO_ACCUM, SEP_POLICY_DYNAMIC | SEP_POLICY_NO_ACCUM]
POLICY_PARAMS = [(4, 6, 5, 9), (2, 1, 3, 1), (3, 10, 70, 20), (1, 40, 300, 7), (4, 64, 64, 256)]


def sim_for(params, policy):
    a, s, p, w = params
    return oracle.CacheSim(a, s, p, w, SEP_IDS, dynamic=bool(policy & SEP_POLICY_DYNAMIC),
                           accumulate=not (policy & SEP_POLICY_NO_ACCUM))


@pytest.mark.parametrize("params", PARAMS, ids=[str(p) for p in PARAMS])
def test_single_token_updates_match_simulation(params):
    single_token_updates(params, 0)


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("params", POLICY_PARAMS, ids=[str(p) for p in POLICY_PARAMS])
def test_policy_single_token_updates_match_simulation(params, policy):
    single_token_updates(params, policy)


def single_token_updates(params, policy):
    a, s, p, w = params
    T = min(3 * (a + s + p + w) + 50, 1400)
    st = Stream(zlib.crc32(repr(params).encode()), 2, 4, 2, 64, T, 0.3)
    cache = guarded_cache(2, 2, 64, a, s, p, w, policy=policy)
    sims = [sim_for(params, policy) for _ in range(2)]
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    every = max(1, T // 60)
    for t in range(T):
        st.push_gpu(cache, t, t + 1, d_sep)
        for b in range(2):
            sims[b].push(oracle.Entry(t, int(st.ids[b, t])))
        if t % every == 0 or t == T - 1:
            check_cache(cache, sims, st)


def _cuts(T, mode, params, rng):
    """Chunk boundaries of a bulk replay: `random` (6 random cuts), `small`
    (chunks of 2..7 tokens: compactions straddle call boundaries) or `wrap`
    (a partial first call, then one call longer than the whole cache, so
    separators still in the recent ring survive while new rows overwrite it)."""
    a, s, p, w = params
    if mode == "random":
        return sorted(set([0, T] + rng.integers(1, T, 6).tolist()))
    if mode == "small":
        cuts = [0]
        while cuts[-1] < T:
            cuts.append(min(T, cuts[-1] + int(rng.integers(2, 8))))
        return cuts
    first = min(T - 1, a + w + (p + w) // 2 + 1)
    return [0, first, T]


@pytest.mark.parametrize("mode", ["random", "small", "wrap"])
@pytest.mark.parametrize("params", PARAMS, ids=[str(p) for p in PARAMS])
def test_bulk_updates_equal_single_updates(params, mode):
    bulk_equals_single(params, mode, 0)


@pytest.mark.parametrize("mode", ["random", "wrap"])
@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("params", POLICY_PARAMS, ids=[str(p) for p in POLICY_PARAMS])
def test_policy_bulk_updates_equal_single_updates(params, policy, mode):
    bulk_equals_single(params, mode, policy)


def bulk_equals_single(params, mode, policy):
    a, s, p, w = params
    T = min(4 * (a + s + p + w) + 77, 2000)
    st = Stream(zlib.crc32(repr(params).encode()) + 1, 3, 4, 2, 128, T, 0.25)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    one = guarded_cache(3, 2, 128, a, s, p, w, policy=policy)
    bulk = guarded_cache(3, 2, 128, a, s, p, w, policy=policy)
    for t in range(T):
        st.push_gpu(one, t, t + 1, d_sep)
    cuts = _cuts(T, mode, params, np.random.default_rng(T))
    for t0, t1 in zip(cuts[:-1], cuts[1:]):
        st.push_gpu(bulk, t0, t1, d_sep)
    torch.cuda.synchronize()
    assert torch.equal(one.state[:, :4], bulk.state[:, :4])    # word 4 records the last call
    assert torch.equal(one.pos, bulk.pos)
    assert torch.equal(one.tok, bulk.tok)
    sims = [sim_for(params, policy) for _ in range(3)]
    for b in range(3):
        sims[b].push_many([oracle.Entry(t, int(st.ids[b, t])) for t in range(T)])
    check_cache(bulk, sims, st)
    check_cache(one, sims, st)


DECODE_CASES = [
    # B, Hq, Hkv, D,  a, s,  p,  w,  T
    (2, 32, 8, 128, 4, 64, 64, 256, 700),
    (1, 8, 8, 64, 2, 5, 3, 11, 90),
    (3, 16, 1, 128, 0, 7, 9, 33, 300),
    (1, 12, 3, 64, 4, 20, 2, 40, 5),      # cache still filling the initial block
    (2, 4, 2, 128, 4, 0, 0, 50, 200),     # StreamingLLM mode
    (1, 16, 16, 128, 4, 256, 28, 512, 1500),
    # the dynamic trigger and no accumulation (the recent ring grows past p + w)
    (2, 32, 8, 128, 4, 64, 16, 96, 700, SEP_POLICY_DYNAMIC),
    (1, 8, 2, 64, 2, 9, 5, 20, 300, SEP_POLICY_DYNAMIC | SEP_POLICY_NO_ACCUM),
]


@pytest.mark.parametrize("split", [True, False], ids=["split", "whole"])
@pytest.mark.parametrize("case", DECODE_CASES, ids=[str(c) for c in DECODE_CASES])
def test_decode_matches_oracle(case, split):
    B, Hq, Hkv, D, a, s, p, w, T = case[:9]
    policy = case[9] if len(case) > 9 else 0
    st = Stream(zlib.crc32(repr(case).encode()), B, Hq, Hkv, D, T + 40, 0.2)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    cache = guarded_cache(B, Hkv, D, a, s, p, w, policy=policy, split=split)
    sims = [sim_for((a, s, p, w), policy) for _ in range(B)]
    st.push_gpu(cache, 0, T, d_sep)
    for b in range(B):
        sims[b].push_many([oracle.Entry(t, int(st.ids[b, t])) for t in range(T)])
    scale = 1.0 / math.sqrt(D)
    for t in range(T, T + 40):
        q = to_dev(np.ascontiguousarray(st.q[:, t]), "bf16")
        kn = to_dev(np.ascontiguousarray(st.k[:, :, t]), "bf16")
        vn = to_dev(np.ascontiguousarray(st.v[:, :, t]), "bf16")
        out, lse = sep_attn_decode(q, kn, vn, cache, scale, return_lse=True,
                                   out=guarded_empty((B, Hq, D), torch.bfloat16),
                                   lse=guarded_empty((B, Hq), torch.float32))
        o = from_dev(out)
        l_gpu = from_dev(lse)
        for b in range(B):
            keys = [e.pos for e in sims[b].keys()] + [t]
            kk = gen.bf16_bits_to_f64(st.k[b][:, keys])
            vv = gen.bf16_bits_to_f64(st.v[b][:, keys])
            o_ref, l_ref = oracle.decode_attention(gen.bf16_bits_to_f64(st.q[b, t]), kk, vv, scale)
            check_close(o[b], o_ref, "bf16", f"{case} step {t} b {b}")
            assert np.max(np.abs(l_gpu[b] - l_ref)) < 1e-3
        st.push_gpu(cache, t, t + 1, d_sep)
        for b in range(B):
            sims[b].push(oracle.Entry(t, int(st.ids[b, t])))
