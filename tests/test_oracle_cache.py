"""Pins of the oracle's four-block cache simulation.

References other than the simulation itself: the closed form of the cache
state (compaction count and compacted prefix computed from t alone),
invariants the pages fix (initial tokens never evicted, every block within
its cap, retained set = initial + separators + window), the StreamingLLM
special case (initial + last w tokens), the parameter contract printed on
the pages, the decode key set as a prefill mask row, and planted mistakes.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import cache as ocache

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))


def param_cases(count=120, seed=61):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        a = int(rng.integers(0, 6))
        if rng.random() < 0.15:
            s, p = 0, 0
        else:
            s = int(rng.integers(1, 12))
            p = int(rng.integers(1, 12))
        w = int(rng.integers(1, 14))
        dens = float(rng.choice([0.0, 0.1, 0.4, 1.0]))
        T = int(rng.integers(0, 160))
        flags = rng.random(T) < dens
        yield a, s, p, w, flags


def run_sim(a, s, p, w, flags, check_each=None):
    sim = oracle.CacheSim(a, s, p, w, sep_ids=[1])
    for t, f in enumerate(flags):
        sim.push(oracle.Entry(pos=t, tok=int(f)))
        if check_each:
            check_each(sim, t + 1)
    return sim


def test_simulation_matches_closed_form_every_step():
    for a, s, p, w, flags in param_cases():
        def chk(sim, t):
            assert sim.positions() == tuple(oracle.closed_form_positions(flags, t, a, s, p, w)), \
                (a, s, p, w, t)
            assert sim.compactions == oracle.n_compactions(t, a, p, w)
        run_sim(a, s, p, w, flags, chk)


def test_invariants_every_step():
    for a, s, p, w, flags in param_cases(seed=67):
        def chk(sim, t):
            I, S, R = sim.positions()
            assert sim.occupancy() <= a + s + p + w
            assert I == list(range(min(a, t)))               # initial never evicted
            assert len(S) <= s and len(R) <= p + w
            if R:
                assert R == list(range(R[0], R[0] + len(R)))  # one contiguous run
                assert R[-1] == t - 1
                cend = R[0]
                # below the window, only separators survive (besides I)
                assert all(flags[x] for x in S) and all(x < cend for x in S)
                assert S == sorted(S)
            for e in sim.keys():                             # id stays with its position
                assert e.tok == int(flags[e.pos])
        run_sim(a, s, p, w, flags, chk)


def test_streamingllm_special_case_keeps_initial_and_last_w():
    """s = p = 0: P1 "Streaming-SepLLM" evict_nonlocal_and_noninitial keeps
    the initial tokens and the local window only."""
    rng = np.random.default_rng(71)
    for a, w in [(4, 8), (0, 3), (2, 1)]:
        flags = rng.random(100) < 0.5
        def chk(sim, t):
            I, S, R = sim.positions()
            assert S == []
            assert I + R == list(range(min(a, t))) + list(range(max(a, t - w), t))
        run_sim(a, 0, 0, w, flags, chk)


def test_bulk_equals_single_pushes():
    for a, s, p, w, flags in param_cases(count=40, seed=73):
        one = run_sim(a, s, p, w, flags)
        bulk = oracle.CacheSim(a, s, p, w, sep_ids=[1])
        cut = len(flags) // 3
        bulk.push_many([oracle.Entry(t, int(flags[t])) for t in range(cut)])
        bulk.push_many([oracle.Entry(t, int(flags[t])) for t in range(cut, len(flags))])
        assert bulk.positions() == one.positions()


def test_parameter_contract_from_pages():
    d = GOLD["sepcache_demo"]
    a, s, w, c = d["init_cache_size"], d["sep_cache_size"], d["local_size"], d["cache_size"]
    p = c - a - s - w                     # the past window takes the rest of the budget
    assert p == 124
    oracle.check_cache_params(a, s, p, w)  # a + s + w < c holds
    with pytest.raises(ValueError):
        oracle.check_cache_params(a, s, 0, w)      # init + sep + local == cache: rejected
    with pytest.raises(ValueError):
        oracle.check_cache_params(a, s, p, 0)      # local must be > 0
    with pytest.raises(ValueError):
        oracle.check_cache_params(-1, s, p, w)     # init must be >= 0
    oracle.check_cache_params(4, 0, 0, 252)        # StreamingLLM: local == cache - init


def test_decode_key_set_is_prefill_mask_row():
    """With s at least the number of separators, the keys a decode step
    reads (cache after t tokens, plus token t) are row t of the prefill mask
    with window n_t = t - cend + 1, where cend starts the window block."""
    rng = np.random.default_rng(79)
    for _ in range(40):
        a = int(rng.integers(0, 5))
        p = int(rng.integers(1, 9))
        w = int(rng.integers(1, 9))
        T = int(rng.integers(1, 120))
        flags = rng.random(T) < 0.3
        s = T + 1
        sim = oracle.CacheSim(a, s, p, w, sep_ids=[1])
        for t in range(T):
            keys = sorted([e.pos for e in sim.keys()] + [t])
            K = oracle.n_compactions(t, a, p, w)
            cend = a + K * (p + 1) if t > a else t
            n_t = t - cend + 1
            row = oracle.mask_rows(flags[:t + 1], a, max(n_t, 1), [t])[0]
            assert keys == np.flatnonzero(row).tolist(), (a, p, w, t)
            sim.push(oracle.Entry(t, int(flags[t])))


def test_decode_oracle_equals_prefill_row_attention():
    rng = np.random.default_rng(83)
    a, s, p, w, T, D = 2, 64, 3, 5, 40, 8
    flags = rng.random(T) < 0.3
    q = rng.standard_normal((4, T, D))
    k = rng.standard_normal((2, T, D))
    v = rng.standard_normal((2, T, D))
    sim = oracle.CacheSim(a, s, p, w, sep_ids=[1])
    scale = 1 / math.sqrt(D)
    for t in range(T):
        keys = [e.pos for e in sim.keys()] + [t]
        o, lse = oracle.decode_attention(q[:, t], k[:, keys], v[:, keys], scale)
        K = oracle.n_compactions(t, a, p, w)
        cend = a + K * (p + 1) if t > a else t
        row = oracle.mask_rows(flags[:T], a, t - cend + 1, [t])
        o2, lse2 = oracle.attention_rows(q[:, [t]], k, v, row, scale, kv_head_of=[0, 0, 1, 1])
        assert np.allclose(o, o2[:, 0], atol=1e-12) and np.allclose(lse, lse2[:, 0], atol=1e-12)
        sim.push(oracle.Entry(t, int(flags[t])))


# ----------------------------------------------------------- planted mistakes
class _MutCompactP(ocache.CacheSim):
    """compacts p entries instead of p + 1"""
    def push(self, e):
        self.t += 1
        if len(self.I) < self.a:
            self.I.append(e)
            return
        self.R.append(e)
        if len(self.R) > self.p + self.w:
            for _ in range(self.p):
                x = self.R.popleft()
                if x.tok in self.sep_set:
                    self.S.append(x)
                    if len(self.S) > self.s:
                        self.S.popleft()


class _MutLifo(ocache.CacheSim):
    """evicts the newest separator instead of the oldest"""
    def push(self, e):
        self.t += 1
        if len(self.I) < self.a:
            self.I.append(e)
            return
        self.R.append(e)
        if len(self.R) > self.p + self.w:
            for _ in range(self.p + 1):
                x = self.R.popleft()
                if x.tok in self.sep_set:
                    if len(self.S) >= self.s:
                        continue
                    self.S.append(x)


class _MutKeepAll(ocache.CacheSim):
    """keeps the non-separators of the past window too"""
    def push(self, e):
        self.t += 1
        if len(self.I) < self.a:
            self.I.append(e)
            return
        self.R.append(e)
        if len(self.R) > self.p + self.w:
            for _ in range(self.p + 1):
                self.S.append(self.R.popleft())
                if len(self.S) > self.s:
                    self.S.popleft()


@pytest.mark.parametrize("mutant", [_MutCompactP, _MutLifo, _MutKeepAll])
def test_planted_cache_mistakes_fail_the_pin(mutant):
    caught = False
    for a, s, p, w, flags in param_cases(count=60, seed=89):
        sim = mutant(a, s, p, w, sep_ids=[1])
        for t, f in enumerate(flags):
            sim.push(oracle.Entry(t, int(f)))
            if sim.positions() != tuple(oracle.closed_form_positions(flags, t + 1, a, s, p, w)):
                caught = True
                break
        if caught:
            break
    assert caught
