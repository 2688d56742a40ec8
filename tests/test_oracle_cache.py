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


# ----------------------------------------------------------- policy variants
# P1 "KV Cache Manager" prints the compression step as pseudo-code: when the
# cache holds more than cache_size entries, the separators of the past window
# (R without its last w entries) join S (SEP_ACCUMULATION) or replace it, and
# S keeps its last sep_cache_size entries (USE_MAX_SEP_CACHE).
POLICIES = [(False, True), (True, True), (False, False), (True, False)]   # (dynamic, accumulate)


def run_policy(a, s, p, w, flags, dynamic, accumulate, check_each=None):
    sim = oracle.CacheSim(a, s, p, w, sep_ids=[1], dynamic=dynamic, accumulate=accumulate)
    for t, f in enumerate(flags):
        before = (sim.occupancy(), sim.compacted, list(sim.S))
        sim.push(oracle.Entry(pos=t, tok=int(f)))
        if check_each:
            check_each(sim, t + 1, before)
    return sim


def test_hand_worked_policy_trace():
    """a=1, s=2, p=1, w=2 (c = 6), separators at positions 2, 3 and 6, worked
    by hand from the pseudo-code. Dynamic trigger, accumulating: R grows to
    [1..5] (cache 6); pushing 6 makes 7 > 6, so the past window [1, 2, 3, 4]
    is compressed, S = [2, 3], R = [5, 6]; pushing 8 (cache 7) compresses
    [5, 6]: S = [2, 3, 6] -> last 2 = [3, 6], R = [7, 8]; pushing 10
    compresses [7, 8] (no separator), R = [9, 10]. Without accumulation the
    compression at 8 leaves S = [6], the cache then holds 1 + 1 + |R| and
    only pushing 11 exceeds 6: [7, 8, 9] is compressed, S = [], R = [10, 11].
    Fixed caps, without accumulation: R exceeds p + w = 3 at 4, 6, 8, 10,
    each time S becomes the separators of the two oldest entries."""
    flags = np.zeros(12, bool)
    flags[[2, 3, 6]] = True
    want = {
        (True, True): {5: ([0], [], [1, 2, 3, 4, 5]), 6: ([0], [2, 3], [5, 6]),
                       8: ([0], [3, 6], [7, 8]), 10: ([0], [3, 6], [9, 10]),
                       11: ([0], [3, 6], [9, 10, 11])},
        (True, False): {6: ([0], [2, 3], [5, 6]), 8: ([0], [6], [7, 8]),
                        10: ([0], [6], [7, 8, 9, 10]), 11: ([0], [], [10, 11])},
        (False, False): {4: ([0], [2], [3, 4]), 6: ([0], [3], [5, 6]), 8: ([0], [6], [7, 8]),
                         10: ([0], [], [9, 10])},
    }
    for pol, states in want.items():
        sim = oracle.CacheSim(1, 2, 1, 2, sep_ids=[1], dynamic=pol[0], accumulate=pol[1])
        for t in range(12):
            sim.push(oracle.Entry(t, int(flags[t])))
            if t in states:
                assert sim.positions() == states[t], (pol, t)


def test_policy_simulation_matches_compression_points():
    for a, s, p, w, flags in param_cases(count=100, seed=97):
        for dyn, acc in POLICIES:
            def chk(sim, t, before):
                assert sim.positions() == tuple(oracle.policy_positions(flags, t, a, s, p, w, dyn, acc)), \
                    (a, s, p, w, t, dyn, acc)
                assert sim.compacted == (sim.R[0].pos if sim.R else t) - a if t > a else sim.compacted == 0
            run_policy(a, s, p, w, flags, dyn, acc, chk)
        assert all(oracle.policy_positions(flags, t, a, s, p, w) ==
                   oracle.closed_form_positions(flags, t, a, s, p, w) for t in range(len(flags) + 1))


def test_dynamic_trigger_is_the_cache_size():
    """Dynamic rule: the cache never holds more than c entries after a push,
    and a compression happens exactly when the push would exceed c."""
    for a, s, p, w, flags in param_cases(count=80, seed=101):
        c = a + s + p + w
        for acc in (True, False):
            def chk(sim, t, before):
                occ0, comp0, _ = before
                assert sim.occupancy() <= c
                compressed = sim.compacted != comp0
                assert compressed == (t > a and occ0 + 1 > c), (a, s, p, w, t)
                if compressed:
                    assert len(sim.R) == w
            run_policy(a, s, p, w, flags, True, acc, chk)


def test_dynamic_with_full_separator_cache_has_fixed_spacing():
    """Once S holds s entries (accumulating), the dynamic rule compresses
    every p + 1 tokens, p + 1 entries at a time, as the fixed rule does."""
    for a, s, p, w, flags in param_cases(count=80, seed=103):
        full = [False]
        def chk(sim, t, before):
            _, comp0, S0 = before
            if len(S0) == s and s > 0:
                full[0] = True
            if full[0] and sim.compacted != comp0:
                assert sim.compacted - comp0 == p + 1
        run_policy(a, s, p, w, flags, True, True, chk)


def test_no_accumulation_keeps_only_the_last_window():
    for a, s, p, w, flags in param_cases(count=80, seed=107):
        for dyn in (False, True):
            def chk(sim, t, before):
                _, comp0, S0 = before
                Spos = [e.pos for e in sim.S]
                if sim.compacted != comp0:
                    lo, hi = a + comp0, a + sim.compacted
                    seps = [x for x in range(lo, hi) if flags[x]]
                    assert Spos == seps[max(0, len(seps) - s):]
                else:
                    assert Spos == [e.pos for e in S0]
            run_policy(a, s, p, w, flags, dyn, False, chk)


def test_streamingllm_is_the_same_under_every_policy():
    rng = np.random.default_rng(109)
    for a, w in [(4, 8), (0, 3), (2, 1)]:
        flags = rng.random(90) < 0.5
        ref = run_policy(a, 0, 0, w, flags, False, True).positions()
        for dyn, acc in POLICIES:
            assert run_policy(a, 0, 0, w, flags, dyn, acc).positions() == ref


class _MutDynIgnoresS(ocache.CacheSim):
    """dynamic trigger that forgets the separator block in the cache size"""
    def push(self, e):
        self.t += 1
        if len(self.I) < self.a:
            self.I.append(e)
            return
        self.R.append(e)
        if len(self.I) + len(self.R) > self.c:
            batch = [self.R.popleft() for _ in range(len(self.R) - self.w)]
            for x in batch:
                if x.tok in self.sep_set:
                    self.S.append(x)
                    if len(self.S) > self.s:
                        self.S.popleft()
            self.compacted += len(batch)


class _MutNoAccumKeepsOld(ocache.CacheSim):
    """SEP_ACCUMULATION off, but the old separators are kept anyway"""
    def __init__(self, *args, **kw):
        super().__init__(*args, **kw)
        self.accumulate = True


@pytest.mark.parametrize("mutant,dyn,acc", [(_MutDynIgnoresS, True, True), (_MutNoAccumKeepsOld, True, False),
                                            (_MutNoAccumKeepsOld, False, False)])
def test_planted_policy_mistakes_fail_the_pin(mutant, dyn, acc):
    caught = False
    for a, s, p, w, flags in param_cases(count=60, seed=113):
        sim = mutant(a, s, p, w, sep_ids=[1], dynamic=dyn, accumulate=acc)
        for t, f in enumerate(flags):
            sim.push(oracle.Entry(t, int(f)))
            if sim.positions() != tuple(oracle.policy_positions(flags, t + 1, a, s, p, w, dyn, acc)):
                caught = True
                break
        if caught:
            break
    assert caught
