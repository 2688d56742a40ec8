"""Pins of the oracle's flags, mask, compaction and tile classes.

Each check compares the oracle with something other than itself: a
set-based brute force written from the visibility rule, special cases whose
mask is a textbook triangle or band, values the pages print, and a
row-count closed form. The planted-mistake tests at the end show that a
plausible slip in the oracle (off-by-one window, dropped term, wrong index)
fails these pins.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import mask as omask

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")))
pytestmark = pytest.mark.filterwarnings("ignore")


def brute_visible(flags, a, n):
    """Kept keys of each query as Python sets: the first a tokens, the n most
    recent positions (self included) and the separators, none in the future."""
    S = len(flags)
    M = np.zeros((S, S), dtype=bool)
    for i in range(S):
        kept = set()
        for j in range(S):
            if j > i:
                continue
            if j < a:
                kept.add(j)
            if i - j < n:
                kept.add(j)
            if flags[j]:
                kept.add(j)
        for j in kept:
            M[i, j] = True
    return M


def random_cases(count=60, seed=7, smax=48):
    rng = np.random.default_rng(seed)
    for _ in range(count):
        S = int(rng.integers(1, smax + 1))
        a = int(rng.integers(0, 9))
        n = int(rng.integers(1, S + 6))
        p = float(rng.choice([0.0, 0.05, 0.3, 0.5, 1.0]))
        flags = rng.random(S) < p
        yield S, a, n, flags


def test_is_sep_brute_force_and_pages_ids():
    sep = GOLD["llama3_separator_ids"]["value"]
    rng = np.random.default_rng(3)
    ids = np.concatenate([np.array(sep), rng.integers(0, 130000, 500)])
    got = oracle.is_sep(ids, sep)
    want = np.array([any(int(x) == s for s in sep) for x in ids])
    assert np.array_equal(got, want)
    assert got[:len(sep)].all()
    # ids that are separators for Pythia but not for Llama 3 are not flagged
    pythia_only = [x for x in GOLD["pythia_separator_ids"]["value"] if x not in sep]
    assert not oracle.is_sep(np.array(pythia_only), sep).any()


def test_mask_matches_brute_force():
    for S, a, n, flags in random_cases():
        assert np.array_equal(oracle.sep_mask(flags, a, n), brute_visible(flags, a, n)), (S, a, n)


def test_mask_rows_equals_full_mask_rows():
    for S, a, n, flags in random_cases(count=20, seed=11, smax=200):
        rows = sorted(set(np.random.default_rng(S).integers(0, S, 7).tolist()))
        assert np.array_equal(oracle.mask_rows(flags, a, n, rows), oracle.sep_mask(flags, a, n)[rows])


def test_special_cases_reduce_to_triangles_and_bands():
    rng = np.random.default_rng(5)
    S = 40
    tril = np.tril(np.ones((S, S), dtype=bool))
    flags = rng.random(S) < 0.2
    # window at least as long as the sequence: ordinary causal attention
    assert np.array_equal(oracle.sep_mask(flags, 3, S, ), tril)
    assert np.array_equal(oracle.sep_mask(flags, 0, S + 10), tril)
    # every token a separator: causal
    assert np.array_equal(oracle.sep_mask(np.ones(S, bool), 0, 1), tril)
    # every token initial: causal
    assert np.array_equal(oracle.sep_mask(np.zeros(S, bool), S, 1), tril)
    # no separators, no initial tokens: sliding window of width n
    for n in (1, 2, 5, 17):
        band = np.tri(S, S, 0, dtype=bool) & ~np.tri(S, S, -n, dtype=bool)
        assert np.array_equal(oracle.sep_mask(np.zeros(S, bool), 0, n), band)
    # n = 1 and nothing else: each query sees only itself
    assert np.array_equal(oracle.sep_mask(np.zeros(S, bool), 0, 1), np.eye(S, dtype=bool))


def test_init_tok_max_idx_example_from_pages():
    ex = GOLD["init_tok_max_idx_example"]
    a = ex["init_tok_max_idx"] + 1          # a counts the kept initial tokens
    S = 30
    M = oracle.sep_mask(np.zeros(S, bool), a, 4)
    last = M[S - 1]
    assert sorted(np.flatnonzero(last[:10]).tolist()) == ex["kept_indices"]


def test_compaction_brute_force_and_invariants():
    for S, a, n, flags in random_cases(count=40, seed=13, smax=300):
        rank, sep_pos, count = oracle.compact(flags)
        r = 0
        want_rank = []
        want_pos = []
        for j in range(S):
            want_rank.append(r)
            if flags[j]:
                want_pos.append(j)
                r += 1
        want_rank.append(r)
        assert rank.tolist() == want_rank
        assert count == r == int(np.sum(flags))
        assert sep_pos[:count].tolist() == want_pos
        assert (sep_pos[count:] == -1).all()
        for k in range(count):
            assert flags[sep_pos[k]] and rank[sep_pos[k]] == k


def test_row_count_closed_form():
    """|row i| = min(i+1, a) + (i+1 - max(lo, a))^+ + (rank[max(lo,a)] - rank[a])^+,
    lo = max(i-n+1, 0): initial keys, then the window above the initial
    block, then the separators between the initial block and the window."""
    for S, a, n, flags in random_cases(count=40, seed=17, smax=400):
        rank, _, _ = oracle.compact(flags)
        M = oracle.sep_mask(flags, a, n)
        for i in range(S):
            lo = max(i - n + 1, 0)
            hi = max(lo, min(a, S))
            want = min(i + 1, a) + max(0, i + 1 - hi) + max(0, int(rank[hi] - rank[min(a, S)]))
            assert M[i].sum() == want, (S, a, n, i)


def brute_tile_class(M, tq, tk):
    S_q, S_k = M.shape
    out = np.zeros((-(-S_q // tq), -(-S_k // tk)), dtype=np.uint8)
    for qt in range(out.shape[0]):
        for kt in range(out.shape[1]):
            seen_vis = seen_hid = False
            for i in range(qt * tq, min(S_q, (qt + 1) * tq)):
                for j in range(kt * tk, min(S_k, (kt + 1) * tk)):
                    if M[i, j]:
                        seen_vis = True
                    else:
                        seen_hid = True
            out[qt, kt] = 2 if (seen_vis and seen_hid) else (1 if seen_vis else 0)
    return out


def test_tile_class_brute_force_and_slabs():
    for S, a, n, flags in random_cases(count=25, seed=19, smax=100):
        M = oracle.sep_mask(flags, a, n)
        for tq, tk in ((4, 4), (8, 16), (16, 8), (1, 1)):
            tc = oracle.tile_class(M, tq, tk)
            assert np.array_equal(tc, brute_tile_class(M, tq, tk))
            assert np.array_equal(oracle.tile_class_slabs(flags, a, n, tq, tk), tc)
        assert np.array_equal(oracle.tile_class(M, 1, 1), M.astype(np.uint8))
        # a block above the diagonal is never fully visible
        tc = oracle.tile_class(M, 8, 8)
        for qt in range(tc.shape[0]):
            for kt in range(qt + 1, tc.shape[1]):
                assert tc[qt, kt] == 0


# ----------------------------------------------------------- planted mistakes
def _mut_window_off_by_one(flags, a, n):
    S = len(flags)
    keep = np.zeros((S, S), bool)
    keep[:, flags] = True
    keep[:, :a] = True
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    keep |= (i - j >= 0) & (i - j <= n)          # <= instead of <
    return keep & (j <= i)


def _mut_no_initial(flags, a, n):
    return omask.sep_mask(flags, 0, n)


def _mut_no_causal(flags, a, n):
    S = len(flags)
    keep = np.zeros((S, S), bool)
    keep[:, flags] = True
    keep[:, :a] = True
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    keep |= (i - j >= 0) & (i - j < n)
    return keep


def _mut_sep_rows(flags, a, n):
    S = len(flags)
    keep = np.zeros((S, S), bool)
    keep[flags, :] = True                        # rows instead of columns
    keep[:, :a] = True
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    keep |= (i - j >= 0) & (i - j < n)
    return keep & (j <= i)


@pytest.mark.parametrize("mutant", [_mut_window_off_by_one, _mut_no_initial, _mut_no_causal,
                                    _mut_sep_rows])
def test_planted_mask_mistakes_fail_the_pin(mutant):
    caught = any(not np.array_equal(mutant(flags, a, n), brute_visible(flags, a, n))
                 for S, a, n, flags in random_cases())
    assert caught
