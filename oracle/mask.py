"""Separator flags, the Sep-Attention mask M, compaction and tile classes.

Test infrastructure only (see the package docstring for who may import it).

Readings of the pages used here:
  * ``a`` counts initial tokens: key j is initial iff j < a. P1 "Initial
    Tokens" gives ``init_tok_max_idx = 2`` as keeping indices 0, 1, 2, i.e.
    a = init_tok_max_idx + 1; SepCache's ``init_cache_size`` is that count.
  * the neighbouring window keeps key j for query i iff 0 <= i - j < n
    (the query itself included), so n = 1 means "self only".
  * the three kinds of kept keys are joined by OR, then intersected with
    the causal triangle (P1 "SepAttention", build_prefill_mask).
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def is_sep(ids: np.ndarray, sep_ids: Sequence[int]) -> np.ndarray:
    """Separator flag of each token: its id belongs to the separator id set.

    P1 "Separator Tokens" (the set depends on the tokenizer) and P1
    "SepAttention" (the mask builder first marks tokens whose id is in the
    separator list)."""
    return np.isin(np.asarray(ids), np.asarray(list(sep_ids), dtype=np.int64))


def sep_mask(flags: np.ndarray, a: int, n: int) -> np.ndarray:
    """The 0/1 mask M[i, j] of one sequence (bool, [S, S]).

    P2 §1.2: M[i, j] = 1 lets query i attend key j; 0 sends the score to -inf.
    Built in the order P1 "SepAttention" describes for build_prefill_mask:
    separator columns, then the initial columns, then the local triangular
    window band, all OR-ed together, then AND with the lower-triangular
    causal mask."""
    flags = np.asarray(flags, dtype=bool)
    S = flags.shape[0]
    keep = np.zeros((S, S), dtype=bool)
    keep[:, flags] = True                         # separator columns
    keep[:, :max(0, min(a, S))] = True            # initial columns
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    keep |= (i - j >= 0) & (i - j < n)            # local window band
    return keep & (j <= i)                        # causal


def mask_rows(flags: np.ndarray, a: int, n: int, rows: Sequence[int]) -> np.ndarray:
    """Rows ``rows`` of M (bool, [len(rows), S]) without building all of M.

    Same definition as ``sep_mask``, evaluated only on the requested rows."""
    flags = np.asarray(flags, dtype=bool)
    S = flags.shape[0]
    i = np.asarray(list(rows), dtype=np.int64)[:, None]
    j = np.arange(S)[None, :]
    keep = np.broadcast_to(flags[None, :], (i.shape[0], S)).copy()
    keep[:, :max(0, min(a, S))] = True
    keep |= (i - j >= 0) & (i - j < n)
    return keep & (j <= i)


def compact(flags: np.ndarray):
    """Prefix-sum stream compaction of the separator flags of one sequence.

    rank[j]    = number of separators at positions < j, for j = 0..S
                 (so rank[S] is the separator count);
    sep_pos[r] = position of the r-th separator (increasing), -1 past count.

    This is the index form of P1 "KV Cache Manager" (compress_past_win_2_seps
    keeps only the separator entries of a window, in order)."""
    flags = np.asarray(flags, dtype=bool)
    S = flags.shape[0]
    rank = np.zeros(S + 1, dtype=np.int64)
    rank[1:] = np.cumsum(flags)
    count = int(rank[S])
    sep_pos = np.full(S, -1, dtype=np.int64)
    sep_pos[:count] = np.flatnonzero(flags)
    return rank, sep_pos, count


def tile_class(M: np.ndarray, tq: int, tk: int) -> np.ndarray:
    """Class of each (tq x tk) block of M: 0 = no pair visible,
    1 = every pair visible, 2 = some visible and some not.

    The blocks are those of a block-sparse map of M, the role P1
    "Flex Attention Kernel" gives to create_block_mask. Edge blocks cover only
    the rows/columns that exist."""
    S_q, S_k = M.shape
    nq = -(-S_q // tq)
    nk = -(-S_k // tk)
    out = np.zeros((nq, nk), dtype=np.uint8)
    for qt in range(nq):
        for kt in range(nk):
            blk = M[qt * tq:(qt + 1) * tq, kt * tk:(kt + 1) * tk]
            if blk.all():
                out[qt, kt] = 1
            elif blk.any():
                out[qt, kt] = 2
    return out


def tile_class_slabs(flags: np.ndarray, a: int, n: int, tq: int, tk: int,
                     qtiles: Sequence[int] | None = None) -> np.ndarray:
    """``tile_class`` for long sequences: M is built one row-slab of tq rows
    at a time (``mask_rows``), never whole. Returns the rows ``qtiles`` of the
    class map (all rows by default)."""
    S = len(flags)
    nq = -(-S // tq)
    nk = -(-S // tk)
    qts = list(range(nq)) if qtiles is None else list(qtiles)
    out = np.zeros((len(qts), nk), dtype=np.uint8)
    full = (S // tk) * tk
    for r, qt in enumerate(qts):
        rows = range(qt * tq, min(S, (qt + 1) * tq))
        slab = mask_rows(flags, a, n, rows)
        if full:
            blocks = slab[:, :full].reshape(slab.shape[0], full // tk, tk)
            all_ = blocks.all(axis=(0, 2))
            any_ = blocks.any(axis=(0, 2))
            out[r, :full // tk] = np.where(all_, 1, np.where(any_, 2, 0))
        if full < S:                      # last, shorter key tile
            blk = slab[:, full:]
            out[r, nk - 1] = 1 if blk.all() else (2 if blk.any() else 0)
    return out
