"""List-based simulation of SepLLM's four-block KV cache, and its closed form.

Test infrastructure only (see the package docstring for who may import it).

The blocks (P2 §1.3; P3 §3.3 table; P1 "SepCache" parameter names):
  I  initial cache    the first ``a`` tokens, never evicted (P3 §3.3: fixed);
  S  separator cache  separators saved from the past window, at most ``s``,
                      oldest evicted first (P3 §3.3; P1 "KV Cache Manager":
                      keep the last sep_cache_size separators);
  R  = P ++ L         the past window P followed by the local window L, one
                      contiguous run of the most recent tokens; the local
                      window overflows into the past window (P3 §3.3).

Reading of when the past window is compacted (the pages leave it open; P1
"KV Cache Manager" compresses once the cache exceeds its size, P3 §3.3
compresses the past window once it is full): every block has a fixed cap.
When pushing a token would make |R| = p + w + 1, the oldest p + 1 entries of
R are taken out; in order, each separator among them is appended to S (and S
drops its oldest entry while |S| > s); the non-separators are discarded.
Both SEP_ACCUMULATION and USE_MAX_SEP_CACHE are on, as in the SepLLM branch
of P1 "Streaming-SepLLM". With s = 0 and p = 0 the same rule keeps only
initial + local tokens: the StreamingLLM baseline of P1 "Streaming-SepLLM".

Policy variants (P1 "KV Cache Manager", the compression pseudo-code):
  dynamic=True     the trigger of that pseudo-code: compress as soon as the
                   whole cache (I + S + R, after the push) holds more than
                   c = a + s + p + w entries. The past window is then R
                   without its last w entries, so while S is not full R
                   grows past p + w. With S full this is the fixed rule.
  accumulate=False SEP_ACCUMULATION off: S becomes the separators of the
                   compressed past window alone (then capped to its last s).
In both rules a compression takes R minus its last w entries (in the fixed
rule that is exactly the oldest p + 1). USE_MAX_SEP_CACHE = False (an
unbounded S) has no fixed-size form and is not modelled.

Order within one streaming step (P1 "Streaming-SepLLM" evaluation loop:
forward with the cache, then update ids, then compress): the decode
attention of token t reads I ++ S ++ R (the state after tokens 0..t-1) plus
token t itself; the update then pushes t.
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass
from typing import Any, List, Sequence

import numpy as np


def check_cache_params(a: int, s: int, p: int, w: int) -> None:
    """The parameter contract of P1 "Streaming 参数约束", restated with
    c = a + s + p + w: cache_size > 0, init >= 0, local > 0,
    cache >= init + local; for SepLLM also sep > 0 and init + sep + local <
    cache (i.e. p >= 1); for StreamingLLM local == cache - init (s = p = 0)."""
    if a < 0 or w <= 0 or s < 0 or p < 0:
        raise ValueError("need a >= 0, w > 0, s >= 0, p >= 0")
    sepllm = s > 0 and p > 0
    streaming = s == 0 and p == 0
    if not (sepllm or streaming):
        raise ValueError("either s > 0 and p > 0 (SepLLM) or s = p = 0 (StreamingLLM)")


@dataclass
class Entry:
    pos: int
    tok: int
    k: Any = None      # [Hkv, D] rows of this token, or None when only ids matter
    v: Any = None


class CacheSim:
    """The four blocks as Python lists, one token at a time."""

    def __init__(self, a: int, s: int, p: int, w: int, sep_ids: Sequence[int],
                 dynamic: bool = False, accumulate: bool = True):
        check_cache_params(a, s, p, w)
        self.a, self.s, self.p, self.w = a, s, p, w
        self.c = a + s + p + w
        self.dynamic, self.accumulate = dynamic, accumulate
        self.sep_set = set(int(x) for x in sep_ids)
        self.I: List[Entry] = []
        self.S: deque = deque()
        self.R: deque = deque()
        self.t = 0
        self.compactions = 0
        self.compacted = 0          # entries taken out of R so far (= cend - a)

    def push(self, e: Entry) -> None:
        """Insert the next token of the stream (its position must be t)."""
        assert e.pos == self.t
        self.t += 1
        if len(self.I) < self.a:
            self.I.append(e)
            return
        self.R.append(e)
        if self.dynamic:
            due = len(self.I) + len(self.S) + len(self.R) > self.c
        else:
            due = len(self.R) > self.p + self.w
        if due:
            batch = [self.R.popleft() for _ in range(len(self.R) - self.w)]
            if not self.accumulate:
                self.S.clear()
            for x in batch:
                if x.tok in self.sep_set:
                    self.S.append(x)
                    if len(self.S) > self.s:
                        self.S.popleft()
            self.compactions += 1
            self.compacted += len(batch)

    def push_many(self, entries: Sequence[Entry]) -> None:
        """A bulk insert is the same as inserting the tokens one by one."""
        for e in entries:
            self.push(e)

    def keys(self) -> List[Entry]:
        """Retained entries in block order I, S, R (each oldest first)."""
        return list(self.I) + list(self.S) + list(self.R)

    def occupancy(self) -> int:
        return len(self.I) + len(self.S) + len(self.R)

    def positions(self):
        return ([e.pos for e in self.I], [e.pos for e in self.S], [e.pos for e in self.R])


def n_compactions(t: int, a: int, p: int, w: int) -> int:
    """Number of compactions after tokens 0..t-1: each one happens when the
    (p + w + 1)-th entry enters R, and leaves w entries behind."""
    m = t - a
    if m <= 0:
        return 0
    return max(0, (m - w) // (p + 1))


def closed_form_positions(flags: np.ndarray, t: int, a: int, s: int, p: int, w: int):
    """Positions held by I, S, R after tokens 0..t-1, without simulating.

    With m = t - a and K compactions, the compacted prefix is [a, cend) with
    cend = a + K (p + 1); S is the last s separators in it, R = [cend, t)."""
    if t - a <= 0:
        return list(range(t)), [], []
    K = n_compactions(t, a, p, w)
    cend = a + K * (p + 1)
    seps = [x for x in range(a, cend) if flags[x]]
    S = seps[max(0, len(seps) - s):] if s > 0 else []
    return list(range(a)), S, list(range(cend, t))


def policy_positions(flags: np.ndarray, t: int, a: int, s: int, p: int, w: int,
                     dynamic: bool = False, accumulate: bool = True):
    """Positions held by I, S, R after tokens 0..t-1, from the compression
    points alone (no per-token lists).

    R is always [cend, t). Pushing position x makes the cache hold
    a + |S| + (x + 1 - cend) entries, so the next compression is at
    x = cend + c - a - |S| (dynamic: the whole cache exceeds c) or at
    x = cend + p + w (fixed: R exceeds p + w); it moves cend to x + 1 - w
    and sets S from the separators in the old [cend, x + 1 - w)."""
    if t <= a:
        return list(range(t)), [], []
    c = a + s + p + w
    cend, S = a, []
    while True:
        x = cend + (c - a - len(S) if dynamic else p + w)
        if x >= t:
            break
        new_cend = x + 1 - w
        batch = [z for z in range(cend, new_cend) if flags[z]]
        S = S + batch if accumulate else batch
        S = S[len(S) - s:] if len(S) > s else S
        cend = new_cend
    return list(range(a)), S, list(range(cend, t))
