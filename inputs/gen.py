"""Seeded synthetic inputs shared by the oracle and the GPU path.

Only random draws and number-format conversion live here; nothing of the
Sep-Attention method (no separator test, mask, attention or cache rule).

Every array is addressable on its own: each (config seed, sequence b, tensor
tag, head) triple seeds its own NumPy PCG64 stream, so a test can generate a
single sequence or a single head of a large workload without generating the
rest, and get the same values as a run that generated everything.

Floating-point inputs are drawn as N(0,1) in float64 and rounded once to the
workload's storage format: float32 (round-to-nearest-even), or bfloat16 by
round-to-nearest-even applied to the float32 bit pattern. bfloat16 data is
returned as ``uint16`` bit patterns; ``bf16_bits_to_f64`` widens them
exactly.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import Sequence

import numpy as np

TAG_IDS, TAG_Q, TAG_K, TAG_V, TAG_HK, TAG_HV, TAG_DO = 0, 1, 2, 3, 4, 5, 6   # TAG_DO: upstream gradient dL/dO


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.default_rng([int(seed)] + [int(k) for k in key])


# ---------------------------------------------------------------- formats
def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bfloat16 bits (RNE on the float32 pattern)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def round_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    if dtype == "f32":
        return x64.astype(np.float32)
    raise ValueError(dtype)


def storage_to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------- token ids
def _complement(sep_ids: Sequence[int], vocab: int) -> np.ndarray:
    mark = np.zeros(vocab, dtype=bool)
    mark[np.asarray([s for s in sep_ids if 0 <= s < vocab], dtype=np.int64)] = True
    return np.flatnonzero(~mark).astype(np.int32)


def ids_iid(rng: np.random.Generator, S: int, sep_ids: Sequence[int], vocab: int,
            p_sep: float) -> np.ndarray:
    """Per token: with probability p_sep an id drawn uniformly from the
    separator list, otherwise an id drawn uniformly from the rest of the
    vocabulary."""
    sep = np.asarray(sep_ids, dtype=np.int32)
    comp = _complement(sep_ids, vocab)
    u = rng.random(S)
    pick_sep = sep[rng.integers(0, len(sep), S)] if len(sep) else np.zeros(S, np.int32)
    pick_other = comp[rng.integers(0, len(comp), S)]
    return np.where(u < p_sep, pick_sep, pick_other).astype(np.int32)


def ids_runs(rng: np.random.Generator, S: int, sep_ids: Sequence[int], vocab: int,
             run_mean: float) -> np.ndarray:
    """Segments of length 1 + Poisson(run_mean - 1): each segment is
    (length - 1) non-separator ids followed by one separator id; the last
    segment is cut at S."""
    sep = np.asarray(sep_ids, dtype=np.int32)
    comp = _complement(sep_ids, vocab)
    n_seg = int(S / max(run_mean, 1.0) * 1.5) + 16
    lengths = 1 + rng.poisson(run_mean - 1.0, n_seg)
    while lengths.sum() < S:
        lengths = np.concatenate([lengths, 1 + rng.poisson(run_mean - 1.0, n_seg)])
    ends = np.cumsum(lengths) - 1
    ends = ends[ends < S]
    out = comp[rng.integers(0, len(comp), S)].astype(np.int32)
    out[ends] = sep[rng.integers(0, len(sep), len(ends))]
    return out


def prefill_ids(cfg, b: int) -> np.ndarray:
    rng = _rng(cfg.seed, b, TAG_IDS)
    if cfg.id_mode == "iid":
        return ids_iid(rng, cfg.S, cfg.sep_ids, cfg.vocab, cfg.p_sep)
    if cfg.id_mode == "runs":
        return ids_runs(rng, cfg.S, cfg.sep_ids, cfg.vocab, cfg.run_mean)
    raise ValueError(cfg.id_mode)


# ---------------------------------------------------------------- tensors
BLOCK_ROWS = 16384


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_rows(seed: int, key: Sequence[int], rows: int, D: int, dtype: str) -> np.ndarray:
    """rows x D values ~ N(0,1) in float64, rounded once to the storage dtype.

    Rows come in blocks of BLOCK_ROWS; block j is drawn from its own stream
    seeded by (seed, *key, j), so blocks are generated in parallel threads
    and the result does not depend on the thread count."""
    st = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((rows, D), dtype=st)
    nblk = -(-rows // BLOCK_ROWS)

    def fill(j):
        r0 = j * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        x = _rng(seed, *key, j).standard_normal((r1 - r0, D))
        out[r0:r1] = round_storage(x, dtype)

    if nblk <= 1:
        for j in range(nblk):
            fill(j)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def prefill_head(cfg, b: int, tag: int, h: int) -> np.ndarray:
    """One head of Q (tag TAG_Q), K/V (TAG_K/TAG_V) or the upstream gradient
    dL/dO (TAG_DO): [S, D] in storage format."""
    return normal_rows(cfg.seed, (b, tag, h), cfg.S, cfg.D, cfg.dtype)


def prefill_inputs(cfg, batches: Sequence[int] | None = None, heads_q: Sequence[int] | None = None):
    """ids [B,S] int32, q [B,Hq,S,D], k/v [B,Hkv,S,D] in storage format."""
    bs = list(range(cfg.B)) if batches is None else list(batches)
    hq = list(range(cfg.Hq)) if heads_q is None else list(heads_q)
    st = np.uint16 if cfg.dtype == "bf16" else np.float32
    ids = np.stack([prefill_ids(cfg, b) for b in bs])
    q = np.empty((len(bs), len(hq), cfg.S, cfg.D), st)
    k = np.empty((len(bs), cfg.Hkv, cfg.S, cfg.D), st)
    v = np.empty_like(k)
    for i, b in enumerate(bs):
        for j, h in enumerate(hq):
            q[i, j] = prefill_head(cfg, b, TAG_Q, h)
        for g in range(cfg.Hkv):
            k[i, g] = prefill_head(cfg, b, TAG_K, g)
            v[i, g] = prefill_head(cfg, b, TAG_V, g)
    return {"ids": ids, "q": q, "k": k, "v": v}


# ---------------------------------------------------------------- streams
def stream_ids(cfg, b: int, length: int | None = None) -> np.ndarray:
    """Token ids of sequence b: history followed by the decode steps."""
    total = cfg.history + cfg.steps if length is None else length
    return ids_iid(_rng(cfg.seed, b, TAG_IDS), total, cfg.sep_ids, cfg.vocab, cfg.p_sep)


def stream_pool(cfg, b: int, pool: int | None = None):
    """Per-step rows of sequence b: q [pool,Hq,D], k/v [pool,Hkv,D]."""
    P = cfg.pool if pool is None else pool
    q = normal_rows(cfg.seed, (b, TAG_Q), P * cfg.Hq, cfg.D, cfg.dtype).reshape(P, cfg.Hq, cfg.D)
    k = normal_rows(cfg.seed, (b, TAG_K), P * cfg.Hkv, cfg.D, cfg.dtype).reshape(P, cfg.Hkv, cfg.D)
    v = normal_rows(cfg.seed, (b, TAG_V), P * cfg.Hkv, cfg.D, cfg.dtype).reshape(P, cfg.Hkv, cfg.D)
    return q, k, v


def history_kv(cfg, b: int):
    """History K/V of sequence b: [Hkv, history, D] each, storage format."""
    k = np.stack([normal_rows(cfg.seed, (b, TAG_HK, g), cfg.history, cfg.D, cfg.dtype)
                  for g in range(cfg.Hkv)])
    v = np.stack([normal_rows(cfg.seed, (b, TAG_HV, g), cfg.history, cfg.D, cfg.dtype)
                  for g in range(cfg.Hkv)])
    return k, v


# ---------------------------------------------------------------- on the device
def device_normal(shape, seed: int, tag: int, dtype: str = "bf16", device="cuda"):
    """A [shape] tensor ~ N(0,1) drawn on the GPU by torch's generator seeded
    with (seed, tag), rounded once to the storage dtype (bf16: torch's
    round-to-nearest-even from float32). For large workloads whose host draw
    would take minutes; tests copy back the rows the oracle reads. Same
    distribution as ``normal_rows``, not the same values."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(tag))
    x = torch.randn(tuple(shape), generator=g, device=device)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "f32":
        return x
    raise ValueError(dtype)

