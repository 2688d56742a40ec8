"""GPU parity of sep_mask_build and sep_index_compact against the oracle.

Integer outputs must match bit for bit: separator flags, tile classes, the
dense mask, ranks, compacted positions and counts. Cases: the three prefill
workloads at full size (1 x 512, 1 x 8192, 1 x 131072 tokens) plus small and
ragged shapes, all-separator, no-separator and single-token sequences.
sep_mask_compact (flags and compaction in one launch) must write exactly
the same four arrays.
"""
import numpy as np
import pytest
import torch

import oracle
from inputs import configs, gen
from kv_cache_compression_sep_amd import sep_index_compact, sep_mask_build, sep_mask_compact

from .gpu_util import guarded_empty, to_dev

pytestmark = pytest.mark.gpu


def _ids_for(cfg):
    return np.stack([gen.prefill_ids(cfg, b) for b in range(cfg.B)])


def _small_cases():
    rng = np.random.default_rng(501)
    cases = []
    for S in (1, 2, 3, 5, 63, 64, 65, 127, 300, 1000, 4097):
        for p in (0.0, 0.1, 1.0):
            B = int(rng.integers(1, 4))
            ids = np.where(rng.random((B, S)) < p, rng.integers(0, 8, (B, S)),
                           rng.integers(8, 1000, (B, S))).astype(np.int32)
            a = int(rng.integers(0, 9))
            n = int(rng.integers(1, S + 6))
            cases.append((ids, a, n))
    return cases


def _check_flags_tiles_compact(ids, sep_ids, a, n, tiles=((64, 64), (32, 64), (16, 48)),
                               dense=None, qtile_sample=None):
    B, S = ids.shape
    d_ids = to_dev(ids)
    d_sep = to_dev(np.asarray(sep_ids, np.int32))
    want_dense = dense if dense is not None else S <= 2048
    for tq, tk in tiles:
        flags, tc, dm = sep_mask_build(
            d_ids, d_sep, a, n, tiles=(tq, tk), is_sep=guarded_empty((B, S), torch.uint8),
            tile_class=guarded_empty((B, -(-S // tq), -(-S // tk)), torch.uint8),
            dense_mask=guarded_empty((B, S, S), torch.uint8) if want_dense else None)
        torch.cuda.synchronize()
        flags_h = flags.cpu().numpy()
        tc_h = tc.cpu().numpy()
        for b in range(B):
            f_ref = oracle.is_sep(ids[b], sep_ids)
            assert np.array_equal(flags_h[b], f_ref.astype(np.uint8))
            qts = qtile_sample if qtile_sample is not None else None
            tc_ref = oracle.tile_class_slabs(f_ref, a, n, tq, tk, qts)
            got = tc_h[b] if qts is None else tc_h[b][qts]
            assert np.array_equal(got, tc_ref), (b, tq, tk)
            if want_dense:
                M = oracle.sep_mask(f_ref, a, n)
                assert np.array_equal(dm[b].cpu().numpy(), M.astype(np.uint8))
    rank, sep_pos, count = sep_index_compact(flags, rank=guarded_empty((B, S + 1), torch.int32),
                                             sep_pos=guarded_empty((B, S), torch.int32),
                                             count=guarded_empty((B,), torch.int32))
    torch.cuda.synchronize()
    rank_h, pos_h, cnt_h = rank.cpu().numpy(), sep_pos.cpu().numpy(), count.cpu().numpy()
    for b in range(B):
        r_ref, p_ref, c_ref = oracle.compact(oracle.is_sep(ids[b], sep_ids))
        assert np.array_equal(rank_h[b], r_ref)
        assert np.array_equal(pos_h[b], p_ref)
        assert cnt_h[b] == c_ref


def test_small_and_ragged_shapes():
    for ids, a, n in _small_cases():
        _check_flags_tiles_compact(ids, list(range(8)), a, n)


def test_empty_separator_set_and_duplicates():
    rng = np.random.default_rng(503)
    ids = rng.integers(0, 20, (2, 333)).astype(np.int32)
    _check_flags_tiles_compact(ids, [], 3, 7)
    _check_flags_tiles_compact(ids, [5, 5, 5, 7], 3, 7)
    _check_flags_tiles_compact(ids, list(range(64)), 0, 1)


def test_tiny_prefill_workload_full():
    cfg = configs.TINY_PREFILL
    _check_flags_tiles_compact(_ids_for(cfg), cfg.sep_ids, cfg.a, cfg.n, dense=True)


def test_llama3_layer_workload_full():
    cfg = configs.LLAMA3_LAYER_PREFILL
    _check_flags_tiles_compact(_ids_for(cfg), cfg.sep_ids, cfg.a, cfg.n, tiles=((64, 64),),
                               dense=True)


def test_long_prefill_workload_flags_ranks_sampled_tiles():
    cfg = configs.LONG_PREFILL
    nqt = cfg.S // 64
    rng = np.random.default_rng(505)
    sample = sorted(set([0, 1, 2, 3, nqt - 2, nqt - 1] + rng.integers(0, nqt, 24).tolist()))
    _check_flags_tiles_compact(_ids_for(cfg), cfg.sep_ids, cfg.a, cfg.n, tiles=((64, 64),),
                               dense=False, qtile_sample=sample)


def _check_fused(ids, sep_ids):
    B, S = ids.shape
    flags, rank, sep_pos, count = sep_mask_compact(
        to_dev(ids), to_dev(np.asarray(sep_ids, np.int32)), is_sep=guarded_empty((B, S), torch.uint8),
        rank=guarded_empty((B, S + 1), torch.int32), sep_pos=guarded_empty((B, S), torch.int32),
        count=guarded_empty((B,), torch.int32))
    torch.cuda.synchronize()
    f_h, r_h, p_h, c_h = flags.cpu().numpy(), rank.cpu().numpy(), sep_pos.cpu().numpy(), count.cpu().numpy()
    for b in range(B):
        f_ref = oracle.is_sep(ids[b], sep_ids)
        r_ref, p_ref, c_ref = oracle.compact(f_ref)
        assert np.array_equal(f_h[b], f_ref.astype(np.uint8)), (S, b)
        assert np.array_equal(r_h[b], r_ref), (S, b)
        assert np.array_equal(p_h[b], p_ref), (S, b)
        assert c_h[b] == c_ref


def test_fused_mask_compact_small_and_ragged():
    """Rows of S % 4 != 0 (scalar path), S % 4 == 0 with rank rows that are
    or are not 16-byte aligned (B > 1), more than one 4096-flag chunk."""
    for ids, _, _ in _small_cases():
        _check_fused(ids, list(range(8)))
    rng = np.random.default_rng(507)
    for B, S in ((3, 8), (2, 4096), (4, 12288), (3, 4100)):
        ids = np.where(rng.random((B, S)) < 0.2, rng.integers(0, 8, (B, S)),
                       rng.integers(8, 1000, (B, S))).astype(np.int32)
        _check_fused(ids, list(range(8)))
    _check_fused(rng.integers(0, 20, (2, 333)).astype(np.int32), [])


def test_fused_mask_compact_workloads():
    for cfg in (configs.LLAMA3_LAYER_PREFILL, configs.LONG_PREFILL):
        _check_fused(_ids_for(cfg), cfg.sep_ids)
