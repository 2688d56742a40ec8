"""sep_attn_prefill_backward_noalloc (its per-row workspace in a fixed array
of the library) against sep_attn_prefill_backward (the caller's workspace),
through the C ABI, on two calls in a row, the second with a smaller input
than the first, then the first shape again.

dq and the dK/dV of window keys are written without atomics, so they must be
bit-identical to the existing entry point's; the dK/dV of initial and
separator keys are summed with fp32 atomics in a varying order, so there the
two results must agree within the derived error bound of the backward's
parity tests, and both must be within that bound of the fp64 oracle.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from kv_cache_compression_sep_amd import (sep_attn_prefill, sep_attn_prefill_backward,
                                          sep_attn_prefill_backward_noalloc, sep_index_compact, sep_mask_build)

from .gpu_util import from_dev, guarded_empty, to_dev
from .test_gpu_prefill_backward import LSE_TOL, OPERAND_ROUNDING, U32, check_bound, grad_bounds

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, S,   D,   a, n,  p_sep, dtype
    (2, 8, 2, 300, 128, 4, 32, 0.15, "bf16"),
    (1, 4, 1, 77, 64, 2, 9, 0.3, "bf16"),          # smaller than the first
    (2, 8, 2, 300, 128, 4, 32, 0.15, "bf16"),      # the first shape again, after a smaller call
    (1, 6, 3, 150, 64, 3, 20, 0.2, "f32"),
]


def _inputs(case):
    B, Hq, Hkv, S, D, a, n, p, dtype = case
    rng = np.random.default_rng(zlib.crc32(repr(("noalloc", case)).encode()))
    ids = np.where(rng.random((B, S)) < p, rng.integers(0, 8, (B, S)), rng.integers(8, 1000, (B, S))).astype(np.int32)
    x = [gen.round_storage(rng.standard_normal(shape), dtype) for shape in
         ((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D), (B, Hq, S, D))]
    return ids, x


def test_noalloc_backward_equals_the_workspace_entry_point():
    for case in CASES:
        B, Hq, Hkv, S, D, a, n, p, dtype = case
        print(f"noalloc backward case {case}", flush=True)
        ids, (q, k, v, dout) = _inputs(case)
        flags, _, _ = sep_mask_build(to_dev(ids), to_dev(np.arange(8, dtype=np.int32)), a, n)
        rank, sep_pos, _ = sep_index_compact(flags)
        tq, tk, tv, tdo = (to_dev(x, dtype) for x in (q, k, v, dout))
        scale = 1.0 / math.sqrt(D)
        out, lse = sep_attn_prefill(tq, tk, tv, flags, rank, sep_pos, a, n, scale, return_lse=True)
        f32 = torch.float32
        ref = sep_attn_prefill_backward(tq, tk, tv, out, tdo, lse, flags, rank, sep_pos, a, n, scale)
        got = sep_attn_prefill_backward_noalloc(tq, tk, tv, out, tdo, lse, flags, rank, sep_pos, a, n, scale,
                                                guarded_empty((B, Hq, S, D), f32), guarded_empty((B, Hkv, S, D), f32),
                                                guarded_empty((B, Hkv, S, D), f32))
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]), (case, "dq differs from sep_attn_prefill_backward")
        out_h = from_dev(out)
        G = Hq // Hkv
        eps = math.expm1(LSE_TOL[dtype]) + OPERAND_ROUNDING[dtype] + 8 * U32
        gamma = (D + G * S) * U32 / (1 - (D + G * S) * U32)
        for b in range(B):
            f = [gen.storage_to_f64(x[b], dtype) for x in (q, k, v, dout)]
            f_sep = oracle.is_sep(ids[b], list(range(8)))
            M = oracle.sep_mask(f_sep, a, n)
            glob = np.flatnonzero(f_sep | (np.arange(S) < a))
            win = np.setdiff1d(np.arange(S), glob)
            rq, rk, rv, _ = oracle.attention_backward(f[0], f[1], f[2], M, scale, f[3], out=out_h[b])
            bq, bk, bv, _ = grad_bounds(f[0], f[1], f[2], out_h[b], f[3], M, scale)
            for name, gg, rr, bb, rf in (("dk", got[1], ref[1], bk, rk), ("dv", got[2], ref[2], bv, rv)):
                gb, rb = from_dev(gg[b]), from_dev(rr[b])
                assert np.array_equal(gb[:, win], rb[:, win]), (case, b, name, "window keys differ")
                check_bound(gb, rb, bb, 2 * (eps + gamma), f"{case} b={b} {name} vs sep_attn_prefill_backward")
                check_bound(gb, rf, bb, eps + gamma, f"{case} b={b} {name} vs oracle")
            check_bound(from_dev(got[0][b]), rq, bq, eps + gamma, f"{case} b={b} dq vs oracle")

