"""GPU parity of sep_attn_prefill_chunk against oracle.chunk_attention.

A cache is filled from a seeded stream (bulk sep_cache_update), mirrored by
oracle.CacheSim; the next C tokens of the stream form the chunk. Every
output element is compared with the oracle's attention over the retained
entries plus the chunk under the window n, within the bf16 tolerance, and
the log-sum-exp within the bf16 prefill's lse tolerance. Cases cover every
cache policy, a cache still filling its initial block, StreamingLLM mode,
chunks of 1 to 1030 tokens (several query tiles, ragged tails), windows of
1 to past the whole cache, GQA 1/2/4/8 and D = 64 / 128. Chunks are chained
(attend, then insert with sep_cache_update, then the next chunk), one token
with a wide window equals sep_attn_decode, and two windows on one cache
(a model's layers) each match the oracle.
"""
import ctypes
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from kv_cache_compression_sep_amd import (SEP_POLICY_DYNAMIC, SEP_POLICY_NO_ACCUM, SepCache, _lib,
                                          chunk_workspace_bytes, sep_attn_decode, sep_attn_prefill_chunk)

from .gpu_util import check_close, from_dev, guarded_empty, to_dev
from .test_gpu_cache_decode import SEP_IDS, Stream, sim_for

pytestmark = pytest.mark.gpu
LSE_TOL = 4e-3   # the forward's bf16 bound: test_gpu_prefill.py


def chunk_inputs(st, t0, t1):
    q = to_dev(np.ascontiguousarray(st.q[:, t0:t1].transpose(0, 2, 1, 3)), "bf16")     # [B, Hq, C, D]
    k = to_dev(np.ascontiguousarray(st.k[:, :, t0:t1]), "bf16")
    v = to_dev(np.ascontiguousarray(st.v[:, :, t0:t1]), "bf16")
    ids = to_dev(np.ascontiguousarray(st.ids[:, t0:t1]))
    return q, k, v, ids


def oracle_chunk(st, sim, b, t0, t1, a, n, scale):
    entries = [oracle.Entry(e.pos, e.tok, gen.bf16_bits_to_f64(st.k[b][:, e.pos]),
                            gen.bf16_bits_to_f64(st.v[b][:, e.pos])) for e in sim.keys()]
    q = gen.bf16_bits_to_f64(st.q[b, t0:t1].transpose(1, 0, 2))
    k = gen.bf16_bits_to_f64(st.k[b][:, t0:t1])
    v = gen.bf16_bits_to_f64(st.v[b][:, t0:t1])
    return oracle.chunk_attention(entries, q, k, v, st.ids[b, t0:t1], t0, a, n, SEP_IDS, scale)


def check_chunk(st, cache, sims, t0, t1, n, d_sep, tag):
    a = cache.a
    scale = 1.0 / math.sqrt(st.D)
    q, k, v, ids = chunk_inputs(st, t0, t1)
    B, Hq, C, D = q.shape
    ws = guarded_empty((chunk_workspace_bytes(cache, C),), torch.uint8)
    out, lse = sep_attn_prefill_chunk(q, k, v, ids, cache, d_sep, n, scale, return_lse=True, workspace=ws,
                                      out=guarded_empty((B, Hq, C, D), torch.bfloat16),
                                      lse=guarded_empty((B, Hq, C), torch.float32))
    o = from_dev(out)
    l_gpu = from_dev(lse)
    for b in range(st.B):
        o_ref, l_ref = oracle_chunk(st, sims[b], b, t0, t1, a, n, scale)
        check_close(o[b], o_ref, "bf16", f"{tag} b={b}")
        assert np.max(np.abs(l_gpu[b] - l_ref)) < LSE_TOL, tag
    return k, v, ids


CASES = [
    # B, Hq, Hkv, D,  a, s,  p,  w,   T,   C,    n,   policy
    (2, 32, 8, 128, 4, 64, 64, 256, 900, 300, 256, 0),
    (1, 8, 2, 128, 4, 64, 64, 256, 900, 1030, 64, 0),
    (2, 8, 8, 64, 2, 5, 3, 11, 90, 37, 5, 0),
    (1, 16, 2, 128, 4, 20, 8, 40, 3, 50, 16, 0),           # cache still filling the initial block
    (1, 4, 1, 128, 4, 0, 0, 50, 200, 64, 30, 0),           # StreamingLLM mode
    (2, 16, 4, 128, 4, 64, 16, 96, 700, 129, 100, SEP_POLICY_DYNAMIC),
    (1, 8, 1, 64, 2, 9, 5, 20, 300, 200, 7, SEP_POLICY_DYNAMIC | SEP_POLICY_NO_ACCUM),
    (1, 6, 3, 64, 3, 32, 16, 64, 400, 257, 1, SEP_POLICY_NO_ACCUM),   # window 1
    (1, 8, 2, 128, 4, 64, 32, 128, 500, 96, 100000, 0),    # window past the whole cache
    (1, 8, 8, 128, 4, 64, 64, 256, 0, 300, 256, 0),        # empty cache: plain prefill of the chunk
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_chunk_matches_oracle(case):
    B, Hq, Hkv, D, a, s, p, w, T, C, n, policy = case
    print(f"chunk case {case}", flush=True)
    st = Stream(zlib.crc32(repr(("chunk", case)).encode()), B, Hq, Hkv, D, T + C, 0.12)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    cache = SepCache(B, Hkv, D, a, s, p, w, policy=policy)
    sims = [sim_for((a, s, p, w), policy) for _ in range(B)]
    if T > 0:
        st.push_gpu(cache, 0, T, d_sep)
        for b in range(B):
            sims[b].push_many([oracle.Entry(x, int(st.ids[b, x])) for x in range(T)])
    check_chunk(st, cache, sims, T, T + C, n, d_sep, str(case))


def test_chained_chunks_with_cache_updates():
    """Attend, insert, attend the next chunk: a prompt streamed into the cache
    in chunks of uneven length."""
    B, Hq, Hkv, D, a, s, p, w = 2, 16, 4, 128, 4, 32, 16, 64
    bounds = [0, 100, 161, 400, 401, 700]
    st = Stream(4242, B, Hq, Hkv, D, bounds[-1], 0.15)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    cache = SepCache(B, Hkv, D, a, s, p, w)
    sims = [sim_for((a, s, p, w), 0) for _ in range(B)]
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        k, v, ids = check_chunk(st, cache, sims, t0, t1, 48, d_sep, f"chunk {t0}..{t1}")
        from kv_cache_compression_sep_amd import sep_cache_update
        sep_cache_update(cache, k, v, ids, d_sep)
        for b in range(B):
            sims[b].push_many([oracle.Entry(x, int(st.ids[b, x])) for x in range(t0, t1)])


def test_one_token_with_a_wide_window_is_decode():
    B, Hq, Hkv, D, a, s, p, w, T = 2, 32, 8, 128, 4, 64, 64, 256, 1000
    st = Stream(77, B, Hq, Hkv, D, T + 1, 0.12)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    cache = SepCache(B, Hkv, D, a, s, p, w)
    st.push_gpu(cache, 0, T, d_sep)
    q, k, v, ids = chunk_inputs(st, T, T + 1)
    oc = sep_attn_prefill_chunk(q, k, v, ids, cache, d_sep, cache.slots + 1)
    od = sep_attn_decode(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(), cache)
    torch.cuda.synchronize()
    check_close(from_dev(oc)[:, :, 0], from_dev(od).astype(np.float64), "bf16", "chunk of one vs decode")


def test_layer_windows_on_one_cache():
    """Two layers with their own windows read the same cache."""
    B, Hq, Hkv, D, a, s, p, w, T, C = 1, 8, 2, 128, 4, 64, 64, 256, 800, 200
    st = Stream(78, B, Hq, Hkv, D, T + C, 0.12)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    cache = SepCache(B, Hkv, D, a, s, p, w)
    sims = [sim_for((a, s, p, w), 0)]
    st.push_gpu(cache, 0, T, d_sep)
    sims[0].push_many([oracle.Entry(x, int(st.ids[0, x])) for x in range(T)])
    outs = []
    for n in (32, 300):
        check_chunk(st, cache, sims, T, T + C, n, d_sep, f"layer window {n}")
        q, k, v, ids = chunk_inputs(st, T, T + C)
        outs.append(from_dev(sep_attn_prefill_chunk(q, k, v, ids, cache, d_sep, n)))
    assert np.max(np.abs(outs[0] - outs[1])) > 0.05


def test_chunk_rejects_a_small_workspace():
    cache = SepCache(1, 2, 128, 4, 16, 8, 32)
    C = 10
    q = torch.zeros((1, 8, C, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 2, C, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((1, C), dtype=torch.int32, device="cuda")
    sep = torch.zeros((1,), dtype=torch.int32, device="cuda")
    need = chunk_workspace_bytes(cache, C)
    ws = torch.empty((need - 256,), dtype=torch.uint8, device="cuda")
    # the binding refuses it before any C call ...
    with pytest.raises(ValueError):
        sep_attn_prefill_chunk(q, kv, kv, ids, cache, sep, 8, workspace=ws)
    # ... and so does the C entry point, which launches nothing then
    out = torch.empty_like(q)
    st = cache.struct()
    code = _lib.load().sep_attn_prefill_chunk(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), ids.data_ptr(), C,
                                              sep.data_ptr(), 1, ctypes.byref(st), 8, 8, 0.088, ws.data_ptr(),
                                              need - 256, out.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert code == _lib.SEP_ERR_WORKSPACE
