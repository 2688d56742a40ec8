"""GPU parity of sep_decode_update (decode, then the single-token update, in
one call) against the oracle and against the two calls it stands for.

Every step must give the outputs of sep_attn_decode (or sep_attn_decode_rope)
followed by sep_cache_update bit for bit, and leave the cache (K/V, pos, tok
and state words) bit for bit as those calls do; state word 7, the arrival
count of the fused launch, must read 0 between calls. The cache is also
checked against the list-based simulation and the decode outputs against
fp64 attention over the retained keys plus the current token (bf16
tolerance), every few steps. Cases cover the split lists (B * Hkv <= 64
with a work buffer), the fused whole-list launch (B * Hkv < 256 otherwise)
across cache policies, StreamingLLM mode, D = 64 / 128, GQA 1..8, with and
without RoPE position shifting, compressions at many steps, and the
two-launch fallback (B * Hkv >= 256).
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from inputs import gen
from kv_cache_compression_sep_amd import (SEP_POLICY_DYNAMIC, SEP_POLICY_NO_ACCUM, SepCache, sep_attn_decode,
                                          sep_attn_decode_rope, sep_cache_update, sep_decode_update,
                                          sep_rope_table)

from .gpu_util import check_close, from_dev, guarded_cache, guarded_empty, to_dev
from .test_gpu_cache_decode import SEP_IDS, Stream, check_cache, sim_for

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, D,  a, s,  p,  w,   T0, steps, policy, rope
    (1, 32, 8, 128, 4, 64, 64, 256, 300, 160, 0, False),
    (1, 32, 8, 128, 4, 64, 64, 256, 380, 70, 0, True),
    (2, 16, 4, 128, 4, 6, 5, 9, 20, 60, 0, False),           # a compression every 6 steps
    (3, 8, 8, 64, 2, 3, 2, 4, 3, 40, SEP_POLICY_DYNAMIC, False),
    (1, 12, 3, 64, 0, 5, 3, 7, 0, 50, SEP_POLICY_NO_ACCUM, True),
    (2, 8, 1, 128, 1, 4, 6, 5, 10, 50, SEP_POLICY_DYNAMIC | SEP_POLICY_NO_ACCUM, False),
    (1, 4, 2, 128, 4, 0, 0, 12, 5, 40, 0, False),            # StreamingLLM mode
    (8, 16, 8, 64, 4, 6, 5, 9, 30, 30, 0, False),            # B * Hkv = 64: the largest split
    (12, 16, 8, 64, 4, 6, 5, 9, 30, 30, 0, False),           # B * Hkv = 96: whole lists even with a work buffer
    (40, 16, 8, 64, 4, 6, 5, 9, 30, 30, 0, False),           # B * Hkv = 320: the two launches
]


@pytest.mark.parametrize("split", [True, False], ids=["split", "whole"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fused_step_equals_two_calls_and_oracle(case, split):
    B, Hq, Hkv, D, a, s, p, w, T0, steps, policy, rope = case
    print(f"decode+update case {case} split={split}", flush=True)
    st = Stream(zlib.crc32(repr(("fused", case)).encode()), B, Hq, Hkv, D, T0 + steps, 0.25)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    fused = guarded_cache(B, Hkv, D, a, s, p, w, policy=policy, split=split)
    plain = guarded_cache(B, Hkv, D, a, s, p, w, policy=policy, split=split)
    assert (fused.work is not None) == (split and B * Hkv <= 64)
    sims = [sim_for((a, s, p, w), policy) for _ in range(B)]
    if T0 > 0:
        st.push_gpu(fused, 0, T0, d_sep)
        st.push_gpu(plain, 0, T0, d_sep)
        for b in range(B):
            sims[b].push_many([oracle.Entry(t, int(st.ids[b, t])) for t in range(T0)])
    table = sep_rope_table(500000.0, D, fused.slots + 1) if rope else None
    scale = 1.0 / math.sqrt(D)
    for t in range(T0, T0 + steps):
        q = to_dev(np.ascontiguousarray(st.q[:, t]), "bf16")
        kn = to_dev(np.ascontiguousarray(st.k[:, :, t]), "bf16")
        vn = to_dev(np.ascontiguousarray(st.v[:, :, t]), "bf16")
        ids = to_dev(np.ascontiguousarray(st.ids[:, t]))
        of, lf = sep_decode_update(q, kn, vn, ids, fused, d_sep, scale, rope=table, return_lse=True,
                                   out=guarded_empty((B, Hq, D), torch.bfloat16),
                                   lse=guarded_empty((B, Hq), torch.float32))
        if rope:
            op, lp = sep_attn_decode_rope(q, kn, vn, plain, table, scale, return_lse=True)
        else:
            op, lp = sep_attn_decode(q, kn, vn, plain, scale, return_lse=True)
        sep_cache_update(plain, kn[:, :, None].contiguous(), vn[:, :, None].contiguous(), ids[:, None].contiguous(),
                         d_sep)
        torch.cuda.synchronize()
        assert torch.equal(of.view(torch.int16), op.view(torch.int16)), t
        assert torch.equal(lf, lp), t
        for name in ("k", "v", "pos", "tok", "state"):
            x, y = getattr(fused, name), getattr(plain, name)
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), (t, name)
        assert int(fused.state[:, 7].abs().max()) == 0
        if (t - T0) % 7 == 0 or t == T0 + steps - 1:
            o = from_dev(of)
            l_gpu = from_dev(lf)
            for b in range(B):
                keys = [e.pos for e in sims[b].keys()] + [t]
                kk = gen.bf16_bits_to_f64(st.k[b][:, keys])
                vv = gen.bf16_bits_to_f64(st.v[b][:, keys])
                qq = gen.bf16_bits_to_f64(st.q[b, t])
                if rope:
                    o_ref, l_ref = oracle.decode_attention_shifted(qq, kk, vv, scale, 500000.0)
                else:
                    o_ref, l_ref = oracle.decode_attention(qq, kk, vv, scale)
                check_close(o[b], o_ref, "bf16", f"{case} step {t} b {b}")
                assert np.max(np.abs(l_gpu[b] - l_ref)) < 1e-3
        for b in range(B):
            sims[b].push(oracle.Entry(t, int(st.ids[b, t])))
        if (t - T0) % 11 == 0 or t == T0 + steps - 1:
            check_cache(fused, sims, st)
