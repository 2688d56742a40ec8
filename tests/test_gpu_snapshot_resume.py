"""Checkpoint and resume of a streaming cache.

The cache is fully described by its caller-owned buffers (k, v, pos, tok and
the state words); the library keeps no state of its own. Copying the buffers
out at step k and back into another cache must therefore let that cache
resume the stream and reproduce the uninterrupted run bit for bit: every
later decode output and log-sum-exp, and the final K/V, pos, tok and state.
Cases cover every cache policy, StreamingLLM mode, a restore into a cache
that held another stream, and a snapshot taken between bulk updates.
"""
import zlib

import numpy as np
import pytest
import torch

from kv_cache_compression_sep_amd import SEP_POLICY_DYNAMIC, SEP_POLICY_NO_ACCUM, SepCache, sep_decode_update

from .gpu_util import guarded_cache, to_dev
from .test_gpu_cache_decode import SEP_IDS, Stream

pytestmark = pytest.mark.gpu
BUFFERS = ("k", "v", "pos", "tok", "state")

CASES = [
    # B, Hq, Hkv, D,  a, s,  p,  w,  T0, k_snap, steps, policy
    (2, 32, 8, 128, 4, 64, 64, 256, 500, 37, 150, 0),
    (3, 8, 2, 64, 2, 5, 3, 11, 40, 9, 80, SEP_POLICY_DYNAMIC),
    (1, 16, 4, 128, 4, 20, 8, 40, 100, 61, 120, SEP_POLICY_NO_ACCUM),
    (2, 8, 8, 64, 0, 7, 9, 33, 0, 50, 120, SEP_POLICY_DYNAMIC | SEP_POLICY_NO_ACCUM),
    (1, 4, 2, 128, 4, 0, 0, 12, 30, 20, 60, 0),           # StreamingLLM mode
    (40, 16, 8, 64, 4, 6, 5, 9, 30, 11, 40, 0),           # B * Hkv >= 256: the two-launch step
]


def run_steps(cache, st, t0, t1, d_sep):
    outs = []
    for t in range(t0, t1):
        o, lse = sep_decode_update(to_dev(np.ascontiguousarray(st.q[:, t]), "bf16"),
                                   to_dev(np.ascontiguousarray(st.k[:, :, t]), "bf16"),
                                   to_dev(np.ascontiguousarray(st.v[:, :, t]), "bf16"),
                                   to_dev(np.ascontiguousarray(st.ids[:, t])), cache, d_sep, return_lse=True)
        outs.append((o.view(torch.int16).clone(), lse.clone()))
    return outs


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_snapshot_restore_resume_is_bit_exact(case):
    B, Hq, Hkv, D, a, s, p, w, T0, k_snap, steps, policy = case
    print(f"snapshot case {case}", flush=True)
    st = Stream(zlib.crc32(repr(("snap", case)).encode()), B, Hq, Hkv, D, T0 + steps, 0.2)
    d_sep = to_dev(np.asarray(SEP_IDS, np.int32))
    ref = guarded_cache(B, Hkv, D, a, s, p, w, policy=policy)
    if T0:
        st.push_gpu(ref, 0, T0 // 2, d_sep)
        st.push_gpu(ref, T0 // 2, T0, d_sep)
    head = run_steps(ref, st, T0, T0 + k_snap, d_sep)
    torch.cuda.synchronize()
    snap = {name: getattr(ref, name).clone().cpu() for name in BUFFERS}      # checkpoint to host memory
    tail = run_steps(ref, st, T0 + k_snap, T0 + steps, d_sep)
    torch.cuda.synchronize()
    assert len(head) == k_snap

    # restore into a cache that first runs another stream, so nothing of the
    # new cache's own history survives the restore
    other = Stream(zlib.crc32(repr(("other", case)).encode()), B, Hq, Hkv, D, 64, 0.5)
    res = guarded_cache(B, Hkv, D, a, s, p, w, policy=policy)
    other.push_gpu(res, 0, 64, d_sep)
    for name in BUFFERS:
        getattr(res, name).copy_(snap[name].cuda())
    resumed = run_steps(res, st, T0 + k_snap, T0 + steps, d_sep)
    torch.cuda.synchronize()
    for i, ((o1, l1), (o2, l2)) in enumerate(zip(tail, resumed)):
        assert torch.equal(o1, o2), (case, "decode output", T0 + k_snap + i)
        assert torch.equal(l1, l2), (case, "lse", T0 + k_snap + i)
    for name in BUFFERS:
        x, y = getattr(ref, name), getattr(res, name)
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        assert torch.equal(x, y), (case, name)
