"""The two streaming workloads at full size, against the oracle, on the entry
point the benchmark times (sep_decode_update: decode, then the single-token
update of the same token).

Streaming decode, batch 1 (4,194,304-token stream, a=4 s=64 p=64 w=256):
the first 65,536 steps run on the GPU; every decode output is compared with
the oracle, and the full cache state (positions, ids and K/V bytes of every
block, in logical order; the arrival word 7 reads 0) at every 4096th step.

Batched decode, 64 sequences (32,768-token histories, a=4 s=256 p=28
w=512): the histories are ingested with one bulk update, then 1024 steps
run. Every sequence is compared in full: the cache after the history, the
cache every 128 steps, every decode output, and the decode with RoPE
position shifting every 128 steps; the final cache positions are also
compared with the closed form.

The oracle decodes are evaluated many steps per call (tests/stream_check.py:
masked attention whose row for step t marks exactly that step's keys).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from inputs import configs, gen
from kv_cache_compression_sep_amd import (SepCache, sep_attn_decode_rope, sep_cache_update, sep_decode_update,
                                          sep_rope_table)

from .gpu_util import check_close, from_dev, guarded_cache, slots_of, to_dev
from .stream_check import decode_steps

pytestmark = pytest.mark.gpu
ROPE_BASE = 500000.0     # Llama 3


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def snapshot(cache):
    return {name: getattr(cache, name).clone() for name in ("state", "pos", "tok", "k", "v")}


def compare_state(cache, snap, b, sim, ids, k_of, v_of):
    """The snapshot of sequence b against the simulation, block by block.
    k_of(positions) -> [Hkv, len, D] uint16 rows of those positions."""
    st = snap["state"]
    assert int(st[b, 0]) == sim.t
    assert int(st[b, 7]) == 0, "arrival word of sep_decode_update not cleared"
    pos = snap["pos"][b].cpu().numpy()
    tok = snap["tok"][b].cpu().numpy()
    kc = bits(snap["k"][b])
    vc = bits(snap["v"][b])
    I, S, R = slots_of(cache, b, state=st)
    for slots, want in zip((I, S, R), sim.positions()):
        assert pos[slots].tolist() == want
        assert tok[slots].tolist() == [int(ids[x]) for x in want]
        if want:
            assert np.array_equal(kc[:, slots], k_of(want))
            assert np.array_equal(vc[:, slots], v_of(want))
    dead = sorted(set(range(cache.slots)) - set(I) - set(S) - set(R))
    assert (pos[dead] == -1).all() and (tok[dead] == -1).all()
    assert sim.occupancy() <= cache.c


@pytest.mark.timeout(1200)
def test_stream_decode_first_65536_steps():
    cfg = configs.STREAM_DECODE
    steps = cfg.check_steps
    ids = gen.stream_ids(cfg, 0, cfg.history + cfg.steps)
    qp, kp, vp = gen.stream_pool(cfg, 0)
    print(f"[stream] pools ready, {steps} steps on sep_decode_update", flush=True)
    dq, dk, dv = to_dev(qp, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16")
    d_ids = to_dev(ids[:steps].copy())
    d_sep = to_dev(np.asarray(cfg.sep_ids, np.int32))
    cache = guarded_cache(1, cfg.Hkv, cfg.D, cfg.a, cfg.s, cfg.p, cfg.w)
    outs = torch.empty((steps, cfg.Hq, cfg.D), dtype=torch.bfloat16, device="cuda")
    lses = torch.empty((steps, cfg.Hq), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(cfg.D)
    snaps = {}
    for t in range(steps):
        sep_decode_update(dq[t:t + 1], dk[t:t + 1], dv[t:t + 1], d_ids[t:t + 1], cache, d_sep, scale,
                          out=outs[t:t + 1], lse=lses[t:t + 1])
        if (t + 1) % cfg.check_every == 0:
            snaps[t + 1] = snapshot(cache)
    torch.cuda.synchronize()
    print("[stream] gpu steps done", flush=True)
    o_gpu = from_dev(outs)
    l_gpu = from_dev(lses)
    k_of = lambda xs: np.ascontiguousarray(kp[xs].transpose(1, 0, 2))
    v_of = lambda xs: np.ascontiguousarray(vp[xs].transpose(1, 0, 2))

    def kv_rows(pos):
        return gen.bf16_bits_to_f64(k_of(pos)), gen.bf16_bits_to_f64(v_of(pos))

    def after_push(t, sim):
        if (t + 1) in snaps:
            compare_state(cache, snaps[t + 1], 0, sim, ids, k_of, v_of)

    sim = oracle.CacheSim(cfg.a, cfg.s, cfg.p, cfg.w, cfg.sep_ids)
    worst = 0.0
    chunk = 8192
    for c0 in range(0, steps, chunk):
        o_ref, l_ref, _ = decode_steps(sim, ids, c0, c0 + chunk, lambda s0, s1: qp[s0:s1], kv_rows, scale,
                                       seg=64, after_push=after_push)
        worst = max(worst, check_close(o_gpu[c0:c0 + chunk], o_ref, "bf16", f"steps {c0}..{c0 + chunk}"))
        assert np.max(np.abs(l_gpu[c0:c0 + chunk] - l_ref)) < 1e-3
        print(f"[stream] oracle through step {c0 + chunk}, worst err {worst:.3e}", flush=True)
    assert sim.t == steps


@pytest.mark.timeout(1200)
def test_batched_decode_workload_all_sequences():
    cfg = configs.BATCHED_DECODE
    B, Hq, Hkv, D, H, steps = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.history, cfg.steps
    ids = np.stack([gen.stream_ids(cfg, b) for b in range(B)])       # [B, H + steps]
    hk = gen.device_normal((B, Hkv, H, D), cfg.seed, gen.TAG_HK)
    hv = gen.device_normal((B, Hkv, H, D), cfg.seed, gen.TAG_HV)
    pq = gen.device_normal((B, steps, Hq, D), cfg.seed, gen.TAG_Q)
    pk = gen.device_normal((B, steps, Hkv, D), cfg.seed, gen.TAG_K)
    pv = gen.device_normal((B, steps, Hkv, D), cfg.seed, gen.TAG_V)
    d_ids = to_dev(ids)
    d_sep = to_dev(np.asarray(cfg.sep_ids, np.int32))
    cache = guarded_cache(B, Hkv, D, cfg.a, cfg.s, cfg.p, cfg.w)
    sep_cache_update(cache, hk, hv, d_ids[:, :H].contiguous(), d_sep)
    torch.cuda.synchronize()
    print("[batched] history ingested", flush=True)
    snaps = {0: snapshot(cache)}
    scale = 1.0 / math.sqrt(D)
    outs = torch.empty((steps, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lses = torch.empty((steps, B, Hq), dtype=torch.float32, device="cuda")
    # every 128th step also decodes with RoPE position shifting (Llama-3 base),
    # on the cache as it stands before that step
    table = sep_rope_table(ROPE_BASE, D, cache.slots + 1)
    rope_steps = list(range(0, steps, 128)) + [steps - 1]
    routs = torch.empty((len(rope_steps), B, Hq, D), dtype=torch.bfloat16, device="cuda")
    for j in range(steps):
        qj = pq[:, j].contiguous()
        kj = pk[:, j].contiguous()
        vj = pv[:, j].contiguous()
        if j in rope_steps:
            sep_attn_decode_rope(qj, kj, vj, cache, table, scale, out=routs[rope_steps.index(j)])
        sep_decode_update(qj, kj, vj, d_ids[:, H + j].contiguous(), cache, d_sep, scale, out=outs[j],
                          lse=lses[j])
        if (j + 1) % cfg.check_every == 0:
            snaps[j + 1] = snapshot(cache)
    torch.cuda.synchronize()
    print("[batched] gpu steps done", flush=True)

    # host copies: the history rows each sequence still holds after the
    # ingest (later steps only drop them or keep them), and every step's rows
    sims = [oracle.CacheSim(cfg.a, cfg.s, cfg.p, cfg.w, cfg.sep_ids) for _ in range(B)]
    hist_pos, hist_k, hist_v = [], [], []
    for b in range(B):
        sims[b].push_many([oracle.Entry(x, int(ids[b, x])) for x in range(H)])
        need = np.asarray(sum(sims[b].positions(), []), np.int64)
        idx = torch.from_numpy(need).cuda()
        hist_pos.append(need)
        hist_k.append(bits(hk[b].index_select(1, idx)))
        hist_v.append(bits(hv[b].index_select(1, idx)))
    pool_q, pool_k, pool_v = bits(pq), bits(pk), bits(pv)
    o_gpu = from_dev(outs)
    l_gpu = from_dev(lses)
    r_gpu = from_dev(routs)
    print("[batched] host copies ready", flush=True)

    def rows_of(b, kind):
        hist = hist_k[b] if kind == "k" else hist_v[b]
        pool = pool_k[b] if kind == "k" else pool_v[b]

        def f(xs):
            xs = np.asarray(xs, np.int64)
            out = np.empty((Hkv, len(xs), D), np.uint16)
            old = xs < H
            r = np.searchsorted(hist_pos[b], xs[old])
            assert np.array_equal(hist_pos[b][r], xs[old])
            out[:, old] = hist[:, r]
            out[:, ~old] = pool[xs[~old] - H].transpose(1, 0, 2)
            return out
        return f

    worst = rope_vs_exact = 0.0
    for b in range(B):
        kr, vr = rows_of(b, "k"), rows_of(b, "v")
        compare_state(cache, snaps[0], b, sims[b], ids[b], kr, vr)

        def after_push(t, sim, b=b, kr=kr, vr=vr):
            if (t + 1 - H) in snaps:
                compare_state(cache, snaps[t + 1 - H], b, sim, ids[b], kr, vr)

        def kv_rows(pos, kr=kr, vr=vr):
            return gen.bf16_bits_to_f64(kr(pos)), gen.bf16_bits_to_f64(vr(pos))

        o_ref, l_ref, kept = decode_steps(sims[b], ids[b], H, H + steps,
                                          lambda s0, s1, b=b: pool_q[b, s0 - H:s1 - H], kv_rows, scale, seg=32,
                                          after_push=after_push, keep=[H + j for j in rope_steps])
        worst = max(worst, check_close(o_gpu[:, b], o_ref, "bf16", f"seq {b}"))
        assert np.max(np.abs(l_gpu[:, b] - l_ref)) < 1e-3, b
        for i, j in enumerate(rope_steps):
            keys = kept[H + j]
            kk, vv = kv_rows(keys)
            qq = gen.bf16_bits_to_f64(pool_q[b, j])
            r_ref, _ = oracle.decode_attention_shifted(qq, kk, vv, scale, ROPE_BASE)
            check_close(r_gpu[i, b], r_ref, "bf16", f"seq {b} step {j} rope")
            # the same step with the rotated operands kept exact (not rounded
            # to bf16): reported, and held to the same tolerance
            r_exact, _ = oracle.decode_attention_shifted(qq, kk, vv, scale, ROPE_BASE, to_bf16=False)
            rope_vs_exact = max(rope_vs_exact, check_close(r_gpu[i, b], r_exact, "bf16",
                                                           f"seq {b} step {j} rope vs exact rotation"))
        if b % 8 == 7:
            print(f"[batched] sequences 0..{b} match, worst err {worst:.3e}, RoPE decode vs unrounded "
                  f"rotation {rope_vs_exact:.3e}", flush=True)
    flags_all = oracle.is_sep(ids, cfg.sep_ids)
    for b in range(B):
        I, S, R = oracle.closed_form_positions(flags_all[b], H + steps, cfg.a, cfg.s, cfg.p, cfg.w)
        pos = cache.pos[b].cpu().numpy()
        for slots, want in zip(slots_of(cache, b), (I, S, R)):
            assert pos[slots].tolist() == want, b
