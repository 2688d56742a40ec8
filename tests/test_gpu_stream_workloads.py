"""The two streaming workloads at full size, against the oracle.

Streaming decode, batch 1 (4,194,304-token stream, a=4 s=64 p=64 w=256):
the first 65,536 steps run decode + update on the GPU; every decode output
is compared with the oracle, and the full cache state (positions, ids and
K/V bytes of every block, in logical order) at every 4096th step.

Batched decode, 64 sequences (32,768-token histories, a=4 s=256 p=28
w=512): the histories are ingested with one bulk update, then 1024 decode +
update steps run. Four sequences are compared in full (cache every 128
steps, every decode output, and the decode with RoPE position shifting
every 128 steps); for all 64 the cache positions and ids are compared with
the closed form after the history and at the end.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from inputs import configs, gen
from kv_cache_compression_sep_amd import (SepCache, sep_attn_decode, sep_attn_decode_rope, sep_cache_update,
                                          sep_rope_table)

from .gpu_util import check_close, from_dev, to_dev

pytestmark = pytest.mark.gpu
ROPE_BASE = 500000.0     # Llama 3


def logical(cache, b):
    return cache.slots_of(b)


def compare_state(cache, b, sim, ids, k_of, v_of):
    """k_of(positions) -> [Hkv, len, D] uint16 rows of those positions."""
    pos = cache.pos[b].cpu().numpy()
    tok = cache.tok[b].cpu().numpy()
    kc = cache.k[b].view(torch.int16).cpu().numpy().view(np.uint16)
    vc = cache.v[b].view(torch.int16).cpu().numpy().view(np.uint16)
    for slots, want in zip(logical(cache, b), sim.positions()):
        assert pos[slots].tolist() == want
        assert tok[slots].tolist() == [int(ids[x]) for x in want]
        if want:
            assert np.array_equal(kc[:, slots], k_of(want))
            assert np.array_equal(vc[:, slots], v_of(want))


@pytest.mark.timeout(1500)
def test_stream_decode_first_65536_steps():
    cfg = configs.STREAM_DECODE
    steps = cfg.check_steps
    ids = gen.stream_ids(cfg, 0, cfg.history + cfg.steps)
    qp, kp, vp = gen.stream_pool(cfg, 0)
    print(f"[stream] pools ready, {steps} steps", flush=True)
    dq, dk, dv = to_dev(qp, "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16")
    d_ids = to_dev(ids[:steps].copy())
    d_sep = to_dev(np.asarray(cfg.sep_ids, np.int32))
    cache = SepCache(1, cfg.Hkv, cfg.D, cfg.a, cfg.s, cfg.p, cfg.w)
    outs = torch.empty((steps, cfg.Hq, cfg.D), dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / math.sqrt(cfg.D)
    snaps = {}
    for t in range(steps):
        sep_attn_decode(dq[t:t + 1], dk[t:t + 1], dv[t:t + 1], cache, scale, out=outs[t:t + 1])
        sep_cache_update(cache, dk[t:t + 1].view(1, cfg.Hkv, 1, cfg.D),
                         dv[t:t + 1].view(1, cfg.Hkv, 1, cfg.D), d_ids[t:t + 1].view(1, 1), d_sep)
        if (t + 1) % cfg.check_every == 0:
            snaps[t + 1] = (cache.state.clone(), cache.pos.clone(), cache.tok.clone(),
                            cache.k.clone(), cache.v.clone())
    torch.cuda.synchronize()
    print("[stream] gpu steps done", flush=True)
    o_gpu = from_dev(outs)
    sim = oracle.CacheSim(cfg.a, cfg.s, cfg.p, cfg.w, cfg.sep_ids)
    kf = gen.bf16_bits_to_f64(kp)  # [pool, Hkv, D]
    vf = gen.bf16_bits_to_f64(vp)
    qf = gen.bf16_bits_to_f64(qp)
    k_of = lambda xs: np.ascontiguousarray(kp[xs].transpose(1, 0, 2))
    v_of = lambda xs: np.ascontiguousarray(vp[xs].transpose(1, 0, 2))
    worst = 0.0
    for t in range(steps):
        keys = [e.pos for e in sim.keys()] + [t]
        o_ref, _ = oracle.decode_attention(qf[t], kf[keys].transpose(1, 0, 2),
                                           vf[keys].transpose(1, 0, 2), scale)
        worst = max(worst, check_close(o_gpu[t], o_ref, "bf16", f"step {t}"))
        sim.push(oracle.Entry(t, int(ids[t])))
        if (t + 1) in snaps:
            st, pos, tok, kk, vv = snaps[t + 1]
            view = SepCache.__new__(SepCache)
            view.a, view.s, view.p, view.w, view.c = cfg.a, cfg.s, cfg.p, cfg.w, cfg.c
            view.ring, view.policy = cfg.p + cfg.w, 0
            view.state, view.pos, view.tok, view.k, view.v = st, pos, tok, kk, vv
            compare_state(view, 0, sim, ids, k_of, v_of)
            assert sim.occupancy() <= cfg.c
        if t % 8192 == 0:
            print(f"[stream] oracle at step {t}, worst err {worst:.3e}", flush=True)
    print(f"[stream] worst decode err {worst:.3e}", flush=True)


@pytest.mark.timeout(1500)
def test_batched_decode_workload():
    cfg = configs.BATCHED_DECODE
    B, Hq, Hkv, D, H = cfg.B, cfg.Hq, cfg.Hkv, cfg.D, cfg.history
    checked = [0, 21, 42, 63]
    ids = np.stack([gen.stream_ids(cfg, b) for b in range(B)])       # [B, H + steps]
    torch.manual_seed(1234)
    hk = torch.randn((B, Hkv, H, D), device="cuda").to(torch.bfloat16)
    hv = torch.randn((B, Hkv, H, D), device="cuda").to(torch.bfloat16)
    pq = torch.randn((B, cfg.steps, Hq, D), device="cuda").to(torch.bfloat16)
    pk = torch.randn((B, cfg.steps, Hkv, D), device="cuda").to(torch.bfloat16)
    pv = torch.randn((B, cfg.steps, Hkv, D), device="cuda").to(torch.bfloat16)
    host = {}
    for b in checked:
        k_h, v_h = gen.history_kv(cfg, b)
        q_p, k_p, v_p = gen.stream_pool(cfg, b)
        host[b] = (k_h, v_h, q_p, k_p, v_p)
        hk[b] = to_dev(k_h, "bf16")
        hv[b] = to_dev(v_h, "bf16")
        pq[b] = to_dev(q_p, "bf16")
        pk[b] = to_dev(k_p, "bf16")
        pv[b] = to_dev(v_p, "bf16")
    print("[batched] inputs ready", flush=True)
    d_ids = to_dev(ids)
    d_sep = to_dev(np.asarray(cfg.sep_ids, np.int32))
    cache = SepCache(B, Hkv, D, cfg.a, cfg.s, cfg.p, cfg.w)
    sep_cache_update(cache, hk, hv, d_ids[:, :H].contiguous(), d_sep)
    torch.cuda.synchronize()
    flags_all = oracle.is_sep(ids, cfg.sep_ids)
    for b in range(B):
        I, S, R = oracle.closed_form_positions(flags_all[b], H, cfg.a, cfg.s, cfg.p, cfg.w)
        pos = cache.pos[b].cpu().numpy()
        for slots, want in zip(logical(cache, b), (I, S, R)):
            assert pos[slots].tolist() == want, b
    sims = {}
    for b in checked:
        sims[b] = oracle.CacheSim(cfg.a, cfg.s, cfg.p, cfg.w, cfg.sep_ids)
        sims[b].push_many([oracle.Entry(x, int(ids[b, x])) for x in range(H)])

    def rows_of(b, kind):
        k_h, v_h, _, k_p, v_p = host[b]
        hist = k_h if kind == "k" else v_h
        pool = k_p if kind == "k" else v_p
        def f(xs):
            out = np.empty((Hkv, len(xs), D), np.uint16)
            for i, x in enumerate(xs):
                out[:, i] = hist[:, x] if x < H else pool[x - H]
            return out
        return f

    for b in checked:
        compare_state(cache, b, sims[b], ids[b], rows_of(b, "k"), rows_of(b, "v"))
    print("[batched] history ingest matches", flush=True)
    scale = 1.0 / math.sqrt(D)
    outs = torch.empty((cfg.steps, B, Hq, D), dtype=torch.bfloat16, device="cuda")
    # every 128th step also runs with RoPE position shifting (Llama-3 base)
    table = sep_rope_table(ROPE_BASE, D, cache.slots + 1)
    rope_steps = list(range(0, cfg.steps, 128)) + [cfg.steps - 1]
    routs = torch.empty((len(rope_steps), B, Hq, D), dtype=torch.bfloat16, device="cuda")
    snaps = {}
    for j in range(cfg.steps):
        qj = pq[:, j].contiguous()
        kj = pk[:, j].contiguous()
        vj = pv[:, j].contiguous()
        sep_attn_decode(qj, kj, vj, cache, scale, out=outs[j])
        if j in rope_steps:
            sep_attn_decode_rope(qj, kj, vj, cache, table, scale, out=routs[rope_steps.index(j)])
        sep_cache_update(cache, kj.view(B, Hkv, 1, D), vj.view(B, Hkv, 1, D),
                         d_ids[:, H + j:H + j + 1].contiguous(), d_sep)
        if (j + 1) % cfg.check_every == 0:
            snaps[j + 1] = (cache.state.clone(), cache.pos.clone(), cache.tok.clone(),
                            cache.k.clone(), cache.v.clone())
    torch.cuda.synchronize()
    o_all = outs[:, checked].float().cpu().numpy().astype(np.float64)
    r_all = routs[:, checked].float().cpu().numpy().astype(np.float64)
    print("[batched] gpu steps done", flush=True)
    for i, b in enumerate(checked):
        k_h, v_h, q_p, k_p, v_p = host[b]
        kr, vr = rows_of(b, "k"), rows_of(b, "v")
        for j in range(cfg.steps):
            t = H + j
            keys = [e.pos for e in sims[b].keys()] + [t]
            kk = gen.bf16_bits_to_f64(kr(keys))
            vv = gen.bf16_bits_to_f64(vr(keys))
            o_ref, _ = oracle.decode_attention(gen.bf16_bits_to_f64(q_p[j]), kk, vv, scale)
            check_close(o_all[j, i], o_ref, "bf16", f"seq {b} step {j}")
            if j in rope_steps:
                r_ref, _ = oracle.decode_attention_shifted(gen.bf16_bits_to_f64(q_p[j]), kk, vv, scale, ROPE_BASE)
                check_close(r_all[rope_steps.index(j), i], r_ref, "bf16", f"seq {b} step {j} rope")
            sims[b].push(oracle.Entry(t, int(ids[b, t])))
            if (j + 1) in snaps:
                st, pos, tok, kc, vc = snaps[j + 1]
                view = SepCache.__new__(SepCache)
                view.a, view.s, view.p, view.w, view.c = cfg.a, cfg.s, cfg.p, cfg.w, cfg.c
                view.ring, view.policy = cfg.p + cfg.w, 0
                view.state, view.pos, view.tok, view.k, view.v = st, pos, tok, kc, vc
                compare_state(view, b, sims[b], ids[b], kr, vr)
        print(f"[batched] sequence {b} matches", flush=True)
    T_end = H + cfg.steps
    for b in range(B):
        I, S, R = oracle.closed_form_positions(flags_all[b], T_end, cfg.a, cfg.s, cfg.p, cfg.w)
        pos = cache.pos[b].cpu().numpy()
        for slots, want in zip(logical(cache, b), (I, S, R)):
            assert pos[slots].tolist() == want, b
