"""GPU parity of sep_attn_prefill_backward against the fp64 oracle.

The GPU forward (sep_attn_prefill) supplies out and lse, as a training step
would; the oracle's gradients use the same out for delta = rowsum(dout * out)
(oracle.attention_backward's ``out``) and the exact softmax weights.

Acceptance, element by element, for g in (dq, dk, dv):
    |g_gpu - g_ref| <= (eps + gamma) * B_g
where B_g is the same sum taken over absolute values:
    aS_ij = P_ij (sum_d |dO_id||V_jd| + sum_d |dO_id||out_id|)
    B_dq  = scale aS |K|,  B_dk = scale sum_h aS^T |Q|,  B_dv = sum_h P^T |dO|.
eps bounds the relative error of the recomputed weights P = exp(s - lse)
that the forward's lse carries: |lse_gpu - lse| <= delta_lse gives
|P_gpu / P - 1| <= exp(delta_lse) - 1 (delta_lse = 4e-3 for bf16, whose
forward sums bf16-rounded weights, and 1e-5 for fp32; both are the
forward's own log-sum-exp tolerances), plus a few ulp of the hardware exp2.
gamma = n u / (1 - n u), u = 2^-24, is the worst-case error of an fp32 sum
of n terms, with n = D + G S the longest chain of fp32 operations (dot
products of length D, then sums over at most G S query rows). With bf16
inputs the products run on the bf16 MFMA: P (for dV) and dS (for dQ, dK)
are rounded to bf16 first, which moves each term by at most 2^-8 of itself
(round to nearest even, 8 significant bits), so eps gains 2^-8 there; Q, K,
V and dO enter exactly. A wrong index, a dropped term or a mask error
shifts an element by a multiple of a single weight's contribution, far
above (eps + gamma) B at these sizes.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from inputs import configs, gen
from kv_cache_compression_sep_amd import (sep_attn_prefill, sep_attn_prefill_backward, sep_index_compact,
                                          sep_mask_build)

from .gpu_util import from_dev, guarded_empty, to_dev

pytestmark = pytest.mark.gpu

LSE_TOL = {"bf16": 4e-3, "f32": 1e-5}   # the forward's: test_gpu_prefill.py
OPERAND_ROUNDING = {"bf16": 2.0 ** -8, "f32": 0.0}   # P and dS rounded to bf16 (8 significant bits)
U32 = 2.0 ** -24


def run_gpu(ids, q, k, v, dout, sep_ids, a, n, dtype, scale):
    d_ids = to_dev(ids)
    flags, _, _ = sep_mask_build(d_ids, to_dev(np.asarray(sep_ids, np.int32)), a, n)
    rank, sep_pos, _ = sep_index_compact(flags)
    tq, tk, tv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    out, lse = sep_attn_prefill(tq, tk, tv, flags, rank, sep_pos, a, n, scale, return_lse=True)
    B, Hq, S, _ = q.shape
    Hkv, D = k.shape[1], q.shape[3]
    f32 = torch.float32
    delta = guarded_empty((B, Hq, S), f32)
    gq, gk, gv = sep_attn_prefill_backward(tq, tk, tv, out, to_dev(dout, dtype), lse, flags, rank, sep_pos,
                                           a, n, scale, delta=delta, dq=guarded_empty((B, Hq, S, D), f32),
                                           dk=guarded_empty((B, Hkv, S, D), f32),
                                           dv=guarded_empty((B, Hkv, S, D), f32))
    torch.cuda.synchronize()
    return from_dev(out), from_dev(gq), from_dev(gk), from_dev(gv), from_dev(delta)


def grad_bounds(q, k, v, out, dout, M, scale):
    """Absolute-value sums B_dq, B_dk, B_dv and B_delta (see the module
    docstring) of one sequence, float64."""
    Hq, S, D = q.shape
    G = Hq // k.shape[0]
    _, _, P = oracle.attention(q, k, v, M, scale, return_weights=True)
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    bdelta = (np.abs(dout) * np.abs(out)).sum(-1)
    for h in range(Hq):
        g = h // G
        aS = P[h] * (np.abs(dout[h]) @ np.abs(v[g]).T + bdelta[h][:, None])
        bq[h] = scale * (aS @ np.abs(k[g]))
        bk[g] += scale * (aS.T @ np.abs(q[h]))
        bv[g] += P[h].T @ np.abs(dout[h])
    return bq, bk, bv, bdelta


def check_bound(got, ref, bound, rel, what):
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite"
    err = np.abs(got - ref)
    lim = rel * bound + 1e-30
    worst = np.unravel_index(np.argmax(err / lim), err.shape)
    assert np.all(err <= lim), (f"{what}: err {err[worst]:.3e} > {lim[worst]:.3e} at {worst} "
                                f"(ref {ref[worst]:.5f}, got {got[worst]:.5f}, max err {err.max():.3e})")
    print(f"{what}: max err {err.max():.3e}, max err / bound {np.max(err / lim):.3f}", flush=True)


def rand_inputs(rng, B, Hq, Hkv, S, D, p_sep, dtype):
    ids = np.where(rng.random((B, S)) < p_sep, rng.integers(0, 8, (B, S)),
                   rng.integers(8, 1000, (B, S))).astype(np.int32)
    q = gen.round_storage(rng.standard_normal((B, Hq, S, D)), dtype)
    k = gen.round_storage(rng.standard_normal((B, Hkv, S, D)), dtype)
    v = gen.round_storage(rng.standard_normal((B, Hkv, S, D)), dtype)
    dout = gen.round_storage(rng.standard_normal((B, Hq, S, D)), dtype)
    return ids, q, k, v, dout


def check_case(ids, q, k, v, dout, sep_ids, a, n, dtype, tag):
    B, Hq, S, D = q.shape
    G = Hq // k.shape[1]
    scale = 1.0 / math.sqrt(D)
    out, gq, gk, gv, delta = run_gpu(ids, q, k, v, dout, sep_ids, a, n, dtype, scale)
    nterms = D + G * S
    gamma = nterms * U32 / (1 - nterms * U32)
    eps = math.expm1(LSE_TOL[dtype]) + OPERAND_ROUNDING[dtype] + 8 * U32
    for b in range(B):
        M = oracle.sep_mask(oracle.is_sep(ids[b], sep_ids), a, n)
        f = [gen.storage_to_f64(x[b], dtype) for x in (q, k, v, dout)]
        rq, rk, rv, rdelta = oracle.attention_backward(*f[:3], M, scale, f[3], out=out[b])
        bq, bk, bv, bdelta = grad_bounds(f[0], f[1], f[2], out[b], f[3], M, scale)
        check_bound(delta[b], rdelta, bdelta, (D + 2) * U32, f"{tag} b={b} delta")
        check_bound(gq[b], rq, bq, eps + gamma, f"{tag} b={b} dq")
        check_bound(gk[b], rk, bk, eps + gamma, f"{tag} b={b} dk")
        check_bound(gv[b], rv, bv, eps + gamma, f"{tag} b={b} dv")


CASES = [
    # B, Hq, Hkv, S,   D,   a,   n,   p_sep
    (1, 4, 1, 97, 64, 4, 16, 0.1),
    (2, 8, 2, 300, 128, 4, 64, 0.12),
    (1, 8, 1, 513, 128, 0, 1, 0.3),       # window 1: a key sees only itself and the globals
    (1, 2, 2, 257, 64, 9, 300, 0.05),     # window longer than the sequence
    (1, 16, 2, 200, 128, 4, 32, 0.0),     # no separators, G = 8
    (1, 16, 1, 130, 64, 2, 8, 1.0),       # every token a separator, G = 16
    (1, 3, 1, 190, 128, 500, 4, 0.1),     # more initial tokens than tokens, G = 3
    (1, 4, 4, 1, 128, 4, 256, 0.5),       # a single token
    (1, 2, 1, 33, 128, 1, 2, 0.2),
    (1, 32, 8, 1100, 128, 4, 256, 0.12),  # Llama-3 head shape, ragged S, several 256-row chunks
    (1, 6, 3, 777, 64, 3, 100, 0.08),     # G = 2
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_prefill_backward_small_cases(case, dtype):
    B, Hq, Hkv, S, D, a, n, p = case
    print(f"backward case {case} {dtype}", flush=True)
    rng = np.random.default_rng(zlib.crc32(repr(("bwd", case, dtype)).encode()))
    ids, q, k, v, dout = rand_inputs(rng, B, Hq, Hkv, S, D, p, dtype)
    check_case(ids, q, k, v, dout, list(range(8)), a, n, dtype, f"{case} {dtype}")


def test_prefill_backward_repeat_is_stable():
    """Two calls on the same inputs: the band kernels' results are
    deterministic; only the global keys' atomic sums may differ, within a
    few ulp of their magnitude."""
    rng = np.random.default_rng(151)
    ids, q, k, v, dout = rand_inputs(rng, 1, 8, 2, 600, 128, 0.1, "bf16")
    r1 = run_gpu(ids, q, k, v, dout, list(range(8)), 4, 64, "bf16", 1 / math.sqrt(128))
    r2 = run_gpu(ids, q, k, v, dout, list(range(8)), 4, 64, "bf16", 1 / math.sqrt(128))
    assert np.array_equal(r1[0], r2[0]) and np.array_equal(r1[1], r2[1])
    for x, y in zip(r1[2:4], r2[2:4]):
        assert np.max(np.abs(x - y)) <= 1e-5 * np.max(np.abs(x))


def sampled_bounds(q, k, v, dout, out, M, scale, rows, keys):
    """B_dq at the sampled rows and B_dk, B_dv at the sampled keys of one kv
    head group (q, dout, out [G, S, D]; k, v [S, D]), with the exact lse."""
    G, S, D = q.shape
    lse = np.empty((G, S))
    for r0 in range(0, S, 512):
        _, lse[:, r0:r0 + 512] = oracle.attention_rows(q[:, r0:r0 + 512], k[None], v[None], M[r0:r0 + 512],
                                                       scale, [0] * G)
    bdelta = (np.abs(dout) * np.abs(out)).sum(-1)
    bq = np.empty((G, len(rows), D))
    bk = np.zeros((len(keys), D))
    bv = np.zeros((len(keys), D))
    for h in range(G):
        x = scale * (q[h, rows] @ k.T)
        x[~M[rows]] = -np.inf
        Pr = np.exp(x - lse[h, rows][:, None])
        bq[h] = scale * ((Pr * (np.abs(dout[h, rows]) @ np.abs(v).T + bdelta[h, rows][:, None])) @ np.abs(k))
        x = scale * (q[h] @ k[keys].T)
        x[~M[:, keys]] = -np.inf
        Pc = np.exp(x - lse[h][:, None])
        bk += scale * ((Pc * (np.abs(dout[h]) @ np.abs(v[keys]).T + bdelta[h][:, None])).T @ np.abs(q[h]))
        bv += Pc.T @ np.abs(dout[h])
    return bq, bk, bv


@pytest.mark.timeout(900)
def test_llama3_layer_workload_sampled():
    """The Llama-3-8B layer workload (1 x 8192 tokens, 32/8 heads, D = 128,
    bf16) in the benchmark's launch configuration: every head is on the GPU;
    one kv head's group is host-generated and checked on sampled query rows
    (first, last and random) and sampled keys (initial, early and late
    separators, window keys, the last keys)."""
    cfg = configs.LLAMA3_LAYER_PREFILL
    B, Hq, Hkv, S, D = cfg.B, cfg.Hq, cfg.Hkv, cfg.S, cfg.D
    G = Hq // Hkv
    g = 5
    heads = list(range(g * G, g * G + G))
    scale = 1.0 / math.sqrt(D)
    ids = np.stack([gen.prefill_ids(cfg, 0)])
    torch.manual_seed(0)
    bf = dict(device="cuda")
    q = torch.randn((B, Hq, S, D), **bf).to(torch.bfloat16)
    dout = torch.randn((B, Hq, S, D), **bf).to(torch.bfloat16)
    k = torch.randn((B, Hkv, S, D), **bf).to(torch.bfloat16)
    v = torch.randn((B, Hkv, S, D), **bf).to(torch.bfloat16)
    xq = np.stack([gen.prefill_head(cfg, 0, gen.TAG_Q, h) for h in heads])
    xdo = np.stack([gen.prefill_head(cfg, 0, gen.TAG_DO, h) for h in heads])
    xk = gen.prefill_head(cfg, 0, gen.TAG_K, g)
    xv = gen.prefill_head(cfg, 0, gen.TAG_V, g)
    for i, h in enumerate(heads):
        q[0, h] = to_dev(xq[i], "bf16")
        dout[0, h] = to_dev(xdo[i], "bf16")
    k[0, g] = to_dev(xk, "bf16")
    v[0, g] = to_dev(xv, "bf16")
    flags, _, _ = sep_mask_build(to_dev(ids), to_dev(np.asarray(cfg.sep_ids, np.int32)), cfg.a, cfg.n)
    rank, sep_pos, _ = sep_index_compact(flags)
    out, lse = sep_attn_prefill(q, k, v, flags, rank, sep_pos, cfg.a, cfg.n, scale, return_lse=True)
    gq, gk, gv = sep_attn_prefill_backward(q, k, v, out, dout, lse, flags, rank, sep_pos, cfg.a, cfg.n, scale)
    torch.cuda.synchronize()

    f = oracle.is_sep(ids[0], cfg.sep_ids)
    seps = np.flatnonzero(f[cfg.a:]) + cfg.a
    band = np.flatnonzero(~f[cfg.a:]) + cfg.a
    rng = np.random.default_rng(521)
    rows = sorted(set(list(range(0, 64)) + list(range(S - 64, S)) + rng.integers(0, S, 128).tolist()))
    keys = sorted(set(list(range(cfg.a)) + seps[:8].tolist() + rng.choice(seps, 24).tolist() +
                      band[:8].tolist() + rng.choice(band, 48).tolist() + list(range(S - 8, S))))
    got_q = from_dev(gq[0, heads][:, rows])
    got_k = from_dev(gk[0, g, keys])
    got_v = from_dev(gv[0, g, keys])
    out_g = from_dev(out[0, heads])

    M = oracle.sep_mask(f, cfg.a, cfg.n)
    x64 = [gen.storage_to_f64(x, "bf16") for x in (xq, xk, xv, xdo)]
    rq, rk, rv = oracle.attention_backward_sampled(x64[0], x64[1], x64[2], x64[3], out_g, M, scale, rows, keys)
    bq, bk, bv = sampled_bounds(x64[0], x64[1], x64[2], x64[3], out_g, M, scale, rows, keys)
    nterms = D + G * S
    rel = math.expm1(LSE_TOL["bf16"]) + OPERAND_ROUNDING["bf16"] + 8 * U32 + nterms * U32 / (1 - nterms * U32)
    check_bound(got_q, rq, bq, rel, f"{cfg.name} dq")
    check_bound(got_k, rk, bk, rel, f"{cfg.name} dk")
    check_bound(got_v, rv, bv, rel, f"{cfg.name} dv")
