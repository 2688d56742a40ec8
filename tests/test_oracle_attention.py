"""Pins of the oracle's masked softmax attention (prefill and decode).

References other than the oracle itself: a pure-Python triple loop with
``math.exp``; PyTorch's float64 CPU scaled_dot_product_attention on the
special cases where the Sep-Attention mask is the causal triangle or a
sliding-window band; SciPy's softmax/logsumexp on the visible entries of a
row; and invariants (weights sum to 1, outputs inside the convex hull of the
visible values, invariance under a joint permutation of keys and mask
columns).
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp, softmax

import oracle


def rand_case(rng, Hq, Hkv, S, D, a, n, p_sep):
    q = rng.standard_normal((Hq, S, D))
    k = rng.standard_normal((Hkv, S, D))
    v = rng.standard_normal((Hkv, S, D))
    flags = rng.random(S) < p_sep
    return q, k, v, flags


def loop_attention(q, k, v, flags, a, n, scale):
    Hq, S, D = q.shape
    G = Hq // k.shape[0]
    out = np.zeros_like(q)
    for h in range(Hq):
        g = h // G
        for i in range(S):
            js = [j for j in range(i + 1) if j < a or i - j < n or flags[j]]
            sc = [scale * sum(q[h, i, d] * k[g, j, d] for d in range(D)) for j in js]
            m = max(sc)
            e = [math.exp(x - m) for x in sc]
            z = sum(e)
            for d in range(D):
                out[h, i, d] = sum(e[t] * v[g, js[t], d] for t in range(len(js))) / z
    return out


def test_triple_loop_brute_force():
    rng = np.random.default_rng(21)
    for (Hq, Hkv, S, D, a, n, ps) in [(2, 1, 17, 4, 2, 3, 0.3), (4, 2, 23, 3, 0, 1, 0.5),
                                      (1, 1, 12, 5, 4, 20, 0.0), (2, 2, 19, 2, 1, 4, 1.0)]:
        q, k, v, flags = rand_case(rng, Hq, Hkv, S, D, a, n, ps)
        scale = 1.0 / math.sqrt(D)
        M = oracle.sep_mask(flags, a, n)
        o, _ = oracle.attention(q, k, v, M, scale)
        assert np.allclose(o, loop_attention(q, k, v, flags, a, n, scale), atol=1e-12, rtol=0)


def _sdpa(q, k, v, scale, causal=False, mask=None):
    G = q.shape[0] // k.shape[0]
    kk = torch.from_numpy(np.repeat(k, G, axis=0))
    vv = torch.from_numpy(np.repeat(v, G, axis=0))
    qq = torch.from_numpy(q)
    am = None if mask is None else torch.from_numpy(mask)
    return torch.nn.functional.scaled_dot_product_attention(
        qq, kk, vv, attn_mask=am, is_causal=causal, scale=scale).numpy()


def test_long_window_is_causal_attention():
    rng = np.random.default_rng(23)
    for (Hq, Hkv, S, D) in [(4, 2, 64, 16), (2, 2, 96, 8), (8, 2, 33, 32)]:
        q, k, v, flags = rand_case(rng, Hq, Hkv, S, D, 4, S, 0.2)
        scale = 1 / math.sqrt(D)
        o, _ = oracle.attention(q, k, v, oracle.sep_mask(flags, 4, S), scale)
        assert np.allclose(o, _sdpa(q, k, v, scale, causal=True), atol=1e-12, rtol=0)


def test_no_separators_no_initial_is_sliding_window():
    rng = np.random.default_rng(29)
    S, D = 80, 16
    q, k, v, _ = rand_case(rng, 2, 1, S, D, 0, 1, 0.0)
    for n in (1, 7, 33):
        band = np.tri(S, S, 0, dtype=bool) & ~np.tri(S, S, -n, dtype=bool)
        o, _ = oracle.attention(q, k, v, oracle.sep_mask(np.zeros(S, bool), 0, n), 0.25)
        assert np.allclose(o, _sdpa(q, k, v, 0.25, mask=band), atol=1e-12, rtol=0)


def test_weights_rows_sum_to_one_and_match_scipy():
    rng = np.random.default_rng(31)
    S, D, a, n = 70, 8, 3, 9
    q, k, v, flags = rand_case(rng, 2, 1, S, D, a, n, 0.15)
    M = oracle.sep_mask(flags, a, n)
    o, lse, w = oracle.attention(q, k, v, M, 0.5, return_weights=True)
    assert np.all(np.abs(w.sum(-1) - 1.0) < 1e-12)
    assert np.all(w[:, ~M] == 0.0)
    for h in range(2):
        for i in range(S):
            js = np.flatnonzero(M[i])
            sc = 0.5 * (k[0, js] @ q[h, i])
            assert np.allclose(w[h, i, js], softmax(sc), atol=1e-14, rtol=0)
            assert abs(lse[h, i] - logsumexp(sc)) < 1e-12


def test_outputs_in_convex_hull_of_visible_values():
    rng = np.random.default_rng(37)
    S, D, a, n = 90, 6, 4, 5
    q, k, v, flags = rand_case(rng, 3, 1, S, D, a, n, 0.1)
    q *= 4.0  # sharp softmax
    M = oracle.sep_mask(flags, a, n)
    o, _ = oracle.attention(q, k, v, M, 1.0)
    for i in range(S):
        vis = v[0, M[i]]
        assert np.all(o[:, i] <= vis.max(0) + 1e-12) and np.all(o[:, i] >= vis.min(0) - 1e-12)


def test_joint_key_permutation_invariance():
    rng = np.random.default_rng(41)
    S, D, a, n = 50, 8, 2, 6
    q, k, v, flags = rand_case(rng, 2, 2, S, D, a, n, 0.2)
    M = oracle.sep_mask(flags, a, n)
    o, _ = oracle.attention(q, k, v, M, 0.3)
    perm = rng.permutation(S)
    # permute keys/values and mask columns only (queries stay in place)
    o2 = np.empty_like(o)
    for h in range(2):
        x = 0.3 * q[h] @ k[h][perm].T
        x[~M[:, perm]] = -np.inf
        o2[h] = softmax(x, axis=1) @ v[h][perm]
    assert np.allclose(o, o2, atol=1e-12, rtol=0)


def test_attention_rows_equals_full():
    rng = np.random.default_rng(43)
    S, D, a, n = 120, 16, 4, 10
    q, k, v, flags = rand_case(rng, 4, 2, S, D, a, n, 0.1)
    M = oracle.sep_mask(flags, a, n)
    o, lse = oracle.attention(q, k, v, M, 0.25)
    rows = [0, 1, 5, 63, 119]
    o2, lse2 = oracle.attention_rows(q[:, rows], k, v, oracle.mask_rows(flags, a, n, rows), 0.25,
                                     kv_head_of=[h // 2 for h in range(4)])
    assert np.allclose(o[:, rows], o2, atol=1e-13, rtol=0)
    assert np.allclose(lse[:, rows], lse2, atol=1e-13, rtol=0)


def test_decode_over_full_prefix_is_causal_row():
    rng = np.random.default_rng(47)
    S, D = 40, 8
    q, k, v, flags = rand_case(rng, 4, 2, S, D, 0, S, 0.0)
    ref = _sdpa(q, k, v, 0.2, causal=True)
    for t in (0, 1, 17, S - 1):
        o, _ = oracle.decode_attention(q[:, t], k[:, :t + 1], v[:, :t + 1], 0.2)
        assert np.allclose(o, ref[:, t], atol=1e-12, rtol=0)


# ----------------------------------------------------------- planted mistakes
def _mut_no_scale(q, k, v, M, scale):
    return oracle.attention(q, k, v, M, 1.0)[0]


def _mut_wrong_gqa(q, k, v, M, scale):
    Hq = q.shape[0]
    Hkv = k.shape[0]
    out = np.empty_like(q)
    for h in range(Hq):
        g = h % Hkv                        # interleaved instead of grouped
        x = scale * q[h] @ k[g].T
        x[~M] = -np.inf
        out[h] = softmax(x, axis=1) @ v[g]
    return out


def _mut_transposed_mask(q, k, v, M, scale):
    Mt = M.T | np.eye(M.shape[0], dtype=bool)
    return oracle.attention(q, k, v, Mt, scale)[0]


@pytest.mark.parametrize("mutant", [_mut_no_scale, _mut_wrong_gqa, _mut_transposed_mask])
def test_planted_attention_mistakes_fail_the_pin(mutant):
    rng = np.random.default_rng(53)
    q, k, v, flags = rand_case(rng, 4, 2, 14, 3, 2, 3, 0.3)
    M = oracle.sep_mask(flags, 2, 3)
    ref = loop_attention(q, k, v, flags, 2, 3, 1 / math.sqrt(3))
    assert not np.allclose(mutant(q, k, v, M, 1 / math.sqrt(3)), ref, atol=1e-9)


# ------------------------------------------------------------ backward pass
def _loss(q, k, v, M, scale, dout):
    out, _ = oracle.attention(q, k, v, M, scale)
    return float((out * dout).sum())


def test_backward_matches_finite_differences():
    """dL/dx for L = sum(dout * O), by central differences of the forward
    oracle (no gradient formula involved), on tiny GQA cases."""
    rng = np.random.default_rng(131)
    for Hq, Hkv, S, D, a, n in [(2, 1, 7, 3, 1, 2), (4, 2, 9, 2, 2, 3), (2, 2, 6, 4, 0, 1)]:
        q, k, v, flags = rand_case(rng, Hq, Hkv, S, D, a, n, 0.3)
        M = oracle.sep_mask(flags, a, n)
        dout = rng.standard_normal((Hq, S, D))
        scale = 0.7
        dq, dk, dv, _ = oracle.attention_backward(q, k, v, M, scale, dout)
        eps = 1e-6
        for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp = x.copy(); xp[idx] += eps
                xm = x.copy(); xm[idx] -= eps
                args_p = dict(q=q, k=k, v=v); args_p[name] = xp
                args_m = dict(q=q, k=k, v=v); args_m[name] = xm
                num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], M, scale, dout) -
                            _loss(args_m["q"], args_m["k"], args_m["v"], M, scale, dout)) / (2 * eps)
            assert np.max(np.abs(num - g)) < 1e-7 * max(1.0, np.max(np.abs(g))), (name, Hq, Hkv, S)


def test_backward_matches_torch_autograd():
    """PyTorch's float64 autograd through a dense masked softmax attention
    written here with torch ops (GQA by repeating the kv heads)."""
    rng = np.random.default_rng(137)
    Hq, Hkv, S, D, a, n = 8, 2, 40, 16, 3, 5
    q, k, v, flags = rand_case(rng, Hq, Hkv, S, D, a, n, 0.15)
    M = oracle.sep_mask(flags, a, n)
    dout = rng.standard_normal((Hq, S, D))
    scale = 1 / math.sqrt(D)
    dq, dk, dv, delta = oracle.attention_backward(q, k, v, M, scale, dout)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = Hq // Hkv
    kk = tk.repeat_interleave(G, dim=0)
    vv = tv.repeat_interleave(G, dim=0)
    x = scale * (tq @ kk.transpose(1, 2))
    x = x.masked_fill(~torch.tensor(M), float("-inf"))
    out = torch.softmax(x, dim=-1) @ vv
    (out * torch.tensor(dout)).sum().backward()
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-11)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-11)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-11)
    assert np.allclose(delta, (out.detach().numpy() * dout).sum(-1), atol=1e-12)


def _bwd_no_delta(q, k, v, M, scale, dout):
    """dS = P * dP, the softmax's row term forgotten"""
    _, _, P = oracle.attention(q, k, v, M, scale, return_weights=True)
    G = q.shape[0] // k.shape[0]
    dq = np.stack([scale * ((P[h] * (dout[h] @ v[h // G].T)) @ k[h // G]) for h in range(q.shape[0])])
    return dq


def _bwd_dq_no_scale(q, k, v, M, scale, dout):
    dq, _, _, _ = oracle.attention_backward(q, k, v, M, scale, dout)
    return dq / scale


def _bwd_dk_last_head_only(q, k, v, M, scale, dout):
    """dK from the last query head of each group instead of their sum"""
    G = q.shape[0] // k.shape[0]
    _, dk1, _, _ = oracle.attention_backward(q[G - 1::G], k, v, M, scale, dout[G - 1::G])
    return dk1


@pytest.mark.parametrize("mutant,which", [(_bwd_no_delta, 0), (_bwd_dq_no_scale, 0),
                                          (_bwd_dk_last_head_only, 1)])
def test_planted_backward_mistakes_fail_the_pin(mutant, which):
    rng = np.random.default_rng(139)
    Hq, Hkv, S, D, a, n = 4, 2, 8, 3, 1, 2
    q, k, v, flags = rand_case(rng, Hq, Hkv, S, D, a, n, 0.3)
    M = oracle.sep_mask(flags, a, n)
    dout = rng.standard_normal((Hq, S, D))
    scale = 0.7
    x = (q, k)[which]
    g = mutant(q, k, v, M, scale, dout)
    eps = 1e-6
    num = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy(); xp[idx] += eps
        xm = x.copy(); xm[idx] -= eps
        if which == 0:
            num[idx] = (_loss(xp, k, v, M, scale, dout) - _loss(xm, k, v, M, scale, dout)) / (2 * eps)
        else:
            num[idx] = (_loss(q, xp, v, M, scale, dout) - _loss(q, xm, v, M, scale, dout)) / (2 * eps)
    assert np.max(np.abs(num - g)) > 1e-4


def test_backward_delta_uses_the_given_output():
    rng = np.random.default_rng(149)
    q, k, v, flags = rand_case(rng, 2, 1, 12, 4, 1, 3, 0.3)
    M = oracle.sep_mask(flags, 1, 3)
    dout = rng.standard_normal((2, 12, 4))
    exact, _ = oracle.attention(q, k, v, M, 0.5)
    a = oracle.attention_backward(q, k, v, M, 0.5, dout)
    b = oracle.attention_backward(q, k, v, M, 0.5, dout, out=exact)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    c = oracle.attention_backward(q, k, v, M, 0.5, dout, out=exact + 0.01)
    assert np.allclose(c[3], a[3] + 0.01 * dout.sum(-1))
    assert np.array_equal(c[2], a[2])                     # dv does not involve delta


@pytest.mark.parametrize("G,S,a,n,p_sep,chunk", [(3, 41, 2, 5, 0.2, 7), (1, 30, 0, 1, 0.0, 512),
                                                  (4, 25, 30, 3, 0.5, 4)])
def test_backward_sampled_matches_full_backward(G, S, a, n, p_sep, chunk):
    """The row/column form agrees with attention_backward (itself pinned by
    finite differences and autograd) on every sampled row and key, with a
    stored output that differs from the exact one."""
    rng = np.random.default_rng(G * 1000 + S)
    q, k, v, flags = rand_case(rng, G, 1, S, 8, a, n, p_sep)
    M = oracle.sep_mask(flags, a, n)
    dout = rng.standard_normal((G, S, 8))
    exact, _ = oracle.attention(q, k, v, M, 0.3)
    stored = exact + 1e-3 * rng.standard_normal(exact.shape)
    rq, rk, rv, _ = oracle.attention_backward(q, k, v, M, 0.3, dout, out=stored)
    rows = sorted(set([0, S - 1] + rng.integers(0, S, 6).tolist()))
    keys = sorted(set([0, 1, S - 1] + rng.integers(0, S, 6).tolist() + np.flatnonzero(flags)[:3].tolist()))
    sq, sk, sv = oracle.attention_backward_sampled(q, k[0], v[0], dout, stored, M, 0.3, rows, keys,
                                                   row_chunk=chunk)
    assert np.allclose(sq, rq[:, rows], rtol=1e-12, atol=1e-12)
    assert np.allclose(sk, rk[0, keys], rtol=1e-12, atol=1e-12)
    assert np.allclose(sv, rv[0, keys], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- chunk attention
def _entries(ids, k, v, positions):
    return [oracle.Entry(int(p), int(ids[p]), k[:, p], v[:, p]) for p in positions]


def _chunk_case(rng, Hq, Hkv, T, D, p_sep):
    ids = np.where(rng.random(T) < p_sep, rng.integers(0, 4, T), rng.integers(4, 100, T))
    q = rng.standard_normal((Hq, T, D))
    k = rng.standard_normal((Hkv, T, D))
    v = rng.standard_normal((Hkv, T, D))
    return ids, q, k, v


@pytest.mark.parametrize("a,n,C", [(2, 5, 7), (0, 1, 12), (3, 40, 9)])
def test_chunk_on_an_empty_cache_is_prefill(a, n, C):
    rng = np.random.default_rng(a * 100 + n)
    ids, q, k, v = _chunk_case(rng, 4, 2, C, 8, 0.3)
    o, l = oracle.chunk_attention([], q, k, v, ids, 0, a, n, range(4), 0.4)
    M = oracle.sep_mask(oracle.is_sep(ids, range(4)), a, n)
    o2, l2 = oracle.attention(q, k, v, M, 0.4)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-13)


@pytest.mark.parametrize("t,C,a,n", [(30, 10, 3, 6), (5, 20, 2, 3), (50, 1, 4, 9)])
def test_chunk_without_eviction_is_prefill_rows(t, C, a, n):
    """A cache that still holds every past token: the chunk's rows are rows
    t..t+C-1 of the prefill over the whole sequence."""
    rng = np.random.default_rng(t + C)
    ids, q, k, v = _chunk_case(rng, 6, 3, t + C, 8, 0.25)
    entries = _entries(ids, k, v, rng.permutation(t))          # any order
    o, l = oracle.chunk_attention(entries, q[:, t:], k[:, t:], v[:, t:], ids[t:], t, a, n, range(4), 0.3)
    M = oracle.sep_mask(oracle.is_sep(ids, range(4)), a, n)
    o2, l2 = oracle.attention(q, k, v, M, 0.3)
    assert np.allclose(o, o2[:, t:], atol=1e-12) and np.allclose(l, l2[:, t:], atol=1e-12)


def test_chunk_of_one_with_a_wide_window_is_decode():
    """C = 1 and a window past every retained entry: the decode step over
    the cache's keys plus the token itself."""
    rng = np.random.default_rng(3)
    T = 200
    ids, q, k, v = _chunk_case(rng, 4, 2, T + 1, 8, 0.2)
    sim = oracle.CacheSim(2, 5, 4, 9, range(4))
    sim.push_many([oracle.Entry(p, int(ids[p]), k[:, p], v[:, p]) for p in range(T)])
    o, _ = oracle.chunk_attention(sim.keys(), q[:, T:], k[:, T:], v[:, T:], ids[T:], T, 2, T + 1, range(4), 0.5)
    keys = [e.pos for e in sim.keys()] + [T]
    o2, _ = oracle.decode_attention(q[:, T], k[:, keys], v[:, keys], 0.5)
    assert np.allclose(o[:, 0], o2, atol=1e-13)


def test_chunk_brute_force_loop():
    """Tiny case with an arbitrary retained subset: a per-row Python loop."""
    rng = np.random.default_rng(17)
    t, C, a, n, D = 14, 5, 2, 3, 4
    ids, q, k, v = _chunk_case(rng, 2, 1, t + C, D, 0.4)
    kept = sorted(rng.choice(t, 8, replace=False).tolist())
    o, _ = oracle.chunk_attention(_entries(ids, k, v, kept), q[:, t:], k[:, t:], v[:, t:], ids[t:], t, a, n,
                                  range(4), 0.7)
    for h in range(2):
        for i in range(C):
            tau = t + i
            js = [p for p in kept + list(range(t, tau + 1))
                  if p < a or ids[p] < 4 or tau - p < n]
            s = [0.7 * float(np.dot(q[h, tau], k[0, p])) for p in js]
            m = max(s)
            w = [math.exp(x - m) for x in s]
            ref = sum(wi / sum(w) * v[0, p] for wi, p in zip(w, js))
            assert np.allclose(o[h, i], ref, atol=1e-12)


def test_chunk_planted_mistakes_are_caught():
    rng = np.random.default_rng(19)
    t, C, a, n = 40, 12, 2, 5
    ids, q, k, v = _chunk_case(rng, 2, 1, t + C, 8, 0.3)
    kept = sorted(rng.choice(t, 25, replace=False).tolist())
    good, _ = oracle.chunk_attention(_entries(ids, k, v, kept), q[:, t:], k[:, t:], v[:, t:], ids[t:], t, a, n,
                                     range(4), 0.5)
    wider, _ = oracle.chunk_attention(_entries(ids, k, v, kept), q[:, t:], k[:, t:], v[:, t:], ids[t:], t, a,
                                      n + 1, range(4), 0.5)
    assert not np.allclose(good, wider, atol=1e-6)             # the window's edge matters
    nosep, _ = oracle.chunk_attention(_entries(ids, k, v, kept), q[:, t:], k[:, t:], v[:, t:], ids[t:], t, a,
                                      n, [], 0.5)
    assert not np.allclose(good, nosep, atol=1e-6)             # separators in the cache and the chunk
