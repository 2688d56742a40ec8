"""Masked scaled-softmax attention in float64.

Test infrastructure only (see the package docstring for who may import it).

P2 §1.2: scores are the scaled dot products of queries with keys; entries
where M = 0 are set to -inf before the softmax; the softmax weights then
average the values. The pages say "scaled" without the factor; callers pass
``scale`` (1/sqrt(D) in every workload here).

Grouped-query attention: with Hq query heads and Hkv key/value heads,
query head h reads key/value head h // (Hq // Hkv). The pages do not
discuss GQA; this is the usual grouping of consecutive query heads.
"""
from __future__ import annotations

import numpy as np


def _softmax_rows(x: np.ndarray):
    """Row softmax of x (-inf allowed, at least one finite entry per row).
    Returns (weights, row max, row sum of exp)."""
    mx = x.max(axis=-1, keepdims=True)
    e = np.exp(x - mx)
    den = e.sum(axis=-1, keepdims=True)
    return e / den, mx[..., 0], den[..., 0]


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, M: np.ndarray, scale: float,
              return_weights: bool = False):
    """Prefill attention of one sequence.

    q [Hq, S, D], k/v [Hkv, S, D] (float64), M [S, S] bool.
    Returns O [Hq, S, D] and lse [Hq, S] (natural log of the softmax
    denominator plus the row max), and the weights [Hq, S, S] on request."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Hq, S, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    out = np.empty((Hq, S, D))
    lse = np.empty((Hq, S))
    weights = np.empty((Hq, S, S)) if return_weights else None
    for h in range(Hq):
        g = h // G
        x = scale * (q[h] @ k[g].T)
        x[~M] = -np.inf
        p, mx, den = _softmax_rows(x)
        out[h] = p @ v[g]
        lse[h] = mx + np.log(den)
        if return_weights:
            weights[h] = p
    if return_weights:
        return out, lse, weights
    return out, lse


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, M: np.ndarray, scale: float,
                       dout: np.ndarray, out: np.ndarray = None):
    """Gradients of the prefill attention of one sequence (the training use of
    Sep-Attention: P1 "Training-SepLLM" trains through the same mask).

    For L = sum(dout * O), with P the softmax weights of query head h over
    kv head g = h // G (P2 §1.2: scaled scores, -inf where M = 0):
        dV_g  = sum over the G heads h of P_h^T dout_h
        dP_h  = dout_h V_g^T
        dS_h  = P_h * (dP_h - rowsum(dout_h * O_h))
        dQ_h  = scale * dS_h K_g
        dK_g  = scale * sum over the heads h of dS_h^T Q_h
    (the chain rule through the row softmax: d softmax = P * (dP - (P dP)
    summed over the row), and rowsum(P * dP) = rowsum(dout * O)).
    q/dout [Hq, S, D], k/v [Hkv, S, D], M [S, S] bool; float64. ``out``, when
    given, is the forward output a caller stored (e.g. rounded to bf16):
    delta is then rowsum(dout * out), as a backward that is handed that
    tensor computes it; by default it is the exact O.
    Returns dq [Hq, S, D], dk, dv [Hkv, S, D] and delta [Hq, S]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    Hq, S, D = q.shape
    Hkv = k.shape[0]
    G = Hq // Hkv
    exact, _, P = attention(q, k, v, M, scale, return_weights=True)
    out = exact if out is None else np.asarray(out, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = (dout * out).sum(axis=-1)
    for h in range(Hq):
        g = h // G
        dv[g] += P[h].T @ dout[h]
        dP = dout[h] @ v[g].T
        dS = P[h] * (dP - delta[h][:, None])
        dq[h] = scale * (dS @ k[g])
        dk[g] += scale * (dS.T @ q[h])
    return dq, dk, dv, delta


def attention_rows(q_rows, k, v, M_rows, scale, kv_head_of):
    """Prefill attention for a subset of query rows.

    q_rows [H', R, D]; k/v [Hkv, S, D]; M_rows [R, S] bool (rows of M for the
    same R queries); kv_head_of[i] is the key/value head that q_rows[i] reads.
    Returns O [H', R, D] and lse [H', R]."""
    q_rows = np.asarray(q_rows, np.float64)
    H, R, D = q_rows.shape
    out = np.empty((H, R, D))
    lse = np.empty((H, R))
    for i in range(H):
        g = int(kv_head_of[i])
        x = scale * (q_rows[i] @ np.asarray(k[g], np.float64).T)
        x[~M_rows] = -np.inf
        p, mx, den = _softmax_rows(x)
        out[i] = p @ np.asarray(v[g], np.float64)
        lse[i] = mx + np.log(den)
    return out, lse


def attention_backward_sampled(q, k, v, dout, out, M, scale, rows, keys, row_chunk: int = 512):
    """Selected elements of attention_backward for one key/value head and the
    G query heads that read it, at sizes where the [S, S] weights of every
    head do not fit.

    q, dout, out [G, S, D]; k, v [S, D]; M [S, S] bool; ``out`` is the
    forward output the backward is handed (delta = rowsum(dout * out), as in
    attention_backward). Returns dq[:, rows] [G, R, D], dk[keys] and
    dv[keys] [J, D].

    Same definitions as attention_backward, evaluated on rows and columns:
    the lse of every query row comes from attention_rows (row chunks of M);
    P_ij = exp(scale q_i.k_j - lse_i) where M[i, j], else 0; dP_ij =
    dout_i.v_j; dS_ij = P_ij (dP_ij - delta_i). A query row gives dq_i =
    scale sum_j dS_ij k_j; a key column gives dv_j = sum_h sum_i P_ij dout_i
    and dk_j = scale sum_h sum_i dS_ij q_i."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    dout = np.asarray(dout, np.float64)
    out = np.asarray(out, np.float64)
    G, S, D = q.shape
    rows = np.asarray(list(rows), dtype=np.int64)
    keys = np.asarray(list(keys), dtype=np.int64)
    lse = np.empty((G, S))
    for r0 in range(0, S, row_chunk):
        r1 = min(S, r0 + row_chunk)
        _, lse[:, r0:r1] = attention_rows(q[:, r0:r1], k[None], v[None], M[r0:r1], scale, [0] * G)
    delta = (dout * out).sum(axis=-1)
    dq = np.empty((G, len(rows), D))
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    Mc = M[:, keys]
    for h in range(G):
        x = scale * (q[h, rows] @ k.T)
        x[~M[rows]] = -np.inf
        Pr = np.exp(x - lse[h, rows][:, None])
        dq[h] = scale * ((Pr * (dout[h, rows] @ v.T - delta[h, rows][:, None])) @ k)
        x = scale * (q[h] @ k[keys].T)
        x[~Mc] = -np.inf
        Pc = np.exp(x - lse[h][:, None])
        dv += Pc.T @ dout[h]
        dk += scale * ((Pc * (dout[h] @ v[keys].T - delta[h][:, None])).T @ q[h])
    return dq, dk, dv


def chunk_attention(cache_entries, q, k, v, ids, t: int, a: int, n: int, sep_ids, scale: float):
    """Attention of a chunk of C new tokens over a live cache and the chunk.

    P1 "SepAttention": build_generate_mask applies the prefill keep rule
    (initial OR separator OR local window, AND causal) to the rows of new
    queries, one row in plain decode, C rows here; P1 names a local window
    for generation (generate_local_window_size) next to the prefill one, and
    a window per layer, so n is an argument of each call. P2 §1.3: the cache
    holds only what was retained, so the keys are the retained entries plus
    the chunk.

    cache_entries: the retained entries (any order), each an Entry with pos,
    tok and k, v rows [Hkv, D]; q [Hq, C, D], k/v [Hkv, C, D], ids [C]: the
    chunk, at positions t .. t+C-1. Query tau = t + i sees key j (position
    p, token id x) iff p <= tau and (p < a or x is a separator or
    tau - p < n). Returns O [Hq, C, D] and lse [Hq, C]."""
    q = np.asarray(q, np.float64)
    Hq, C, D = q.shape
    Hkv = np.asarray(k).shape[0]
    pos = np.array([e.pos for e in cache_entries] + list(range(t, t + C)), dtype=np.int64)
    tok = np.array([e.tok for e in cache_entries] + list(np.asarray(ids)), dtype=np.int64)
    kk = np.concatenate([np.asarray([e.k for e in cache_entries], np.float64).reshape(-1, Hkv, D)
                         .transpose(1, 0, 2), np.asarray(k, np.float64)], axis=1)
    vv = np.concatenate([np.asarray([e.v for e in cache_entries], np.float64).reshape(-1, Hkv, D)
                         .transpose(1, 0, 2), np.asarray(v, np.float64)], axis=1)
    sep = np.isin(tok, np.asarray(list(sep_ids), dtype=np.int64))
    tau = np.arange(t, t + C, dtype=np.int64)[:, None]
    p = pos[None, :]
    M = (p <= tau) & ((p < a) | sep[None, :] | (tau - p < n))
    G = Hq // Hkv
    return attention_rows(q, kk, vv, M, scale, [h // G for h in range(Hq)])


def decode_attention(q: np.ndarray, keys_k: np.ndarray, keys_v: np.ndarray, scale: float):
    """Attention of one decode step over an explicit key list, no further mask.

    q [Hq, D]; keys_k/keys_v [Hkv, L, D] (the retained keys in any order,
    the current token included). P1 "SepAttention" (build_generate_mask: the
    same keep rule for a single query) and P2 §1.3 (only the kept KV are
    read). Returns o [Hq, D] and lse [Hq]."""
    q = np.asarray(q, np.float64)
    keys_k = np.asarray(keys_k, np.float64)
    keys_v = np.asarray(keys_v, np.float64)
    Hq, D = q.shape
    Hkv = keys_k.shape[0]
    G = Hq // Hkv
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for h in range(Hq):
        g = h // G
        x = scale * (keys_k[g] @ q[h])
        p, mx, den = _softmax_rows(x[None, :])
        out[h] = p[0] @ keys_v[g]
        lse[h] = mx[0] + np.log(den[0])
    return out, lse
