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
