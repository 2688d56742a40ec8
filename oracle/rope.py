"""Rotary position embedding with position shifting, for streaming decode.

Test infrastructure only (see the package docstring for who may import it).

P1 "Streaming-SepLLM" and its note that streaming is not an ordinary
evaluation entry: the streaming setting needs positional-encoding shifting,
which the code base implements for Llama in its pos_shift module. The pages
give no formula. The readings, in the order they are applied:

* RoPE as published (Su et al., "RoFormer: Enhanced Transformer with Rotary
  Position Embedding", 2021, section 3.4): feature pair i of a vector at
  position m is rotated by the angle m * theta_i, theta_i = base^(-2 i / D),
  i = 0 .. D/2 - 1.
* Llama's arrangement of the pairs (the pages name Llama's module): pair i
  is (x_i, x_{i + D/2}), rotated as
      x_i'       = x_i cos(m theta_i) - x_{i+D/2} sin(m theta_i)
      x_{i+D/2}' = x_{i+D/2} cos(m theta_i) + x_i sin(m theta_i).
* Shifting: keys are cached before rotation. At each decode step the
  retained keys take the positions 0 .. L-1 in cache order (initial block,
  separators, recent window, each oldest first: CacheSim.keys()), and the
  current token, query and key alike, takes position L.
* Precision: the rotated query and keys are held in bfloat16, the format the
  cache stores them in, before the attention products (round to nearest,
  ties to even, applied once to the exact rotation).
"""
from __future__ import annotations

import numpy as np

from .attention import decode_attention


def rope_angles(positions, D: int, base: float) -> np.ndarray:
    """Angles m * theta_i, [len(positions), D/2], float64."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / D)
    return np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]


def rotate(x: np.ndarray, positions, base: float) -> np.ndarray:
    """RoPE of x [..., P, D] (rows at the given P positions), float64."""
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    h = D // 2
    ang = rope_angles(positions, D, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even; values in bfloat16's normal range."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def decode_attention_shifted(q, keys_k, keys_v, scale: float, base: float, to_bf16: bool = True):
    """One decode step with position shifting.

    q [Hq, D] (the current token's query, before rotation); keys_k/keys_v
    [Hkv, L + 1, D], the retained keys in cache order followed by the current
    token, before rotation. Key u is rotated to position u and the query to
    position L; with ``to_bf16`` both are rounded to bfloat16. Returns o [Hq, D]
    and lse [Hq] (decode_attention on the rotated operands)."""
    keys_k = np.asarray(keys_k, np.float64)
    n = keys_k.shape[1]
    qr = rotate(np.asarray(q, np.float64)[:, None, :], [n - 1], base)[:, 0]
    kr = rotate(keys_k, np.arange(n), base)
    if to_bf16:
        qr, kr = round_bf16(qr), round_bf16(kr)
    return decode_attention(qr, kr, keys_v, scale)
