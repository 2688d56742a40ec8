"""Pins of the oracle's rotary position embedding and position shifting.

References other than the oracle itself: the closed form of a plane
rotation by 1 radian; RoPE's complex form (pair i as the complex number
x_i + j x_{i+D/2}, multiplied by exp(j m theta_i)); the invariants of a
rotation (position 0 is the identity, norms are kept, a dot product depends
only on the position difference); PyTorch's float32 -> bfloat16 conversion
and hand-picked ties for the rounding; and, for the shifted decode step, the
relative form <R(a) q, R(b) k> = <q, R(b - a) k> written as a loop over keys.
Planted mistakes (pairs interleaved, the sign of the sine, the exponent of
theta, the query at position 0) each fail one of these.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def complex_rope(x, pos, base):
    D = x.shape[-1]
    h = D // 2
    z = x[..., :h] + 1j * x[..., h:]
    theta = np.array([base ** (-2.0 * i / D) for i in range(h)])
    z = z * np.exp(1j * np.asarray(pos, np.float64)[:, None] * theta[None, :])
    return np.concatenate([z.real, z.imag], axis=-1)


def test_rotation_by_one_radian():
    # D = 2: theta_0 = base^0 = 1, so position 1 turns (1, 0) by 1 rad
    y = oracle.rotate(np.array([[1.0, 0.0]]), [1], 500000.0)
    assert np.allclose(y, [[0.5403023058681398, 0.8414709848078965]], atol=1e-15)
    y = oracle.rotate(np.array([[0.0, 2.0]]), [3], 10.0)
    assert np.allclose(y, [[-2 * math.sin(3.0), 2 * math.cos(3.0)]], atol=1e-14)


def test_second_pair_frequency():
    # D = 4, base 100: theta_1 = 100^(-1/2) = 0.1; pair 1 is (x_1, x_3)
    y = oracle.rotate(np.array([[0.0, 1.0, 0.0, 0.0]]), [5], 100.0)
    assert np.allclose(y, [[0.0, math.cos(0.5), 0.0, math.sin(0.5)]], atol=1e-15)


@pytest.mark.parametrize("D,base", [(8, 10000.0), (64, 500000.0), (128, 500000.0)])
def test_complex_form(D, base):
    rng = np.random.default_rng(D)
    x = rng.standard_normal((3, 17, D))
    pos = rng.integers(0, 70000, 17)
    assert np.allclose(oracle.rotate(x, pos, base), complex_rope(x, pos, base), atol=1e-9)


def test_rotation_invariants():
    rng = np.random.default_rng(5)
    D = 64
    q = rng.standard_normal((40, D))
    k = rng.standard_normal((40, D))
    assert np.array_equal(oracle.rotate(q, np.zeros(40), 1e4), q)
    pa = rng.integers(0, 5000, 40)
    pb = rng.integers(0, 5000, 40)
    qa = oracle.rotate(q, pa, 1e4)
    h = D // 2
    assert np.allclose(qa[:, :h] ** 2 + qa[:, h:] ** 2, q[:, :h] ** 2 + q[:, h:] ** 2)
    dots = np.sum(qa * oracle.rotate(k, pb, 1e4), axis=-1)
    c = 1234
    dots_c = np.sum(oracle.rotate(q, pa + c, 1e4) * oracle.rotate(k, pb + c, 1e4), axis=-1)
    assert np.allclose(dots, dots_c, atol=1e-9)


def test_round_bf16_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-20, 20, 100000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    u = 2.0 ** -8                          # half a bfloat16 ulp at 1
    assert oracle.round_bf16(np.array([1 + u]))[0] == 1.0
    assert oracle.round_bf16(np.array([1 + 3 * u]))[0] == 1 + 4 * u
    assert oracle.round_bf16(np.array([-(1 + 3 * u)]))[0] == -(1 + 4 * u)
    assert oracle.round_bf16(np.array([1 + u * 1.0001]))[0] == 1 + 2 * u
    assert oracle.round_bf16(np.array([0.0]))[0] == 0.0


def relative_loop(q, keys_k, keys_v, scale, base):
    """Score of key u = <q, R((u - n + 1) theta) k_u>: the query stays put and
    each key turns by its offset from the query's position; no rounding."""
    Hq, D = q.shape
    Hkv, n, _ = keys_k.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    for hq in range(Hq):
        g = hq // G
        s = []
        for u in range(n):
            kr = oracle.rotate(keys_k[g, u][None], [u - (n - 1)], base)[0]
            s.append(scale * float(np.dot(q[hq], kr)))
        m = max(s)
        wts = [math.exp(x - m) for x in s]
        tot = sum(wts)
        out[hq] = sum(wt / tot * keys_v[g, u] for u, wt in enumerate(wts))
    return out


@pytest.mark.parametrize("Hq,Hkv,n,D", [(4, 2, 9, 8), (3, 1, 1, 4), (2, 2, 30, 16)])
def test_shifted_decode_matches_relative_form(Hq, Hkv, n, D):
    rng = np.random.default_rng(Hq * 100 + n)
    q = rng.standard_normal((Hq, D))
    kk = rng.standard_normal((Hkv, n, D))
    vv = rng.standard_normal((Hkv, n, D))
    o, lse = oracle.decode_attention_shifted(q, kk, vv, 0.4, 10000.0, to_bf16=False)
    assert np.allclose(o, relative_loop(q, kk, vv, 0.4, 10000.0), atol=1e-12)
    if n == 1:
        assert np.allclose(o, np.repeat(vv[:, 0], Hq // Hkv, axis=0))


def test_shifted_decode_rounds_both_operands():
    rng = np.random.default_rng(11)
    q = rng.standard_normal((2, 16))
    kk = rng.standard_normal((1, 12, 16))
    vv = rng.standard_normal((1, 12, 16))
    o, _ = oracle.decode_attention_shifted(q, kk, vv, 0.25, 500000.0)
    qr = oracle.round_bf16(oracle.rotate(q[:, None], [11], 500000.0)[:, 0])
    kr = oracle.round_bf16(oracle.rotate(kk, np.arange(12), 500000.0))
    o2, _ = oracle.decode_attention(qr, kr, vv, 0.25)
    assert np.array_equal(o, o2)
    o3, _ = oracle.decode_attention_shifted(q, kk, vv, 0.25, 500000.0, to_bf16=False)
    assert 0 < np.max(np.abs(o - o3)) < 0.05


def test_planted_mistakes_are_caught(monkeypatch):
    rng = np.random.default_rng(13)
    x = rng.standard_normal((5, 16))
    pos = rng.integers(1, 900, 5)
    good = complex_rope(x, pos, 10000.0)

    def interleaved(x, positions, base):          # pairs (2i, 2i+1) instead of (i, i + D/2)
        ang = oracle.rope_angles(positions, x.shape[-1], base)
        y = x.copy()
        y[..., 0::2] = x[..., 0::2] * np.cos(ang) - x[..., 1::2] * np.sin(ang)
        y[..., 1::2] = x[..., 1::2] * np.cos(ang) + x[..., 0::2] * np.sin(ang)
        return y

    def sign(x, positions, base):
        return oracle.rotate(x, -np.asarray(positions), base)

    def exponent(x, positions, base):              # theta_i = base^(-i/D)
        return oracle.rotate(x, positions, math.sqrt(base))

    for bad in (interleaved, sign, exponent):
        assert not np.allclose(bad(x, pos, 10000.0), good, atol=1e-6), bad.__name__
    # the query at position 0 instead of n - 1
    q = rng.standard_normal((2, 8))
    kk = rng.standard_normal((1, 6, 8))
    vv = rng.standard_normal((1, 6, 8))
    ref = relative_loop(q, kk, vv, 0.5, 100.0)
    kr = oracle.rotate(kk, np.arange(6), 100.0)
    wrong, _ = oracle.decode_attention(q, kr, vv, 0.5)
    assert not np.allclose(wrong, ref, atol=1e-6)
