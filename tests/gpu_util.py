"""Helpers shared by the GPU parity tests: tensor transfer and the
floating-point acceptance criterion.

Criterion for attention outputs: max |o_gpu - o_ref| <= tol + ulp_out(o_ref)/2,
with tol = 1e-2 for bf16 I/O and 1e-5 for fp32 I/O, and ulp_out the unit in
the last place of the output format at |o_ref| (bf16: 2^(floor(log2|x|) - 7);
fp32: 2^(floor(log2|x|) - 23)). The half-ulp term is the unavoidable
rounding of a correct result to the output format (in bf16 it alone reaches
0.0156 for |o| >= 4).
"""
import numpy as np
import torch

from inputs import gen

TOL = {"bf16": 1e-2, "f32": 1e-5}


def to_dev(x: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_dev(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy float64 (exact for bf16/fp32), ints unchanged."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return gen.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    return t.numpy()


def half_ulp(ref: np.ndarray, dtype: str) -> np.ndarray:
    mant = 7 if dtype == "bf16" else 23
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1e-30)))
    return np.where(a > 0, 0.5 * np.exp2(e - mant), 0.0)


def check_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "") -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = TOL[dtype] + half_ulp(ref, dtype)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (
        f"{what}: max err {err.max():.3e} (bound at worst {bound[worst]:.3e}, ref {ref[worst]:.4f}, "
        f"got {got[worst]:.4f} at {worst})")
    return float(err.max())
