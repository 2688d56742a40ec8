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

# ---------------------------------------------------------------- guard canaries
# Device outputs are placed inside a larger allocation whose bytes before and
# after the tensor hold a fixed pattern; after each GPU test the patterns are
# compared (tests/conftest.py), so a kernel that writes outside its output is
# caught even when the write lands in memory no other check reads.
GUARD_BYTES = 4096          # a multiple of 256: the tensor keeps the allocation's alignment
GUARD_PATTERN = 0xA5
_guards = []


def guarded_empty(shape, dtype, fill=None, device="cuda") -> torch.Tensor:
    """A contiguous device tensor of `shape`/`dtype` with guard bytes around
    it; filled with `fill` when given (else the guard pattern)."""
    shape = tuple(int(x) for x in shape)
    esz = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape)) if shape else 1
    body = -(-n * esz // 256) * 256
    buf = torch.full((GUARD_BYTES + body + GUARD_BYTES,), GUARD_PATTERN, dtype=torch.uint8, device=device)
    t = buf[GUARD_BYTES:GUARD_BYTES + n * esz].view(dtype).view(shape)
    if fill is not None:
        t.fill_(fill)
    _guards.append((buf, n * esz, f"{tuple(shape)} {dtype}"))
    return t


def guarded_like(x: torch.Tensor) -> torch.Tensor:
    t = guarded_empty(x.shape, x.dtype, device=x.device)
    t.copy_(x)
    return t


def reset_guards():
    _guards.clear()


def check_guards():
    """Assert that no guard byte of any guarded tensor changed."""
    bad = []
    for buf, nbytes, what in _guards:
        head = buf[:GUARD_BYTES]
        tail = buf[GUARD_BYTES + nbytes:]
        if bool((head != GUARD_PATTERN).any()) or bool((tail != GUARD_PATTERN).any()):
            bad.append(what)
    _guards.clear()
    assert not bad, f"a kernel wrote outside its output: guard bytes changed around {bad}"


def guarded_cache(*args, **kw):
    """A SepCache whose k, v, pos, tok and state live in guarded buffers."""
    from kv_cache_compression_sep_amd import SepCache
    c = SepCache(*args, **kw)
    c.k, c.v = guarded_like(c.k), guarded_like(c.v)
    c.pos, c.tok, c.state = guarded_like(c.pos), guarded_like(c.tok), guarded_like(c.state)
    if c.work is not None:
        c.work = guarded_like(c.work)
    return c


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


def slots_of(cache, b: int, state=None):
    """Slots of sequence b's retained entries per block, oldest first:
    (initial, separator ring, recent ring), from its state words (the slot
    layout of sep_cache in include/sepattn.h). ``state`` overrides the
    cache's own state tensor (for a snapshot)."""
    st = cache.state if state is None else state
    t, ncomp, head, cnt = [int(x) for x in st[b, :4].cpu().numpy()]
    a, s = cache.a, cache.s
    I = list(range(min(a, t)))
    S = [a + (head - cnt + i) % s for i in range(cnt)] if s > 0 else []
    cend = a + ncomp
    R = [a + s + (x - a) % cache.ring for x in range(max(cend, a), t)] if t > a else []
    return I, S, R

