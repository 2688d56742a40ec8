"""Sep-Attention hot path for AMD Instinct MI355X (gfx950).

Python binding of ``libsepattn.so`` (C ABI in ``include/sepattn.h``). The
functions carry the C entry points' names and take PyTorch tensors on the
GPU; the binding only checks tensor properties, allocates outputs when the
caller does not pass them, and hands raw pointers and the current HIP
stream to the library. All computation happens in the HIP kernels.

    is_sep, tiles, dense = sep_mask_build(ids, sep_ids, a, n, ...)
    rank, sep_pos, count = sep_index_compact(is_sep)
    out, lse             = sep_attn_prefill(q, k, v, is_sep, rank, sep_pos, a, n)
    cache = SepCache(B, Hkv, D, a, s, p, w)     # four-block KV cache
    o, lse = sep_attn_decode(q, k_new, v_new, cache)
    sep_cache_update(cache, k_new, v_new, ids_new, sep_ids)
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import SepError, SEP_BF16, SEP_F32  # noqa: F401

__all__ = ["sep_mask_build", "sep_index_compact", "sep_mask_compact", "sep_attn_prefill", "sep_attn_prefill_backward",
           "sep_attn_prefill_backward_noalloc", "SEP_NOALLOC_MAX_ROWS",
           "sep_attn_decode", "sep_attn_decode_rope", "sep_decode_update", "sep_rope_table", "sep_attn_prefill_chunk",
           "chunk_workspace_bytes", "decode_work_bytes",
           "sep_cache_update", "sep_cache_reset", "SepCache", "SepError", "library_version",
           "SEP_POLICY_DYNAMIC", "SEP_POLICY_NO_ACCUM"]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _need_shape(t, name, shape, dtype, device=None):
    """t must be a contiguous GPU tensor of exactly this shape and dtype (and
    on `device` when given): the C ABI cannot see tensor sizes, so a wrong
    size here would make a kernel read or write out of bounds."""
    _need(t, name, dtype)
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _out(t, name, shape, dtype, device):
    """The caller's output tensor after checking it, or a new one."""
    if t is None:
        return torch.empty(tuple(shape), dtype=dtype, device=device)
    _need_shape(t, name, shape, dtype, device)
    return t


def _dtype_code(t) -> int:
    if t.dtype == torch.bfloat16:
        return SEP_BF16
    if t.dtype == torch.float32:
        return SEP_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def library_version() -> int:
    return _lib.load().sep_version()


def sep_mask_build(ids, sep_ids, a: int, n: int, *, is_sep=None, tiles: tuple | None = None,
                   tile_class=None, dense: bool = False, dense_mask=None):
    """Separator flags [B,S] u8; optional tile classes for ``tiles=(tq, tk)``
    and the dense mask [B,S,S] u8 (S <= 8192)."""
    lib = _lib.load()
    _need(ids, "ids", torch.int32, 2)
    _need(sep_ids, "sep_ids", torch.int32, 1)
    B, S = ids.shape
    dev = ids.device
    is_sep = _out(is_sep, "is_sep", (B, S), torch.uint8, dev)
    tq = tk = 0
    if tiles is not None:
        tq, tk = (int(x) for x in tiles)
        if tq < 1 or tk < 1:
            raise ValueError("tiles must be positive")
        tile_class = _out(tile_class, "tile_class", (B, -(-S // tq), -(-S // tk)), torch.uint8, dev)
    elif tile_class is not None:
        raise ValueError("tile_class needs tiles=(tq, tk)")
    if dense or dense_mask is not None:
        dense_mask = _out(dense_mask, "dense_mask", (B, S, S), torch.uint8, dev)
    code = lib.sep_mask_build(ids.data_ptr(), B, S, _ptr(sep_ids) if sep_ids.numel() else None,
                              sep_ids.numel(), a, n, is_sep.data_ptr(), _ptr(tile_class), tq, tk,
                              _ptr(dense_mask), _stream())
    _lib.check("sep_mask_build", code)
    return is_sep, tile_class, dense_mask


def sep_index_compact(is_sep, *, rank=None, sep_pos=None, count=None):
    """rank [B,S+1] i32, sep_pos [B,S] i32, count [B] i32."""
    lib = _lib.load()
    _need(is_sep, "is_sep", torch.uint8, 2)
    B, S = is_sep.shape
    dev = is_sep.device
    rank = _out(rank, "rank", (B, S + 1), torch.int32, dev)
    sep_pos = _out(sep_pos, "sep_pos", (B, S), torch.int32, dev)
    count = _out(count, "count", (B,), torch.int32, dev)
    code = lib.sep_index_compact(is_sep.data_ptr(), B, S, rank.data_ptr(), sep_pos.data_ptr(),
                                 count.data_ptr(), _stream())
    _lib.check("sep_index_compact", code)
    return rank, sep_pos, count


def sep_mask_compact(ids, sep_ids, *, is_sep=None, rank=None, sep_pos=None, count=None):
    """Flags and compaction in one launch: returns is_sep [B,S] u8, rank
    [B,S+1] i32, sep_pos [B,S] i32, count [B] i32."""
    lib = _lib.load()
    _need(ids, "ids", torch.int32, 2)
    _need(sep_ids, "sep_ids", torch.int32, 1)
    B, S = ids.shape
    dev = ids.device
    is_sep = _out(is_sep, "is_sep", (B, S), torch.uint8, dev)
    rank = _out(rank, "rank", (B, S + 1), torch.int32, dev)
    sep_pos = _out(sep_pos, "sep_pos", (B, S), torch.int32, dev)
    count = _out(count, "count", (B,), torch.int32, dev)
    code = lib.sep_mask_compact(ids.data_ptr(), B, S, _ptr(sep_ids) if sep_ids.numel() else None,
                                sep_ids.numel(), is_sep.data_ptr(), rank.data_ptr(), sep_pos.data_ptr(),
                                count.data_ptr(), _stream())
    _lib.check("sep_mask_compact", code)
    return is_sep, rank, sep_pos, count


def _need_index(is_sep, rank, sep_pos, B, S, dev):
    _need_shape(is_sep, "is_sep", (B, S), torch.uint8, dev)
    _need_shape(rank, "rank", (B, S + 1), torch.int32, dev)
    _need_shape(sep_pos, "sep_pos", (B, S), torch.int32, dev)


def sep_attn_prefill(q, k, v, is_sep, rank, sep_pos, a: int, n: int, scale: float | None = None, *,
                     out=None, return_lse: bool = False, lse=None):
    """Sep-Attention prefill: q [B,Hq,S,D], k/v [B,Hkv,S,D] (bf16 or fp32)."""
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, None, 4)
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share a dtype")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or k.device != dev or v.device != dev:
        raise ValueError("k/v must be [B, Hkv, S, D] matching q, on q's device")
    _need_index(is_sep, rank, sep_pos, B, S, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out(out, "out", q.shape, q.dtype, dev)
    if return_lse or lse is not None:
        lse = _out(lse, "lse", (B, Hq, S), torch.float32, dev)
    code = lib.sep_attn_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), B, Hq,
                                Hkv, S, D, is_sep.data_ptr(), rank.data_ptr(), sep_pos.data_ptr(),
                                a, n, float(scale), out.data_ptr(), _ptr(lse), _stream())
    _lib.check("sep_attn_prefill", code)
    return (out, lse) if return_lse else out


def sep_attn_prefill_backward(q, k, v, out, dout, lse, is_sep, rank, sep_pos, a: int, n: int,
                              scale: float | None = None, *, dq=None, dk=None, dv=None, delta=None):
    """Gradients of sep_attn_prefill for L = sum(dout * out): returns float32
    dq [B,Hq,S,D], dk, dv [B,Hkv,S,D]. `out` and `lse` are the forward's."""
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, None, 4)
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise ValueError("q, k, v, out, dout must share a dtype")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k/v must be [B, Hkv, S, D]; out/dout [B, Hq, S, D]")
    if any(t.device != dev for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out, dout must be on one device")
    _need_shape(lse, "lse", (B, Hq, S), torch.float32, dev)
    _need_index(is_sep, rank, sep_pos, B, S, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    f32 = torch.float32
    dq = _out(dq, "dq", (B, Hq, S, D), f32, dev)
    dk = _out(dk, "dk", (B, Hkv, S, D), f32, dev)
    dv = _out(dv, "dv", (B, Hkv, S, D), f32, dev)
    delta = _out(delta, "delta", (B, Hq, S), f32, dev)
    code = lib.sep_attn_prefill_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         dout.data_ptr(), lse.data_ptr(), _dtype_code(q), B, Hq, Hkv, S, D,
                                         is_sep.data_ptr(), rank.data_ptr(), sep_pos.data_ptr(), a, n,
                                         float(scale), delta.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                         dv.data_ptr(), _stream())
    _lib.check("sep_attn_prefill_backward", code)
    return dq, dk, dv


def sep_attn_prefill_backward_noalloc(q, k, v, out, dout, lse, is_sep, rank, sep_pos, a: int, n: int,
                                      scale: float | None, dq, dk, dv):
    """sep_attn_prefill_backward with its per-row workspace in a fixed device
    array of the library (no allocation by the library or by this binding;
    the caller passes dq, dk, dv). B * Hq * S <= SEP_NOALLOC_MAX_ROWS; calls
    that overlap on one GPU race on the array."""
    lib = _lib.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _need(t, name, None, 4)
    if not (q.dtype == k.dtype == v.dtype == out.dtype == dout.dtype):
        raise ValueError("q, k, v, out, dout must share a dtype")
    B, Hq, S, D = q.shape
    Hkv = k.shape[1]
    dev = q.device
    if k.shape != (B, Hkv, S, D) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k/v must be [B, Hkv, S, D]; out/dout [B, Hq, S, D]")
    if any(t.device != dev for t in (k, v, out, dout)):
        raise ValueError("q, k, v, out, dout must be on one device")
    _need_shape(lse, "lse", (B, Hq, S), torch.float32, dev)
    _need_index(is_sep, rank, sep_pos, B, S, dev)
    _need_shape(dq, "dq", (B, Hq, S, D), torch.float32, dev)
    _need_shape(dk, "dk", (B, Hkv, S, D), torch.float32, dev)
    _need_shape(dv, "dv", (B, Hkv, S, D), torch.float32, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    code = lib.sep_attn_prefill_backward_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                                 dout.data_ptr(), lse.data_ptr(), _dtype_code(q), B, Hq, Hkv, S, D,
                                                 is_sep.data_ptr(), rank.data_ptr(), sep_pos.data_ptr(), a, n,
                                                 float(scale), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), _stream())
    _lib.check("sep_attn_prefill_backward_noalloc", code)
    return dq, dk, dv


SEP_NOALLOC_MAX_ROWS = 1 << 22

# cache policies (sep_cache.policy in include/sepattn.h)
SEP_POLICY_DYNAMIC = 1     # compress when the whole cache exceeds c = a + s + p + w
SEP_POLICY_NO_ACCUM = 2    # SEP_ACCUMULATION off: a compression replaces the separators
STATE_WORDS = 8


class SepCache:
    """A batch of four-block caches in device memory (layout: see sep_cache
    in include/sepattn.h). ``policy`` combines SEP_POLICY_DYNAMIC and
    SEP_POLICY_NO_ACCUM; the recent ring has p + w slots, or s + p + w under
    SEP_POLICY_DYNAMIC. With ``split`` (the default) the cache also carries
    the work buffer that lets decode split each list over several workgroups
    when there are few (sequence, kv head) pairs (sized for up to 16 query
    heads per kv head)."""

    MAX_GROUP = 16

    def __init__(self, B: int, Hkv: int, D: int, a: int, s: int, p: int, w: int,
                 dtype=torch.bfloat16, device="cuda", policy: int = 0, split: bool = True):
        self.B, self.Hkv, self.D = B, Hkv, D
        self.a, self.s, self.p, self.w = a, s, p, w
        self.policy = int(policy)
        self.c = a + s + p + w
        self.ring = p + w + (s if self.policy & SEP_POLICY_DYNAMIC else 0)
        self.slots = a + s + self.ring
        self.dtype = dtype
        dev = torch.device(device)
        self.k = torch.zeros((B, Hkv, self.slots, D), dtype=dtype, device=dev)
        self.v = torch.zeros_like(self.k)
        self.pos = torch.full((B, self.slots), -1, dtype=torch.int32, device=dev)
        self.tok = torch.full((B, self.slots), -1, dtype=torch.int32, device=dev)
        self.state = torch.zeros((B, STATE_WORDS), dtype=torch.int64, device=dev)
        self.work = None
        if split:
            need = decode_work_bytes(self, Hkv * self.MAX_GROUP)
            if need:
                self.work = torch.empty((need,), dtype=torch.uint8, device=dev)

    def struct(self) -> _lib.SepCacheStruct:
        """The sep_cache view of this cache, after checking that its tensors
        still have the shapes the C side will assume."""
        dev = self.k.device
        _need_shape(self.k, "cache.k", (self.B, self.Hkv, self.slots, self.D), self.dtype, dev)
        _need_shape(self.v, "cache.v", (self.B, self.Hkv, self.slots, self.D), self.dtype, dev)
        _need_shape(self.pos, "cache.pos", (self.B, self.slots), torch.int32, dev)
        _need_shape(self.tok, "cache.tok", (self.B, self.slots), torch.int32, dev)
        _need_shape(self.state, "cache.state", (self.B, STATE_WORDS), torch.int64, dev)
        work, work_bytes = None, 0
        if self.work is not None:
            _need(self.work, "cache.work", torch.uint8, 1)
            if self.work.device != dev:
                raise ValueError("cache.work must be on the cache's device")
            work, work_bytes = self.work.data_ptr(), self.work.numel()
        return _lib.SepCacheStruct(self.a, self.s, self.p, self.w, self.B, self.Hkv, self.D,
                                   _dtype_code(self.k), self.k.data_ptr(), self.v.data_ptr(),
                                   self.pos.data_ptr(), self.tok.data_ptr(), self.state.data_ptr(),
                                   self.policy, work, work_bytes)

    def reset(self):
        sep_cache_reset(self)

    def n_seen(self):
        return self.state[:, 0]


def _need_same_device(cache, **tensors):
    dev = cache.k.device
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} must be on the cache's device {dev}, got {t.device}")


def sep_cache_reset(cache: SepCache):
    st = cache.struct()
    _lib.check("sep_cache_reset", _lib.load().sep_cache_reset(ctypes.byref(st), _stream()))


def sep_cache_update(cache: SepCache, k_new, v_new, ids_new, sep_ids):
    """Append T tokens per sequence: k_new/v_new [B,Hkv,T,D], ids_new [B,T] i32."""
    lib = _lib.load()
    _need(k_new, "k_new", cache.dtype, 4)
    _need(v_new, "v_new", cache.dtype, 4)
    _need(ids_new, "ids_new", torch.int32, 2)
    _need(sep_ids, "sep_ids", torch.int32, 1)
    B, Hkv, T, D = k_new.shape
    if (B, Hkv, D) != (cache.B, cache.Hkv, cache.D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, Hkv, T, D] of the cache")
    if ids_new.shape != (B, T):
        raise ValueError("ids_new must be [B, T]")
    _need_same_device(cache, k_new=k_new, v_new=v_new, ids_new=ids_new, sep_ids=sep_ids)
    st = cache.struct()
    code = lib.sep_cache_update(ctypes.byref(st), k_new.data_ptr(), v_new.data_ptr(),
                                ids_new.data_ptr(), T,
                                _ptr(sep_ids) if sep_ids.numel() else None, sep_ids.numel(),
                                _stream())
    _lib.check("sep_cache_update", code)


def decode_work_bytes(cache: "SepCache", Hq: int) -> int:
    """Work-buffer bytes the decode calls need to split their lists for Hq
    query heads (0: they never split this cache)."""
    st = cache.struct()
    return int(_lib.load().sep_decode_work_bytes(ctypes.byref(st), Hq))


def chunk_workspace_bytes(cache: "SepCache", C: int) -> int:
    """Workspace bytes sep_attn_prefill_chunk needs for a chunk of C tokens."""
    st = cache.struct()
    return int(_lib.load().sep_chunk_workspace_bytes(ctypes.byref(st), C))


def sep_attn_prefill_chunk(q, k, v, ids, cache: "SepCache", sep_ids, n: int, scale: float | None = None, *,
                           workspace=None, out=None, return_lse: bool = False, lse=None):
    """A chunk of C new tokens over the live cache and itself: q [B,Hq,C,D],
    k/v [B,Hkv,C,D] (bf16), ids [B,C] int32, window n. The cache is not
    modified (insert the chunk with sep_cache_update afterwards)."""
    lib = _lib.load()
    _need(q, "q", cache.dtype, 4)
    _need(k, "k", cache.dtype, 4)
    _need(v, "v", cache.dtype, 4)
    _need(ids, "ids", torch.int32, 2)
    _need(sep_ids, "sep_ids", torch.int32, 1)
    B, Hq, C, D = q.shape
    if (B, D) != (cache.B, cache.D) or k.shape != (B, cache.Hkv, C, D) or v.shape != k.shape:
        raise ValueError("shapes do not match the cache")
    if ids.shape != (B, C):
        raise ValueError("ids must be [B, C]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _need_same_device(cache, q=q, k=k, v=v, ids=ids, sep_ids=sep_ids)
    dev = q.device
    need = chunk_workspace_bytes(cache, C)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    else:
        _need(workspace, "workspace", torch.uint8, 1)
        if workspace.device != dev:
            raise ValueError("workspace must be on the cache's device")
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, {need} needed")
    out = _out(out, "out", q.shape, q.dtype, dev)
    if return_lse or lse is not None:
        lse = _out(lse, "lse", (B, Hq, C), torch.float32, dev)
    st = cache.struct()
    code = lib.sep_attn_prefill_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), ids.data_ptr(), C,
                                      sep_ids.data_ptr(), sep_ids.numel(), ctypes.byref(st), Hq, n, float(scale),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      out.data_ptr(), _ptr(lse), _stream())
    _lib.check("sep_attn_prefill_chunk", code)
    return (out, lse) if return_lse else out


def sep_rope_table(base: float, D: int, n_pos: int, *, out=None, device="cuda"):
    """(cos, sin) of p * base^(-2i/D) for p < n_pos, i < D/2: float32 [n_pos, D/2, 2]."""
    lib = _lib.load()
    dev = out.device if isinstance(out, torch.Tensor) else torch.device(device)
    out = _out(out, "out", (n_pos, D // 2, 2), torch.float32, dev)
    code = lib.sep_rope_table(float(base), D, n_pos, out.data_ptr(), _stream())
    _lib.check("sep_rope_table", code)
    return out


def sep_attn_decode_rope(q, k_new, v_new, cache: SepCache, rope, scale: float | None = None, *, out=None,
                         return_lse: bool = False, lse=None):
    """sep_attn_decode with rotary embedding at shifted positions (cached keys
    and k_new unrotated; `rope` from sep_rope_table with at least
    cache.slots + 1 rows)."""
    lib = _lib.load()
    _need(q, "q", cache.dtype, 3)
    _need(k_new, "k_new", cache.dtype, 3)
    _need(v_new, "v_new", cache.dtype, 3)
    _need(rope, "rope", torch.float32, 3)
    B, Hq, D = q.shape
    if (B, D) != (cache.B, cache.D) or k_new.shape != (B, cache.Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("shapes do not match the cache")
    if rope.shape[1:] != (D // 2, 2):
        raise ValueError("rope must be [n_pos, D/2, 2]")
    _need_same_device(cache, q=q, k_new=k_new, v_new=v_new, rope=rope)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    if return_lse or lse is not None:
        lse = _out(lse, "lse", (B, Hq), torch.float32, q.device)
    st = cache.struct()
    code = lib.sep_attn_decode_rope(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), ctypes.byref(st), Hq,
                                    float(scale), rope.data_ptr(), rope.shape[0], out.data_ptr(), _ptr(lse),
                                    _stream())
    _lib.check("sep_attn_decode_rope", code)
    return (out, lse) if return_lse else out


def sep_decode_update(q, k_new, v_new, ids_new, cache: SepCache, sep_ids, scale: float | None = None, *,
                      rope=None, out=None, return_lse: bool = False, lse=None):
    """One streaming step: the decode of q [B,Hq,D] with k_new/v_new
    [B,Hkv,D] (bf16) over the cache (with `rope`, at shifted positions),
    then the insertion of that token (ids_new [B] int32) into the cache;
    equal to sep_attn_decode (or sep_attn_decode_rope) then
    sep_cache_update, in one launch where the decode runs wide."""
    lib = _lib.load()
    _need(q, "q", cache.dtype, 3)
    _need(k_new, "k_new", cache.dtype, 3)
    _need(v_new, "v_new", cache.dtype, 3)
    _need(ids_new, "ids_new", torch.int32, 1)
    _need(sep_ids, "sep_ids", torch.int32, 1)
    B, Hq, D = q.shape
    if (B, D) != (cache.B, cache.D) or k_new.shape != (B, cache.Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("shapes do not match the cache")
    if ids_new.shape != (B,):
        raise ValueError("ids_new must be [B]")
    if rope is not None:
        _need(rope, "rope", torch.float32, 3)
        if rope.shape[1:] != (D // 2, 2):
            raise ValueError("rope must be [n_pos, D/2, 2]")
    _need_same_device(cache, q=q, k_new=k_new, v_new=v_new, ids_new=ids_new, sep_ids=sep_ids, rope=rope)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    if return_lse or lse is not None:
        lse = _out(lse, "lse", (B, Hq), torch.float32, q.device)
    st = cache.struct()
    code = lib.sep_decode_update(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), ids_new.data_ptr(),
                                 _ptr(sep_ids) if sep_ids.numel() else None, sep_ids.numel(), ctypes.byref(st),
                                 Hq, float(scale), _ptr(rope), 0 if rope is None else rope.shape[0],
                                 out.data_ptr(), _ptr(lse), _stream())
    _lib.check("sep_decode_update", code)
    return (out, lse) if return_lse else out


def sep_attn_decode(q, k_new, v_new, cache: SepCache, scale: float | None = None, *, out=None,
                    return_lse: bool = False, lse=None):
    """One decode step: q [B,Hq,D], k_new/v_new [B,Hkv,D] (bf16)."""
    lib = _lib.load()
    _need(q, "q", cache.dtype, 3)
    _need(k_new, "k_new", cache.dtype, 3)
    _need(v_new, "v_new", cache.dtype, 3)
    B, Hq, D = q.shape
    if (B, D) != (cache.B, cache.D) or k_new.shape != (B, cache.Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("shapes do not match the cache")
    _need_same_device(cache, q=q, k_new=k_new, v_new=v_new)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out(out, "out", q.shape, q.dtype, q.device)
    if return_lse or lse is not None:
        lse = _out(lse, "lse", (B, Hq), torch.float32, q.device)
    st = cache.struct()
    code = lib.sep_attn_decode(q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), ctypes.byref(st),
                               Hq, float(scale), out.data_ptr(), _ptr(lse), _stream())
    _lib.check("sep_attn_decode", code)
    return (out, lse) if return_lse else out
