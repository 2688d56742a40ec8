"""The C ABI on the host: the library loads, exports every function that
include/sepattn.h declares, and rejects invalid arguments with the documented
status codes before touching the GPU (validation runs before any HIP call,
so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from kv_cache_compression_sep_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sepattn.h")
FAKE = 4096  # a non-NULL, 16-byte aligned host address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsepattn.so is not built (run __graft_entry__.build())")
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:int|size_t|const char\*)\s+(sep_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_five_entry_points():
    names = header_functions()
    for fn in ("sep_mask_build", "sep_index_compact", "sep_attn_prefill", "sep_attn_decode",
               "sep_cache_update"):
        assert fn in names


def test_every_declared_function_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for fn in header_functions():
        assert fn in exported, fn
        assert hasattr(lib, fn)
    assert set(_lib.SIGNATURES) == set(header_functions())


def test_version_and_status_strings(lib):
    assert lib.sep_version() >= 10100
    for code in range(-7, 1):
        assert lib.sep_status_string(code)
    assert lib.sep_status_string(-99) == b"unknown status"


def test_struct_layout_matches_header():
    # 8 int32, 5 pointers, the int32 policy (padded to 8 bytes), the work
    # pointer and its size
    assert ctypes.sizeof(_lib.SepCacheStruct) == 8 * 4 + 5 * 8 + 8 + 2 * 8
    assert _lib.SepCacheStruct.k.offset == 32
    assert _lib.SepCacheStruct.policy.offset == 72
    assert _lib.SepCacheStruct.work.offset == 80
    assert _lib.SepCacheStruct.work_bytes.offset == 88


def test_mask_build_argument_checks(lib):
    f = lib.sep_mask_build
    E = _lib
    assert f(None, 1, 8, FAKE, 1, 4, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_NULL
    assert f(FAKE, 1, 8, FAKE, 1, 4, 2, None, None, 0, 0, None, None) == E.SEP_ERR_NULL
    assert f(FAKE, 0, 8, FAKE, 1, 4, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_SHAPE
    assert f(FAKE, 1, 0, FAKE, 1, 4, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_SHAPE
    assert f(FAKE, 1, 8, FAKE, 65, 4, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_SHAPE
    assert f(FAKE, 1, 8, None, 3, 4, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_NULL
    assert f(FAKE, 1, 8, FAKE, 1, -1, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_PARAM
    assert f(FAKE, 1, 8, FAKE, 1, 4, 0, FAKE, None, 0, 0, None, None) == E.SEP_ERR_PARAM
    assert f(FAKE, 1, 8, FAKE, 1, 4, 2, FAKE, FAKE, 0, 8, None, None) == E.SEP_ERR_SHAPE
    assert f(FAKE, 1, 9000, FAKE, 1, 4, 2, FAKE, None, 0, 0, FAKE, None) == E.SEP_ERR_SHAPE
    assert f(FAKE + 4, 1, 8, FAKE, 1, 4, 2, FAKE, None, 0, 0, None, None) == E.SEP_ERR_ALIGN


def test_index_compact_argument_checks(lib):
    f = lib.sep_index_compact
    assert f(None, 1, 8, FAKE, FAKE, None, None) == _lib.SEP_ERR_NULL
    assert f(FAKE, 1, 8, None, FAKE, None, None) == _lib.SEP_ERR_NULL
    assert f(FAKE, 0, 8, FAKE, FAKE, None, None) == _lib.SEP_ERR_SHAPE


def _prefill(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, B=1, Hq=32, Hkv=8, S=64, D=128, is_sep=FAKE,
                rank=FAKE, sep_pos=FAKE, a=4, n=16, scale=0.088, out=FAKE, lse=None, st=None)
    args.update(kw)
    return lib.sep_attn_prefill(*args.values())


def test_prefill_argument_checks(lib):
    E = _lib
    assert _prefill(lib, q=None) == E.SEP_ERR_NULL
    assert _prefill(lib, rank=None) == E.SEP_ERR_NULL
    assert _prefill(lib, dtype=7) == E.SEP_ERR_DTYPE
    assert _prefill(lib, Hq=30) == E.SEP_ERR_SHAPE        # not a multiple of Hkv
    assert _prefill(lib, Hq=8 * 17) == E.SEP_ERR_SHAPE    # group larger than 16
    assert _prefill(lib, D=96) == E.SEP_ERR_SHAPE
    assert _prefill(lib, S=0) == E.SEP_ERR_SHAPE
    assert _prefill(lib, a=-1) == E.SEP_ERR_PARAM
    assert _prefill(lib, n=0) == E.SEP_ERR_PARAM
    assert _prefill(lib, scale=0.0) == E.SEP_ERR_PARAM
    assert _prefill(lib, scale=float("nan")) == E.SEP_ERR_PARAM
    assert _prefill(lib, out=FAKE + 2) == E.SEP_ERR_ALIGN


def _backward(lib, **kw):
    args = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, dout=FAKE, lse=FAKE, dtype=1, B=1, Hq=32, Hkv=8, S=64,
                D=128, is_sep=FAKE, rank=FAKE, sep_pos=FAKE, a=4, n=16, scale=0.088, delta=FAKE, dq=FAKE,
                dk=FAKE, dv=FAKE, st=None)
    args.update(kw)
    return lib.sep_attn_prefill_backward(*args.values())


def test_prefill_backward_argument_checks(lib):
    E = _lib
    for name in ("q", "dout", "lse", "delta", "dq", "dk", "dv", "sep_pos"):
        assert _backward(lib, **{name: None}) == E.SEP_ERR_NULL, name
    assert _backward(lib, dtype=7) == E.SEP_ERR_DTYPE
    assert _backward(lib, Hq=30) == E.SEP_ERR_SHAPE
    assert _backward(lib, D=96) == E.SEP_ERR_SHAPE
    assert _backward(lib, S=0) == E.SEP_ERR_SHAPE
    assert _backward(lib, S=2097152 + 1) == E.SEP_ERR_SHAPE     # past SEP_MAX_BACKWARD_S
    assert _backward(lib, n=0) == E.SEP_ERR_PARAM
    assert _backward(lib, a=-1) == E.SEP_ERR_PARAM
    assert _backward(lib, scale=float("inf")) == E.SEP_ERR_PARAM
    for name in ("out", "dout", "dq", "dk", "dv"):
        assert _backward(lib, **{name: FAKE + 4}) == E.SEP_ERR_ALIGN, name


def _cache(**kw):
    d = dict(a=4, s=64, p=64, w=256, B=1, Hkv=8, D=128, dtype=1, k=FAKE, v=FAKE, pos=FAKE,
             tok=FAKE, state=FAKE, policy=0)
    d.update(kw)
    return _lib.SepCacheStruct(*d.values())


def test_cache_contract_from_the_pages(lib):
    """P1 "Streaming 参数约束": cache > 0, init >= 0, local > 0,
    cache >= init + local; SepLLM: sep > 0 and init + sep + local < cache;
    StreamingLLM: local == cache - init (here s = p = 0)."""
    E = _lib
    upd = lambda c: lib.sep_cache_update(ctypes.byref(c), FAKE, FAKE, FAKE, 1, FAKE, 1, None)
    assert upd(_cache(w=0)) == E.SEP_ERR_PARAM             # local must be > 0
    assert upd(_cache(a=-1)) == E.SEP_ERR_PARAM            # init must be >= 0
    assert upd(_cache(p=0)) == E.SEP_ERR_PARAM             # init + sep + local == cache
    assert upd(_cache(s=0)) == E.SEP_ERR_PARAM             # sep must be > 0 for SepLLM
    assert upd(_cache(s=9000)) == E.SEP_ERR_PARAM          # beyond the ring limit
    assert upd(_cache(D=80)) == E.SEP_ERR_SHAPE
    assert upd(_cache(dtype=5)) == E.SEP_ERR_DTYPE
    assert upd(_cache(pos=None)) == E.SEP_ERR_NULL
    assert upd(_cache(k=FAKE + 8)) == E.SEP_ERR_ALIGN
    assert lib.sep_cache_update(None, FAKE, FAKE, FAKE, 1, FAKE, 1, None) == E.SEP_ERR_NULL
    c = _cache()
    assert lib.sep_cache_update(ctypes.byref(c), FAKE, FAKE, FAKE, 0, FAKE, 1, None) == E.SEP_ERR_SHAPE
    assert lib.sep_cache_update(ctypes.byref(c), None, FAKE, FAKE, 1, FAKE, 1, None) == E.SEP_ERR_NULL
    assert lib.sep_cache_reset(ctypes.byref(_cache(w=0)), None) == E.SEP_ERR_PARAM


def test_cache_policy_checks(lib):
    """Policy bits: SEP_POLICY_DYNAMIC (1) and SEP_POLICY_NO_ACCUM (2) only; the
    dynamic trigger's recent ring (s + p + w slots) is bounded."""
    E = _lib
    upd = lambda c: lib.sep_cache_update(ctypes.byref(c), FAKE, FAKE, FAKE, 1, FAKE, 1, None)
    assert upd(_cache(policy=4)) == E.SEP_ERR_PARAM
    assert upd(_cache(policy=-1)) == E.SEP_ERR_PARAM
    assert upd(_cache(policy=1, s=64, p=16384, w=16384)) == E.SEP_ERR_PARAM   # ring 32832 > 32768
    for pol in (1, 2, 3):
        c = _cache(policy=pol)
        assert lib.sep_cache_update(ctypes.byref(c), FAKE, FAKE, FAKE, 0, FAKE, 1, None) == E.SEP_ERR_SHAPE


def test_decode_argument_checks(lib):
    E = _lib
    c = _cache()
    dec = lambda cc, **kw: lib.sep_attn_decode(
        kw.get("q", FAKE), FAKE, FAKE, ctypes.byref(cc), kw.get("Hq", 32), kw.get("scale", 0.1),
        FAKE, None, None)
    assert dec(c, q=None) == E.SEP_ERR_NULL
    assert dec(c, Hq=12) == E.SEP_ERR_SHAPE
    assert dec(c, Hq=8 * 17) == E.SEP_ERR_SHAPE
    assert dec(c, scale=-1.0) == E.SEP_ERR_PARAM
    assert dec(_cache(dtype=0)) == E.SEP_ERR_DTYPE
    assert dec(_cache(s=0)) == E.SEP_ERR_PARAM           # s = 0 needs p = 0
    assert dec(c, q=FAKE + 2) == E.SEP_ERR_ALIGN


def test_rope_argument_checks(lib):
    E = _lib
    tab = lambda **kw: lib.sep_rope_table(kw.get("base", 500000.0), kw.get("D", 128), kw.get("n", 10),
                                          kw.get("t", FAKE), None)
    assert tab(t=None) == E.SEP_ERR_NULL
    assert tab(D=96) == E.SEP_ERR_SHAPE
    assert tab(n=0) == E.SEP_ERR_SHAPE
    assert tab(base=1.0) == E.SEP_ERR_PARAM
    assert tab(base=float("nan")) == E.SEP_ERR_PARAM
    assert tab(t=FAKE + 8) == E.SEP_ERR_ALIGN
    c = _cache()                                         # 4 + 64 + (64 + 256) slots
    dec = lambda cc, **kw: lib.sep_attn_decode_rope(
        FAKE, FAKE, FAKE, ctypes.byref(cc), 32, 0.1, kw.get("rope", FAKE), kw.get("npos", 389), FAKE, None, None)
    assert dec(c, rope=None) == E.SEP_ERR_NULL
    assert dec(c, npos=388) == E.SEP_ERR_PARAM           # fewer rows than slots + 1
    assert dec(_cache(policy=1), npos=389) == E.SEP_ERR_PARAM   # dynamic ring: s + p + w slots
    assert dec(c, rope=FAKE + 4) == E.SEP_ERR_ALIGN
    assert dec(_cache(dtype=0)) == E.SEP_ERR_DTYPE


def test_decode_update_argument_checks(lib):
    E = _lib
    c = _cache()                                         # 4 + 64 + (64 + 256) slots, 8 kv heads
    du = lambda cc, **kw: lib.sep_decode_update(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("ids", FAKE), FAKE, kw.get("nsep", 4), ctypes.byref(cc),
        kw.get("Hq", 32), kw.get("scale", 0.1), kw.get("rope", None), kw.get("npos", 0), kw.get("out", FAKE),
        None, None)
    assert du(c, q=None) == E.SEP_ERR_NULL
    assert du(c, ids=None) == E.SEP_ERR_NULL
    assert du(c, out=None) == E.SEP_ERR_NULL
    assert du(c, nsep=65) == E.SEP_ERR_SHAPE
    assert du(c, Hq=12) == E.SEP_ERR_SHAPE                # not a multiple of Hkv = 8
    assert du(c, scale=0.0) == E.SEP_ERR_PARAM
    assert du(c, rope=FAKE, npos=388) == E.SEP_ERR_PARAM  # fewer rows than slots + 1
    assert du(c, q=FAKE + 4) == E.SEP_ERR_ALIGN
    assert du(c, rope=FAKE + 4, npos=389) == E.SEP_ERR_ALIGN
    assert du(_cache(dtype=0)) == E.SEP_ERR_DTYPE


def test_chunk_argument_checks(lib):
    E = _lib
    c = _cache()                                          # 4 + 64 + 320 slots, 8 kv heads, D = 128
    need = lib.sep_chunk_workspace_bytes(ctypes.byref(c), 100)
    assert need >= 2 * 8 * (388 + 100) * 128 * 2
    assert lib.sep_chunk_workspace_bytes(ctypes.byref(c), 0) == 0
    ch = lambda cc, **kw: lib.sep_attn_prefill_chunk(
        kw.get("q", FAKE), FAKE, FAKE, kw.get("ids", FAKE), kw.get("C", 100), FAKE, kw.get("nsep", 4),
        ctypes.byref(cc), kw.get("Hq", 32), kw.get("n", 64), 0.1, kw.get("ws", 1 << 20), kw.get("wsb", need),
        FAKE, None, None)
    assert ch(c, q=None) == E.SEP_ERR_NULL
    assert ch(c, ids=None) == E.SEP_ERR_NULL
    assert ch(c, nsep=65) == E.SEP_ERR_SHAPE
    assert ch(c, C=0) == E.SEP_ERR_SHAPE
    assert ch(c, Hq=12) == E.SEP_ERR_SHAPE
    assert ch(c, n=0) == E.SEP_ERR_PARAM
    assert ch(c, ws=None) == E.SEP_ERR_WORKSPACE
    assert ch(c, wsb=need - 1) == E.SEP_ERR_WORKSPACE
    assert ch(c, ws=(1 << 20) + 16) == E.SEP_ERR_WORKSPACE
    assert ch(c, q=FAKE + 2) == E.SEP_ERR_ALIGN
    assert ch(_cache(dtype=0)) == E.SEP_ERR_DTYPE


def test_mask_compact_argument_checks(lib):
    E = _lib
    f = lambda **kw: lib.sep_mask_compact(kw.get("ids", FAKE), kw.get("B", 1), kw.get("S", 64), FAKE,
                                          kw.get("nsep", 4), kw.get("flags", FAKE), kw.get("rank", FAKE), FAKE,
                                          None, None)
    assert f(ids=None) == E.SEP_ERR_NULL
    assert f(rank=None) == E.SEP_ERR_NULL
    assert f(S=0) == E.SEP_ERR_SHAPE
    assert f(nsep=65) == E.SEP_ERR_SHAPE
    assert f(flags=FAKE + 1) == E.SEP_ERR_ALIGN
    assert f(ids=FAKE + 4) == E.SEP_ERR_ALIGN


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_validation_under_address_and_undefined_behavior_sanitizers(tmp_path):
    """api.hip's argument validation, compiled for the host only with ASan and
    UBSan (no recovery) and linked against stand-in launchers that count
    calls (tests/abi_host/stubs.hip), driven through every entry point's
    status codes by tests/abi_host/driver.cpp."""
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    here = os.path.join(ROOT, "tests", "abi_host")
    csrc = os.path.join(ROOT, "kv_cache_compression_sep_amd", "csrc")
    inc = [f"-I{os.path.join(ROOT, 'include')}", f"-I{csrc}"]
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    objs = []
    for src in (os.path.join(csrc, "api.hip"), os.path.join(here, "stubs.hip"), os.path.join(here, "driver.cpp")):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip", "--cuda-host-only"]          # host code only; the driver needs HIP's headers
        cmd = [hipcc, *lang, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", *san, *inc, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-4000:]
        objs.append(obj)
    exe = str(tmp_path / "abi_driver")
    r = subprocess.run([hipcc, *san, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "abi validation ok" in r.stdout


def test_noalloc_backward_argument_checks(lib):
    """The no-alloc backward checks its arguments like the backward, then
    refuses more query rows than its fixed array holds, all before any HIP
    call."""
    f = lib.sep_attn_prefill_backward_noalloc

    def call(S=64, q=FAKE, dq=FAKE, B=1, Hq=32):
        return f(q, FAKE, FAKE, FAKE, FAKE, FAKE, 1, B, Hq, 8, S, 128, FAKE, FAKE, FAKE, 4, 16, 0.088, dq, FAKE,
                 FAKE, None)
    rows = 1 << 22
    assert call(q=None) == _lib.SEP_ERR_NULL
    assert call(dq=None) == _lib.SEP_ERR_NULL
    assert call(dq=FAKE + 4) == _lib.SEP_ERR_ALIGN
    assert call(S=0) == _lib.SEP_ERR_SHAPE
    assert call(S=rows // 32 + 1) == _lib.SEP_ERR_WORKSPACE
    assert call(S=rows // 64 + 1, B=2) == _lib.SEP_ERR_WORKSPACE
    assert call(S=2_000_000, B=2_000_000, Hq=2_000_000 // 8 * 8) == _lib.SEP_ERR_SHAPE   # group > 16 first
    assert call(S=1 << 21, B=1 << 30, Hq=16) == _lib.SEP_ERR_WORKSPACE

