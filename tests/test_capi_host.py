"""The C ABI on the host: the built library loads, exports every function
include/ws.h declares, and rejects bad arguments before touching a GPU.

No call here reaches a kernel launch: each one fails validation, which
happens on the host before any HIP call. Device pointers are fake addresses
that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

from cached_block_causal_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced


def _header_functions():
    text = open(os.path.join(ROOT, "include", "ws.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ws_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libws.so is not built (run __graft_entry__.build())")
    return L.lib()


def _err(lib):
    return lib.ws_last_error().decode()


def test_every_declared_function_is_exported(lib):
    names = _header_functions()
    assert set(names) == set(L.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)


def test_status_strings(lib):
    for s in range(8):
        assert lib.ws_status_string(s)
    assert lib.ws_status_string(0) == b"ok"


def _cache(heads=2, d=128, cap=100, length=10, k=FAKE, v=FAKE + 4096):
    return L.WsKvCache(k, v, heads, d, cap, length)


def test_append_validation(lib):
    c = _cache()
    args = lambda **kw: dict(dict(ks=FAKE, vs=FAKE, n=5, h=4, hb=0, lay=0), **kw)
    def call(cache, **kw):
        a = args(**kw)
        return lib.ws_kv_append(ctypes.byref(cache) if cache is not None else None, a["ks"],
                                a["vs"], a["n"], a["h"], a["hb"], a["lay"], None)
    assert call(None) == L.WS_ERR_NULL
    assert call(c, n=91) == L.WS_ERR_CAPACITY and c.len == 10 and "capacity" in _err(lib)
    assert call(c, hb=3) == L.WS_ERR_SHAPE            # heads [3, 5) of 4
    assert call(c, hb=-1) == L.WS_ERR_SHAPE
    assert call(c, n=-1) == L.WS_ERR_SHAPE
    assert call(c, lay=2) == L.WS_ERR_UNSUPPORTED
    assert call(_cache(d=96)) == L.WS_ERR_UNSUPPORTED
    assert call(_cache(length=101)) == L.WS_ERR_SHAPE
    assert call(c, ks=None) == L.WS_ERR_NULL
    assert call(c, ks=FAKE + 8) == L.WS_ERR_ALIGN
    assert call(_cache(k=FAKE + 2)) == L.WS_ERR_ALIGN
    assert call(c, n=0, ks=None, vs=None) == L.WS_OK and c.len == 10   # no-op
    assert c.len == 10


def test_append_segments_validation(lib):
    c = _cache()
    def segs(*items):
        arr = (L.WsKvSegment * max(1, len(items)))()
        for i, it in enumerate(items):
            arr[i] = L.WsKvSegment(*it)
        return arr
    ok = (FAKE, FAKE, 5, 4, 0, L.WS_TOKEN_MAJOR)
    empty = (None, None, 0, 4, 0, L.WS_HEAD_MAJOR)
    call = lambda s, n: lib.ws_kv_append_segments(ctypes.byref(c), s, n, None)
    assert lib.ws_kv_append_segments(ctypes.byref(c), None, 1, None) == L.WS_ERR_NULL
    assert call(segs(ok), 0) == L.WS_ERR_SHAPE
    assert call(segs(ok, ok, ok, ok, ok), 5) == L.WS_ERR_SHAPE
    assert call(segs(ok, (FAKE, FAKE, 5, 4, 0, 2)), 2) == L.WS_ERR_UNSUPPORTED
    assert call(segs(ok, (FAKE, FAKE, -1, 4, 0, 0)), 2) == L.WS_ERR_SHAPE
    assert call(segs(ok, (FAKE, FAKE, 5, 4, 3, 0)), 2) == L.WS_ERR_SHAPE   # heads [3, 5) of 4
    # 45 + 46 tokens do not fit the 90 free rows: refused as a whole
    assert call(segs((FAKE, FAKE, 45, 4, 0, 0), (FAKE, FAKE, 46, 2, 0, 1)), 2) == L.WS_ERR_CAPACITY
    assert c.len == 10 and "capacity" in _err(lib)
    assert call(segs(ok, (None, FAKE, 5, 4, 0, 0)), 2) == L.WS_ERR_NULL
    assert call(segs((FAKE + 8, FAKE, 5, 4, 0, 0), ok), 2) == L.WS_ERR_ALIGN
    assert call(segs(empty, empty), 2) == L.WS_OK and c.len == 10     # nothing to write


def _attn(lib, cache, **kw):
    a = dict(q=FAKE, nq=50, ks=None, vs=None, ns=0, units=1, qb=[0, 50], kend=[10], scale=0.1,
             splits=1, out=FAKE, ws=None, wsb=0)
    a.update(kw)
    qb = (ctypes.c_int32 * len(a["qb"]))(*a["qb"])
    ke = (ctypes.c_int32 * len(a["kend"]))(*a["kend"])
    return lib.ws_block_causal_attn(ctypes.byref(cache), a["q"], a["nq"], a["ks"], a["vs"],
                                    a["ns"], a["units"], qb, ke, a["scale"], a["splits"],
                                    a["out"], a["ws"], a["wsb"], None)


def test_attention_validation(lib):
    c = _cache()
    assert _attn(lib, c, kend=[11]) == L.WS_ERR_SHAPE             # beyond len + n_self
    assert _attn(lib, c, kend=[0]) == L.WS_ERR_SHAPE
    assert _attn(lib, c, qb=[0, 49]) == L.WS_ERR_SHAPE            # does not end at n_q
    assert _attn(lib, c, qb=[1, 50]) == L.WS_ERR_SHAPE
    assert _attn(lib, c, units=2, qb=[0, 30, 20], kend=[5, 10]) == L.WS_ERR_SHAPE
    assert _attn(lib, c, units=2, qb=[0, 20, 50], kend=[8, 5]) == L.WS_ERR_SHAPE
    assert _attn(lib, c, units=0) == L.WS_ERR_SHAPE
    # more than WS_MAX_UNITS units with queries: their table needs the workspace
    live = list(range(71))
    assert _attn(lib, c, nq=70, units=70, qb=live, kend=[10] * 70) == L.WS_ERR_WORKSPACE
    assert _attn(lib, c, nq=70, units=70, qb=live, kend=[10] * 70, ws=FAKE,
                 wsb=lib.ws_attn_workspace_bytes(2, 70, 128, 1) - 4) == L.WS_ERR_WORKSPACE
    assert _attn(lib, c, nq=70, units=70, qb=live, kend=list(range(10, 0, -1)) * 7) == L.WS_ERR_SHAPE
    assert _attn(lib, c, scale=0.0) == L.WS_ERR_SHAPE
    assert _attn(lib, c, scale=float("nan")) == L.WS_ERR_SHAPE
    assert _attn(lib, c, splits=-1) == L.WS_ERR_SHAPE
    assert _attn(lib, c, splits=257) == L.WS_ERR_SHAPE
    assert _attn(lib, c, q=None) == L.WS_ERR_NULL
    assert _attn(lib, c, ns=4, kend=[14]) == L.WS_ERR_NULL         # own tokens without buffers
    assert _attn(lib, c, out=FAKE + 4) == L.WS_ERR_ALIGN
    assert _attn(lib, c, splits=4) == L.WS_ERR_WORKSPACE
    need = lib.ws_attn_workspace_bytes(2, 50, 128, 4)
    assert _attn(lib, c, splits=4, ws=FAKE, wsb=need - 1) == L.WS_ERR_WORKSPACE
    assert _attn(lib, c, splits=4, ws=FAKE + 8, wsb=need) == L.WS_ERR_ALIGN
    assert _attn(lib, _cache(d=80)) == L.WS_ERR_UNSUPPORTED
    assert _attn(lib, c, nq=0, qb=[0, 0], q=None, out=None) == L.WS_OK  # no-op


def test_merge_and_euler_validation(lib):
    assert lib.ws_attn_merge(2, 10, 96, 2, FAKE, 1 << 20, FAKE, None) == L.WS_ERR_UNSUPPORTED
    assert lib.ws_attn_merge(2, 10, 128, 0, FAKE, 1 << 20, FAKE, None) == L.WS_ERR_SHAPE
    assert lib.ws_attn_merge(2, 10, 128, 2, None, 1 << 20, FAKE, None) == L.WS_ERR_WORKSPACE
    assert lib.ws_attn_merge(2, 10, 128, 2, FAKE, 8, FAKE, None) == L.WS_ERR_WORKSPACE
    assert lib.ws_attn_merge(2, 10, 128, 1, None, 0, None, None) == L.WS_OK   # nothing to merge
    assert lib.ws_fm_euler_step(None, FAKE, 10, 0.25, None) == L.WS_ERR_NULL
    assert lib.ws_fm_euler_step(FAKE, FAKE, -1, 0.25, None) == L.WS_ERR_SHAPE
    assert lib.ws_fm_euler_step(FAKE, FAKE, 10, float("inf"), None) == L.WS_ERR_SHAPE
    assert lib.ws_fm_euler_step(FAKE + 4, FAKE, 10, 0.25, None) == L.WS_ERR_ALIGN
    assert lib.ws_fm_euler_step(None, None, 0, 0.25, None) == L.WS_OK


def test_split_planning_is_host_only_and_sized(lib):
    assert lib.ws_attn_default_splits(0, 10, 128, 100) == 1
    # one split: nothing, or room for a unit table of up to n_q units
    assert lib.ws_attn_workspace_bytes(10, 64, 128, 1) == 0
    assert lib.ws_attn_workspace_bytes(10, 920, 128, 1) == (2 * 920 + 1) * 4
    for heads, nq, d, nk in [(10, 920, 128, 61880), (40, 920, 128, 61880), (24, 252, 128, 9372),
                             (40, 4, 128, 244772), (4, 252, 64, 804)]:
        s = lib.ws_attn_default_splits(heads, nq, d, nk)
        assert 1 <= s <= 256
        need = lib.ws_attn_workspace_bytes(heads, nq, d, s)
        assert need >= (s > 1) * s * heads * nq * (d + 1) * 4 + (nq > 64) * (2 * nq + 1) * 4
    # at most 32 queries: one round of 1024 one-wave workgroups, at most a
    # quarter of the 32-key tiles per split
    assert lib.ws_attn_default_splits(40, 4, 128, 244772) == 25
    assert lib.ws_attn_default_splits(10, 32, 128, 244772) == 102
    assert lib.ws_attn_default_splits(3, 1, 64, 200) == 1
    assert lib.ws_attn_default_splits(2000, 4, 128, 244772) == 1


def test_c_abi_demo_compiles_as_c99():
    """include/ws.h is a C header: the plain-C demo builds with gcc -std=c99
    -Wall -Wextra against libws.so."""
    from cached_block_causal_amd import build as b
    path = b.build_demo()
    assert os.path.exists(path)


def test_host_code_clean_under_asan_and_ubsan(tmp_path):
    """The library's host code (argument validation, split planning, status
    text) called from C under AddressSanitizer and UndefinedBehaviorSanitizer:
    tests/capi_errors.c makes every refused call and runs the planning
    functions over extreme sizes; neither sanitizer may report anything.
    The sanitizers instrument host code only (no call reaches a GPU)."""
    import subprocess
    from cached_block_causal_amd import build as b
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(b.hipcc())))
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    if not os.path.exists(clang):
        pytest.skip("ROCm clang not found")
    lib = str(tmp_path / "libws.so")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    r = subprocess.run([b.hipcc(), f"--offload-arch={b.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC",
                        "-shared", *san, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        "-I", b.INCLUDE, "-I", b.CSRC, *[os.path.join(b.CSRC, s) for s in b.SOURCES],
                        "-o", lib], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "capi_errors")
    r = subprocess.run([clang, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
                        "-fno-omit-frame-pointer", "-I", b.INCLUDE,
                        os.path.join(ROOT, "tests", "capi_errors.c"), lib,
                        f"-Wl,-rpath,{tmp_path}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}",
                        "-o", exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
               ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and "capi_errors ok" in r.stdout, r.stdout + r.stderr[-3000:]
