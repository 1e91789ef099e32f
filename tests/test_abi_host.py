"""Host-side checks of the C-ABI library that need no GPU: it loads, exports
every symbol include/csa2.h declares, sizes workspaces, and rejects invalid
arguments with the documented status before enqueuing anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def csa():
    import fp4_kv_cache_index_amd as csa
    if not os.path.exists(csa.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    csa.lib()
    return csa


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(csa2_\w+)\s*\(", src, re.M)))


def test_exports_every_declared_symbol(csa):
    syms = declared_symbols()
    assert set(syms) == set(csa.EXPORTS), syms
    L = csa.lib()
    for s in syms:
        assert hasattr(L, s), s


def test_roofline_helper_exports_its_header():
    """libcsa2_roofline.so (the streaming-read ceiling helper) exports every
    symbol include/csa2_roofline.h declares and rejects bad arguments before
    touching a device."""
    import fp4_kv_cache_index_amd as csa
    src = open(os.path.join(ROOT, "include", "csa2_roofline.h")).read()
    syms = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(csa2roof_\w+)\s*\(", src, re.M)))
    assert syms == ["csa2roof_stream_read"]
    L = ctypes.CDLL(csa.ROOF_LIB_PATH)
    f = L.csa2roof_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    p = ctypes.c_void_p(FAKE)
    assert f(None, 16, p, 1, None) == -1
    assert f(p, 15, p, 1, None) == -1
    assert f(ctypes.c_void_p(FAKE + 8), 16, p, 1, None) == -1
    assert f(p, 16, None, 1, None) == -1
    assert f(p, 16, p, 0, None) == -1
    assert f(p, 0, p, 1, None) == 0


def test_status_strings_and_version(csa):
    for code in (csa.OK, csa.EINVAL, csa.ECAPACITY, csa.EWORKSPACE, csa.EUNSUPPORTED, csa.EHIP, csa.EDEVICE):
        assert csa.status_string(code) and csa.status_string(code) != "unknown status"
    assert csa.status_string(12345) == "unknown status"
    assert "gfx950" in csa.version() and not csa.version().endswith("debug")


def test_debug_library_exports_and_version(csa):
    """The debug library exports the same symbols, says it is the debug build,
    and keeps its internals in a namespace of its own (both load side by side)."""
    D = csa.debug_lib()
    for s in declared_symbols():
        assert hasattr(D, s), s
    assert D.csa2_version().decode().endswith("debug")
    assert D.csa2_workspace_bytes(csa.OP_INDEX, 16, 1, 131072) == csa.workspace_bytes(csa.OP_INDEX, 16, 1, 131072)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", csa.DEBUG_LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        assert "10csa2_debug" in out.stdout and "4csa2" not in out.stdout  # mangled namespace names


@pytest.fixture(params=["release", "debug"])
def L(request, csa):
    """Each host-validation test runs against both libraries: the debug one
    validates exactly as the release one does."""
    return csa.lib() if request.param == "release" else csa.debug_lib()


def test_workspace_sizes(csa):
    ws = csa.workspace_bytes
    assert ws(csa.OP_INDEX, 0, 1, 100) == 0 and ws(7, 1, 1, 100) == 0
    a = ws(csa.OP_INDEX, 16, 1, 131072)
    assert a > 0 and ws(csa.OP_INDEX, 32, 1, 131072) > a and ws(csa.OP_INDEX, 16, 1, 262144) > a
    assert ws(csa.OP_ATTEND, 16, 1, 0) > 0
    assert ws(csa.OP_ATTEND, 1, 2048, 0) == 0  # enough queries: no split, no workspace
    assert ws(csa.OP_ATTEND, 1, 300, 0) > 0  # 300 queries split in two


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def cache(csa, B=2, cap=100, ratio=1, **over):
    c = csa.CacheStruct(FAKE, FAKE, FAKE, FAKE, FAKE, B, cap, ratio)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_append_rejections(csa, L):
    p = ctypes.c_void_p(FAKE)
    q = L.csa2_quantize_append
    assert q(None, p, None, p, 1, 0, None) == csa.EINVAL
    assert q(ctypes.byref(cache(csa, ratio=3)), p, None, p, 1, 0, None) == csa.EINVAL   # T % r
    assert q(ctypes.byref(cache(csa, ratio=0)), p, p, p, 1, 0, None) == csa.EINVAL      # ratio 1..16
    assert q(ctypes.byref(cache(csa, ratio=17)), p, p, p, 17, 0, None) == csa.EINVAL
    assert q(ctypes.byref(cache(csa, ratio=4)), p, None, p, 4, 0, None) == csa.EINVAL   # logits missing
    assert q(ctypes.byref(cache(csa, ratio=2)), p, p, p, 3, 0, None) == csa.EINVAL      # T % r
    assert q(ctypes.byref(cache(csa, ratio=2)), p, None, p, 2, 0, None) == csa.EINVAL   # logits missing
    assert q(ctypes.byref(cache(csa, ratio=1)), p, p, p, 2, 0, None) == csa.EINVAL      # logits given
    assert q(ctypes.byref(cache(csa, cap=10)), p, None, p, 4, 7, None) == csa.ECAPACITY
    assert q(ctypes.byref(cache(csa)), p, None, p, -1, 0, None) == csa.EINVAL
    assert q(ctypes.byref(cache(csa, kv_codes=None)), p, None, p, 1, 0, None) == csa.EINVAL
    assert q(ctypes.byref(cache(csa, cap=1 << 30)), p, None, p, 1, 0, None) == csa.EUNSUPPORTED
    assert q(ctypes.byref(cache(csa)), ctypes.c_void_p(FAKE + 4), None, p, 1, 0, None) == csa.EINVAL  # misaligned
    assert q(ctypes.byref(cache(csa)), p, None, p, 0, 0, None) == csa.OK  # nothing to do


def test_append_proj_rejections(csa, L):
    """The projected append validates like the plain one, and needs its w_ik."""
    p = ctypes.c_void_p(FAKE)
    q = L.csa2_quantize_append_proj
    assert q(None, p, None, p, 1, 0, None) == csa.EINVAL
    assert q(ctypes.byref(cache(csa, ratio=3)), p, None, p, 1, 0, None) == csa.EINVAL   # T % r
    assert q(ctypes.byref(cache(csa, ratio=0)), p, p, p, 1, 0, None) == csa.EINVAL      # ratio 1..16
    assert q(ctypes.byref(cache(csa, ratio=17)), p, p, p, 17, 0, None) == csa.EINVAL
    assert q(ctypes.byref(cache(csa, ratio=4)), p, None, p, 4, 0, None) == csa.EINVAL   # logits missing
    assert q(ctypes.byref(cache(csa, ratio=2)), p, p, p, 3, 0, None) == csa.EINVAL      # T % r
    assert q(ctypes.byref(cache(csa, ratio=2)), p, None, p, 2, 0, None) == csa.EINVAL   # logits missing
    assert q(ctypes.byref(cache(csa, cap=10)), p, None, p, 4, 7, None) == csa.ECAPACITY
    assert q(ctypes.byref(cache(csa)), p, None, None, 1, 0, None) == csa.EINVAL          # no w_ik
    assert q(ctypes.byref(cache(csa)), p, None, ctypes.c_void_p(FAKE + 2), 1, 0, None) == csa.EINVAL  # misaligned
    assert q(ctypes.byref(cache(csa)), p, None, p, 0, 0, None) == csa.OK  # nothing to do
    # and the plain append still needs its ik rows
    assert L.csa2_quantize_append(ctypes.byref(cache(csa)), p, None, None, 1, 0, None) == csa.EINVAL


def test_swa_rejections(csa, L):
    p = ctypes.c_void_p(FAKE)
    s = L.csa2_swa_append
    assert s(p, 0, p, p, 1, 1, None) == csa.EINVAL
    assert s(p, 128, p, p, 1, 129, None) == csa.EINVAL
    assert s(None, 128, p, p, 1, 1, None) == csa.EINVAL
    assert s(p, 128, p, None, 1, 1, None) == csa.EINVAL
    assert s(p, 128, p, p, 0, 1, None) == csa.OK


def test_compress_rejections(csa, L):
    p = ctypes.c_void_p(FAKE)
    c = L.csa2_compress
    assert c(p, p, 1, 3, 2, p, None) == csa.EINVAL  # T % ratio
    assert c(p, None, 1, 4, 2, p, None) == csa.EINVAL  # ratio 2 needs logits
    assert c(p, p, 1, 4, 1, p, None) == csa.EINVAL  # ratio 1 takes none
    assert c(p, p, 1, 34, 17, p, None) == csa.EINVAL  # ratio above 16
    assert c(None, p, 1, 4, 2, p, None) == csa.EINVAL
    assert c(p, p, 1, 4, 2, None, None) == csa.EINVAL
    assert c(p, p, -1, 4, 2, p, None) == csa.EINVAL
    assert c(p, p, 0, 4, 2, p, None) == csa.OK and c(p, p, 3, 0, 2, p, None) == csa.OK


def test_attend_noalloc_rejections(csa, L):
    """Host checks of the no-allocation attention call, all before any device use."""
    p = ctypes.c_void_p(FAKE)
    a = L.csa2_sparse_attend_noalloc
    c = ctypes.byref(cache(csa, B=1, cap=100))
    # 1,021 queries need two splits of partials, 64.1 MiB: more than the library's array
    assert csa.workspace_bytes(csa.OP_ATTEND, 1, 1021, 100) > (64 << 20)
    assert a(c, p, p, 128, None, None, 0, p, None, 0.1, p, None, 1021, None) == csa.EWORKSPACE
    assert csa.workspace_bytes(csa.OP_ATTEND, 1, 1020, 100) <= (64 << 20)
    assert csa.workspace_bytes(csa.OP_ATTEND, 1, 1025, 100) == 0
    assert a(c, p, p, 0, None, None, 0, p, None, 0.1, p, None, 1, None) == csa.EINVAL      # S < 1
    assert a(c, p, p, 128, p, None, 1, p, None, 0.1, p, None, 1, None) == csa.EINVAL      # swa_x without swa_len
    assert a(c, p, p, 128, None, None, 0, p, None, 0.1, p, None, -1, None) == csa.EINVAL  # Q < 0
    assert a(c, p, p, 128, None, None, 0, p, None, 0.1, p, None, 0, None) == csa.OK       # nothing to do
    assert a(ctypes.byref(cache(csa, B=0)), p, p, 128, None, None, 0, p, None, 0.1, p, None, 1, None) == csa.OK


def test_index_rejections(csa, L):
    p = ctypes.c_void_p(FAKE)
    f = L.csa2_index_score_topk
    c = ctypes.byref(cache(csa, cap=131072))
    assert f(c, 5, p, None, None, None, p, None, 1, p, 1 << 40, None) == csa.EINVAL          # mode
    assert f(c, csa.FULL, p, None, None, p, p, None, 1, p, 1 << 40, None) == csa.EINVAL      # pool_in on Full
    assert f(c, csa.REINDEX, p, None, None, None, p, None, 1, p, 1 << 40, None) == csa.EINVAL  # no pool_in
    assert f(c, csa.REINDEX, p, None, None, p, p, p, 1, p, 1 << 40, None) == csa.EINVAL     # pool_out on Reindex
    assert f(c, csa.FULL, None, None, None, None, p, None, 1, p, 1 << 40, None) == csa.EINVAL
    assert f(c, csa.FULL, p, None, None, None, p, None, 1, p, 16, None) == csa.EWORKSPACE
    assert f(c, csa.FULL, p, None, None, None, p, None, 1, None, 0, None) == csa.EWORKSPACE
    assert f(c, csa.FULL, p, None, None, None, p, None, -1, p, 1 << 40, None) == csa.EINVAL
    big = ctypes.byref(cache(csa, cap=(1 << 23) + 1))
    assert f(big, csa.FULL, p, None, None, None, p, None, 1, p, 1 << 40, None) == csa.EUNSUPPORTED
    assert f(c, csa.FULL, p, None, None, None, p, None, 0, None, 0, None) == csa.OK


def test_attend_rejections(csa, L):
    p = ctypes.c_void_p(FAKE)
    a = L.csa2_sparse_attend
    c = ctypes.byref(cache(csa, B=16))
    big_ws = 1 << 40
    # (cache, topk, swa, S, swa_x, swa_len, swa_T, q, q_pos, sm_scale, out, lse, Q, ws, ws_bytes, stream)
    assert a(c, p, p, 0, None, None, 0, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL        # S
    assert a(c, None, p, 128, None, None, 0, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL   # topk
    assert a(c, p, p, 128, None, None, 0, p, None, 1.0, None, None, 1, p, big_ws, None) == csa.EINVAL   # out
    assert a(c, p, p, 128, None, None, 0, p, None, 1.0, p, None, 1, p, 8, None) == csa.EWORKSPACE
    assert a(ctypes.byref(cache(csa, kv_scales=None)), p, p, 128, None, None, 0, p, None, 1.0, p, None, 1, p,
             big_ws, None) == csa.EINVAL
    # fused window append: x, its lengths and T come together, 1 <= T <= S
    assert a(c, p, p, 128, p, None, 1, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL          # no swa_len
    assert a(c, p, p, 128, p, p, 0, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL             # T = 0
    assert a(c, p, p, 128, p, p, 129, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL           # T > S
    assert a(c, p, p, 128, None, p, 0, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL          # stray len
    assert a(c, p, p, 128, None, None, 3, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL       # stray T
    odd = ctypes.c_void_p(FAKE + 4)
    assert a(c, odd, p, 128, None, None, 0, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL     # topk align
    assert a(c, p, p, 128, odd, p, 1, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL           # x align
    assert a(c, p, None, 128, p, p, 1, p, None, 1.0, p, None, 1, p, big_ws, None) == csa.EINVAL          # no ring
    # zero queries and no append: nothing to do
    assert a(c, None, None, 128, None, None, 0, None, None, 1.0, None, None, 0, None, 0, None) == csa.OK