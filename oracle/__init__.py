"""CPU oracle for the CSA2 decode hot path: TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes front end of liboracle.so (csa2_oracle.c).  Only tests,
``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may import
this package; the GPU path never does.  Argument meanings follow the C-ABI of the
GPU library, but nothing is shared with it.

Every function takes and returns plain numpy arrays in the layouts below:

* main-KV codes ``[B][cap][256]`` u8 (byte i: channel 2i low nibble, 2i+1 high),
  scales ``[B][cap][32]`` u8 E4M3 (channels 16g..16g+15);
* indexer K ``[B][cap][64]`` u8 E4M3 with one fp32 scale per entry ``[B][cap]``;
* lengths ``[B]`` int32 (entries present);
* sliding window ``[B][S][512]`` u8 E4M3, token p in slot p mod S;
* indexer queries ``[B][Q][4][64]`` fp32, head weights ``[B][Q][4]`` fp32 or None;
* attention queries ``[B][Q][16][512]`` (bf16 values, passed as fp32).
"""
import ctypes
import os

import numpy as np

from . import build as _build

D = 512
GROUP = 16
TOPK = 512
POOL_BLOCKS = 2048
BLOCK = 8
POOL = POOL_BLOCKS * BLOCK
WIN = 128
IH = 4
ID = 64
HEADS = 16
FULL = 0
REINDEX = 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        _lib = ctypes.CDLL(path)
        _declare(_lib)
    return _lib


def _declare(L):
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_encode.restype = ctypes.c_uint8
    L.orc_e4m3_encode.argtypes = [ctypes.c_float]
    L.orc_e2m1_value.restype = ctypes.c_double
    L.orc_e2m1_value.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_encode.restype = ctypes.c_uint8
    L.orc_e2m1_encode.argtypes = [ctypes.c_float]
    L.orc_footprint_bytes_per_token.restype = ctypes.c_double
    L.orc_main_entry_bytes.restype = ctypes.c_int
    L.orc_indexer_entry_bytes.restype = ctypes.c_int
    L.orc_quantize_main_rows.argtypes = [f32p, i64, u8p, u8p]
    L.orc_dequant_main_rows.argtypes = [u8p, u8p, i64, f64p]
    L.orc_quantize_ik_rows.argtypes = [f32p, i64, u8p, f32p]
    L.orc_compress_pairs.argtypes = [f32p, f32p, i64, f32p]
    L.orc_compress.argtypes = [f32p, f32p, ctypes.c_int32, i64, f32p]
    L.orc_quantize_query.argtypes = [f32p, u8p, f32p]
    L.orc_entry_score.restype = ctypes.c_double
    L.orc_entry_score.argtypes = [u8p, f32p, f32p, u8p, ctypes.c_float]
    L.orc_quantize_append.restype = ctypes.c_int
    L.orc_quantize_append.argtypes = [u8p, u8p, u8p, f32p, i32p, i32, i32, i32, f32p, f32p, f32p, i32]
    L.orc_swa_append.restype = ctypes.c_int
    L.orc_swa_append.argtypes = [u8p, i32, f32p, i32p, i32, i32]
    L.orc_index_topk.restype = ctypes.c_int
    L.orc_index_topk.argtypes = [u8p, f32p, i32p, i32, i32, i32, ctypes.c_int, f32p, f32p, i32p, i32p,
                                 i32p, i32p, i32, f64p]
    L.orc_attend.restype = ctypes.c_int
    L.orc_attend.argtypes = [u8p, u8p, i32p, i32, i32, i32, i32p, u8p, i32, f32p, i32p, ctypes.c_float,
                             f64p, f64p, i32]
    L.orc_num_threads.restype = ctypes.c_int
    L.orc_set_threads.restype = None
    L.orc_set_threads.argtypes = [ctypes.c_int]


def _p(a, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError(f"{what}: oracle precondition violated (code {rc})")


# ----------------------------------------------------------------- codecs
def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code) & 0xFF)


def e4m3_encode(x: float) -> int:
    return int(lib().orc_e4m3_encode(float(x)))


def e2m1_value(nibble: int) -> float:
    return lib().orc_e2m1_value(int(nibble) & 0xF)


def e2m1_encode(x: float) -> int:
    return int(lib().orc_e2m1_encode(float(x)))


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_encode_array(x) -> np.ndarray:
    x = _c(np.asarray(x), np.float32).ravel()
    return np.array([e4m3_encode(v) for v in x], dtype=np.uint8)


def e4m3_decode_array(codes) -> np.ndarray:
    return e4m3_table()[np.asarray(codes, dtype=np.uint8)]


def footprint_bytes_per_token() -> float:
    return lib().orc_footprint_bytes_per_token()


def main_entry_bytes() -> int:
    return lib().orc_main_entry_bytes()


def indexer_entry_bytes() -> int:
    return lib().orc_indexer_entry_bytes()


# ------------------------------------------------------------- row helpers
def quantize_main(x):
    """fp32 rows [..., 512] -> (codes [..., 256] u8, scales [..., 32] u8)."""
    x = _c(x, np.float32)
    lead = x.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    codes = np.empty(lead + (D // 2,), np.uint8)
    scales = np.empty(lead + (D // GROUP,), np.uint8)
    lib().orc_quantize_main_rows(_p(x, ctypes.c_float), n, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8))
    return codes, scales


def dequant_main(codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    lead = codes.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (D,), np.float64)
    lib().orc_dequant_main_rows(_p(codes, ctypes.c_uint8), _p(scales, ctypes.c_uint8), n, _p(out, ctypes.c_double))
    return out


def quantize_ik(k):
    """fp32 rows [..., 64] -> (codes [..., 64] u8, scales [...] fp32)."""
    k = _c(k, np.float32)
    lead = k.shape[:-1]
    n = int(np.prod(lead)) if lead else 1
    codes = np.empty(lead + (ID,), np.uint8)
    scales = np.empty(lead, np.float32)
    lib().orc_quantize_ik_rows(_p(k, ctypes.c_float), n, _p(codes, ctypes.c_uint8), _p(scales, ctypes.c_float))
    return codes, scales


def compress_pairs(x, z):
    """[2n][512] tokens + logits -> [n][512] fp32 entries (ratio 2)."""
    x = _c(x, np.float32)
    z = _c(z, np.float32)
    n = x.shape[0] // 2
    out = np.empty((n, D), np.float32)
    lib().orc_compress_pairs(_p(x, ctypes.c_float), _p(z, ctypes.c_float), n, _p(out, ctypes.c_float))
    return out


def compress(x, z, m):
    """[m n][512] tokens + logits -> [n][512] fp32 entries: the ratio-2 rule
    over m consecutive tokens (per-channel softmax of the logits weighting the
    values, fp64 sums in token order, one rounding)."""
    x = _c(x, np.float32)
    z = _c(z, np.float32)
    n = x.shape[0] // m
    out = np.empty((n, D), np.float32)
    lib().orc_compress(_p(x, ctypes.c_float), _p(z, ctypes.c_float), int(m), n, _p(out, ctypes.c_float))
    return out


def project_ik(entries, w_ik):
    """Indexer K derived from main-KV entries (ai.info "Methodology in Plain
    English": CSA2 takes indexer K from a projection of the main KV entries).
    entries [..., 512] fp32, w_ik [512][64] fp32 channel-major:
    k[d] = sum_c w_ik[c][d] * entry[c], each product exact in fp64, summed in
    fp64 (a library matmul), rounded once to fp32."""
    e = np.asarray(entries, np.float32).astype(np.float64)
    w = np.asarray(w_ik, np.float32).astype(np.float64)
    assert w.shape == (D, ID)
    return (e @ w).astype(np.float32)


def quantize_query(iq):
    iq = _c(iq, np.float32).reshape(IH, ID)
    q8 = np.empty((IH, ID), np.uint8)
    sq = np.empty((IH,), np.float32)
    lib().orc_quantize_query(_p(iq, ctypes.c_float), _p(q8, ctypes.c_uint8), _p(sq, ctypes.c_float))
    return q8, sq


def entry_score(q8, sq, w, k8, sk) -> float:
    q8 = _c(q8, np.uint8)
    sq = _c(sq, np.float32)
    w = _c(w, np.float32)
    k8 = _c(k8, np.uint8)
    return float(lib().orc_entry_score(_p(q8, ctypes.c_uint8), _p(sq, ctypes.c_float), _p(w, ctypes.c_float),
                                       _p(k8, ctypes.c_uint8), float(sk)))


# ------------------------------------------------------------------- cache
class Cache:
    """Host copy of one KV-owning layer's global cache."""

    def __init__(self, batch: int, capacity: int, ratio: int = 1):
        self.B, self.cap, self.ratio = int(batch), int(capacity), int(ratio)
        self.kv_codes = np.zeros((batch, capacity, D // 2), np.uint8)
        self.kv_scales = np.zeros((batch, capacity, D // GROUP), np.uint8)
        self.ik_codes = np.zeros((batch, capacity, ID), np.uint8)
        self.ik_scales = np.zeros((batch, capacity), np.float32)
        self.length = np.zeros((batch,), np.int32)


def quantize_append(cache: Cache, kv, ik, logits=None):
    kv = _c(kv, np.float32)
    ik = _c(ik, np.float32)
    logits = _c(logits, np.float32)
    T = kv.shape[1]
    rc = lib().orc_quantize_append(_p(cache.kv_codes, ctypes.c_uint8), _p(cache.kv_scales, ctypes.c_uint8),
                                   _p(cache.ik_codes, ctypes.c_uint8), _p(cache.ik_scales, ctypes.c_float),
                                   _p(cache.length, ctypes.c_int32), cache.B, cache.cap, cache.ratio,
                                   _p(kv, ctypes.c_float), _p(logits, ctypes.c_float), _p(ik, ctypes.c_float), T)
    _check(rc, "quantize_append")


def quantize_append_proj(cache: Cache, kv, w_ik, logits=None):
    """quantize_append with each new entry's indexer K = project_ik(entry), the
    entry being the token row (ratio 1) or the tokens it compresses (ratio 2 or more)."""
    kv = _c(kv, np.float32)
    if cache.ratio == 2:
        logits = _c(logits, np.float32)
        entries = np.stack([compress_pairs(kv[b], logits[b]) for b in range(kv.shape[0])])
    elif cache.ratio > 2:
        logits = _c(logits, np.float32)
        entries = np.stack([compress(kv[b], logits[b], cache.ratio) for b in range(kv.shape[0])])
    else:
        entries = kv
    quantize_append(cache, kv, project_ik(entries, w_ik), logits=logits)


def swa_append(swa, x, seq_len):
    """swa [B][S][512] u8 (updated in place); x [B][T][512] fp32; seq_len [B]."""
    x = _c(x, np.float32)
    seq_len = _c(seq_len, np.int32)
    assert swa.flags.c_contiguous and swa.dtype == np.uint8
    B, T = x.shape[0], x.shape[1]
    rc = lib().orc_swa_append(_p(swa, ctypes.c_uint8), swa.shape[1], _p(x, ctypes.c_float),
                              _p(seq_len, ctypes.c_int32), B, T)
    _check(rc, "swa_append")


def index_topk(cache: Cache, mode: int, iq, iw=None, q_pos=None, pool_in=None, want_pool=False,
               want_scores=False):
    """Returns (topk [B][Q][512], pool [B][Q][16384] or None, scores [B][Q][cap] or None)."""
    iq = _c(iq, np.float32)
    B, Q = iq.shape[0], iq.shape[1]
    iw = _c(iw, np.float32)
    q_pos = _c(q_pos, np.int32)
    pool_in = _c(pool_in, np.int32)
    topk = np.empty((B, Q, TOPK), np.int32)
    pool = np.empty((B, Q, POOL), np.int32) if want_pool else None
    scores = np.empty((B, Q, cache.cap), np.float64) if want_scores else None
    rc = lib().orc_index_topk(_p(cache.ik_codes, ctypes.c_uint8), _p(cache.ik_scales, ctypes.c_float),
                              _p(cache.length, ctypes.c_int32), cache.B, cache.cap, cache.ratio, int(mode),
                              _p(iq, ctypes.c_float), _p(iw, ctypes.c_float), _p(q_pos, ctypes.c_int32),
                              _p(pool_in, ctypes.c_int32), _p(topk, ctypes.c_int32), _p(pool, ctypes.c_int32), Q,
                              _p(scores, ctypes.c_double))
    _check(rc, "index_topk")
    return topk, pool, scores


def attend(cache: Cache, topk, swa, q, sm_scale, q_pos=None):
    """Returns (out [B][Q][16][512] fp64, lse [B][Q][16] fp64)."""
    topk = _c(topk, np.int32)
    q = _c(q, np.float32)
    q_pos = _c(q_pos, np.int32)
    swa = _c(swa, np.uint8)
    B, Q = q.shape[0], q.shape[1]
    out = np.empty((B, Q, HEADS, D), np.float64)
    lse = np.empty((B, Q, HEADS), np.float64)
    rc = lib().orc_attend(_p(cache.kv_codes, ctypes.c_uint8), _p(cache.kv_scales, ctypes.c_uint8),
                          _p(cache.length, ctypes.c_int32), cache.B, cache.cap, cache.ratio,
                          _p(topk, ctypes.c_int32), _p(swa, ctypes.c_uint8), swa.shape[1], _p(q, ctypes.c_float),
                          _p(q_pos, ctypes.c_int32), float(sm_scale), _p(out, ctypes.c_double),
                          _p(lse, ctypes.c_double), Q)
    _check(rc, "attend")
    return out, lse


def num_threads() -> int:
    return lib().orc_num_threads()


def set_threads(n: int) -> None:
    """Threads for the oracle's parallel loops (timing only: results do not
    depend on the count)."""
    lib().orc_set_threads(int(n))
