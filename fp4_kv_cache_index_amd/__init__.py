"""CSA2 decode hot path for MI355X (gfx950): Python binding of libcsa2.so.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  The C-ABI, with the
meaning, layout and ownership of every argument, is include/csa2.h; the
function names here are the same.  If the library is not built this module
raises on first use: there is no fallback path.
"""
import contextlib
import ctypes
import os

import torch

D = 512
GROUP = 16
TOPK = 512
POOL_BLOCKS = 2048
BLOCK = 8
POOL = POOL_BLOCKS * BLOCK
WIN = 128
IDX_HEADS = 4
IDX_DIM = 64
HEADS = 16

FULL = 0
REINDEX = 1
OP_INDEX = 0
OP_ATTEND = 1

OK = 0
EINVAL = -1
ECAPACITY = -2
EWORKSPACE = -3
EUNSUPPORTED = -4
EHIP = -5
EDEVICE = -6  # debug library: an earlier call found a device precondition violated

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")
# the same library with the kernels' device-side precondition checks on
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2_debug.so")
# measurement helper (the streaming-read ceiling), not part of the method
ROOF_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2_roofline.so")
_lib = None
_debug_lib = None


class CSA2Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status) if _lib else status} ({status})")


class CacheStruct(ctypes.Structure):
    _fields_ = [("kv_codes", ctypes.c_void_p), ("kv_scales", ctypes.c_void_p), ("ik_codes", ctypes.c_void_p),
                ("ik_scales", ctypes.c_void_p), ("length", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("ratio", ctypes.c_int32)]


EXPORTS = ("csa2_quantize_append", "csa2_quantize_append_proj", "csa2_compress", "csa2_swa_append", "csa2_index_score_topk",
           "csa2_append_index_score_topk", "csa2_sparse_attend", "csa2_sparse_attend_noalloc",
           "csa2_workspace_bytes", "csa2_status_string", "csa2_version")


def _load(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cp = ctypes.POINTER(CacheStruct)
    L.csa2_quantize_append.restype = ctypes.c_int
    L.csa2_quantize_append.argtypes = [cp, vp, vp, vp, i32, i32, vp]
    L.csa2_quantize_append_proj.restype = ctypes.c_int
    L.csa2_quantize_append_proj.argtypes = [cp, vp, vp, vp, i32, i32, vp]
    L.csa2_compress.restype = ctypes.c_int
    L.csa2_compress.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    L.csa2_swa_append.restype = ctypes.c_int
    L.csa2_swa_append.argtypes = [vp, i32, vp, vp, i32, i32, vp]
    L.csa2_index_score_topk.restype = ctypes.c_int
    L.csa2_index_score_topk.argtypes = [cp, ctypes.c_int, vp, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.csa2_append_index_score_topk.restype = ctypes.c_int
    L.csa2_append_index_score_topk.argtypes = [cp, vp, vp, i32, i32, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.csa2_sparse_attend.restype = ctypes.c_int
    L.csa2_sparse_attend.argtypes = [cp, vp, vp, i32, vp, vp, i32, vp, vp, ctypes.c_float, vp, vp, i32, vp, sz, vp]
    L.csa2_sparse_attend_noalloc.restype = ctypes.c_int
    L.csa2_sparse_attend_noalloc.argtypes = [cp, vp, vp, i32, vp, vp, i32, vp, vp, ctypes.c_float, vp, vp, i32, vp]
    L.csa2_workspace_bytes.restype = sz
    L.csa2_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32]
    L.csa2_status_string.restype = ctypes.c_char_p
    L.csa2_status_string.argtypes = [ctypes.c_int]
    L.csa2_version.restype = ctypes.c_char_p
    return L


def lib():
    """Load libcsa2.so (built in-tree by __graft_entry__.build()), or the debug
    library when the environment sets CSA2_DEBUG=1."""
    global _lib
    if _lib is None:
        _lib = _load(DEBUG_LIB_PATH if os.environ.get("CSA2_DEBUG") == "1" else LIB_PATH)
    return _lib


def debug_lib():
    """The debug library (device-side precondition checks, CSA2_EDEVICE on the
    next call after a violation), loaded beside the release one."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


@contextlib.contextmanager
def using(L):
    """Route this module's calls through the library handle L (say debug_lib())
    inside the block."""
    global _lib
    prev = lib()
    _lib = L
    try:
        yield L
    finally:
        _lib = prev


def status_string(status: int) -> str:
    return lib().csa2_status_string(int(status)).decode()


def version() -> str:
    return lib().csa2_version().decode()


def workspace_bytes(op: int, B: int, Q: int, capacity: int) -> int:
    return int(lib().csa2_workspace_bytes(int(op), int(B), int(Q), int(capacity)))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(rc, what):
    if rc != OK:
        raise CSA2Error(rc, what)


def _expect(t, dtype, shape, name):
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


class Cache:
    """One KV-owning (Full) layer's global cache on the GPU (layout in csa2.h).

    ``host_len_bound`` is a host-side upper bound of every sequence length; the
    binding advances it on each append and passes it to the capacity check.
    """

    def __init__(self, batch, capacity, ratio=1, device="cuda"):
        self.batch, self.capacity, self.ratio = int(batch), int(capacity), int(ratio)
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.kv_codes = z((batch, capacity, D // 2), torch.uint8)
        self.kv_scales = z((batch, capacity, D // GROUP), torch.uint8)
        self.ik_codes = z((batch, capacity, IDX_DIM), torch.uint8)
        self.ik_scales = z((batch, capacity), torch.float32)
        self.length = z((batch,), torch.int32)
        self.host_len_bound = 0

    def struct(self) -> CacheStruct:
        return CacheStruct(self.kv_codes.data_ptr(), self.kv_scales.data_ptr(), self.ik_codes.data_ptr(),
                           self.ik_scales.data_ptr(), self.length.data_ptr(), self.batch, self.capacity,
                           self.ratio)


def quantize_append(cache: Cache, kv, ik, logits=None, stream=None):
    B, T = kv.shape[0], kv.shape[1]
    _expect(kv, torch.float32, (cache.batch, T, D), "kv")
    _expect(ik, torch.float32, (cache.batch, T // cache.ratio, IDX_DIM), "ik")
    if logits is not None:
        _expect(logits, torch.float32, (cache.batch, T, D), "logits")
    st = cache.struct()
    rc = lib().csa2_quantize_append(ctypes.byref(st), _ptr(kv), _ptr(logits), _ptr(ik), T, cache.host_len_bound,
                                    _stream(stream))
    _check(rc, "csa2_quantize_append")
    cache.host_len_bound += T // cache.ratio


def quantize_append_proj(cache: Cache, kv, w_ik, logits=None, stream=None):
    """csa2_quantize_append_proj: the new entries' indexer K is w_ik [512][64] applied to each entry."""
    B, T = kv.shape[0], kv.shape[1]
    _expect(kv, torch.float32, (cache.batch, T, D), "kv")
    _expect(w_ik, torch.float32, (D, IDX_DIM), "w_ik")
    if logits is not None:
        _expect(logits, torch.float32, (cache.batch, T, D), "logits")
    st = cache.struct()
    rc = lib().csa2_quantize_append_proj(ctypes.byref(st), _ptr(kv), _ptr(logits), _ptr(w_ik), T,
                                         cache.host_len_bound, _stream(stream))
    _check(rc, "csa2_quantize_append_proj")
    cache.host_len_bound += T // cache.ratio


def compress(kv, ratio, logits=None, out=None, stream=None):
    """csa2_compress: [B][T][512] token latents -> [B][T/ratio][512] fp32 entries."""
    B, T = kv.shape[0], kv.shape[1]
    _expect(kv, torch.float32, (B, T, D), "kv")
    if logits is not None:
        _expect(logits, torch.float32, (B, T, D), "logits")
    if out is None:
        out = torch.empty((B, T // ratio, D), dtype=torch.float32, device=kv.device)
    _expect(out, torch.float32, (B, T // ratio, D), "out")
    rc = lib().csa2_compress(_ptr(kv), _ptr(logits), B, T, ratio, _ptr(out), _stream(stream))
    _check(rc, "csa2_compress")
    return out


def swa_append(swa, x, seq_len, stream=None):
    B, S = swa.shape[0], swa.shape[1]
    T = x.shape[1]
    _expect(swa, torch.uint8, (B, S, D), "swa")
    _expect(x, torch.float32, (B, T, D), "x")
    _expect(seq_len, torch.int32, (B,), "seq_len")
    rc = lib().csa2_swa_append(_ptr(swa), S, _ptr(x), _ptr(seq_len), B, T, _stream(stream))
    _check(rc, "csa2_swa_append")


def index_score_topk(cache: Cache, mode, iq, topk_out, iw=None, q_pos=None, pool_in=None, pool_out=None, ws=None,
                     stream=None):
    B, Q = iq.shape[0], iq.shape[1]
    _expect(iq, torch.float32, (cache.batch, Q, IDX_HEADS, IDX_DIM), "iq")
    _expect(topk_out, torch.int32, (cache.batch, Q, TOPK), "topk_out")
    if iw is not None:
        _expect(iw, torch.float32, (cache.batch, Q, IDX_HEADS), "iw")
    if q_pos is not None:
        _expect(q_pos, torch.int32, (cache.batch, Q), "q_pos")
    if pool_in is not None:
        _expect(pool_in, torch.int32, (cache.batch, Q, POOL), "pool_in")
    if pool_out is not None:
        _expect(pool_out, torch.int32, (cache.batch, Q, POOL), "pool_out")
    need = workspace_bytes(OP_INDEX, cache.batch, Q, cache.capacity)
    if ws is None and need:
        ws = torch.zeros(need, dtype=torch.uint8, device=iq.device)
    st = cache.struct()
    rc = lib().csa2_index_score_topk(ctypes.byref(st), int(mode), _ptr(iq), _ptr(iw), _ptr(q_pos), _ptr(pool_in),
                                     _ptr(topk_out), _ptr(pool_out), Q, _ptr(ws),
                                     ws.numel() if ws is not None else 0, _stream(stream))
    _check(rc, "csa2_index_score_topk")


def append_index_score_topk(cache: Cache, kv, ik, iq, topk_out, iw=None, q_pos=None, pool_out=None, ws=None,
                            stream=None):
    """csa2_append_index_score_topk: the Full layer's append of kv/ik ([B][T][512],
    [B][T][64], ratio 1) and its scoring with Top-512 (and pool), in one call."""
    T = kv.shape[1]
    Q = iq.shape[1]
    _expect(kv, torch.float32, (cache.batch, T, D), "kv")
    _expect(ik, torch.float32, (cache.batch, T, IDX_DIM), "ik")
    _expect(iq, torch.float32, (cache.batch, Q, IDX_HEADS, IDX_DIM), "iq")
    _expect(topk_out, torch.int32, (cache.batch, Q, TOPK), "topk_out")
    if iw is not None:
        _expect(iw, torch.float32, (cache.batch, Q, IDX_HEADS), "iw")
    if q_pos is not None:
        _expect(q_pos, torch.int32, (cache.batch, Q), "q_pos")
    if pool_out is not None:
        _expect(pool_out, torch.int32, (cache.batch, Q, POOL), "pool_out")
    need = workspace_bytes(OP_INDEX, cache.batch, Q, cache.capacity)
    if ws is None and need:
        ws = torch.zeros(need, dtype=torch.uint8, device=iq.device)
    st = cache.struct()
    rc = lib().csa2_append_index_score_topk(ctypes.byref(st), _ptr(kv), _ptr(ik), T, cache.host_len_bound, _ptr(iq),
                                            _ptr(iw), _ptr(q_pos), _ptr(topk_out), _ptr(pool_out), Q, _ptr(ws),
                                            ws.numel() if ws is not None else 0, _stream(stream))
    _check(rc, "csa2_append_index_score_topk")
    cache.host_len_bound += T


def sparse_attend(cache: Cache, topk, swa, q, out, sm_scale, lse=None, q_pos=None, ws=None, stream=None,
                  swa_x=None, swa_len=None):
    """Attention of one layer; with `swa_x` ([B][T][512] f32) and `swa_len` ([B]
    i32 tokens after the append) the layer's new window tokens are appended to
    `swa` in the same launch first."""
    B, Q = q.shape[0], q.shape[1]
    S = swa.shape[1]
    _expect(q, torch.bfloat16, (cache.batch, Q, HEADS, D), "q")
    _expect(out, torch.bfloat16, (cache.batch, Q, HEADS, D), "out")
    _expect(topk, torch.int32, (cache.batch, Q, TOPK), "topk")
    _expect(swa, torch.uint8, (cache.batch, S, D), "swa")
    if lse is not None:
        _expect(lse, torch.float32, (cache.batch, Q, HEADS), "lse")
    if q_pos is not None:
        _expect(q_pos, torch.int32, (cache.batch, Q), "q_pos")
    T = 0
    if swa_x is not None:
        T = swa_x.shape[1]
        _expect(swa_x, torch.float32, (cache.batch, T, D), "swa_x")
        _expect(swa_len, torch.int32, (cache.batch,), "swa_len")
    need = workspace_bytes(OP_ATTEND, cache.batch, Q, cache.capacity)
    if ws is None and need:
        ws = torch.zeros(need, dtype=torch.uint8, device=q.device)
    st = cache.struct()
    rc = lib().csa2_sparse_attend(ctypes.byref(st), _ptr(topk), _ptr(swa), S, _ptr(swa_x), _ptr(swa_len), T,
                                  _ptr(q), _ptr(q_pos), float(sm_scale), _ptr(out), _ptr(lse), Q, _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(stream))
    _check(rc, "csa2_sparse_attend")


def sparse_attend_noalloc(cache: Cache, topk, swa, q, out, sm_scale, lse=None, q_pos=None, stream=None,
                          swa_x=None, swa_len=None):
    """csa2_sparse_attend_noalloc: sparse_attend with the split partials in the
    library's own per-GPU device array (no workspace, no allocation)."""
    Q = q.shape[1]
    S = swa.shape[1]
    _expect(q, torch.bfloat16, (cache.batch, Q, HEADS, D), "q")
    _expect(out, torch.bfloat16, (cache.batch, Q, HEADS, D), "out")
    _expect(topk, torch.int32, (cache.batch, Q, TOPK), "topk")
    _expect(swa, torch.uint8, (cache.batch, S, D), "swa")
    if lse is not None:
        _expect(lse, torch.float32, (cache.batch, Q, HEADS), "lse")
    if q_pos is not None:
        _expect(q_pos, torch.int32, (cache.batch, Q), "q_pos")
    T = 0
    if swa_x is not None:
        T = swa_x.shape[1]
        _expect(swa_x, torch.float32, (cache.batch, T, D), "swa_x")
        _expect(swa_len, torch.int32, (cache.batch,), "swa_len")
    st = cache.struct()
    rc = lib().csa2_sparse_attend_noalloc(ctypes.byref(st), _ptr(topk), _ptr(swa), S, _ptr(swa_x), _ptr(swa_len), T,
                                          _ptr(q), _ptr(q_pos), float(sm_scale), _ptr(out), _ptr(lse), Q,
                                          _stream(stream))
    _check(rc, "csa2_sparse_attend_noalloc")
