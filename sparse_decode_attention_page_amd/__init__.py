"""EntmaxKV decode hot path on one MI355X: Python binding of libentmaxkv.so.

Thin ctypes marshalling over the C ABI declared in ``include/entmaxkv.h``: every
function takes torch tensors that already live on the GPU, checks their shapes and
dtypes, and passes raw device pointers plus the current HIP stream.  All the
computation happens in the library's HIP kernels; there is no fallback path.  If
the library is missing, the first call raises.

Names, argument order and semantics follow the C ABI:
``build_page_meta``, ``score_pages``, ``select_pages_topk``, ``select_pages_gauss``,
``entmax_decode_sparse``, ``entmax_decode_full``, ``softmax_decode_full``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libentmaxkv.so")
_lib = None

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
(CALL_SCORE, CALL_TOPK, CALL_GAUSS, CALL_DECODE_SPARSE, CALL_DECODE_FULL, CALL_SOFTMAX, CALL_SOFTMAX_SPARSE,
 CALL_TOPK_GROUP, CALL_GAUSS_GROUP, CALL_DECODE_GROUP) = range(1, 11)

EXPORTS = ("build_page_meta", "score_pages", "build_page_meta_f8", "score_pages_f8", "append_token",
           "select_pages_topk", "select_pages_gauss", "select_pages_topk_group", "select_pages_gauss_group",
           "entmax_decode_sparse_group",
           "entmax_decode_sparse", "entmax_decode_full", "softmax_decode_full", "softmax_decode_sparse",
           "entmaxkv_workspace_bytes", "entmaxkv_status_string", "entmaxkv_gauss_hermite16",
           "entmaxkv_stream_read")


class EntmaxKVError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn}: status {status} ({status_string(status)})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_phys_pages", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_double)]


def load(path: str | None = None):
    """Load libentmaxkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m sparse_decode_attention_page_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, sz, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    sh = ctypes.POINTER(Shape)
    lib.entmaxkv_workspace_bytes.restype = sz
    lib.entmaxkv_workspace_bytes.argtypes = [sh, i32]
    lib.entmaxkv_status_string.restype = ctypes.c_char_p
    lib.entmaxkv_status_string.argtypes = [i32]
    lib.entmaxkv_gauss_hermite16.restype = None
    lib.entmaxkv_gauss_hermite16.argtypes = [vp, vp]
    lib.entmaxkv_stream_read.restype = i32
    lib.entmaxkv_stream_read.argtypes = [vp, sz, vp, vp]
    lib.build_page_meta.restype = i32
    lib.build_page_meta.argtypes = [sh, vp, vp, vp, vp, vp, vp]
    lib.score_pages.restype = i32
    lib.score_pages.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.append_token.restype = i32
    lib.append_token.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, i32, vp]
    lib.build_page_meta_f8.restype = i32
    lib.build_page_meta_f8.argtypes = [sh, vp, vp, vp, vp, vp, vp]
    lib.score_pages_f8.restype = i32
    lib.score_pages_f8.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.select_pages_topk.restype = i32
    lib.select_pages_topk.argtypes = [sh, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.select_pages_gauss.restype = i32
    lib.select_pages_gauss.argtypes = [sh, vp, vp, vp, vp, dbl, dbl, dbl, vp, vp, vp, vp, vp, sz, vp]
    lib.select_pages_topk_group.restype = i32
    lib.select_pages_topk_group.argtypes = [sh, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.select_pages_gauss_group.restype = i32
    lib.select_pages_gauss_group.argtypes = [sh, vp, vp, vp, vp, dbl, dbl, dbl, vp, vp, vp, vp, vp, sz, vp]
    lib.entmax_decode_sparse_group.restype = i32
    lib.entmax_decode_sparse_group.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, dbl, i32, vp, vp, vp, vp, sz, vp]
    lib.entmax_decode_sparse.restype = i32
    lib.entmax_decode_sparse.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, dbl, i32, vp, vp, vp, vp, sz, vp]
    lib.softmax_decode_sparse.restype = i32
    lib.softmax_decode_sparse.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.entmax_decode_full.restype = i32
    lib.entmax_decode_full.argtypes = [sh, vp, vp, vp, vp, vp, dbl, i32, vp, vp, vp, vp, sz, vp]
    lib.softmax_decode_full.restype = i32
    lib.softmax_decode_full.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().entmaxkv_status_string(int(status)).decode()


def stream_read(src, sink, stream=None):
    """Measurement probe: read every byte of the device tensor src once with
    coalesced 16-byte loads (sink: a device int32/uint32 tensor of >= 1 element)."""
    st = load().entmaxkv_stream_read(_ptr(src, name="src"), src.numel() * src.element_size(),
                                     _ptr(sink, name="sink"), _stream(stream))
    _check("entmaxkv_stream_read", st)


def gauss_hermite16():
    """The library's 16-point Gauss-Hermite rule (nodes, weights for exp(-x^2))."""
    x = (ctypes.c_double * 16)()
    w = (ctypes.c_double * 16)()
    load().entmaxkv_gauss_hermite16(x, w)
    return list(x), list(w)


# ----------------------------------------------------------------- marshalling
def _torch():
    import torch
    return torch


def make_shape(q, k_pool, page_table, scale: float = 0.0) -> Shape:
    """Shape from q [B, Hq, d], k_pool [phys, Hkv, P, d], page_table [B, max_pages]."""
    torch = _torch()
    B, Hq, d = q.shape
    phys, Hkv, P, d2 = k_pool.shape
    if d2 != d or page_table.shape[0] != B:
        raise ValueError("inconsistent q / k_pool / page_table shapes")
    if q.dtype == torch.bfloat16:
        dt = BF16
    elif q.dtype == torch.float32:
        dt = F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    return Shape(B, Hq, Hkv, d, P, page_table.shape[1], phys, dt, float(scale))


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(shape: Shape, which_call: int) -> int:
    return int(load().entmaxkv_workspace_bytes(ctypes.byref(shape), int(which_call)))


def workspace(shape: Shape, which_call: int, device="cuda"):
    """A uint8 device tensor big enough for `which_call` (or None if none is needed)."""
    n = workspace_bytes(shape, which_call)
    if n == 0:
        return None
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def _ws(shape, which, ws):
    if ws is None:
        ws = workspace(shape, which)
    if ws is None:
        return None, 0, None
    return _ptr(ws, name="ws"), ws.numel() * ws.element_size(), ws


def _check(fn, st):
    if st != OK:
        raise EntmaxKVError(fn, st)


def _kv_dtype(shape: Shape):
    torch = _torch()
    return torch.bfloat16 if shape.dtype == BF16 else torch.float32


def build_page_meta(shape: Shape, k_pool, page_table, seq_lens, meta, from_token=None, stream=None):
    torch = _torch()
    kd = _kv_dtype(shape)
    st = load().build_page_meta(ctypes.byref(shape), _ptr(k_pool, kd, "k_pool"),
                                _ptr(page_table, torch.int32, "page_table"),
                                _ptr(seq_lens, torch.int32, "seq_lens"),
                                _ptr(from_token, torch.int32, "from_token"), _ptr(meta, kd, "meta"),
                                _stream(stream))
    _check("build_page_meta", st)
    return meta


def meta_f8_empty(shape: Shape):
    """A zeroed compact-metadata tensor: uint8 [num_phys, Hkv, 6d]."""
    torch = _torch()
    return torch.zeros((shape.num_phys_pages, shape.n_kv_heads, 6 * shape.head_dim), dtype=torch.uint8,
                       device="cuda")


def _meta_f8(shape: Shape, meta):
    torch = _torch()
    need = shape.num_phys_pages * shape.n_kv_heads * 6 * shape.head_dim
    if meta.numel() * meta.element_size() < need:
        raise ValueError(f"compact metadata needs {need} bytes")
    return _ptr(meta, torch.uint8, "meta")


def build_page_meta_f8(shape: Shape, k_pool, page_table, seq_lens, meta, from_token=None, stream=None):
    """Compact records: k_min / k_max bf16, mean / var OCP FP8 E4M3 (uint8 meta)."""
    torch = _torch()
    st = load().build_page_meta_f8(ctypes.byref(shape), _ptr(k_pool, _kv_dtype(shape), "k_pool"),
                                   _ptr(page_table, torch.int32, "page_table"),
                                   _ptr(seq_lens, torch.int32, "seq_lens"),
                                   _ptr(from_token, torch.int32, "from_token"), _meta_f8(shape, meta),
                                   _stream(stream))
    _check("build_page_meta_f8", st)
    return meta


def append_token(shape: Shape, k_new, v_new, k_pool, v_pool, page_table, seq_lens, meta, compact=False,
                 stream=None):
    """Write token seq_lens[b] - 1's K and V rows (k_new / v_new [B, Hkv, d]) into the pools and
    rebuild that page's metadata (compact records when compact=True)."""
    torch = _torch()
    kd = _kv_dtype(shape)
    st = load().append_token(ctypes.byref(shape), _ptr(k_new, kd, "k_new"), _ptr(v_new, kd, "v_new"),
                             _ptr(k_pool, kd, "k_pool"), _ptr(v_pool, kd, "v_pool"),
                             _ptr(page_table, torch.int32, "page_table"), _ptr(seq_lens, torch.int32, "seq_lens"),
                             _meta_f8(shape, meta) if compact else _ptr(meta, kd, "meta"), 1 if compact else 0,
                             _stream(stream))
    _check("append_token", st)
    return meta


def score_pages_f8(shape: Shape, q, meta, page_table, seq_lens, box, mu, var, ws=None, stream=None):
    torch = _torch()
    wp, wn, keep = _ws(shape, CALL_SCORE, ws)
    st = load().score_pages_f8(ctypes.byref(shape), _ptr(q, _kv_dtype(shape), "q"), _meta_f8(shape, meta),
                               _ptr(page_table, torch.int32, "page_table"),
                               _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(box, torch.float32, "box"),
                               _ptr(mu, torch.float32, "mu"), _ptr(var, torch.float32, "var"), wp, wn,
                               _stream(stream))
    _check("score_pages_f8", st)
    return box, mu, var


def score_pages(shape: Shape, q, meta, page_table, seq_lens, box, mu, var, ws=None, stream=None):
    torch = _torch()
    kd = _kv_dtype(shape)
    wp, wn, keep = _ws(shape, CALL_SCORE, ws)
    st = load().score_pages(ctypes.byref(shape), _ptr(q, kd, "q"), _ptr(meta, kd, "meta"),
                            _ptr(page_table, torch.int32, "page_table"),
                            _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(box, torch.float32, "box"),
                            _ptr(mu, torch.float32, "mu"), _ptr(var, torch.float32, "var"), wp, wn,
                            _stream(stream))
    _check("score_pages", st)
    return box, mu, var


def select_pages_topk(shape: Shape, box, seq_lens, k, sel_idx, sel_cnt, seq_mask=None, ws=None,
                      stream=None):
    torch = _torch()
    wp, wn, keep = _ws(shape, CALL_TOPK, ws)
    st = load().select_pages_topk(ctypes.byref(shape), _ptr(box, torch.float32, "box"),
                                  _ptr(seq_lens, torch.int32, "seq_lens"), int(k),
                                  _ptr(seq_mask, torch.uint8, "seq_mask"),
                                  _ptr(sel_idx, torch.int32, "sel_idx"),
                                  _ptr(sel_cnt, torch.int32, "sel_cnt"), wp, wn, _stream(stream))
    _check("select_pages_topk", st)
    return sel_idx, sel_cnt


def select_pages_gauss(shape: Shape, box, mu, var, seq_lens, alpha, delta, sel_idx, sel_cnt,
                       n_sigma=3.0, seq_mask=None, tau_hat=None, ws=None, stream=None):
    torch = _torch()
    wp, wn, keep = _ws(shape, CALL_GAUSS, ws)
    st = load().select_pages_gauss(ctypes.byref(shape), _ptr(box, torch.float32, "box"),
                                   _ptr(mu, torch.float32, "mu"), _ptr(var, torch.float32, "var"),
                                   _ptr(seq_lens, torch.int32, "seq_lens"), float(alpha), float(delta),
                                   float(n_sigma), _ptr(seq_mask, torch.uint8, "seq_mask"),
                                   _ptr(sel_idx, torch.int32, "sel_idx"),
                                   _ptr(sel_cnt, torch.int32, "sel_cnt"),
                                   _ptr(tau_hat, torch.float64, "tau_hat"), wp, wn, _stream(stream))
    _check("select_pages_gauss", st)
    return sel_idx, sel_cnt


def select_pages_topk_group(shape: Shape, box, seq_lens, k, sel_idx, sel_cnt, seq_mask=None, ws=None,
                            stream=None):
    """One set per KV head: sel_idx int32 [B, Hkv, max_pages], sel_cnt int32 [B, Hkv]."""
    torch = _torch()
    wp, wn, keep = _ws(shape, CALL_TOPK_GROUP, ws)
    st = load().select_pages_topk_group(ctypes.byref(shape), _ptr(box, torch.float32, "box"),
                                        _ptr(seq_lens, torch.int32, "seq_lens"), int(k),
                                        _ptr(seq_mask, torch.uint8, "seq_mask"),
                                        _ptr(sel_idx, torch.int32, "sel_idx"),
                                        _ptr(sel_cnt, torch.int32, "sel_cnt"), wp, wn, _stream(stream))
    _check("select_pages_topk_group", st)
    return sel_idx, sel_cnt


def select_pages_gauss_group(shape: Shape, box, mu, var, seq_lens, alpha, delta, sel_idx, sel_cnt,
                             n_sigma=3.0, seq_mask=None, tau_hat=None, ws=None, stream=None):
    """One set per KV head: the union of the group's per-head Gaussian sets."""
    torch = _torch()
    wp, wn, keep = _ws(shape, CALL_GAUSS_GROUP, ws)
    st = load().select_pages_gauss_group(ctypes.byref(shape), _ptr(box, torch.float32, "box"),
                                         _ptr(mu, torch.float32, "mu"), _ptr(var, torch.float32, "var"),
                                         _ptr(seq_lens, torch.int32, "seq_lens"), float(alpha), float(delta),
                                         float(n_sigma), _ptr(seq_mask, torch.uint8, "seq_mask"),
                                         _ptr(sel_idx, torch.int32, "sel_idx"),
                                         _ptr(sel_cnt, torch.int32, "sel_cnt"),
                                         _ptr(tau_hat, torch.float64, "tau_hat"), wp, wn, _stream(stream))
    _check("select_pages_gauss_group", st)
    return sel_idx, sel_cnt


def entmax_decode_sparse_group(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt,
                               alpha, out, tau=None, weights_out=None, tau_method=0, ws=None, stream=None):
    """entmax_decode_sparse with one kept set per KV head (sel_idx [B, Hkv, max_pages])."""
    torch = _torch()
    kd = _kv_dtype(shape)
    wp, wn, keep = _ws(shape, CALL_DECODE_GROUP, ws)
    st = load().entmax_decode_sparse_group(ctypes.byref(shape), _ptr(q, kd, "q"), _ptr(k_pool, kd, "k_pool"),
                                           _ptr(v_pool, kd, "v_pool"), _ptr(page_table, torch.int32, "page_table"),
                                           _ptr(seq_lens, torch.int32, "seq_lens"),
                                           _ptr(sel_idx, torch.int32, "sel_idx"),
                                           _ptr(sel_cnt, torch.int32, "sel_cnt"), float(alpha), int(tau_method),
                                           _ptr(out, torch.float32, "out"), _ptr(tau, torch.float64, "tau"),
                                           _ptr(weights_out, torch.float32, "weights_out"), wp, wn,
                                           _stream(stream))
    _check("entmax_decode_sparse_group", st)
    return out


def entmax_decode_sparse(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt,
                         alpha, out, tau=None, weights_out=None, tau_method=0, ws=None, stream=None):
    torch = _torch()
    kd = _kv_dtype(shape)
    wp, wn, keep = _ws(shape, CALL_DECODE_SPARSE, ws)
    st = load().entmax_decode_sparse(ctypes.byref(shape), _ptr(q, kd, "q"), _ptr(k_pool, kd, "k_pool"),
                                     _ptr(v_pool, kd, "v_pool"), _ptr(page_table, torch.int32, "page_table"),
                                     _ptr(seq_lens, torch.int32, "seq_lens"),
                                     _ptr(sel_idx, torch.int32, "sel_idx"),
                                     _ptr(sel_cnt, torch.int32, "sel_cnt"), float(alpha), int(tau_method),
                                     _ptr(out, torch.float32, "out"), _ptr(tau, torch.float64, "tau"),
                                     _ptr(weights_out, torch.float32, "weights_out"), wp, wn,
                                     _stream(stream))
    _check("entmax_decode_sparse", st)
    return out


def entmax_decode_full(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, alpha, out, tau=None,
                       weights_out=None, tau_method=0, ws=None, stream=None):
    torch = _torch()
    kd = _kv_dtype(shape)
    wp, wn, keep = _ws(shape, CALL_DECODE_FULL, ws)
    st = load().entmax_decode_full(ctypes.byref(shape), _ptr(q, kd, "q"), _ptr(k_pool, kd, "k_pool"),
                                   _ptr(v_pool, kd, "v_pool"), _ptr(page_table, torch.int32, "page_table"),
                                   _ptr(seq_lens, torch.int32, "seq_lens"), float(alpha), int(tau_method),
                                   _ptr(out, torch.float32, "out"), _ptr(tau, torch.float64, "tau"),
                                   _ptr(weights_out, torch.float32, "weights_out"), wp, wn,
                                   _stream(stream))
    _check("entmax_decode_full", st)
    return out


def softmax_decode_sparse(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out,
                          lse=None, ws=None, stream=None):
    """Softmax attention over the kept pages (the selection entmax_decode_sparse takes)."""
    torch = _torch()
    kd = _kv_dtype(shape)
    wp, wn, keep = _ws(shape, CALL_SOFTMAX_SPARSE, ws)
    st = load().softmax_decode_sparse(ctypes.byref(shape), _ptr(q, kd, "q"), _ptr(k_pool, kd, "k_pool"),
                                      _ptr(v_pool, kd, "v_pool"), _ptr(page_table, torch.int32, "page_table"),
                                      _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(sel_idx, torch.int32, "sel_idx"),
                                      _ptr(sel_cnt, torch.int32, "sel_cnt"), _ptr(out, torch.float32, "out"),
                                      _ptr(lse, torch.float32, "lse"), wp, wn, _stream(stream))
    _check("softmax_decode_sparse", st)
    return out


def softmax_decode_full(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, out, lse=None,
                        ws=None, stream=None):
    torch = _torch()
    kd = _kv_dtype(shape)
    wp, wn, keep = _ws(shape, CALL_SOFTMAX, ws)
    st = load().softmax_decode_full(ctypes.byref(shape), _ptr(q, kd, "q"), _ptr(k_pool, kd, "k_pool"),
                                    _ptr(v_pool, kd, "v_pool"), _ptr(page_table, torch.int32, "page_table"),
                                    _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(out, torch.float32, "out"),
                                    _ptr(lse, torch.float32, "lse"), wp, wn, _stream(stream))
    _check("softmax_decode_full", st)
    return out
