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
# another build of the library (the host-side sanitizer run) may be named by ENTMAXKV_LIB
LIB_PATH = os.environ.get("ENTMAXKV_LIB") or os.path.join(_HERE, "libentmaxkv.so")
_lib = None

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_TOO_LARGE = range(6)
F32, BF16 = 0, 1
(CALL_SCORE, CALL_TOPK, CALL_GAUSS, CALL_DECODE_SPARSE, CALL_DECODE_FULL, CALL_SOFTMAX, CALL_SOFTMAX_SPARSE,
 CALL_TOPK_GROUP, CALL_GAUSS_GROUP, CALL_DECODE_GROUP, CALL_SCORE_GAUSS) = range(1, 12)

EXPORTS = ("build_page_meta", "score_pages", "build_page_meta_f8", "score_pages_f8", "append_token",
           "select_pages_topk", "select_pages_gauss", "select_pages_topk_group", "select_pages_gauss_group",
           "entmax_decode_sparse_group",
           "entmax_decode_sparse", "entmax_decode_full", "softmax_decode_full", "softmax_decode_sparse",
           "entmaxkv_workspace_bytes", "entmaxkv_status_string", "entmaxkv_gauss_hermite16",
           "entmaxkv_stream_read", "score_pages_noalloc", "entmaxkv_score_scratch_bytes",
           "entmaxkv_decode_workspace_bytes", "score_select_pages_gauss")


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
    """Load libentmaxkv.so (raises if it has not been built).

    torch is imported first: its HIP runtime is then the one in the process and
    the library binds to it (both carry the soname libamdhip64.so.7).  Loaded
    the other way round, torch would bring a second HIP runtime and the
    library's launches would fail."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} not found: build it with `python -m sparse_decode_attention_page_amd.build`")
    import torch  # noqa: F401  (one HIP runtime per process: torch's)
    lib = ctypes.CDLL(p)
    vp, i32, sz, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
    sh = ctypes.POINTER(Shape)
    lib.entmaxkv_workspace_bytes.restype = sz
    lib.entmaxkv_workspace_bytes.argtypes = [sh, i32]
    lib.entmaxkv_decode_workspace_bytes.restype = sz
    lib.entmaxkv_decode_workspace_bytes.argtypes = [sh, i32, ctypes.c_int64]
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
    lib.score_pages_noalloc.restype = i32
    lib.score_pages_noalloc.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.entmaxkv_score_scratch_bytes.restype = sz
    lib.entmaxkv_score_scratch_bytes.argtypes = []
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
    lib.score_select_pages_gauss.restype = i32
    lib.score_select_pages_gauss.argtypes = [sh, vp, vp, vp, vp, vp, vp, vp, dbl, dbl, dbl, vp, vp, vp, vp, vp, sz,
                                             vp]
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


def _ptr(t, dtype=None, name="tensor", numel=None):
    """Device pointer of t after the checks the kernels rely on: at least `numel`
    elements (the extent the shape implies), on the device, contiguous, dtype."""
    if t is None:
        return None
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements; the shape needs {numel}")
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


def decode_workspace_bytes(shape: Shape, which_call: int, max_kept_pages: int) -> int:
    """Bytes of a decode workspace holding `max_kept_pages` kept pages summed
    over the query-head rows (which_call: CALL_DECODE_SPARSE, _GROUP, _FULL)."""
    return int(load().entmaxkv_decode_workspace_bytes(ctypes.byref(shape), int(which_call), int(max_kept_pages)))


def workspace(shape: Shape, which_call: int, device="cuda", max_kept_pages=None):
    """A uint8 device tensor big enough for `which_call` (or None if none is
    needed); for the decode calls, max_kept_pages bounds the kept pages summed
    over the query-head rows (None: every row's full set)."""
    if max_kept_pages is not None:
        n = decode_workspace_bytes(shape, which_call, max_kept_pages)
    else:
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


def _call(fn, shape: Shape, which, ws, args, stream):
    """Run a workspace-taking call: args are the already checked pointers and
    scalars between the shape and the workspace; the workspace is allocated only
    after every argument has passed its checks."""
    wp, wn, keep = _ws(shape, which, ws)
    st = getattr(load(), fn)(ctypes.byref(shape), *args, wp, wn, _stream(stream))
    _check(fn, st)


def _kv_dtype(shape: Shape):
    torch = _torch()
    return torch.bfloat16 if shape.dtype == BF16 else torch.float32


class _N:
    """Element counts of every buffer a call reads or writes, from the shape."""

    def __init__(self, s: Shape):
        B, Hq, Hkv, d, P, MP, NP = (s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.page_size, s.max_pages,
                                    s.num_phys_pages)
        self.q = self.out = B * Hq * d
        self.pool = NP * Hkv * P * d
        self.meta = NP * Hkv * 4 * d
        self.meta_f8 = NP * Hkv * 6 * d
        self.page_table = B * MP
        self.batch = B            # seq_lens, seq_mask, from_token
        self.rows = B * Hq        # sel_cnt, tau, tau_hat, lse
        self.per_page = B * Hq * MP   # box, mu, var, sel_idx
        self.grows = B * Hkv      # group sel_cnt
        self.gper_page = B * Hkv * MP  # group sel_idx
        self.weights = B * Hq * MP * P
        self.token_rows = B * Hkv * d  # k_new, v_new


def build_page_meta(shape: Shape, k_pool, page_table, seq_lens, meta, from_token=None, stream=None):
    torch = _torch()
    kd, n = _kv_dtype(shape), _N(shape)
    st = load().build_page_meta(ctypes.byref(shape), _ptr(k_pool, kd, "k_pool", n.pool),
                                _ptr(page_table, torch.int32, "page_table", n.page_table),
                                _ptr(seq_lens, torch.int32, "seq_lens", n.batch),
                                _ptr(from_token, torch.int32, "from_token", n.batch),
                                _ptr(meta, kd, "meta", n.meta), _stream(stream))
    _check("build_page_meta", st)
    return meta


def meta_f8_empty(shape: Shape):
    """A zeroed compact-metadata tensor: uint8 [num_phys, Hkv, 6d]."""
    torch = _torch()
    return torch.zeros((shape.num_phys_pages, shape.n_kv_heads, 6 * shape.head_dim), dtype=torch.uint8,
                       device="cuda")


def _meta_f8(shape: Shape, meta):
    return _ptr(meta, _torch().uint8, "meta", _N(shape).meta_f8)


def build_page_meta_f8(shape: Shape, k_pool, page_table, seq_lens, meta, from_token=None, stream=None):
    """Compact records: k_min / k_max bf16, mean / var OCP FP8 E4M3 (uint8 meta)."""
    torch = _torch()
    n = _N(shape)
    st = load().build_page_meta_f8(ctypes.byref(shape), _ptr(k_pool, _kv_dtype(shape), "k_pool", n.pool),
                                   _ptr(page_table, torch.int32, "page_table", n.page_table),
                                   _ptr(seq_lens, torch.int32, "seq_lens", n.batch),
                                   _ptr(from_token, torch.int32, "from_token", n.batch), _meta_f8(shape, meta),
                                   _stream(stream))
    _check("build_page_meta_f8", st)
    return meta


def append_token(shape: Shape, k_new, v_new, k_pool, v_pool, page_table, seq_lens, meta, compact=False,
                 stream=None):
    """Write token seq_lens[b] - 1's K and V rows (k_new / v_new [B, Hkv, d]) into the pools and
    rebuild that page's metadata (compact records when compact=True)."""
    torch = _torch()
    kd, n = _kv_dtype(shape), _N(shape)
    st = load().append_token(ctypes.byref(shape), _ptr(k_new, kd, "k_new", n.token_rows),
                             _ptr(v_new, kd, "v_new", n.token_rows), _ptr(k_pool, kd, "k_pool", n.pool),
                             _ptr(v_pool, kd, "v_pool", n.pool), _ptr(page_table, torch.int32, "page_table", n.page_table),
                             _ptr(seq_lens, torch.int32, "seq_lens", n.batch),
                             _meta_f8(shape, meta) if compact else _ptr(meta, kd, "meta", n.meta), 1 if compact else 0,
                             _stream(stream))
    _check("append_token", st)
    return meta


def _score_args(shape: Shape, q, page_table, seq_lens, box, mu, var):
    torch = _torch()
    n = _N(shape)
    return (_ptr(q, _kv_dtype(shape), "q", n.q), _ptr(page_table, torch.int32, "page_table", n.page_table),
            _ptr(seq_lens, torch.int32, "seq_lens", n.batch), _ptr(box, torch.float32, "box", n.per_page),
            _ptr(mu, torch.float32, "mu", n.per_page), _ptr(var, torch.float32, "var", n.per_page))


def score_pages_f8(shape: Shape, q, meta, page_table, seq_lens, box, mu, var, ws=None, stream=None):
    qp, pt, sl, bp, mp, vp = _score_args(shape, q, page_table, seq_lens, box, mu, var)
    _call("score_pages_f8", shape, CALL_SCORE, ws, (qp, _meta_f8(shape, meta), pt, sl, bp, mp, vp), stream)
    return box, mu, var


def score_pages(shape: Shape, q, meta, page_table, seq_lens, box, mu, var, ws=None, stream=None):
    qp, pt, sl, bp, mp, vp = _score_args(shape, q, page_table, seq_lens, box, mu, var)
    mt = _ptr(meta, _kv_dtype(shape), "meta", _N(shape).meta)
    _call("score_pages", shape, CALL_SCORE, ws, (qp, mt, pt, sl, bp, mp, vp), stream)
    return box, mu, var


def score_pages_noalloc(shape: Shape, q, meta, page_table, seq_lens, box, mu, var, stream=None):
    """score_pages without a workspace: the library's static device scratch holds
    the coefficient table (calls that overlap on one GPU race)."""
    qp, pt, sl, bp, mp, vp = _score_args(shape, q, page_table, seq_lens, box, mu, var)
    mt = _ptr(meta, _kv_dtype(shape), "meta", _N(shape).meta)
    _check("score_pages_noalloc", load().score_pages_noalloc(ctypes.byref(shape), qp, mt, pt, sl, bp, mp, vp,
                                                             _stream(stream)))
    return box, mu, var


def score_scratch_bytes() -> int:
    return int(load().entmaxkv_score_scratch_bytes())


def _sel_args(shape: Shape, sel_idx, sel_cnt, group=False):
    torch = _torch()
    n = _N(shape)
    return (_ptr(sel_idx, torch.int32, "sel_idx", n.gper_page if group else n.per_page),
            _ptr(sel_cnt, torch.int32, "sel_cnt", n.grows if group else n.rows))


def _gauss_args(shape: Shape, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask):
    torch = _torch()
    n = _N(shape)
    return (_ptr(box, torch.float32, "box", n.per_page), _ptr(mu, torch.float32, "mu", n.per_page),
            _ptr(var, torch.float32, "var", n.per_page), _ptr(seq_lens, torch.int32, "seq_lens", n.batch),
            float(alpha), float(delta), float(n_sigma), _ptr(seq_mask, torch.uint8, "seq_mask", n.batch))


def _topk_args(shape: Shape, box, seq_lens, k, seq_mask):
    torch = _torch()
    n = _N(shape)
    return (_ptr(box, torch.float32, "box", n.per_page), _ptr(seq_lens, torch.int32, "seq_lens", n.batch), int(k),
            _ptr(seq_mask, torch.uint8, "seq_mask", n.batch))


def select_pages_topk(shape: Shape, box, seq_lens, k, sel_idx, sel_cnt, seq_mask=None, ws=None,
                      stream=None):
    args = (*_topk_args(shape, box, seq_lens, k, seq_mask), *_sel_args(shape, sel_idx, sel_cnt))
    _call("select_pages_topk", shape, CALL_TOPK, ws, args, stream)
    return sel_idx, sel_cnt


def select_pages_gauss(shape: Shape, box, mu, var, seq_lens, alpha, delta, sel_idx, sel_cnt,
                       n_sigma=3.0, seq_mask=None, tau_hat=None, ws=None, stream=None):
    args = (*_gauss_args(shape, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask),
            *_sel_args(shape, sel_idx, sel_cnt), _ptr(tau_hat, _torch().float64, "tau_hat", _N(shape).rows))
    _call("select_pages_gauss", shape, CALL_GAUSS, ws, args, stream)
    return sel_idx, sel_cnt


def score_select_pages_gauss(shape: Shape, q, meta, page_table, seq_lens, box, mu, var, alpha, delta,
                             sel_idx, sel_cnt, n_sigma=3.0, seq_mask=None, tau_hat=None, ws=None, stream=None):
    """score_pages then select_pages_gauss in one call (the selector's bracket
    comes from the scoring launch); the same outputs as the two calls in turn."""
    torch = _torch()
    n = _N(shape)
    qp, pt, sl, bp, mp, vp = _score_args(shape, q, page_table, seq_lens, box, mu, var)
    mt = _ptr(meta, _kv_dtype(shape), "meta", n.meta)
    args = (qp, mt, pt, sl, bp, mp, vp, float(alpha), float(delta), float(n_sigma),
            _ptr(seq_mask, torch.uint8, "seq_mask", n.batch), *_sel_args(shape, sel_idx, sel_cnt),
            _ptr(tau_hat, torch.float64, "tau_hat", n.rows))
    _call("score_select_pages_gauss", shape, CALL_SCORE_GAUSS, ws, args, stream)
    return box, mu, var, sel_idx, sel_cnt


def select_pages_topk_group(shape: Shape, box, seq_lens, k, sel_idx, sel_cnt, seq_mask=None, ws=None,
                            stream=None):
    """One set per KV head: sel_idx int32 [B, Hkv, max_pages], sel_cnt int32 [B, Hkv]."""
    args = (*_topk_args(shape, box, seq_lens, k, seq_mask), *_sel_args(shape, sel_idx, sel_cnt, group=True))
    _call("select_pages_topk_group", shape, CALL_TOPK_GROUP, ws, args, stream)
    return sel_idx, sel_cnt


def select_pages_gauss_group(shape: Shape, box, mu, var, seq_lens, alpha, delta, sel_idx, sel_cnt,
                             n_sigma=3.0, seq_mask=None, tau_hat=None, ws=None, stream=None):
    """One set per KV head: the union of the group's per-head Gaussian sets."""
    args = (*_gauss_args(shape, box, mu, var, seq_lens, alpha, delta, n_sigma, seq_mask),
            *_sel_args(shape, sel_idx, sel_cnt, group=True),
            _ptr(tau_hat, _torch().float64, "tau_hat", _N(shape).rows))
    _call("select_pages_gauss_group", shape, CALL_GAUSS_GROUP, ws, args, stream)
    return sel_idx, sel_cnt


def _decode_args(shape: Shape, q, k_pool, v_pool, page_table, seq_lens):
    torch = _torch()
    kd, n = _kv_dtype(shape), _N(shape)
    return (_ptr(q, kd, "q", n.q), _ptr(k_pool, kd, "k_pool", n.pool), _ptr(v_pool, kd, "v_pool", n.pool),
            _ptr(page_table, torch.int32, "page_table", n.page_table), _ptr(seq_lens, torch.int32, "seq_lens", n.batch))


def _out_args(shape: Shape, out, tau, weights_out):
    torch = _torch()
    n = _N(shape)
    return (_ptr(out, torch.float32, "out", n.out), _ptr(tau, torch.float64, "tau", n.rows),
            _ptr(weights_out, torch.float32, "weights_out", n.weights))


def entmax_decode_sparse_group(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt,
                               alpha, out, tau=None, weights_out=None, tau_method=0, ws=None, stream=None):
    """entmax_decode_sparse with one kept set per KV head (sel_idx [B, Hkv, max_pages])."""
    args = (*_decode_args(shape, q, k_pool, v_pool, page_table, seq_lens),
            *_sel_args(shape, sel_idx, sel_cnt, group=True), float(alpha), int(tau_method),
            *_out_args(shape, out, tau, weights_out))
    _call("entmax_decode_sparse_group", shape, CALL_DECODE_GROUP, ws, args, stream)
    return out


def entmax_decode_sparse(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt,
                         alpha, out, tau=None, weights_out=None, tau_method=0, ws=None, stream=None):
    args = (*_decode_args(shape, q, k_pool, v_pool, page_table, seq_lens), *_sel_args(shape, sel_idx, sel_cnt),
            float(alpha), int(tau_method), *_out_args(shape, out, tau, weights_out))
    _call("entmax_decode_sparse", shape, CALL_DECODE_SPARSE, ws, args, stream)
    return out


def entmax_decode_full(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, alpha, out, tau=None,
                       weights_out=None, tau_method=0, ws=None, stream=None):
    args = (*_decode_args(shape, q, k_pool, v_pool, page_table, seq_lens), float(alpha), int(tau_method),
            *_out_args(shape, out, tau, weights_out))
    _call("entmax_decode_full", shape, CALL_DECODE_FULL, ws, args, stream)
    return out


def softmax_decode_sparse(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, sel_idx, sel_cnt, out,
                          lse=None, ws=None, stream=None):
    """Softmax attention over the kept pages (the selection entmax_decode_sparse takes)."""
    torch = _torch()
    n = _N(shape)
    args = (*_decode_args(shape, q, k_pool, v_pool, page_table, seq_lens), *_sel_args(shape, sel_idx, sel_cnt),
            _ptr(out, torch.float32, "out", n.out), _ptr(lse, torch.float32, "lse", n.rows))
    _call("softmax_decode_sparse", shape, CALL_SOFTMAX_SPARSE, ws, args, stream)
    return out


def softmax_decode_full(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, out, lse=None,
                        ws=None, stream=None):
    torch = _torch()
    n = _N(shape)
    args = (*_decode_args(shape, q, k_pool, v_pool, page_table, seq_lens), _ptr(out, torch.float32, "out", n.out),
            _ptr(lse, torch.float32, "lse", n.rows))
    _call("softmax_decode_full", shape, CALL_SOFTMAX, ws, args, stream)
    return out
