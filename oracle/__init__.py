"""Plain fp64 CPU oracle for the EntmaxKV decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The product path (``sparse_decode_attention_page_amd``)
never imports it, and the two share no code.

The C source (``oracle.c``) follows "Resumen Tecnico: EntmaxKV - Decodificacion
Consciente del Soporte para Atencion Entmax" (gist.science/es/paper/2605.21649),
sections 2.A-2.C and 3; each C function cites the passage it implements.

Arrays are numpy.  KV-dtype tensors are passed as their raw storage: ``float32``
arrays for fp32 data, ``uint16`` arrays holding bfloat16 bit patterns for bf16.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_OVERRIDE = os.environ.get("ENTMAXKV_ORACLE_LIB")  # another build of oracle.c (the sanitizer run)
_lib = None
_FLAGS = ["-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared"]


def build() -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, no FMA contraction)."""
    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-O2", *_FLAGS, "-o", _SO + ".tmp", src, "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def build_sanitized(out: str) -> str:
    """Compile oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer
    (any report aborts) into `out`; load it with ENTMAXKV_ORACLE_LIB=out in a
    process started with gcc's libasan preloaded."""
    src = os.path.join(_HERE, "oracle.c")
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", *_FLAGS, "-o", out, src, "-lm"]
    subprocess.check_call(cmd)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    src = os.path.join(_HERE, "oracle.c")
    if _OVERRIDE:
        so = _OVERRIDE
    else:
        so = _SO
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
            build()
    lib = ctypes.CDLL(so)
    _lib = lib
    vp = ctypes.c_void_p
    lib.orc_round_bf16.restype = ctypes.c_double
    lib.orc_round_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_f32.restype = ctypes.c_double
    lib.orc_round_f32.argtypes = [ctypes.c_double]
    lib.orc_round_f32_up.restype = ctypes.c_double
    lib.orc_round_f32_up.argtypes = [ctypes.c_double]
    lib.orc_gauss_hermite16.argtypes = [vp, vp]
    lib.orc_build_page_meta.argtypes = [vp] * 6
    lib.orc_build_page_meta_f8.argtypes = [vp] * 6
    lib.orc_score_pages.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp]
    lib.orc_score_pages_f8.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_select_topk.argtypes = [vp, vp, vp, ctypes.c_int32, vp, vp, ctypes.c_int32, vp, vp]
    lib.orc_select_gauss.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, ctypes.c_double,
                                     ctypes.c_double, vp, vp, ctypes.c_int32, vp, vp, vp]
    lib.orc_select_topk_group.argtypes = [vp, vp, vp, ctypes.c_int32, vp, vp, ctypes.c_int32, vp, vp]
    lib.orc_select_gauss_group.argtypes = [vp, vp, vp, vp, vp, ctypes.c_double, ctypes.c_double,
                                           ctypes.c_double, vp, vp, ctypes.c_int32, vp, vp, vp]
    lib.orc_entmax_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_double, vp,
                                      ctypes.c_int32, vp, vp, vp]
    lib.orc_softmax_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp, vp]
    lib.orc_gauss_mass.restype = ctypes.c_double
    lib.orc_gauss_mass.argtypes = [vp, vp, vp, ctypes.c_int32, ctypes.c_double, ctypes.c_double]
    lib.orc_entmax_tau.restype = ctypes.c_double
    lib.orc_entmax_tau.argtypes = [vp, ctypes.c_int64, ctypes.c_double]
    return lib


class _Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("P", ctypes.c_int32), ("max_pages", ctypes.c_int32),
                ("num_phys", ctypes.c_int32), ("dtype", ctypes.c_int32), ("scale", ctypes.c_double)]


@dataclass
class Shape:
    B: int
    Hq: int
    Hkv: int
    d: int
    P: int
    max_pages: int
    num_phys: int
    dtype: str  # "f32" or "bf16"
    scale: float = 0.0

    def c(self) -> _Shape:
        return _Shape(self.B, self.Hq, self.Hkv, self.d, self.P, self.max_pages, self.num_phys,
                      0 if self.dtype == "f32" else 1, self.scale)


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _raw(a, shape: Shape):
    want = np.float32 if shape.dtype == "f32" else np.uint16
    assert a.dtype == want, f"expected {want} storage, got {a.dtype}"
    return np.ascontiguousarray(a)


def _rows(rows):
    if rows is None:
        return None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    return r, len(r)


def round_bf16(x: float) -> float:
    return _load().orc_round_bf16(float(x))


def round_f32(x: float) -> float:
    return _load().orc_round_f32(float(x))


def round_f32_up(x: float) -> float:
    return _load().orc_round_f32_up(float(x))


def e4m3_decode(code: int) -> float:
    """Value of an OCP FP8 E4M3 code (0..255)."""
    return _load().orc_e4m3_decode(int(code) & 0xFF)


def e4m3_encode(x: float) -> int:
    """Nearest E4M3 code (ties to even, saturating at +-448, NaN -> 0x7F)."""
    return int(_load().orc_e4m3_encode(float(x)))


def gauss_hermite16():
    x = np.zeros(16)
    w = np.zeros(16)
    _load().orc_gauss_hermite16(_p(x), _p(w))
    return x, w


def build_page_meta(shape: Shape, k_pool, page_table, seq_lens, from_token=None, meta=None):
    lib = _load()
    k_pool = _raw(k_pool, shape)
    if meta is None:
        meta = np.zeros((shape.num_phys, shape.Hkv, 4, shape.d), dtype=k_pool.dtype)
    meta = np.ascontiguousarray(meta)
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ft = None if from_token is None else np.ascontiguousarray(from_token, dtype=np.int32)
    sh = shape.c()
    lib.orc_build_page_meta(ctypes.byref(sh), _p(k_pool), _p(pt), _p(sl), _p(ft), _p(meta))
    return meta


def build_page_meta_f8(shape: Shape, k_pool, page_table, seq_lens, from_token=None, meta=None):
    """Compact records (bf16 keys): uint8 [num_phys][Hkv][6d] holding k_min and
    k_max as bf16 and the mean and variance as E4M3."""
    assert shape.dtype == "bf16", "compact metadata is defined for bf16 keys"
    lib = _load()
    k_pool = _raw(k_pool, shape)
    if meta is None:
        meta = np.zeros((shape.num_phys, shape.Hkv, 6 * shape.d), dtype=np.uint8)
    meta = np.ascontiguousarray(meta)
    assert meta.dtype == np.uint8 and meta.nbytes == shape.num_phys * shape.Hkv * 6 * shape.d
    pt = np.ascontiguousarray(page_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    ft = None if from_token is None else np.ascontiguousarray(from_token, dtype=np.int32)
    sh = shape.c()
    lib.orc_build_page_meta_f8(ctypes.byref(sh), _p(k_pool), _p(pt), _p(sl), _p(ft), _p(meta))
    return meta


def score_pages_f8(shape: Shape, q, meta, page_table, seq_lens, rows=None):
    """score_pages over compact records."""
    lib = _load()
    n = shape.B * shape.Hq * shape.max_pages
    box = np.full(n, np.nan, np.float32)
    mu = np.full(n, np.nan, np.float32)
    var = np.full(n, np.nan, np.float32)
    r, nr = _rows(rows)
    m = np.ascontiguousarray(meta)
    assert m.dtype == np.uint8
    sh = shape.c()
    lib.orc_score_pages_f8(ctypes.byref(sh), _p(_raw(q, shape)), _p(m),
                           _p(np.ascontiguousarray(page_table, dtype=np.int32)),
                           _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), _p(r), nr,
                           _p(box), _p(mu), _p(var))
    s3 = (shape.B, shape.Hq, shape.max_pages)
    return box.reshape(s3), mu.reshape(s3), var.reshape(s3)


def score_pages(shape: Shape, q, meta, page_table, seq_lens, rows=None):
    lib = _load()
    n = shape.B * shape.Hq * shape.max_pages
    box = np.full(n, np.nan, np.float32)
    mu = np.full(n, np.nan, np.float32)
    var = np.full(n, np.nan, np.float32)
    r, nr = _rows(rows)
    sh = shape.c()
    lib.orc_score_pages(ctypes.byref(sh), _p(_raw(q, shape)), _p(_raw(meta, shape)),
                        _p(np.ascontiguousarray(page_table, dtype=np.int32)),
                        _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), _p(r), nr,
                        _p(box), _p(mu), _p(var))
    s3 = (shape.B, shape.Hq, shape.max_pages)
    return box.reshape(s3), mu.reshape(s3), var.reshape(s3)


def select_topk(shape: Shape, box, seq_lens, k, seq_mask=None, rows=None):
    lib = _load()
    sel = np.full((shape.B, shape.Hq, shape.max_pages), -1, np.int32)
    cnt = np.full((shape.B, shape.Hq), -1, np.int32)
    r, nr = _rows(rows)
    m = None if seq_mask is None else np.ascontiguousarray(seq_mask, dtype=np.uint8)
    sh = shape.c()
    lib.orc_select_topk(ctypes.byref(sh), _p(np.ascontiguousarray(box, dtype=np.float32)),
                        _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), int(k), _p(m), _p(r), nr,
                        _p(sel), _p(cnt))
    return sel, cnt


def select_gauss(shape: Shape, box, mu, var, seq_lens, alpha, delta, n_sigma=3.0, seq_mask=None,
                 rows=None):
    lib = _load()
    sel = np.full((shape.B, shape.Hq, shape.max_pages), -1, np.int32)
    cnt = np.full((shape.B, shape.Hq), -1, np.int32)
    tau = np.full((shape.B, shape.Hq), np.nan)
    r, nr = _rows(rows)
    m = None if seq_mask is None else np.ascontiguousarray(seq_mask, dtype=np.uint8)
    sh = shape.c()
    box_c, mu_c, var_c = (np.ascontiguousarray(a, dtype=np.float32) for a in (box, mu, var))
    lib.orc_select_gauss(ctypes.byref(sh), _p(box_c), _p(mu_c), _p(var_c),
                         _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), float(alpha),
                         float(delta), float(n_sigma), _p(m), _p(r), nr, _p(sel), _p(cnt), _p(tau))
    return sel, cnt, tau


def select_topk_group(shape: Shape, box, seq_lens, k, seq_mask=None, rows=None):
    """One set per KV head: top-k of the largest box over the group's heads.
    rows: group rows b*Hkv+g.  Returns sel [B][Hkv][max_pages], cnt [B][Hkv]."""
    lib = _load()
    sel = np.full((shape.B, shape.Hkv, shape.max_pages), -1, np.int32)
    cnt = np.full((shape.B, shape.Hkv), -1, np.int32)
    r, nr = _rows(rows)
    m = None if seq_mask is None else np.ascontiguousarray(seq_mask, dtype=np.uint8)
    sh = shape.c()
    lib.orc_select_topk_group(ctypes.byref(sh), _p(np.ascontiguousarray(box, dtype=np.float32)),
                              _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), int(k), _p(m), _p(r), nr,
                              _p(sel), _p(cnt))
    return sel, cnt


def select_gauss_group(shape: Shape, box, mu, var, seq_lens, alpha, delta, n_sigma=3.0, seq_mask=None,
                       rows=None):
    """One set per KV head: the union of the group's per-head Gaussian sets.
    Returns sel [B][Hkv][max_pages], cnt [B][Hkv], tau_hat [B][Hq]."""
    lib = _load()
    sel = np.full((shape.B, shape.Hkv, shape.max_pages), -1, np.int32)
    cnt = np.full((shape.B, shape.Hkv), -1, np.int32)
    tau = np.full((shape.B, shape.Hq), np.nan)
    r, nr = _rows(rows)
    m = None if seq_mask is None else np.ascontiguousarray(seq_mask, dtype=np.uint8)
    sh = shape.c()
    box_c, mu_c, var_c = (np.ascontiguousarray(a, dtype=np.float32) for a in (box, mu, var))
    lib.orc_select_gauss_group(ctypes.byref(sh), _p(box_c), _p(mu_c), _p(var_c),
                               _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), float(alpha),
                               float(delta), float(n_sigma), _p(m), _p(r), nr, _p(sel), _p(cnt), _p(tau))
    return sel, cnt, tau


def expand_group_selection(shape: Shape, sel_g, cnt_g):
    """Per-query-head copies of a group selection (head h reads group h // G)."""
    G = shape.Hq // shape.Hkv
    return (np.ascontiguousarray(np.repeat(np.asarray(sel_g), G, axis=1)),
            np.ascontiguousarray(np.repeat(np.asarray(cnt_g), G, axis=1)))


def entmax_decode(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, alpha, sel_idx=None,
                  sel_cnt=None, rows=None, want_weights=False):
    """Sparse decode over (sel_idx, sel_cnt); full-cache decode when sel_idx is None."""
    lib = _load()
    out = np.full((shape.B, shape.Hq, shape.d), np.nan)
    tau = np.full((shape.B, shape.Hq), np.nan)
    w = np.zeros((shape.B, shape.Hq, shape.max_pages * shape.P)) if want_weights else None
    r, nr = _rows(rows)
    si = None if sel_idx is None else np.ascontiguousarray(sel_idx, dtype=np.int32)
    sc = None if sel_cnt is None else np.ascontiguousarray(sel_cnt, dtype=np.int32)
    sh = shape.c()
    lib.orc_entmax_decode(ctypes.byref(sh), _p(_raw(q, shape)), _p(_raw(k_pool, shape)),
                          _p(_raw(v_pool, shape)), _p(np.ascontiguousarray(page_table, dtype=np.int32)),
                          _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), _p(si), _p(sc),
                          float(alpha), _p(r), nr, _p(out), _p(tau), _p(w))
    return out, tau, w


def softmax_decode(shape: Shape, q, k_pool, v_pool, page_table, seq_lens, rows=None, sel_idx=None,
                   sel_cnt=None):
    """Softmax attention over every cached token, or over the kept pages when a
    selection (sel_idx [B][Hq][max_pages], sel_cnt [B][Hq]) is given."""
    lib = _load()
    out = np.full((shape.B, shape.Hq, shape.d), np.nan)
    lse = np.full((shape.B, shape.Hq), np.nan)
    r, nr = _rows(rows)
    si = None if sel_idx is None else np.ascontiguousarray(sel_idx, dtype=np.int32)
    sc = None if sel_cnt is None else np.ascontiguousarray(sel_cnt, dtype=np.int32)
    sh = shape.c()
    lib.orc_softmax_decode(ctypes.byref(sh), _p(_raw(q, shape)), _p(_raw(k_pool, shape)),
                           _p(_raw(v_pool, shape)), _p(np.ascontiguousarray(page_table, dtype=np.int32)),
                           _p(np.ascontiguousarray(seq_lens, dtype=np.int32)), _p(si), _p(sc), _p(r), nr,
                           _p(out), _p(lse))
    return out, lse


def entmax_tau(scores, alpha) -> float:
    """alpha-entmax threshold (score units) of a 1-D score vector, by bisection."""
    s = np.ascontiguousarray(scores, dtype=np.float64)
    return _load().orc_entmax_tau(_p(s), len(s), float(alpha))


def gauss_mass(mu, var, n, alpha, tau) -> float:
    """F(tau) of the Gaussian selector for explicit pages (mu, var float32; n fill counts)."""
    mu = np.ascontiguousarray(mu, dtype=np.float32)
    var = np.ascontiguousarray(var, dtype=np.float32)
    n = np.ascontiguousarray(n, dtype=np.int32)
    return _load().orc_gauss_mass(_p(mu), _p(var), _p(n), len(mu), float(alpha), float(tau))
