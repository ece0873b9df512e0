"""CPU checks of the C-ABI library: it loads without a GPU, exports every
function include/entmaxkv.h declares, rejects bad arguments with the documented
status before launching anything, and sizes workspaces."""
import ctypes
import os
import re

import numpy as np
import pytest

import sparse_decode_attention_page_amd as E

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "entmaxkv.h")

FAKE = ctypes.c_void_p(256)  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_hot_path():
    names = declared_functions()
    for n in ("build_page_meta", "score_pages", "select_pages_topk", "select_pages_gauss",
              "entmax_decode_sparse", "entmax_decode_full", "softmax_decode_full"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = E.load()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert missing == []
    assert set(declared_functions()) <= set(E.EXPORTS)


def shape(**kw):
    base = dict(batch=1, n_q_heads=32, n_kv_heads=8, head_dim=64, page_size=64, max_pages=16384,
                num_phys_pages=16384, dtype=E.BF16, scale=0.0)
    base.update(kw)
    return E.Shape(**base)


@pytest.mark.parametrize("bad,status", [
    (dict(n_kv_heads=7), E.ERR_INVALID_ARGUMENT),      # Hq % Hkv
    (dict(batch=0), E.ERR_INVALID_ARGUMENT),
    (dict(max_pages=0), E.ERR_INVALID_ARGUMENT),
    (dict(dtype=5), E.ERR_INVALID_ARGUMENT),
    (dict(scale=-1.0), E.ERR_INVALID_ARGUMENT),
    (dict(head_dim=96), E.ERR_UNSUPPORTED),
    (dict(page_size=8), E.ERR_UNSUPPORTED),
    (dict(n_q_heads=48, n_kv_heads=3), E.ERR_UNSUPPORTED),  # group of 16
])
def test_bad_shapes(bad, status):
    lib = E.load()
    s = shape(**bad)
    assert lib.score_pages(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == status
    assert lib.softmax_decode_full(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == status
    assert E.workspace_bytes(s, E.CALL_GAUSS) == 0


def test_bad_arguments():
    lib = E.load()
    s = ctypes.byref(shape())
    big = 1 << 40
    # null required pointers
    assert lib.score_pages(s, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None) == E.ERR_INVALID_ARGUMENT
    assert lib.build_page_meta(s, FAKE, FAKE, FAKE, None, None, None) == E.ERR_INVALID_ARGUMENT
    # k <= 0
    assert lib.select_pages_topk(s, FAKE, FAKE, 0, None, FAKE, FAKE, None, 0, None) == E.ERR_INVALID_ARGUMENT
    # alpha <= 1, negative delta / n_sigma
    for a, dl, ns in ((1.0, 0.5, 3.0), (0.5, 0.5, 3.0), (1.5, -0.1, 3.0), (1.5, 0.5, -1.0),
                      (float("nan"), 0.5, 3.0)):
        assert lib.select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, a, dl, ns, None, FAKE, FAKE, None, FAKE,
                                      big, None) == E.ERR_INVALID_ARGUMENT
    assert lib.entmax_decode_sparse(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 0, FAKE, None, None,
                                    FAKE, big, None) == E.ERR_INVALID_ARGUMENT
    # sort closed form only for alpha == 2; unknown tau method
    assert lib.entmax_decode_full(s, FAKE, FAKE, FAKE, FAKE, FAKE, 1.5, 1, FAKE, None, None, FAKE, big,
                                  None) == E.ERR_INVALID_ARGUMENT
    assert lib.entmax_decode_full(s, FAKE, FAKE, FAKE, FAKE, FAKE, 2.0, 7, FAKE, None, None, FAKE, big,
                                  None) == E.ERR_INVALID_ARGUMENT
    # the fused score + Gaussian selection checks both steps' arguments
    assert lib.score_select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.0, 0.5, 3.0, None, FAKE, FAKE,
                                        None, FAKE, big, None) == E.ERR_INVALID_ARGUMENT
    assert lib.score_select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.5, 0.5, 3.0, None, None, FAKE,
                                        None, FAKE, big, None) == E.ERR_INVALID_ARGUMENT
    # sparse decode needs a selection
    assert lib.entmax_decode_sparse(s, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1.5, 0, FAKE, None, None,
                                    FAKE, big, None) == E.ERR_INVALID_ARGUMENT


def test_noalloc_rejects_shapes_beyond_its_scratch():
    """score_pages_noalloc checks its static scratch before launching anything."""
    lib = E.load()
    cap = E.score_scratch_bytes()
    assert cap == 4 << 20
    big = shape(batch=64, head_dim=128)  # 32 B * 64 * 32 * 128 = 8 MiB of coefficients
    assert lib.score_pages_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == \
        E.ERR_TOO_LARGE
    assert "scratch" in E.status_string(E.ERR_TOO_LARGE)
    s = ctypes.byref(shape())
    assert lib.score_pages_noalloc(s, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.ERR_INVALID_ARGUMENT


def test_workspace_too_small_or_misaligned():
    lib = E.load()
    sh = shape()
    s = ctypes.byref(sh)
    need = E.workspace_bytes(sh, E.CALL_GAUSS)
    assert need > 0
    assert lib.select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, 1.5, 0.5, 3.0, None, FAKE, FAKE, None, FAKE,
                                  need - 1, None) == E.ERR_WORKSPACE
    assert lib.select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, 1.5, 0.5, 3.0, None, FAKE, FAKE, None, None,
                                  need, None) == E.ERR_WORKSPACE
    assert lib.select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, 1.5, 0.5, 3.0, None, FAKE, FAKE, None,
                                  ctypes.c_void_p(264), need, None) == E.ERR_INVALID_ARGUMENT
    fused = E.workspace_bytes(sh, E.CALL_SCORE_GAUSS)
    assert fused >= need + E.workspace_bytes(sh, E.CALL_SCORE)
    assert lib.score_select_pages_gauss(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1.5, 0.5, 3.0, None, FAKE, FAKE,
                                        None, FAKE, fused - 1, None) == E.ERR_WORKSPACE
    for call in (E.CALL_SCORE, E.CALL_DECODE_SPARSE, E.CALL_DECODE_FULL, E.CALL_SOFTMAX):
        assert E.workspace_bytes(sh, call) > 0
    assert E.workspace_bytes(sh, 99) == 0
    assert "workspace" in E.status_string(E.ERR_WORKSPACE)


def test_library_gauss_hermite_rule():
    x, w = E.gauss_hermite16()
    xn, wn = np.polynomial.hermite.hermgauss(16)
    assert np.max(np.abs(np.array(x) - xn)) < 1e-13
    assert np.max(np.abs(np.array(w) - wn) / wn) < 1e-11
    assert abs(sum(w) - np.sqrt(np.pi)) < 1e-14
