"""GPU parity of the entmax decodes on long selections.

Rows here keep many tokens, and with a small score scale many candidates.
Two batch shapes: 8 query-head rows (a set per query head goes to the
per-item decode: chunk blocks, merge, register or workspace solve) and 68
rows (the slice decode: lone blocks over rounds of entries, chunked rows
merged by their last block, and above 32768 entries the helper steps --
histogram window, moments and window solve, split gather -- or for a generic
alpha passes over the workspace).  Same bars as the small cases: thresholds
to 1e-12, bit-exact supports, weights to 1e-5, outputs to the KV-dtype
tolerance; a repeated call gives the same bits.
"""
import numpy as np
import pytest

import sparse_decode_attention_page_amd as E
from gpu_util import Dev, decode_check
from sparse_decode_attention_page_amd import synth

pytestmark = pytest.mark.gpu

# score scales: default 1/sqrt(d) (few candidates), 0.08 (candidates that
# still fit LDS), 0.02 and 0.01 (alpha = 1.5: 1k-4k candidates per row, solved
# from registers, and some rows beyond), 0.002 (every token a candidate and in
# the support: solved over the workspace)
SCALES = [0.0, 0.08, 0.02, 0.01, 0.002]


# (batch, contexts): 8 rows, and 68 rows (past the per-item decode's row limit)
SHAPES = [(2, (20000, 9001)), (17, (20000, 9001) * 8 + (4000,))]


@pytest.fixture(scope="module", params=[(s, b) for b in range(len(SHAPES)) for s in SCALES],
                ids=lambda p: f"rows{SHAPES[p[1]][0] * 4}_scale{p[0]}")
def large(request):
    scale, bi = request.param
    B, ctx = SHAPES[bi]
    inp = synth.random_small(11, B=B, Hq=4, Hkv=2, d=64, P=16, dtype="bf16", ctx=ctx, planted_per_kv=5)
    return inp, Dev(inp, scale=scale)


def _selections(inp, seed=5):
    """Per row: all pages, a random half, a contiguous run, a single page."""
    rng = np.random.default_rng(seed)
    sel = np.full((inp.B, inp.Hq, inp.max_pages), -1, np.int32)
    cnt = np.zeros((inp.B, inp.Hq), np.int32)
    for b in range(inp.B):
        npg = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        for h in range(inp.Hq):
            kind = (b * inp.Hq + h) % 4
            if kind == 0:
                s = np.arange(npg)
            elif kind == 1:
                s = np.sort(rng.choice(npg, size=max(1, npg // 2), replace=False))
            elif kind == 2:
                lo = int(rng.integers(0, max(1, npg - 300)))
                s = np.arange(lo, min(npg, lo + 300))
            else:
                s = np.array([npg - 1])
            sel[b, h, :len(s)] = s
            cnt[b, h] = len(s)
    return sel, cnt


@pytest.mark.parametrize("alpha,method", [(1.5, 0), (2.0, 0), (2.0, 1), (1.25, 0)])
def test_entmax_decode_sparse_long_rows(large, alpha, method):
    inp, D = large
    sel, cnt = _selections(inp)
    decode_check(inp, D, alpha, sel, cnt, tau_method=method)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_entmax_decode_full_long_rows(large, alpha):
    inp, D = large
    decode_check(inp, D, alpha, None, None, full=True)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_entmax_decode_long_rows_repeat_bitwise(large, alpha):
    """Two calls on the same inputs give identical out, tau and weights (the
    helper steps merge integer counts and fixed-order partials)."""
    import torch
    inp, D = large
    sel, cnt = _selections(inp)
    si, ci = torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda()
    res = []
    for _ in range(2):
        out = torch.full((inp.B, inp.Hq, inp.d), np.nan, device="cuda")
        tau = torch.full((inp.B, inp.Hq), np.nan, dtype=torch.float64, device="cuda")
        w = torch.full((inp.B, inp.Hq, inp.max_pages * inp.P), np.nan, device="cuda")
        E.entmax_decode_sparse(D.shape, D.q, D.k, D.v, D.pt, D.sl, si, ci, alpha, out, tau=tau, weights_out=w)
        res.append((out.cpu().numpy(), tau.cpu().numpy(), w.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


@pytest.mark.parametrize("scale", [0.0, 0.002], ids=["scale_default", "scale0.002"])
def test_entmax_decode_sparse_very_long_row(scale):
    """One context of 262,144 tokens in pages of 16 (16,384 pages): row 0 keeps
    every page (32 chunk blocks of 8,192 tokens, so a chunk's later tokens are
    read again between its passes, and the merge looks pages up in memory
    rather than LDS: more than 2,048 items), row 1 a random 60% of them."""
    inp = synth.random_small(12, B=1, Hq=2, Hkv=1, d=64, P=16, dtype="bf16", ctx=(262144,), planted_per_kv=5)
    D = Dev(inp, scale=scale)
    npg = inp.max_pages
    assert npg == 16384
    rng = np.random.default_rng(3)
    sel = np.full((1, 2, npg), -1, np.int32)
    cnt = np.zeros((1, 2), np.int32)
    sel[0, 0] = np.arange(npg)
    cnt[0, 0] = npg
    half = np.sort(rng.choice(npg, size=int(0.6 * npg), replace=False))
    sel[0, 1, :len(half)] = half
    cnt[0, 1] = len(half)
    decode_check(inp, D, 1.5, sel, cnt)
