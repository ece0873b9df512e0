"""GPU parity: each C-ABI call against the CPU oracle on the same seeded inputs.

Bars: page metadata, page scores (stored float32 bits), page sets and entmax
supports are bit-exact; outputs are within 2e-3 relative L2 per row for bf16 KV
and 1e-5 for fp32 KV (fp32 accumulation of exact fp64-decided weights);
thresholds agree to 1e-12 relative.
"""
import numpy as np
import pytest

from gpu_util import TOL, Dev, decode_check, dev, host_raw, rel_l2_rows, sets_equal, torch
from sparse_decode_attention_page_amd import synth
import sparse_decode_attention_page_amd as E
import oracle

pytestmark = pytest.mark.gpu

SMALL = [
    # (seed, B, Hq, Hkv, d, P, dtype, ctx)
    (0, 2, 4, 2, 64, 16, "bf16", (700, 333)),
    (1, 1, 8, 2, 128, 32, "bf16", (1500,)),
    (2, 3, 2, 1, 64, 64, "f32", (4096, 65, 1)),
    (3, 2, 8, 1, 64, 32, "bf16", (3000, 2017)),
    (4, 1, 1, 1, 64, 16, "f32", (4096,)),
    # more than 64 query-head rows: a set per query head goes to the slice decode
    (5, 5, 16, 4, 64, 16, "bf16", (1000, 333, 2048, 1, 4000)),
    (6, 3, 32, 4, 128, 32, "f32", (3000, 700, 1)),
]


def small(seed, B, Hq, Hkv, d, P, dtype, ctx):
    return synth.random_small(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, P=P, dtype=dtype, ctx=ctx, planted_per_kv=5)


@pytest.fixture(scope="module", params=SMALL, ids=lambda c: f"s{c[0]}_B{c[1]}_H{c[2]}x{c[3]}_d{c[4]}_P{c[5]}_{c[6]}")
def case(request):
    inp = small(*request.param)
    D = Dev(inp)
    meta_o = oracle.build_page_meta(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens)
    box_o, mu_o, var_o = oracle.score_pages(D.oshape, inp.q, meta_o, inp.page_table, inp.seq_lens)
    return inp, D, meta_o, (box_o, mu_o, var_o)


def _valid_mask(inp):
    m = np.zeros((inp.B, inp.Hq, inp.max_pages), bool)
    for b in range(inp.B):
        npg = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        m[b, :, :npg] = True
    return m


def test_build_page_meta(case):
    inp, D, meta_o, _ = case
    meta = D.zeros_meta()
    E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta)
    got = host_raw(meta, inp.dtype)
    assert np.array_equal(got, meta_o)


def test_build_page_meta_append(case):
    inp, D, meta_o, _ = case
    t = torch()
    meta = D.zeros_meta()
    from_tok = np.maximum(inp.seq_lens - 1, 0).astype(np.int32)  # one new token per sequence
    E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta, from_token=t.from_numpy(from_tok).cuda())
    got = host_raw(meta, inp.dtype)
    want = oracle.build_page_meta(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens, from_token=from_tok,
                                  meta=np.zeros_like(meta_o))
    assert np.array_equal(got, want)


def test_score_pages(case):
    inp, D, meta_o, (box_o, mu_o, var_o) = case
    meta = D.zeros_meta()
    E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta)
    box, mu, var = D.per_page(), D.per_page(), D.per_page()
    E.score_pages(D.shape, D.q, meta, D.pt, D.sl, box, mu, var)
    m = _valid_mask(inp)
    for got, want in ((box, box_o), (mu, mu_o), (var, var_o)):
        g = got.cpu().numpy()
        assert np.array_equal(g[m].view(np.uint32), want[m].view(np.uint32))
        assert np.all(np.isnan(g[~m]))  # pages past N_b untouched


def test_build_page_meta_f8(case):
    inp, D, _, _ = case
    t = torch()
    if inp.dtype != "bf16":
        with pytest.raises(E.EntmaxKVError, match="status 2"):
            E.build_page_meta_f8(D.shape, D.k, D.pt, D.sl, E.meta_f8_empty(D.shape))
        return
    meta = E.meta_f8_empty(D.shape)
    E.build_page_meta_f8(D.shape, D.k, D.pt, D.sl, meta)
    want = oracle.build_page_meta_f8(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens)
    assert np.array_equal(meta.cpu().numpy(), want)
    # append path: only the pages holding each sequence's newest token
    from_tok = np.maximum(inp.seq_lens - 1, 0).astype(np.int32)
    meta2 = E.meta_f8_empty(D.shape)
    E.build_page_meta_f8(D.shape, D.k, D.pt, D.sl, meta2, from_token=t.from_numpy(from_tok).cuda())
    want2 = oracle.build_page_meta_f8(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens, from_token=from_tok,
                                      meta=np.zeros_like(want))
    assert np.array_equal(meta2.cpu().numpy(), want2)


def test_score_pages_f8_and_gauss(case):
    inp, D, _, _ = case
    if inp.dtype != "bf16":
        with pytest.raises(E.EntmaxKVError, match="status 2"):
            E.score_pages_f8(D.shape, D.q, E.meta_f8_empty(D.shape), D.pt, D.sl, D.per_page(), D.per_page(),
                             D.per_page())
        return
    meta = E.meta_f8_empty(D.shape)
    E.build_page_meta_f8(D.shape, D.k, D.pt, D.sl, meta)
    box, mu, var = D.per_page(), D.per_page(), D.per_page()
    E.score_pages_f8(D.shape, D.q, meta, D.pt, D.sl, box, mu, var)
    meta_o = oracle.build_page_meta_f8(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens)
    bo, mo, vo = oracle.score_pages_f8(D.oshape, inp.q, meta_o, inp.page_table, inp.seq_lens)
    m = _valid_mask(inp)
    for got, want in ((box, bo), (mu, mo), (var, vo)):
        g = got.cpu().numpy()
        assert np.array_equal(g[m].view(np.uint32), want[m].view(np.uint32))
        assert np.all(np.isnan(g[~m]))
    # the Gaussian selector on the compact scores (same kernels, other inputs)
    sel, cnt = D.sel_buffers()
    E.select_pages_gauss(D.shape, box, mu, var, D.sl, 1.5, 0.5, sel, cnt)
    so, co, _ = oracle.select_gauss(D.oshape, bo, mo, vo, inp.seq_lens, 1.5, 0.5)
    assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co) == []


@pytest.mark.parametrize("k", [1, 3, 17, 1000])
def test_select_topk(case, k):
    inp, D, _, (box_o, _, _) = case
    box = torch().from_numpy(box_o).cuda()
    sel, cnt = D.sel_buffers()
    E.select_pages_topk(D.shape, box, D.sl, k, sel, cnt)
    so, co = oracle.select_topk(D.oshape, box_o, inp.seq_lens, k)
    assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co) == []


@pytest.mark.parametrize("mp", [1000, 16384, 17500])
@pytest.mark.parametrize("k", [1, 64, 999])
def test_select_topk_ties_and_long_rows(mp, k):
    """Top-k on bounds with many ties (40 distinct values), NaN and both signed
    zeros, over rows of 1,000 and 16,384 pages (one batch of keys, held in
    registers for every pass) and 17,500 pages (two batches, read again each
    pass), one row ragged; bit-exact sets against the oracle (ties to the
    lowest page index, NaN last)."""
    t = torch()
    B, Hq, P = 2, 4, 16  # one KV head of four query heads
    rng = np.random.default_rng(mp * 7 + k)
    box = (rng.integers(0, 40, size=(B, Hq, mp)).astype(np.float32) * 0.25 - 3.0).astype(np.float32)
    box[0, 0, rng.integers(0, mp, 25)] = np.nan
    box[1, 2, rng.integers(0, mp, 25)] = -0.0
    box[1, 2, rng.integers(0, mp, 25)] = 0.0
    seq_lens = np.array([mp * P, (mp - 37) * P - 5], dtype=np.int32)
    shape = E.Shape(B, Hq, 1, 64, P, mp, mp * B, E.BF16, 0.0)
    oshape = oracle.Shape(B, Hq, 1, 64, P, mp, mp * B, "bf16", 0.0)
    sel = t.full((B, Hq, mp), -7, dtype=t.int32, device="cuda")
    cnt = t.full((B, Hq), -7, dtype=t.int32, device="cuda")
    E.select_pages_topk(shape, t.from_numpy(box).cuda(), dev(seq_lens, "i32"), k, sel, cnt)
    so, co = oracle.select_topk(oshape, box, seq_lens, k)
    assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co) == []


@pytest.mark.parametrize("alpha,delta", [(1.5, 0.5), (2.0, 0.5), (1.5, 0.0), (2.0, 1.5), (1.25, 0.5)])
def test_select_gauss(case, alpha, delta):
    inp, D, _, (box_o, mu_o, var_o) = case
    t = torch()
    box, mu, var = (t.from_numpy(a).cuda() for a in (box_o, mu_o, var_o))
    sel, cnt = D.sel_buffers()
    tau = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
    E.select_pages_gauss(D.shape, box, mu, var, D.sl, alpha, delta, sel, cnt, tau_hat=tau)
    so, co, to = oracle.select_gauss(D.oshape, box_o, mu_o, var_o, inp.seq_lens, alpha, delta)
    assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co) == []
    tg = tau.cpu().numpy()
    assert np.allclose(tg, to, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("alpha,delta", [(1.5, 0.5), (2.0, 0.5), (1.5, 0.0), (1.25, 0.5)])
def test_score_select_gauss_fused(case, alpha, delta):
    """score_select_pages_gauss: box/mu/var, sets and tau_hat are the bits of
    score_pages then select_pages_gauss, and match the oracle (sets exactly,
    tau_hat to 1e-12); a masked sequence's rows are left untouched."""
    inp, D, meta_o, (box_o, mu_o, var_o) = case
    t = torch()
    meta = D.zeros_meta()
    E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta)
    mask = np.ones(inp.B, np.uint8)
    if inp.B > 1:
        mask[1] = 0
    mk = t.from_numpy(mask).cuda()
    box, mu, var = D.per_page(), D.per_page(), D.per_page()
    sel, cnt = D.sel_buffers()
    tau = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
    for _ in range(2):  # the second call reuses the workspace (its counters were left at zero)
        ws = E.workspace(D.shape, E.CALL_SCORE_GAUSS) if _ == 0 else ws
        E.score_select_pages_gauss(D.shape, D.q, meta, D.pt, D.sl, box, mu, var, alpha, delta, sel, cnt,
                                   seq_mask=mk, tau_hat=tau, ws=ws)
    box2, mu2, var2 = D.per_page(), D.per_page(), D.per_page()
    E.score_pages(D.shape, D.q, meta, D.pt, D.sl, box2, mu2, var2)
    sel2, cnt2 = D.sel_buffers()
    tau2 = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
    E.select_pages_gauss(D.shape, box2, mu2, var2, D.sl, alpha, delta, sel2, cnt2, seq_mask=mk, tau_hat=tau2)
    for a, b in ((box, box2), (mu, mu2), (var, var2)):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))
    assert np.array_equal(cnt.cpu().numpy(), cnt2.cpu().numpy())
    assert np.array_equal(sel.cpu().numpy(), sel2.cpu().numpy())
    tg = tau.cpu().numpy()
    assert np.array_equal(tg.view(np.uint64), tau2.cpu().numpy().view(np.uint64))
    so, co, to = oracle.select_gauss(D.oshape, box_o, mu_o, var_o, inp.seq_lens, alpha, delta, seq_mask=mask)
    keep = mask.astype(bool)
    sg, cg = sel.cpu().numpy(), cnt.cpu().numpy()
    assert sets_equal(sg[keep], cg[keep], so[keep], co[keep]) == []
    assert np.allclose(tg[keep], to[keep], rtol=1e-12, atol=1e-12)
    assert np.all(cg[~keep] == -1) and np.all(np.isnan(tg[~keep]))


def test_score_select_gauss_fused_invalid_pages(case):
    """Pages whose record holds a NaN (box, mu and var then non-finite) are
    skipped by the fused call's bracket exactly as by the selector's own: the
    same sets and tau_hat bits as the two calls in turn."""
    inp, D, _, _ = case
    t = torch()
    meta = D.zeros_meta()
    E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta)
    pt = inp.page_table
    for b in range(inp.B):  # the first and the last page of every sequence, KV head 0
        npg = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        for p_ in {0, npg - 1}:
            meta[int(pt[b, p_]), 0, 0, 0] = float("nan")
    out = []
    for fused in (True, False):
        box, mu, var = D.per_page(), D.per_page(), D.per_page()
        sel, cnt = D.sel_buffers()
        tau = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
        if fused:
            E.score_select_pages_gauss(D.shape, D.q, meta, D.pt, D.sl, box, mu, var, 1.5, 0.5, sel, cnt,
                                       tau_hat=tau)
        else:
            E.score_pages(D.shape, D.q, meta, D.pt, D.sl, box, mu, var)
            E.select_pages_gauss(D.shape, box, mu, var, D.sl, 1.5, 0.5, sel, cnt, tau_hat=tau)
        out.append((sel.cpu().numpy(), cnt.cpu().numpy(), tau.cpu().numpy(), box.cpu().numpy()))
    (s1, c1, t1, b1), (s2, c2, t2, b2) = out
    assert np.isnan(b1[:, 0]).any()  # the planted NaN reached the scores
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert np.array_equal(t1.view(np.uint64), t2.view(np.uint64))


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25])
def test_entmax_decode_sparse_topk(case, alpha):
    inp, D, _, (box_o, _, _) = case
    so, co = oracle.select_topk(D.oshape, box_o, inp.seq_lens, 7)
    decode_check(inp, D, alpha, so, co)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_entmax_decode_sparse_gauss(case, alpha):
    inp, D, _, (box_o, mu_o, var_o) = case
    so, co, _ = oracle.select_gauss(D.oshape, box_o, mu_o, var_o, inp.seq_lens, alpha, 0.5)
    decode_check(inp, D, alpha, so, co)


def test_entmax_decode_sparse_sort_alpha2(case):
    inp, D, _, (box_o, _, _) = case
    so, co = oracle.select_topk(D.oshape, box_o, inp.seq_lens, 9)
    decode_check(inp, D, 2.0, so, co, tau_method=1)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_entmax_decode_full(case, alpha):
    inp, D, _, _ = case
    decode_check(inp, D, alpha, None, None, full=True)


def test_entmax_decode_full_sort_alpha2(case):
    """The full-cache decode with the sparsemax sort form (tau_method 1)."""
    inp, D, _, _ = case
    decode_check(inp, D, 2.0, None, None, full=True, tau_method=1)


def test_softmax_decode_full(case):
    inp, D, _, _ = case
    t = torch()
    out = t.full((inp.B, inp.Hq, inp.d), np.nan, dtype=t.float32, device="cuda")
    lse = t.full((inp.B, inp.Hq), np.nan, dtype=t.float32, device="cuda")
    E.softmax_decode_full(D.shape, D.q, D.k, D.v, D.pt, D.sl, out, lse=lse)
    oo, lo = oracle.softmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens)
    assert rel_l2_rows(out.cpu().numpy(), oo) <= TOL[inp.dtype]
    assert np.allclose(lse.cpu().numpy(), lo, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("policy", ["topk", "gauss"])
def test_softmax_decode_sparse(case, policy):
    """Softmax over the oracle's own selection of each case."""
    inp, D, _, (box_o, mu_o, var_o) = case
    t = torch()
    if policy == "topk":
        so, co = oracle.select_topk(D.oshape, box_o, inp.seq_lens, 7)
    else:
        so, co, _ = oracle.select_gauss(D.oshape, box_o, mu_o, var_o, inp.seq_lens, 1.5, 0.5)
    out = t.full((inp.B, inp.Hq, inp.d), np.nan, dtype=t.float32, device="cuda")
    lse = t.full((inp.B, inp.Hq), np.nan, dtype=t.float32, device="cuda")
    E.softmax_decode_sparse(D.shape, D.q, D.k, D.v, D.pt, D.sl, t.from_numpy(so).cuda(), t.from_numpy(co).cuda(),
                            out, lse=lse)
    oo, lo = oracle.softmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                   sel_idx=so, sel_cnt=co)
    assert rel_l2_rows(out.cpu().numpy(), oo) <= TOL[inp.dtype]
    assert np.allclose(lse.cpu().numpy(), lo, rtol=1e-5, atol=1e-5)


def test_softmax_decode_sparse_edge_cases(case):
    """Bad selections give NaN rows, an empty one zeros and lse = -inf, as in the oracle."""
    inp, D, _, _ = case
    t = torch()
    MP = inp.max_pages
    so = np.zeros((inp.B, inp.Hq, MP), np.int32)
    co = np.zeros((inp.B, inp.Hq), np.int32)
    rows = inp.B * inp.Hq
    flat_s, flat_c = so.reshape(rows, MP), co.reshape(rows)
    for r in range(rows):
        b = r // inp.Hq
        np_b = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        kind = r % 4
        if kind == 0:      # empty
            flat_c[r] = 0
        elif kind == 1:    # count above N_b
            flat_c[r] = np_b + 1
            flat_s[r, :np_b + 1 if np_b + 1 <= MP else MP] = np.arange(min(np_b + 1, MP))
        elif kind == 2 and np_b >= 2:  # not ascending
            flat_c[r] = 2
            flat_s[r, :2] = [1, 0]
        else:              # every page
            flat_c[r] = np_b
            flat_s[r, :np_b] = np.arange(np_b)
    out = t.full((inp.B, inp.Hq, inp.d), 7.0, dtype=t.float32, device="cuda")
    lse = t.full((inp.B, inp.Hq), 7.0, dtype=t.float32, device="cuda")
    E.softmax_decode_sparse(D.shape, D.q, D.k, D.v, D.pt, D.sl, t.from_numpy(so).cuda(), t.from_numpy(co).cuda(),
                            out, lse=lse)
    oo, lo = oracle.softmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                   sel_idx=so, sel_cnt=co)
    og, lg = out.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(np.isnan(og), np.isnan(oo)) and np.array_equal(np.isnan(lg), np.isnan(lo))
    fin = ~np.isnan(lo)
    assert np.array_equal(np.isinf(lg[fin]), np.isinf(lo[fin]))
    ok = ~np.isnan(oo).any(axis=-1)
    assert rel_l2_rows(og[ok][None], oo[ok][None]) <= TOL[inp.dtype] if ok.any() else True


# ------------------------------------------------------- group-shared selection
def _group_decode_check(inp, D, alpha, sg, cg, tau_method=0):
    """entmax_decode_sparse_group against the oracle decoding every head over
    its group's set (the expanded selection)."""
    t = torch()
    out = t.full((inp.B, inp.Hq, inp.d), np.nan, dtype=t.float32, device="cuda")
    tau = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
    w = t.full((inp.B, inp.Hq, inp.max_pages * inp.P), np.nan, dtype=t.float32, device="cuda")
    E.entmax_decode_sparse_group(D.shape, D.q, D.k, D.v, D.pt, D.sl, t.from_numpy(sg).cuda(), t.from_numpy(cg).cuda(),
                                 alpha, out, tau=tau, weights_out=w, tau_method=tau_method)
    se, ce = oracle.expand_group_selection(D.oshape, sg, cg)
    oo, to, wo = oracle.entmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                      alpha, se, ce, want_weights=True)
    og, tg, wg = out.cpu().numpy(), tau.cpu().numpy(), w.cpu().numpy()
    assert np.array_equal(np.isnan(og).any(-1), np.isnan(oo).any(-1)), "malformed rows differ"
    ok = ~np.isnan(oo).any(-1)
    assert np.array_equal(np.isnan(tg), np.isnan(to))
    fin = ~np.isnan(to)
    assert np.allclose(tg[fin], to[fin], rtol=1e-12, atol=1e-12)
    assert np.array_equal(wg[ok] > 0, wo[ok] > 0), "support differs"
    assert np.max(np.abs(wg[ok] - wo[ok]), initial=0.0) < 1e-5
    if ok.any():
        assert rel_l2_rows(og[ok][None], oo[ok][None]) <= TOL[inp.dtype]


@pytest.mark.parametrize("policy", ["topk", "gauss"])
def test_group_selection_and_decode(case, policy):
    inp, D, meta_o, (box_o, mu_o, var_o) = case
    t = torch()
    B, Hkv, MP = inp.B, inp.Hkv, inp.max_pages
    box, mu, var = (t.from_numpy(a).cuda() for a in (box_o, mu_o, var_o))
    sel = t.full((B, Hkv, MP), -1, dtype=t.int32, device="cuda")
    cnt = t.full((B, Hkv), -1, dtype=t.int32, device="cuda")
    if policy == "topk":
        for k in (1, 5, 1000):
            E.select_pages_topk_group(D.shape, box, D.sl, k, sel, cnt)
            so, co = oracle.select_topk_group(D.oshape, box_o, inp.seq_lens, k)
            assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co) == []
    else:
        tau = t.full((B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
        E.select_pages_gauss_group(D.shape, box, mu, var, D.sl, 1.5, 0.5, sel, cnt, tau_hat=tau)
        so, co, to = oracle.select_gauss_group(D.oshape, box_o, mu_o, var_o, inp.seq_lens, 1.5, 0.5)
        assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co) == []
        assert np.allclose(tau.cpu().numpy(), to, rtol=1e-12, atol=1e-12)
    for alpha in (1.5, 2.0):
        _group_decode_check(inp, D, alpha, so, co)
    _group_decode_check(inp, D, 2.0, so, co, tau_method=1)


def test_group_decode_edge_cases(case):
    """Empty, over-long, non-ascending and full group sets, as the oracle rules them."""
    inp, D, _, _ = case
    MP = inp.max_pages
    sg = np.zeros((inp.B, inp.Hkv, MP), np.int32)
    cg = np.zeros((inp.B, inp.Hkv), np.int32)
    for b in range(inp.B):
        np_b = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        for g in range(inp.Hkv):
            kind = (b * inp.Hkv + g) % 4
            if kind == 0:
                cg[b, g] = 0
            elif kind == 1:
                cg[b, g] = np_b + 1
                sg[b, g, :min(np_b + 1, MP)] = np.arange(min(np_b + 1, MP))
            elif kind == 2 and np_b >= 2:
                cg[b, g] = 2
                sg[b, g, :2] = [1, 0]
            else:
                cg[b, g] = np_b
                sg[b, g, :np_b] = np.arange(np_b)
    _group_decode_check(inp, D, 1.5, sg, cg)


# ------------------------------------------------------------ streaming append
@pytest.mark.parametrize("compact", [False, True])
def test_append_token(case, compact):
    """append_token writes token L_b - 1 into its slot and rebuilds that page's
    record: pools and metadata bit-exact against the pools updated on the host
    and the oracle's rebuild from that token; a sequence whose page entry is
    out of range stays untouched."""
    inp, D, _, _ = case
    t = torch()
    if compact and inp.dtype != "bf16":
        with pytest.raises(E.EntmaxKVError, match="status 2"):
            rows = D.q[:, :inp.Hkv].contiguous()
            E.append_token(D.shape, rows, rows, D.k.clone(), D.v.clone(), D.pt, D.sl, E.meta_f8_empty(D.shape),
                           compact=True)
        return
    rng = np.random.default_rng(31)
    B, Hkv, d, P = inp.B, inp.Hkv, inp.d, inp.P
    kn = synth._store(rng.standard_normal((B, Hkv, d), dtype=np.float32), inp.dtype)
    vn = synth._store(rng.standard_normal((B, Hkv, d), dtype=np.float32), inp.dtype)
    pt = inp.page_table.copy()
    if B > 1:  # the last sequence's newest page: an out-of-range entry
        pt[B - 1, (int(inp.seq_lens[B - 1]) - 1) // P] = inp.num_phys
    k_exp, v_exp = inp.k_pool.copy(), inp.v_pool.copy()
    for b in range(B):
        L = int(inp.seq_lens[b])
        ph = pt[b, (L - 1) // P]
        if L >= 1 and 0 <= ph < inp.num_phys:
            k_exp[ph, :, (L - 1) % P, :] = kn[b]
            v_exp[ph, :, (L - 1) % P, :] = vn[b]
    build = oracle.build_page_meta_f8 if compact else oracle.build_page_meta
    meta0 = build(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens)
    from_tok = np.maximum(inp.seq_lens - 1, 0).astype(np.int32)
    meta_exp = build(D.oshape, k_exp, pt, inp.seq_lens, from_token=from_tok, meta=meta0.copy())
    kind = D.kind
    k, v = D.k.clone(), D.v.clone()
    if compact:
        meta = t.from_numpy(meta0.copy()).cuda()
    else:
        meta = D.zeros_meta()
        E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta)
    E.append_token(D.shape, dev(kn, kind), dev(vn, kind), k, v, dev(pt, "i32"), D.sl, meta, compact=compact)
    assert np.array_equal(host_raw(k, inp.dtype), k_exp) and np.array_equal(host_raw(v, inp.dtype), v_exp)
    got = meta.cpu().numpy() if compact else host_raw(meta, inp.dtype)
    assert np.array_equal(got, meta_exp)


@pytest.mark.parametrize("dtype,compact", [("bf16", False), ("bf16", True), ("f32", False)])
def test_append_token_edges(dtype, compact):
    """append_token at the page boundaries and the degenerate lengths: eight
    sequences of 700 tokens in pages of 16 (cap 704) append with L = 1 (first
    token), 16 (last slot of page 0), 17 and 33 (first slot of a new page), 700,
    704 (the cap), 0 (nothing written) and 720 (clamped to the cap, as in every
    call).  Pools and records bit-exact against the host update and the
    oracle's rebuild of the touched pages."""
    inp = small(7, 8, 4, 2, 64, 16, dtype, (700,) * 8)
    D = Dev(inp)
    B, P, MP = inp.B, inp.P, inp.max_pages
    new_sl = np.array([1, 16, 17, 33, 700, 704, 0, 720], dtype=np.int32)
    cap = MP * P
    rng = np.random.default_rng(41)
    kn = synth._store(rng.standard_normal((B, inp.Hkv, inp.d), dtype=np.float32), dtype)
    vn = synth._store(rng.standard_normal((B, inp.Hkv, inp.d), dtype=np.float32), dtype)
    k_exp, v_exp = inp.k_pool.copy(), inp.v_pool.copy()
    for b in range(B):
        L = min(max(int(new_sl[b]), 0), cap)
        if L >= 1:
            ph = inp.page_table[b, (L - 1) // P]
            assert 0 <= ph < inp.num_phys
            k_exp[ph, :, (L - 1) % P, :] = kn[b]
            v_exp[ph, :, (L - 1) % P, :] = vn[b]
    build = oracle.build_page_meta_f8 if compact else oracle.build_page_meta
    meta0 = build(D.oshape, inp.k_pool, inp.page_table, inp.seq_lens)
    from_tok = np.maximum(np.minimum(new_sl, cap) - 1, 0).astype(np.int32)
    meta_exp = build(D.oshape, k_exp, inp.page_table, new_sl, from_token=from_tok, meta=meta0.copy())
    t = torch()
    k, v = D.k.clone(), D.v.clone()
    meta = t.from_numpy(meta0.copy()).cuda() if compact else dev(meta0, D.kind)
    E.append_token(D.shape, dev(kn, D.kind), dev(vn, D.kind), k, v, D.pt, dev(new_sl, "i32"), meta,
                   compact=compact)
    assert np.array_equal(host_raw(k, dtype), k_exp) and np.array_equal(host_raw(v, dtype), v_exp)
    got = meta.cpu().numpy() if compact else host_raw(meta, dtype)
    assert np.array_equal(got, meta_exp)
