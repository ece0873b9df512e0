"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (same generator, same calls, same workspaces).

The oracle recomputes sampled query rows one by one: page metadata of the
sampled sequences and page scores of the sampled rows (stored values bit for
bit: both sides add the same exact products in coordinate order), the page
sets of both selectors computed from the GPU's own scores (bit-exact), the
sparse and full-cache entmax outputs, thresholds and supports, and the
full-cache softmax output (tolerances as in the small cases).  The last test
runs the oracle's whole chain from the seeded inputs (its own metadata, scores,
selections and decodes) against the GPU's chain on the sampled rows and logs
the margin of every cut.
"""
import numpy as np
import pytest

from gpu_util import (TOL, gauss_keep_margin, log_margin, rel_l2_rows, sets_equal, support_margin, topk_gap,
                      torch)
import sparse_decode_attention_page_amd as E
from sparse_decode_attention_page_amd import synth
import oracle

pytestmark = pytest.mark.gpu

N_SAMPLE = 3


def _rows_sample(B, Hq, seed):
    rng = np.random.default_rng(seed)
    rows = {0, B * Hq - 1}
    rows.update(int(r) for r in rng.choice(B * Hq, size=min(N_SAMPLE, B * Hq), replace=False))
    return sorted(rows)


@pytest.fixture(scope="module", params=list(synth.WORKLOADS))
def full(request):
    t = torch()
    wl = synth.WORKLOADS[request.param]
    print(f"\n[full-size] generating {wl.name}", flush=True)
    inp = synth.make_device(wl, 0)
    shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
    osh = oracle.Shape(inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages, inp.num_phys, inp.dtype, 0.0)
    B, Hq, MP = inp.B, inp.Hq, inp.max_pages
    meta = t.zeros((inp.num_phys, inp.Hkv, 4, inp.d), dtype=inp.k_pool.dtype, device="cuda")
    E.build_page_meta(shape, inp.k_pool, inp.page_table, inp.seq_lens, meta)
    box = t.full((B, Hq, MP), np.nan, device="cuda")
    mu, var = t.full_like(box, np.nan), t.full_like(box, np.nan)
    E.score_pages(shape, inp.q, meta, inp.page_table, inp.seq_lens, box, mu, var)
    rows = _rows_sample(B, Hq, 7)
    host = {k: inp.host(k) for k in ("q", "k_pool", "v_pool", "page_table", "seq_lens")}
    t.cuda.synchronize()
    return dict(wl=wl, inp=inp, shape=shape, osh=osh, meta=meta, box=box, mu=mu, var=var, rows=rows, host=host)


def _take_rows(a, rows):
    a = np.asarray(a)
    return a.reshape(-1, *a.shape[2:])[rows]


def test_full_meta_sampled_sequences(full):
    inp, h = full["inp"], full["host"]
    bs = sorted({r // inp.Hq for r in full["rows"]})
    sl = np.zeros_like(h["seq_lens"])
    sl[bs] = h["seq_lens"][bs]  # the oracle rebuilds the sampled sequences' pages only
    want = oracle.build_page_meta(full["osh"], h["k_pool"], h["page_table"], sl)
    t = torch()
    got = full["meta"].view(t.int16).cpu().numpy().view(np.uint16) if inp.dtype == "bf16" else full["meta"].cpu().numpy()
    for b in bs:
        npg = (int(h["seq_lens"][b]) + inp.P - 1) // inp.P
        phys = h["page_table"][b, :npg]
        assert np.array_equal(got[phys], want[phys]), f"metadata of sequence {b} differs"


def test_full_score_sampled_rows(full):
    inp, h, rows = full["inp"], full["host"], full["rows"]
    t = torch()
    meta_h = full["meta"].view(t.int16).cpu().numpy().view(np.uint16) if inp.dtype == "bf16" else full["meta"].cpu().numpy()
    bo, mo, vo = oracle.score_pages(full["osh"], h["q"], meta_h, h["page_table"], h["seq_lens"], rows=rows)
    for got, want in ((full["box"], bo), (full["mu"], mo), (full["var"], vo)):
        g = _take_rows(got.cpu().numpy(), rows)
        w = _take_rows(want, rows)
        for i, r in enumerate(rows):
            npg = (int(h["seq_lens"][r // inp.Hq]) + inp.P - 1) // inp.P
            gi, wi = g[i, :npg], w[i, :npg]
            bad = np.flatnonzero(gi.view(np.int32) != wi.view(np.int32))
            assert bad.size == 0, f"row {r}: {bad.size} stored scores differ, first at page {bad[:5]}"


def test_full_meta_and_score_f8_sampled(full):
    """Compact records (E4M3 mean / variance) at full size: metadata of the
    sampled sequences and scores of the sampled rows bit-exact."""
    inp, h, rows = full["inp"], full["host"], full["rows"]
    if inp.dtype != "bf16":
        pytest.skip("compact metadata holds bf16 bounds")
    t = torch()
    m8 = E.meta_f8_empty(full["shape"])
    E.build_page_meta_f8(full["shape"], inp.k_pool, inp.page_table, inp.seq_lens, m8)
    B, Hq, MP = inp.B, inp.Hq, inp.max_pages
    box = t.full((B, Hq, MP), np.nan, device="cuda")
    mu, var = t.full_like(box, np.nan), t.full_like(box, np.nan)
    E.score_pages_f8(full["shape"], inp.q, m8, inp.page_table, inp.seq_lens, box, mu, var)
    got_meta = m8.cpu().numpy()
    bs = sorted({r // inp.Hq for r in rows})
    sl = np.zeros_like(h["seq_lens"])
    sl[bs] = h["seq_lens"][bs]
    want = oracle.build_page_meta_f8(full["osh"], h["k_pool"], h["page_table"], sl)
    for b in bs:
        npg = (int(h["seq_lens"][b]) + inp.P - 1) // inp.P
        phys = h["page_table"][b, :npg]
        assert np.array_equal(got_meta[phys], want[phys]), f"compact metadata of sequence {b} differs"
    bo, mo, vo = oracle.score_pages_f8(full["osh"], h["q"], got_meta, h["page_table"], h["seq_lens"], rows=rows)
    for got, wnt in ((box, bo), (mu, mo), (var, vo)):
        g = _take_rows(got.cpu().numpy(), rows)
        w = _take_rows(wnt, rows)
        for i, r in enumerate(rows):
            npg = (int(h["seq_lens"][r // inp.Hq]) + inp.P - 1) // inp.P
            bad = np.flatnonzero(g[i, :npg].view(np.int32) != w[i, :npg].view(np.int32))
            assert bad.size == 0, f"row {r}: {bad.size} compact scores differ, first at page {bad[:5]}"


def _select(full, policy):
    t = torch()
    inp, wl = full["inp"], full["wl"]
    B, Hq, MP = inp.B, inp.Hq, inp.max_pages
    sel = t.full((B, Hq, MP), -1, dtype=t.int32, device="cuda")
    cnt = t.full((B, Hq), -1, dtype=t.int32, device="cuda")
    tau = t.full((B, Hq), np.nan, dtype=t.float64, device="cuda")
    if policy == "topk":
        E.select_pages_topk(full["shape"], full["box"], inp.seq_lens, wl.topk, sel, cnt)
    else:
        E.select_pages_gauss(full["shape"], full["box"], full["mu"], full["var"], inp.seq_lens, wl.alphas[0],
                             wl.delta, sel, cnt, tau_hat=tau)
    return sel, cnt, tau


@pytest.mark.parametrize("policy", ["topk", "gauss"])
def test_full_selection_sampled_rows(full, policy):
    inp, h, rows, wl = full["inp"], full["host"], full["rows"], full["wl"]
    sel, cnt, tau = _select(full, policy)
    box, mu, var = (full[k].cpu().numpy() for k in ("box", "mu", "var"))
    if policy == "topk":
        so, co = oracle.select_topk(full["osh"], box, h["seq_lens"], wl.topk, rows=rows)
    else:
        so, co, to = oracle.select_gauss(full["osh"], box, mu, var, h["seq_lens"], wl.alphas[0], wl.delta, rows=rows)
        tg = tau.cpu().numpy().reshape(-1)[rows]
        assert np.allclose(tg, to.reshape(-1)[rows], rtol=1e-12, atol=1e-12)
    assert sets_equal(sel.cpu().numpy(), cnt.cpu().numpy(), so, co, rows=set(rows)) == []


def test_full_gauss_selection_is_deterministic(full):
    """Two calls of the Gaussian selector on the same scores give the same
    tau_hat bits and the same sets (integer counts, fixed-order sums)."""
    t = torch()
    s1, c1, t1 = _select(full, "gauss")
    s2, c2, t2 = _select(full, "gauss")
    assert t.equal(c1, c2)
    assert t.equal(s1, s2)
    assert t.equal(t1.view(t.int64), t2.view(t.int64)), "tau_hat bits differ between two runs"


def test_full_fused_score_select_gauss(full):
    """score_select_pages_gauss at the full size (the benchmark's step): box,
    mu and var, the sets and the tau_hat bits equal score_pages followed by
    select_pages_gauss, on every row."""
    t = torch()
    inp, wl = full["inp"], full["wl"]
    B, Hq, MP = inp.B, inp.Hq, inp.max_pages
    box, mu, var = (t.full((B, Hq, MP), np.nan, device="cuda") for _ in range(3))
    sel = t.full((B, Hq, MP), -1, dtype=t.int32, device="cuda")
    cnt = t.full((B, Hq), -1, dtype=t.int32, device="cuda")
    tau = t.full((B, Hq), np.nan, dtype=t.float64, device="cuda")
    E.score_select_pages_gauss(full["shape"], inp.q, full["meta"], inp.page_table, inp.seq_lens, box, mu, var,
                               wl.alphas[0], wl.delta, sel, cnt, tau_hat=tau)
    s2, c2, t2 = _select(full, "gauss")
    for a, b in ((box, full["box"]), (mu, full["mu"]), (var, full["var"])):
        assert t.equal(a.view(t.int32), b.view(t.int32))
    assert t.equal(cnt, c2)
    assert t.equal(sel, s2)
    assert t.equal(tau.view(t.int64), t2.view(t.int64))


@pytest.mark.parametrize("kind", ["sparse_gauss", "sparse_topk", "full"])
def test_full_entmax_sampled_rows(full, kind):
    t = torch()
    inp, h, rows, wl = full["inp"], full["host"], full["rows"], full["wl"]
    B, Hq, MP, P, d = inp.B, inp.Hq, inp.max_pages, inp.P, inp.d
    alpha = wl.alphas[0]
    out = t.full((B, Hq, d), np.nan, device="cuda")
    tau = t.full((B, Hq), np.nan, dtype=t.float64, device="cuda")
    w = t.full((B, Hq, MP * P), np.nan, device="cuda")
    if kind == "full":
        E.entmax_decode_full(full["shape"], inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, alpha,
                             out, tau=tau, weights_out=w)
        oo, to, wo = oracle.entmax_decode(full["osh"], h["q"], h["k_pool"], h["v_pool"], h["page_table"],
                                          h["seq_lens"], alpha, rows=rows, want_weights=True)
    else:
        sel, cnt, _ = _select(full, "gauss" if kind == "sparse_gauss" else "topk")
        E.entmax_decode_sparse(full["shape"], inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, sel, cnt,
                               alpha, out, tau=tau, weights_out=w)
        oo, to, wo = oracle.entmax_decode(full["osh"], h["q"], h["k_pool"], h["v_pool"], h["page_table"],
                                          h["seq_lens"], alpha, sel.cpu().numpy(), cnt.cpu().numpy(), rows=rows,
                                          want_weights=True)
    og = _take_rows(out.cpu().numpy(), rows)
    tg = tau.cpu().numpy().reshape(-1)[rows]
    wg = w.view(B * Hq, -1)[rows].cpu().numpy()
    oo, to, wo = _take_rows(oo, rows), to.reshape(-1)[rows], _take_rows(wo, rows)
    assert np.allclose(tg, to, rtol=1e-12, atol=1e-12)
    assert np.array_equal(wg > 0, wo > 0), "support differs"
    assert np.max(np.abs(wg - wo)) < 1e-5
    assert rel_l2_rows(og, oo) <= TOL[inp.dtype]


def test_full_softmax_sampled_rows(full):
    t = torch()
    inp, h, rows = full["inp"], full["host"], full["rows"]
    out = t.full((inp.B, inp.Hq, inp.d), np.nan, device="cuda")
    lse = t.full((inp.B, inp.Hq), np.nan, device="cuda")
    E.softmax_decode_full(full["shape"], inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, out, lse=lse)
    oo, lo = oracle.softmax_decode(full["osh"], h["q"], h["k_pool"], h["v_pool"], h["page_table"], h["seq_lens"],
                                   rows=rows)
    assert rel_l2_rows(_take_rows(out.cpu().numpy(), rows), _take_rows(oo, rows)) <= TOL[inp.dtype]
    assert np.allclose(lse.cpu().numpy().reshape(-1)[rows], lo.reshape(-1)[rows], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("policy", ["gauss", "topk"])
def test_full_softmax_sparse_sampled_rows(full, policy):
    """Softmax over the kept pages of the GPU's own selection, against the oracle
    on the same selection (sampled rows)."""
    t = torch()
    inp, h, rows = full["inp"], full["host"], full["rows"]
    sel, cnt, _ = _select(full, policy)
    out = t.full((inp.B, inp.Hq, inp.d), np.nan, device="cuda")
    lse = t.full((inp.B, inp.Hq), np.nan, device="cuda")
    E.softmax_decode_sparse(full["shape"], inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, sel, cnt,
                            out, lse=lse)
    oo, lo = oracle.softmax_decode(full["osh"], h["q"], h["k_pool"], h["v_pool"], h["page_table"], h["seq_lens"],
                                   rows=rows, sel_idx=sel.cpu().numpy(), sel_cnt=cnt.cpu().numpy())
    assert rel_l2_rows(_take_rows(out.cpu().numpy(), rows), _take_rows(oo, rows)) <= TOL[inp.dtype]
    assert np.allclose(lse.cpu().numpy().reshape(-1)[rows], lo.reshape(-1)[rows], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("policy", ["gauss", "topk"])
def test_full_group_selection_and_decode_sampled(full, policy):
    """Group-shared selection (one set per KV head) and the group decode at full
    size: the sampled rows' groups against the oracle on the GPU's own scores."""
    t = torch()
    inp, h, rows, wl = full["inp"], full["host"], full["rows"], full["wl"]
    B, Hq, Hkv, MP, P, d = inp.B, inp.Hq, inp.Hkv, inp.max_pages, inp.P, inp.d
    G = Hq // Hkv
    alpha = wl.alphas[0]
    sel = t.full((B, Hkv, MP), -1, dtype=t.int32, device="cuda")
    cnt = t.full((B, Hkv), -1, dtype=t.int32, device="cuda")
    box, mu, var = (full[k].cpu().numpy() for k in ("box", "mu", "var"))
    grows = sorted({(r // Hq) * Hkv + (r % Hq) // G for r in rows})
    if policy == "topk":
        E.select_pages_topk_group(full["shape"], full["box"], inp.seq_lens, wl.topk, sel, cnt)
        so, co = oracle.select_topk_group(full["osh"], box, h["seq_lens"], wl.topk, rows=grows)
    else:
        E.select_pages_gauss_group(full["shape"], full["box"], full["mu"], full["var"], inp.seq_lens, alpha,
                                   wl.delta, sel, cnt)
        so, co, _ = oracle.select_gauss_group(full["osh"], box, mu, var, h["seq_lens"], alpha, wl.delta, rows=grows)
    sg, cg = sel.cpu().numpy(), cnt.cpu().numpy()
    assert sets_equal(sg, cg, so, co, rows=set(grows)) == []
    out = t.full((B, Hq, d), np.nan, device="cuda")
    tau = t.full((B, Hq), np.nan, dtype=t.float64, device="cuda")
    w = t.full((B, Hq, MP * P), np.nan, device="cuda")
    E.entmax_decode_sparse_group(full["shape"], inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, sel, cnt,
                                 alpha, out, tau=tau, weights_out=w)
    se, ce = oracle.expand_group_selection(full["osh"], sg, cg)
    oo, to, wo = oracle.entmax_decode(full["osh"], h["q"], h["k_pool"], h["v_pool"], h["page_table"], h["seq_lens"],
                                      alpha, se, ce, rows=rows, want_weights=True)
    og = _take_rows(out.cpu().numpy(), rows)
    tg = tau.cpu().numpy().reshape(-1)[rows]
    wg = w.view(B * Hq, -1)[rows].cpu().numpy()
    oo, to, wo = _take_rows(oo, rows), to.reshape(-1)[rows], _take_rows(wo, rows)
    assert np.allclose(tg, to, rtol=1e-12, atol=1e-12)
    assert np.array_equal(wg > 0, wo > 0), "support differs"
    assert np.max(np.abs(wg - wo)) < 1e-5
    assert rel_l2_rows(og, oo) <= TOL[inp.dtype]


def _policies(wl, b):
    """Selection policies a sequence uses (the mixed workload alternates them by sequence)."""
    if wl.policy == "mixed":
        return ("topk",) if b % 2 == 0 else ("gauss",)
    return {"gauss": ("gauss",), "topk": ("topk",), "both": ("gauss", "topk")}[wl.policy]


def test_full_chain_end_to_end(full):
    """The oracle's chain (its own metadata -> scores -> selection -> decode, from
    the seeded inputs) against the GPU's on the sampled rows: page sets and
    supports bit-exact, thresholds to 1e-12, weights to 1e-5, outputs to the
    dtype's tolerance; the margin of every cut is logged."""
    t = torch()
    inp, h, rows, wl = full["inp"], full["host"], full["rows"], full["wl"]
    osh = full["osh"]
    B, Hq, MP, P, d, G = inp.B, inp.Hq, inp.max_pages, inp.P, inp.d, inp.Hq // inp.Hkv
    scale = 1.0 / np.sqrt(d)
    bs = sorted({r // Hq for r in rows})
    sl_s = np.zeros_like(h["seq_lens"])
    sl_s[bs] = h["seq_lens"][bs]
    meta_o = oracle.build_page_meta(osh, h["k_pool"], h["page_table"], sl_s)
    bo, mo, vo = oracle.score_pages(osh, h["q"], meta_o, h["page_table"], h["seq_lens"], rows=rows)
    checked = 0
    for policy in ("gauss", "topk"):
        prow = [r for r in rows if policy in _policies(wl, r // Hq)]
        if not prow:
            continue
        sel, cnt, tau_hat = _select(full, policy)
        if policy == "gauss":
            so, co, to = oracle.select_gauss(osh, bo, mo, vo, h["seq_lens"], wl.alphas[0], wl.delta, rows=prow)
            tg = tau_hat.cpu().numpy().reshape(-1)[prow]
            assert np.allclose(tg, to.reshape(-1)[prow], rtol=1e-12, atol=1e-12), "tau_hat"
        else:
            so, co = oracle.select_topk(osh, bo, h["seq_lens"], wl.topk, rows=prow)
        sg, cg = sel.cpu().numpy(), cnt.cpu().numpy()
        for r in prow:
            b, hh = divmod(r, Hq)
            npg = (int(h["seq_lens"][b]) + P - 1) // P
            if policy == "gauss":
                m = gauss_keep_margin(bo[b, hh], mo[b, hh], vo[b, hh], npg, float(to[b, hh]), wl.delta)
            else:
                m = topk_gap(bo[b, hh], npg, wl.topk)
            log_margin(wl.name, policy + " keep", r, m)
        bad = sets_equal(sg, cg, so, co, rows=set(prow))
        assert bad == [], f"{policy} page sets differ from the oracle chain: {bad[:4]}"
        for alpha in wl.alphas:
            out = t.full((B, Hq, d), np.nan, device="cuda")
            tau = t.full((B, Hq), np.nan, dtype=t.float64, device="cuda")
            w = t.full((B, Hq, MP * P), np.nan, device="cuda")
            E.entmax_decode_sparse(full["shape"], inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                   sel, cnt, alpha, out, tau=tau, weights_out=w)
            oo, tdo, wo = oracle.entmax_decode(osh, h["q"], h["k_pool"], h["v_pool"], h["page_table"], h["seq_lens"],
                                               alpha, so, co, rows=prow, want_weights=True)
            og = _take_rows(out.cpu().numpy(), prow)
            tg = tau.cpu().numpy().reshape(-1)[prow]
            wg = w.view(B * Hq, -1)[prow].cpu().numpy()
            assert np.allclose(tg, tdo.reshape(-1)[prow], rtol=1e-12, atol=1e-12), "decode tau"
            assert np.array_equal(wg > 0, _take_rows(wo, prow) > 0), "support differs"
            assert np.max(np.abs(wg - _take_rows(wo, prow))) < 1e-5
            assert rel_l2_rows(og, _take_rows(oo, prow)) <= TOL[inp.dtype]
            for r in prow:
                b, hh = divmod(r, Hq)
                m = support_margin(h["q"][b, hh], h["k_pool"], hh // G, h["page_table"][b], int(h["seq_lens"][b]),
                                   P, so[b, hh], int(co[b, hh]), float(tdo[b, hh]), scale, inp.dtype)
                log_margin(wl.name, f"support a={alpha}", r, m)
            checked += len(prow)
    assert checked > 0
