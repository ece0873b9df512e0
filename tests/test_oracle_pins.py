"""Pins for the CPU oracle against facts fixed outside the oracle itself.

Every test here runs on the CPU.  Each pin is chosen so that a plausible mistake in
the oracle (a dropped term, a wrong sign or index, a transposed operand, a wrong
rounding) fails at least one of them:

* Gauss-Hermite rule  -> numpy.polynomial.hermite.hermgauss and the Gaussian moments
* storage roundings    -> brute force over the neighbouring representable values
* page metadata        -> numpy min/max and exact rational mean/variance
* FP8 E4M3 codec       -> torch.float8_e4m3fn for every code, brute-force nearest
                          with ties to even for the encoder
* page scores          -> brute-force token scores (upper bound, equality cases,
                          mean identity, one-coordinate variance identity)
* top-k                -> numpy lexsort
* Gaussian selector    -> polynomial regime closed forms, the sigma = 0 reduction to
                          the exact token entmax, keep-rule invariants
* entmax threshold     -> sparsemax / 1.5-entmax sort closed forms (golden file),
                          softmax limit, support containment and the 2*B*delta bound
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from sparse_decode_attention_page_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def shape_of(inp, orc):
    return orc.Shape(inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages, inp.num_phys, inp.dtype)


def f64(a, dtype):
    return synth.storage_to_f64(a, dtype)


# --------------------------------------------------------------------------- GH16
def test_gauss_hermite_vs_numpy(orc):
    x, w = orc.gauss_hermite16()
    xn, wn = np.polynomial.hermite.hermgauss(16)
    assert np.max(np.abs(x - xn)) < 1e-13
    assert np.max(np.abs(w - wn) / wn) < 1e-11
    # exact for polynomials of degree <= 31: int x^(2k) e^{-x^2} = Gamma(k + 1/2)
    for k in range(16):
        assert math.isclose(np.sum(w * x ** (2 * k)), math.gamma(k + 0.5), rel_tol=1e-12)
        assert abs(np.sum(w * x ** (2 * k + 1))) < 1e-9 * math.gamma(k + 1)


# --------------------------------------------------------------------- roundings
def _bf16_neighbours(x):
    """Exact RNE to bf16 by brute force over representable neighbours."""
    f = np.float32(x)
    bits = int(np.array(f).view(np.uint32)) & 0xFFFF0000
    cands = []
    for delta in (-0x10000, 0, 0x10000, 0x20000):
        b = (bits + delta) & 0xFFFFFFFF
        v = np.array(b, dtype=np.uint32).view(np.float32)
        if np.isfinite(v):
            cands.append(float(v))
    X = Fraction(x)
    best = min(cands, key=lambda c: (abs(Fraction(c) - X),
                                     (int(np.array(np.float32(c)).view(np.uint32)) >> 16) & 1))
    return best


def test_round_bf16_brute_force(orc):
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(400) * 10.0 ** rng.integers(-30, 30, 400))
    # exact ties: halfway between two bf16 values (ties-to-even either way)
    vals += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(2.0 + 2.0 ** -7), 3.0 * 2.0 ** -130]
    vals += [2.0 ** -133 * 0.5, 2.0 ** -133 * 1.5, 1e-40, -1e-39]
    for v in vals:
        got = orc.round_bf16(v)
        assert got == _bf16_neighbours(v), v
    assert orc.round_bf16(3.5e38) == math.inf
    assert orc.round_bf16(1.0 + 2.0 ** -8) == 1.0          # tie -> even
    assert orc.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_round_f32_up(orc):
    rng = np.random.default_rng(6)
    for v in list(rng.standard_normal(300) * 10.0 ** rng.integers(-20, 20, 300)) + [0.1, -0.1, -1e-50]:
        r = orc.round_f32_up(v)
        assert r >= v and np.float32(r) == r
        below = float(np.nextafter(np.float32(r), np.float32(-np.inf)))
        assert below < v
    assert orc.round_f32_up(1.0) == 1.0


# ---------------------------------------------------------------- page metadata
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_build_page_meta_definitions(orc, dtype):
    inp = synth.random_small(1, B=2, Hq=2, Hkv=2, d=64, P=16, dtype=dtype, ctx=(53, 16))
    sh = shape_of(inp, orc)
    # garbage in the unfilled tail slots must not leak into the statistics
    k = inp.k_pool.copy()
    kf = f64(k, dtype)
    for b in range(inp.B):
        L = int(inp.seq_lens[b])
        last = (L - 1) // inp.P
        n = L - last * inp.P
        if n < inp.P:
            phys = inp.page_table[b, last]
            big = synth._store(np.full((inp.P - n, inp.d), 1e4, np.float32), dtype)
            k[phys, :, n:, :] = big
    meta = orc.build_page_meta(sh, k, inp.page_table, inp.seq_lens)
    mf = f64(meta, dtype)
    rnd = (lambda v: float(np.float32(v))) if dtype == "f32" else orc.round_bf16
    for b in range(inp.B):
        L = int(inp.seq_lens[b])
        for p in range((L + inp.P - 1) // inp.P):
            phys = inp.page_table[b, p]
            n = min(inp.P, L - p * inp.P)
            for g in range(inp.Hkv):
                toks = kf[phys, g, :n, :]
                assert np.array_equal(mf[phys, g, 0], toks.min(axis=0))
                assert np.array_equal(mf[phys, g, 1], toks.max(axis=0))
                for i in range(0, inp.d, 7):
                    col = [Fraction(float(t)) for t in toks[:, i]]
                    mean = sum(col) / n
                    var = sum(c * c for c in col) / n - mean * mean
                    assert mf[phys, g, 2, i] == rnd(float(mean))
                    assert abs(mf[phys, g, 3, i] - rnd(float(max(var, 0)))) <= 4e-16 * float(
                        sum(c * c for c in col) / n) + 1e-300
                # population variance (ddof = 0)
                npv = toks.var(axis=0)
                tol = (1e-6 if dtype == "f32" else 8e-3) * np.maximum(npv, 1e-30) + 1e-12
                assert np.all(np.abs(mf[phys, g, 3] - npv) <= tol)


# ------------------------------------------------------------ compact metadata
def _e4m3_table():
    import torch
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_decode_vs_torch(orc):
    tab = _e4m3_table()
    got = np.array([orc.e4m3_decode(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(tab))
    ok = ~np.isnan(tab)
    assert np.array_equal(got[ok], tab[ok])
    assert orc.e4m3_decode(0x7E) == 448.0 and orc.e4m3_decode(0x01) == 2.0 ** -9


def _e4m3_nearest(x, tab):
    """Brute force: nearest finite code, ties to the even code, +-448 saturation."""
    if math.isnan(x):
        return 0x7F
    sgn = 0x80 if math.copysign(1.0, x) < 0 else 0
    a = abs(x)
    pos = [(c, tab[c]) for c in range(0x7F)]  # 0x00 .. 0x7E, finite, non-negative
    best = min(pos, key=lambda cv: (abs(cv[1] - a), cv[0] & 1))
    return sgn | best[0]


def test_e4m3_encode_brute_force(orc):
    tab = _e4m3_table()
    rng = np.random.default_rng(3)
    xs = list(np.exp(rng.uniform(np.log(2.0 ** -13), np.log(600.0), 400)) * rng.choice([-1.0, 1.0], 400))
    fin = [tab[c] for c in range(0x7F)]
    xs += fin + [-v for v in fin]
    xs += [(a + b) / 2 for a, b in zip(fin[:-1], fin[1:])]          # every tie
    xs += [np.nextafter((a + b) / 2, 0) for a, b in zip(fin[:-1], fin[1:])]
    xs += [0.0, -0.0, 447.9, 448.0, 463.9, 464.0, 1e9, -1e9, 2.0 ** -10, 3 * 2.0 ** -10, float("nan")]
    for x in xs:
        assert orc.e4m3_encode(float(x)) == _e4m3_nearest(float(x), tab), x


def test_e4m3_encode_vs_torch_cast(orc):
    import torch
    rng = np.random.default_rng(4)
    x = (np.exp(rng.uniform(np.log(2.0 ** -12), np.log(440.0), 3000)) * rng.choice([-1.0, 1.0], 3000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([orc.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_build_page_meta_f8_definitions(orc):
    inp = synth.random_small(5, B=2, Hq=2, Hkv=2, d=64, P=16, dtype="bf16", ctx=(53, 16))
    sh = shape_of(inp, orc)
    meta4 = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    m8 = orc.build_page_meta_f8(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    assert m8.shape == (inp.num_phys, inp.Hkv, 6 * inp.d) and m8.dtype == np.uint8
    tab = _e4m3_table()
    kf = f64(inp.k_pool, "bf16")
    d = inp.d
    for b in range(inp.B):
        L = int(inp.seq_lens[b])
        for p in range((L + inp.P - 1) // inp.P):
            phys = inp.page_table[b, p]
            n = min(inp.P, L - p * inp.P)
            for g in range(inp.Hkv):
                rec = m8[phys, g]
                # bounds: the same bf16 bits as the four-row record
                assert np.array_equal(rec[:4 * d].view(np.uint16), meta4[phys, g, :2].reshape(-1))
                toks = kf[phys, g, :n, :]
                for i in range(d):
                    col = [Fraction(float(t)) for t in toks[:, i]]
                    mean = sum(col) / n
                    var = max(sum(c * c for c in col) / n - mean * mean, Fraction(0))
                    assert rec[4 * d + i] == _e4m3_nearest(float(mean), tab)
                    assert rec[5 * d + i] == _e4m3_nearest(float(var), tab)


def test_score_pages_f8_definitions(orc):
    inp = synth.random_small(6, B=2, Hq=4, Hkv=2, d=64, P=16, dtype="bf16", ctx=(300, 77))
    sh = shape_of(inp, orc)
    meta4 = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    m8 = orc.build_page_meta_f8(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box4, _, _ = orc.score_pages(sh, inp.q, meta4, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages_f8(sh, inp.q, m8, inp.page_table, inp.seq_lens)
    tab = _e4m3_table()
    qf = f64(inp.q, "bf16")
    c = 1.0 / math.sqrt(inp.d)
    G, d = inp.Hq // inp.Hkv, inp.d
    for b in range(inp.B):
        npg = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        # the box reads the same bounds as the four-row record
        assert np.array_equal(box[b, :, :npg], box4[b, :, :npg])
        for h in range(inp.Hq):
            q = qf[b, h]
            for p in range(npg):
                rec = m8[inp.page_table[b, p], h // G]
                mean, vv = tab[rec[4 * d:5 * d]], tab[rec[5 * d:6 * d]]
                # exact sums of exact products, rounded once
                m_exact = math.fsum(float(x) for x in q * mean)
                v_exact = math.fsum(float(x) for x in (q * q) * vv)
                for got, want in ((mu[b, h, p], np.float32(c * m_exact)), (var[b, h, p], np.float32(c * c * v_exact))):
                    ulp = abs(int(np.array(got).view(np.int32)) - int(np.array(want).view(np.int32)))
                    assert ulp <= 1, (b, h, p, got, want)


def test_build_page_meta_from_token(orc):
    inp = synth.random_small(2, B=2, Hq=2, Hkv=1, d=64, P=16, dtype="bf16", ctx=(100, 40))
    sh = shape_of(inp, orc)
    full = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    sentinel = np.full_like(full, 0x7F7F)
    part = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens,
                               from_token=np.array([70, 0], np.int32), meta=sentinel.copy())
    # b=0: pages 4..6 rebuilt (tokens >= 70 live in page 70 // 16 = 4 onwards); b=1: all
    for p in range(7):
        phys = inp.page_table[0, p]
        want = full[phys] if p >= 4 else sentinel[phys]
        assert np.array_equal(part[phys], want), p
    for p in range(3):
        assert np.array_equal(part[inp.page_table[1, p]], full[inp.page_table[1, p]])


# ---------------------------------------------------------------- page scoring
def _token_scores(inp, b, h, p):
    G = inp.Hq // inp.Hkv
    phys = inp.page_table[b, p]
    n = min(inp.P, int(inp.seq_lens[b]) - p * inp.P)
    K = f64(inp.k_pool[phys, h // G, :n], inp.dtype)
    q = f64(inp.q[b, h], inp.dtype)
    return (K @ q) / math.sqrt(inp.d)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_box_is_upper_bound_and_exact_for_single_token(orc, dtype):
    # ctx 81 = 5 full pages + a one-token page
    inp = synth.random_small(3, B=1, Hq=4, Hkv=2, d=64, P=16, dtype=dtype, ctx=(81,))
    sh = shape_of(inp, orc)
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    for h in range(inp.Hq):
        for p in range(6):
            s = _token_scores(inp, 0, h, p)
            assert box[0, h, p] >= s.max()
        # one-token page: k_min = k_max = k, so the bound is the score itself (rounded up)
        s = _token_scores(inp, 0, h, 5)
        assert len(s) == 1
        assert box[0, h, 5] == orc.round_f32_up(float(s[0]))
        assert mu[0, h, 5] == np.float32(s[0]) or abs(mu[0, h, 5] - s[0]) < 1e-2 * (dtype == "bf16")
        if dtype == "f32":
            assert var[0, h, 5] == 0.0


def test_mu_is_mean_score_and_var_one_coordinate(orc):
    # fp32 storage keeps mean/var nearly exact, so the identities can be checked tightly
    inp = synth.random_small(4, B=1, Hq=2, Hkv=1, d=64, P=16, dtype="f32", ctx=(64,))
    # page 1: keys that differ only in coordinate 3 -> the diagonal model is exact
    base = np.random.default_rng(0).standard_normal(64).astype(np.float32)
    for j in range(16):
        row = base.copy()
        row[3] = np.float32(j * 0.37 - 2.0)
        inp.k_pool[inp.page_table[0, 1], 0, j] = row
    sh = shape_of(inp, orc)
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    for h in range(2):
        for p in range(4):
            s = _token_scores(inp, 0, h, p)
            assert abs(mu[0, h, p] - s.mean()) < 1e-5
        s = _token_scores(inp, 0, h, 1)
        assert abs(var[0, h, 1] - s.var()) < 1e-5 * s.var()
        # a page with generic keys: sigma^2 is the diagonal part, below the true variance only by
        # the off-diagonal covariance; it must match sum_i q_i^2 var_i / d
        q = f64(inp.q[0, h], "f32")
        K = f64(inp.k_pool[inp.page_table[0, 2], 0], "f32")
        assert abs(var[0, h, 2] - np.sum(q * q * K.var(axis=0)) / 64) < 1e-5


def test_score_rows_subset_matches_full(orc):
    inp = synth.random_small(5, B=2, Hq=4, Hkv=2, dtype="bf16", ctx=(90, 33))
    sh = shape_of(inp, orc)
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    a = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    b = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens, rows=[5, 2])
    for x, y in zip(a, b):
        assert np.array_equal(x[1, 1], y[1, 1], equal_nan=True)
        assert np.array_equal(x[0, 2], y[0, 2], equal_nan=True)


# ------------------------------------------------------------------------ top-k
def test_topk_vs_lexsort(orc):
    rng = np.random.default_rng(7)
    B, Hq, mp = 2, 3, 50
    sh = orc.Shape(B, Hq, 1, 64, 16, mp, 100, "bf16")
    box = rng.standard_normal((B, Hq, mp)).astype(np.float32)
    box[0, 0, 10:20] = 0.5                   # ties
    box[0, 1, 5] = np.nan
    box[1, 2, :] = -0.0
    box[1, 2, ::3] = 0.0
    seq = np.array([16 * 50, 16 * 37 - 5], np.int32)
    for k in (1, 7, 37, 64):
        sel, cnt = orc.select_topk(sh, box, seq, k)
        for b in range(B):
            npg = (int(seq[b]) + 15) // 16
            for h in range(Hq):
                key = np.where(np.isnan(box[b, h, :npg]), -np.inf, box[b, h, :npg]).astype(np.float64)
                order = np.lexsort((np.arange(npg), -key))
                want = np.sort(order[:min(k, npg)])
                assert cnt[b, h] == len(want)
                assert np.array_equal(sel[b, h, :cnt[b, h]], want)


def test_topk_group_vs_lexsort_of_head_max(orc):
    rng = np.random.default_rng(17)
    B, Hkv, G, mp = 2, 2, 3, 40
    sh = orc.Shape(B, Hkv * G, Hkv, 64, 16, mp, 100, "bf16")
    box = rng.standard_normal((B, Hkv * G, mp)).astype(np.float32)
    box[0, 0:3, 10:20] = 0.5                    # ties across pages
    box[0, 1, 5] = np.nan                       # one head's NaN: the others decide
    box[1, 3:6, 7] = np.nan                     # every head NaN: ranks last
    seq = np.array([16 * 40, 16 * 31 - 5], np.int32)
    for k in (1, 6, 31, 64):
        sel, cnt = orc.select_topk_group(sh, box, seq, k)
        assert sel.shape == (B, Hkv, mp)
        for b in range(B):
            npg = (int(seq[b]) + 15) // 16
            for g in range(Hkv):
                blk = box[b, g * G:(g + 1) * G, :npg].astype(np.float64)
                key = np.where(np.isnan(blk), -np.inf, blk).max(axis=0)
                order = np.lexsort((np.arange(npg), -key))
                want = np.sort(order[:min(k, npg)])
                assert cnt[b, g] == len(want)
                assert np.array_equal(sel[b, g, :cnt[b, g]], want)


def test_group_selection_reduces_to_per_head_for_one_head_groups(orc):
    inp = synth.random_small(8, B=2, Hq=3, Hkv=3, d=64, P=16, dtype="bf16", ctx=(900, 333), planted_per_kv=3)
    sh = shape_of(inp, orc)
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    s1, c1 = orc.select_topk(sh, box, inp.seq_lens, 9)
    s2, c2 = orc.select_topk_group(sh, box, inp.seq_lens, 9)
    assert np.array_equal(c1, c2) and all(np.array_equal(s1[b, h, :c1[b, h]], s2[b, h, :c2[b, h]])
                                          for b in range(2) for h in range(3))
    s1, c1, t1 = orc.select_gauss(sh, box, mu, var, inp.seq_lens, 1.5, 0.5)
    s2, c2, t2 = orc.select_gauss_group(sh, box, mu, var, inp.seq_lens, 1.5, 0.5)
    assert np.array_equal(c1, c2) and np.array_equal(t1, t2)
    assert all(np.array_equal(s1[b, h, :c1[b, h]], s2[b, h, :c2[b, h]]) for b in range(2) for h in range(3))


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_gauss_group_is_union_and_discards_less(orc, alpha):
    inp = synth.random_small(9, B=2, Hq=8, Hkv=2, d=64, P=16, dtype="bf16", ctx=(2000, 700), planted_per_kv=8)
    sh = shape_of(inp, orc)
    G = inp.Hq // inp.Hkv
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    sh_, ch_, th_ = orc.select_gauss(sh, box, mu, var, inp.seq_lens, alpha, 0.0)
    sg, cg, tg = orc.select_gauss_group(sh, box, mu, var, inp.seq_lens, alpha, 0.0)
    assert np.array_equal(th_, tg)
    _, _, wfull = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, alpha,
                                    want_weights=True)
    P = inp.P
    for b in range(inp.B):
        for g in range(inp.Hkv):
            gset = set(sg[b, g, :cg[b, g]].tolist())
            heads = [set(sh_[b, g * G + j, :ch_[b, g * G + j]].tolist()) for j in range(G)]
            assert gset == set().union(*heads)
            assert sg[b, g, :cg[b, g]].tolist() == sorted(gset)
            for j in range(G):
                h = g * G + j
                w = wfull[b, h]
                out_own = sum(w[p * P:(p + 1) * P].sum() for p in range(len(w) // P) if p not in heads[j])
                out_grp = sum(w[p * P:(p + 1) * P].sum() for p in range(len(w) // P) if p not in gset)
                assert out_grp <= out_own + 1e-15   # a superset of the kept pages discards less mass
    # decoding over the group set is decoding each head over the expanded selection
    se, ce = orc.expand_group_selection(sh, sg, cg)
    assert se.shape == (inp.B, inp.Hq, inp.max_pages) and np.array_equal(ce[:, :G], np.repeat(cg[:, :1], G, 1))


# ------------------------------------------------------------ Gaussian selector
def test_gauss_polynomial_regime_closed_form(orc):
    # every quadrature node above tau: the rule is exact for the polynomial integrand
    # alpha=1.5 (beta=2): E[(aS - tau)^2] = (a mu - tau)^2 + a^2 sigma^2
    mu = np.array([0.3, 0.1], np.float32)
    var = np.array([0.01, 0.0025], np.float32)
    n = np.array([4, 3], np.int32)
    a = 0.5
    for tau in (-2.0, -1.5):
        want = sum(int(n[p]) * ((a * float(mu[p]) - tau) ** 2 + a * a * float(var[p])) for p in range(2))
        assert math.isclose(orc.gauss_mass(mu, var, n, 1.5, tau), want, rel_tol=1e-13)
    # alpha=2 (beta=1): E[S - tau] = mu - tau
    for tau in (-1.0, -0.7):
        want = sum(int(n[p]) * (float(mu[p]) - tau) for p in range(2))
        assert math.isclose(orc.gauss_mass(mu, var, n, 2.0, tau), want, rel_tol=1e-13)


def _row_shape(orc, npg, P):
    return orc.Shape(1, 1, 1, 64, P, npg, npg, "f32")


def test_gauss_tau_polynomial_regime_root(orc):
    # one page, n = 4, sigma = 0.1, alpha = 1.5: root of 4[(a mu - t)^2 + a^2 s^2] = 1
    mu = np.array([[[0.8]]], np.float32)
    var = np.array([[[0.01]]], np.float32)
    box = np.array([[[5.0]]], np.float32)
    sh = _row_shape(orc, 1, 4)
    sel, cnt, tau = orc.select_gauss(sh, box, mu, var, np.array([4], np.int32), 1.5, 0.0)
    a = 0.5
    root_x = a * float(mu.ravel()[0]) - math.sqrt(0.25 - a * a * float(var.ravel()[0]))
    assert abs(tau[0, 0] - root_x / a) < 1e-13
    # alpha = 2: 4 (mu - t) = 1 (sigma = 0.01 keeps every node above the root)
    var = np.array([[[1e-4]]], np.float32)
    sel, cnt, tau = orc.select_gauss(sh, box, mu, var, np.array([4], np.int32), 2.0, 0.0)
    assert abs(tau[0, 0] - (float(mu.ravel()[0]) - 0.25)) < 1e-13


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.3])
def test_gauss_sigma_zero_reduces_to_token_entmax(orc, alpha):
    # sigma_p = 0: each page is n_p tokens of score mu_p and F is the exact token mass
    rng = np.random.default_rng(8)
    npg, P = 40, 8
    mu = rng.standard_normal(npg).astype(np.float32)
    var = np.zeros(npg, np.float32)
    L = npg * P - 3
    fills = [min(P, L - p * P) for p in range(npg)]
    tokens = np.concatenate([[float(mu[p])] * fills[p] for p in range(npg)])
    tau_tok = orc.entmax_tau(tokens, alpha)
    sh = _row_shape(orc, npg, P)
    sel, cnt, tau = orc.select_gauss(sh, (mu + 10).reshape(1, 1, -1), mu.reshape(1, 1, -1),
                                     var.reshape(1, 1, -1), np.array([L], np.int32), alpha, 0.0)
    assert abs(tau[0, 0] - tau_tok) < 1e-12 * max(1.0, abs(tau_tok))
    # Delta = 0, est = mu: keep exactly the pages holding support tokens (mu > tau) or ties
    kept = set(sel[0, 0, :cnt[0, 0]].tolist())
    assert kept == {p for p in range(npg) if mu[p] >= tau[0, 0]}


def test_gauss_keep_rule_properties(orc):
    inp = synth.random_small(9, B=1, Hq=2, Hkv=1, d=64, P=16, dtype="bf16", ctx=(2000,))
    sh = shape_of(inp, orc)
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    npg = 125
    for alpha in (1.5, 2.0):
        prev = None
        for delta in (0.0, 0.25, 0.5, 2.0, 100.0):
            sel, cnt, tau = orc.select_gauss(sh, box, mu, var, inp.seq_lens, alpha, delta)
            for h in range(2):
                kept = set(sel[0, h, :cnt[0, h]].tolist())
                thr = tau[0, h] - delta
                est = np.minimum(mu[0, h, :npg].astype(np.float64) + 3 * np.sqrt(var[0, h, :npg].astype(np.float64)),
                                 box[0, h, :npg].astype(np.float64))
                want = {p for p in range(npg) if est[p] >= thr - 1e-12}
                maybe = {p for p in range(npg) if abs(est[p] - thr) < 1e-12}
                if want:
                    assert kept - maybe == want - maybe
                else:
                    assert kept == {int(np.argmax(est))}
                assert list(sel[0, h, :cnt[0, h]]) == sorted(kept)
                # F(tau_hat) >= 1 > F(tau_hat + eps): tau_hat is the bisection limit
                n = np.full(npg, 16, np.int32)
                tx = tau[0, h] * (alpha - 1)
                assert orc.gauss_mass(mu[0, h, :npg], var[0, h, :npg], n, alpha, tx) >= 1.0
                assert orc.gauss_mass(mu[0, h, :npg], var[0, h, :npg], n, alpha, tx + 1e-9) < 1.0
            if prev is not None:  # larger Delta keeps a superset
                for h in range(2):
                    assert set(prev[0, h, :pcnt[0, h]]) <= set(sel[0, h, :cnt[0, h]])
            prev, pcnt = sel, cnt
        assert all(cnt[0, h] == npg for h in range(2))  # Delta = 100 keeps everything


# ---------------------------------------------------------- entmax threshold
def test_entmax_closed_form_golden(orc):
    gold = json.load(open(os.path.join(GOLD, "entmax_closed_forms.json")))
    for c in gold["cases"]:
        s = np.array(c["scores"], np.float64)
        tau = orc.entmax_tau(s, c["alpha"])
        assert abs(tau - c["tau"]) < 1e-14, c
        a = c["alpha"] - 1
        p = np.maximum(a * s - a * tau, 0) ** (1 / a)
        assert np.allclose(p, c["p"], atol=1e-14)


def _sparsemax_tau(z):
    zs = np.sort(z)[::-1]
    cs = np.cumsum(zs)
    k = np.arange(1, len(z) + 1)
    kstar = k[1 + k * zs > cs].max()
    return (cs[kstar - 1] - 1) / kstar


def _entmax15_tau_sort(z):
    x = np.sort(z / 2)[::-1]
    best = None
    for k in range(1, len(x) + 1):
        m = x[:k].mean()
        ss = np.sum((x[:k] - m) ** 2)
        if ss > 1:
            break
        t = m - math.sqrt((1 - ss) / k)
        if t <= x[k - 1]:
            best = t
    return best * 2  # score units


@pytest.mark.parametrize("seed", range(6))
def test_entmax_tau_vs_sort_forms(orc, seed):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(50 + 40 * seed) * (0.5 + seed)
    assert abs(orc.entmax_tau(z, 2.0) - _sparsemax_tau(z)) < 1e-13 * max(1, abs(_sparsemax_tau(z)))
    t15 = _entmax15_tau_sort(z)
    assert abs(orc.entmax_tau(z, 1.5) - t15) < 1e-13 * max(1, abs(t15))


def test_entmax_near_one_is_softmax(orc):
    z = np.random.default_rng(1).standard_normal(30)
    inp_tau = orc.entmax_tau(z, 1.0005)
    a = 0.0005
    p = np.maximum(a * z - a * inp_tau, 0) ** (1 / a)
    p /= p.sum()
    assert np.max(np.abs(p - scipy.special.softmax(z))) < 2e-3


def _decode_inputs(orc, seed=11, dtype="bf16", ctx=(700, 333), alpha=1.5):
    inp = synth.random_small(seed, B=2, Hq=4, Hkv=2, d=64, P=16, dtype=dtype, ctx=ctx, planted_per_kv=6)
    return inp, shape_of(inp, orc)


@pytest.mark.parametrize("alpha", [1.5, 2.0, 1.25, 3.0])
def test_entmax_weights_and_output(orc, alpha):
    inp, sh = _decode_inputs(orc, alpha=alpha)
    out, tau, w = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                    alpha, want_weights=True)
    for b in range(inp.B):
        L = int(inp.seq_lens[b])
        for h in range(inp.Hq):
            s = np.concatenate([_token_scores(inp, b, h, p) for p in range((L + 15) // 16)])
            p = w[b, h, :L]
            assert abs(p.sum() - 1) < 1e-12 and np.all(p >= 0)
            assert np.all(w[b, h, L:] == 0)
            # p_t > 0 exactly when the score beats the threshold
            assert np.array_equal(p > 0, s > tau[b, h])
            if alpha == 2.0:
                assert abs(tau[b, h] - _sparsemax_tau(s)) < 1e-12
            if alpha == 1.5:
                assert abs(tau[b, h] - _entmax15_tau_sort(s)) < 1e-12
            # o = sum_t p_t v_t as a matrix product over the gathered V rows
            G = inp.Hq // inp.Hkv
            V = np.concatenate([f64(inp.v_pool[inp.page_table[b, pg], h // G,
                                               :min(16, L - pg * 16)], inp.dtype)
                                for pg in range((L + 15) // 16)])
            assert np.allclose(out[b, h], p @ V, atol=1e-12)


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_support_containment_is_exact(orc, alpha):
    # EntmaxKV summary section 3: S subset of I_keep  =>  delta = 0 and the sparse output is exact
    inp, sh = _decode_inputs(orc, seed=12)
    out, tau, w = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                    alpha, want_weights=True)
    sel = np.zeros((inp.B, inp.Hq, inp.max_pages), np.int32)
    cnt = np.zeros((inp.B, inp.Hq), np.int32)
    for b in range(inp.B):
        for h in range(inp.Hq):
            pages = sorted({t // 16 for t in np.nonzero(w[b, h])[0]})
            extra = [p for p in range((int(inp.seq_lens[b]) + 15) // 16) if p % 5 == 0]
            pages = sorted(set(pages) | set(extra))
            sel[b, h, :len(pages)] = pages
            cnt[b, h] = len(pages)
    o2, t2, w2 = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                   alpha, sel, cnt, want_weights=True)
    assert np.max(np.abs(o2 - out)) < 1e-12 * np.max(np.abs(out))
    assert np.max(np.abs(t2 - tau)) < 1e-12
    assert np.max(np.abs(w2 - w)) < 1e-12


@pytest.mark.parametrize("alpha", [1.5, 2.0])
def test_truncation_bound(orc, alpha):
    # ||o - o~|| <= 2 B delta (EntmaxKV summary section 3), and tau~ <= tau, p~ >= p on T
    inp, sh = _decode_inputs(orc, seed=13)
    out, tau, w = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                    alpha, want_weights=True)
    rng = np.random.default_rng(0)
    for trial in range(4):
        sel = np.zeros((inp.B, inp.Hq, inp.max_pages), np.int32)
        cnt = np.zeros((inp.B, inp.Hq), np.int32)
        for b in range(inp.B):
            npg = (int(inp.seq_lens[b]) + 15) // 16
            for h in range(inp.Hq):
                pages = np.sort(rng.choice(npg, size=max(1, npg // 3), replace=False))
                sel[b, h, :len(pages)] = pages
                cnt[b, h] = len(pages)
        o2, t2, w2 = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table,
                                       inp.seq_lens, alpha, sel, cnt, want_weights=True)
        G = inp.Hq // inp.Hkv
        for b in range(inp.B):
            L = int(inp.seq_lens[b])
            for h in range(inp.Hq):
                kept = np.zeros(inp.max_pages * 16, bool)
                for p in sel[b, h, :cnt[b, h]]:
                    kept[p * 16:(p + 1) * 16] = True
                kept[L:] = False
                delta = w[b, h][~kept].sum()
                V = np.stack([f64(inp.v_pool[inp.page_table[b, t // 16], h // G, t % 16], inp.dtype)
                              for t in range(L)])
                Bn = np.max(np.linalg.norm(V, axis=1))
                err = np.linalg.norm(out[b, h] - o2[b, h])
                assert err <= 2 * Bn * delta + 1e-12
                assert t2[b, h] <= tau[b, h] + 1e-15
                assert np.all(w2[b, h][kept] >= w[b, h][kept] - 1e-15)


def test_decode_rejects_bad_selection(orc):
    inp, sh = _decode_inputs(orc, seed=14)
    sel = np.zeros((inp.B, inp.Hq, inp.max_pages), np.int32)
    cnt = np.ones((inp.B, inp.Hq), np.int32) * 2
    sel[:, :, 0] = 3
    sel[:, :, 1] = 1  # not ascending
    out, tau, _ = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                    1.5, sel, cnt)
    assert np.all(np.isnan(out)) and np.all(np.isnan(tau))


# -------------------------------------------------------------------- softmax
def test_softmax_vs_scipy(orc):
    inp, sh = _decode_inputs(orc, seed=15, dtype="f32")
    out, lse = orc.softmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens)
    G = inp.Hq // inp.Hkv
    for b in range(inp.B):
        L = int(inp.seq_lens[b])
        for h in range(inp.Hq):
            s = np.concatenate([_token_scores(inp, b, h, p) for p in range((L + 15) // 16)])
            V = np.stack([f64(inp.v_pool[inp.page_table[b, t // 16], h // G, t % 16], "f32")
                          for t in range(L)])
            assert np.allclose(out[b, h], scipy.special.softmax(s) @ V, atol=1e-12)
            assert abs(lse[b, h] - scipy.special.logsumexp(s)) < 1e-12


def _some_selection(inp, seed, keep_frac=0.3):
    """A seeded selection: ascending kept pages per row, at least one page."""
    rng = np.random.default_rng(seed)
    sel = np.zeros((inp.B, inp.Hq, inp.max_pages), np.int32)
    cnt = np.zeros((inp.B, inp.Hq), np.int32)
    for b in range(inp.B):
        np_b = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        for h in range(inp.Hq):
            k = max(1, int(keep_frac * np_b))
            pages = np.sort(rng.choice(np_b, size=k, replace=False))
            sel[b, h, :k] = pages
            cnt[b, h] = k
    return sel, cnt


def test_softmax_over_selection_vs_scipy(orc):
    """Softmax over the kept pages only: scipy's softmax / logsumexp of the kept
    tokens' scores, the identity 1 - exp(lse_T - lse_full) = softmax mass of the
    discarded tokens (the discarded-mass notion of section 3), and a full
    selection reproducing the full-cache result."""
    inp, sh = _decode_inputs(orc, seed=16, dtype="f32")
    sel, cnt = _some_selection(inp, 16)
    out, lse = orc.softmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                  sel_idx=sel, sel_cnt=cnt)
    out_f, lse_f = orc.softmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens)
    G = inp.Hq // inp.Hkv
    for b in range(inp.B):
        L = int(inp.seq_lens[b])
        for h in range(inp.Hq):
            kept = sel[b, h, :cnt[b, h]]
            s = np.concatenate([_token_scores(inp, b, h, p) for p in kept])
            V = np.concatenate([f64(inp.v_pool[inp.page_table[b, p], h // G, :min(16, L - p * 16)], "f32")
                                for p in kept])
            assert np.allclose(out[b, h], scipy.special.softmax(s) @ V, atol=1e-12)
            assert abs(lse[b, h] - scipy.special.logsumexp(s)) < 1e-12
            s_all = np.concatenate([_token_scores(inp, b, h, p) for p in range((L + 15) // 16)])
            p_all = scipy.special.softmax(s_all)
            dropped = np.ones(len(s_all), bool)
            for p in kept:
                dropped[p * 16:min(L, (p + 1) * 16)] = False
            assert abs((1.0 - math.exp(lse[b, h] - lse_f[b, h])) - p_all[dropped].sum()) < 1e-12
    # every page kept: the full-cache softmax
    full_sel = np.zeros_like(sel)
    full_cnt = np.zeros_like(cnt)
    for b in range(inp.B):
        np_b = (int(inp.seq_lens[b]) + 15) // 16
        full_sel[b, :, :np_b] = np.arange(np_b)
        full_cnt[b, :] = np_b
    out_a, lse_a = orc.softmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                      sel_idx=full_sel, sel_cnt=full_cnt)
    assert np.array_equal(out_a, out_f) and np.array_equal(lse_a, lse_f)


def test_softmax_selection_edge_cases(orc):
    inp, sh = _decode_inputs(orc, seed=17)
    sel = np.zeros((inp.B, inp.Hq, inp.max_pages), np.int32)
    cnt = np.zeros((inp.B, inp.Hq), np.int32)
    cnt[0, 0] = 2
    sel[0, 0, :2] = [3, 1]           # not ascending -> NaN
    cnt[0, 1] = -1                   # negative count -> NaN
    cnt[1, 0] = 0                    # empty -> zeros, lse = -inf
    cnt[1, 1] = 1
    sel[1, 1, 0] = 10 ** 6           # page beyond N_b -> NaN
    out, lse = orc.softmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                  rows=[0, 1, 4, 5], sel_idx=sel, sel_cnt=cnt)
    assert np.all(np.isnan(out[0, 0])) and np.isnan(lse[0, 0])
    assert np.all(np.isnan(out[0, 1])) and np.isnan(lse[0, 1])
    assert np.all(out[1, 0] == 0.0) and lse[1, 0] == -np.inf
    assert np.all(np.isnan(out[1, 1])) and np.isnan(lse[1, 1])


def test_tiny_workload_end_to_end(orc):
    """The 4k-token fp32 workload: both selectors run and the sparse result obeys section 3."""
    inp = synth.make("tiny_4k", 0)
    sh = shape_of(inp, orc)
    meta = orc.build_page_meta(sh, inp.k_pool, inp.page_table, inp.seq_lens)
    box, mu, var = orc.score_pages(sh, inp.q, meta, inp.page_table, inp.seq_lens)
    of, tf, wf = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens,
                                   1.5, want_weights=True)
    support = set(np.nonzero(wf[0, 0])[0].tolist())
    planted = {t for (_, _, t) in inp.planted[0]}
    assert planted <= support
    for sel, cnt in (orc.select_topk(sh, box, inp.seq_lens, 32),
                     orc.select_gauss(sh, box, mu, var, inp.seq_lens, 1.5, 0.5)[:2]):
        os_, ts, ws = orc.entmax_decode(sh, inp.q, inp.k_pool, inp.v_pool, inp.page_table,
                                        inp.seq_lens, 1.5, sel, cnt, want_weights=True)
        kept = {t for p in sel[0, 0, :cnt[0, 0]] for t in range(p * 16, p * 16 + 16)}
        delta = sum(wf[0, 0, t] for t in support - kept)
        if support <= kept:
            assert np.max(np.abs(os_ - of)) < 1e-12
        else:
            assert delta > 0
