"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP library through its binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np

import oracle
import sparse_decode_attention_page_amd as E
from sparse_decode_attention_page_amd import synth


def torch():
    import torch as _t
    return _t


def dev(a, kind):
    """numpy -> device tensor; kind in {"kv_bf16", "kv_f32", "i32", "u8", "f32", "f64"}."""
    t = torch()
    a = np.ascontiguousarray(a)
    if kind == "kv_bf16":
        return t.from_numpy(a.view(np.int16)).view(t.bfloat16).cuda()
    if kind == "kv_f32":
        return t.from_numpy(a.astype(np.float32)).cuda()
    if kind == "i32":
        return t.from_numpy(a.astype(np.int32)).cuda()
    if kind == "u8":
        return t.from_numpy(a.astype(np.uint8)).cuda()
    if kind == "f32":
        return t.from_numpy(a.astype(np.float32)).cuda()
    return t.from_numpy(a.astype(np.float64)).cuda()


def host_raw(x, dtype):
    """device KV-dtype tensor -> numpy raw storage (uint16 bits for bf16)."""
    t = torch()
    if dtype == "bf16":
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


class Dev:
    """Device copy of a synth.Inputs instance."""

    def __init__(self, inp: synth.Inputs, scale=0.0):
        t = torch()
        self.inp = inp
        kind = "kv_bf16" if inp.dtype == "bf16" else "kv_f32"
        self.kind = kind
        self.q = dev(inp.q, kind)
        self.k = dev(inp.k_pool, kind)
        self.v = dev(inp.v_pool, kind)
        self.pt = dev(inp.page_table, "i32")
        self.sl = dev(inp.seq_lens, "i32")
        self.shape = E.make_shape(self.q, self.k, self.pt, scale)
        self.oshape = oracle.Shape(inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages, inp.num_phys,
                                   inp.dtype, scale)
        self.kv_dtype = t.bfloat16 if inp.dtype == "bf16" else t.float32

    def zeros_meta(self):
        t = torch()
        i = self.inp
        return t.zeros((i.num_phys, i.Hkv, 4, i.d), dtype=self.kv_dtype, device="cuda")

    def per_page(self, fill=np.nan, dtype=None):
        t = torch()
        i = self.inp
        return t.full((i.B, i.Hq, i.max_pages), fill, dtype=dtype or t.float32, device="cuda")

    def sel_buffers(self):
        t = torch()
        i = self.inp
        return (t.full((i.B, i.Hq, i.max_pages), -1, dtype=t.int32, device="cuda"),
                t.full((i.B, i.Hq), -1, dtype=t.int32, device="cuda"))


TOL = {"bf16": 2e-3, "f32": 1e-5}


def decode_check(inp, D, alpha, sel_o, cnt_o, full=False, tau_method=0):
    """Run one entmax decode call and compare out, tau, support and weights with the oracle."""
    t = torch()
    out = t.full((inp.B, inp.Hq, inp.d), np.nan, dtype=t.float32, device="cuda")
    tau = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
    w = t.full((inp.B, inp.Hq, inp.max_pages * inp.P), np.nan, dtype=t.float32, device="cuda")
    if full:
        E.entmax_decode_full(D.shape, D.q, D.k, D.v, D.pt, D.sl, alpha, out, tau=tau, weights_out=w,
                             tau_method=tau_method)
        oo, to, wo = oracle.entmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table,
                                          inp.seq_lens, alpha, want_weights=True)
    else:
        E.entmax_decode_sparse(D.shape, D.q, D.k, D.v, D.pt, D.sl, t.from_numpy(sel_o).cuda(),
                               t.from_numpy(cnt_o).cuda(), alpha, out, tau=tau, weights_out=w,
                               tau_method=tau_method)
        oo, to, wo = oracle.entmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table,
                                          inp.seq_lens, alpha, sel_o, cnt_o, want_weights=True)
    og, tg, wg = out.cpu().numpy(), tau.cpu().numpy(), w.cpu().numpy()
    assert np.allclose(tg, to, rtol=1e-12, atol=1e-12)
    assert np.array_equal(wg > 0, wo > 0), "support differs"
    assert np.max(np.abs(wg - wo)) < 1e-5
    assert rel_l2_rows(og, oo) <= TOL[inp.dtype]


def rel_l2_rows(a, b):
    """max over rows of ||a - b|| / ||b|| (rows = all but the last axis)."""
    a = np.asarray(a, np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, np.float64).reshape(-1, np.shape(b)[-1])
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def sets_equal(sel_a, cnt_a, sel_b, cnt_b, rows=None):
    """Compare two (sel_idx, sel_cnt) pairs row by row; returns list of mismatching rows."""
    bad = []
    B, Hq = cnt_b.shape
    for b in range(B):
        for h in range(Hq):
            r = b * Hq + h
            if rows is not None and r not in rows:
                continue
            ca, cb = int(cnt_a[b, h]), int(cnt_b[b, h])
            if ca != cb or not np.array_equal(sel_a[b, h, :ca], sel_b[b, h, :cb]):
                bad.append((b, h, ca, cb))
    return bad


# Cut margins of the end-to-end comparisons: (workload, cut, row, margin)
# lines, printed in the terminal summary (tests/conftest.py).  A decision's
# margin is its distance from the cut relative to max(1, |cut|); margins below
# MARGIN_FLAG could flip under a last-bit difference of the threshold.
MARGIN_LOG: list = []
MARGIN_FLAG = 1e-12


def gauss_keep_margin(box, mu, var, n_pages, tau_hat, delta, n_sigma=3.0):
    """Smallest |min(mu + n_sigma sigma, box) - (tau_hat - delta)| over a row's valid pages."""
    bx = np.asarray(box[:n_pages], np.float64)
    m = np.asarray(mu[:n_pages], np.float64)
    v = np.asarray(var[:n_pages], np.float64)
    ok = np.isfinite(bx) & np.isfinite(m) & np.isfinite(v)
    if not ok.any() or not np.isfinite(tau_hat):
        return np.inf
    est = np.minimum(m[ok] + n_sigma * np.sqrt(np.maximum(v[ok], 0.0)), bx[ok])
    thr = tau_hat - delta
    return float(np.min(np.abs(est - thr)) / max(1.0, abs(thr)))


def topk_gap(box, n_pages, k):
    """Relative gap between the k-th and (k+1)-th largest box of a row (inf when every page is kept);
    ties are decided by page index on both sides, so a zero gap is not a risk."""
    if n_pages <= k:
        return np.inf
    b = np.asarray(box[:n_pages], np.float64)
    b = np.sort(np.where(np.isnan(b), -np.inf, b))[::-1]
    return float((b[k - 1] - b[k]) / max(1.0, abs(b[k - 1])))


def support_margin(q_row, k_pool, g, page_table_row, seq_len, P, sel_row, cnt, tau, scale, dtype):
    """Smallest |s_t - tau| (score units) over the tokens of a row's kept pages (KV head g)."""
    if cnt <= 0 or not np.isfinite(tau):
        return np.inf
    qf = synth.storage_to_f64(q_row, dtype)
    worst = np.inf
    for p in sel_row[:cnt]:
        n = min(P, seq_len - int(p) * P)
        kf = synth.storage_to_f64(k_pool[int(page_table_row[p]), g][:n], dtype)  # [n, d]
        s = scale * (kf @ qf)
        worst = min(worst, float(np.min(np.abs(s - tau))))
    return worst / max(1.0, abs(tau))


def log_margin(workload, cut, row, margin):
    flag = "  << below %.0e" % MARGIN_FLAG if margin < MARGIN_FLAG else ""
    MARGIN_LOG.append(f"{workload:18s} {cut:14s} row {row:5d}  margin {margin:.3e}{flag}")
