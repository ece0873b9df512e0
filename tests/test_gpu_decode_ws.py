"""Decode workspaces sized by a bound on the kept pages.

A workspace from decode_workspace_bytes(shape, call, n) holds n kept pages
summed over the query-head rows, laid out in row order.  With n = the total
kept pages every row matches the oracle; with less, the rows whose pages fit
still match and the others read NaN (out and tau)."""
import numpy as np
import pytest

import oracle
import sparse_decode_attention_page_amd as E
from gpu_util import TOL, Dev, rel_l2_rows, torch
from sparse_decode_attention_page_amd import synth

pytestmark = pytest.mark.gpu


def _sets(inp, rng):
    sel = np.full((inp.B, inp.Hq, inp.max_pages), -1, np.int32)
    cnt = np.zeros((inp.B, inp.Hq), np.int32)
    for b in range(inp.B):
        npg = (int(inp.seq_lens[b]) + inp.P - 1) // inp.P
        for h in range(inp.Hq):
            k = int(rng.integers(0, npg + 1))
            s = np.sort(rng.choice(npg, size=k, replace=False))
            sel[b, h, :k] = s
            cnt[b, h] = k
    return sel, cnt


@pytest.mark.parametrize("group", [False, True], ids=["per_head", "group"])
def test_decode_workspace_by_kept_pages(group):
    inp = synth.random_small(21, B=2, Hq=4, Hkv=2, d=64, P=16, dtype="bf16", ctx=(3000, 1700), planted_per_kv=4)
    D = Dev(inp)
    t = torch()
    rng = np.random.default_rng(4)
    G = inp.Hq // inp.Hkv
    if group:
        gs, gc = _sets(inp, rng)
        gs, gc = gs[:, :inp.Hkv].copy(), gc[:, :inp.Hkv].copy()
        sel, cnt = np.repeat(gs, G, axis=1), np.repeat(gc, G, axis=1)
        call, si, ci = E.CALL_DECODE_GROUP, gs, gc
    else:
        sel, cnt = _sets(inp, rng)
        call, si, ci = E.CALL_DECODE_SPARSE, sel, cnt
    oo, to, _ = oracle.entmax_decode(D.oshape, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, 1.5,
                                     sel, cnt)
    flat = cnt.reshape(-1).astype(np.int64)
    ends = np.cumsum(flat)
    total = int(ends[-1])
    checked_nan = False
    for cap in (total, total - 1, total - 40, int(ends[2]), 1):
        ws = E.workspace(D.shape, call, max_kept_pages=cap)
        assert ws.numel() == E.decode_workspace_bytes(D.shape, call, cap)
        assert ws.numel() <= E.workspace_bytes(D.shape, call)
        out = t.full((inp.B, inp.Hq, inp.d), np.nan, device="cuda")
        tau = t.full((inp.B, inp.Hq), np.nan, dtype=t.float64, device="cuda")
        fn = E.entmax_decode_sparse_group if group else E.entmax_decode_sparse
        fn(D.shape, D.q, D.k, D.v, D.pt, D.sl, t.from_numpy(si).cuda(), t.from_numpy(ci).cuda(), 1.5, out, tau=tau,
           ws=ws)
        og, tg = out.cpu().numpy().reshape(-1, inp.d), tau.cpu().numpy().reshape(-1)
        # capacity: the largest n whose size fits the bytes (alignment may add a few pages)
        held = cap
        while E.decode_workspace_bytes(D.shape, call, held + 1) <= ws.numel() and held < total + 64:
            held += 1
        fits = ends <= held
        if group:  # a group's G rows fit or fail together (the last row of the group decides)
            fits = np.repeat(fits.reshape(-1, G).all(axis=1), G)
        ok_o, ok_t = oo.reshape(-1, inp.d)[fits], to.reshape(-1)[fits]
        assert np.allclose(tg[fits], ok_t, rtol=1e-12, atol=1e-12, equal_nan=True)
        if fits.any():
            assert rel_l2_rows(og[fits], ok_o) <= TOL["bf16"]
        assert np.all(np.isnan(og[~fits])) and np.all(np.isnan(tg[~fits])), cap
        checked_nan |= bool((~fits).any())
    assert checked_nan  # some capacity left rows out
