"""HIP-graph capture of the decode step: every replay against the same calls made
eagerly.

Two graphs on a 8,192-token, 32/8-head, bf16 slice with pages of 16:

* the decode step (score_pages -> select_pages_gauss / select_pages_topk ->
  entmax_decode_sparse, the group-shared forms with one set per KV head, the
  compact-record scorer, softmax over the kept pages, score and Gaussian
  selection as one call) captured once; before each
  of four replays the query
  is overwritten eagerly, and the replay's page sets, counts and outputs are
  compared with an eager run on the same query;
* the streaming step of the EntmaxKV summary (section 2, pages' metadata kept
  up to date as they fill): append one token's K and V to its page and rebuild
  that page's metadata (append_token, or torch writes + build_page_meta from
  the new token), then score, select and decode with the context one token
  longer.  Four replays grow the context by four
  tokens; a copy driven eagerly takes the same steps, and metadata, sets and
  outputs must agree after every replay.

Page sets, counts, metadata and outputs must match bit for bit: every sum in
the step is taken in a fixed order (the Gaussian selector's counts are integer
adds, its moments fixed-order sums), so a replay repeats the eager run exactly.
"""
import numpy as np
import pytest

import sparse_decode_attention_page_amd as E
from sparse_decode_attention_page_amd import synth

pytestmark = pytest.mark.gpu

CTX = 8192


def _inputs(seed):
    import torch
    wl = synth.WORKLOADS["gqa_32k"]
    inp = synth.make_device(wl, seed, ctx_override=CTX)
    shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
    meta = torch.zeros((inp.num_phys, inp.Hkv, 4, inp.d), dtype=inp.k_pool.dtype, device="cuda")
    E.build_page_meta(shape, inp.k_pool, inp.page_table, inp.seq_lens, meta)
    torch.cuda.synchronize()
    return wl, inp, shape, meta


class _Step:
    """Static buffers and one decode step over them."""

    def __init__(self, shape, inp, policy, alpha, delta, k):
        import torch
        B, Hq, MP, d = inp.B, inp.Hq, inp.max_pages, inp.d
        self.shape, self.policy, self.alpha, self.delta, self.k = shape, policy, alpha, delta, k
        self.box = torch.empty((B, Hq, MP), device="cuda")
        self.mu, self.var = torch.empty_like(self.box), torch.empty_like(self.box)
        nset = inp.Hkv if policy.endswith("_group") else Hq  # group policies: one set per KV head
        self.sel = torch.full((B, nset, MP), -7, dtype=torch.int32, device="cuda")
        self.cnt = torch.full((B, nset), -7, dtype=torch.int32, device="cuda")
        self.out = torch.full((B, Hq, d), float("nan"), device="cuda")
        self.ws_s = E.workspace(shape, E.CALL_SCORE)
        self.ws_g = E.workspace(shape, E.CALL_GAUSS)
        self.ws_t = E.workspace(shape, E.CALL_TOPK)
        self.ws_d = E.workspace(shape, E.CALL_DECODE_SPARSE)
        self.ws_gg = E.workspace(shape, E.CALL_GAUSS_GROUP)
        self.ws_tg = E.workspace(shape, E.CALL_TOPK_GROUP)
        self.ws_dg = E.workspace(shape, E.CALL_DECODE_GROUP)
        self.ws_sm = E.workspace(shape, E.CALL_SOFTMAX_SPARSE)
        self.ws_sg = E.workspace(shape, E.CALL_SCORE_GAUSS)
        self.meta8 = None

    def __call__(self, q, k_pool, v_pool, meta, pt, sl):
        if self.policy == "gauss_fused":  # score and Gaussian selection in one call
            E.score_select_pages_gauss(self.shape, q, meta, pt, sl, self.box, self.mu, self.var, self.alpha,
                                       self.delta, self.sel, self.cnt, ws=self.ws_sg)
            E.entmax_decode_sparse(self.shape, q, k_pool, v_pool, pt, sl, self.sel, self.cnt, self.alpha,
                                   self.out, ws=self.ws_d)
            return
        if self.policy == "gauss_f8":  # compact records, built once from the same keys
            if self.meta8 is None:
                self.meta8 = E.meta_f8_empty(self.shape)
                E.build_page_meta_f8(self.shape, k_pool, pt, sl, self.meta8)
            E.score_pages_f8(self.shape, q, self.meta8, pt, sl, self.box, self.mu, self.var, ws=self.ws_s)
        else:
            E.score_pages(self.shape, q, meta, pt, sl, self.box, self.mu, self.var, ws=self.ws_s)
        if self.policy in ("gauss", "gauss_f8", "gauss_softmax"):
            E.select_pages_gauss(self.shape, self.box, self.mu, self.var, sl, self.alpha, self.delta,
                                 self.sel, self.cnt, ws=self.ws_g)
        elif self.policy == "topk":
            E.select_pages_topk(self.shape, self.box, sl, self.k, self.sel, self.cnt, ws=self.ws_t)
        elif self.policy == "gauss_group":
            E.select_pages_gauss_group(self.shape, self.box, self.mu, self.var, sl, self.alpha, self.delta,
                                       self.sel, self.cnt, ws=self.ws_gg)
        else:
            E.select_pages_topk_group(self.shape, self.box, sl, self.k, self.sel, self.cnt, ws=self.ws_tg)
        if self.policy.endswith("_group"):
            E.entmax_decode_sparse_group(self.shape, q, k_pool, v_pool, pt, sl, self.sel, self.cnt, self.alpha,
                                         self.out, ws=self.ws_dg)
        elif self.policy == "gauss_softmax":
            E.softmax_decode_sparse(self.shape, q, k_pool, v_pool, pt, sl, self.sel, self.cnt, self.out,
                                    ws=self.ws_sm)
        else:
            E.entmax_decode_sparse(self.shape, q, k_pool, v_pool, pt, sl, self.sel, self.cnt, self.alpha,
                                   self.out, ws=self.ws_d)


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def _same_sets(a, b, tag):
    import torch
    assert torch.equal(a.cnt, b.cnt), f"{tag}: sel_cnt differs"
    MP = a.sel.shape[-1]
    inside = torch.arange(MP, device="cuda")[None, None, :] < a.cnt[:, :, None]
    assert torch.equal(torch.where(inside, a.sel, -1), torch.where(inside, b.sel, -1)), f"{tag}: sel_idx differs"


def _close(x, y, tag):
    """Bitwise equality of two float outputs (the step is deterministic)."""
    import torch
    assert bool(torch.isfinite(x).all()), f"{tag}: non-finite output"
    assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (
        f"{tag}: outputs differ (max abs {float((x - y).abs().max()):.3e})")


@pytest.mark.parametrize("policy", ["gauss", "topk", "gauss_group", "topk_group", "gauss_f8", "gauss_softmax",
                                    "gauss_fused"])
def test_graph_replays_match_eager_step(policy):
    import torch
    wl, inp, shape, meta = _inputs(11)
    alpha = wl.alphas[0]
    q_static = inp.q.clone()
    gstep = _Step(shape, inp, policy, alpha, wl.delta, 16)
    estep = _Step(shape, inp, policy, alpha, wl.delta, 16)
    gstep(q_static, inp.k_pool, inp.v_pool, meta, inp.page_table, inp.seq_lens)  # warm
    torch.cuda.synchronize()
    g = _capture(lambda: gstep(q_static, inp.k_pool, inp.v_pool, meta, inp.page_table, inp.seq_lens))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for r in range(4):
        qn = torch.randn(inp.q.shape, generator=gen, device="cuda").to(inp.q.dtype)
        q_static.copy_(qn)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        estep(qn, inp.k_pool, inp.v_pool, meta, inp.page_table, inp.seq_lens)
        torch.cuda.synchronize()
        tag = f"{policy} replay {r}"
        _same_sets(gstep, estep, tag)
        _close(gstep.out, estep.out, tag)


@pytest.mark.parametrize("append", ["append_token", "torch_index_put"])
def test_graph_streaming_step_matches_eager(append):
    import torch
    wl, inp, shape, meta = _inputs(12)
    alpha, P = wl.alphas[0], inp.P
    n_steps = 4
    ptl = inp.page_table.long()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9)
    knew = torch.randn((inp.B, inp.Hkv, inp.d), generator=gen, device="cuda").to(inp.k_pool.dtype)
    vnew = torch.randn((inp.B, inp.Hkv, inp.d), generator=gen, device="cuda").to(inp.v_pool.dtype)

    class Stream:
        def __init__(self):
            self.k = inp.k_pool.clone()
            self.v = inp.v_pool.clone()
            self.meta = meta.clone()
            self.seq = (inp.seq_lens - (n_steps + 1)).to(torch.int32)
            self.step = _Step(shape, inp, "gauss", alpha, wl.delta, 16)

        def __call__(self):
            self.seq.add_(1)
            if append == "append_token":
                E.append_token(shape, knew, vnew, self.k, self.v, inp.page_table, self.seq, self.meta)
            else:
                pos = (self.seq - 1).long()
                ph = torch.gather(ptl, 1, (pos // P).unsqueeze(1)).squeeze(1)
                slot = pos % P
                self.k[ph, :, slot, :] = knew
                self.v[ph, :, slot, :] = vnew
                E.build_page_meta(shape, self.k, inp.page_table, self.seq, self.meta, from_token=self.seq - 1)
            self.step(inp.q, self.k, self.v, self.meta, inp.page_table, self.seq)

    gs, es = Stream(), Stream()
    gs()  # warm: first token
    es()
    torch.cuda.synchronize()
    g = _capture(gs)
    for r in range(n_steps - 1):
        g.replay()
        torch.cuda.synchronize()
        es()
        torch.cuda.synchronize()
        tag = f"streaming replay {r}"
        assert torch.equal(gs.seq, es.seq), f"{tag}: context length differs"
        assert torch.equal(gs.k, es.k) and torch.equal(gs.v, es.v), f"{tag}: K/V pools differ"
        assert torch.equal(gs.meta.view(torch.int16), es.meta.view(torch.int16)), f"{tag}: metadata differs"
        _same_sets(gs.step, es.step, tag)
        _close(gs.step.out, es.step.out, tag)
    # after the last replay the context is back at its full length: the
    # appended metadata equals a full rebuild over the final pools
    assert int(gs.seq[0]) == int(inp.seq_lens[0]) - 1
    full = torch.zeros_like(gs.meta)
    E.build_page_meta(shape, gs.k, inp.page_table, gs.seq, full)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), gs.meta.view(torch.int16)), "appended metadata != full rebuild"
    np.testing.assert_array_equal(gs.seq.cpu().numpy(), es.seq.cpu().numpy())
