#!/usr/bin/env python3
"""EntmaxKV sparse decode benchmark on one MI355X.

One step = one decode step of one layer for the whole batch, inputs resident in
HBM: score_pages -> select_pages_gauss (or top-k) -> entmax_decode_sparse, all
through the HIP library (libentmaxkv.so).  Default workload: 1,048,576-token
context, B=1, 32 query heads over 8 KV heads, d=64, bf16 K/V, pages of 64,
alpha=1.5, Gaussian selection with Delta=0.5.

The timed loop rotates over R input replicas (metadata, q and K/V pools) so
that each step reads its bytes from HBM rather than from the 256 MB last-level
cache.  Steps are replayed from HIP graphs (one per replica) unless --no-graph.

Prints one JSON line (the last line of stdout).
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse entmax decode us/step @1M ctx; HBM GB/s (% peak); speedup vs full-cache"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_1m")
    ap.add_argument("--policy", default="gauss", choices=["gauss", "topk"])
    ap.add_argument("--replicas", type=int, default=6)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming multi-step decode timing")
    ap.add_argument("--no-passage", action="store_true",
                    help="skip the quality-matched leg (the step on the passage variant of the workload)")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the compact-metadata and group-shared-selection variants of the step")
    ap.add_argument("--selector-sweep", action="store_true",
                    help="time select_pages_topk (k=64) and select_pages_gauss over contexts 32k..1M "
                         "(one JSON line with the table), then exit")
    ap.add_argument("--config-sweep", action="store_true",
                    help="step time (HIP-graph replay; Gaussian selection through score_select_pages_gauss and "
                         "Top-k) and the full-cache softmax / entmax times on each smaller workload (4k, 32k, "
                         "128k tokens); one JSON line with the table, then exit")
    ap.add_argument("--quality", action="store_true",
                    help="approximation quality vs KV budget on every synthetic workload (recall of the "
                         "full-cache entmax support, discarded mass and relative output error of entmax and "
                         "softmax under the same kept pages); one JSON line, then exit")
    ap.add_argument("--oracle-1t", action="store_true",
                    help="time the oracle's step on the tiny and 32k workloads (CPU only; run with "
                         "OMP_NUM_THREADS=1 by the CPU-baseline leg), print one JSON line, then exit")
    ap.add_argument("--only", default="", choices=["", "score", "step", "full", "copy"],
                    help="profiling aid: run only score_pages, only the step, only the full-cache entmax and "
                         "softmax decodes, or a plain 1 GiB device copy (the calibration of the HBM byte "
                         "counters), then exit")
    return ap.parse_args()


def main():
    args = parse()
    if args.oracle_1t:
        print(json.dumps(oracle_small_steps()), flush=True)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus N > 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_decode_attention_page_amd as E
    from sparse_decode_attention_page_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    E.load()
    if args.only == "copy":
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {src.nbytes} bytes x4")
        return
    if args.selector_sweep:
        selector_sweep(args)
        return
    if args.quality:
        quality_sweep(args)
        return
    if args.config_sweep:
        config_sweep(args)
        return
    wl = synth.WORKLOADS[args.workload]
    alpha = wl.alphas[0]
    t0 = time.time()
    inp = synth.make_device(wl, args.seed)
    torch.cuda.synchronize()
    log(f"[bench] generated {wl.name} on device in {time.time() - t0:.1f}s: B={inp.B} Hq={inp.Hq} "
        f"Hkv={inp.Hkv} d={inp.d} P={inp.P} pages/seq={inp.max_pages}")
    shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
    B, Hq, Hkv, d, P, MP = inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages
    dev = "cuda"

    # ---- replicas: metadata, q and K/V pools (distinct HBM copies)
    R = max(1, args.replicas)
    reps = []
    meta0 = torch.zeros((inp.num_phys, Hkv, 4, d), dtype=inp.k_pool.dtype, device=dev)
    E.build_page_meta(shape, inp.k_pool, inp.page_table, inp.seq_lens, meta0)
    torch.cuda.synchronize()
    for r in range(R):
        if r == 0:
            reps.append((inp.q, inp.k_pool, inp.v_pool, meta0))
        else:
            reps.append((inp.q.clone(), inp.k_pool.clone(), inp.v_pool.clone(), meta0.clone()))
    torch.cuda.synchronize()
    log(f"[bench] {R} replicas ready ({R * (2 * inp.k_pool.nbytes + meta0.nbytes) / 2**30:.1f} GiB)")

    box = torch.empty((B, Hq, MP), device=dev)
    mu = torch.empty_like(box)
    var = torch.empty_like(box)
    sel = torch.empty((B, Hq, MP), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hq), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, d), device=dev)
    ws_s = E.workspace(shape, E.CALL_SCORE)
    ws_g = E.workspace(shape, E.CALL_GAUSS)
    ws_t = E.workspace(shape, E.CALL_TOPK)
    ws_d = None  # sized by the kept pages below
    sl, pt = inp.seq_lens, inp.page_table

    def score(r):
        q, k, v, meta = reps[r]
        E.score_pages(shape, q, meta, pt, sl, box, mu, var, ws=ws_s)

    def select():
        if args.policy == "gauss":
            E.select_pages_gauss(shape, box, mu, var, sl, alpha, wl.delta, sel, cnt, ws=ws_g)
        else:
            E.select_pages_topk(shape, box, sl, wl.topk or 64, sel, cnt, ws=ws_t)

    def decode(r):
        q, k, v, meta = reps[r]
        E.entmax_decode_sparse(shape, q, k, v, pt, sl, sel, cnt, alpha, out, ws=ws_d)

    ws_sg = E.workspace(shape, E.CALL_SCORE_GAUSS)

    def score_select(r):
        """score + selection: one call for the Gaussian policy (the selector's
        bracket comes from the scoring launch), score_pages + select_pages_topk
        otherwise."""
        if args.policy == "gauss":
            q, k, v, meta = reps[r]
            E.score_select_pages_gauss(shape, q, meta, pt, sl, box, mu, var, alpha, wl.delta, sel, cnt, ws=ws_sg)
        else:
            score(r)
            select()

    def step(r):
        score_select(r)
        decode(r)

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def time_calls(fn, n, per_call=True):
        """Average duration of fn(i) with HIP events on the current stream."""
        ts = []
        for i in range(n):
            a, b = ev(), ev()
            a.record()
            fn(i)
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in ts])) * 1e3  # us

    # ---- the decode workspace holds the kept pages of a first selection with
    # a margin (twice, at least every row's mean plus 64 pages per row)
    score(0)
    select()
    torch.cuda.synchronize()
    kept0 = int(cnt.sum())
    ws_d = E.workspace(shape, E.CALL_DECODE_SPARSE, max_kept_pages=2 * kept0 + 64 * B * Hq)
    ws_dense = E.workspace_bytes(shape, E.CALL_DECODE_SPARSE)
    log(f"[bench] decode workspace {ws_d.numel() / 2**20:.1f} MiB for {kept0} kept pages "
        f"(every page: {ws_dense / 2**20:.1f} MiB)")

    # ---- warm up every call once (also builds lazily computed constants)
    for r in range(R):
        step(r)
    torch.cuda.synchronize()

    if args.only == "score":
        for i in range(args.steps):
            score(i % R)
        torch.cuda.synchronize()
        return
    if args.only == "step":
        for i in range(args.steps):
            step(i % R)
        torch.cuda.synchronize()
        return
    if args.only == "full":
        ws_sm = E.workspace(shape, E.CALL_SOFTMAX)
        ws_f = E.workspace(shape, E.CALL_DECODE_FULL)
        for i in range(args.steps):
            q, k, v, meta = reps[i % R]
            E.entmax_decode_full(shape, q, k, v, pt, sl, alpha, out, ws=ws_f)
            E.softmax_decode_full(shape, q, k, v, pt, sl, out, ws=ws_sm)
        torch.cuda.synchronize()
        return

    # ---- the timed step loop
    graphs = None
    if not args.no_graph:
        try:
            graphs = []
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for r in range(R):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        step(r)
                    graphs.append(g)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
        except Exception as e:  # capture unsupported: time eager launches
            log(f"[bench] graph capture failed ({e}); timing eager launches")
            graphs = None

    def run_step(i):
        if graphs:
            graphs[i % R].replay()
        else:
            step(i % R)

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    a, b = ev(), ev()
    a.record()
    for i in range(args.steps):
        run_step(i)
    b.record()
    torch.cuda.synchronize()
    step_us = a.elapsed_time(b) * 1e3 / args.steps
    log(f"[bench] step: {step_us:.2f} us ({'graph' if graphs else 'eager'})")

    # ---- score_pages launch duration: HIP events around a graph of back-to-back
    # launches (rotating replicas) on the stream they run on
    n_sc = 4 * R
    score_us = None
    try:
        gsc = torch.cuda.CUDAGraph()
        s2 = torch.cuda.Stream()
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s2):
            with torch.cuda.graph(gsc, stream=s2):
                for i in range(n_sc):
                    score(i % R)
        torch.cuda.current_stream().wait_stream(s2)
        gsc.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(5):
            gsc.replay()
        b.record()
        torch.cuda.synchronize()
        score_us = a.elapsed_time(b) * 1e3 / (5 * n_sc)
    except Exception as e:  # capture unsupported: events around eager launches
        log(f"[bench] score graph failed ({e})")
    # ---- per-call breakdown (eager, events around each call, rotating replicas)
    n = max(3 * R, 12)
    score_eager_us = time_calls(lambda i: score(i % R), n)
    if score_us is None:
        score_us = score_eager_us
    sel_us = time_calls(lambda i: select(), n)
    dec_us = time_calls(lambda i: decode(i % R), n)
    log(f"[bench] score_pages per launch (graph of {n_sc}): {score_us:.2f} us; eager per call: score "
        f"{score_eager_us:.2f} us, select {sel_us:.2f} us, decode {dec_us:.2f} us")

    # ---- top-k selection (k=64 unless the workload names one) on the same scores
    k_top = wl.topk or 64
    sel2 = torch.empty_like(sel)
    cnt2 = torch.empty_like(cnt)
    E.select_pages_topk(shape, box, sl, k_top, sel2, cnt2, ws=ws_t)
    torch.cuda.synchronize()
    topk_us = time_calls(lambda i: E.select_pages_topk(shape, box, sl, k_top, sel2, cnt2, ws=ws_t), n)

    # ---- metadata append for the new token: rebuild the page holding each
    # sequence's last token (build_page_meta with from_token = L_b - 1)
    from_tok = (sl - 1).clamp(min=0).to(torch.int32)
    meta_scratch = reps[0][3].clone()

    def append(i):
        E.build_page_meta(shape, reps[0][1], pt, sl, meta_scratch, from_token=from_tok)

    append(0)
    torch.cuda.synchronize()
    append_us = time_calls(append, n)
    del meta_scratch

    # ---- a measured stream read on this GPU (the library's read probe over a
    # 2 GiB K/V replica, rotating replicas so each pass reads HBM): the practical
    # ceiling next to the 8 TB/s peak
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for r in range(R):
        E.stream_read(reps[r][1], sink)
    torch.cuda.synchronize()
    sr_us = time_calls(lambda i: E.stream_read(reps[i % R][1 + (i // R) % 2], sink), 2 * R)
    stream_gbs = reps[0][1].nbytes / (sr_us * 1e-6) / 1e9
    log(f"[bench] top-k select {topk_us:.2f} us, metadata append {append_us:.2f} us, "
        f"stream read {stream_gbs:.0f} GB/s")

    # ---- streaming decode: one graph per step appends the new token's K and V
    # to its page and rebuilds that page's metadata (append_token, one launch),
    # then scores, selects and decodes with the context one token longer (the
    # context grows from L - n_total to L over the replays); on copies of
    # replica 0
    stream_res = None
    if not args.no_stream:
        try:
            n_st, n_wu = 50, 5
            k2, v2, meta2 = reps[0][1].clone(), reps[0][2].clone(), reps[0][3].clone()
            seq2 = (sl - (n_st + n_wu + 1)).clamp(min=1).to(torch.int32)
            knew = torch.randn((B, Hkv, d), device=dev).to(k2.dtype)
            vnew = torch.randn((B, Hkv, d), device=dev).to(v2.dtype)
            sel3, cnt3 = torch.empty_like(sel), torch.empty_like(cnt)
            out3 = torch.empty_like(out)

            def stream_step():
                seq2.add_(1)
                E.append_token(shape, knew, vnew, k2, v2, pt, seq2, meta2)
                if args.policy == "gauss":
                    E.score_select_pages_gauss(shape, reps[0][0], meta2, pt, seq2, box, mu, var, alpha, wl.delta,
                                               sel3, cnt3, ws=ws_sg)
                else:
                    E.score_pages(shape, reps[0][0], meta2, pt, seq2, box, mu, var, ws=ws_s)
                    E.select_pages_topk(shape, box, seq2, wl.topk or 64, sel3, cnt3, ws=ws_t)
                E.entmax_decode_sparse(shape, reps[0][0], k2, v2, pt, seq2, sel3, cnt3, alpha, out3, ws=ws_d)

            stream_step()  # warm (also the first token)
            torch.cuda.synchronize()
            gst = torch.cuda.CUDAGraph()
            s3 = torch.cuda.Stream()
            s3.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s3):
                with torch.cuda.graph(gst, stream=s3):
                    stream_step()
            torch.cuda.current_stream().wait_stream(s3)
            for _ in range(n_wu - 1):
                gst.replay()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for _ in range(n_st):
                gst.replay()
            b.record()
            torch.cuda.synchronize()
            st_us = a.elapsed_time(b) * 1e3 / n_st
            L_end = int(seq2.max().item())
            stream_res = {"us_per_step": round(st_us, 3), "steps": n_st,
                          "context_end": L_end, "context_start": L_end - n_st,
                          "step": "append_token (K/V row + page metadata) + " +
                                  ("score_select_pages_gauss" if args.policy == "gauss"
                                   else "score_pages + select_pages_topk") +
                                  " + entmax_decode_sparse, one HIP graph per step"}
            # append_token's own launch duration: a graph of 20 launches (the
            # same token rewritten, so every launch does the same work)
            gap = torch.cuda.CUDAGraph()
            s3.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s3):
                with torch.cuda.graph(gap, stream=s3):
                    for _ in range(20):
                        E.append_token(shape, knew, vnew, k2, v2, pt, seq2, meta2)
            torch.cuda.current_stream().wait_stream(s3)
            gap.replay()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for _ in range(5):
                gap.replay()
            b.record()
            torch.cuda.synchronize()
            ap_us = a.elapsed_time(b) * 1e3 / 100
            stream_res["append_token_us"] = round(ap_us, 2)
            log(f"[bench] streaming step (append + metadata + step): {st_us:.2f} us; append_token per launch "
                f"(graph of 20): {ap_us:.2f} us")
            del k2, v2, meta2
        except Exception as e:  # capture unsupported
            log(f"[bench] streaming step failed ({e})")

    # ---- variants of the step: compact metadata (score_pages_f8 on E4M3 mean /
    # variance records) and group-shared selection (one kept set per KV head,
    # each kept page read once for the G query heads); one graph per replica
    variants, var_sets = None, {}
    rec8_bytes = 6 * d
    if not args.no_variants:
        try:
            meta8 = []
            for r in range(R):
                m8 = E.meta_f8_empty(shape)
                E.build_page_meta_f8(shape, reps[r][1], pt, sl, m8)
                meta8.append(m8)
            selg = torch.empty((B, Hkv, MP), dtype=torch.int32, device=dev)
            cntg = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
            ws_gg = E.workspace(shape, E.CALL_GAUSS_GROUP)
            ws_tg = E.workspace(shape, E.CALL_TOPK_GROUP)
            ws_dg = E.workspace(shape, E.CALL_DECODE_GROUP)

            def v_step(r, f8, grp):
                q, k, v, meta = reps[r]
                if f8:
                    E.score_pages_f8(shape, q, meta8[r], pt, sl, box, mu, var, ws=ws_s)
                else:
                    E.score_pages(shape, q, meta, pt, sl, box, mu, var, ws=ws_s)
                if not grp:
                    select()
                    decode(r)
                    return
                if args.policy == "gauss":
                    E.select_pages_gauss_group(shape, box, mu, var, sl, alpha, wl.delta, selg, cntg, ws=ws_gg)
                else:
                    E.select_pages_topk_group(shape, box, sl, wl.topk or 64, selg, cntg, ws=ws_tg)
                E.entmax_decode_sparse_group(shape, q, k, v, pt, sl, selg, cntg, alpha, out, ws=ws_dg)

            def graph_us(fn, n_rep):
                gs = []
                sv = torch.cuda.Stream()
                sv.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(sv):
                    for r in range(R):
                        g = torch.cuda.CUDAGraph()
                        with torch.cuda.graph(g, stream=sv):
                            fn(r)
                        gs.append(g)
                torch.cuda.current_stream().wait_stream(sv)
                for i in range(max(args.warmup, R)):
                    gs[i % R].replay()
                torch.cuda.synchronize()
                a, b = ev(), ev()
                a.record()
                for i in range(n_rep):
                    gs[i % R].replay()
                b.record()
                torch.cuda.synchronize()
                return a.elapsed_time(b) * 1e3 / n_rep

            variants = {}
            for name, f8, grp in (("separate_calls", False, False), ("compact_meta", True, False),
                                  ("group_sets", False, True), ("compact_meta_group_sets", True, True)):
                us = graph_us(lambda r, f8=f8, grp=grp: v_step(r, f8, grp), args.steps)
                v_step(0, f8, grp)  # replica 0's selection, for the quality figures below
                torch.cuda.synchronize()
                if grp:
                    var_sets[name] = (selg.repeat_interleave(Hq // Hkv, dim=1).clone(),
                                      cntg.repeat_interleave(Hq // Hkv, dim=1).clone(),
                                      float(cntg.double().mean()))
                else:
                    var_sets[name] = (sel.clone(), cnt.clone(), None)
                variants[name] = {"step_us": round(us, 2), "speedup_vs_step": round(step_us / us, 3)}
                if grp:
                    variants[name]["kept_pages_per_kv_head_mean"] = round(var_sets[name][2], 2)
                log(f"[bench] variant {name}: step {us:.2f} us")
            # score_pages_f8 per launch, as for score_pages
            sc8_us = graph_us(lambda r: [E.score_pages_f8(shape, reps[(r + j) % R][0], meta8[(r + j) % R], pt, sl,
                                                          box, mu, var, ws=ws_s) for j in range(4)], 5 * R) / 4
            variants["compact_meta"]["score_pages_f8_us"] = round(sc8_us, 2)
            log(f"[bench] score_pages_f8 per launch: {sc8_us:.2f} us")
            step(0)  # the main step's state again (replica 0)
            torch.cuda.synchronize()
            del meta8
        except Exception as e:
            log(f"[bench] variants failed ({e})")
            variants = None

    # ---- algorithmic bytes of the dominant kernel (score_pages)
    seq = sl.cpu().numpy().astype(np.int64)
    npg = (seq + P - 1) // P
    esz = inp.k_pool.element_size()
    rec = 4 * d * esz
    # metadata records + q + box/mu/var outputs + page-table entries
    score_bytes = int(npg.sum() * Hkv * rec + B * Hq * d * esz + Hq * npg.sum() * 12 + npg.sum() * 4)
    score_gbs = score_bytes / (score_us * 1e-6) / 1e9
    if variants and "score_pages_f8_us" in variants.get("compact_meta", {}):
        b8 = int(npg.sum() * Hkv * rec8_bytes + B * Hq * d * esz + Hq * npg.sum() * 12 + npg.sum() * 4)
        t8 = variants["compact_meta"]["score_pages_f8_us"]
        variants["compact_meta"]["score_pages_f8_roofline"] = {
            "bound": "hbm", "algorithmic_bytes": b8, "achieved": round(b8 / (t8 * 1e-6) / 1e9, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(b8 / (t8 * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    # ---- selection statistics and decode bytes
    torch.cuda.synchronize()
    step(0)
    torch.cuda.synchronize()
    cnt_h = cnt.cpu().numpy()
    sel_h = sel.cpu().numpy()
    union = 0
    G = Hq // Hkv
    for bb in range(B):
        for g in range(Hkv):
            s_ = set()
            for h in range(g * G, (g + 1) * G):
                s_.update(sel_h[bb, h, :cnt_h[bb, h]].tolist())
            union += len(s_)
    per_head_pages = int(cnt_h.sum())
    log(f"[bench] kept pages per row: min {cnt_h.min()} median {int(np.median(cnt_h))} max {cnt_h.max()} "
        f"(of {MP})")
    dec_bytes = per_head_pages * 2 * P * d * esz  # K and V of every kept page (per head)
    step_bytes = score_bytes + Hq * npg.sum() * 12 + dec_bytes  # + selector reads of box/mu/var

    result = {
        "metric": METRIC,
        "value": round(step_us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-kv/f64-score/f32-acc",
        "dtype_detail": ("K/V and q bf16; scores, thresholds and weights p_t fp64 (exact bf16 products); "
                         "the weighted V sum accumulated in fp32"),
        "data": "synthetic",
        "config": {
            "workload": (f"{wl.name}: B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, {wl.dtype} K/V, "
                         f"{int(seq.max())} tokens in pages of {P}; alpha={alpha}, "
                         + (f"Gaussian selection Delta={wl.delta}" if args.policy == "gauss"
                            else f"top-k {wl.topk or 64}")),
            "step": ("score_select_pages_gauss (score_pages + select_pages_gauss in one call)"
                     if args.policy == "gauss" else "score_pages + select_pages_topk") + " + entmax_decode_sparse",
            "replicas": R,
            "launch": "hip graph replay" if graphs else "eager",
            "kv_dtype": wl.dtype,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "score_pages",
            "achieved": round(score_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(score_gbs / HBM_PEAK_GBS, 4),
            "traffic": score_traffic(args.workload),
            "algorithmic_bytes": score_bytes,
            "launch_us": round(score_us, 3),
            "stream_read_GBps": round(stream_gbs, 1),
            "frac_of_stream_read": round(score_gbs / stream_gbs, 4),
        },
        "breakdown_us": {"score_pages": round(score_us, 3), "select": round(sel_us, 3),
                         "entmax_decode_sparse": round(dec_us, 3), "select_topk": round(topk_us, 3),
                         "metadata_append": round(append_us, 3),
                         "note": "select/decode/top-k/append: eager, per call; append = rebuild of "
                                 "the page holding each sequence's newest token"},
        "selection": {"pages_per_head_mean": round(per_head_pages / (B * Hq), 2),
                      "kv_group_union_pages": union, "pages_per_seq": int(npg.max())},
        "streaming": stream_res,
        "variants": variants,
        "step_algorithmic_bytes": int(step_bytes),
        "step_GBps": round(step_bytes / (step_us * 1e-6) / 1e9, 1),
    }

    # ---- comparators: the library's own full-cache softmax and entmax decodes
    if not args.no_comparators:
        ws_sm = E.workspace(shape, E.CALL_SOFTMAX)
        ws_f = E.workspace(shape, E.CALL_DECODE_FULL)
        out2 = torch.empty_like(out)

        def sm(i):
            q, k, v, meta = reps[i % R]
            E.softmax_decode_full(shape, q, k, v, pt, sl, out2, ws=ws_sm)

        def ef(i):
            q, k, v, meta = reps[i % R]
            E.entmax_decode_full(shape, q, k, v, pt, sl, alpha, out2, ws=ws_f)

        sm(0)
        torch.cuda.synchronize()
        sm_us = time_calls(sm, max(R, 6))
        t1 = time.time()
        ef(0)
        torch.cuda.synchronize()
        n_ef = 3 if time.time() - t1 < 2.0 else 1
        ef_us = time_calls(ef, n_ef)
        kv_bytes = int(npg.sum() * P * Hkv * 2 * d * esz)
        result["comparators_us"] = {"softmax_decode_full": round(sm_us, 2),
                                    "entmax_decode_full": round(ef_us, 2),
                                    "softmax_full_GBps": round(kv_bytes / (sm_us * 1e-6) / 1e9, 1)}
        result["speedup"] = {"vs_full_softmax": round(sm_us / step_us, 2),
                             "vs_full_entmax": round(ef_us / step_us, 2)}
        log(f"[bench] full softmax {sm_us:.1f} us, full entmax {ef_us:.1f} us")

        # ---- entmax vs softmax under the same kept set (the step's selection):
        # discarded probability mass delta and relative output error against each
        # one's full-cache result (untimed), and the softmax-over-kept-pages time
        ws_ss = E.workspace(shape, E.CALL_SOFTMAX_SPARSE)
        q0, k0, v0, _ = reps[0]
        step(0)
        torch.cuda.synchronize()
        out_es = out.clone()
        wfull = torch.empty((B, Hq, MP * P), device=dev)
        out_ef = torch.empty_like(out)
        E.entmax_decode_full(shape, q0, k0, v0, pt, sl, alpha, out_ef, weights_out=wfull, ws=ws_f)
        out_sf = torch.empty_like(out)
        lse_f = torch.empty((B, Hq), device=dev)
        E.softmax_decode_full(shape, q0, k0, v0, pt, sl, out_sf, lse=lse_f, ws=ws_sm)
        out_ss = torch.empty_like(out)
        lse_s = torch.empty((B, Hq), device=dev)
        E.softmax_decode_sparse(shape, q0, k0, v0, pt, sl, sel, cnt, out_ss, lse=lse_s, ws=ws_ss)
        torch.cuda.synchronize()
        # unused slots go to a spare column MP (a shared target of True and
        # False writes would leave the kept flag to the write order)
        keep = torch.zeros((B, Hq, MP + 1), dtype=torch.bool, device=dev)
        ar = torch.arange(MP, device=dev)
        valid = ar[None, None, :] < cnt[:, :, None]
        keep.scatter_(2, torch.where(valid, sel, torch.full_like(sel, MP)).long(), valid)
        keep = keep[:, :, :MP]
        kept_mass = (wfull.view(B, Hq, MP, P).double().sum(-1) * keep).sum(-1)
        d_ent = (1.0 - kept_mass).clamp(min=0.0)
        d_sm = (1.0 - torch.exp((lse_s - lse_f).double())).clamp(min=0.0)

        def rel(a, b):
            return (torch.linalg.vector_norm((a - b).double(), dim=-1)
                    / torch.linalg.vector_norm(b.double(), dim=-1).clamp(min=1e-30))

        e_ent, e_sm = rel(out_es, out_ef), rel(out_ss, out_sf)
        ss_us = time_calls(lambda i: E.softmax_decode_sparse(shape, reps[i % R][0], reps[i % R][1], reps[i % R][2],
                                                             pt, sl, sel, cnt, out_ss, ws=ws_ss), max(R, 6))
        # the variants' selections on replica 0: discarded entmax mass and the
        # relative error of their outputs against the full-cache entmax
        if variants:
            for name, (vs, vc, _) in var_sets.items():
                vk = torch.zeros((B, Hq, MP + 1), dtype=torch.bool, device=dev)
                vin = ar[None, None, :] < vc[:, :, None]
                vk.scatter_(2, torch.where(vin, vs, torch.full_like(vs, MP)).long(), vin)
                vkeep = vk[:, :, :MP]
                d_v = (1.0 - (wfull.view(B, Hq, MP, P).double().sum(-1) * vkeep).sum(-1)).clamp(min=0.0)
                out_v = torch.empty_like(out)
                E.entmax_decode_sparse(shape, q0, k0, v0, pt, sl, vs.contiguous(), vc.contiguous(), alpha, out_v,
                                       ws=ws_d)
                torch.cuda.synchronize()
                variants[name]["delta_entmax_mean"] = float(d_v.mean())
                variants[name]["rel_err_entmax_mean"] = float(rel(out_v, out_ef).mean())
                variants[name]["kept_pages_per_head_mean"] = round(float(vc.double().mean()), 2)
        result["same_kept_set"] = {
            "selection": "step's " + args.policy + " selection",
            "delta_entmax_mean": float(d_ent.mean()), "delta_entmax_max": float(d_ent.max()),
            "delta_softmax_mean": float(d_sm.mean()), "delta_softmax_max": float(d_sm.max()),
            "rel_err_entmax_mean": float(e_ent.mean()), "rel_err_entmax_max": float(e_ent.max()),
            "rel_err_softmax_mean": float(e_sm.mean()), "rel_err_softmax_max": float(e_sm.max()),
            "softmax_decode_sparse_us": round(ss_us, 2),
        }
        log(f"[bench] same kept set: delta entmax {float(d_ent.mean()):.3e} vs softmax {float(d_sm.mean()):.3e}; "
            f"rel err entmax {float(e_ent.mean()):.3e} vs softmax {float(e_sm.mean()):.3e}; "
            f"softmax over kept pages {ss_us:.1f} us")
        del wfull

    result["decode_workspace"] = {"bytes": int(ws_d.numel()), "kept_pages_bound": 2 * kept0 + 64 * B * Hq,
                                  "every_page_bytes": int(ws_dense)}

    # ---- quality-matched leg: the same step where the kept pages hold the support
    if not args.no_passage and (wl.name + "_passage") in synth.WORKLOADS:
        del reps
        torch.cuda.empty_cache()
        try:
            result["quality_matched"] = passage_leg(args, wl.name + "_passage")
        except Exception as e:
            log(f"[bench] passage leg failed ({e})")

    # ---- CPU baseline: the oracle on a bounded sample of the same workload
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, shape, wl, alpha, args.policy)

    print(json.dumps(result), flush=True)


def passage_leg(args, name):
    """The step on the passage variant of the workload (runs of 16 planted keys
    along the query, so the selection keeps the pages holding the entmax
    support): step time over HIP-graph replays of two replicas, the full-cache
    softmax and entmax times, and the discarded entmax mass and relative output
    error of the sparse decode against the full-cache entmax."""
    import numpy as np
    import torch

    import sparse_decode_attention_page_amd as E
    from sparse_decode_attention_page_amd import synth

    wl = synth.WORKLOADS[name]
    alpha = wl.alphas[0]
    inp = synth.make_device(wl, args.seed)
    shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
    B, Hq, Hkv, d, P, MP = inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages
    meta = torch.zeros((inp.num_phys, Hkv, 4, d), dtype=inp.k_pool.dtype, device="cuda")
    E.build_page_meta(shape, inp.k_pool, inp.page_table, inp.seq_lens, meta)
    reps = [(inp.q, inp.k_pool, inp.v_pool, meta),
            (inp.q.clone(), inp.k_pool.clone(), inp.v_pool.clone(), meta.clone())]
    box = torch.empty((B, Hq, MP), device="cuda")
    mu, var = torch.empty_like(box), torch.empty_like(box)
    sel = torch.empty((B, Hq, MP), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, d), device="cuda")
    sl, pt = inp.seq_lens, inp.page_table
    ws_sg = E.workspace(shape, E.CALL_SCORE_GAUSS)

    def select(r):
        q, k, v, m = reps[r]
        E.score_select_pages_gauss(shape, q, m, pt, sl, box, mu, var, alpha, wl.delta, sel, cnt, ws=ws_sg)

    select(0)
    torch.cuda.synchronize()
    kept = int(cnt.sum())
    ws_d = E.workspace(shape, E.CALL_DECODE_SPARSE, max_kept_pages=2 * kept + 64 * B * Hq)

    def step(r):
        q, k, v, m = reps[r]
        select(r)
        E.entmax_decode_sparse(shape, q, k, v, pt, sl, sel, cnt, alpha, out, ws=ws_d)

    for r in range(2):
        step(r)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(s):
        for r in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                step(r)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(max(args.warmup, 2)):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(args.steps):
        graphs[i % 2].replay()
    b.record()
    torch.cuda.synchronize()
    step_us = a.elapsed_time(b) * 1e3 / args.steps
    # comparators on the same inputs (eager, events around each call)
    ws_sm, ws_f = E.workspace(shape, E.CALL_SOFTMAX), E.workspace(shape, E.CALL_DECODE_FULL)
    out2 = torch.empty_like(out)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(n):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.mean([x.elapsed_time(y) for x, y in ts])) * 1e3

    q0, k0, v0, m0 = reps[0]
    sm_us = timed(lambda: E.softmax_decode_full(shape, q0, k0, v0, pt, sl, out2, ws=ws_sm), 6)
    ef_us = timed(lambda: E.entmax_decode_full(shape, q0, k0, v0, pt, sl, alpha, out2, ws=ws_f), 3)
    # quality of replica 0's step against the full-cache entmax
    step(0)
    wfull = torch.empty((B, Hq, MP * P), device="cuda")
    out_f = torch.empty_like(out)
    E.entmax_decode_full(shape, q0, k0, v0, pt, sl, alpha, out_f, weights_out=wfull, ws=ws_f)
    torch.cuda.synchronize()
    keep = torch.zeros((B, Hq, MP + 1), dtype=torch.bool, device="cuda")
    ar = torch.arange(MP, device="cuda")
    valid = ar[None, None, :] < cnt[:, :, None]
    keep.scatter_(2, torch.where(valid, sel, torch.full_like(sel, MP)).long(), valid)
    kept_mass = (wfull.view(B, Hq, MP, P).double().sum(-1) * keep[:, :, :MP]).sum(-1)
    delta = (1.0 - kept_mass).clamp(min=0.0)
    rel = (torch.linalg.vector_norm((out - out_f).double(), dim=-1)
           / torch.linalg.vector_norm(out_f.double(), dim=-1).clamp(min=1e-30))
    res = {"workload": (f"{name}: B={B}, Hq={Hq}, Hkv={Hkv}, d={d}, {wl.dtype} K/V, {int(sl.max())} tokens in "
                        f"pages of {P}; alpha={alpha}, Gaussian selection Delta={wl.delta}"),
           "step_us": round(step_us, 2), "softmax_decode_full_us": round(sm_us, 2),
           "entmax_decode_full_us": round(ef_us, 2),
           "speedup_vs_full_softmax": round(sm_us / step_us, 2), "speedup_vs_full_entmax": round(ef_us / step_us, 2),
           "kept_pages_per_head_mean": round(float(cnt.double().mean()), 2),
           "delta_entmax_mean": float(delta.mean()), "delta_entmax_max": float(delta.max()),
           "rel_err_entmax_mean": float(rel.mean()), "rel_err_entmax_max": float(rel.max()),
           "launch": "hip graph replay (2 replicas)"}
    log(f"[bench] quality-matched leg ({name}): step {step_us:.2f} us, full softmax {sm_us:.1f} us, full entmax "
        f"{ef_us:.1f} us; delta entmax {res['delta_entmax_mean']:.3e}, rel err {res['rel_err_entmax_mean']:.3e}")
    return res


def config_sweep(args):
    """The step on each smaller workload: score + selection + sparse entmax decode
    as HIP-graph replays over two replicas, once with the Gaussian selection
    (score_select_pages_gauss) and once with Top-k (score_pages +
    select_pages_topk), for every alpha the workload lists; beside them the
    full-cache softmax and entmax decodes (eager, events around each call)."""
    import numpy as np
    import torch

    import sparse_decode_attention_page_amd as E
    from sparse_decode_attention_page_amd import synth

    ev = lambda: torch.cuda.Event(enable_timing=True)
    rows = []
    for name in ("tiny_4k", "gqa_32k", "gqa_128k"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_device(wl, args.seed)
        shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
        B, Hq, Hkv, d, P, MP = inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages
        meta = torch.zeros((inp.num_phys, Hkv, 4, d), dtype=inp.k_pool.dtype, device="cuda")
        E.build_page_meta(shape, inp.k_pool, inp.page_table, inp.seq_lens, meta)
        reps = [(inp.q, inp.k_pool, inp.v_pool, meta),
                (inp.q.clone(), inp.k_pool.clone(), inp.v_pool.clone(), meta.clone())]
        sl, pt = inp.seq_lens, inp.page_table
        box = torch.empty((B, Hq, MP), device="cuda")
        mu, var = torch.empty_like(box), torch.empty_like(box)
        sel = torch.empty((B, Hq, MP), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
        out = torch.empty((B, Hq, d), device="cuda")
        ws_s, ws_t = E.workspace(shape, E.CALL_SCORE), E.workspace(shape, E.CALL_TOPK)
        ws_sg = E.workspace(shape, E.CALL_SCORE_GAUSS)
        ws_d = E.workspace(shape, E.CALL_DECODE_SPARSE)
        k_top = wl.topk or 64

        def graph_us(fn):
            fn(0), fn(1)
            torch.cuda.synchronize()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            gs = []
            with torch.cuda.stream(s):
                for r in range(2):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=s):
                        fn(r)
                    gs.append(g)
            torch.cuda.current_stream().wait_stream(s)
            for i in range(max(args.warmup, 2)):
                gs[i % 2].replay()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for i in range(args.steps):
                gs[i % 2].replay()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / args.steps

        def eager_us(fn, n=10):
            fn()
            torch.cuda.synchronize()
            a, b = ev(), ev()
            a.record()
            for _ in range(n):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / n

        q0, k0, v0, m0 = reps[0]
        ws_sm, ws_f = E.workspace(shape, E.CALL_SOFTMAX), E.workspace(shape, E.CALL_DECODE_FULL)
        sm_us = eager_us(lambda: E.softmax_decode_full(shape, q0, k0, v0, pt, sl, out, ws=ws_sm))
        for alpha in wl.alphas:
            def gauss_step(r, alpha=alpha):
                q, k, v, m = reps[r]
                E.score_select_pages_gauss(shape, q, m, pt, sl, box, mu, var, alpha, wl.delta, sel, cnt, ws=ws_sg)
                E.entmax_decode_sparse(shape, q, k, v, pt, sl, sel, cnt, alpha, out, ws=ws_d)

            def topk_step(r, alpha=alpha):
                q, k, v, m = reps[r]
                E.score_pages(shape, q, m, pt, sl, box, mu, var, ws=ws_s)
                E.select_pages_topk(shape, box, sl, k_top, sel, cnt, ws=ws_t)
                E.entmax_decode_sparse(shape, q, k, v, pt, sl, sel, cnt, alpha, out, ws=ws_d)

            g_us = graph_us(gauss_step)
            gauss_step(0)
            torch.cuda.synchronize()
            g_kept = float(cnt.double().mean())
            t_us = graph_us(topk_step)
            ef_us = eager_us(lambda: E.entmax_decode_full(shape, q0, k0, v0, pt, sl, alpha, out, ws=ws_f))
            row = {"workload": name, "B": B, "Hq": Hq, "Hkv": Hkv, "d": d, "P": P, "kv_dtype": wl.dtype,
                   "context": int(sl.max()), "alpha": alpha, "delta": wl.delta, "topk": k_top,
                   "step_gauss_us": round(g_us, 2), "gauss_kept_pages_per_head_mean": round(g_kept, 2),
                   "step_topk_us": round(t_us, 2), "pages_per_seq": MP,
                   "softmax_decode_full_us": round(sm_us, 2), "entmax_decode_full_us": round(ef_us, 2)}
            log(f"[configs] {row}")
            rows.append(row)
        del inp, reps, meta
        torch.cuda.empty_cache()
    print(json.dumps({"config_sweep": rows, "unit": "us per step (graph replay) / per call (full-cache, eager)"}),
          flush=True)


def selector_sweep(args):
    """Top-k (k=64) vs Gaussian selection time as the context grows, on the
    long-context workload's shapes (B=1, 32 query / 8 KV heads, d=64, pages of
    64); scores come from score_pages on freshly built metadata."""
    import numpy as np
    import torch

    import sparse_decode_attention_page_amd as E
    from sparse_decode_attention_page_amd import synth

    wl = synth.WORKLOADS["long_1m"]
    alpha = wl.alphas[0]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rows = []
    for ctx in (32768, 131072, 524288, 1048576, 4194304):
        inp = synth.make_device(wl, args.seed, ctx_override=ctx)
        shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
        B, Hq, Hkv, d, MP = inp.B, inp.Hq, inp.Hkv, inp.d, inp.max_pages
        meta = torch.zeros((inp.num_phys, Hkv, 4, d), dtype=inp.k_pool.dtype, device="cuda")
        E.build_page_meta(shape, inp.k_pool, inp.page_table, inp.seq_lens, meta)
        box = torch.empty((B, Hq, MP), device="cuda"); mu = torch.empty_like(box); var = torch.empty_like(box)
        sel = torch.empty((B, Hq, MP), dtype=torch.int32, device="cuda")
        cnt = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
        E.score_pages(shape, inp.q, meta, inp.page_table, inp.seq_lens, box, mu, var,
                      ws=E.workspace(shape, E.CALL_SCORE))
        ws_t, ws_g = E.workspace(shape, E.CALL_TOPK), E.workspace(shape, E.CALL_GAUSS)
        ws_s, ws_sg = E.workspace(shape, E.CALL_SCORE), E.workspace(shape, E.CALL_SCORE_GAUSS)
        calls = {"topk64": lambda: E.select_pages_topk(shape, box, inp.seq_lens, 64, sel, cnt, ws=ws_t),
                 "gauss": lambda: E.select_pages_gauss(shape, box, mu, var, inp.seq_lens, alpha, wl.delta,
                                                       sel, cnt, ws=ws_g),
                 "score": lambda: E.score_pages(shape, inp.q, meta, inp.page_table, inp.seq_lens, box, mu, var,
                                                ws=ws_s),
                 "score_select_gauss": lambda: E.score_select_pages_gauss(shape, inp.q, meta, inp.page_table,
                                                                          inp.seq_lens, box, mu, var, alpha,
                                                                          wl.delta, sel, cnt, ws=ws_sg)}
        row = {"context": ctx, "pages": MP}
        for name, fn in calls.items():
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(20):
                a, b = ev(), ev()
                a.record(); fn(); b.record()
                ts.append((a, b))
            torch.cuda.synchronize()
            row[name + "_us"] = round(float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3, 2)
            if name == "gauss":
                row["gauss_kept_pages_mean"] = round(float(cnt.float().mean().item()), 2)
        log(f"[sweep] {row}")
        rows.append(row)
        del inp, meta, box, mu, var, sel, cnt
        torch.cuda.empty_cache()
    print(json.dumps({"selector_sweep": rows, "unit": "us per call (median of 20, eager)",
                      "workload": "long_1m shapes at the listed contexts"}), flush=True)


def quality_sweep(args):
    """Approximation quality against the KV budget (the comparison of the
    EntmaxKV summary, sections 3 and 4, on synthetic inputs).  For every
    workload, alpha and selector setting: kept pages per head, recall of the
    full-cache entmax support S (|S n T| / |S|, T the tokens of the kept
    pages), the discarded probability mass delta of entmax (full-cache weights
    outside T) and of softmax (1 - exp(lse_T - lse_full)), the relative output
    error ||o - o~|| / ||o|| of each decoded over T, and the largest ratio of
    that error to its bound 2 B delta (B = largest value norm of the row's
    sequence and KV head).  Every number comes from this library's kernels."""
    import numpy as np
    import torch

    import sparse_decode_attention_page_amd as E
    from sparse_decode_attention_page_amd import synth

    dev = "cuda"
    rows = []
    for name in ("tiny_4k", "gqa_32k", "gqa_128k", "long_1m", "batch16_ragged", "gqa_128k_passage",
                 "long_1m_passage"):
        wl = synth.WORKLOADS[name]
        inp = synth.make_device(wl, args.seed)
        shape = E.make_shape(inp.q, inp.k_pool, inp.page_table)
        B, Hq, Hkv, d, P, MP = inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages
        G = Hq // Hkv
        sl, pt, q, kp, vp = inp.seq_lens, inp.page_table, inp.q, inp.k_pool, inp.v_pool
        meta = torch.zeros((inp.num_phys, Hkv, 4, d), dtype=kp.dtype, device=dev)
        E.build_page_meta(shape, kp, pt, sl, meta)
        box = torch.empty((B, Hq, MP), device=dev)
        mu, var = torch.empty_like(box), torch.empty_like(box)
        E.score_pages(shape, q, meta, pt, sl, box, mu, var)
        ntok = MP * P
        valid = torch.arange(ntok, device=dev)[None, :] < sl[:, None]            # [B][ntok]
        # B of the bound: the largest value norm over the row's sequence and KV head
        vn = torch.linalg.vector_norm(vp.float(), dim=-1)                         # [phys][Hkv][P]
        vnb = vn[pt.clamp(min=0).long()].permute(0, 2, 1, 3).reshape(B, Hkv, ntok)
        vnb = torch.where(valid[:, None, :], vnb, torch.zeros_like(vnb))
        bnd = vnb.amax(-1).repeat_interleave(G, dim=1).double()                  # [B][Hq]
        out_sf = torch.empty((B, Hq, d), device=dev)
        lse_f = torch.empty((B, Hq), device=dev)
        E.softmax_decode_full(shape, q, kp, vp, pt, sl, out_sf, lse=lse_f)
        sel = torch.empty((B, Hq, MP), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, Hq), dtype=torch.int32, device=dev)
        out_es, out_ss = torch.empty_like(out_sf), torch.empty_like(out_sf)
        lse_s = torch.empty_like(lse_f)
        ar = torch.arange(MP, device=dev)
        settings = [("topk", {"k": k}) for k in (4, 16, 64, 256) if k < MP]
        settings += [("gauss", {"delta": dl, "n_sigma": ns})
                     for dl, ns in ((0.5, 2.0), (0.5, 3.0), (0.5, 4.0), (0.5, 6.0), (0.0, 3.0), (1.0, 3.0),
                                    (2.0, 3.0))]

        def rel(a, b):
            return (torch.linalg.vector_norm((a - b).double(), dim=-1),
                    torch.linalg.vector_norm(b.double(), dim=-1))

        for alpha in wl.alphas:
            wfull = torch.empty((B, Hq, ntok), device=dev)
            out_ef = torch.empty_like(out_sf)
            E.entmax_decode_full(shape, q, kp, vp, pt, sl, alpha, out_ef, weights_out=wfull)
            supp = wfull > 0
            n_supp = supp.sum(-1).double()
            for kind, par in settings:
                if kind == "topk":
                    E.select_pages_topk(shape, box, sl, par["k"], sel, cnt)
                else:
                    E.select_pages_gauss(shape, box, mu, var, sl, alpha, par["delta"], sel, cnt,
                                         n_sigma=par["n_sigma"])
                E.entmax_decode_sparse(shape, q, kp, vp, pt, sl, sel, cnt, alpha, out_es)
                E.softmax_decode_sparse(shape, q, kp, vp, pt, sl, sel, cnt, out_ss, lse=lse_s)
                torch.cuda.synchronize()
                inside = ar[None, None, :] < cnt[:, :, None]
                keep = torch.zeros((B, Hq, MP + 1), dtype=torch.bool, device=dev)   # column MP: unused slots
                keep.scatter_(2, torch.where(inside, sel, torch.full_like(sel, MP)).long(), inside)
                T = keep[:, :, :MP].repeat_interleave(P, dim=2) & valid[:, None, :]
                recall = (supp & T).sum(-1).double() / n_supp.clamp(min=1)
                d_ent = (wfull.double() * (~T)).sum(-1)
                d_sm = (-torch.expm1((lse_s - lse_f).double())).clamp(min=0.0)
                ee, ne = rel(out_es, out_ef)
                es, ns_ = rel(out_ss, out_sf)
                r_ent, r_sm = ee / ne.clamp(min=1e-30), es / ns_.clamp(min=1e-30)
                big_e, big_s = d_ent > 1e-6, d_sm > 1e-6
                ratio_e = float((ee / (2 * bnd * d_ent))[big_e].max()) if bool(big_e.any()) else None
                ratio_s = float((es / (2 * bnd * d_sm))[big_s].max()) if bool(big_s.any()) else None
                exact = ~big_e
                row = {"workload": name, "alpha": alpha, "selector": kind, **par,
                       "kept_pages_mean": round(float(cnt.double().mean()), 2),
                       "kept_token_frac": float(T.sum(-1).double().mean() / sl.double().mean()),
                       "support_mean": round(float(n_supp.mean()), 1),
                       "recall_mean": float(recall.mean()), "recall_min": float(recall.min()),
                       "rows_support_kept": float((recall == 1.0).double().mean()),
                       "delta_entmax_mean": float(d_ent.mean()), "delta_softmax_mean": float(d_sm.mean()),
                       "rel_err_entmax_mean": float(r_ent.mean()), "rel_err_softmax_mean": float(r_sm.mean()),
                       "rows_entmax_less_mass": float((d_ent <= d_sm).double().mean()),
                       "err_over_bound_max_entmax": ratio_e, "err_over_bound_max_softmax": ratio_s,
                       "err_where_delta0_max": float(ee[exact].max()) if bool(exact.any()) else None}
                log(f"[quality] {name} a={alpha} {kind} {par}: pages {row['kept_pages_mean']} "
                    f"recall {row['recall_mean']:.3f} delta ent {row['delta_entmax_mean']:.3e} "
                    f"sm {row['delta_softmax_mean']:.3e} relerr ent {row['rel_err_entmax_mean']:.3e} "
                    f"sm {row['rel_err_softmax_mean']:.3e}")
                rows.append(row)
            del wfull, supp
        del inp, meta, box, mu, var, vn, vnb
        torch.cuda.empty_cache()
    print(json.dumps({"quality_sweep": rows, "seed": args.seed,
                      "note": "selection on box/mu/var from score_pages; T = tokens of the kept pages"}),
          flush=True)


SCORE_SOURCES = ("sparse_decode_attention_page_amd/csrc/score.hip", "sparse_decode_attention_page_amd/csrc/common.hpp")


def score_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def score_traffic(workload):
    """HBM bytes per score_pages launch from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a plain copy), or None when the
    scorer's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"score_pages_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != score_sources_sha():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, shape, wl, alpha, policy):
    """The oracle (plain fp64 C, OpenMP over query rows) on the same workload:
    score_pages + selection + sparse decode for every query row, repeated until
    about 10 s of work have run (the metadata build is not part of a step).  A
    workload whose step would take the oracle more than ~30 s is cut to whole
    KV-head groups of batch 0 and scaled to the full step."""
    import numpy as np
    import oracle

    B, Hq, Hkv = inp.B, inp.Hq, inp.Hkv
    G = Hq // Hkv
    osh = oracle.Shape(B, Hq, Hkv, inp.d, inp.P, inp.max_pages, inp.num_phys, inp.dtype)
    t0 = time.time()
    k = inp.host("k_pool")
    v = inp.host("v_pool")
    q = inp.host("q")
    pt = inp.page_table.cpu().numpy()
    sl = inp.seq_lens.cpu().numpy()
    meta = oracle.build_page_meta(osh, k, pt, sl)
    log(f"[bench] oracle inputs ready in {time.time() - t0:.1f}s")

    def step(rows):
        t1 = time.perf_counter()
        box, mu, var = oracle.score_pages(osh, q, meta, pt, sl, rows=rows)
        if policy == "gauss":
            sel, cnt, _ = oracle.select_gauss(osh, box, mu, var, sl, alpha, wl.delta, rows=rows)
        else:
            sel, cnt = oracle.select_topk(osh, box, sl, wl.topk or 64, rows=rows)
        oracle.entmax_decode(osh, q, k, v, pt, sl, alpha, sel, cnt, rows=rows)
        return time.perf_counter() - t1

    all_rows = list(range(B * Hq))
    probe = all_rows[:G]
    dt_probe = step(probe)
    omp = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    # rows run in parallel over min(rows, threads) threads
    est_full = dt_probe * len(all_rows) / len(probe) * min(len(probe), omp) / min(len(all_rows), omp)
    if est_full <= 30.0:
        rows = all_rows
        reps = max(1, int(10.0 / max(est_full, 1e-3)))
    else:
        groups = max(1, min(Hkv, int(30.0 / est_full * Hkv)))
        rows = list(range(groups * G))
        reps = 1
    total = 0.0
    for _ in range(reps):
        total += step(rows)
    dt = total / reps
    scale = len(all_rows) / len(rows)
    threads = min(len(rows), omp, os.cpu_count() or 1)
    sample = (f"score+select+sparse decode of {len(rows)} of {len(all_rows)} query rows, "
              f"{reps} run(s) averaged ({total:.1f}s of work)"
              + (f", scaled x{scale:g}" if scale != 1 else ""))
    log(f"[bench] cpu baseline: {dt * scale * 1e3:.1f} ms/step ({sample}, {threads} threads)")
    res = {"value": round(dt * scale * 1e6, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
           "sample": sample, "cpu_model": cpu_model()}
    # one thread on the two small workloads, in a child process that never touches the GPU
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-1t"],
                           env=dict(os.environ, OMP_NUM_THREADS="1"), capture_output=True, text=True,
                           timeout=300)
        res["single_thread_us_per_step"] = json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:  # reported, never fatal
        res["single_thread_us_per_step"] = {"error": str(e)[:200]}
    log(f"[bench] oracle, one thread: {res['single_thread_us_per_step']}")
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def oracle_small_steps():
    """The oracle's step (score + Gaussian selection + sparse decode, every query
    row) on the 4k-token and 32k-token workloads, repeated to about a second of
    work each; us per step."""
    import oracle
    from sparse_decode_attention_page_amd import synth

    out = {}
    for name in ("tiny_4k", "gqa_32k"):
        wl = synth.WORKLOADS[name]
        inp = synth.make(wl, 0)
        osh = oracle.Shape(inp.B, inp.Hq, inp.Hkv, inp.d, inp.P, inp.max_pages, inp.num_phys, inp.dtype)
        meta = oracle.build_page_meta(osh, inp.k_pool, inp.page_table, inp.seq_lens)
        alpha = wl.alphas[0]
        n, total = 0, 0.0
        while total < 1.0 and n < 1000:
            t1 = time.perf_counter()
            box, mu, var = oracle.score_pages(osh, inp.q, meta, inp.page_table, inp.seq_lens)
            sel, cnt, _ = oracle.select_gauss(osh, box, mu, var, inp.seq_lens, alpha, wl.delta)
            oracle.entmax_decode(osh, inp.q, inp.k_pool, inp.v_pool, inp.page_table, inp.seq_lens, alpha,
                                 sel, cnt)
            total += time.perf_counter() - t1
            n += 1
        out[name] = round(total / n * 1e6, 1)
    return out


if __name__ == "__main__":
    main()
