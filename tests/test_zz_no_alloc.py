"""score_pages_noalloc (no workspace: the library's static device scratch)
against score_pages with a caller workspace, through the C ABI, on two calls in
a row -- the second with a smaller input, so the scratch holds the first call's
table when the second starts.  Outputs must agree bit for bit (same kernel,
same fixed-order fp64 sums), and with the oracle."""
import numpy as np
import pytest

import oracle
import sparse_decode_attention_page_amd as E
from sparse_decode_attention_page_amd import synth
from gpu_util import Dev, torch

pytestmark = pytest.mark.gpu

CASES = [  # (seed, B, Hq, Hkv, d, P, dtype, ctx): the second is smaller than the first
    (3, 2, 32, 8, 128, 32, "bf16", (9000, 4100)),
    (4, 1, 8, 2, 64, 16, "bf16", (1500,)),
]


def _run(case):
    seed, B, Hq, Hkv, d, P, dtype, ctx = case
    t = torch()
    inp = synth.random_small(seed, B=B, Hq=Hq, Hkv=Hkv, d=d, P=P, dtype=dtype, ctx=ctx)
    D = Dev(inp)
    meta = D.zeros_meta()
    E.build_page_meta(D.shape, D.k, D.pt, D.sl, meta)
    ref = [D.per_page() for _ in range(3)]
    got = [D.per_page() for _ in range(3)]
    E.score_pages(D.shape, D.q, meta, D.pt, D.sl, *ref)
    E.score_pages_noalloc(D.shape, D.q, meta, D.pt, D.sl, *got)
    t.cuda.synchronize()
    for r, g, name in zip(ref, got, ("box", "mu", "var")):
        rb, gb = r.view(t.int32), g.view(t.int32)  # NaN fill past each row's pages compares as bits
        assert t.equal(rb, gb), f"{name} differs from score_pages (case {case[:1]})"
    meta_h = meta.view(t.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else meta.cpu().numpy()
    bo, mo, vo = oracle.score_pages(D.oshape, inp.q, meta_h, inp.page_table, inp.seq_lens)
    for g, w in zip(got, (bo, mo, vo)):
        gh = g.cpu().numpy()
        for b in range(B):
            npg = (int(inp.seq_lens[b]) + P - 1) // P
            assert np.array_equal(gh[b, :, :npg].view(np.int32), w[b, :, :npg].view(np.int32))


def test_noalloc_matches_score_pages_twice():
    need = [32 * c[1] * c[2] * c[4] for c in CASES]
    assert need[1] < need[0] <= E.score_scratch_bytes()
    for case in CASES:
        _run(case)
