"""CPU checks of the Python binding: every wrapper checks each tensor's element
count against the shape (and that it lives on the device) before the library
is called or a workspace allocated, so an undersized buffer raises ValueError
instead of reaching a kernel."""
import pytest
import torch

import sparse_decode_attention_page_amd as E

B, HQ, HKV, D, P, MP, NP = 2, 8, 2, 64, 16, 12, 30


def shape():
    return E.Shape(B, HQ, HKV, D, P, MP, NP, E.BF16, 0.0)


class Dev(torch.Tensor):
    """A host tensor that reports itself as a device tensor, so that the size
    checks of every argument are reached (no call below gets past them)."""

    @property
    def is_cuda(self):
        return True


def t(n, dtype=torch.float32):
    return torch.zeros(n, dtype=dtype)


def full_args():
    """Correctly sized (CPU) tensors for every buffer of the hot-path calls."""
    bf, i32, f32, f64 = torch.bfloat16, torch.int32, torch.float32, torch.float64
    return dict(q=t(B * HQ * D, bf), k_pool=t(NP * HKV * P * D, bf), v_pool=t(NP * HKV * P * D, bf),
                meta=t(NP * HKV * 4 * D, bf), page_table=t(B * MP, i32), seq_lens=t(B, i32),
                box=t(B * HQ * MP), mu=t(B * HQ * MP), var=t(B * HQ * MP), sel_idx=t(B * HQ * MP, i32),
                sel_cnt=t(B * HQ, i32), out=t(B * HQ * D, f32), tau=t(B * HQ, f64),
                weights_out=t(B * HQ * MP * P, f32), lse=t(B * HQ, f32), meta8=t(NP * HKV * 6 * D, torch.uint8),
                k_new=t(B * HKV * D, bf), v_new=t(B * HKV * D, bf))


CALLS = {
    "score_pages": lambda a: E.score_pages(shape(), a["q"], a["meta"], a["page_table"], a["seq_lens"], a["box"],
                                           a["mu"], a["var"]),
    "select_pages_topk": lambda a: E.select_pages_topk(shape(), a["box"], a["seq_lens"], 4, a["sel_idx"],
                                                       a["sel_cnt"]),
    "select_pages_gauss": lambda a: E.select_pages_gauss(shape(), a["box"], a["mu"], a["var"], a["seq_lens"], 1.5,
                                                         0.5, a["sel_idx"], a["sel_cnt"], tau_hat=a["tau"]),
    "entmax_decode_sparse": lambda a: E.entmax_decode_sparse(shape(), a["q"], a["k_pool"], a["v_pool"],
                                                             a["page_table"], a["seq_lens"], a["sel_idx"],
                                                             a["sel_cnt"], 1.5, a["out"], tau=a["tau"],
                                                             weights_out=a["weights_out"]),
    "entmax_decode_full": lambda a: E.entmax_decode_full(shape(), a["q"], a["k_pool"], a["v_pool"], a["page_table"],
                                                         a["seq_lens"], 1.5, a["out"], tau=a["tau"],
                                                         weights_out=a["weights_out"]),
    "softmax_decode_full": lambda a: E.softmax_decode_full(shape(), a["q"], a["k_pool"], a["v_pool"],
                                                           a["page_table"], a["seq_lens"], a["out"], lse=a["lse"]),
    "softmax_decode_sparse": lambda a: E.softmax_decode_sparse(shape(), a["q"], a["k_pool"], a["v_pool"],
                                                               a["page_table"], a["seq_lens"], a["sel_idx"],
                                                               a["sel_cnt"], a["out"], lse=a["lse"]),
    "build_page_meta": lambda a: E.build_page_meta(shape(), a["k_pool"], a["page_table"], a["seq_lens"], a["meta"]),
    "build_page_meta_f8": lambda a: E.build_page_meta_f8(shape(), a["k_pool"], a["page_table"], a["seq_lens"],
                                                         a["meta8"]),
    "score_pages_f8": lambda a: E.score_pages_f8(shape(), a["q"], a["meta8"], a["page_table"], a["seq_lens"],
                                                 a["box"], a["mu"], a["var"]),
    "append_token": lambda a: E.append_token(shape(), a["k_new"], a["v_new"], a["k_pool"], a["v_pool"],
                                             a["page_table"], a["seq_lens"], a["meta"]),
    "append_token_f8": lambda a: E.append_token(shape(), a["k_new"], a["v_new"], a["k_pool"], a["v_pool"],
                                                a["page_table"], a["seq_lens"], a["meta8"], compact=True),
}

# the buffers each call reads or writes
USES = {
    "score_pages": ("q", "meta", "page_table", "seq_lens", "box", "mu", "var"),
    "select_pages_topk": ("box", "seq_lens", "sel_idx", "sel_cnt"),
    "select_pages_gauss": ("box", "mu", "var", "seq_lens", "sel_idx", "sel_cnt", "tau"),
    "entmax_decode_sparse": ("q", "k_pool", "v_pool", "page_table", "seq_lens", "sel_idx", "sel_cnt", "out", "tau",
                             "weights_out"),
    "entmax_decode_full": ("q", "k_pool", "v_pool", "page_table", "seq_lens", "out", "tau", "weights_out"),
    "softmax_decode_full": ("q", "k_pool", "v_pool", "page_table", "seq_lens", "out", "lse"),
    "softmax_decode_sparse": ("q", "k_pool", "v_pool", "page_table", "seq_lens", "sel_idx", "sel_cnt", "out", "lse"),
    "build_page_meta": ("k_pool", "page_table", "seq_lens", "meta"),
    "build_page_meta_f8": ("k_pool", "page_table", "seq_lens", "meta8"),
    "score_pages_f8": ("q", "meta8", "page_table", "seq_lens", "box", "mu", "var"),
    "append_token": ("k_new", "v_new", "k_pool", "v_pool", "page_table", "seq_lens", "meta"),
    "append_token_f8": ("k_new", "v_new", "k_pool", "v_pool", "page_table", "seq_lens", "meta8"),
}


@pytest.mark.parametrize("call", sorted(CALLS))
def test_undersized_buffers_raise(call):
    for name in USES[call]:
        a = {k: v.as_subclass(Dev) for k, v in full_args().items()}
        a[name] = a[name][:-1]  # one element short
        with pytest.raises(ValueError, match="elements"):
            CALLS[call](a)


@pytest.mark.parametrize("call", sorted(CALLS))
def test_host_tensors_raise(call):
    with pytest.raises(ValueError, match="device tensor"):
        CALLS[call](full_args())


def test_group_selection_sizes():
    a = {k: v.as_subclass(Dev) for k, v in full_args().items()}
    gsel, gcnt = t(B * HKV * MP, torch.int32).as_subclass(Dev), t(B * HKV, torch.int32).as_subclass(Dev)
    with pytest.raises(ValueError, match="elements"):
        E.select_pages_topk_group(shape(), a["box"], a["seq_lens"], 4, gsel[:-1], gcnt)
    with pytest.raises(ValueError, match="elements"):
        E.select_pages_gauss_group(shape(), a["box"], a["mu"], a["var"], a["seq_lens"], 1.5, 0.5, gsel, gcnt[:-1])
    with pytest.raises(ValueError, match="elements"):
        E.entmax_decode_sparse_group(shape(), a["q"], a["k_pool"], a["v_pool"], a["page_table"], a["seq_lens"],
                                     gsel, gcnt[:-1], 1.5, a["out"])
