"""Seeded synthetic decode workloads (inputs only -- none of the method's arithmetic).

This module is the one piece shared by the HIP path's tests/benchmark and the
CPU oracle: it draws q, a paged K/V pool, a page table and sequence lengths.
Everything is numpy ``default_rng(seed)`` (PCG64) float32 draws, stored as
float32 or rounded to bfloat16 (round-to-nearest-even) as the workload says.

The EntmaxKV summary ("Resumen Tecnico: EntmaxKV ...", gist.science/es/paper/
2605.21649, section 4) evaluates on long-context retrieval/LM suites and on
efficiency runs up to 1M tokens; none of those inputs exist here.  These
workloads stand in for them: Gaussian keys with planted "needle" tokens whose
key points along the query (k = g q/|q| + N(0, 0.1^2) per coordinate, g = 4), at
the context lengths the summary reports.  The "_passage" variants plant runs of
16 such tokens with g = 8 instead: short passages that stand out of the bulk.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    P: int
    dtype: str                 # "f32" | "bf16"
    ctx: tuple                 # per-sequence context lengths (len B) or a (lo, hi) range drawn per b
    ragged: bool = False
    planted_per_kv: int = 0
    planted_layout: str = "random"   # "random" | "even"
    drift_per_1k: float = 0.0
    diffuse_first_half: bool = False
    shuffle_pages: bool = False
    alphas: tuple = (1.5,)
    topk: int = 0
    delta: float = 0.5
    policy: str = "gauss"      # "gauss" | "topk" | "mixed" (even b top-k, odd b Gaussian)
    needle_gain: float = 4.0   # planted key = needle_gain * q/|q| + noise (score ~ needle_gain)
    needle_run: int = 1        # consecutive planted tokens per item (a short passage when > 1)
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # tiny exact check: 1 head, fp32, 4096 tokens in 256 pages of 16
    "tiny_4k": Workload("tiny_4k", 1, 1, 1, 64, 16, "f32", (4096,), planted_per_kv=8,
                        alphas=(1.5,), topk=32, delta=0.5, policy="both"),
    # GQA slice: 32 q heads / 8 KV heads, bf16, 32k tokens, pages of 16, drifting keys
    "gqa_32k": Workload("gqa_32k", 1, 32, 8, 64, 16, "bf16", (32768,), planted_per_kv=16,
                        drift_per_1k=0.05, alphas=(1.5,), topk=64, delta=0.5, policy="both"),
    # 128k tokens, pages of 32, 64 evenly spaced needles per KV head
    "gqa_128k": Workload("gqa_128k", 1, 32, 8, 64, 32, "bf16", (131072,), planted_per_kv=64,
                         planted_layout="even", alphas=(1.5, 2.0), topk=64, delta=0.5, policy="both"),
    # long-context decode: 1M tokens, pages of 64 (about 2 GiB of K+V)
    "long_1m": Workload("long_1m", 1, 32, 8, 64, 64, "bf16", (1048576,), planted_per_kv=32,
                        alphas=(1.5,), topk=64, delta=0.5, policy="gauss"),
    # batched ragged decode: 16 sequences of 16k..256k tokens, d=128, shuffled page pool
    "batch16_ragged": Workload("batch16_ragged", 16, 32, 8, 128, 32, "bf16", (16384, 262144),
                               ragged=True, planted_per_kv=64, diffuse_first_half=True,
                               shuffle_pages=True, alphas=(1.5,), topk=128, delta=0.5,
                               policy="mixed"),
}
# the same shapes with planted passages: runs of 16 consecutive tokens whose
# keys point along the query, scoring ~8 against a bulk maximum of ~5 at 1M
# tokens (the few relevant passages a retrieval query attends to)
WORKLOADS["gqa_128k_passage"] = Workload("gqa_128k_passage", 1, 32, 8, 64, 32, "bf16", (131072,),
                                         planted_per_kv=64, planted_layout="even", alphas=(1.5, 2.0),
                                         topk=64, delta=0.5, policy="both", needle_gain=8.0, needle_run=16)
WORKLOADS["long_1m_passage"] = Workload("long_1m_passage", 1, 32, 8, 64, 64, "bf16", (1048576,),
                                        planted_per_kv=32, alphas=(1.5,), topk=64, delta=0.5,
                                        policy="gauss", needle_gain=8.0, needle_run=16)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return (a if dtype == "f32" else bf16_bits_to_f32(a)).astype(np.float64)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32) if dtype == "f32" else to_bf16_bits(x)


@dataclass
class Inputs:
    wl: Workload
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    P: int
    dtype: str
    max_pages: int
    num_phys: int
    q: np.ndarray            # [B][Hq][d] storage dtype
    k_pool: np.ndarray       # [num_phys][Hkv][P][d]
    v_pool: np.ndarray
    page_table: np.ndarray   # int32 [B][max_pages]
    seq_lens: np.ndarray     # int32 [B]
    planted: list            # per b: list of (kv_head, q_head, token position)
    seq_mask_topk: np.ndarray  # uint8 [B]: rows that use the top-k policy
    seq_mask_gauss: np.ndarray


def make(wl: Workload | str, seed: int = 0, ctx_override=None, shuffle=None) -> Inputs:
    """Draw one seeded instance of a workload.

    ctx_override: replace the context length(s) (tests use it to shrink a workload
    while keeping its structure).  shuffle: force a shuffled physical page pool.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, P = wl.B, wl.Hq, wl.Hkv, wl.d, wl.P
    G = Hq // Hkv
    if ctx_override is not None:
        ctx = list(ctx_override) if np.ndim(ctx_override) else [int(ctx_override)] * B
        ctx = (ctx * B)[:B] if len(ctx) < B else ctx
    elif wl.ragged:
        ctx = [int(x) for x in rng.integers(wl.ctx[0], wl.ctx[1] + 1, size=B)]
    else:
        ctx = [int(wl.ctx[0])] * B
    seq_lens = np.asarray(ctx, dtype=np.int32)
    npages = [(L + P - 1) // P for L in ctx]
    max_pages = max(max(npages), 1)
    num_phys = sum(npages)
    do_shuffle = wl.shuffle_pages if shuffle is None else shuffle
    perm = rng.permutation(num_phys) if do_shuffle else np.arange(num_phys)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        page_table[b, : npages[b]] = perm[off: off + npages[b]]
        off += npages[b]

    qf = rng.standard_normal((B, Hq, d), dtype=np.float32)
    q = _store(qf, wl.dtype)
    qs = storage_to_f64(q, wl.dtype)

    k_pool = np.zeros((num_phys, Hkv, P, d), dtype=np.float32 if wl.dtype == "f32" else np.uint16)
    v_pool = np.zeros_like(k_pool)
    planted = []
    for b in range(B):
        L, nb = ctx[b], npages[b]
        diffuse = wl.diffuse_first_half and b < B // 2
        plist = []
        for g in range(Hkv):
            # keys and values of every logical page of this (b, g), position-major
            kf = rng.standard_normal((nb * P, d), dtype=np.float32)
            vf = rng.standard_normal((nb * P, d), dtype=np.float32)
            if diffuse:
                kf *= np.float32(8.0 / np.sqrt(L))
            if wl.drift_per_1k:
                r = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=d)
                t = np.arange(nb * P, dtype=np.float32)[:, None]
                kf += np.float32(wl.drift_per_1k) * r[None, :] * t / np.float32(1000.0)
            if wl.planted_per_kv and not diffuse:
                n = min(wl.planted_per_kv, L)
                if wl.planted_layout == "even":
                    pos = ((np.arange(n) + 0.5) * L / n).astype(np.int64)
                else:
                    pos = np.sort(rng.choice(L, size=n, replace=False))
                for j, t0 in enumerate(pos):
                    h = g * G + (j % G)
                    qv = qs[b, h]
                    for t in range(int(t0), min(int(t0) + wl.needle_run, L)):
                        noise = rng.standard_normal(d, dtype=np.float32) * np.float32(0.1)
                        kf[t] = (float(wl.needle_gain) * qv / np.linalg.norm(qv)).astype(np.float32) + noise
                        plist.append((g, h, int(t)))
            if L < nb * P:  # slots past the end of the sequence stay zero
                kf[L:] = 0.0
                vf[L:] = 0.0
            ks, vs = _store(kf, wl.dtype), _store(vf, wl.dtype)
            phys = page_table[b, :nb]
            k_pool[phys, g] = ks.reshape(nb, P, d)
            v_pool[phys, g] = vs.reshape(nb, P, d)
        planted.append(plist)

    if wl.policy == "mixed":
        mt = np.array([1 if b % 2 == 0 else 0 for b in range(B)], dtype=np.uint8)
    elif wl.policy == "topk":
        mt = np.ones(B, np.uint8)
    elif wl.policy == "gauss":
        mt = np.zeros(B, np.uint8)
    else:  # both policies evaluated on every row
        mt = np.ones(B, np.uint8)
    mg = (1 - mt).astype(np.uint8) if wl.policy == "mixed" else (
        np.ones(B, np.uint8) if wl.policy in ("gauss", "both") else np.zeros(B, np.uint8))
    return Inputs(wl, seed, B, Hq, Hkv, d, P, wl.dtype, max_pages, num_phys, q, k_pool, v_pool,
                  page_table, seq_lens, planted, mt, mg)


def random_small(seed: int, B=2, Hq=4, Hkv=2, d=64, P=16, dtype="bf16", ctx=(200, 77),
                 shuffle=True, planted_per_kv=4, scale_keys=1.0) -> Inputs:
    """Small ragged instance for parity tests (several tiles, a ragged tail)."""
    wl = Workload("small", B, Hq, Hkv, d, P, dtype, tuple(ctx), planted_per_kv=planted_per_kv,
                  shuffle_pages=shuffle, topk=4, delta=0.5, policy="both")
    inp = make(wl, seed, ctx_override=list(ctx), shuffle=shuffle)
    if scale_keys != 1.0:
        kf = storage_to_f64(inp.k_pool, dtype) * scale_keys
        inp.k_pool = _store(kf.astype(np.float32), dtype)
    return inp


@dataclass
class DeviceInputs:
    """A workload drawn directly on the GPU (torch Philox, seeded).  Same recipe
    as make(); different random stream.  Tensors: q [B][Hq][d], k_pool/v_pool
    [num_phys][Hkv][P][d] (bf16 or fp32), page_table/seq_lens int32."""
    wl: Workload
    seed: int
    B: int
    Hq: int
    Hkv: int
    d: int
    P: int
    dtype: str
    max_pages: int
    num_phys: int
    q: object
    k_pool: object
    v_pool: object
    page_table: object
    seq_lens: object
    planted: list
    seq_mask_topk: object
    seq_mask_gauss: object

    def host(self, name):
        """Raw host storage of a tensor (uint16 bit patterns for bf16), for the oracle."""
        import torch
        t = getattr(self, name)
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()


def make_device(wl: Workload | str, seed: int = 0, ctx_override=None, device="cuda") -> DeviceInputs:
    import torch
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    hgen = torch.Generator()
    hgen.manual_seed(int(seed))
    B, Hq, Hkv, d, P = wl.B, wl.Hq, wl.Hkv, wl.d, wl.P
    G = Hq // Hkv
    if ctx_override is not None:
        ctx = list(ctx_override) if np.ndim(ctx_override) else [int(ctx_override)] * B
        ctx = (ctx * B)[:B] if len(ctx) < B else ctx
    elif wl.ragged:
        ctx = [int(x) for x in torch.randint(wl.ctx[0], wl.ctx[1] + 1, (B,), generator=hgen)]
    else:
        ctx = [int(wl.ctx[0])] * B
    npages = [(L + P - 1) // P for L in ctx]
    max_pages = max(max(npages), 1)
    num_phys = sum(npages)
    perm = torch.randperm(num_phys, generator=hgen) if wl.shuffle_pages else torch.arange(num_phys)
    pt = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        pt[b, : npages[b]] = perm[off: off + npages[b]].to(torch.int32)
        off += npages[b]
    kdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q = torch.randn((B, Hq, d), generator=gen, device=device, dtype=torch.float32).to(kdt)
    qs = q.to(torch.float64)
    k_pool = torch.zeros((num_phys, Hkv, P, d), dtype=kdt, device=device)
    v_pool = torch.zeros_like(k_pool)
    planted = []
    for b in range(B):
        L, nb = ctx[b], npages[b]
        diffuse = wl.diffuse_first_half and b < B // 2
        phys = pt[b, :nb].to(device=device, dtype=torch.int64)
        plist = []
        for g in range(Hkv):
            kf = torch.randn((nb * P, d), generator=gen, device=device, dtype=torch.float32)
            vf = torch.randn((nb * P, d), generator=gen, device=device, dtype=torch.float32)
            if diffuse:
                kf *= 8.0 / float(np.sqrt(L))
            if wl.drift_per_1k:
                r = torch.randint(0, 2, (d,), generator=gen, device=device).to(torch.float32) * 2 - 1
                t = torch.arange(nb * P, device=device, dtype=torch.float32)[:, None]
                kf += float(wl.drift_per_1k) * r[None, :] * t / 1000.0
            if wl.planted_per_kv and not diffuse:
                n = min(wl.planted_per_kv, L)
                if wl.planted_layout == "even":
                    pos = ((torch.arange(n, dtype=torch.float64) + 0.5) * L / n).to(torch.int64)
                else:
                    pos = torch.sort(torch.randperm(L, generator=hgen)[:n]).values
                hs = torch.tensor([g * G + (j % G) for j in range(n)], device=device)
                qv = qs[b, hs]                                           # [n, d]
                dirs = (float(wl.needle_gain) * qv / torch.linalg.norm(qv, dim=1, keepdim=True)).to(torch.float32)
                for o in range(wl.needle_run):
                    noise = torch.randn((n, d), generator=gen, device=device, dtype=torch.float32) * 0.1
                    tt = pos + o
                    ok = tt < L
                    kf[tt[ok].to(device)] = (dirs + noise)[ok.to(device)]
                    plist += [(g, int(hs[j]), int(tt[j])) for j in range(n) if bool(ok[j])]
            if L < nb * P:
                kf[L:] = 0.0
                vf[L:] = 0.0
            k_pool[phys, g] = kf.view(nb, P, d).to(kdt)
            v_pool[phys, g] = vf.view(nb, P, d).to(kdt)
            del kf, vf
        planted.append(plist)
    if wl.policy == "mixed":
        mt = np.array([1 if b % 2 == 0 else 0 for b in range(B)], dtype=np.uint8)
        mg = 1 - mt
    elif wl.policy == "topk":
        mt, mg = np.ones(B, np.uint8), np.zeros(B, np.uint8)
    elif wl.policy == "gauss":
        mt, mg = np.zeros(B, np.uint8), np.ones(B, np.uint8)
    else:
        mt, mg = np.ones(B, np.uint8), np.ones(B, np.uint8)
    return DeviceInputs(wl, seed, B, Hq, Hkv, d, P, wl.dtype, max_pages, num_phys, q, k_pool, v_pool,
                        pt.to(device), torch.tensor(ctx, dtype=torch.int32, device=device), planted,
                        torch.from_numpy(mt.astype(np.uint8)).to(device),
                        torch.from_numpy(mg.astype(np.uint8)).to(device))
