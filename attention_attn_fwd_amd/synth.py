"""Seeded synthetic inputs for sink attention (CPU torch tensors).

This module only draws random numbers; it holds none of the attention
arithmetic.  Tests feed the same draws to the HIP library and to the fp64
oracle, and bench.py times the library on them.

Workload shapes are gpt-oss shaped: 64 query heads over 8 KV heads, head
dimension 64, alternating sliding-window-128 / full-causal layers (Megatron-LM
issue "gpt-oss implementation", "Alternating Sliding-Window Attention
Pattern"), and a decode batch of 128 sequences of at most 1024 tokens (the
serve command in tpu-inference PR "[GPT-OSS] JAX implementation of GPT-OSS":
max-num-seqs 128, max-model-len 1024).  Values are bf16 draws of N(0, std^2)
and the per-head sinks fp32 draws of N(0, 1).

Draw order inside one generator: (decode lengths), q, k, v, sinks, (dout).
"""

from dataclasses import dataclass

import torch

__all__ = ["PrefillCase", "DecodeCase", "PagedDecodeCase", "VarlenCase", "CONFIGS", "make_prefill", "make_dout",
           "make_decode", "make_paged_decode", "make_varlen", "draw_doc_lengths", "config_inputs", "VARLEN_WORKLOAD",
           "varlen_workload"]

SLIDING_WINDOW = 128


@dataclass
class PrefillCase:
    q: torch.Tensor      # bf16 [B, S, Hq, D]
    k: torch.Tensor      # bf16 [B, S, Hkv, D]
    v: torch.Tensor      # bf16 [B, S, Hkv, D]
    sinks: torch.Tensor  # fp32 [Hq]
    scale: float


@dataclass
class DecodeCase:
    q: torch.Tensor           # bf16 [N, Hq, D]
    k_cache: torch.Tensor     # bf16 [T, Hkv, D]
    v_cache: torch.Tensor     # bf16 [T, Hkv, D]
    cu_seqlens: torch.Tensor  # int32 [N + 1]
    sinks: torch.Tensor       # fp32 [Hq]
    max_seqlen: int
    scale: float


def _normal_bf16(gen, shape, std):
    x = torch.randn(shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(torch.bfloat16)


def make_prefill(B, S, Hq, Hkv, D=64, std=1.0, seed=0, scale=None):
    gen = torch.Generator().manual_seed(seed)
    q = _normal_bf16(gen, (B, S, Hq, D), std)
    k = _normal_bf16(gen, (B, S, Hkv, D), std)
    v = _normal_bf16(gen, (B, S, Hkv, D), std)
    sinks = torch.randn((Hq,), generator=gen, dtype=torch.float32)
    return PrefillCase(q, k, v, sinks, (1.0 / D ** 0.5) if scale is None else scale)


def make_dout(shape, seed):
    gen = torch.Generator().manual_seed(seed)
    return _normal_bf16(gen, shape, 1.0)


def make_decode(N, Hq, Hkv, D=64, max_len=1024, seed=0, lengths=None, std=1.0):
    """Packed decode batch; lengths ~ U{1..max_len} unless given explicitly."""
    gen = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = torch.randint(1, max_len + 1, (N,), generator=gen, dtype=torch.int64)
    else:
        lengths = torch.as_tensor(lengths, dtype=torch.int64)
    cu = torch.zeros(N + 1, dtype=torch.int64)
    cu[1:] = torch.cumsum(lengths, 0)
    T = int(cu[-1])
    q = _normal_bf16(gen, (N, Hq, D), std)
    kc = _normal_bf16(gen, (T, Hkv, D), std)
    vc = _normal_bf16(gen, (T, Hkv, D), std)
    sinks = torch.randn((Hq,), generator=gen, dtype=torch.float32)
    max_seqlen = max(1, int(lengths.max())) if N > 0 else 1
    return DecodeCase(q, kc, vc, cu.to(torch.int32), sinks, max_seqlen, 1.0 / D ** 0.5)


@dataclass
class PagedDecodeCase:
    q: torch.Tensor            # bf16 [N, Hq, D]
    k_pages: torch.Tensor      # bf16 [P, page_size, Hkv, D]
    v_pages: torch.Tensor      # bf16 [P, page_size, Hkv, D]
    block_table: torch.Tensor  # int32 [N, pages_per_seq]
    seq_lens: torch.Tensor     # int32 [N]
    sinks: torch.Tensor        # fp32 [Hq]
    ring_tokens: int           # 0 = linear cache
    max_seqlen: int
    scale: float
    full: DecodeCase           # the same sequences as one packed cache (every position kept)


def make_paged_decode(N, Hq, Hkv, page_size, D=64, max_len=1024, seed=0, lengths=None, ring_tokens=0,
                      spare_pages=3):
    """A paged decode batch holding the sequences of make_decode(N, ..., seed):
    each sequence's positions are written in order into its slots (slot t, or
    t mod ring_tokens for a ring, so later positions overwrite earlier ones),
    through a block table of randomly permuted page indices.  Slots never
    written hold 1e4 (a misread would show)."""
    full = make_decode(N, Hq, Hkv, D=D, max_len=max_len, seed=seed, lengths=lengths)
    lens = (full.cu_seqlens[1:] - full.cu_seqlens[:-1]).tolist()
    if ring_tokens:
        pps = ring_tokens // page_size
    else:
        pps = max(1, (max(lens + [1]) + page_size - 1) // page_size)
    n_pages = N * pps + spare_pages
    gen = torch.Generator().manual_seed(seed + 7919)
    perm = torch.randperm(n_pages, generator=gen)[: N * pps].to(torch.int32)
    block_table = perm.reshape(N, pps).contiguous()
    k_pages = torch.full((n_pages, page_size, Hkv, D), 1e4).to(torch.bfloat16)
    v_pages = torch.full((n_pages, page_size, Hkv, D), 1e4).to(torch.bfloat16)
    for n, L in enumerate(lens):
        base = int(full.cu_seqlens[n])
        for t in range(L):
            slot = t % ring_tokens if ring_tokens else t
            page = int(block_table[n, slot // page_size])
            k_pages[page, slot % page_size] = full.k_cache[base + t]
            v_pages[page, slot % page_size] = full.v_cache[base + t]
    return PagedDecodeCase(full.q, k_pages, v_pages, block_table, torch.tensor(lens, dtype=torch.int32),
                           full.sinks, ring_tokens, full.max_seqlen, full.scale, full)


@dataclass
class VarlenCase:
    q: torch.Tensor           # bf16 [T, Hq, D]
    k: torch.Tensor           # bf16 [T, Hkv, D]
    v: torch.Tensor           # bf16 [T, Hkv, D]
    cu_seqlens: torch.Tensor  # int32 [N + 1]; document b = rows cu[b] .. cu[b+1]-1
    sinks: torch.Tensor       # fp32 [Hq]
    max_seqlen: int
    scale: float


def draw_doc_lengths(total, max_len, gen):
    """Document lengths ~ U{1..max_len} drawn until they cover `total` tokens;
    the last one is cut so that the lengths sum to `total` exactly."""
    lengths, left = [], total
    while left > 0:
        L = int(torch.randint(1, max_len + 1, (1,), generator=gen))
        lengths.append(min(L, left))
        left -= lengths[-1]
    return lengths


def make_varlen(Hq, Hkv, D=64, lengths=None, total=None, max_len=None, std=1.0, seed=0, lead=0, tail=0,
                scale=None):
    """Documents packed back to back along the token dimension.

    Lengths are given explicitly or drawn by draw_doc_lengths(total, max_len).
    `lead` / `tail` rows before the first and after the last document belong
    to no document (their values are drawn like the rest).  Draw order:
    (lengths), q, k, v, sinks.
    """
    gen = torch.Generator().manual_seed(seed)
    if lengths is None:
        lengths = draw_doc_lengths(total, max_len, gen)
    lengths = [int(x) for x in lengths]
    cu = [lead]
    for L in lengths:
        cu.append(cu[-1] + L)
    T = cu[-1] + tail
    q = _normal_bf16(gen, (T, Hq, D), std)
    k = _normal_bf16(gen, (T, Hkv, D), std)
    v = _normal_bf16(gen, (T, Hkv, D), std)
    sinks = torch.randn((Hq,), generator=gen, dtype=torch.float32)
    max_seqlen = max([1] + lengths)
    return VarlenCase(q, k, v, torch.tensor(cu, dtype=torch.int32), sinks, max_seqlen,
                      (1.0 / D ** 0.5) if scale is None else scale)


# The five workloads.  Each prefill config runs one sliding-window-128 layer
# and one full-causal layer (window 0) over the same tensors.
CONFIGS = {
    "small_b1_s512_h8x1": dict(kind="fwd", B=1, S=512, Hq=8, Hkv=1, std=1.0, seed=1000),
    "prefill_b4_s4096_h64x8": dict(kind="fwd", B=4, S=4096, Hq=64, Hkv=8, std=1.0, seed=1001),
    "long_b1_s65536_h64x8": dict(kind="fwd", B=1, S=65536, Hq=64, Hkv=8, std=0.5, seed=1002),
    "train_b4_s4096_h64x8": dict(kind="bwd", B=4, S=4096, Hq=64, Hkv=8, std=1.0, seed=1001,
                                  dout_seed=1003),
    "decode_n128_l1024_h64x8": dict(kind="decode", N=128, Hq=64, Hkv=8, max_len=1024,
                                       seed=1004),
}


# Packed-document prefill: the token count and heads of the B=4, S=4096
# workload, cut into documents of U{1..4096} tokens (the pages give no
# document-length mix; this is the plainest one that spans short and
# full-length documents).
VARLEN_WORKLOAD = dict(name="varlen_t16384_docs_u1_4096_h64x8", total=16384, max_len=4096, Hq=64, Hkv=8,
                       seed=1005, dout_seed=1006)


def varlen_workload():
    """(VarlenCase, dout) of the packed-document workload (CPU tensors)."""
    w = VARLEN_WORKLOAD
    case = make_varlen(w["Hq"], w["Hkv"], total=w["total"], max_len=w["max_len"], seed=w["seed"], scale=0.125)
    return case, make_dout(tuple(case.q.shape), w["dout_seed"])


def config_inputs(name):
    """Inputs of one named workload (CPU tensors)."""
    c = CONFIGS[name]
    if c["kind"] == "decode":
        return make_decode(c["N"], c["Hq"], c["Hkv"], max_len=c["max_len"], seed=c["seed"])
    case = make_prefill(c["B"], c["S"], c["Hq"], c["Hkv"], std=c["std"], seed=c["seed"],
                        scale=0.125)
    if c["kind"] == "bwd":
        return case, make_dout(tuple(case.q.shape), c["dout_seed"])
    return case
