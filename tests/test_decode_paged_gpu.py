"""Paged and ring-buffer decode against the fp64 oracle (GPU)."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_decode_paged

from _util import check_out_lse, f64, need_gpu

pytestmark = pytest.mark.gpu

EDGE_LENGTHS = [1, 2, 15, 16, 17, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 1024, 0]


def _run(case, window, dev, max_seqlen=None):
    t = [x.to(dev) for x in (case.q, case.k_pages, case.v_pages, case.block_table, case.seq_lens, case.sinks)]
    out, lse = attn.decode_paged(*t, case.max_seqlen if max_seqlen is None else max_seqlen, window, case.scale,
                                 ring_tokens=case.ring_tokens)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, window):
    return ref_decode_paged(f64(case.q), f64(case.k_pages), f64(case.v_pages), case.block_table.numpy(),
                            case.seq_lens.numpy(), f64(case.sinks), case.ring_tokens, window, case.scale)


# pages of 1-4 tokens take the per-lane lookup, 8 and more the wave-uniform one
@pytest.mark.parametrize("page_size", [1, 4, 8, 16, 64, 256])
@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("heads", [(64, 8), (8, 1), (128, 2)])
def test_paged_linear(page_size, window, heads):
    dev = need_gpu()
    case = synth.make_paged_decode(len(EDGE_LENGTHS), *heads, page_size, lengths=EDGE_LENGTHS,
                                   seed=page_size + window + heads[0])
    print(f"paged ps={page_size} W={window} heads={heads}", flush=True)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"paged ps={page_size} W={window}")


@pytest.mark.parametrize("ring,window,page_size", [(128, 128, 16), (128, 100, 16), (256, 128, 64), (128, 1, 128)])
def test_ring(ring, window, page_size):
    dev = need_gpu()
    lengths = [1, window, window + 1, ring, ring + 1, 3 * ring + 7, 1000, 0, 65]
    case = synth.make_paged_decode(len(lengths), 64, 8, page_size, lengths=lengths, seed=ring + window,
                                   ring_tokens=ring)
    print(f"ring R={ring} W={window} ps={page_size}", flush=True)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"ring R={ring} W={window}")


@pytest.mark.parametrize("window", [0, 128])
def test_paged_equals_packed_decode_bitwise(window):
    """Same rows in the same order: the paged kernel must reproduce the packed
    cache kernel bit for bit, at the 128 x U{1..1024} workload."""
    dev = need_gpu()
    case = synth.make_paged_decode(128, 64, 8, 16, seed=1004)
    out_p, lse_p = _run(case, window, dev)
    f = case.full
    t = [x.to(dev) for x in (f.q, f.k_cache, f.v_cache, f.cu_seqlens, f.sinks)]
    out_c, lse_c = attn.decode(*t, f.max_seqlen, window, f.scale)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_c) and torch.equal(lse_p, lse_c)


def test_paged_long_sequence_chunked():
    """One long sequence is cut into chunks and merged; pages of 16 tokens."""
    dev = need_gpu()
    case = synth.make_paged_decode(1, 64, 8, 16, lengths=[20000], seed=15)
    out, lse = _run(case, 0, dev)
    ro, rl = _oracle(case, 0)
    check_out_lse(f64(out), f64(lse), ro, rl, "paged long")


@pytest.mark.parametrize("page_size", [8, 16, 4])
def test_paged_window_chunked(page_size):
    """Few sequences with a window of 1000: the visible range starts at
    L - 1000 (not a multiple of 8) and is cut into chunks, so a lane group's
    8 rows often straddle a page boundary."""
    dev = need_gpu()
    lengths = [20000, 3001, 1000, 999]
    case = synth.make_paged_decode(len(lengths), 64, 8, page_size, lengths=lengths, seed=40 + page_size)
    print(f"paged window chunked ps={page_size}", flush=True)
    out, lse = _run(case, 1000, dev)
    ro, rl = _oracle(case, 1000)
    check_out_lse(f64(out), f64(lse), ro, rl, f"paged W=1000 ps={page_size}")
