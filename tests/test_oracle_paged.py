"""Pins of the paged-cache oracle (CPU): reading a paged or ring cache through
its block table must give back exactly the rows of the packed cache it was
written from, and the decode over them must equal the packed-cache decode."""

import numpy as np
import pytest

from attention_attn_fwd_amd import synth
from oracle import gather_paged, ref_decode, ref_decode_paged

from _util import f64

LENGTHS = [1, 2, 15, 16, 17, 63, 64, 65, 200, 0, 129]


def _visible_rows(case, window):
    """The packed cache's visible rows per sequence, by plain slicing."""
    f = case.full
    ks, vs = [], []
    for n in range(len(case.seq_lens)):
        b, e = int(f.cu_seqlens[n]), int(f.cu_seqlens[n + 1])
        lo = max(b, e - window) if window > 0 else b
        ks.append(f64(f.k_cache[lo:e]))
        vs.append(f64(f.v_cache[lo:e]))
    return np.concatenate(ks), np.concatenate(vs)


@pytest.mark.parametrize("page_size", [1, 16, 64])
@pytest.mark.parametrize("window", [0, 1, 128])
def test_linear_pages_give_back_the_packed_rows(page_size, window):
    case = synth.make_paged_decode(len(LENGTHS), 4, 2, page_size, lengths=LENGTHS, seed=11)
    kc, vc, cu = gather_paged(f64(case.k_pages), f64(case.v_pages), case.block_table.numpy(),
                              case.seq_lens.numpy(), 0, window)
    rk, rv = _visible_rows(case, window)
    assert np.array_equal(kc, rk) and np.array_equal(vc, rv)
    assert np.abs(kc).max() < 100  # no never-written slot (1e4) was read


@pytest.mark.parametrize("ring,window", [(128, 128), (128, 100), (256, 128), (16, 16)])
def test_ring_keeps_exactly_the_window(ring, window):
    lengths = [1, window - 1, window, window + 1, ring, ring + 1, 3 * ring + 7, 0]
    case = synth.make_paged_decode(len(lengths), 4, 2, 16, lengths=lengths, seed=12, ring_tokens=ring)
    kc, vc, cu = gather_paged(f64(case.k_pages), f64(case.v_pages), case.block_table.numpy(),
                              case.seq_lens.numpy(), ring, window)
    rk, rv = _visible_rows(case, window)
    assert np.array_equal(kc, rk) and np.array_equal(vc, rv)


def test_ring_narrower_than_the_window_is_rejected():
    case = synth.make_paged_decode(2, 4, 2, 16, lengths=[40, 50], seed=13, ring_tokens=32)
    with pytest.raises(AssertionError):
        gather_paged(f64(case.k_pages), f64(case.v_pages), case.block_table.numpy(), case.seq_lens.numpy(), 32, 64)


@pytest.mark.parametrize("ring,window", [(0, 0), (0, 128), (128, 128)])
def test_paged_decode_equals_packed_decode(ring, window):
    lengths = [1, 16, 100, 300, 0, 129]
    case = synth.make_paged_decode(len(lengths), 8, 2, 16, lengths=lengths, seed=14, ring_tokens=ring)
    f = case.full
    ro, rl = ref_decode(f64(f.q), f64(f.k_cache), f64(f.v_cache), f.cu_seqlens.numpy(), f64(f.sinks), window,
                        f.scale)
    po, pl = ref_decode_paged(f64(case.q), f64(case.k_pages), f64(case.v_pages), case.block_table.numpy(),
                              case.seq_lens.numpy(), f64(case.sinks), ring, window, case.scale)
    np.testing.assert_allclose(po, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(pl, rl, rtol=0, atol=1e-12)
