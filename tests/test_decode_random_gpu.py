"""Decode parity over a fixed set of random configurations (GPU): packed,
paged and ring caches; sequence counts on both sides of the ranked-order
limit; KV head counts that leave a head block partly empty; windows below,
at and above the small-window limit; empty sequences.  Every case against
the fp64 oracle, outputs NaN-filled first."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_decode, ref_decode_paged

from _util import check_out_lse, f64, need_gpu

pytestmark = pytest.mark.gpu


def _configs():
    rng = np.random.default_rng(20261203)
    out = []
    for i in range(24):
        Hkv = int(rng.choice([1, 2, 3, 8]))
        G = int(rng.choice([1, 4, 8, 16]))
        N = int(rng.choice([1, 5, 37, 200, 256, 300]))
        window = int(rng.choice([0, 0, 1, 100, 128, 256, 257, 1000]))
        cache = ["packed", "paged", "ring"][i % 3]
        page = int(rng.choice([1, 8, 16, 64]))
        max_len = int(rng.choice([64, 700, 1500]))
        out.append((i, Hkv, G, N, window, cache, page, max_len))
    # one chunk per sequence without a window: the ranked order, over the
    # packed cache and both paged paths that take it
    out += [(24, 8, 8, 200, 0, "packed", 16, 1024), (25, 8, 8, 200, 0, "paged", 8, 1024),
            (26, 3, 8, 200, 0, "paged", 1, 1024)]
    return out


@pytest.mark.parametrize("cfg", _configs(), ids=lambda c: f"c{c[0]}")
def test_decode_random_config(cfg):
    i, Hkv, G, N, window, cache, page, max_len = cfg
    dev = need_gpu()
    rng = np.random.default_rng(1000 + i)
    lengths = rng.integers(0, max_len + 1, size=N)
    lengths[rng.random(N) < 0.1] = 0
    lengths = lengths.tolist()
    Hq = G * Hkv
    if cache == "ring" and window == 0:
        window = 128  # a ring holds a sliding layer's keys
    print(f"random decode c{i}: N={N} Hq={Hq} Hkv={Hkv} W={window} {cache} page={page} max_len={max_len}",
          flush=True)
    o = torch.full((N, Hq, 64), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((N, Hq), float("nan"), device=dev)
    if cache == "packed":
        case = synth.make_decode(N, Hq, Hkv, lengths=lengths, seed=2000 + i)
        t = [x.to(dev) for x in (case.q, case.k_cache, case.v_cache, case.cu_seqlens, case.sinks)]
        attn.decode(*t, case.max_seqlen, window, case.scale, out=o, lse=lse)
        ro, rl = ref_decode(f64(case.q), f64(case.k_cache), f64(case.v_cache), case.cu_seqlens.numpy(),
                            f64(case.sinks), window, case.scale)
    else:
        ring = 0
        if cache == "ring":
            ring = max(page, 1 << int(np.ceil(np.log2(max(window, 1)))))
        case = synth.make_paged_decode(N, Hq, Hkv, page, lengths=lengths, seed=2000 + i, ring_tokens=ring)
        t = [x.to(dev) for x in (case.q, case.k_pages, case.v_pages, case.block_table, case.seq_lens, case.sinks)]
        attn.decode_paged(*t, case.max_seqlen, window, case.scale, ring_tokens=ring, out=o, lse=lse)
        ro, rl = ref_decode_paged(f64(case.q), f64(case.k_pages), f64(case.v_pages), case.block_table.numpy(),
                                  case.seq_lens.numpy(), f64(case.sinks), ring, window, case.scale)
    torch.cuda.synchronize()
    check_out_lse(f64(o), f64(lse), ro, rl, f"random decode c{i}")
