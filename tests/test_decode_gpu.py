"""Decode parity of the HIP path against the fp64 oracle (GPU)."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_decode

from _util import seed_of, check_out_lse, f64, need_gpu

pytestmark = pytest.mark.gpu


def _run(case, window, dev, max_seqlen=None):
    t = [x.to(dev) for x in (case.q, case.k_cache, case.v_cache, case.cu_seqlens, case.sinks)]
    out, lse = attn.decode(*t, case.max_seqlen if max_seqlen is None else max_seqlen, window, case.scale)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, window):
    return ref_decode(f64(case.q), f64(case.k_cache), f64(case.v_cache), case.cu_seqlens.numpy(),
                      f64(case.sinks), window, case.scale)


@pytest.mark.parametrize("window", [128, 0])
def test_decode_workload(window):
    dev = need_gpu()
    case = synth.config_inputs("decode_n128_l1024_h64x8")
    print(f"decode workload W={window}", flush=True)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"decode workload W={window}")


EDGE_LENGTHS = [1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1000, 1024]


@pytest.mark.parametrize("window", [0, 1, 127, 128, 129])
@pytest.mark.parametrize("heads", [(64, 8), (8, 1), (8, 8), (6, 2), (40, 1), (128, 1), (64, 2), (16, 1)])
def test_decode_edge_lengths(window, heads):
    dev = need_gpu()
    Hq, Hkv = heads
    case = synth.make_decode(len(EDGE_LENGTHS), Hq, Hkv, lengths=EDGE_LENGTHS, seed=window + 3 * Hq)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"edges W={window} heads={heads}")


def test_decode_empty_sequences():
    dev = need_gpu()
    lengths = [0, 5, 0, 300, 0]
    case = synth.make_decode(len(lengths), 8, 1, lengths=lengths, seed=5)
    case.sinks[3] = -np.inf
    out, lse = _run(case, 0, dev, max_seqlen=1024)
    ro, rl = _oracle(case, 0)
    o, l = f64(out), f64(lse)
    for n in (0, 2, 4):
        assert (o[n] == 0).all()
        np.testing.assert_array_equal(l[n], f64(case.sinks))
    check_out_lse(o[[1, 3]], l[[1, 3]], ro[[1, 3]], rl[[1, 3]], "non-empty rows")


@pytest.mark.parametrize("window", [0, 200])
def test_decode_fewer_keys_than_workgroups(window):
    """max_seqlen 4096 (the chunk plan cuts each sequence's visible range
    into several chunks) with 6 keys in all: most chunks are empty, empty
    sequences see only the sink."""
    dev = need_gpu()
    lengths = [0, 1, 2, 0, 3, 0]
    case = synth.make_decode(len(lengths), 16, 2, lengths=lengths, seed=7 + window)
    out, lse = _run(case, window, dev, max_seqlen=4096)
    ro, rl = _oracle(case, window)
    o, l = f64(out), f64(lse)
    for n in (0, 3, 5):
        assert (o[n] == 0).all()
        np.testing.assert_array_equal(l[n], f64(case.sinks))
    check_out_lse(o[[1, 2, 4]], l[[1, 2, 4]], ro[[1, 2, 4]], rl[[1, 2, 4]], f"sparse W={window}")


@pytest.mark.parametrize("N", [512, 600])
def test_decode_many_sequences(N):
    """More sequences than CUs: one workgroup per (sequence, KV-head group),
    several per CU."""
    dev = need_gpu()
    case = synth.make_decode(N, 8, 1, max_len=300, seed=17 + N)
    out, lse = _run(case, 0, dev)
    ro, rl = _oracle(case, 0)
    check_out_lse(f64(out), f64(lse), ro, rl, f"N={N}")


@pytest.mark.parametrize("N", [255, 256, 257])
def test_decode_ranked_order(N):
    """With one chunk per sequence and at most 256 sequences (two KV heads
    per workgroup, no small window) every workgroup ranks the sequences by
    visible tiles itself and takes its item from that order.  Lengths with
    many ties (the rank breaks them by index) and empty sequences; outputs
    start as NaN, so an item taken twice or never shows.  Every sequence's
    result must also not depend on where it sits in the batch: a permuted
    batch gives the same bits per sequence."""
    dev = need_gpu()
    gen = np.random.default_rng(900 + N)
    lengths = gen.choice([0, 1, 63, 64, 65, 500, 1000, 1024], size=N).tolist()
    lengths[: 4] = [1024, 0, 1024, 1]
    case = synth.make_decode(N, 64, 8, lengths=lengths, seed=31 + N)
    print(f"ranked decode N={N}", flush=True)

    def run(c):
        t = [x.to(dev) for x in (c.q, c.k_cache, c.v_cache, c.cu_seqlens, c.sinks)]
        o = torch.full((N, 64, 64), float("nan"), dtype=torch.bfloat16, device=dev)
        l = torch.full((N, 64), float("nan"), device=dev)
        attn.decode(*t, c.max_seqlen, 0, c.scale, out=o, lse=l)
        torch.cuda.synchronize()
        return o, l

    out, lse = run(case)
    ro, rl = _oracle(case, 0)
    check_out_lse(f64(out), f64(lse), ro, rl, f"ranked N={N}")

    perm = gen.permutation(N)
    lp = [lengths[i] for i in perm]
    cu = case.cu_seqlens.long()
    rows = torch.cat([torch.arange(int(cu[i]), int(cu[i + 1])) for i in perm]) if sum(lp) else torch.zeros(0, dtype=torch.long)
    cup = torch.zeros(N + 1, dtype=torch.int32)
    cup[1:] = torch.cumsum(torch.tensor(lp, dtype=torch.int64), 0).to(torch.int32)
    pt = torch.as_tensor(perm, dtype=torch.long)
    pc = synth.DecodeCase(case.q[pt], case.k_cache[rows], case.v_cache[rows], cup, case.sinks, case.max_seqlen,
                          case.scale)
    out_p, lse_p = run(pc)
    pd = torch.as_tensor(perm, dtype=torch.long, device=dev)
    assert torch.equal(out_p, out[pd]) and torch.equal(lse_p, lse[pd])


@pytest.mark.parametrize("window", [0, 128])
def test_decode_multi_step(window):
    """Append one token per sequence and decode again, five times over; every
    step is compared with the oracle on the grown cache."""
    dev = need_gpu()
    gen = torch.Generator().manual_seed(77)
    N, Hq, Hkv, D = 16, 64, 8, 64
    lengths = torch.randint(120, 300, (N,), generator=gen).tolist()
    lengths[0], lengths[1] = 1, 127
    seqs_k = [torch.randn(L, Hkv, D, generator=gen).to(torch.bfloat16) for L in lengths]
    seqs_v = [torch.randn(L, Hkv, D, generator=gen).to(torch.bfloat16) for L in lengths]
    sinks = torch.randn(Hq, generator=gen)
    for step in range(5):
        q = torch.randn(N, Hq, D, generator=gen).to(torch.bfloat16)
        lens = [s.shape[0] for s in seqs_k]
        cu = torch.zeros(N + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lens), 0)
        case = synth.DecodeCase(q, torch.cat(seqs_k), torch.cat(seqs_v), cu, sinks, max(lens), 0.125)
        out, lse = _run(case, window, dev)
        ro, rl = _oracle(case, window)
        check_out_lse(f64(out), f64(lse), ro, rl, f"step {step}")
        # the next token's K/V join every cache
        for n in range(N):
            seqs_k[n] = torch.cat([seqs_k[n], torch.randn(1, Hkv, D, generator=gen).to(torch.bfloat16)])
            seqs_v[n] = torch.cat([seqs_v[n], torch.randn(1, Hkv, D, generator=gen).to(torch.bfloat16)])


def test_decode_matches_prefill_last_row():
    """Decode of the last token equals row L-1 of the GPU prefill (both
    within the bar of the oracle; compared to each other here)."""
    dev = need_gpu()
    S = 700
    case = synth.make_prefill(1, S, 16, 2, seed=12)
    for window in (0, 128):
        out_p, lse_p = attn.fwd(case.q.to(dev), case.k.to(dev), case.v.to(dev), case.sinks.to(dev), window,
                                case.scale)
        cu = torch.tensor([0, S], dtype=torch.int32, device=dev)
        out_d, lse_d = attn.decode(case.q[0, S - 1:S].to(dev).contiguous(), case.k[0].to(dev), case.v[0].to(dev),
                                   cu, case.sinks.to(dev), S, window, case.scale)
        torch.cuda.synchronize()
        assert (out_d.float() - out_p[0, S - 1].float()).abs().max().item() <= 1e-2
        assert (lse_d[0] - lse_p[0, :, S - 1]).abs().max().item() <= 1e-3


@pytest.mark.parametrize("window", [0, 128, 1000])
@pytest.mark.parametrize("lengths", [[65536], [1024] * 31 + [700], [3000, 1, 64, 2049]],
                         ids=["one_long", "n32", "mixed"])
def test_decode_chunked(window, lengths):
    """Few (sequence, KV group) pairs: sequences are cut into chunks, each
    chunk walked by one wave per KV head, and merged afterwards (window
    1000: the visible range starts inside the sequence and is cut too;
    window 128 is decoded unsplit)."""
    dev = need_gpu()
    case = synth.make_decode(len(lengths), 64, 8, lengths=lengths, seed=seed_of(lengths, window))
    print(f"decode chunked n={len(lengths)} max={max(lengths)} W={window}", flush=True)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"chunked W={window}")


def test_decode_is_deterministic():
    dev = need_gpu()
    case = synth.make_decode(32, 64, 8, max_len=1024, seed=13)
    a = _run(case, 0, dev)
    b = _run(case, 0, dev)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("workload", ["n128_l1024", "n8_l1024", "one_65536"])
def test_decode_split_count_invariance(workload, window):
    """The result must not depend on how a sequence's keys are cut into
    chunks: the same inputs decoded under the chunk plans of max_seqlen =
    the longest sequence, 4x and 64x it (the plan follows max_seqlen and the
    number of sequences) each match the oracle, and agree with one another
    within 3e-3 (max) and 3e-4 (mean) on out and 2e-5 on lse.  (Plans do
    differ beyond one bf16 ulp: each chunk rounds its probabilities to bf16
    against its own running maximum, an error of the size the oracle bar
    already admits for each plan, ~1e-3 here.)"""
    dev = need_gpu()
    if workload == "n128_l1024":
        case = synth.config_inputs("decode_n128_l1024_h64x8")
    elif workload == "n8_l1024":
        case = synth.make_decode(8, 64, 8, max_len=1024, seed=seed_of("t3", window))
    else:
        case = synth.make_decode(1, 64, 8, lengths=[65536], seed=seed_of("t3long", window))
    Lmax = int(np.diff(case.cu_seqlens.numpy()).max())
    ro, rl = _oracle(case, window)
    results = []
    for ms in (Lmax, 4 * Lmax, 64 * Lmax):
        ws = attn.decode_workspace_size(case.q.shape[0], 64, 8, 64, ms, window)
        print(f"decode T3 {workload} W={window} max_seqlen={ms} workspace={ws}", flush=True)
        out, lse = _run(case, window, dev, max_seqlen=ms)
        check_out_lse(f64(out), f64(lse), ro, rl, f"{workload} W={window} max_seqlen={ms}")
        results.append((f64(out), f64(lse)))
    (o0, l0) = results[0]
    for o, l in results[1:]:
        d = np.abs(o - o0)
        print(f"plans differ: out max {d.max():.2e} mean {d.mean():.2e}, lse max {np.abs(l - l0).max():.2e}")
        assert d.max() <= 3e-3 and d.mean() <= 3e-4
        assert np.abs(l - l0).max() <= 2e-5


def test_decode_reuses_one_workspace():
    """One workspace serves a run of calls with different plans, windows and
    sequence counts: every call matches the one with a fresh workspace bit
    for bit (the kernels are deterministic and overwrite what they read)."""
    dev = need_gpu()
    cases = [synth.make_decode(128, 64, 8, max_len=1024, seed=61),
             synth.make_decode(8, 64, 8, max_len=1024, seed=62),
             synth.make_decode(3, 64, 8, lengths=[3000, 1, 2049], seed=63)]
    need = max(attn.decode_workspace_size(c.q.shape[0], 64, 8, 64, c.max_seqlen, w) for c in cases for w in (0, 128))
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dev)  # stale bytes must not matter
    for rep in range(2):
        for ci, case in enumerate(cases):
            for window in (0, 128):
                t = [x.to(dev) for x in (case.q, case.k_cache, case.v_cache, case.cu_seqlens, case.sinks)]
                ref = attn.decode(*t, case.max_seqlen, window, case.scale)
                got = attn.decode(*t, case.max_seqlen, window, case.scale, workspace=ws)
                torch.cuda.synchronize()
                assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]), (rep, ci, window)
