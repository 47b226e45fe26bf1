"""Packed-document (variable-length) prefill forward and backward against the
fp64 oracle (GPU), through the C ABI.

Documents are packed along the token dimension (document b = rows
cu[b] .. cu[b+1]-1) and attention is confined to each.  Layouts cover empty
documents, one-token documents, lengths that end inside a tile, and rows
before the first / after the last document (which must stay untouched)."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_bwd_varlen, ref_fwd_varlen

from _util import (GRAD_REL_L2, check_grads_by_group, check_out_lse, f64, nan_grads, need_gpu, oracle_map, rel_l2,
                   seed_of)

pytestmark = pytest.mark.gpu

SENTINEL = 77.0  # prefilled into outputs; rows in no document must keep it


def _dev(case, dev):
    return [t.to(dev) for t in (case.q, case.k, case.v, case.cu_seqlens, case.sinks)]


def _inside(cu, T):
    m = np.zeros(T, dtype=bool)
    for b in range(len(cu) - 1):
        m[int(cu[b]):int(cu[b + 1])] = True
    return m


def _fwd(case, window, dev):
    q, k, v, cu, s = _dev(case, dev)
    T, Hq, _ = q.shape
    out = torch.full_like(q, SENTINEL)
    lse = torch.full((Hq, T), SENTINEL, dtype=torch.float32, device=dev)
    attn.fwd_varlen(q, k, v, cu, s, case.max_seqlen, window, case.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _bwd(case, out, lse, dout, window, dev):
    q, k, v, cu, s = _dev(case, dev)
    grads = (torch.full_like(q, SENTINEL), torch.full_like(k, SENTINEL), torch.full_like(v, SENTINEL),
             torch.full((q.shape[1],), SENTINEL, dtype=torch.float32, device=dev))
    attn.bwd_varlen(q, k, v, cu, s, out, lse, dout.to(dev), case.max_seqlen, window, case.scale, grads=grads)
    torch.cuda.synchronize()
    return grads


def _check_grads(grads, ref, inside, what, heads=None, kv_heads=None):
    dq, dk, dv, ds = (f64(t) for t in grads)
    rdq, rdk, rdv, rds = ref
    dq, dk, dv, rdq, rdk, rdv = dq[inside], dk[inside], dv[inside], rdq[inside], rdk[inside], rdv[inside]
    if heads is not None:
        dq, rdq, ds, rds = dq[:, heads], rdq[:, heads], ds[heads], rds[heads]
        dk, rdk, dv, rdv = dk[:, kv_heads], rdk[:, kv_heads], dv[:, kv_heads], rdv[:, kv_heads]
    errs = {n: rel_l2(a, r) for n, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv),
                                               ("dsinks", ds, rds))}
    msg = f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items())
    print(msg, flush=True)
    for e in errs.values():
        assert e <= GRAD_REL_L2, msg


LAYOUTS = [  # document lengths, rows before, rows after
    ([300], 0, 0),
    ([1, 64, 65, 0, 130, 31, 200], 0, 0),
    ([129, 0, 0, 257, 3], 5, 11),
    ([700, 1, 1, 450], 0, 7),
    ([0, 0, 17], 40, 0),
]
HEADS = [(8, 1), (16, 2), (6, 2), (1, 1), (64, 1)]


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: "L%d-%d-%d" % (len(l[0]), l[1], l[2]))
@pytest.mark.parametrize("heads", HEADS, ids=lambda h: "H%dx%d" % h)
@pytest.mark.parametrize("window", [0, 1, 128])
def test_varlen_fwd_bwd(layout, heads, window):
    dev = need_gpu()
    lengths, lead, tail = layout
    Hq, Hkv = heads
    case = synth.make_varlen(Hq, Hkv, lengths=lengths, lead=lead, tail=tail, seed=seed_of(layout, heads, window))
    dout = synth.make_dout(tuple(case.q.shape), seed=seed_of("dout", layout, heads, window))
    print(f"varlen lengths={lengths} lead={lead} tail={tail} heads={heads} W={window}", flush=True)
    T = case.q.shape[0]
    inside = _inside(case.cu_seqlens.tolist(), T)
    out, lse = _fwd(case, window, dev)
    ro, rl = ref_fwd_varlen(f64(case.q), f64(case.k), f64(case.v), case.cu_seqlens.numpy(), f64(case.sinks),
                            window, case.scale)
    check_out_lse(f64(out)[inside], f64(lse)[:, inside], ro[inside], rl[:, inside], f"varlen W={window}")
    assert (out[torch.from_numpy(~inside).to(dev)] == SENTINEL).all()
    assert (lse[:, torch.from_numpy(~inside).to(dev)] == SENTINEL).all()
    grads = _bwd(case, out, lse, dout, window, dev)
    ref = ref_bwd_varlen(f64(case.q), f64(case.k), f64(case.v), case.cu_seqlens.numpy(), f64(case.sinks),
                         f64(dout), window, case.scale)
    _check_grads(grads, ref, inside, f"varlen bwd W={window}")
    gap = torch.from_numpy(~inside).to(dev)
    for t in grads[:3]:
        assert (t[gap] == SENTINEL).all()


@pytest.mark.parametrize("window", [0, 128])
def test_varlen_equal_lengths_match_dense_bitwise(window):
    """N documents of one length S are the dense [N, S] batch: same kernels,
    same arithmetic, so every output is bit-identical (lse transposed)."""
    dev = need_gpu()
    N, S, Hq, Hkv = 3, 333, 16, 2
    case = synth.make_varlen(Hq, Hkv, lengths=[S] * N, seed=31 + window)
    dout = synth.make_dout(tuple(case.q.shape), seed=32)
    out, lse = _fwd(case, window, dev)
    grads = _bwd(case, out, lse, dout, window, dev)
    q, k, v, _, s = _dev(case, dev)
    D = q.shape[2]
    qd, kd, vd = q.view(N, S, Hq, D), k.view(N, S, Hkv, D), v.view(N, S, Hkv, D)
    dout_d = dout.to(dev).view(N, S, Hq, D)
    out_d, lse_d = attn.fwd(qd, kd, vd, s, window, case.scale)
    grads_d = attn.bwd(qd, kd, vd, s, out_d, lse_d, dout_d, window, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(N, S, Hq, D), out_d)
    assert torch.equal(lse.view(Hq, N, S).transpose(0, 1), lse_d)
    for a, b in zip(grads[:3], grads_d[:3]):
        assert torch.equal(a.view(b.shape), b)
    assert torch.equal(grads[3], grads_d[3])


def test_varlen_no_document_rows():
    """Every document empty: nothing is written but dsinks, which is the
    empty sum 0."""
    dev = need_gpu()
    case = synth.make_varlen(8, 1, lengths=[0, 0, 0], lead=10, tail=6, seed=41)
    dout = synth.make_dout(tuple(case.q.shape), seed=42)
    out, lse = _fwd(case, 0, dev)
    assert (out == SENTINEL).all() and (lse == SENTINEL).all()
    grads = _bwd(case, out, lse, dout, 0, dev)
    for t in grads[:3]:
        assert (t == SENTINEL).all()
    assert (grads[3] == 0).all()


@pytest.mark.parametrize("window", [128, 0])
def test_varlen_workload_whole(window):
    """The packed-document workload bench.py times (16384 tokens in
    documents of U{1..4096} tokens, 64q/8kv heads), in the same launch
    configuration: every output, lse and gradient element of every document
    and KV group against the oracle (run per document and KV group on the
    host's cores), into NaN-filled gradient buffers."""
    dev = need_gpu()
    case, dout = synth.varlen_workload()
    cu = case.cu_seqlens.numpy()
    T, Hq, D = case.q.shape
    Hkv = case.k.shape[1]
    G = Hq // Hkv
    print(f"varlen workload W={window} docs={len(cu) - 1}", flush=True)
    assert _inside(cu, T).all()  # the documents tile the token rows
    out, lse = _fwd(case, window, dev)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    q, k, v, sk, do = f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout)
    tasks = [(b, c) for b in range(len(cu) - 1) for c in range(Hkv) if cu[b + 1] > cu[b]]

    def fwd_one(t):
        b, c = t
        a, e, hs = int(cu[b]), int(cu[b + 1]), slice(c * G, (c + 1) * G)
        return ref_fwd_varlen(q[a:e, hs], k[a:e, c:c + 1], v[a:e, c:c + 1], np.array([0, e - a]), sk[hs], window,
                              case.scale)

    ro, rl = np.full((T, Hq, D), np.nan), np.full((Hq, T), np.nan)
    for (b, c), (o, l) in zip(tasks, oracle_map(fwd_one, tasks)):
        a, e, hs = int(cu[b]), int(cu[b + 1]), slice(c * G, (c + 1) * G)
        ro[a:e, hs], rl[hs, a:e] = o, l
    check_out_lse(f64(out), f64(lse), ro, rl, f"varlen workload W={window}")

    q_, k_, v_, cu_, s_ = _dev(case, dev)
    grads = attn.bwd_varlen(q_, k_, v_, cu_, s_, out, lse, dout.to(dev), case.max_seqlen, window, case.scale,
                            grads=nan_grads(q_, k_, v_, Hq))
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t.float()).all()

    def bwd_one(t):
        b, c = t
        a, e, hs = int(cu[b]), int(cu[b + 1]), slice(c * G, (c + 1) * G)
        return ref_bwd_varlen(q[a:e, hs], k[a:e, c:c + 1], v[a:e, c:c + 1], np.array([0, e - a]), sk[hs],
                              do[a:e, hs], window, case.scale)

    rdq, rdk, rdv, rds = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape), np.zeros(Hq)
    for (b, c), (gq, gk, gv, gs) in zip(tasks, oracle_map(bwd_one, tasks)):
        a, e, hs = int(cu[b]), int(cu[b + 1]), slice(c * G, (c + 1) * G)
        rdq[a:e, hs], rdk[a:e, c], rdv[a:e, c] = gq, gk[:, 0], gv[:, 0]
        rds[hs] += gs
    got = [f64(t) for t in grads]
    check_grads_by_group([got[0][None], got[1][None], got[2][None], got[3]],
                         [rdq[None], rdk[None], rdv[None], rds], Hkv, f"varlen workload bwd W={window}")
