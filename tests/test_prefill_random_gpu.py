"""Forward and backward parity over a fixed set of random configurations
(GPU): dense batches and packed documents; sequence and document lengths that
end inside a tile; group sizes that do and do not divide a workgroup's 256
columns or the backward's 64-column steps; windows of one key, around the
64-key tile, around 128, drawn at random, and at or above the sequence
length; softmax scales below 1/sqrt(D); sinks of -inf, 0, drawn and dominant
values mixed over the heads.  Inputs keep the magnitudes of the workloads
(unit or half normal), where the output bars are set.  Every case against the
fp64 oracle, outputs and gradients NaN-filled first."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_bwd_varlen, ref_fwd_varlen

from _util import (GRAD_REL_L2, check_grads_by_group, check_out_lse, f64, nan_grads, nan_like, need_gpu,
                   ref_bwd_groups, ref_fwd_groups, rel_l2)

pytestmark = pytest.mark.gpu


def _mixed_sinks(sinks, rng):
    """Some heads without a sink (-inf), some with a zero or dominant one."""
    s = sinks.clone()
    u = rng.random(s.numel())
    s[torch.from_numpy(u < 0.2)] = float("-inf")
    s[torch.from_numpy((u >= 0.2) & (u < 0.3))] = 0.0
    s[torch.from_numpy((u >= 0.3) & (u < 0.4))] = 4.0
    return s


def _window(rng, S, kind=None):
    kind = int(rng.integers(0, 6)) if kind is None else kind
    if kind == 0:
        return 0
    if kind == 1:
        return 1
    if kind == 2:
        return int(rng.choice([63, 64, 65]))
    if kind == 3:
        return int(rng.choice([127, 128, 129]))
    if kind == 4:
        return int(rng.integers(2, max(3, S)))
    return S + int(rng.integers(0, 3))  # every key visible: the full-causal layer


def _dense_configs():
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(16):
        B = int(rng.choice([1, 2, 3]))
        S = int(rng.integers(16, 600))
        Hkv = int(rng.choice([1, 2, 3, 8]))
        G = int(rng.choice([1, 2, 3, 5, 8, 12, 16]))
        window = _window(rng, S)
        scale = float(rng.choice([0.125, 0.1, 0.0625]))
        std = float(rng.choice([1.0, 0.5]))
        out.append((i, B, S, Hkv, G, window, scale, std))
    return out


@pytest.mark.parametrize("cfg", _dense_configs(), ids=lambda c: f"d{c[0]}")
def test_prefill_random_dense(cfg):
    i, B, S, Hkv, G, window, scale, std = cfg
    dev = need_gpu()
    Hq = G * Hkv
    rng = np.random.default_rng(3000 + i)
    case = synth.make_prefill(B, S, Hq, Hkv, std=std, seed=4000 + i, scale=scale)
    sinks = _mixed_sinks(case.sinks, rng)
    dout = synth.make_dout(tuple(case.q.shape), seed=5000 + i)
    print(f"random prefill d{i}: B={B} S={S} Hq={Hq} Hkv={Hkv} W={window} scale={scale} std={std}", flush=True)
    q, k, v, s, do = (t.to(dev) for t in (case.q, case.k, case.v, sinks, dout))
    out = nan_like(q.shape, torch.bfloat16, dev)
    lse = nan_like((B, Hq, S), torch.float32, dev)
    attn.fwd(q, k, v, s, window, scale, out=out, lse=lse)
    grads = attn.bwd(q, k, v, s, out, lse, do, window, scale, grads=nan_grads(q, k, v, Hq))
    torch.cuda.synchronize()
    qf, kf, vf, sf = f64(case.q), f64(case.k), f64(case.v), f64(sinks)
    ro, rl = ref_fwd_groups(qf, kf, vf, sf, window, scale)
    check_out_lse(f64(out), f64(lse), ro, rl, f"random prefill d{i}")
    ref = ref_bwd_groups(qf, kf, vf, sf, f64(dout), window, scale)
    check_grads_by_group([f64(t) for t in grads], ref, Hkv, f"random prefill bwd d{i}")


def _varlen_configs():
    rng = np.random.default_rng(20261205)
    out = []
    for i in range(8):
        Hkv = int(rng.choice([1, 2, 8]))
        G = int(rng.choice([1, 4, 8, 12]))
        n_docs = int(rng.integers(1, 8))
        lengths = rng.integers(1, 400, size=n_docs)
        lengths[rng.random(n_docs) < 0.15] = 0
        lengths[rng.random(n_docs) < 0.15] = 1
        lead = int(rng.choice([0, 0, int(rng.integers(1, 20))]))
        tail = int(rng.choice([0, 0, int(rng.integers(1, 20))]))
        window = _window(rng, int(lengths.max()), kind=i % 6)
        out.append((i, Hkv, G, [int(x) for x in lengths], lead, tail, window))
    return out


@pytest.mark.parametrize("cfg", _varlen_configs(), ids=lambda c: f"v{c[0]}")
def test_prefill_random_varlen(cfg):
    i, Hkv, G, lengths, lead, tail, window = cfg
    dev = need_gpu()
    Hq = G * Hkv
    rng = np.random.default_rng(6000 + i)
    case = synth.make_varlen(Hq, Hkv, lengths=lengths, lead=lead, tail=tail, seed=7000 + i)
    sinks = _mixed_sinks(case.sinks, rng)
    dout = synth.make_dout(tuple(case.q.shape), seed=8000 + i)
    T = case.q.shape[0]
    cu = case.cu_seqlens.numpy()
    inside = np.zeros(T, dtype=bool)
    for b in range(len(cu) - 1):
        inside[cu[b]:cu[b + 1]] = True
    print(f"random varlen v{i}: lengths={lengths} lead={lead} tail={tail} Hq={Hq} Hkv={Hkv} W={window}",
          flush=True)
    q, k, v, c, s, do = (t.to(dev) for t in (case.q, case.k, case.v, case.cu_seqlens, sinks, dout))
    out = nan_like(q.shape, torch.bfloat16, dev)
    lse = nan_like((Hq, T), torch.float32, dev)
    attn.fwd_varlen(q, k, v, c, s, case.max_seqlen, window, case.scale, out=out, lse=lse)
    grads = attn.bwd_varlen(q, k, v, c, s, out, lse, do, case.max_seqlen, window, case.scale,
                            grads=nan_grads(q, k, v, Hq))
    torch.cuda.synchronize()
    qf, kf, vf, sf, dof = f64(case.q), f64(case.k), f64(case.v), f64(sinks), f64(dout)
    o_, l_ = f64(out), f64(lse)
    if inside.any():
        ro, rl = ref_fwd_varlen(qf, kf, vf, cu, sf, window, case.scale)
        check_out_lse(o_[inside], l_[:, inside], ro[inside], rl[:, inside], f"random varlen v{i}")
    # rows in no document are left as they were
    assert np.isnan(o_[~inside]).all() and np.isnan(l_[:, ~inside]).all()
    got = [f64(t) for t in grads]
    for t in got[:3]:
        assert np.isnan(t[~inside]).all()
    assert np.isfinite(got[3]).all()
    rdq, rdk, rdv, rds = ref_bwd_varlen(qf, kf, vf, cu, sf, dof, window, case.scale)
    if inside.any():
        errs = {n: rel_l2(a[inside], r[inside]) for n, a, r in (("dq", got[0], rdq), ("dk", got[1], rdk),
                                                                   ("dv", got[2], rdv))}
        errs["dsinks"] = rel_l2(got[3], rds)
        msg = f"random varlen bwd v{i}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items())
        print(msg, flush=True)
        assert all(e <= GRAD_REL_L2 for e in errs.values()), msg
    else:
        assert (got[3] == 0).all()
