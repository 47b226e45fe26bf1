"""Backward parity of the HIP path against the fp64 oracle (GPU).

The HIP backward consumes the HIP forward's own bf16 out and fp32 lse (as in
training); the oracle recomputes its own fp64 forward."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_bwd

from _util import GRAD_REL_L2, check_grads_by_group, f64, nan_grads, need_gpu, ref_bwd_groups, rel_l2, seed_of

pytestmark = pytest.mark.gpu


def _run(case, dout, window, dev):
    q, k, v, s = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    do = dout.to(dev)
    out, lse = attn.fwd(q, k, v, s, window, case.scale)
    grads = attn.bwd(q, k, v, s, out, lse, do, window, case.scale)
    torch.cuda.synchronize()
    return grads


def _check(grads, ref, what, heads=None, kv_heads=None):
    dq, dk, dv, ds = (f64(t) for t in grads)
    rdq, rdk, rdv, rds = ref
    if heads is not None:
        dq, rdq = dq[:, :, heads], rdq[:, :, heads]
        ds, rds = ds[heads], rds[heads]
        dk, rdk = dk[:, :, kv_heads], rdk[:, :, kv_heads]
        dv, rdv = dv[:, :, kv_heads], rdv[:, :, kv_heads]
    errs = {n: rel_l2(a, r) for n, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv),
                                               ("dsinks", ds, rds))}
    msg = f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items())
    print(msg, flush=True)
    for n, e in errs.items():
        assert e <= GRAD_REL_L2, msg
    return errs


def _oracle(case, dout, window, **kw):
    return ref_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout), window, case.scale, **kw)


SMALL = [  # B, S, Hq, Hkv  (S = 1 over 4 batches: one key per head makes a single
           # batch's relative L2 hinge on one possibly cancelling dS sum)
    (4, 1, 8, 1), (1, 17, 8, 1), (2, 129, 8, 1), (1, 300, 8, 8), (1, 700, 8, 1), (2, 77, 16, 2),
    (1, 200, 6, 2), (1, 333, 1, 1), (1, 260, 4, 4),
    (2, 200, 16, 8), (3, 150, 24, 8),  # B * Hkv = 16, 24: the XCD-aware order with 2, 3 groups per XCD
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dS%dH%dx%d" % s)
@pytest.mark.parametrize("window", [0, 1, 127, 128, 129])
def test_bwd_small_shapes(shape, window):
    dev = need_gpu()
    B, S, Hq, Hkv = shape
    case = synth.make_prefill(B, S, Hq, Hkv, seed=seed_of(shape, window, "bwd"))
    dout = synth.make_dout(tuple(case.q.shape), seed=S + window)
    print(f"bwd shape={shape} window={window}", flush=True)
    grads = _run(case, dout, window, dev)
    check_grads_by_group([f64(t) for t in grads], _oracle(case, dout, window), Hkv, f"{shape} W={window}")


@pytest.mark.parametrize("heads", [(16, 1), (32, 1), (64, 1), (128, 1), (12, 1), (80, 2)], ids=lambda h: "H%dx%d" % h)
@pytest.mark.parametrize("window", [0, 128])
def test_bwd_large_groups(heads, window):
    """Group sizes up to the supported 128 (the key-outer kernel's 64-column
    steps hold 64 / G positions when G divides 64, else a column walk by
    division; the query-outer kernel's 128 columns hold 128 / G positions)."""
    dev = need_gpu()
    Hq, Hkv = heads
    case = synth.make_prefill(1, 190, Hq, Hkv, seed=seed_of(heads, window, "bwdG"))
    dout = synth.make_dout(tuple(case.q.shape), seed=seed_of(heads, window, "doutG"))
    print(f"bwd heads={heads} window={window}", flush=True)
    grads = _run(case, dout, window, dev)
    _check(grads, _oracle(case, dout, window), f"heads={heads} W={window}")


@pytest.mark.parametrize("sink", [-np.inf, 5.0])
@pytest.mark.parametrize("window", [0, 128])
def test_bwd_extreme_sinks(sink, window):
    dev = need_gpu()
    case = synth.make_prefill(1, 300, 8, 1, seed=21)
    case.sinks[:] = sink
    dout = synth.make_dout(tuple(case.q.shape), seed=22)
    grads = _run(case, dout, window, dev)
    ref = _oracle(case, dout, window)
    if sink == -np.inf:
        assert (grads[3] == 0).all()
        ref = ref[:3] + (np.ones(8),)  # dsink is exactly zero; compare the rest
        grads = grads[:3] + (torch.ones(8),)
    _check(grads, ref, f"sink={sink} W={window}")


def test_bwd_is_deterministic():
    dev = need_gpu()
    case = synth.make_prefill(2, 600, 16, 2, seed=23)
    dout = synth.make_dout(tuple(case.q.shape), seed=24)
    a = _run(case, dout, 0, dev)
    b = _run(case, dout, 0, dev)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("window", [128, 0])
def test_bwd_training_workload_whole(window):
    """The training shape (B=4, S=4096, 64q/8kv) in the launch configuration
    bench.py times: every gradient element of all eight KV groups against the
    oracle (run per batch and KV group on the host's cores), into NaN-filled
    gradient buffers."""
    dev = need_gpu()
    case, dout = synth.config_inputs("train_b4_s4096_h64x8")
    print(f"bwd B4 S4096 W={window}", flush=True)
    q, k, v, s = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse = attn.fwd(q, k, v, s, window, case.scale)
    grads = attn.bwd(q, k, v, s, out, lse, dout.to(dev), window, case.scale, grads=nan_grads(q, k, v, q.shape[2]))
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t.float()).all()
    ref = ref_bwd_groups(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout), window, case.scale)
    check_grads_by_group([f64(t) for t in grads], ref, k.shape[2], f"B4 S4096 W={window}")
