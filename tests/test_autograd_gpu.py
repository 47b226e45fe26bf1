"""The autograd wrapper against the fp64 oracle (GPU)."""

import numpy as np
import pytest
import torch
import torch.utils.checkpoint

from attention_attn_fwd_amd import synth
from attention_attn_fwd_amd.autograd import sink_attention
from oracle import ref_bwd, ref_fwd

from _util import GRAD_REL_L2, check_out_lse, f64, need_gpu, rel_l2

pytestmark = pytest.mark.gpu


def _leaves(case, dev):
    return [t.to(dev).requires_grad_(True) for t in (case.q, case.k, case.v, case.sinks)]


@pytest.mark.parametrize("window", [0, 128])
def test_autograd_matches_oracle(window):
    dev = need_gpu()
    case = synth.make_prefill(2, 300, 16, 2, seed=41)
    dout = synth.make_dout(tuple(case.q.shape), seed=42)
    q, k, v, s = _leaves(case, dev)
    out, lse = sink_attention(q, k, v, s, window, case.scale, return_lse=True)
    (out.float() * dout.to(dev).float()).sum().backward()
    torch.cuda.synchronize()
    ro, rl = ref_fwd(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), window, case.scale)
    check_out_lse(f64(out.detach()), f64(lse), ro, rl, f"autograd fwd W={window}")
    ref = ref_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout), window, case.scale)
    for t, r, n in zip((q, k, v, s), ref, ("dq", "dk", "dv", "dsinks")):
        assert t.grad is not None and t.grad.dtype == t.dtype, n
        e = rel_l2(f64(t.grad), r)
        print(f"{n} rel L2 {e:.2e}", flush=True)
        assert e <= GRAD_REL_L2, n


def test_autograd_partial_requires_grad_and_noncontiguous_dout():
    dev = need_gpu()
    case = synth.make_prefill(1, 200, 8, 1, seed=43)
    q = case.q.to(dev).requires_grad_(True)
    k, v, s = (t.to(dev) for t in (case.k, case.v, case.sinks))
    out = sink_attention(q, k, v, s, 128)
    g = torch.randn(out.shape[::-1], device=dev).to(torch.bfloat16).permute(3, 2, 1, 0)  # non-contiguous
    out.backward(g)
    torch.cuda.synchronize()
    ref = ref_bwd(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(g.cpu()), 128, case.scale)
    assert k.grad is None and v.grad is None and s.grad is None
    assert rel_l2(f64(q.grad), ref[0]) <= GRAD_REL_L2


def test_autograd_under_checkpoint_is_bitwise_equal():
    dev = need_gpu()
    case = synth.make_prefill(1, 256, 8, 1, seed=44)
    dout = synth.make_dout(tuple(case.q.shape), seed=45).to(dev)
    grads = []
    for use_ckpt in (False, True):
        q, k, v, s = _leaves(case, dev)
        f = lambda a, b, c, d: sink_attention(a, b, c, d, 0)
        out = torch.utils.checkpoint.checkpoint(f, q, k, v, s, use_reentrant=False) if use_ckpt else f(q, k, v, s)
        out.backward(dout)
        torch.cuda.synchronize()
        grads.append([t.grad.clone() for t in (q, k, v, s)])
    for a, b in zip(*grads):
        assert torch.equal(a, b)
