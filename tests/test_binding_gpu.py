"""The Python binding refuses caller buffers the kernels would overrun and
tensors on another device, before any launch (GPU: the checks need device
tensors)."""

import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth

from _util import need_gpu

pytestmark = pytest.mark.gpu


def _prefill(dev):
    case = synth.make_prefill(1, 64, 8, 1, seed=3)
    return case, [t.to(dev) for t in (case.q, case.k, case.v, case.sinks)]


def test_fwd_rejects_wrong_output_buffers():
    dev = need_gpu()
    case, (q, k, v, s) = _prefill(dev)
    with pytest.raises(ValueError, match="out must have shape"):
        attn.fwd(q, k, v, s, 0, case.scale, out=torch.empty_like(q)[:, :32])
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.fwd(q, k, v, s, 0, case.scale, lse=torch.empty(1, 8, 32, device=dev))
    with pytest.raises(ValueError, match="sinks must be on a HIP device"):
        attn.fwd(q, k, v, case.sinks, 0, case.scale)
    with pytest.raises(ValueError, match="k_rot must have shape"):
        attn.fwd_rope(q, k, v, s, attn.rope_table(64, 10000.0), 0, case.scale, k_rot=torch.empty_like(q))


def test_bwd_rejects_wrong_gradient_buffers_and_workspace():
    dev = need_gpu()
    case, (q, k, v, s) = _prefill(dev)
    out, lse = attn.fwd(q, k, v, s, 0, case.scale)
    dout = torch.ones_like(q)
    bad = (torch.empty_like(q), torch.empty_like(q), torch.empty_like(v), torch.empty(8, device=dev))
    with pytest.raises(ValueError, match="dk must have shape"):
        attn.bwd(q, k, v, s, out, lse, dout, 0, case.scale, grads=bad)
    with pytest.raises(ValueError, match="workspace is on cpu"):
        attn.bwd(q, k, v, s, out, lse, dout, 0, case.scale, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()


def test_decode_and_rope_reject_wrong_output_buffers():
    dev = need_gpu()
    dec = synth.make_decode(4, 8, 1, max_len=100, seed=4)
    t = [x.to(dev) for x in (dec.q, dec.k_cache, dec.v_cache, dec.cu_seqlens, dec.sinks)]
    with pytest.raises(ValueError, match="lse must have shape"):
        attn.decode(*t, dec.max_seqlen, 0, dec.scale, lse=torch.empty(4, 4, device=dev))
    with pytest.raises(ValueError, match="table must have shape"):
        attn.rope_table(100, 10000.0, out=torch.empty(50, 32, 2, device=dev))
    x = torch.zeros(10, 2, 64, dtype=torch.bfloat16, device=dev)
    pos = torch.zeros(10, dtype=torch.int32, device=dev)
    with pytest.raises(ValueError, match="out must have shape"):
        attn.rope_rows(x, pos, attn.rope_table(16, 10000.0), out=torch.empty(5, 2, 64, dtype=torch.bfloat16,
                                                                              device=dev))
    torch.cuda.synchronize()
