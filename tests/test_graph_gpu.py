"""The ABI calls under HIP graph capture (GPU).

Every entry point launches on the caller's stream and makes no allocation,
host synchronisation or memset, so a caller can capture it.  Each graph is
replayed several times with eager launches and synchronisations between the
replays, and every replay must equal the eager result bit for bit (all
kernels are deterministic)."""

import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth

from _util import need_gpu

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("window", [0, 128])
def test_prefill_fwd_bwd_graph_replays(window):
    dev = need_gpu()
    case = synth.make_prefill(2, 700, 16, 2, seed=31)
    other = synth.make_prefill(2, 700, 16, 2, seed=32)
    q, k, v, s = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    q2, k2, v2 = (t.to(dev) for t in (other.q, other.k, other.v))
    do = synth.make_dout(tuple(case.q.shape), seed=33).to(dev)
    B, S, Hq, D = q.shape
    ref_o, ref_l = attn.fwd(q, k, v, s, window, case.scale)
    ref_g = attn.bwd(q, k, v, s, ref_o, ref_l, do, window, case.scale)
    torch.cuda.synchronize()

    o, l = torch.empty_like(q), torch.empty(B, Hq, S, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty(Hq, device=dev))
    ws = torch.empty(max(1, attn.bwd_workspace_size(B, S, Hq, k.shape[2], D, window)), dtype=torch.uint8,
                     device=dev)

    def body():
        attn.fwd(q, k, v, s, window, case.scale, out=o, lse=l)
        attn.bwd(q, k, v, s, o, l, do, window, case.scale, workspace=ws, grads=grads)

    g = _capture(body)
    for rep in range(3):
        for t in (o, l, *grads):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"replay {rep}: fwd differs"
        for a, b in zip(grads, ref_g):
            assert torch.equal(a, b), f"replay {rep}: bwd differs"
        # eager work on other inputs between the replays
        attn.fwd(q2, k2, v2, s, window, case.scale)
        torch.cuda.synchronize()


@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("lengths", [None, [40000, 3, 700]], ids=["n64", "chunked"])
def test_decode_graph_replays(window, lengths):
    dev = need_gpu()
    N = 64 if lengths is None else len(lengths)
    case = synth.make_decode(N, 64, 8, max_len=1024, lengths=lengths, seed=34)
    t = [x.to(dev) for x in (case.q, case.k_cache, case.v_cache, case.cu_seqlens, case.sinks)]
    ref_o, ref_l = attn.decode(*t, case.max_seqlen, window, case.scale)
    torch.cuda.synchronize()
    o, l = torch.empty_like(ref_o), torch.empty_like(ref_l)
    need = attn.decode_workspace_size(N, 64, 8, 64, case.max_seqlen, window)
    ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    g = _capture(lambda: attn.decode(*t, case.max_seqlen, window, case.scale, out=o, lse=l, workspace=ws))
    for rep in range(3):
        o.fill_(float("nan"))
        l.fill_(float("nan"))
        ws.fill_(0xFF)  # stale partials must not leak into the result
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"replay {rep} differs"
        attn.decode(t[0], t[1], t[2], t[3], t[4], case.max_seqlen, 0, 0.5)
        torch.cuda.synchronize()
