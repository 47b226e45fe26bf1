"""gptoss_attn_decode_noalloc (the decode entry point that allocates nothing:
its split partials live in the library's per-GPU scratch array) against
gptoss_attn_decode with a caller workspace, through the C ABI (GPU)."""

import ctypes

import pytest
import torch

from attention_attn_fwd_amd import _lib, synth

from _util import need_gpu

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(lib, case, window, dev):
    """(out, lse) of the no-allocation entry point and of the workspace one,
    each into NaN-filled outputs."""
    q, kc, vc, cu, sk = (x.to(dev) for x in (case.q, case.k_cache, case.v_cache, case.cu_seqlens, case.sinks))
    N, Hq, D = q.shape
    Hkv = kc.shape[1]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = []
    for noalloc in (True, False):
        out = torch.full((N, Hq, D), float("nan"), dtype=torch.bfloat16, device=dev)
        lse = torch.full((N, Hq), float("nan"), dtype=torch.float32, device=dev)
        args = [_ptr(q), _ptr(kc), _ptr(vc), _ptr(cu), _ptr(sk), N, Hq, Hkv, D, case.max_seqlen, window,
                ctypes.c_float(case.scale), _ptr(out), _ptr(lse)]
        if noalloc:
            st = lib.gptoss_attn_decode_noalloc(*args, stream)
        else:
            need = lib.gptoss_attn_decode_workspace_size(N, Hq, Hkv, D, case.max_seqlen, window)
            ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
            st = lib.gptoss_attn_decode(*args, _ptr(ws), ctypes.c_size_t(ws.numel()), stream)
        _lib.check(st, lib)
        res.append((out, lse))
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("window", [0, 1000])
def test_noalloc_matches_workspace_decode_twice(window):
    """Two calls in a row, the second with a smaller input: both the same bit
    for bit as gptoss_attn_decode with its own workspace (the same kernels;
    the first call's partials left in the scratch array do not leak into the
    second).  The first input is cut into chunks, so the scratch array is used
    (a window of 128 keys is decoded unsplit; 1000 is cut)."""
    dev = need_gpu()
    lib = _lib.load()
    big = synth.make_decode(8, 64, 8, lengths=[2048, 1, 700, 1500, 64, 2047, 333, 1024], seed=71 + window)
    small = synth.make_decode(3, 64, 8, lengths=[900, 5, 400], seed=72 + window)
    assert lib.gptoss_attn_decode_workspace_size(8, 64, 8, 64, big.max_seqlen, window) > 0
    for case in (big, small):
        print(f"noalloc decode N={case.q.shape[0]} max_seqlen={case.max_seqlen} W={window}", flush=True)
        (o1, l1), (o2, l2) = _both(lib, case, window, dev)
        assert torch.isfinite(o1.float()).all() and torch.isfinite(l1).all()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_noalloc_workload_without_partials():
    """The 128-sequence decode workload (one chunk per sequence: the scratch
    array is not needed) gives the workspace entry point's result."""
    dev = need_gpu()
    lib = _lib.load()
    case = synth.config_inputs("decode_n128_l1024_h64x8")
    for window in (0, 128):
        (o1, l1), (o2, l2) = _both(lib, case, window, dev)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
