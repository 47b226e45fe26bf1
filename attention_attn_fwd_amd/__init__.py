"""MI355X (gfx950) sink attention: causal / sliding-window grouped-query
attention with a learned per-head sink logit, behind a C ABI.

Python layer = argument marshalling over libgptoss_attn.so (see
include/gptoss_attn.h).  torch provides device memory and the current stream;
all computation runs in the library's HIP kernels.

    out, lse = fwd(q, k, v, sinks, window, scale)
    dq, dk, dv, dsinks = bwd(q, k, v, sinks, out, lse, dout, window, scale)
    out, lse = decode(q, k_cache, v_cache, cu_seqlens, sinks, max_seqlen, window, scale)
    out, lse = decode_paged(q, k_pages, v_pages, block_table, seq_lens, sinks, max_seqlen, window, scale,
                            ring_tokens)
    out, lse = fwd_varlen(q, k, v, cu_seqlens, sinks, max_seqlen, window, scale)     # packed documents
    dq, dk, dv, dsinks = bwd_varlen(q, k, v, cu_seqlens, sinks, out, lse, dout, max_seqlen, window, scale)
    table = rope_table(positions, base, factor, orig_ctx, alpha, beta)          # YaRN rotary table
    out, lse, k_rot = fwd_rope(q, k, v, sinks, table, window, scale)            # RoPE fused into prefill
    out, lse = decode_rope(q, k_cache, v_cache, cu_seqlens, sinks, table, max_seqlen, window, scale)
    y = rope_rows(x, positions, table)                                          # rotate rows (cache append)
    dq, dk, dv, dsinks = bwd_rope(q, k_rot, v, sinks, table, out, lse, dout, window, scale)  # grads wrt unrotated q, k

Training: attention_attn_fwd_amd.autograd.sink_attention (torch autograd over
fwd/bwd).
"""

import torch

from . import _lib
from ._lib import AttnError

__all__ = ["fwd", "bwd", "decode", "decode_noalloc", "decode_paged", "fwd_varlen", "bwd_varlen", "bwd_workspace_size",
           "bwd_varlen_workspace_size", "decode_workspace_size", "decode_workspace", "rope_table", "rope_rows", "fwd_rope", "decode_rope",
           "bwd_rope", "bwd_rope_workspace_size",
           "AttnError", "abi_version"]


def _need(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on(dev, *named):
    """Every (tensor, name) pair lives on device `dev`."""
    for t, name in named:
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev} (all tensors of a call on one device)")


def _buffer(t, name, dtype, shape, dev):
    """A caller-provided output buffer: exact dtype, shape, contiguity and
    device (the kernels write exactly that many elements)."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _on(dev, (t, name))
    return t


def _workspace(ws, need, dev):
    """The caller's workspace (any dtype, contiguous, on `dev`) or a new one;
    returns (tensor, size in bytes).  The library checks the size."""
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous torch.Tensor")
    _on(dev, (ws, "workspace"))
    return ws, ws.numel() * ws.element_size()


def _grads(grads, q, k, v, Hq):
    """Gradient buffers: new ones, or the caller's (dq, dk, dv, dsinks) checked
    against q, k, v and Hq."""
    if grads is None:
        return (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                torch.empty((Hq,), dtype=torch.float32, device=q.device))
    dq, dk, dv, dsinks = grads
    for t, n, ref in ((dq, "dq", q), (dk, "dk", k), (dv, "dv", v)):
        _buffer(t, n, torch.bfloat16, ref.shape, q.device)
    _buffer(dsinks, "dsinks", torch.float32, (Hq,), q.device)
    return dq, dk, dv, dsinks


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def abi_version():
    return _lib.load().gptoss_attn_abi_version()


def fwd(q, k, v, sinks, window=0, scale=None, out=None, lse=None):
    """Prefill forward.  q [B,S,Hq,D], k/v [B,S,Hkv,D] bf16; sinks [Hq] fp32.

    Returns (out bf16 [B,S,Hq,D], lse fp32 [B,Hq,S]).
    """
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(sinks, "sinks", torch.float32, 1)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or sinks.shape != (Hq,):
        raise ValueError("shape mismatch among q, k, v, sinks")
    _on(q.device, (k, "k"), (v, "v"), (sinks, "sinks"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else _buffer(out, "out", torch.bfloat16, q.shape, q.device)
    lse = (torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None
           else _buffer(lse, "lse", torch.float32, (B, Hq, S), q.device))
    lib = _lib.load()
    st = lib.gptoss_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), sinks.data_ptr(), B, S, Hq, Hkv, D,
                             int(window), scale, out.data_ptr(), lse.data_ptr(), _stream(q.device))
    _lib.check(st, lib)
    return out, lse


def bwd_workspace_size(B, S, Hq, Hkv, D=64, window=0):
    return int(_lib.load().gptoss_attn_bwd_workspace_size(B, S, Hq, Hkv, D, int(window)))


def bwd(q, k, v, sinks, out, lse, dout, window=0, scale=None, workspace=None, grads=None):
    """Backward of sum(dout * out).  Returns (dq, dk, dv bf16, dsinks fp32 [Hq]),
    written into `grads` = (dq, dk, dv, dsinks) when given."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(sinks, "sinks", torch.float32, 1)
    _need(lse, "lse", torch.float32, 3)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if (k.shape != (B, S, Hkv, D) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape
            or lse.shape != (B, Hq, S) or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among backward inputs")
    _on(q.device, (k, "k"), (v, "v"), (sinks, "sinks"), (out, "out"), (lse, "lse"), (dout, "dout"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    dq, dk, dv, dsinks = _grads(grads, q, k, v, Hq)
    workspace, ws_bytes = _workspace(workspace, bwd_workspace_size(B, S, Hq, Hkv, D, window), q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), sinks.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), dout.data_ptr(), B, S, Hq, Hkv, D, int(window), scale,
                             dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dsinks.data_ptr(),
                             workspace.data_ptr(), ws_bytes, _stream(q.device))
    _lib.check(st, lib)
    return dq, dk, dv, dsinks


def _decode_outputs(out, lse, q):
    N, Hq, _ = q.shape
    out = torch.empty_like(q) if out is None else _buffer(out, "out", torch.bfloat16, q.shape, q.device)
    lse = (torch.empty((N, Hq), dtype=torch.float32, device=q.device) if lse is None
           else _buffer(lse, "lse", torch.float32, (N, Hq), q.device))
    return out, lse


def decode_workspace_size(N, Hq, Hkv, D=64, max_seqlen=1, window=0):
    return int(_lib.load().gptoss_attn_decode_workspace_size(N, Hq, Hkv, D, max_seqlen, int(window)))


def decode_workspace(N, Hq, Hkv, max_seqlen, window=0, D=64, device=None):
    """A decode workspace for these sizes (reusable by later calls on one
    stream with the same or smaller sizes)."""
    need = decode_workspace_size(N, Hq, Hkv, D, max_seqlen, window)
    return torch.empty(max(need, 1), dtype=torch.uint8, device=device or torch.device("cuda"))


def decode(q, k_cache, v_cache, cu_seqlens, sinks, max_seqlen, window=0, scale=None, out=None, lse=None,
           workspace=None):
    """Decode one token per sequence.  q [N,Hq,D]; caches [T,Hkv,D] bf16;
    cu_seqlens int32 [N+1] on the device.  Returns (out bf16 [N,Hq,D], lse fp32 [N,Hq])."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(sinks, "sinks", torch.float32, 1)
    N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if (v_cache.shape != k_cache.shape or k_cache.shape[2] != D or cu_seqlens.shape != (N + 1,)
            or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among decode inputs")
    _on(q.device, (k_cache, "k_cache"), (v_cache, "v_cache"), (cu_seqlens, "cu_seqlens"), (sinks, "sinks"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out, lse = _decode_outputs(out, lse, q)
    workspace, ws_bytes = _workspace(workspace, decode_workspace_size(N, Hq, Hkv, D, max_seqlen, window), q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens.data_ptr(),
                                sinks.data_ptr(), N, Hq, Hkv, D, int(max_seqlen), int(window), scale,
                                out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), ws_bytes,
                                _stream(q.device))
    _lib.check(st, lib)
    return out, lse


def decode_noalloc(q, k_cache, v_cache, cu_seqlens, sinks, max_seqlen, window=0, scale=None, out=None, lse=None):
    """decode() through gptoss_attn_decode_noalloc: no workspace; the split
    partials live in the library's per-GPU scratch array (calls that may
    overlap on one GPU race on it)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(sinks, "sinks", torch.float32, 1)
    N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if (v_cache.shape != k_cache.shape or k_cache.shape[2] != D or cu_seqlens.shape != (N + 1,)
            or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among decode inputs")
    _on(q.device, (k_cache, "k_cache"), (v_cache, "v_cache"), (cu_seqlens, "cu_seqlens"), (sinks, "sinks"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out, lse = _decode_outputs(out, lse, q)
    lib = _lib.load()
    st = lib.gptoss_attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens.data_ptr(),
                                        sinks.data_ptr(), N, Hq, Hkv, D, int(max_seqlen), int(window), scale,
                                        out.data_ptr(), lse.data_ptr(), _stream(q.device))
    _lib.check(st, lib)
    return out, lse


def decode_paged(q, k_pages, v_pages, block_table, seq_lens, sinks, max_seqlen, window=0, scale=None,
                 ring_tokens=0, out=None, lse=None, workspace=None):
    """Decode against a paged KV cache.  q [N,Hq,D]; pages [P, page_size, Hkv, D] bf16;
    block_table int32 [N, pages_per_seq] and seq_lens int32 [N] on the device; ring_tokens = 0
    for a linear cache, else the ring size of a sliding layer's cache.  Returns (out, lse)."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(seq_lens, "seq_lens", torch.int32, 1)
    _need(sinks, "sinks", torch.float32, 1)
    N, Hq, D = q.shape
    _, page_size, Hkv, Dk = k_pages.shape
    if (v_pages.shape != k_pages.shape or Dk != D or block_table.shape[0] != N or seq_lens.shape != (N,)
            or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among paged decode inputs")
    _on(q.device, (k_pages, "k_pages"), (v_pages, "v_pages"), (block_table, "block_table"), (seq_lens, "seq_lens"),
        (sinks, "sinks"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out, lse = _decode_outputs(out, lse, q)
    workspace, ws_bytes = _workspace(workspace, decode_workspace_size(N, Hq, Hkv, D, max_seqlen, window), q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                                      seq_lens.data_ptr(), sinks.data_ptr(), N, Hq, Hkv, D, page_size,
                                      block_table.shape[1], int(ring_tokens), int(max_seqlen), int(window), scale,
                                      out.data_ptr(), lse.data_ptr(), workspace.data_ptr(), ws_bytes,
                                      _stream(q.device))
    _lib.check(st, lib)
    return out, lse


def fwd_varlen(q, k, v, cu_seqlens, sinks, max_seqlen, window=0, scale=None, out=None, lse=None):
    """Prefill forward over documents packed along the token dimension.

    q [T,Hq,D], k/v [T,Hkv,D] bf16; cu_seqlens int32 [N+1] on the device
    (document b = rows cu_seqlens[b] .. cu_seqlens[b+1]-1, attention confined
    to it); max_seqlen bounds every document length.  Returns
    (out bf16 [T,Hq,D], lse fp32 [Hq,T]); rows outside every document are not
    written.
    """
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(sinks, "sinks", torch.float32, 1)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    N = cu_seqlens.shape[0] - 1
    if N < 0 or k.shape != (T, Hkv, D) or v.shape != k.shape or sinks.shape != (Hq,):
        raise ValueError("shape mismatch among q, k, v, cu_seqlens, sinks")
    _on(q.device, (k, "k"), (v, "v"), (cu_seqlens, "cu_seqlens"), (sinks, "sinks"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else _buffer(out, "out", torch.bfloat16, q.shape, q.device)
    lse = (torch.empty((Hq, T), dtype=torch.float32, device=q.device) if lse is None
           else _buffer(lse, "lse", torch.float32, (Hq, T), q.device))
    lib = _lib.load()
    st = lib.gptoss_attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                    sinks.data_ptr(), N, T, Hq, Hkv, D, int(max_seqlen), int(window), scale,
                                    out.data_ptr(), lse.data_ptr(), _stream(q.device))
    _lib.check(st, lib)
    return out, lse


def bwd_varlen_workspace_size(T, Hq, Hkv, D=64):
    return int(_lib.load().gptoss_attn_bwd_varlen_workspace_size(T, Hq, Hkv, D))


def bwd_varlen(q, k, v, cu_seqlens, sinks, out, lse, dout, max_seqlen, window=0, scale=None, workspace=None,
               grads=None):
    """Backward of fwd_varlen for sum(dout * out).  Returns (dq, dk, dv bf16,
    dsinks fp32 [Hq]), written into `grads` = (dq, dk, dv, dsinks) when given;
    rows outside every document are not written."""
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(sinks, "sinks", torch.float32, 1)
    _need(lse, "lse", torch.float32, 2)
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    N = cu_seqlens.shape[0] - 1
    if (N < 0 or k.shape != (T, Hkv, D) or v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape
            or lse.shape != (Hq, T) or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among varlen backward inputs")
    _on(q.device, (k, "k"), (v, "v"), (cu_seqlens, "cu_seqlens"), (sinks, "sinks"), (out, "out"), (lse, "lse"),
        (dout, "dout"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    dq, dk, dv, dsinks = _grads(grads, q, k, v, Hq)
    workspace, ws_bytes = _workspace(workspace, bwd_varlen_workspace_size(T, Hq, Hkv, D), q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                    sinks.data_ptr(), out.data_ptr(), lse.data_ptr(), dout.data_ptr(), N, T, Hq,
                                    Hkv, D, int(max_seqlen), int(window), scale, dq.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), dsinks.data_ptr(), workspace.data_ptr(), ws_bytes,
                                    _stream(q.device))
    _lib.check(st, lib)
    return dq, dk, dv, dsinks


def rope_table(positions, base, factor=1.0, orig_ctx=1.0, alpha=1.0, beta=32.0, device=None, out=None):
    """YaRN rotary table fp32 [positions, 32, 2] = (m cos(p h_i), m sin(p h_i))."""
    dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
    out = (torch.empty((int(positions), 32, 2), dtype=torch.float32, device=dev) if out is None
           else _buffer(out, "table", torch.float32, (int(positions), 32, 2), out.device))
    lib = _lib.load()
    st = lib.gptoss_attn_rope_table(out.data_ptr(), int(positions), 64, float(base), float(factor),
                                    float(orig_ctx), float(alpha), float(beta), _stream(out.device))
    _lib.check(st, lib)
    return out


def _need_table(table):
    _need(table, "table", torch.float32, 3)
    if table.shape[1:] != (32, 2):
        raise ValueError("table must be [positions, 32, 2]")


def rope_rows(x, positions, table, out=None, transpose=False):
    """Rotate rows x bf16 [T, H, 64] by positions int32 [T] (device); with
    transpose, apply the adjoint R^T (gradients back to unrotated rows)."""
    _need(x, "x", torch.bfloat16, 3)
    _need(positions, "positions", torch.int32, 1)
    _need_table(table)
    T, H, D = x.shape
    if positions.shape != (T,):
        raise ValueError("positions must be [T]")
    _on(x.device, (positions, "positions"), (table, "table"))
    out = torch.empty_like(x) if out is None else _buffer(out, "out", torch.bfloat16, x.shape, x.device)
    lib = _lib.load()
    st = lib.gptoss_attn_rope_rows(x.data_ptr(), out.data_ptr(), positions.data_ptr(), T, H, D, table.data_ptr(),
                                   table.shape[0], 1 if transpose else 0, _stream(x.device))
    _lib.check(st, lib)
    return out


def fwd_rope(q, k, v, sinks, table, window=0, scale=None, out=None, lse=None, k_rot=None):
    """Prefill forward over RoPE-rotated q and k (token i at position i).
    Returns (out, lse, k_rot) with k_rot the rotated keys [B,S,Hkv,64]."""
    _need(q, "q", torch.bfloat16, 4)
    _need(k, "k", torch.bfloat16, 4)
    _need(v, "v", torch.bfloat16, 4)
    _need(sinks, "sinks", torch.float32, 1)
    _need_table(table)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or sinks.shape != (Hq,):
        raise ValueError("shape mismatch among q, k, v, sinks")
    _on(q.device, (k, "k"), (v, "v"), (sinks, "sinks"), (table, "table"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else _buffer(out, "out", torch.bfloat16, q.shape, q.device)
    lse = (torch.empty((B, Hq, S), dtype=torch.float32, device=q.device) if lse is None
           else _buffer(lse, "lse", torch.float32, (B, Hq, S), q.device))
    k_rot = torch.empty_like(k) if k_rot is None else _buffer(k_rot, "k_rot", torch.bfloat16, k.shape, q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_fwd_rope(q.data_ptr(), k.data_ptr(), v.data_ptr(), sinks.data_ptr(), table.data_ptr(),
                                  table.shape[0], B, S, Hq, Hkv, D, int(window), scale, out.data_ptr(),
                                  lse.data_ptr(), k_rot.data_ptr(), _stream(q.device))
    _lib.check(st, lib)
    return out, lse, k_rot


def decode_rope(q, k_cache, v_cache, cu_seqlens, sinks, table, max_seqlen, window=0, scale=None, out=None, lse=None,
                workspace=None):
    """Decode with q rotated at position L_n - 1; the caches hold rotated keys."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    _need(sinks, "sinks", torch.float32, 1)
    _need_table(table)
    N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if (v_cache.shape != k_cache.shape or k_cache.shape[2] != D or cu_seqlens.shape != (N + 1,)
            or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among decode inputs")
    _on(q.device, (k_cache, "k_cache"), (v_cache, "v_cache"), (cu_seqlens, "cu_seqlens"), (sinks, "sinks"),
        (table, "table"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    out, lse = _decode_outputs(out, lse, q)
    workspace, ws_bytes = _workspace(workspace, decode_workspace_size(N, Hq, Hkv, D, max_seqlen, window), q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_decode_rope(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens.data_ptr(),
                                     sinks.data_ptr(), table.data_ptr(), table.shape[0], N, Hq, Hkv, D,
                                     int(max_seqlen), int(window), scale, out.data_ptr(), lse.data_ptr(),
                                     workspace.data_ptr(), ws_bytes, _stream(q.device))
    _lib.check(st, lib)
    return out, lse


def bwd_rope_workspace_size(B, S, Hq, Hkv, D=64):
    return int(_lib.load().gptoss_attn_bwd_rope_workspace_size(B, S, Hq, Hkv, D))


def bwd_rope(q, k_rot, v, sinks, table, out, lse, dout, window=0, scale=None, workspace=None, grads=None):
    """Backward of fwd_rope for sum(dout * out): (dq, dk, dv, dsinks) with dq,
    dk the gradients with respect to the unrotated q and k.  k_rot is
    fwd_rope's rotated-key output."""
    for t, n in ((q, "q"), (k_rot, "k_rot"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4)
    _need(sinks, "sinks", torch.float32, 1)
    _need(lse, "lse", torch.float32, 3)
    _need_table(table)
    B, S, Hq, D = q.shape
    Hkv = k_rot.shape[2]
    if (k_rot.shape != (B, S, Hkv, D) or v.shape != k_rot.shape or out.shape != q.shape or dout.shape != q.shape
            or lse.shape != (B, Hq, S) or sinks.shape != (Hq,)):
        raise ValueError("shape mismatch among backward inputs")
    _on(q.device, (k_rot, "k_rot"), (v, "v"), (sinks, "sinks"), (table, "table"), (out, "out"), (lse, "lse"),
        (dout, "dout"))
    scale = (1.0 / D ** 0.5) if scale is None else float(scale)
    dq, dk, dv, dsinks = _grads(grads, q, k_rot, v, Hq)
    workspace, ws_bytes = _workspace(workspace, bwd_rope_workspace_size(B, S, Hq, Hkv, D), q.device)
    lib = _lib.load()
    st = lib.gptoss_attn_bwd_rope(q.data_ptr(), k_rot.data_ptr(), v.data_ptr(), sinks.data_ptr(), table.data_ptr(),
                                  table.shape[0], out.data_ptr(), lse.data_ptr(), dout.data_ptr(), B, S, Hq, Hkv, D,
                                  int(window), scale, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dsinks.data_ptr(),
                                  workspace.data_ptr(), ws_bytes, _stream(q.device))
    _lib.check(st, lib)
    return dq, dk, dv, dsinks
