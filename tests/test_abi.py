"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any HIP call."""

import ctypes
import math
import os
import re

import pytest

from attention_attn_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptoss_attn.h")

P = 0x10000  # a 256-byte aligned, never dereferenced stand-in pointer


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gptoss_attn_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS), names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.gptoss_attn_abi_version() == 1


def _fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, sinks=P, B=1, S=16, Hq=8, Hkv=1, D=64, window=0, scale=0.125, out=P, lse=P,
             stream=None)
    a.update(kw)
    return lib.gptoss_attn_fwd(a["q"], a["k"], a["v"], a["sinks"], a["B"], a["S"], a["Hq"], a["Hkv"], a["D"],
                               a["window"], a["scale"], a["out"], a["lse"], a["stream"])


@pytest.mark.parametrize("kw,status,frag", [
    (dict(q=None), 1, "q is NULL"),
    (dict(k=None), 1, "k is NULL"),
    (dict(out=None), 1, "out is NULL"),
    (dict(lse=None), 1, "lse is NULL"),
    (dict(sinks=None), 1, "sinks is NULL"),
    (dict(q=P + 8), 1, "aligned"),
    (dict(lse=P + 2), 1, "aligned"),
    (dict(B=-1), 1, "must be >= 0"),
    (dict(S=-3), 1, "must be >= 0"),
    (dict(Hq=0), 1, ">= 1"),
    (dict(Hkv=0), 1, ">= 1"),
    (dict(Hq=8, Hkv=3), 1, "multiple"),
    (dict(window=-1), 1, "window"),
    (dict(scale=0.0), 1, "softmax_scale"),
    (dict(scale=-1.0), 1, "softmax_scale"),
    (dict(scale=math.inf), 1, "softmax_scale"),
    (dict(scale=math.nan), 1, "softmax_scale"),
    (dict(D=128), 2, "head_dim"),
    (dict(Hq=512, Hkv=1), 2, "group size"),
    (dict(B=65536, S=65536), 1, "exceeds"),
])
def test_fwd_rejects_bad_arguments(lib, kw, status, frag):
    st = _fwd(lib, **kw)
    assert st == status
    assert frag in lib.gptoss_attn_last_error().decode()


def test_zero_sized_problems_are_noops(lib):
    assert _fwd(lib, B=0, q=None, k=None, v=None, sinks=None, out=None, lse=None) == 0
    assert _fwd(lib, S=0, q=None, k=None, v=None, sinks=None, out=None, lse=None) == 0
    st = lib.gptoss_attn_decode(None, None, None, None, None, 0, 8, 1, 64, 1, 0, 0.125, None, None, None, 0,
                                None)
    assert st == 0
    st = lib.gptoss_attn_bwd(*([None] * 7), 0, 4, 8, 1, 64, 0, 0.125, *([None] * 5), 0, None)
    assert st == 0


def _bwd(lib, ws=P, ws_bytes=None, **kw):
    a = dict(B=1, S=256, Hq=8, Hkv=1, D=64, window=0, scale=0.125)
    a.update(kw)
    need = lib.gptoss_attn_bwd_workspace_size(a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["window"])
    ptrs = [P] * 7
    outs = [P] * 4
    if "dq" in kw:
        outs[0] = kw.pop("dq")
    return lib.gptoss_attn_bwd(*ptrs, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["window"], a["scale"],
                               *outs, ws, need if ws_bytes is None else ws_bytes, None), need


def test_bwd_rejects_small_workspace(lib):
    st, need = _bwd(lib)
    if need > 0:
        st, _ = _bwd(lib, ws_bytes=need - 1)
        assert st == 1 and "workspace" in lib.gptoss_attn_last_error().decode()
        st, _ = _bwd(lib, ws=P + 64)
        assert st == 1 and "aligned" in lib.gptoss_attn_last_error().decode()


def test_bwd_rejects_bad_arguments(lib):
    st = lib.gptoss_attn_bwd(*([P] * 7), 1, 64, 8, 3, 64, 0, 0.125, *([P] * 4), P, 1 << 30, None)
    assert st == 1 and "multiple" in lib.gptoss_attn_last_error().decode()
    st = lib.gptoss_attn_bwd(*([P] * 7), 1, 64, 8, 1, 64, 0, 0.125, None, P, P, P, P, 1 << 30, None)
    assert st == 1 and "dq is NULL" in lib.gptoss_attn_last_error().decode()


def _dec(lib, **kw):
    a = dict(q=P, kc=P, vc=P, cu=P, sinks=P, N=2, Hq=64, Hkv=8, D=64, max_seqlen=65536, window=0,
             scale=0.125, out=P, lse=P, ws=P, ws_bytes=None)
    a.update(kw)
    need = lib.gptoss_attn_decode_workspace_size(a["N"], a["Hq"], a["Hkv"], a["D"], a["max_seqlen"],
                                                 a["window"])
    wb = need if a["ws_bytes"] is None else a["ws_bytes"]
    return lib.gptoss_attn_decode(a["q"], a["kc"], a["vc"], a["cu"], a["sinks"], a["N"], a["Hq"], a["Hkv"],
                                  a["D"], a["max_seqlen"], a["window"], a["scale"], a["out"], a["lse"],
                                  a["ws"], wb, None)


@pytest.mark.parametrize("kw,frag", [
    (dict(cu=None), "cu_seqlens is NULL"),
    (dict(max_seqlen=0), "max_seqlen"),
    (dict(max_seqlen=(1 << 30) + 1), "exceeds 2^30"),
    (dict(max_seqlen=2 ** 31 - 1), "exceeds 2^30"),
    (dict(N=-1), "N"),
    (dict(N=70000), "exceeds"),
    (dict(window=-2), "window"),
    (dict(ws_bytes=1), "workspace"),
    (dict(ws=None), "workspace is NULL"),
    (dict(kc=P + 4), "aligned"),
])
def test_decode_rejects_bad_arguments(lib, kw, frag):
    assert _dec(lib, **kw) == 1
    assert frag in lib.gptoss_attn_last_error().decode()


def test_decode_refuses_more_kv_heads_than_its_grid_holds(lib):
    # ceil(131072 / 2) = 65536 workgroup rows: one more than a launch takes
    for call in (lambda: _dec(lib, Hq=131072, Hkv=131072),
                 lambda: _paged(lib, Hq=131072, Hkv=131072)):
        assert call() == 2
        assert "more than 65535" in lib.gptoss_attn_last_error().decode()
    # the largest accepted count gets past the check (and fails later, on the
    # host, at the missing cu_seqlens)
    assert _dec(lib, Hq=131070, Hkv=131070, cu=None) == 1
    assert "cu_seqlens is NULL" in lib.gptoss_attn_last_error().decode()


def test_workspace_size_queries(lib):
    # a long single sequence is cut into chunks whose partials need a workspace
    assert lib.gptoss_attn_decode_workspace_size(1, 64, 8, 64, 65536, 0) > 0
    # 128 sequences of <= 1024 keys fill the chip one chunk each: no partials
    assert lib.gptoss_attn_decode_workspace_size(128, 64, 8, 64, 1024, 0) == 0
    assert lib.gptoss_attn_decode_workspace_size(128, 64, 8, 64, 1024, 128) == 0
    assert lib.gptoss_attn_decode_workspace_size(128, 64, 8, 128, 1024, 0) == 0  # unsupported D
    assert lib.gptoss_attn_bwd_workspace_size(4, 4096, 64, 8, 64, 0) >= 0
    assert lib.gptoss_attn_bwd_workspace_size(4, 4096, 64, 7, 64, 0) == 0


def test_decode_workspace_size_near_the_int32_limit(lib):
    """The chunk plan is computed in 64 bits: up to the largest allowed
    max_seqlen (2^30) the workspace grows with the sequence and never wraps;
    beyond it the size query returns 0 and the entry points refuse the call."""
    sizes = [lib.gptoss_attn_decode_workspace_size(1, 64, 8, 64, L, 0)
             for L in (1 << 16, 1 << 20, 1 << 26, (1 << 30) - 63, 1 << 30)]
    assert all(x > 0 for x in sizes) and sizes == sorted(sizes), sizes
    for L in ((1 << 30) + 1, 2 ** 31 - 64, 2 ** 31 - 63, 2 ** 31 - 1):
        assert lib.gptoss_attn_decode_workspace_size(1, 64, 8, 64, L, 0) == 0
        assert _dec(lib, N=1, max_seqlen=L, ws_bytes=1 << 40) == 1
        assert "exceeds 2^30" in lib.gptoss_attn_last_error().decode()
    # a window bounds the visible keys whatever max_seqlen says
    assert lib.gptoss_attn_decode_workspace_size(1, 64, 8, 64, 1 << 30, 128) == \
        lib.gptoss_attn_decode_workspace_size(1, 64, 8, 64, 128, 128)


def test_error_message_cleared_on_success(lib):
    _fwd(lib, q=None)
    assert lib.gptoss_attn_last_error().decode() != ""
    assert _fwd(lib, B=0) == 0
    assert lib.gptoss_attn_last_error().decode() == ""


def _paged(lib, **kw):
    a = dict(q=P, kp=P, vp=P, bt=P, lens=P, sinks=P, N=2, Hq=64, Hkv=8, D=64, page_size=16, pps=64, ring=0,
             max_seqlen=1024, window=0, scale=0.125, out=P, lse=P, ws=P, ws_bytes=None)
    a.update(kw)
    need = lib.gptoss_attn_decode_workspace_size(a["N"], a["Hq"], a["Hkv"], a["D"], a["max_seqlen"], a["window"])
    wb = need if a["ws_bytes"] is None else a["ws_bytes"]
    return lib.gptoss_attn_decode_paged(a["q"], a["kp"], a["vp"], a["bt"], a["lens"], a["sinks"], a["N"], a["Hq"],
                                        a["Hkv"], a["D"], a["page_size"], a["pps"], a["ring"], a["max_seqlen"],
                                        a["window"], a["scale"], a["out"], a["lse"], a["ws"], wb, None)


@pytest.mark.parametrize("kw,frag", [
    (dict(bt=None), "block_table is NULL"),
    (dict(lens=None), "seq_lens is NULL"),
    (dict(page_size=24), "power of two"),
    (dict(page_size=0), "power of two"),
    (dict(pps=0), "pages_per_seq"),
    (dict(max_seqlen=1025), "linear cache"),
    (dict(ring=128, window=0), "window"),
    (dict(ring=128, window=129), "window"),
    (dict(ring=96, window=64), "power of two"),
    (dict(ring=8, window=8), "multiple of page_size"),
    (dict(ring=2048, window=128), "pages"),
    (dict(ring=-1), "ring_tokens"),
    (dict(kp=P + 2), "aligned"),
])
def test_paged_decode_rejects_bad_arguments(lib, kw, frag):
    assert _paged(lib, **kw) == 1
    assert frag in lib.gptoss_attn_last_error().decode()


def test_paged_decode_zero_sequences_is_a_noop(lib):
    assert _paged(lib, N=0, q=None, kp=None, vp=None, bt=None, lens=None, out=None, lse=None, ws=None) == 0


def test_autograd_wrapper_refuses_host_tensors():
    import torch
    from attention_attn_fwd_amd.autograd import sink_attention
    q = torch.zeros(1, 4, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="HIP device"):
        sink_attention(q, k, k, torch.zeros(8), 0)


def _fwd_varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, cu=P, sinks=P, N=3, T=1000, Hq=64, Hkv=8, D=64, max_seqlen=512, window=0,
             scale=0.125, out=P, lse=P)
    a.update(kw)
    return lib.gptoss_attn_fwd_varlen(a["q"], a["k"], a["v"], a["cu"], a["sinks"], a["N"], a["T"], a["Hq"],
                                      a["Hkv"], a["D"], a["max_seqlen"], a["window"], a["scale"], a["out"],
                                      a["lse"], None)


def _bwd_varlen(lib, **kw):
    a = dict(q=P, k=P, v=P, cu=P, sinks=P, out=P, lse=P, dout=P, N=3, T=1000, Hq=64, Hkv=8, D=64,
             max_seqlen=512, window=0, scale=0.125, dq=P, dk=P, dv=P, dsinks=P, ws=P, ws_bytes=None)
    a.update(kw)
    need = lib.gptoss_attn_bwd_varlen_workspace_size(a["T"], a["Hq"], a["Hkv"], a["D"])
    wb = need if a["ws_bytes"] is None else a["ws_bytes"]
    return lib.gptoss_attn_bwd_varlen(a["q"], a["k"], a["v"], a["cu"], a["sinks"], a["out"], a["lse"], a["dout"],
                                      a["N"], a["T"], a["Hq"], a["Hkv"], a["D"], a["max_seqlen"], a["window"],
                                      a["scale"], a["dq"], a["dk"], a["dv"], a["dsinks"], a["ws"], wb, None)


VARLEN_BAD = [
    (dict(cu=None), "cu_seqlens is NULL"),
    (dict(q=None), "q is NULL"),
    (dict(N=-1), "must be >= 0"),
    (dict(T=-5), "must be >= 0"),
    (dict(max_seqlen=0), "max_seqlen"),
    (dict(N=65536), "exceeds"),
    (dict(T=2 ** 31 - 1), "exceeds 2^31 - 2^16"),
    (dict(Hq=64, Hkv=6), "multiple"),
    (dict(window=-1), "window"),
    (dict(scale=math.nan), "softmax_scale"),
    (dict(k=P + 8), "aligned"),
]


@pytest.mark.parametrize("kw,frag", VARLEN_BAD)
def test_fwd_varlen_rejects_bad_arguments(lib, kw, frag):
    assert _fwd_varlen(lib, **kw) == 1
    assert frag in lib.gptoss_attn_last_error().decode()
    assert _fwd_varlen(lib, D=128) == 2


@pytest.mark.parametrize("kw,frag", VARLEN_BAD + [
    (dict(dq=None), "dq is NULL"),
    (dict(dsinks=None), "dsinks is NULL"),
    (dict(ws_bytes=16), "workspace"),
    (dict(ws=P + 16), "aligned"),
])
def test_bwd_varlen_rejects_bad_arguments(lib, kw, frag):
    assert _bwd_varlen(lib, **kw) == 1
    assert frag in lib.gptoss_attn_last_error().decode()


def test_varlen_zero_sized_problems_are_noops(lib):
    nulls = dict(q=None, k=None, v=None, cu=None, sinks=None, out=None, lse=None)
    assert _fwd_varlen(lib, N=0, **nulls) == 0
    assert _fwd_varlen(lib, T=0, **nulls) == 0
    assert _bwd_varlen(lib, N=0, dout=None, dq=None, dk=None, dv=None, dsinks=None, ws=None, **nulls) == 0


def test_varlen_workspace_size(lib):
    # one {lse, Dvec} pair and one dsink term per (row, head), like the dense backward
    assert lib.gptoss_attn_bwd_varlen_workspace_size(16384, 64, 8, 64) == \
        lib.gptoss_attn_bwd_workspace_size(4, 4096, 64, 8, 64, 0)
    assert lib.gptoss_attn_bwd_varlen_workspace_size(0, 64, 8, 64) == 0
    assert lib.gptoss_attn_bwd_varlen_workspace_size(100, 64, 7, 64) == 0


def _table(lib, **kw):
    a = dict(t=P, P=4096, D=64, base=150000.0, factor=32.0, ctx=4096.0, alpha=1.0, beta=32.0)
    a.update(kw)
    return lib.gptoss_attn_rope_table(a["t"], a["P"], a["D"], a["base"], a["factor"], a["ctx"], a["alpha"],
                                      a["beta"], None)


@pytest.mark.parametrize("kw,status,frag", [
    (dict(t=None), 1, "table is NULL"),
    (dict(t=P + 4), 1, "aligned"),
    (dict(P=0), 1, "positions"),
    (dict(D=128), 2, "head_dim"),
    (dict(base=1.0), 1, "base"),
    (dict(base=math.nan), 1, "base"),
    (dict(factor=0.5), 1, "factor"),
    (dict(ctx=0.0), 1, "original context"),
    (dict(alpha=32.0, beta=32.0), 1, "alpha < beta"),
    (dict(beta=math.inf), 1, "alpha < beta"),
])
def test_rope_table_rejects_bad_arguments(lib, kw, status, frag):
    assert _table(lib, **kw) == status
    assert frag in lib.gptoss_attn_last_error().decode()


def test_rope_rows_and_fused_entry_points_reject_bad_arguments(lib):
    assert lib.gptoss_attn_rope_rows(P, P, None, 4, 8, 64, P, 16, 0, None) == 1
    assert "positions is NULL" in lib.gptoss_attn_last_error().decode()
    assert lib.gptoss_attn_rope_rows(P, P, P, 4, 8, 64, P, 0, 0, None) == 1
    assert lib.gptoss_attn_rope_rows(P, P, P, 4, 8, 32, P, 16, 0, None) == 2
    assert lib.gptoss_attn_rope_rows(None, None, None, 0, 8, 64, P, 16, 1, None) == 0  # T = 0 is a no-op
    # forward: the table must cover S; k_rot is required and must not alias k
    fa = [P, P, P, P, P, 4096, 1, 4097, 64, 8, 64, 0, 0.125, P, P, P, None]
    assert lib.gptoss_attn_fwd_rope(*fa) == 1 and "rope table" in lib.gptoss_attn_last_error().decode()
    fa[7] = 4096
    fa[15] = None
    assert lib.gptoss_attn_fwd_rope(*fa) == 1 and "k_rot is NULL" in lib.gptoss_attn_last_error().decode()
    fa[15] = P
    assert lib.gptoss_attn_fwd_rope(*fa) == 1 and "alias" in lib.gptoss_attn_last_error().decode()
    fa[4] = None
    fa[15] = P + 256
    assert lib.gptoss_attn_fwd_rope(*fa) == 1 and "table is NULL" in lib.gptoss_attn_last_error().decode()
    # decode: the table must cover max_seqlen
    da = [P, P, P, P, P, P, 1000, 2, 64, 8, 64, 1024, 0, 0.125, P, P, P, 1 << 30, None]
    assert lib.gptoss_attn_decode_rope(*da) == 1 and "rope table" in lib.gptoss_attn_last_error().decode()
    da[5] = None
    da[6] = 1024
    assert lib.gptoss_attn_decode_rope(*da) == 1 and "table is NULL" in lib.gptoss_attn_last_error().decode()


def test_bwd_rope_rejects_bad_arguments(lib):
    need = lib.gptoss_attn_bwd_rope_workspace_size(1, 256, 8, 1, 64)
    assert need >= 256 * 8 * 64 * 2
    args = [P, P, P, P, P, 256, P, P, P, 1, 256, 8, 1, 64, 0, 0.125, P, P, P, P, P, need, None]
    assert lib.gptoss_attn_bwd_rope(*args) != 1 or "workspace" not in lib.gptoss_attn_last_error().decode()
    bad = list(args)
    bad[5] = 255  # the table must cover S
    assert lib.gptoss_attn_bwd_rope(*bad) == 1 and "rope table" in lib.gptoss_attn_last_error().decode()
    bad = list(args)
    bad[21] = need - 1
    assert lib.gptoss_attn_bwd_rope(*bad) == 1 and "workspace" in lib.gptoss_attn_last_error().decode()
    bad = list(args)
    bad[4] = None
    assert lib.gptoss_attn_bwd_rope(*bad) == 1 and "table is NULL" in lib.gptoss_attn_last_error().decode()
    assert lib.gptoss_attn_bwd_rope(*([None] * 5), 1, *([None] * 3), 0, 4, 8, 1, 64, 0, 0.125,
                                    *([None] * 5), 0, None) == 0


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: a library that is not built is an error, not a silent
    path through something else."""
    from attention_attn_fwd_amd import _lib
    with pytest.raises(RuntimeError, match="is not built"):
        _lib.load(str(tmp_path / "libgptoss_attn.so"))


def test_decode_noalloc_refuses_plans_beyond_its_scratch(lib):
    """The no-allocation decode holds 4 MiB of split partials per GPU; a call
    whose plan needs more is refused on the host, before any HIP call."""
    N, Hq, Hkv, L = 129, 128, 4, 1024
    need = lib.gptoss_attn_decode_workspace_size(N, Hq, Hkv, 64, L, 0)
    assert need > 4 << 20
    st = lib.gptoss_attn_decode_noalloc(P, P, P, P, P, N, Hq, Hkv, 64, L, 0, 0.125, P, P, None)
    assert st == 1 and "no-allocation" in lib.gptoss_attn_last_error().decode()
    # the same argument checks as gptoss_attn_decode
    st = lib.gptoss_attn_decode_noalloc(P, P, P, None, P, 2, 64, 8, 64, 1024, 0, 0.125, P, P, None)
    assert st == 1 and "cu_seqlens is NULL" in lib.gptoss_attn_last_error().decode()
    st = lib.gptoss_attn_decode_noalloc(P, P, P, P, P, 2, 64, 8, 64, 2 ** 31 - 1, 0, 0.125, P, P, None)
    assert st == 1 and "exceeds 2^30" in lib.gptoss_attn_last_error().decode()
    assert lib.gptoss_attn_decode_noalloc(None, None, None, None, None, 0, 64, 8, 64, 1, 0, 0.125, None, None,
                                          None) == 0
