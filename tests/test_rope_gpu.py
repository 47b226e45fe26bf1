"""RoPE with YaRN scaling fused into prefill and decode, against the oracle
(GPU), through the C ABI: the table kernel, the row rotation, the forward
with rotated q and k (and its rotated-key output), the decode with the
query rotated at its position."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import apply_rope_bf16, ref_bwd_rope, ref_decode_rope, ref_fwd_rope, rope_table

from _util import check_out_lse, f64, need_gpu, seed_of

pytestmark = pytest.mark.gpu

GPTOSS_LIKE = dict(base=150000.0, factor=32.0, orig_ctx=4096.0, alpha=1.0, beta=32.0)
PLAIN = dict(base=10000.0, factor=1.0, orig_ctx=1.0, alpha=1.0, beta=32.0)
OTHER = dict(base=500000.0, factor=8.0, orig_ctx=8192.0, alpha=2.0, beta=16.0)


def _oracle_table(P, params):
    c, s = rope_table(P, 64, params["base"], params["factor"], params["orig_ctx"], params["alpha"],
                      params["beta"])
    return c, s


def _as_device_table(c, s, dev):
    return torch.from_numpy(np.stack([c, s], axis=-1).astype(np.float32)).to(dev).contiguous()


def _bf16_ulp(x):
    return np.exp2(np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126))) - 7)


@pytest.mark.parametrize("params", [GPTOSS_LIKE, PLAIN, OTHER], ids=["yarn32", "plain", "yarn8"])
def test_table_matches_oracle(params):
    dev = need_gpu()
    P = 70000
    tab = attn.rope_table(P, **params)
    torch.cuda.synchronize()
    c, s = _oracle_table(P, params)
    t = tab.cpu().numpy()
    # within one fp32 ulp, or 1e-10 absolute where cos or sin is near a zero
    # crossing: both sides evaluate p h_i in fp64, whose last-bit differences
    # (pow, argument reduction) move the angle by ~1e-11 at p ~ 7e4
    for got, ref in ((t[..., 0], c), (t[..., 1], s)):
        ulp = np.maximum(np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64), 1e-10)
        d = np.abs(got.astype(np.float64) - ref.astype(np.float64))
        assert (d <= ulp).all(), d.max()
        assert (got == ref).mean() > 0.999


def test_rows_bitwise_with_the_oracle_table():
    """Given the oracle's fp32 table, the kernel's rotation is the same fp32
    operations and bf16 rounding as the oracle's: bit-identical."""
    dev = need_gpu()
    rng = np.random.default_rng(1)
    P, T, H = 5000, 700, 8
    c, s = _oracle_table(P, GPTOSS_LIKE)
    x = synth.make_dout((T, H, 64), seed=5)
    pos = rng.integers(0, P, T).astype(np.int32)
    y = attn.rope_rows(x.to(dev), torch.from_numpy(pos).to(dev), _as_device_table(c, s, dev))
    torch.cuda.synchronize()
    ref = apply_rope_bf16(f64(x), pos, c, s)
    np.testing.assert_array_equal(f64(y), ref)
    # in place
    xd = x.to(dev)
    attn.rope_rows(xd, torch.from_numpy(pos).to(dev), _as_device_table(c, s, dev), out=xd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(xd), ref)


SMALL = [(1, 200, 8, 1), (2, 333, 16, 2), (1, 130, 6, 2), (1, 77, 1, 1)]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dS%dH%dx%d" % s)
@pytest.mark.parametrize("window", [0, 128])
@pytest.mark.parametrize("params", [GPTOSS_LIKE, OTHER], ids=["yarn32", "yarn8"])
def test_fwd_rope_small(shape, window, params):
    dev = need_gpu()
    B, S, Hq, Hkv = shape
    case = synth.make_prefill(B, S, Hq, Hkv, seed=seed_of(shape, window, "rope"))
    print(f"fwd_rope shape={shape} W={window} params={params}", flush=True)
    tab = attn.rope_table(max(S, 64), **params)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse, k_rot = attn.fwd_rope(q, k, v, sk, tab, window, case.scale)
    torch.cuda.synchronize()
    c, s = _oracle_table(max(S, 64), params)
    ro, rl, rk = ref_fwd_rope(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), window, case.scale, c, s)
    check_out_lse(f64(out), f64(lse), ro, rl, f"fwd_rope {shape} W={window}")
    d = np.abs(f64(k_rot) - rk)
    assert (d <= _bf16_ulp(rk)).all() and (d == 0).mean() > 0.999


def test_fwd_rope_identity_table_is_fwd():
    dev = need_gpu()
    case = synth.make_prefill(2, 300, 16, 2, seed=11)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    ident = torch.zeros((300, 32, 2), dtype=torch.float32, device=dev)
    ident[..., 0] = 1.0
    for w in (0, 128):
        out, lse, k_rot = attn.fwd_rope(q, k, v, sk, ident, w, case.scale)
        o2, l2 = attn.fwd(q, k, v, sk, w, case.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, o2) and torch.equal(lse, l2) and torch.equal(k_rot, k)


@pytest.mark.parametrize("window", [128, 0])
def test_fwd_rope_workload_sampled_rows(window):
    """B=4, S=4096, 64q/8kv with a YaRN table (factor 32 over a 4096-token
    original context), in the launch configuration bench.py times; every
    rotated key and a sample of output rows against the oracle."""
    dev = need_gpu()
    case = synth.config_inputs("c1_b4_s4096_h64x8")
    print(f"fwd_rope workload W={window}", flush=True)
    B, S, Hq, _ = case.q.shape
    tab = attn.rope_table(S, **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse, k_rot = attn.fwd_rope(q, k, v, sk, tab, window, case.scale)
    torch.cuda.synchronize()
    c, s = _oracle_table(S, GPTOSS_LIKE)
    rng = np.random.default_rng(S + window)
    rows = np.array(sorted(set(range(0, 8)) | {127, 128, 2047, 4095} | set(rng.integers(0, S, 12).tolist())))
    ro, rl, rk = ref_fwd_rope(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), window, case.scale, c, s,
                              rows=rows, heads=list(range(0, Hq, 4)))
    ri = torch.from_numpy(rows).to(dev)
    check_out_lse(f64(out[:, ri]), f64(lse[:, :, ri]), ro[:, rows], rl[:, :, rows], f"fwd_rope C1 W={window}")
    d = np.abs(f64(k_rot) - rk)
    assert (d <= _bf16_ulp(rk)).all()


@pytest.mark.parametrize("window", [0, 128])
def test_decode_rope(window):
    """The 128-sequence decode workload with the query rotated at L - 1; the
    cache holds keys rotated by the oracle (positions 0 .. L - 1)."""
    dev = need_gpu()
    dec = synth.config_inputs("c4_decode_n128_l1024_h64x8")
    cu = dec.cu_seqlens.numpy()
    c, s = _oracle_table(1024, GPTOSS_LIKE)
    pos = np.concatenate([np.arange(int(cu[i + 1] - cu[i])) for i in range(len(cu) - 1)]).astype(np.int64)
    kr = apply_rope_bf16(f64(dec.k_cache), pos, c, s)
    kr_t = torch.from_numpy(kr).to(torch.bfloat16)
    tab = attn.rope_table(1024, **GPTOSS_LIKE)
    print(f"decode_rope W={window}", flush=True)
    out, lse = attn.decode_rope(dec.q.to(dev), kr_t.to(dev), dec.v_cache.to(dev), dec.cu_seqlens.to(dev),
                                dec.sinks.to(dev), tab, dec.max_seqlen, window, dec.scale)
    torch.cuda.synchronize()
    ro, rl = ref_decode_rope(f64(dec.q), kr, f64(dec.v_cache), cu, f64(dec.sinks), window, dec.scale, c, s)
    check_out_lse(f64(out), f64(lse), ro, rl, f"decode_rope W={window}")


def test_prefill_cache_then_decode_rope_matches_prefill_row():
    """A decoder's loop on the GPU alone: prefill a sequence with fwd_rope,
    append the next token's key with rope_rows at its position, decode that
    token with decode_rope; the result equals row L - 1 of a prefill over
    all L tokens (same rotated keys, same query rotation)."""
    dev = need_gpu()
    L = 301
    case = synth.make_prefill(1, L, 8, 1, seed=13)
    tab = attn.rope_table(L, **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out_full, lse_full, krot_full = attn.fwd_rope(q, k, v, sk, tab, 0, case.scale)
    _, _, krot = attn.fwd_rope(q[:, :L - 1].contiguous(), k[:, :L - 1].contiguous(), v[:, :L - 1].contiguous(),
                               sk, tab, 0, case.scale)
    new_key = attn.rope_rows(k[0, L - 1:L].contiguous(), torch.tensor([L - 1], dtype=torch.int32, device=dev), tab)
    cache = torch.cat([krot[0], new_key], 0).contiguous()
    torch.cuda.synchronize()
    assert torch.equal(cache, krot_full[0])
    cu = torch.tensor([0, L], dtype=torch.int32, device=dev)
    o, l = attn.decode_rope(q[0, L - 1:L].contiguous(), cache, v[0].contiguous(), cu, sk, tab, L, 0, case.scale)
    torch.cuda.synchronize()
    assert (o.float() - out_full[0, L - 1].float()).abs().max().item() <= 1e-2
    assert (l[0] - lse_full[0, :, L - 1]).abs().max().item() <= 1e-4


def _rel_errs(grads, ref, heads=None, kv_heads=None):
    from _util import rel_l2
    dq, dk, dv, ds = (f64(t) for t in grads)
    rdq, rdk, rdv, rds = ref
    if heads is not None:
        dq, rdq, ds, rds = dq[:, :, heads], rdq[:, :, heads], ds[heads], rds[heads]
        dk, rdk, dv, rdv = dk[:, :, kv_heads], rdk[:, :, kv_heads], dv[:, :, kv_heads], rdv[:, :, kv_heads]
    return {n: rel_l2(a, r) for n, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv), ("dsinks", ds, rds))}


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dS%dH%dx%d" % s)
@pytest.mark.parametrize("window", [0, 128])
def test_bwd_rope_small(shape, window):
    """Gradients with respect to the unrotated q and k through the fused
    rotation (q rotated in the backward's pre-pass, dq and dk carried back by
    the adjoint rotation)."""
    from _util import GRAD_REL_L2
    dev = need_gpu()
    B, S, Hq, Hkv = shape
    case = synth.make_prefill(B, S, Hq, Hkv, seed=seed_of(shape, window, "bwd_rope"))
    dout = synth.make_dout(tuple(case.q.shape), seed=seed_of("dout", shape, window))
    print(f"bwd_rope shape={shape} W={window}", flush=True)
    tab = attn.rope_table(max(S, 64), **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse, k_rot = attn.fwd_rope(q, k, v, sk, tab, window, case.scale)
    grads = attn.bwd_rope(q, k_rot, v, sk, tab, out, lse, dout.to(dev), window, case.scale)
    torch.cuda.synchronize()
    c, s = _oracle_table(max(S, 64), GPTOSS_LIKE)
    ref = ref_bwd_rope(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout), window, case.scale, c, s)
    errs = _rel_errs(grads, ref)
    print(errs, flush=True)
    assert all(e <= GRAD_REL_L2 for e in errs.values()), errs


@pytest.mark.parametrize("window", [128, 0])
def test_bwd_rope_workload_group(window):
    """The training shape (B=4, S=4096, 64q/8kv) with the YaRN table, in the
    configuration bench.py times; every gradient of KV group 0 (query heads
    0..7, all batches) against the oracle."""
    from _util import GRAD_REL_L2
    dev = need_gpu()
    case, dout = synth.config_inputs("c3_bwd_b4_s4096_h64x8")
    print(f"bwd_rope workload W={window}", flush=True)
    S = case.q.shape[1]
    tab = attn.rope_table(S, **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse, k_rot = attn.fwd_rope(q, k, v, sk, tab, window, case.scale)
    grads = attn.bwd_rope(q, k_rot, v, sk, tab, out, lse, dout.to(dev), window, case.scale)
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t.float()).all()
    c, s = _oracle_table(S, GPTOSS_LIKE)
    heads = list(range(8))
    ref = ref_bwd_rope(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout), window, case.scale, c, s,
                       heads=heads)
    errs = _rel_errs(grads, ref, heads=heads, kv_heads=[0])
    print(errs, flush=True)
    assert all(e <= GRAD_REL_L2 for e in errs.values()), errs


def test_autograd_rope_matches_entry_points():
    """sink_attention_rope through torch autograd gives the fused forward's
    output and the fused backward's gradients, bit for bit."""
    from attention_attn_fwd_amd.autograd import sink_attention_rope
    dev = need_gpu()
    case = synth.make_prefill(2, 257, 16, 2, seed=51)
    dout = synth.make_dout(tuple(case.q.shape), seed=52).to(dev)
    tab = attn.rope_table(257, **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    leaves = [t.detach().clone().requires_grad_(True) for t in (q, k, v, sk)]
    out = sink_attention_rope(*leaves, tab, 128, case.scale)
    out.backward(dout)
    o2, l2, k_rot = attn.fwd_rope(q, k, v, sk, tab, 128, case.scale)
    g2 = attn.bwd_rope(q, k_rot, v, sk, tab, o2, l2, dout, 128, case.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, o2)
    for leaf, g in zip(leaves, g2):
        assert torch.equal(leaf.grad, g)
