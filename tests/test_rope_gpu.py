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

from _util import check_grads_by_group, check_out_lse, f64, nan_grads, nan_like, need_gpu, oracle_map, seed_of

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


def test_rows_match_the_oracle():
    """Rotated rows equal the oracle's bf16 rotation (the exact value rounded
    once) bit for bit; the same in place; and the adjoint rows (transpose)
    equal the oracle's rotation with the sines negated, which is R^T."""
    dev = need_gpu()
    rng = np.random.default_rng(1)
    P, T, H = 5000, 700, 8
    c, s = _oracle_table(P, GPTOSS_LIKE)
    x = synth.make_dout((T, H, 64), seed=5)
    pos = rng.integers(0, P, T).astype(np.int32)
    pd, tab = torch.from_numpy(pos).to(dev), _as_device_table(c, s, dev)
    y = attn.rope_rows(x.to(dev), pd, tab)
    yt = attn.rope_rows(x.to(dev), pd, tab, transpose=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(y), apply_rope_bf16(f64(x), pos, c, s))
    np.testing.assert_array_equal(f64(yt), apply_rope_bf16(f64(x), pos, c, -s))
    xd = x.to(dev)
    attn.rope_rows(xd, pd, tab, out=xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, y)


def test_rows_on_bf16_midpoints():
    """Rotations whose fp64 sum lands exactly on a bf16 midpoint although
    the exact value does not: a = +-2^e with cos = 1 + 2^-8 puts a c on the
    midpoint above a, and a sine of ~2^-62 moves the exact value off it by
    far less than an fp64 ulp.  The exact value's side of the midpoint
    decides (the oracle's rounding), not ties-to-even; both the rotation and
    its adjoint, bit for bit."""
    dev = need_gpu()
    rng = np.random.default_rng(11)
    P, T, H = 64, 512, 4
    c = np.full((P, 32), 1.0 + 2.0 ** -8, dtype=np.float32)
    s = (rng.choice([-1.0, 1.0], (P, 32)) * 2.0 ** -62 * rng.integers(1, 9, (P, 32))).astype(np.float32)
    a = rng.choice([-1.0, 1.0], (T, H, 32)) * np.exp2(rng.integers(-6, 7, (T, H, 32)))
    b = f64(synth.make_dout((T, H, 32), seed=6))
    x = torch.from_numpy(np.concatenate([a, b], axis=-1)).to(torch.bfloat16)
    pos = rng.integers(0, P, T).astype(np.int32)
    pd, tab = torch.from_numpy(pos).to(dev), _as_device_table(c, s, dev)
    y = attn.rope_rows(x.to(dev), pd, tab)
    yt = attn.rope_rows(x.to(dev), pd, tab, transpose=True)
    torch.cuda.synchronize()
    want = apply_rope_bf16(f64(x), pos, c, s)
    # the case is real: ties-to-even on the fp64 sum would round every a c - b s down to |a|
    assert (np.abs(want[..., :32]) > np.abs(a)).mean() > 0.3
    np.testing.assert_array_equal(f64(y), want)
    np.testing.assert_array_equal(f64(yt), apply_rope_bf16(f64(x), pos, c, -s))


def _midpoint_case(B, S, Hq, Hkv, seed):
    """q and k whose first-half elements are +-2^e (e in -3..0) and a table
    with cos = 1 + 2^-8 and sines of ~2^-62: most rotated first-half
    elements have an fp64 sum exactly on a bf16 midpoint."""
    rng = np.random.default_rng(seed)
    case = synth.make_prefill(B, S, Hq, Hkv, seed=seed)
    def pow2_half(t):
        x = f64(t)
        x[..., :32] = rng.choice([-1.0, 1.0], x[..., :32].shape) * np.exp2(rng.integers(-3, 1, x[..., :32].shape))
        return torch.from_numpy(x).to(torch.bfloat16)
    c = np.full((S, 32), 1.0 + 2.0 ** -8, dtype=np.float32)
    s = (rng.choice([-1.0, 1.0], (S, 32)) * 2.0 ** -62 * rng.integers(1, 9, (S, 32))).astype(np.float32)
    return pow2_half(case.q), pow2_half(case.k), case.v, case.sinks, case.scale, c, s


@pytest.mark.parametrize("window", [0, 128])
def test_fused_rotations_on_bf16_midpoints(window):
    """The fused rotations of q (forward, decode, backward) take their exact
    path when an fp64 sum lands on a bf16 midpoint: the backward's rotated q
    (the first part of its workspace) equals the oracle's bit for bit, and
    the forward and decode results match the oracle over the same rotation."""
    dev = need_gpu()
    B, S, Hq, Hkv = 1, 200, 8, 1
    q, k, v, sk, scale, c, s = _midpoint_case(B, S, Hq, Hkv, seed=17 + window)
    tab = _as_device_table(c, s, dev)
    qd, kd, vd, skd = (t.to(dev) for t in (q, k, v, sk))
    out, lse, k_rot = attn.fwd_rope(qd, kd, vd, skd, tab, window, scale)
    dout = synth.make_dout(tuple(q.shape), seed=23)
    ws = torch.empty(attn.bwd_rope_workspace_size(B, S, Hq, Hkv), dtype=torch.uint8, device=dev)
    attn.bwd_rope(qd, k_rot, vd, skd, tab, out, lse, dout.to(dev), window, scale, workspace=ws)
    torch.cuda.synchronize()
    ro, rl, rk = ref_fwd_rope(f64(q), f64(k), f64(v), f64(sk), window, scale, c, s)
    ra, _, _ = ref_fwd_rope(f64(q), f64(k), np.abs(f64(v)), f64(sk), window, scale, c, s)
    np.testing.assert_array_equal(f64(k_rot), rk)
    check_out_lse(f64(out), f64(lse), ro, rl, f"fwd_rope on midpoints W={window}", ref_abs=ra)
    q_rot = ws[:B * S * Hq * 64 * 2].view(torch.bfloat16).view(B, S, Hq, 64)
    want = apply_rope_bf16(f64(q[0]), np.arange(S), c, s)
    assert (np.abs(want[..., :32]) > np.abs(f64(q[0])[..., :32])).mean() > 0.3  # the midpoints are there
    np.testing.assert_array_equal(f64(q_rot[0]), want)
    # decode of the last row, the query rotated at S - 1 in the decode kernel
    cu = torch.tensor([0, S], dtype=torch.int32)
    do_, dl = attn.decode_rope(qd[0, S - 1:S].contiguous(), k_rot[0].contiguous(), vd[0].contiguous(), cu.to(dev), skd,
                               tab, S, window, scale)
    torch.cuda.synchronize()
    rdo, rdl = ref_decode_rope(f64(q[0, S - 1:S]), rk[0], f64(v[0]), cu.numpy(), f64(sk), window, scale, c, s)
    rda, _ = ref_decode_rope(f64(q[0, S - 1:S]), rk[0], np.abs(f64(v[0])), cu.numpy(), f64(sk), window, scale, c, s)
    check_out_lse(f64(do_), f64(dl), rdo, rdl, f"decode_rope on midpoints W={window}", ref_abs=rda)


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
    # sum_j P |v_j|: the oracle's forward of |v| (the rotation leaves v alone)
    ra, _, _ = ref_fwd_rope(f64(case.q), f64(case.k), np.abs(f64(case.v)), f64(case.sinks), window, case.scale, c, s)
    check_out_lse(f64(out), f64(lse), ro, rl, f"fwd_rope {shape} W={window}", ref_abs=ra)
    np.testing.assert_array_equal(f64(k_rot), rk)


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
def test_fwd_rope_workload_whole(window):
    """B=4, S=4096, 64q/8kv with a YaRN table (factor 32 over a 4096-token
    original context), in the launch configuration bench.py times: every
    rotated key, output and lse element against the oracle (per batch and KV
    group on the host's cores), into NaN-filled buffers."""
    dev = need_gpu()
    case = synth.config_inputs("prefill_b4_s4096_h64x8")
    print(f"fwd_rope workload W={window}", flush=True)
    B, S, Hq, D = case.q.shape
    Hkv = case.k.shape[2]
    G = Hq // Hkv
    tab = attn.rope_table(S, **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out = nan_like((B, S, Hq, D), torch.bfloat16, dev)
    lse = nan_like((B, Hq, S), torch.float32, dev)
    k_rot = nan_like((B, S, Hkv, D), torch.bfloat16, dev)
    attn.fwd_rope(q, k, v, sk, tab, window, case.scale, out=out, lse=lse, k_rot=k_rot)
    torch.cuda.synchronize()
    for t in (out, lse, k_rot):
        assert torch.isfinite(t.float()).all()
    c, s = _oracle_table(S, GPTOSS_LIKE)
    qo, ko, vo, so = f64(case.q), f64(case.k), f64(case.v), f64(case.sinks)
    tasks = [(b, g) for b in range(B) for g in range(Hkv)]

    def one(t):
        b, g = t
        hs = slice(g * G, (g + 1) * G)
        args = (qo[b:b + 1, :, hs], ko[b:b + 1, :, g:g + 1])
        o, l, kr = ref_fwd_rope(*args, vo[b:b + 1, :, g:g + 1], so[hs], window, case.scale, c, s)
        # sum_j P |v_j| (the rotation leaves v alone): what rounding P to bf16 can cost
        oa, _, _ = ref_fwd_rope(*args, np.abs(vo[b:b + 1, :, g:g + 1]), so[hs], window, case.scale, c, s)
        return o, l, kr, oa

    ro, rl, rk = np.zeros((B, S, Hq, D)), np.zeros((B, Hq, S)), np.zeros((B, S, Hkv, D))
    ra = np.zeros((B, S, Hq, D))
    for (b, g), (o, l, kr, oa) in zip(tasks, oracle_map(one, tasks)):
        hs = slice(g * G, (g + 1) * G)
        ro[b, :, hs], rl[b, hs], rk[b, :, g], ra[b, :, hs] = o[0], l[0], kr[0, :, 0], oa[0]
    check_out_lse(f64(out), f64(lse), ro, rl, f"fwd_rope B4 S4096 W={window}", ref_abs=ra)
    np.testing.assert_array_equal(f64(k_rot), rk)


@pytest.mark.parametrize("window", [0, 128])
def test_decode_rope(window):
    """The 128-sequence decode workload with the query rotated at L - 1; the
    cache holds keys rotated by the oracle (positions 0 .. L - 1)."""
    dev = need_gpu()
    dec = synth.config_inputs("decode_n128_l1024_h64x8")
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
    ra, _ = ref_decode_rope(f64(dec.q), kr, np.abs(f64(dec.v_cache)), cu, f64(dec.sinks), window, dec.scale, c, s)
    check_out_lse(f64(out), f64(lse), ro, rl, f"decode_rope W={window}", ref_abs=ra)


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
def test_bwd_rope_workload_whole(window):
    """The training shape (B=4, S=4096, 64q/8kv) with the YaRN table, in the
    configuration bench.py times: every gradient element of all eight KV
    groups against the oracle, into NaN-filled gradient buffers."""
    dev = need_gpu()
    case, dout = synth.config_inputs("train_b4_s4096_h64x8")
    print(f"bwd_rope workload W={window}", flush=True)
    B, S, Hq, D = case.q.shape
    Hkv = case.k.shape[2]
    G = Hq // Hkv
    tab = attn.rope_table(S, **GPTOSS_LIKE)
    q, k, v, sk = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse, k_rot = attn.fwd_rope(q, k, v, sk, tab, window, case.scale)
    grads = attn.bwd_rope(q, k_rot, v, sk, tab, out, lse, dout.to(dev), window, case.scale,
                          grads=nan_grads(q, k, v, Hq))
    torch.cuda.synchronize()
    for t in grads:
        assert torch.isfinite(t.float()).all()
    c, s = _oracle_table(S, GPTOSS_LIKE)
    qo, ko, vo, so, do = f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), f64(dout)
    tasks = [(b, g) for b in range(B) for g in range(Hkv)]

    def one(t):
        b, g = t
        hs = slice(g * G, (g + 1) * G)
        return ref_bwd_rope(qo[b:b + 1, :, hs], ko[b:b + 1, :, g:g + 1], vo[b:b + 1, :, g:g + 1], so[hs],
                            do[b:b + 1, :, hs], window, case.scale, c, s)

    rdq, rdk, rdv, rds = np.zeros(qo.shape), np.zeros(ko.shape), np.zeros(vo.shape), np.zeros(Hq)
    for (b, g), (gq, gk, gv, gs) in zip(tasks, oracle_map(one, tasks)):
        hs = slice(g * G, (g + 1) * G)
        rdq[b, :, hs], rdk[b, :, g], rdv[b, :, g] = gq[0], gk[0, :, 0], gv[0, :, 0]
        rds[hs] += gs
    check_grads_by_group([f64(t) for t in grads], (rdq, rdk, rdv, rds), Hkv, f"bwd_rope B4 S4096 W={window}")


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
