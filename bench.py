#!/usr/bin/env python3
"""Benchmark of the sink-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  gpt-oss layer pair at B=4, S=4096, 64 query / 8 KV heads, head_dim 64 --
  forward + backward of the sliding-window-128 layer and of the full-causal
  layer -- plus decode of both layers for 128 sequences with KV lengths
  U{1..1024}.
Inputs and outputs stay resident in HBM; the timed region holds exactly
`--steps` steps between two stream synchronisations.  Each step is one replay
of a HIP graph that holds the step's kernel launches (captured once through
the same C ABI calls), so the host's per-call argument marshalling does not
sit between the kernels; the eager (one ABI call after another) step time is
reported beside it as `ms_per_step_eager`.

value = unmasked FLOPs of the step (forward 4*D, backward 10*D per visible
(batch, query head, query, key) pair; decode 4*D per visible key and head)
divided by the step time, in TFLOP/s.  Per-part figures (TFLOP/s, GB/s and
the fraction of the bounding roof) are printed in `parts`; `parts` also times
paths outside the step: decode through a paged and a ring cache, a training
step through the autograd wrapper, and prefill of packed documents (16384
tokens in documents of U{1..4096} tokens, same heads; FLOPs over the pairs
visible inside each document), and prefill and decode with the YaRN rotary
embedding fused in (the same FLOPs; bytes add the rotated-key write; the
backward counts the plain backward's bytes), decode of one 65536-key
sequence (the long-context workload's next token), and the forward of the small (B=1, S=512, 8q/1kv) and long-context (B=1,
S=65536) workloads.
"""

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
D = 64
WINDOWS = (128, 0)             # sliding layer, full-causal layer
COPY_BYTES = 1 << 30           # calibration copy for the HBM byte counters
NSETS = 4                      # input/output buffer sets used in rotation
ROOT = os.path.dirname(os.path.abspath(__file__))


# the sources each part's kernels and launch come from (measured traffic of a
# part stays valid while these files are unchanged)
PART_SOURCES = {"fwd": ("fwd.hip", "common.h", "launch.h"),
                "bwd": ("bwd.hip", "common.h", "launch.h", "plan.cpp"),
                "decode": ("decode.hip", "decode_paged.hip", "common.h", "launch.h", "plan.cpp")}


def build_source_flags():
    """The build's per-source compiler flags (attention_attn_fwd_amd/build.py
    SOURCE_FLAGS), read without importing the package."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_gptoss_build", os.path.join(ROOT, "attention_attn_fwd_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.SOURCE_FLAGS


def source_digest(part):
    """sha256 over the library sources of `part` (fwd, bwd or decode, the
    packed-document parts as their dense kind) and the extra compiler flags
    the build gives each of them."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_attn_fwd_amd", "csrc")
    flags = build_source_flags()
    for name in PART_SOURCES[part.replace("varlen_", "")]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
        if flags.get(name):
            h.update(b"\0flags\0" + " ".join(flags[name]).encode())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch of `key` (e.g. "bwd_full") from
    profiles/traffic.json (FETCH_SIZE + WRITE_SIZE, calibrated against a
    plain copy), or None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    part = key.rsplit("_", 1)[0]
    if part.replace("varlen_", "") not in PART_SOURCES:
        return None
    if t.get("source_sha256", {}).get(part) != source_digest(part):
        return None
    v = t.get("bytes_per_launch", {}).get(key)
    return None if v is None else float(v)


def pairs_per_head(S, W):
    """Visible (query, key) pairs of one (batch, head): closed form."""
    if W == 0 or W >= S:
        return S * (S + 1) // 2
    return W * (W + 1) // 2 + (S - W) * W


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["fwd", "bwd", "decode", "varlen_fwd", "varlen_bwd", "copy"], default=None,
                    help="run only this part in a loop (for profiling); prints no JSON line.  'copy' "
                         "copies 1 GiB once per step, to calibrate HBM byte counters")
    ap.add_argument("--window", type=int, default=None, choices=list(WINDOWS),
                    help="with --only: run that part for this layer's window only")
    ap.add_argument("--digest-traffic", metavar="DIR", default=None,
                    help="write profiles/traffic.json from the rocprofv3 FETCH_SIZE / WRITE_SIZE csv runs under DIR "
                         "(DIR/<part>_<window>_<counter>/run_counter_collection.csv, one run per part, layer and "
                         "counter, plus DIR/copy_<counter>) and exit; runs no GPU code")
    ap.add_argument("--verbose", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.digest_traffic:
        digest_traffic(args.digest_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the kernels run on one GPU's share "
              "of the work (KV heads, sequences and batch rows shard across GPUs without communication)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_attn_fwd_amd as attn
    from attention_attn_fwd_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = (lambda *a: print(*a, file=sys.stderr, flush=True)) if args.verbose else (lambda *a: None)

    if args.only == "copy":
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"done: copy of {COPY_BYTES} bytes x {args.warmup + args.steps}", flush=True)
        return

    # ---- inputs (seeded, synthetic, gpt-oss shaped), resident in HBM.
    # NSETS copies of every input and output, used in rotation, so that
    # consecutive launches never find their working set in the 256 MB
    # last-level cache (MALL) that the previous launch filled.
    case, dout_cpu = synth.config_inputs("train_b4_s4096_h64x8")
    B, S, Hq, _ = case.q.shape
    Hkv = case.k.shape[2]
    sinks = case.sinks.to(dev)
    dec = synth.config_inputs("decode_n128_l1024_h64x8")
    N = dec.q.shape[0]
    dcu, dsinks_ = dec.cu_seqlens.to(dev), dec.sinks.to(dev)
    lengths = (dec.cu_seqlens[1:] - dec.cu_seqlens[:-1]).tolist()
    scale = case.scale

    sets = []
    for _ in range(NSETS):
        q, k, v, dout = case.q.to(dev), case.k.to(dev), case.v.to(dev), dout_cpu.to(dev)
        sets.append(dict(
            q=q, k=k, v=v, dout=dout,
            outs={w: (torch.empty_like(q), torch.empty(B, Hq, S, device=dev)) for w in WINDOWS},
            grads={w: (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                       torch.empty(Hq, dtype=torch.float32, device=dev)) for w in WINDOWS},
            dq=dec.q.to(dev), dk=dec.k_cache.to(dev), dv=dec.v_cache.to(dev),
            dec_out={w: (torch.empty_like(dec.q, device=dev), torch.empty(N, Hq, device=dev)) for w in WINDOWS}))
    q, k = sets[0]["q"], sets[0]["k"]
    bws = torch.empty(attn.bwd_workspace_size(B, S, Hq, Hkv, D, 0), dtype=torch.uint8, device=dev)
    dws = attn.decode_workspace(N, Hq, Hkv, dec.max_seqlen, 0, device=dev)

    def fwd(w, i=0):
        x = sets[i % NSETS]
        o, l = x["outs"][w]
        attn.fwd(x["q"], x["k"], x["v"], sinks, w, scale, out=o, lse=l)

    def bwd(w, i=0):
        x = sets[i % NSETS]
        o, l = x["outs"][w]
        attn.bwd(x["q"], x["k"], x["v"], sinks, o, l, x["dout"], w, scale, workspace=bws, grads=x["grads"][w])

    def decode(w, i=0):
        x = sets[i % NSETS]
        o, l = x["dec_out"][w]
        attn.decode(x["dq"], x["dk"], x["dv"], dcu, dsinks_, dec.max_seqlen, w, dec.scale, out=o, lse=l,
                    workspace=dws)

    def step(i=0):
        for w in WINDOWS:
            fwd(w, i)
            bwd(w, i)
        for w in WINDOWS:
            decode(w, i)

    # packed documents: 16384 tokens in documents of U{1..4096} tokens, same heads
    vcase, vdout_cpu = synth.varlen_workload()
    vT = vcase.q.shape[0]
    vcu = vcase.cu_seqlens.to(dev)
    vlens = (vcase.cu_seqlens[1:] - vcase.cu_seqlens[:-1]).tolist()
    vsets = []
    for _ in range(NSETS if not args.only or args.only.startswith("varlen") else 0):
        vq, vk, vv = vcase.q.to(dev), vcase.k.to(dev), vcase.v.to(dev)
        vsets.append(dict(q=vq, k=vk, v=vv, dout=vdout_cpu.to(dev),
                          outs={w: (torch.empty_like(vq), torch.empty(Hq, vT, device=dev)) for w in WINDOWS},
                          grads={w: (torch.empty_like(vq), torch.empty_like(vk), torch.empty_like(vv),
                                     torch.empty(Hq, dtype=torch.float32, device=dev)) for w in WINDOWS}))
    vws = torch.empty(attn.bwd_varlen_workspace_size(vT, Hq, Hkv, D), dtype=torch.uint8, device=dev)

    def varlen_fwd(w, i=0):
        x = vsets[i % NSETS]
        o, l = x["outs"][w]
        attn.fwd_varlen(x["q"], x["k"], x["v"], vcu, sinks, vcase.max_seqlen, w, vcase.scale, out=o, lse=l)

    def varlen_bwd(w, i=0):
        x = vsets[i % NSETS]
        o, l = x["outs"][w]
        attn.bwd_varlen(x["q"], x["k"], x["v"], vcu, sinks, o, l, x["dout"], vcase.max_seqlen, w, vcase.scale,
                        workspace=vws, grads=x["grads"][w])

    if args.only:
        fn = {"fwd": fwd, "bwd": bwd, "decode": decode, "varlen_fwd": varlen_fwd,
              "varlen_bwd": varlen_bwd}[args.only]
        wins = WINDOWS if args.window is None else (args.window,)
        if args.only in ("bwd", "varlen_bwd"):
            first = fwd if args.only == "bwd" else varlen_fwd
            for i in range(NSETS):
                for w in wins:
                    first(w, i)  # the backward consumes this layer's forward out/lse
        for i in range(args.warmup + args.steps):
            for w in wins:
                fn(w, i)
        torch.cuda.synchronize()
        print(f"done: {args.only} x {args.warmup + args.steps} per layer", flush=True)
        return

    # ---- work accounting
    flops = {}
    bytes_ = {}
    for w in WINDOWS:
        pairs = B * Hq * pairs_per_head(S, w)
        flops[("fwd", w)] = 4 * D * pairs
        flops[("bwd", w)] = 10 * D * pairs
        # algorithmic bytes: every input read once, every output written once
        bytes_[("fwd", w)] = 2 * (q.numel() + 2 * k.numel() + q.numel()) + 4 * B * Hq * S
        bytes_[("bwd", w)] = (2 * (4 * q.numel() + 2 * k.numel()) + 4 * B * Hq * S + 4 * Hq   # q,out,dout,dq + k,v
                              + 2 * 2 * k.numel() + 4 * Hq)                                  # dk, dv, sinks/dsinks
        vis = sum(min(L, w) if w else L for L in lengths)
        flops[("decode", w)] = 4 * D * Hq * vis
        bytes_[("decode", w)] = (2 * 2 * vis * Hkv * D + 2 * 2 * N * Hq * D + 4 * N * Hq + 4 * Hq
                                 + 4 * (N + 1))
        vpairs = Hq * sum(pairs_per_head(L, w) for L in vlens)
        flops[("varlen_fwd", w)] = 4 * D * vpairs
        flops[("varlen_bwd", w)] = 10 * D * vpairs
        vq_el, vk_el = vT * Hq * D, vT * Hkv * D
        bytes_[("varlen_fwd", w)] = 2 * (2 * vq_el + 2 * vk_el) + 4 * Hq * vT + 4 * len(vlens)
        bytes_[("varlen_bwd", w)] = 2 * (4 * vq_el + 4 * vk_el) + 4 * Hq * vT + 8 * Hq + 4 * len(vlens)

    stream = torch.cuda.current_stream(dev)

    def timed(run, n):
        """ms per call of `run` over n calls bracketed by events on `stream`."""
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(n):
            run()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / n

    # eager step (reported only): warm the library on every buffer set, then
    # one timed pass per set
    for i in range(NSETS):
        step(i)
    it = iter(range(1 << 30))
    ms_eager = timed(lambda: step(next(it)), NSETS)
    g_steps = [capture(lambda: step(i)) for i in range(NSETS)]

    # ---- warmup, then the timed region: exactly `steps` graph replays,
    # rotating over the buffer sets
    for i in range(args.warmup):
        g_steps[i % NSETS].replay()
    it = iter(range(1 << 30))
    ms_per_step = timed(lambda: g_steps[next(it) % NSETS].replay(), args.steps)
    total_flops = sum(f for (name, _), f in flops.items() if not name.startswith("varlen"))
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    g_clock = g_steps[0]  # replayed again at the very end to sample the clocks under this load
    del g_steps

    # ---- per-part launch durations: a graph of `reps` back-to-back calls of
    # one part (rotating over the buffer sets), replayed once untimed, then
    # five times timed; the median replay / reps
    def median_replay(g):
        return sorted(timed(g.replay, 1) for _ in range(5))[2]

    reps = 5 * NSETS  # 20 back-to-back calls per graph
    part_ms = {}
    for name, fn in (("fwd", fwd), ("bwd", bwd), ("decode", decode)):
        for w in WINDOWS:
            g = capture(lambda: [fn(w, i) for i in range(reps)])
            g.replay()
            part_ms[(name, w)] = median_replay(g) / reps
            del g
    # training step of one full-causal layer through the autograd wrapper
    # (forward + backward, the same kernels; timed eagerly, host marshalling
    # included)
    from attention_attn_fwd_amd.autograd import sink_attention
    leaves = [[x[n].detach().requires_grad_(True) for n in ("q", "k", "v")] for x in sets]
    sk_leaf = sinks.detach().requires_grad_(True)

    def train(i):
        qq, kk, vv = leaves[i % NSETS]
        for t in (qq, kk, vv, sk_leaf):  # as zero_grad(set_to_none=True): no accumulation kernels
            t.grad = None
        sink_attention(qq, kk, vv, sk_leaf, 0, scale).backward(sets[i % NSETS]["dout"])

    for i in range(NSETS):
        train(i)
    it = iter(range(1 << 30))
    ms_train = timed(lambda: train(next(it)), 2 * NSETS)
    del leaves

    parts = {}
    for (name, w), ms in part_ms.items():
        tf = flops[(name, w)] / (ms * 1e-3) / 1e12
        gbs = bytes_[(name, w)] / (ms * 1e-3) / 1e9
        ai = flops[(name, w)] / bytes_[(name, w)]
        roof_tf = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
        parts[f"{name}_{'full' if w == 0 else 'w%d' % w}"] = {
            "ms": round(ms, 4), "tflops": round(tf, 2), "gbs": round(gbs, 1),
            "bound": "mfma" if roof_tf >= BF16_PEAK_TFLOPS else "hbm",
            "frac_of_roof": round(tf / roof_tf, 4)}
    # decode through a paged cache (pages of 16 tokens, the full layer) and
    # through a ring cache of 128 slots (the sliding layer), same sequences
    pg = synth.make_paged_decode(N, Hq, Hkv, 16, seed=1004)
    rg = synth.make_paged_decode(N, Hq, Hkv, 16, seed=1004, ring_tokens=128)
    pg_sets = [[t.to(dev) for t in (pg.k_pages, pg.v_pages)] for _ in range(NSETS)]
    rg_sets = [[t.to(dev) for t in (rg.k_pages, rg.v_pages)] for _ in range(NSETS)]
    pg_bt, rg_bt, lens_d = pg.block_table.to(dev), rg.block_table.to(dev), pg.seq_lens.to(dev)
    for label, cs, bt, ring, w in (("decode_paged16_full", pg_sets, pg_bt, 0, 0),
                                   ("decode_ring128_w128", rg_sets, rg_bt, 128, 128)):
        def pfn(i, cs=cs, bt=bt, ring=ring, w=w):
            x = sets[i % NSETS]
            o, l = x["dec_out"][w]
            kp, vp = cs[i % NSETS]
            attn.decode_paged(x["dq"], kp, vp, bt, lens_d, dsinks_, dec.max_seqlen, w, dec.scale, ring_tokens=ring,
                              out=o, lse=l, workspace=dws)
        g = capture(lambda: [pfn(i) for i in range(reps)])
        g.replay()
        ms = median_replay(g) / reps
        del g
        gbs = bytes_[("decode", w)] / (ms * 1e-3) / 1e9
        parts[label] = {"ms": round(ms, 4), "gbs": round(gbs, 1), "bound": "hbm",
                        "frac_of_roof": round(gbs / HBM_PEAK_GBS, 4)}
    del pg_sets, rg_sets
    # decode of the long-context workload's next token: one sequence of
    # 65536 keys, 64q/8kv, both layers (the full layer's chunk plan cuts the
    # sequence into 128 chunks of 512 keys and merges their partials)
    lc = synth.make_decode(1, Hq, Hkv, lengths=[65536], seed=1005)
    lcu, lsk = lc.cu_seqlens.to(dev), lc.sinks.to(dev)
    lsets = [(lc.q.to(dev), lc.k_cache.to(dev), lc.v_cache.to(dev), torch.empty(1, Hq, D, dtype=torch.bfloat16,
              device=dev), torch.empty(1, Hq, device=dev)) for _ in range(NSETS)]
    lws = attn.decode_workspace(1, Hq, Hkv, lc.max_seqlen, 0, device=dev)
    for w in WINDOWS:
        def lfn(i, w=w):
            lq, lk, lv, lo, ll = lsets[i % NSETS]
            attn.decode(lq, lk, lv, lcu, lsk, lc.max_seqlen, w, lc.scale, out=lo, lse=ll, workspace=lws)
        g = capture(lambda: [lfn(i) for i in range(reps)])
        g.replay()
        ms = median_replay(g) / reps
        del g
        vis = min(65536, w) if w else 65536
        by = 2 * 2 * vis * Hkv * D + 2 * 2 * Hq * D + 4 * Hq + 4 * Hq + 8
        gbs = by / (ms * 1e-3) / 1e9
        parts[f"decode_one65536_{'full' if w == 0 else 'w%d' % w}"] = {
            "ms": round(ms, 4), "gbs": round(gbs, 1), "bound": "hbm", "frac_of_roof": round(gbs / HBM_PEAK_GBS, 4)}
    del lsets, lws
    # packed-document prefill (not part of the step): forward and backward
    # per layer, each timed like the parts above
    for w in WINDOWS:
        for i in range(NSETS):
            varlen_fwd(w, i)
    for name, fn in (("varlen_fwd", varlen_fwd), ("varlen_bwd", varlen_bwd)):
        for w in WINDOWS:
            g = capture(lambda: [fn(w, i) for i in range(reps)])
            g.replay()
            ms = median_replay(g) / reps
            del g
            tf = flops[(name, w)] / (ms * 1e-3) / 1e12
            gbs = bytes_[(name, w)] / (ms * 1e-3) / 1e9
            ai = flops[(name, w)] / bytes_[(name, w)]
            roof_tf = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
            parts[f"{name}_{'full' if w == 0 else 'w%d' % w}"] = {
                "ms": round(ms, 4), "tflops": round(tf, 2), "gbs": round(gbs, 1),
                "bound": "mfma" if roof_tf >= BF16_PEAK_TFLOPS else "hbm",
                "frac_of_roof": round(tf / roof_tf, 4)}
    del vsets
    # RoPE with YaRN scaling fused into the prefill (q rotated in the load
    # stage, k once into the rotated-key cache) and into decode (the query);
    # gpt-oss-like table parameters (base 150000, factor 32 over a 4096-token
    # original context, ramp 1..32)
    yarn = dict(base=150000.0, factor=32.0, orig_ctx=4096.0, alpha=1.0, beta=32.0)
    tab = attn.rope_table(max(S, dec.max_seqlen), **yarn)
    krots = [torch.empty_like(x["k"]) for x in sets]

    def fwd_rope(w, i=0):
        x = sets[i % NSETS]
        o, l = x["outs"][w]
        attn.fwd_rope(x["q"], x["k"], x["v"], sinks, tab, w, scale, out=o, lse=l, k_rot=krots[i % NSETS])

    def decode_rope(w, i=0):
        x = sets[i % NSETS]
        o, l = x["dec_out"][w]
        attn.decode_rope(x["dq"], x["dk"], x["dv"], dcu, dsinks_, tab, dec.max_seqlen, w, dec.scale, out=o, lse=l,
                         workspace=dws)

    for name, fn, base in (("fwd_rope", fwd_rope, "fwd"), ("decode_rope", decode_rope, "decode")):
        for w in WINDOWS:
            g = capture(lambda: [fn(w, i) for i in range(reps)])
            g.replay()
            ms = median_replay(g) / reps
            del g
            extra = 2 * 2 * k.numel() if base == "fwd" else 0  # k read and k_rot written by the pre-pass
            tf = flops[(base, w)] / (ms * 1e-3) / 1e12
            gbs = (bytes_[(base, w)] + extra) / (ms * 1e-3) / 1e9
            ai = flops[(base, w)] / (bytes_[(base, w)] + extra)
            roof_tf = min(BF16_PEAK_TFLOPS, ai * HBM_PEAK_GBS / 1e3)
            bound = "mfma" if roof_tf >= BF16_PEAK_TFLOPS else "hbm"
            parts[f"{name}_{'full' if w == 0 else 'w%d' % w}"] = {
                "ms": round(ms, 4), "tflops": round(tf, 2), "gbs": round(gbs, 1), "bound": bound,
                "frac_of_roof": round(tf / roof_tf if bound == "mfma" else gbs / HBM_PEAK_GBS, 4)}
    # backward with RoPE (training): out, lse and k_rot are those fwd_rope
    # left in every buffer set above; the dq kernel rotates q (and leaves it
    # in the workspace for dkdv) and the dq, dk epilogues apply the adjoint
    # rotation.  Algorithmic bytes as the plain backward (q_rot is not an
    # output; its write is overhead the fraction shows)
    rws = torch.empty(attn.bwd_rope_workspace_size(B, S, Hq, Hkv, D), dtype=torch.uint8, device=dev)

    def bwd_rope(w, i=0):
        x = sets[i % NSETS]
        o, l = x["outs"][w]
        attn.bwd_rope(x["q"], krots[i % NSETS], x["v"], sinks, tab, o, l, x["dout"], w, scale, workspace=rws,
                      grads=x["grads"][w])

    for w in WINDOWS:
        g = capture(lambda: [bwd_rope(w, i) for i in range(reps)])
        g.replay()
        ms = median_replay(g) / reps
        del g
        tf = flops[("bwd", w)] / (ms * 1e-3) / 1e12
        gbs = bytes_[("bwd", w)] / (ms * 1e-3) / 1e9
        roof_tf = min(BF16_PEAK_TFLOPS, flops[("bwd", w)] / bytes_[("bwd", w)] * HBM_PEAK_GBS / 1e3)
        parts[f"bwd_rope_{'full' if w == 0 else 'w%d' % w}"] = {
            "ms": round(ms, 4), "tflops": round(tf, 2), "gbs": round(gbs, 1),
            "bound": "mfma" if roof_tf >= BF16_PEAK_TFLOPS else "hbm", "frac_of_roof": round(tf / roof_tf, 4)}
    del krots, rws
    # the small workload (B=1, S=512, 8q/1kv) and the long-context workload
    # (B=1, S=65536, 64q/8kv, values ~ N(0, 0.5^2)): forward of both layers
    for cname, label in (("small_b1_s512_h8x1", "small"), ("long_b1_s65536_h64x8", "long")):
        cc = synth.config_inputs(cname)
        cB, cS, cHq, _ = cc.q.shape
        csets = []
        for _ in range(NSETS):
            cq = cc.q.to(dev)
            csets.append((cq, cc.k.to(dev), cc.v.to(dev), torch.empty_like(cq),
                          torch.empty(cB, cHq, cS, device=dev)))
        csk = cc.sinks.to(dev)
        for w in WINDOWS:
            def cfn(i, w=w):
                cq, ck, cv, co, cl = csets[i % NSETS]
                attn.fwd(cq, ck, cv, csk, w, cc.scale, out=co, lse=cl)
            g = capture(lambda: [cfn(i) for i in range(reps)])
            g.replay()
            ms = median_replay(g) / reps
            del g
            fl = 4 * D * cB * cHq * pairs_per_head(cS, w)
            by = 2 * (2 * cc.q.numel() + 2 * cc.k.numel()) + 4 * cB * cHq * cS
            tf = fl / (ms * 1e-3) / 1e12
            gbs = by / (ms * 1e-3) / 1e9
            roof_tf = min(BF16_PEAK_TFLOPS, fl / by * HBM_PEAK_GBS / 1e3)
            parts[f"{label}_fwd_{'full' if w == 0 else 'w%d' % w}"] = {
                "ms": round(ms, 4), "tflops": round(tf, 2), "gbs": round(gbs, 1),
                "bound": "mfma" if roof_tf >= BF16_PEAK_TFLOPS else "hbm", "frac_of_roof": round(tf / roof_tf, 4)}
        del csets
    tf_train = (flops[("fwd", 0)] + flops[("bwd", 0)]) / (ms_train * 1e-3) / 1e12
    parts["autograd_train_full"] = {"ms": round(ms_train, 4), "tflops": round(tf_train, 2), "bound": "mfma",
                                    "frac_of_roof": round(tf_train / BF16_PEAK_TFLOPS, 4)}
    log(json.dumps(parts, indent=1))

    # Dominant unit of the step: the backward entry point of the full-causal
    # layer (3 launches: dq, dkdv, dsink; dkdv is the largest).  Its
    # duration per call comes from events on the stream its kernels run on,
    # around a graph of back-to-back calls; achieved uses the algorithmic
    # 10*D FLOPs per visible pair.
    ms_b = part_ms[("bwd", 0)]
    ach = flops[("bwd", 0)] / (ms_b * 1e-3) / 1e12
    tb = measured_traffic("bwd_full")
    roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": tb,
                "kernel": "gptoss_attn_bwd, full-causal layer (bwd_dq + bwd_dkdv + bwd_dsink)",
                "ms_per_launch": round(ms_b, 4)}
    ach_f = flops[("fwd", 0)] / (part_ms[("fwd", 0)] * 1e-3) / 1e12
    roofline_fwd = {"bound": "mfma", "achieved": round(ach_f, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach_f / BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic("fwd_full"),
                    "kernel": "fwd_kernel, full-causal layer", "ms_per_launch": round(part_ms[("fwd", 0)], 4)}
    ms_d = part_ms[("decode", 0)]
    gbs_d = bytes_[("decode", 0)] / (ms_d * 1e-3) / 1e9
    roofline_decode = {"bound": "hbm", "achieved": round(gbs_d, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(gbs_d / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode_full"),
                       "kernel": "gptoss_attn_decode, full layer (split + merge)", "ms_per_launch": round(ms_d, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, dout_cpu)

    # the clocks under the step's load, after everything else was timed (so
    # that the load cannot change another measurement): sampled while about
    # 3 s of step replays keep the GPU busy
    n_load = max(1, int(3000 / ms_per_step))
    clocks = sample_clocks(lambda: ([g_clock.replay() for _ in range(n_load)], torch.cuda.synchronize()))
    del g_clock

    line = {
        "metric": "attn fwd/bwd TFLOP/s (unmasked FLOPs) + decode GB/s, % of MI355X roofline",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "ms_per_step_eager": round(ms_eager, 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "gpt-oss sink attention layer pair (sliding-128 + full causal): fwd+bwd at "
                               "B=4 S=4096 Hq=64 Hkv=8 D=64, plus decode N=128 L~U[1,1024]",
                   "global_batch": B, "seq_len": S, "parallelism": "none (1 GPU)"},
        "decode_gbs": {("full" if w == 0 else "w128"): parts["decode_" + ("full" if w == 0 else "w128")]["gbs"]
                       for w in WINDOWS},
        "parts": parts,
        "roofline": roofline,
        "roofline_fwd": roofline_fwd,
        "roofline_decode": roofline_decode,
        "cpu_baseline": cpu,
        "clocks": clocks,
    }
    print(json.dumps(line), flush=True)


PART_KERNELS = {"fwd": ("fwd_kernel",), "varlen_fwd": ("fwd_kernel",),
                "bwd": ("bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_dsink_kernel"),
                "varlen_bwd": ("bwd_dq_kernel", "bwd_dkdv_kernel", "bwd_dsink_kernel"),
                "decode": ("decode_split_kernel", "decode_merge_few_kernel", "decode_merge_kernel")}


def read_counter(path, counter):
    """{kernel: [values per dispatch]} of one rocprofv3 counter csv (KiB)."""
    import csv
    import re
    out = {}
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            m = re.search(r"(\w+_kernel)(<[^>]*>)?\(", row["Kernel_Name"])
            name = m.group(1) if m else row["Kernel_Name"]
            out.setdefault(name, []).append(float(row["Counter_Value"]))
    return out


def digest_traffic(d):
    """profiles/traffic.json from counter runs of `bench.py --only <part>
    --window <w>` (each of the part's kernels averaged over its dispatches),
    scaled by what the counters read for a plain copy of COPY_BYTES: reads
    by COPY_BYTES / FETCH_SIZE of the copy, writes by COPY_BYTES /
    WRITE_SIZE of the copy.  A part with no runs under `d` keeps its
    entries from the existing file while its sources still hash to the
    digest recorded there (its bytes were measured on the same kernels);
    otherwise it is left out."""
    def copy_kib(counter):
        v = read_counter(os.path.join(d, f"copy_{counter}", "run_counter_collection.csv"), counter)
        big = [x for vals in v.values() for x in vals if x * 1024 > COPY_BYTES / 8]
        return sum(big) / len(big)
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            old = json.load(f)
    except (OSError, ValueError):
        old = {}
    rk, wk = copy_kib("FETCH_SIZE"), copy_kib("WRITE_SIZE")
    rcal, wcal = COPY_BYTES / (rk * 1024), COPY_BYTES / (wk * 1024)
    per_launch, per_kernel, digests = {}, {}, {}
    for part, kernels in PART_KERNELS.items():
        if not any(os.path.isdir(os.path.join(d, f"{part}_{w}_{c}"))
                   for w in WINDOWS for c in ("FETCH_SIZE", "WRITE_SIZE")):
            if old.get("source_sha256", {}).get(part) == source_digest(part):
                digests[part] = old["source_sha256"][part]
                for w in WINDOWS:
                    key = f"{part}_{'full' if w == 0 else 'w%d' % w}"
                    if key in old.get("bytes_per_launch", {}):
                        per_launch[key] = old["bytes_per_launch"][key]
                    per_kernel.update({k: v for k, v in old.get("per_kernel_bytes", {}).items()
                                       if k.startswith(key + ":")})
            continue
        missing = [f"{part}_{w}_{c}" for w in WINDOWS for c in ("FETCH_SIZE", "WRITE_SIZE")
                   if not os.path.isdir(os.path.join(d, f"{part}_{w}_{c}"))]
        if missing:
            raise SystemExit(f"{d}: part {part} was measured only in part (missing runs: {', '.join(missing)})")
        digests[part] = source_digest(part)
        for w in WINDOWS:
            key = f"{part}_{'full' if w == 0 else 'w%d' % w}"
            vals = [read_counter(os.path.join(d, f"{part}_{w}_{c}", "run_counter_collection.csv"), c)
                    for c in ("FETCH_SIZE", "WRITE_SIZE")]
            total = 0.0
            for kname in kernels:
                if kname not in vals[0]:  # (the forward calls in a backward run are not the part's)
                    continue
                r = sum(vals[0][kname]) / len(vals[0][kname]) * 1024 * rcal
                wb = sum(vals[1][kname]) / len(vals[1][kname]) * 1024 * wcal
                per_kernel[f"{key}:{kname}"] = [round(r), round(wb)]
                total += r + wb
            per_launch[key] = round(total)
    out = {"source_sha256": digests,
           "read_calibration": rcal, "write_calibration": wcal,
           "calibration": f"plain device copy of {COPY_BYTES} bytes: FETCH_SIZE {rk:.0f} KiB, "
                          f"WRITE_SIZE {wk:.0f} KiB",
           "bytes_per_launch": per_launch, "per_kernel_bytes": per_kernel}
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


def parse_dpm_level(text):
    """Current level of an amdgpu pp_dpm_* file ("1: 2100Mhz *" marks it) in
    MHz, or None."""
    import re
    for line in text.splitlines():
        if line.rstrip().endswith("*"):
            m = re.search(r"(\d+(?:\.\d+)?)\s*mhz", line, re.I)
            if m:
                return float(m.group(1))
    return None


def sample_clocks(load):
    """The GPU's clock levels as the amdgpu driver reports them
    (/sys/class/drm/card*/device/pp_dpm_{sclk,mclk,fclk}, the files rocm-smi
    reads) while `load` (launches that keep the GPU busy for a few seconds)
    runs: a thread reads them every 0.1 s and the median of each is kept.
    None where no such file exists (one GPU per box: the first card that
    has them).  Reported beside the results, never used in them."""
    import glob
    import threading
    import time
    cards = sorted(os.path.dirname(f) for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not cards:
        return None
    dev = cards[0]
    seen = {"sclk": [], "mclk": [], "fclk": []}
    stop = threading.Event()

    def reader():
        time.sleep(0.5)
        while not stop.is_set():
            for k in seen:
                try:
                    with open(os.path.join(dev, f"pp_dpm_{k}")) as f:
                        v = parse_dpm_level(f.read())
                except OSError:
                    v = None
                if v is not None:
                    seen[k].append(v)
            time.sleep(0.1)

    th = threading.Thread(target=reader, daemon=True)
    th.start()
    load()
    stop.set()
    th.join()
    out = {f"{k}_mhz": sorted(v)[len(v) // 2] for k, v in seen.items() if v}
    if not out:
        return None
    out["samples"] = max(len(v) for v in seen.values())
    out["source"] = "amdgpu pp_dpm_* current levels, median over ~3 s of step replays after the timed region"
    return out


def capture(fn):
    """A HIP graph of the launches `fn` makes on the current stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def cpu_baseline(case, dout_cpu):
    """The fp64 oracle timed on this host on a bounded sample of the same step:
    forward + backward of KV groups 0..3 (query heads 0..31) of batch 0 at the
    full S = 4096, for both layers.  Reported in the metric's unit over that
    sample's unmasked FLOPs."""
    from oracle import ref_bwd, ref_fwd

    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [i["num_threads"] for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            cores = min(cores, max(blas))
    except Exception:
        pass
    f64 = lambda t: t.to(torch_float64()).numpy()
    q = f64(case.q[:1])
    k = f64(case.k[:1])
    v = f64(case.v[:1])
    s = f64(case.sinks)
    do = f64(dout_cpu[:1])
    heads = list(range(32))
    S = q.shape[1]
    t = time.perf_counter()
    fl = 0
    for w in WINDOWS:
        ref_fwd(q, k, v, s, w, case.scale, heads=heads)
        ref_bwd(q, k, v, s, do, w, case.scale, heads=heads)
        fl += (4 + 10) * D * len(heads) * pairs_per_head(S, w)
    el = time.perf_counter() - t
    return {"value": round(fl / el / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": "fp64 oracle fwd+bwd of batch 0, query heads 0-31 (KV groups 0-3), S=4096, both layers "
                      f"({el:.1f} s); decode not included"}


def torch_float64():
    import torch
    return torch.float64


if __name__ == "__main__":
    main()
