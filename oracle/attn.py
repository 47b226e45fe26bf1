"""Plain fp64 CPU oracle for sink attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The library (the HIP path behind the C
ABI) never imports, links or calls it, and it shares no code with that path.

What is computed (the method these pages describe, written out as a plain
definition, materialising the masked score rows):

* Attention sinks -- Megatron-LM issue "gpt-oss implementation", section
  "Attention Mechanisms / Attention Sinks"; HF blog "Tricks from OpenAI
  gpt-oss YOU can use with transformers", paragraph on Flash Attention 3 with
  attention sinks; tpu-inference PR "[GPT-OSS] JAX implementation of GPT-OSS",
  review thread on the kernel's ``attention_sink`` argument.  The pages name
  the feature only.  The reading used here: each query head h owns one learned
  logit ``sink[h]`` that joins the softmax denominator of every row and has no
  value vector (so it only drains probability mass); it is not multiplied by
  the softmax scale.
* Alternating sliding-window / full-causal layers -- Megatron-LM issue, section
  "Alternating Sliding-Window Attention Pattern"; HF blog list item "Dynamic
  Sliding Window Layer & Cache"; torchtitan PR "[WIP] Experimental
  implementation of gpt-oss (grouped GEMM MoE + FlexAttention sink/sliding)",
  title and notes.  Reading: ``window == 0`` is full causal; ``window = W >= 1``
  lets query i see keys j with ``i - W < j <= i`` (W keys including itself).
* Grouped-query heads: query head h reads K/V head ``h // (Hq // Hkv)``.
* Documents packed along the token dimension (``ref_fwd_varlen`` /
  ``ref_bwd_varlen``) -- Megatron-LM issue "gpt-oss implementation",
  discussion thread, where a user asks for attention confined to each
  document of a packed sequence (intra-document masking) and gets no answer.
  Reading: document b is rows ``cu[b] .. cu[b+1]-1``; the definition below
  applies to each document on its own (positions restart at 0, rows of other
  documents are never visible); the sink joins every row as usual.
* Decode (one new token per sequence over a packed per-sequence KV cache) is
  row ``L - 1`` of the same definition over that sequence's ``L`` cached keys
  (the HF blog's "Continuous Batching & Paged Attention" and the serve command
  in the tpu-inference PR give the workload; the maths is the prefill row).

Definition, per batch b, query head h, query row i (kv head c = h // G):

    s_ij  = scale * <q[b,i,h,:], k[b,j,c,:]>     for allowed (i, j), else -inf
    M_i   = max(sink_h, max_j s_ij)
    Z_i   = exp(sink_h - M_i) + sum_j exp(s_ij - M_i)
    P_ij  = exp(s_ij - M_i) / Z_i
    out[b,i,h,:] = sum_j P_ij v[b,j,c,:]
    lse[b,h,i]   = M_i + ln Z_i            (natural log, sink included)

Backward of L = sum(dout * out) (the sink's value vector is zero, so its
score gradient is P_sink * (0 - Dvec)):

    Dvec_i  = <dout_i, out_i>
    dS_ij   = P_ij * (<dout_i, v_j> - Dvec_i)
    dq_i    = scale * sum_j dS_ij k_j
    dk_j    = scale * sum_{h in group} sum_i dS_ij q_i
    dv_j    = sum_{h in group} sum_i P_ij dout_i
    dsink_h = - sum_{b,i} exp(sink_h - lse_{b,h,i}) * Dvec_{b,h,i}

Arrays are float64 numpy arrays in the layouts [B, S, H, D] (q, k, v, out,
dout) and [B, H, S] (lse).  Callers upcast bf16 inputs exactly.  The only
library primitives used are numpy's matrix product, exp, log and sums; the
row loop is a memory bound only (every row is independent).

Pins: tests/test_oracle.py checks this module against a scalar brute force,
hand-derived exact cases (tests/golden/hand_cases.json), torch's fp64
scaled_dot_product_attention through an augmented-key reduction, closed forms,
the four invariants, and central finite differences for the backward.
"""

import numpy as np

__all__ = ["allowed_mask", "ref_fwd", "ref_bwd", "ref_decode", "ref_decode_paged", "gather_paged",
           "unmasked_pairs", "ref_fwd_varlen", "ref_bwd_varlen"]


def allowed_mask(rows, keys, window):
    """Boolean [len(rows), len(keys)]: key j visible from query i.

    Causal (j <= i) and, for window W >= 1, inside the window (i - j < W).
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(keys, dtype=np.int64)[None, :]
    ok = j <= i
    if window > 0:
        ok &= (i - j) < window
    return ok


def unmasked_pairs(S, window):
    """Number of allowed (i, j) pairs of one (batch, head) -- counted directly."""
    total = 0
    for i in range(S):
        lo = 0 if window == 0 else max(0, i - window + 1)
        total += i - lo + 1
    return total


def _key_range(rows, window):
    """Keys [lo, hi] that can be visible from any of ``rows``."""
    lo = 0 if window == 0 else max(0, int(np.min(rows)) - window + 1)
    hi = int(np.max(rows))
    return lo, hi


def _row_softmax(s, sink):
    """Return (P, lse) for score rows ``s`` (masked = -inf) and one sink logit."""
    M = np.maximum(sink, s.max(axis=1))
    e = np.exp(s - M[:, None])
    Z = np.exp(sink - M) + e.sum(axis=1)
    return e / Z[:, None], M + np.log(Z)


def ref_fwd(q, k, v, sinks, window, scale, rows=None, heads=None,
            batches=None, row_block=512):
    """Forward: returns (out [B,S,Hq,D], lse [B,Hq,S]) in fp64.

    ``rows``/``heads``/``batches`` restrict which outputs are computed (others
    are left NaN); each computed row uses all of its visible keys, so it is
    exact.  ``row_block`` only bounds memory.
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    out = np.full((B, S, Hq, D), np.nan)
    lse = np.full((B, Hq, S), np.nan)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    batches = range(B) if batches is None else batches
    for b in batches:
        for h in heads:
            c = h // G
            for r0 in range(0, len(rows), row_block):
                rb = rows[r0:r0 + row_block]
                lo, hi = _key_range(rb, window)
                keys = np.arange(lo, hi + 1)
                s = scale * (q[b, rb, h, :] @ k[b, lo:hi + 1, c, :].T)
                s = np.where(allowed_mask(rb, keys, window), s, -np.inf)
                P, l = _row_softmax(s, float(sinks[h]))
                out[b, rb, h, :] = P @ v[b, lo:hi + 1, c, :]
                lse[b, h, rb] = l
    return out, lse


def ref_bwd(q, k, v, sinks, dout, window, scale, heads=None, batches=None):
    """Backward of sum(dout * out): returns (dq, dk, dv, dsinks) in fp64.

    Recomputes the forward (its own fp64 out and lse) per (batch, head).
    With ``heads``/``batches`` given, dq covers those heads only, dk/dv sum the
    contributions of those heads only, and dsinks sums over those batches.
    """
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    dsinks = np.zeros(Hq)
    heads = range(Hq) if heads is None else heads
    batches = range(B) if batches is None else batches
    pos = np.arange(S)
    mask = allowed_mask(pos, pos, window)
    for b in batches:
        for h in heads:
            c = h // G
            Q, K, V, dO = q[b, :, h, :], k[b, :, c, :], v[b, :, c, :], dout[b, :, h, :]
            s = np.where(mask, scale * (Q @ K.T), -np.inf)
            P, lse = _row_softmax(s, float(sinks[h]))
            O = P @ V
            Dvec = (dO * O).sum(axis=1)
            dP = dO @ V.T
            dS = P * (dP - Dvec[:, None])
            dq[b, :, h, :] = scale * (dS @ K)
            dk[b, :, c, :] += scale * (dS.T @ Q)
            dv[b, :, c, :] += P.T @ dO
            dsinks[h] -= np.sum(np.exp(float(sinks[h]) - lse) * Dvec)
    return dq, dk, dv, dsinks


def ref_decode(q, k_cache, v_cache, cu_seqlens, sinks, window, scale):
    """Decode: one query per sequence over its packed KV rows.

    q [N, Hq, D]; k_cache, v_cache [T, Hkv, D]; sequence n owns cache rows
    cu_seqlens[n] .. cu_seqlens[n+1]-1 (L_n of them, the new token's K/V last).
    The query sits at position L_n - 1.  Returns (out [N,Hq,D], lse [N,Hq]).
    An empty sequence (L_n = 0) sees only the sink: out = 0, lse = sink.
    """
    N, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((N, Hq, D))
    lse = np.zeros((N, Hq))
    for n in range(N):
        base, L = int(cu_seqlens[n]), int(cu_seqlens[n + 1] - cu_seqlens[n])
        for h in range(Hq):
            sink = float(sinks[h])
            if L == 0:
                out[n, h, :] = 0.0
                lse[n, h] = sink
                continue
            c = h // G
            keys = np.arange(L)
            ok = allowed_mask([L - 1], keys, window)[0]
            s = scale * (k_cache[base:base + L, c, :] @ q[n, h, :])
            s = np.where(ok, s, -np.inf)[None, :]
            P, l = _row_softmax(s, sink)
            out[n, h, :] = (P @ v_cache[base:base + L, c, :])[0]
            lse[n, h] = l[0]
    return out, lse


def gather_paged(k_pages, v_pages, block_table, seq_lens, ring_tokens, window):
    """The visible K/V rows of every sequence of a paged cache, in position
    order, as a packed cache.

    HF blog "Tricks from OpenAI gpt-oss YOU can use with transformers", items
    "Continuous Batching & Paged Attention" (the cache lives in fixed-size
    pages named by a per-sequence block table) and "Dynamic Sliding Window
    Layer & Cache" (a sliding layer keeps only its last W tokens).  Position t
    of sequence n sits in slot t (linear cache, ring_tokens = 0) or slot
    t mod ring_tokens (ring), i.e. in page block_table[n][slot // page_size]
    at row slot % page_size.  The visible positions are [L - W, L) (all L when
    W = 0); in a ring, positions before L - ring_tokens have been overwritten,
    so W <= ring_tokens is required.

    k_pages, v_pages [P, page_size, Hkv, D]; block_table [N, pages_per_seq];
    seq_lens [N].  Returns (k_cache, v_cache [T, Hkv, D], cu_seqlens [N + 1])
    holding only the visible rows.
    """
    page_size = k_pages.shape[1]
    if ring_tokens:
        assert 1 <= window <= ring_tokens
    ks, vs, cu = [], [], [0]
    for n, L in enumerate(seq_lens):
        L = int(L)
        lo = max(0, L - window) if window > 0 else 0
        for t in range(lo, L):
            slot = t % ring_tokens if ring_tokens else t
            page = int(block_table[n][slot // page_size])
            ks.append(k_pages[page, slot % page_size])
            vs.append(v_pages[page, slot % page_size])
        cu.append(cu[-1] + (L - lo))
    Hkv, D = k_pages.shape[2], k_pages.shape[3]
    kc = np.array(ks).reshape(-1, Hkv, D) if ks else np.zeros((0, Hkv, D))
    vc = np.array(vs).reshape(-1, Hkv, D) if vs else np.zeros((0, Hkv, D))
    return kc, vc, np.array(cu)


def ref_decode_paged(q, k_pages, v_pages, block_table, seq_lens, sinks, ring_tokens, window, scale):
    """Decode against a paged cache: the query of sequence n (position L_n - 1)
    over its visible rows read through the block table (gather_paged); the
    attention itself is ref_decode on those rows (all of them visible)."""
    kc, vc, cu = gather_paged(k_pages, v_pages, block_table, seq_lens, ring_tokens, window)
    return ref_decode(q, kc, vc, cu, sinks, 0, scale)


def ref_fwd_varlen(q, k, v, cu_seqlens, sinks, window, scale, docs=None, heads=None):
    """Forward over packed documents: q [T,Hq,D], k/v [T,Hkv,D].

    Each document is the batch-of-one forward of its own rows.  Returns
    (out [T,Hq,D], lse [Hq,T]); rows outside the computed documents stay NaN.
    ``docs`` / ``heads`` restrict which documents / query heads are computed.
    """
    T, Hq, D = q.shape
    out = np.full((T, Hq, D), np.nan)
    lse = np.full((Hq, T), np.nan)
    n_docs = len(cu_seqlens) - 1
    for b in (range(n_docs) if docs is None else docs):
        a, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if e <= a:
            continue
        o, l = ref_fwd(q[None, a:e], k[None, a:e], v[None, a:e], sinks, window, scale, heads=heads)
        out[a:e] = o[0]
        lse[:, a:e] = l[0]
    return out, lse


def ref_bwd_varlen(q, k, v, cu_seqlens, sinks, dout, window, scale, docs=None, heads=None):
    """Backward of sum(dout * out) over packed documents.

    Returns (dq, dk, dv, dsinks); dq/dk/dv rows outside the computed documents
    stay NaN and dsinks sums the computed documents' rows.  With ``heads``
    given, only those query heads contribute (as in ref_bwd).
    """
    dq = np.full(q.shape, np.nan)
    dk = np.full(k.shape, np.nan)
    dv = np.full(v.shape, np.nan)
    dsinks = np.zeros(q.shape[1])
    n_docs = len(cu_seqlens) - 1
    for b in (range(n_docs) if docs is None else docs):
        a, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        if e <= a:
            continue
        gq, gk, gv, gs = ref_bwd(q[None, a:e], k[None, a:e], v[None, a:e], sinks, dout[None, a:e], window, scale,
                                 heads=heads)
        dq[a:e], dk[a:e], dv[a:e] = gq[0], gk[0], gv[0]
        dsinks += gs
    return dq, dk, dv, dsinks
