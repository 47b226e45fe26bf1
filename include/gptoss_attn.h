/*
 * gptoss_attn.h -- C ABI of the MI355X (gfx950) sink-attention library.
 *
 * The operation (cited pages: Megatron-LM issue "gpt-oss implementation",
 * sections "Attention Sinks" and "Alternating Sliding-Window Attention
 * Pattern"; HF blog "Tricks from OpenAI gpt-oss YOU can use with
 * transformers", the Flash Attention 3 with attention sinks paragraph and the
 * "Dynamic Sliding Window Layer & Cache" / "Continuous Batching & Paged
 * Attention" items; tpu-inference PR "[GPT-OSS] JAX implementation of
 * GPT-OSS", the kernel's attention_sink argument and the serve command):
 *
 *   causal grouped-query attention in which every query head h owns one
 *   learned logit sinks[h] that joins the softmax denominator of each row and
 *   has no value vector.  For batch b, query head h (kv head c = h / G,
 *   G = Hq / Hkv) and query position i:
 *
 *     s_ij   = softmax_scale * dot(q[b,i,h,:], k[b,j,c,:])   visible j only
 *     M_i    = max(sinks[h], max_j s_ij)
 *     Z_i    = exp(sinks[h] - M_i) + sum_j exp(s_ij - M_i)
 *     out[b,i,h,:] = sum_j exp(s_ij - M_i) / Z_i * v[b,j,c,:]
 *     lse[b,h,i]   = M_i + ln Z_i          (natural log, sink included)
 *
 *   Key j is visible from query i when j <= i and, for window W >= 1, also
 *   i - j < W (W keys including the query itself).  window = 0 is full causal;
 *   a window >= S gives the same result as window = 0.  The sink is not
 *   multiplied by softmax_scale; sinks[h] = -INFINITY removes it.
 *
 * Conventions for every entry point
 *   - Tensors are dense, contiguous, row-major, in DEVICE memory of the current
 *     HIP device, and 16-byte aligned.  bf16 is IEEE bfloat16 (stored as
 *     uint16).  Layouts: q/out/dout/dq [B, S, Hq, D]; k/v/dk/dv [B, S, Hkv, D];
 *     lse [B, Hq, S]; sinks/dsinks [Hq].
 *   - head_dim D must be 64 and the group size Hq / Hkv at most 128
 *     (GPTOSS_ERR_UNSUPPORTED otherwise).  The decode entry points also need
 *     ceil(Hkv / 2) * ceil(Hq / Hkv / 32) <= 65535 (their launch's workgroup
 *     rows; GPTOSS_ERR_UNSUPPORTED otherwise).
 *   - The caller owns every buffer (inputs, outputs, workspace).  The library
 *     allocates no device memory and keeps no state between calls beyond a
 *     per-device capability check and the per-thread error message.
 *   - Calls enqueue work on `stream` (a hipStream_t; NULL = the null stream)
 *     and return without synchronising.  Outputs are overwritten, never
 *     accumulated into.  Calls on different streams must not share outputs or
 *     workspace.
 *   - Argument errors are detected on the host before any HIP call and
 *     nothing is written.  A zero-sized problem (B == 0, S == 0, N == 0 or
 *     T == 0) returns GPTOSS_OK without touching memory.  Contents of device buffers
 *     (NaN/Inf in inputs, cu_seqlens values) are caller contracts and are not
 *     checked.
 *   - gptoss_attn_last_error() returns the message of this thread's last
 *     non-OK status.
 */
#ifndef GPTOSS_ATTN_H
#define GPTOSS_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPTOSS_ATTN_ABI_VERSION 1

typedef enum {
    GPTOSS_OK = 0,
    GPTOSS_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, alignment, workspace */
    GPTOSS_ERR_UNSUPPORTED = 2,      /* head_dim != 64, device is not gfx950 */
    GPTOSS_ERR_HIP = 3               /* a HIP runtime call or launch failed */
} gptoss_status;

/* ABI version of the loaded library (GPTOSS_ATTN_ABI_VERSION it was built with). */
int gptoss_attn_abi_version(void);

/* Message for this thread's last non-OK status ("" if none).  The pointer
 * stays valid until the next library call on the same thread. */
const char* gptoss_attn_last_error(void);

/*
 * Prefill forward.  Computes out and lse as defined above.
 *   q      bf16 [B, S, Hq, D]          read
 *   k, v   bf16 [B, S, Hkv, D]         read
 *   sinks  fp32 [Hq]                   read
 *   out    bf16 [B, S, Hq, D]          written (round-to-nearest-even)
 *   lse    fp32 [B, Hq, S]             written
 * Requires B, S >= 0, Hq >= 1, Hkv >= 1, Hq % Hkv == 0, window >= 0,
 * softmax_scale finite and > 0.
 */
gptoss_status gptoss_attn_fwd(const void* q, const void* k, const void* v,
                              const float* sinks, int B, int S, int Hq, int Hkv,
                              int D, int window, float softmax_scale, void* out,
                              float* lse, void* stream);

/*
 * Training backward of the forward above for the loss sum(dout * out):
 *   dq = dL/dq, dk = dL/dk, dv = dL/dv (bf16, RNE), dsinks = dL/dsinks (fp32,
 *   summed over batch and positions).  With Dvec_i = dot(dout_i, out_i):
 *   dS_ij = P_ij (dot(dout_i, v_j) - Dvec_i) and
 *   dsinks[h] = -sum_{b,i} exp(sinks[h] - lse[b,h,i]) * Dvec[b,h,i].
 *   out and lse must be the forward's outputs for the same inputs.
 *   q, k, v, out, dout bf16 (layouts as above); sinks fp32 [Hq];
 *   lse fp32 [B, Hq, S]                          read
 *   dq bf16 [B,S,Hq,D]; dk, dv bf16 [B,S,Hkv,D]; dsinks fp32 [Hq]   written
 *   workspace  device scratch of at least gptoss_attn_bwd_workspace_size()
 *              bytes, 256-byte aligned; its contents on entry do not matter.
 */
size_t gptoss_attn_bwd_workspace_size(int B, int S, int Hq, int Hkv, int D, int window);
gptoss_status gptoss_attn_bwd(const void* q, const void* k, const void* v,
                              const float* sinks, const void* out, const float* lse,
                              const void* dout, int B, int S, int Hq, int Hkv, int D,
                              int window, float softmax_scale, void* dq, void* dk,
                              void* dv, float* dsinks, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Decode: one new query token per sequence against a packed KV cache
 * (split-KV partial softmax per chunk of keys, then an lse merge in which the
 * sink enters exactly once).
 *   q           bf16 [N, Hq, D]                 read
 *   k_cache,
 *   v_cache     bf16 [T, Hkv, D]                read; sequence n owns rows
 *               cu_seqlens[n] .. cu_seqlens[n+1]-1 (L_n rows, the new token's
 *               K/V last); its query sits at position L_n - 1.
 *   cu_seqlens  int32 [N + 1], device, cu_seqlens[0] = 0, non-decreasing
 *   max_seqlen  host-side upper bound of every L_n (>= 1); it sizes the split
 *               grid without reading device memory.  L_n > max_seqlen is a
 *               caller error whose keys beyond max_seqlen are ignored.
 *   out         bf16 [N, Hq, D]   written;  lse fp32 [N, Hq] written.
 *               An empty sequence (L_n = 0) gives out = 0, lse = sinks[h].
 *   max_seqlen  at most 2^30 (INVALID_ARGUMENT above).
 *   workspace   at least gptoss_attn_decode_workspace_size() bytes,
 *               256-byte aligned (split partials; 0 bytes: may be NULL);
 *               contents on entry ignored.
 */
size_t gptoss_attn_decode_workspace_size(int N, int Hq, int Hkv, int D, int max_seqlen,
                                         int window);
gptoss_status gptoss_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                 const int* cu_seqlens, const float* sinks, int N, int Hq,
                                 int Hkv, int D, int max_seqlen, int window,
                                 float softmax_scale, void* out, float* lse,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * gptoss_attn_decode without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same operation, arguments (minus the workspace)
 * and outputs as gptoss_attn_decode.  The split partials live in a
 * library-owned array of 4 MiB in each GPU's memory (held until the process
 * ends; its address is looked up once per device); a call whose plan needs
 * more (gptoss_attn_decode_workspace_size() > 4 MiB) returns
 * GPTOSS_ERR_INVALID_ARGUMENT before any HIP call.  The call allocates nothing.  Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (different
 * streams, concurrent host threads) race and must be serialised by the
 * caller.
 */
gptoss_status gptoss_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         const int* cu_seqlens, const float* sinks, int N, int Hq,
                                         int Hkv, int D, int max_seqlen, int window,
                                         float softmax_scale, void* out, float* lse, void* stream);

/*
 * Decode against a paged KV cache (HF blog "Tricks from OpenAI gpt-oss YOU
 * can use with transformers", items "Continuous Batching & Paged Attention"
 * and "Dynamic Sliding Window Layer & Cache": the cache lives in fixed-size
 * pages named by a per-sequence block table, and a sliding layer need keep
 * only its last W tokens).  Same operation and outputs as gptoss_attn_decode;
 * only the addressing of K/V rows differs.
 *   k_pages,
 *   v_pages     bf16 [num_pages, page_size, Hkv, D]   read; page p holds
 *               page_size token rows of Hkv heads.
 *   block_table int32 [N, pages_per_seq], device: entry [n][i] is the page
 *               holding slots i*page_size .. (i+1)*page_size-1 of sequence n.
 *   seq_lens    int32 [N], device: L_n, tokens of sequence n so far (the new
 *               token included); its query sits at position L_n - 1.
 *   ring_tokens 0: slot of position t is t (linear cache; needs
 *                  max_seqlen <= pages_per_seq * page_size).
 *               R > 0: the cache of every sequence is a ring of R slots,
 *                  position t in slot t mod R (positions t - R and before
 *                  have been overwritten).  Needs window >= 1, window <= R,
 *                  R a power of two, a multiple of page_size, and
 *                  R / page_size <= pages_per_seq.
 *   page_size   a power of two, 1 .. 65536.
 *   workspace   gptoss_attn_decode_workspace_size(N, Hq, Hkv, D, max_seqlen,
 *               window) bytes, 256-byte aligned; contents on entry ignored.
 * Page indices in block_table and the seq_lens values are caller contracts
 * (not checked); a sequence with L_n > max_seqlen sees its first max_seqlen
 * positions only.
 */
gptoss_status gptoss_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                       const int* block_table, const int* seq_lens,
                                       const float* sinks, int N, int Hq, int Hkv, int D,
                                       int page_size, int pages_per_seq, int ring_tokens,
                                       int max_seqlen, int window, float softmax_scale,
                                       void* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Packed variable-length prefill (documents packed back to back in one token
 * dimension, attention confined to each document).  Megatron-LM issue
 * "gpt-oss implementation", discussion thread: a user asks for attention
 * computed within each document of a packed sequence rather than over the
 * whole sequence (intra-document masking); the pages give no answer.  The
 * reading used here: document b is rows cu_seqlens[b] .. cu_seqlens[b+1]-1,
 * its positions restart at 0, and the definition above (sink, causal and
 * window visibility) applies inside each document on its own; rows of other
 * documents are never visible.
 *   q, out          bf16 [T, Hq, D]      (q read, out written)
 *   k, v            bf16 [T, Hkv, D]     read
 *   cu_seqlens      int32 [N + 1], device, non-decreasing, 0 <= cu[0],
 *                   cu[N] <= T.  Rows outside every document are neither
 *                   read as keys nor written.  The kernels clamp the
 *                   offsets into [0, T], so offsets that break this contract
 *                   give unspecified results but no access outside the
 *                   tensors.
 *   max_seqlen      host-side upper bound of every document length (>= 1); it
 *                   sizes the grid without reading device memory.  A longer
 *                   document is a caller error: only its first max_seqlen rows
 *                   are computed and the rest are not written.
 *   lse             fp32 [Hq, T]         written (entry [h][row] for each row
 *                   inside a document)
 * window >= max_seqlen gives the same result as window = 0.
 */
gptoss_status gptoss_attn_fwd_varlen(const void* q, const void* k, const void* v,
                                     const int* cu_seqlens, const float* sinks, int N, int T,
                                     int Hq, int Hkv, int D, int max_seqlen, int window,
                                     float softmax_scale, void* out, float* lse, void* stream);

/*
 * Backward of gptoss_attn_fwd_varlen for the loss sum(dout * out), the
 * per-document counterpart of gptoss_attn_bwd.
 *   q, out, dout    bf16 [T, Hq, D]; k, v bf16 [T, Hkv, D]; lse fp32 [Hq, T]
 *                   as written by the forward                         read
 *   dq bf16 [T, Hq, D]; dk, dv bf16 [T, Hkv, D]                       written
 *                   on the rows inside a document (others not written)
 *   dsinks fp32 [Hq] written: the sum over every document's rows (0 when no
 *                   row lies inside a document).
 *   workspace       gptoss_attn_bwd_varlen_workspace_size(T, Hq, Hkv, D) bytes,
 *                   256-byte aligned; contents on entry ignored.
 */
size_t gptoss_attn_bwd_varlen_workspace_size(int T, int Hq, int Hkv, int D);
gptoss_status gptoss_attn_bwd_varlen(const void* q, const void* k, const void* v,
                                     const int* cu_seqlens, const float* sinks, const void* out,
                                     const float* lse, const void* dout, int N, int T, int Hq,
                                     int Hkv, int D, int max_seqlen, int window,
                                     float softmax_scale, void* dq, void* dk, void* dv,
                                     float* dsinks, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * Rotary position embedding with YaRN scaling, fused into the prefill and
 * decode load stage.  Megatron-LM issue "gpt-oss implementation", section
 * "Positional Encodings / YaRN RoPE Scaling", names YaRN (to 128k+ context)
 * and cites the YaRN paper (arXiv:2309.00071), whose definitions are used;
 * the pages give no formula or parameters.  For pair i = 0..31 of a 64-wide
 * head:
 *   theta_i = base^(-2i/64);  r_i = orig_ctx * theta_i / (2 pi)  (turns over
 *   the original context);  gamma_i = clamp((r_i - alpha) / (beta - alpha),
 *   0, 1);  h_i = (1 - gamma_i) theta_i / factor + gamma_i theta_i;
 *   m = 0.1 ln(factor) + 1 (m = 1 and h_i = theta_i when factor = 1).
 * Element i of a q or k row at position p is rotated with element i + 32:
 *   y_i = x_i c - x_{i+32} s,  y_{i+32} = x_{i+32} c + x_i s,
 *   c = m cos(p h_i), s = m sin(p h_i)  (fp32, from the table below);
 * y is the exact value of that expression (bf16 x, fp32 c and s) rounded
 * once to bf16, nearest even: the attention consumes bf16 q and k.
 *
 * gptoss_attn_rope_table: fills table, fp32 [positions][32][2] = (c, s),
 *   evaluated in fp64.  Requires D == 64, positions >= 1, base > 1,
 *   factor >= 1, and for factor > 1 orig_ctx >= 1 and alpha < beta.
 */
gptoss_status gptoss_attn_rope_table(float* table, int positions, int D, double base, double factor,
                                     double orig_ctx, double alpha, double beta, void* stream);

/*
 * Rotates rows x bf16 [T, H, D] (token t at position positions[t], int32 [T]
 * on the device; positions outside [0, table_positions) are clamped) into y
 * (same layout; y may equal x, otherwise they must not overlap).  Used to
 * append a new token's key to a rotated KV cache.  transpose != 0 applies
 * the adjoint R^T instead (y_i = x_i c + x_{i+32} s, y_{i+32} = x_{i+32} c -
 * x_i s), which carries a gradient with respect to rotated rows back to the
 * unrotated ones.
 */
gptoss_status gptoss_attn_rope_rows(const void* x, void* y, const int* positions, int T, int H, int D,
                                    const float* table, int table_positions, int transpose, void* stream);

/*
 * Prefill forward with the rotation fused: q and k are the unrotated
 * projections [B, S, H, D] (token i of every batch at position i); the
 * operation is gptoss_attn_fwd over the rotated q and k.  k is rotated once
 * by a pre-pass into k_rot (bf16 [B, S, Hkv, D], written; it is also the
 * rotated key cache a decoder keeps; it must not overlap k); q is rotated in
 * the attention kernel's load stage.  table: gptoss_attn_rope_table output
 * with table_positions >= S.
 */
gptoss_status gptoss_attn_fwd_rope(const void* q, const void* k, const void* v, const float* sinks,
                                   const float* table, int table_positions, int B, int S, int Hq, int Hkv,
                                   int D, int window, float softmax_scale, void* out, float* lse, void* k_rot,
                                   void* stream);

/*
 * Decode with the query rotation fused: as gptoss_attn_decode, with q the
 * unrotated projection of the new token, rotated at its position L_n - 1 in
 * the kernel's load stage; the caches hold rotated keys (k_rot of the
 * prefill, then each new token's key through gptoss_attn_rope_rows).
 * table_positions >= max_seqlen.
 */
gptoss_status gptoss_attn_decode_rope(const void* q, const void* k_cache, const void* v_cache,
                                      const int* cu_seqlens, const float* sinks, const float* table,
                                      int table_positions, int N, int Hq, int Hkv, int D, int max_seqlen,
                                      int window, float softmax_scale, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Training backward of gptoss_attn_fwd_rope for the loss sum(dout * out):
 * gradients with respect to the unrotated q and k.  Takes q (unrotated) and
 * k_rot (the forward's rotated keys); the backward of gptoss_attn_bwd runs
 * on the rotated q and k (the dq kernel rotates q, as gptoss_attn_fwd_rope
 * does, and leaves it in the workspace for the dk/dv kernel), and dq, dk are
 * carried back through the adjoint rotation R^T, applied to the fp32
 * gradients before their one rounding to bf16.  The rounding of the rotated
 * q and k to bf16 is not differentiated (its derivative is taken as 1).
 *   q, out, dout bf16 [B, S, Hq, D]; k_rot, v bf16 [B, S, Hkv, D];
 *   lse fp32 [B, Hq, S] as written by gptoss_attn_fwd_rope      read
 *   dq [B,S,Hq,D], dk, dv [B,S,Hkv,D] bf16; dsinks fp32 [Hq]    written
 *   workspace  gptoss_attn_bwd_rope_workspace_size(B, S, Hq, Hkv, D) bytes,
 *              256-byte aligned (the rotated q, then the backward's own).
 */
size_t gptoss_attn_bwd_rope_workspace_size(int B, int S, int Hq, int Hkv, int D);
gptoss_status gptoss_attn_bwd_rope(const void* q, const void* k_rot, const void* v, const float* sinks,
                                   const float* table, int table_positions, const void* out,
                                   const float* lse, const void* dout, int B, int S, int Hq, int Hkv,
                                   int D, int window, float softmax_scale, void* dq, void* dk,
                                   void* dv, float* dsinks, void* workspace,
                                   size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GPTOSS_ATTN_H */
