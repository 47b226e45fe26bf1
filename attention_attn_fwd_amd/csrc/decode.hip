// Split-KV decode of grouped-query sink attention (gfx950).
//
// One new query token per sequence attends to that sequence's packed KV cache
// rows (the decode workload of HF blog "Tricks from OpenAI gpt-oss YOU can
// use with transformers", "Continuous Batching & Paged Attention" and
// "Dynamic Sliding Window Layer & Cache"; batch shape from the serve command
// of tpu-inference PR "[GPT-OSS] JAX implementation of GPT-OSS").  The query
// of sequence n sits at position L_n - 1, so it sees keys
// [max(0, L_n - W), L_n) (all L_n keys when W = 0).
//
// The work is memory bound: every K/V byte is read once and serves all G
// query heads of its KV head.
//   split kernel : grid (chunk of visible keys, group of 4 KV heads x head
//     block, sequence); chunks are only cut when too few (sequence, group)
//     pairs would fill the chip.  Each wave owns one KV head, so the 4 waves of a
//     workgroup stream adjacent 128-byte rows of the same tokens (512
//     contiguous bytes per token for K and again for V).  A wave walks its
//     chunk in 64-key tiles: whole K and V rows (8 lanes per 128-byte row)
//     go through wave-private LDS tiles, K read back as MFMA A operands and V
//     transposed, S^T = K Q^T and O^T = V^T P^T on 32x32x16 bf16 MFMAs with the G query
//     heads as columns, an online softmax across tiles, and the next tile's
//     loads in flight while the current one is computed.  Waves never
//     synchronise.  A sequence that fits in one chunk is finished in place
//     (sink folded in, out and lse written); otherwise the wave writes one
//     partial (unnormalised O, running max m in log2 units, sum l) per head.
//   merge kernels (one wave per (sequence, head) when there are at most 16
//     chunks, one workgroup per (sequence, head) otherwise):
//     m = max(sink, m_s), l = 2^(sink - m) + sum l_s 2^(m_s - m),
//     out = sum O_s 2^(m_s - m) / l, lse = ln2 (m + log2 l).  The sink enters
//     here exactly once.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace gptoss {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;         // KV heads per workgroup, one per wave
constexpr int kTileKeys = 64;     // keys per wave step
constexpr int kPartStride = 68;   // floats per partial: O[64], m, l, pad
// Workgroups the chunking aims for: one per CU.  Cutting the 128 x 1024
// workload finer (512 or more workgroups, merged afterwards) measured slower.
constexpr long long kTargetWorkgroups = 256;


struct DecParams {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int* cu;
    const float* sinks;
    uint16_t* out;
    float* lse;
    float* part;      // [N][Hq][n_splits][kPartStride]
    const int* bt;    // paged cache: block table [N][pps]; nullptr for the contiguous cache
    const int* lens;  // paged cache: L_n per sequence
    const float2* rope;  // (cos, sin) table: q rotated at position L_n - 1 (keys arrive rotated); nullptr = none
    int ps_shift, ps_mask, pps, ring_mask;  // page size = 1 << ps_shift; slot = position & ring_mask
    int Hq, Hkv, G, window, n_splits, n_hblk, max_seqlen;
    int chunk_keys;   // visible keys per chunk (a multiple of 64)
    float c;          // scale * log2(e)
};

__device__ __forceinline__ void seq_range(const DecParams& p, int n, int& base, int& L, int& vis_lo) {
    if (p.bt != nullptr) {
        base = 0;
        L = min(p.lens[n], p.max_seqlen);
    } else {
        base = p.cu[n];
        L = min(p.cu[n + 1] - base, p.max_seqlen);
    }
    vis_lo = p.window > 0 ? max(0, L - p.window) : 0;
}

// The loads of tile t + 1 are issued as soon as tile t has been moved to
// LDS.  (Keeping two to four tiles per wave in flight, at one wave per SIMD,
// measured slower on the 128 x 1024 workload than one tile per wave at two
// workgroups per CU, and so did two waves per KV head taking alternate tiles.)
// kPaged: K/V rows are found through the block table (slot = position &
// ring_mask, page = bt[n][slot >> ps_shift], row = slot & ps_mask); the page
// indices of a tile are loaded one tile ahead of its K/V rows.
template <bool kPaged>
__global__ void __launch_bounds__(kThreads, 2)
decode_split_kernel(DecParams p) {
    __shared__ uint4 ksm[kWaves][kTileUnits];  // one row-major K tile per wave
    __shared__ uint4 vsm[kWaves][kTileUnits];  // one row-major V tile per wave

    const int chunk = blockIdx.x;
    const int kvg = blockIdx.y / p.n_hblk;
    const int hb = blockIdx.y % p.n_hblk;
    const int n = blockIdx.z;
    int base, L, vis_lo;
    seq_range(p, n, base, L, vis_lo);
    const int n_vis = L - vis_lo;
    const int n_act = (n_vis + p.chunk_keys - 1) / p.chunk_keys;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int kvh = kvg * kWaves + wave;
    if (n_act == 0) {
        // empty sequence: only the sink is visible (out = 0, lse = sink)
        if (chunk == 0 && kvh < p.Hkv && hb * 32 + (lane & 31) < p.G) {
            const int hd = kvh * p.G + hb * 32 + (lane & 31);
            uint16_t* orow = p.out + ((size_t)n * p.Hq + hd) * kHeadDim + 32 * (lane >> 5);
#pragma unroll
            for (int i = 0; i < 4; ++i) st16(orow + 8 * i, make_uint4(0, 0, 0, 0));
            if (lane < 32) p.lse[(size_t)n * p.Hq + hd] = p.sinks[hd];
        }
        return;
    }
    if (chunk >= n_act) return;
    if (kvh >= p.Hkv) return;  // waves are independent: no barrier follows
    const int g = lane >> 5, l32 = lane & 31;
    const int G = p.G;
    const int hcol = hb * 32 + l32;  // head within the group
    const bool col_ok = hcol < G;
    const int head = kvh * G + hcol;

    const int c0 = vis_lo + chunk * p.chunk_keys;
    const int c1 = min(c0 + p.chunk_keys, L);  // exclusive
    const int n_tiles = (c1 - c0 + kTileKeys - 1) / kTileKeys;

    const size_t row_stride = (size_t)p.Hkv * kHeadDim;
    const uint16_t* kb = p.kc + ((size_t)base * p.Hkv + kvh) * kHeadDim;
    const uint16_t* vb = p.vc + ((size_t)base * p.Hkv + kvh) * kHeadDim;
    const int* bt_row = kPaged ? p.bt + (size_t)n * p.pps : nullptr;

    // the sink is only needed when a single-chunk sequence is finished, but
    // is loaded here so that its latency hides behind the tiles
    const float sink = col_ok ? p.sinks[head] : 0.0f;
    uint4 qraw[4];
    {
        const uint16_t* qrow = p.q + ((size_t)n * p.Hq + head) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qraw[ks] = make_uint4(0, 0, 0, 0);
            if (col_ok) qraw[ks] = ld16(qrow + 16 * ks + 8 * g);
        }
    }
    // rotary table entries of the query at position L - 1 (pairs d, d + 32
    // are fragments ks and ks + 2), loaded ahead of the first tile
    float4 rcs[2][4];
    if (p.rope != nullptr) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) load_rope8(p.rope, L - 1, 16 * ks + 8 * g, rcs[ks]);
    }

    // tile loads: eight consecutive lanes read one whole 128-byte K or V row
    // (lane loads unit lane % 8 of rows lane / 8 + 8 j), so every load
    // instruction covers 8 full rows; the rows go through the wave's LDS
    // tiles.  Rows past the chunk end re-read its last row: their scores are
    // masked to -inf, so they add exactly 0 to l and to O.
    uint4 kr[8], vr[8];
    int pid[8];  // paged: page of each of this lane's 8 rows of the next tile to load
    auto tile_key = [&](int t, int j) { return min(c0 + t * kTileKeys + (lane >> 3) + 8 * j, c1 - 1); };
    auto load_pids = [&](int t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pid[j] = bt_row[(tile_key(t, j) & p.ring_mask) >> p.ps_shift];
    };
    auto load_tile = [&](int t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = tile_key(t, j);
            size_t row = (size_t)key;
            if (kPaged) row = ((size_t)pid[j] << p.ps_shift) + (size_t)(key & p.ring_mask & p.ps_mask);
            kr[j] = ld16(kb + row * row_stride + 8 * (lane & 7));
            vr[j] = ld16(vb + row * row_stride + 8 * (lane & 7));
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 oacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

    if (kPaged) {
        load_pids(0);
        load_tile(0);
        if (n_tiles > 1) load_pids(1);
    } else {
        load_tile(0);  // n_tiles >= 1 here
    }
    if (p.rope != nullptr) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) rope8(qraw[ks], qraw[ks + 2], rcs[ks]);
    }
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(qraw[ks]);
    for (int t = 0; t < n_tiles; ++t) {
        // K and V tiles -> this wave's LDS tiles.  Only this wave touches
        // them and a wave's LDS operations complete in order, so the previous
        // tile's reads are done; the signal fences keep the compiler from
        // moving LDS accesses across the hand-over.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            ksm[wave][tile_unit((lane >> 3) + 8 * j, lane & 7)] = kr[j];
            vsm[wave][tile_unit((lane >> 3) + 8 * j, lane & 7)] = vr[j];
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (t + 1 < n_tiles) {  // in flight during this tile's compute
            load_tile(t + 1);
            if (kPaged && t + 2 < n_tiles) load_pids(t + 2);
        }
        // S^T = K Q^T; A operand rows are keys in the forward's permuted
        // order, K slots 8 g + 0..7 of step ks are d = 16 ks + 8 g + 0..7
        f32x16 sacc[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sacc[mb] = mfma32(as_bf16x8(ksm[wave][tile_unit(32 * mb + perm_row(l32), 2 * ks + g)]), qf[ks],
                                  sacc[mb]);
        }
        // keys at or beyond c1 are invisible: register r of block mb holds key
        // t0 + 32 mb + 16 (r / 8) + 8 g + r % 8
        const int rem = c1 - (c0 + t * kTileKeys) - 8 * g;
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cr = 32 * mb + 16 * (r >> 3) + (r & 7);
                sacc[mb][r] = cr < rem ? sacc[mb][r] : -INFINITY;
                mx = fmaxf(mx, sacc[mb][r]);
            }
        mx = max_across_halves(mx);
        const float m_new = fmaxf(m_run, mx * p.c);  // finite: every tile has a visible key
        const float alpha = fast_exp2(m_run - m_new);  // m_run = -inf -> 0
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
        m_run = m_new;
        bf16x8 pb[4];
        float la = 0.0f, lb = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r = 8 * (kk & 1) + 2 * j;
                const float e0 = fast_exp2(fmaf(sacc[kk >> 1][r], p.c, -m_run));
                const float e1 = fast_exp2(fmaf(sacc[kk >> 1][r + 1], p.c, -m_run));
                la += e0;
                lb += e1;
                w[j] = pack_bf16x2(e0, e1);
            }
            pb[kk] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        }
        l_run += la + lb;
        // O^T += V^T P^T (V^T rows d = 32 db + l32, keys 16 kk + 8 g + 0..7)
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                oacc[db] = mfma32(tile_read_tr8(vsm[wave], 16 * kk + 8 * g, 32 * db + 16 * (l32 >> 4), l32 & 15),
                                  pb[kk], oacc[db]);
    }

    const float l_tot = sum_across_halves(l_run);
    if (!col_ok) return;
    if (n_act == 1) {
        // finish in place: fold in the sink
        const float s2 = sink * kLog2e;
        const float mf = fmaxf(s2, m_run);
        const float a = fast_exp2(m_run - mf);
        const float lfin = (sink == -INFINITY ? 0.0f : fast_exp2(s2 - mf)) + l_tot * a;
        const float inv = a / lfin;
        uint16_t* orow = p.out + ((size_t)n * p.Hq + head) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * db + 8 * r4 + 4 * g;
                uint2 w;
                w.x = pack_bf16x2(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv);
                w.y = pack_bf16x2(oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
                *reinterpret_cast<uint2*>(orow + d0) = w;
            }
        if (g == 0) p.lse[(size_t)n * p.Hq + head] = (mf + fast_log2(lfin)) * kLn2;
        return;
    }
    float* dst = p.part + (((size_t)n * p.Hq + head) * p.n_splits + chunk) * kPartStride;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = 32 * db + 8 * r4 + 4 * g;
            *reinterpret_cast<float4*>(dst + d0) =
                make_float4(oacc[db][4 * r4 + 0], oacc[db][4 * r4 + 1], oacc[db][4 * r4 + 2], oacc[db][4 * r4 + 3]);
        }
    if (g == 0) {
        dst[64] = m_run;
        dst[65] = l_tot;
    }
}

// Few chunks (at most kFewChunks): one wave per (sequence, head), four heads
// per workgroup; lane = d, the chunks' partials are read in one unrolled pass.
constexpr int kFewChunks = 16;
__global__ void __launch_bounds__(256)
decode_merge_few_kernel(DecParams p) {
    const int n = blockIdx.y;
    const int head = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (head >= p.Hq) return;
    int base, L, vis_lo;
    seq_range(p, n, base, L, vis_lo);
    const int n_act = (L - vis_lo + p.chunk_keys - 1) / p.chunk_keys;
    if (n_act <= 1) return;  // finished by the split kernel
    const int lane = threadIdx.x & 63;
    const float* src = p.part + ((size_t)n * p.Hq + head) * p.n_splits * kPartStride;
    const float sink = p.sinks[head];
    float ms[kFewChunks], ls[kFewChunks], os[kFewChunks];
    float mtot = sink * kLog2e;
#pragma unroll
    for (int s = 0; s < kFewChunks; ++s) {
        if (s < n_act) {
            ms[s] = src[s * kPartStride + 64];
            ls[s] = src[s * kPartStride + 65];
            os[s] = src[s * kPartStride + lane];
            mtot = fmaxf(mtot, ms[s]);
        }
    }
    float l = sink == -INFINITY ? 0.0f : fast_exp2(sink * kLog2e - mtot);
    float o = 0.0f;
#pragma unroll
    for (int s = 0; s < kFewChunks; ++s) {
        if (s < n_act) {
            const float a = fast_exp2(ms[s] - mtot);
            l = fmaf(ls[s], a, l);
            o = fmaf(os[s], a, o);
        }
    }
    const __bf16 rb = (__bf16)(o / l);
    p.out[((size_t)n * p.Hq + head) * kHeadDim + lane] = __builtin_bit_cast(uint16_t, rb);
    if (lane == 0) p.lse[(size_t)n * p.Hq + head] = (mtot + fast_log2(l)) * kLn2;
}

// Many chunks: one workgroup per (sequence, head) with more than one chunk.  The
// block-wide maximum over the chunks' m (and the sink) comes first; then wave
// w sums chunks w, w + 4, ... with lane = d, and wave 0 adds the four sums.
__global__ void __launch_bounds__(256)
decode_merge_kernel(DecParams p) {
    __shared__ float red_o[4][64];
    __shared__ float red_x[4];
    const int head = blockIdx.x, n = blockIdx.y;
    int base, L, vis_lo;
    seq_range(p, n, base, L, vis_lo);
    const int n_act = (L - vis_lo + p.chunk_keys - 1) / p.chunk_keys;
    if (n_act <= 1) return;  // finished by the split kernel (uniform exit)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* src = p.part + ((size_t)n * p.Hq + head) * p.n_splits * kPartStride;
    const float sink = p.sinks[head];
    // maximum over the sink and every chunk's m (log2 units)
    float mx = sink * kLog2e;
    for (int s = tid; s < n_act; s += 256) mx = fmaxf(mx, src[s * kPartStride + 64]);
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if (lane == 0) red_x[wave] = mx;
    __syncthreads();
    const float mtot = fmaxf(fmaxf(red_x[0], red_x[1]), fmaxf(red_x[2], red_x[3]));
    __syncthreads();  // red_x is reused below
    float o = 0.0f, l = 0.0f;
#pragma unroll 4
    for (int s = wave; s < n_act; s += 4) {
        const float* c = src + s * kPartStride;
        const float a = fast_exp2(c[64] - mtot);
        o = fmaf(c[lane], a, o);
        l = fmaf(c[65], a, l);
    }
    red_o[wave][lane] = o;
    if (lane == 0) red_x[wave] = l;
    __syncthreads();
    if (wave != 0) return;
    o = (red_o[0][lane] + red_o[1][lane]) + (red_o[2][lane] + red_o[3][lane]);
    l = (red_x[0] + red_x[1]) + (red_x[2] + red_x[3]);
    if (sink != -INFINITY) l += fast_exp2(sink * kLog2e - mtot);
    const __bf16 rb = (__bf16)(o / l);
    p.out[((size_t)n * p.Hq + head) * kHeadDim + lane] = __builtin_bit_cast(uint16_t, rb);
    if (lane == 0) p.lse[(size_t)n * p.Hq + head] = (mtot + fast_log2(l)) * kLn2;
}

// Chunking plan: about one workgroup per CU over the whole grid.  A sequence
// is cut into chunks only when there are too few (sequence, KV-head group)
// pairs to fill the chip; every chunk but the last per sequence costs a
// partial write and read plus the merge launch, which on the 128 x 1024
// workload cost more than they gain.
struct ChunkPlan { int keys, n; };
ChunkPlan chunk_plan(int N, int Hkv, int G, int max_seqlen, int window) {
    const int vis = window > 0 ? std::min(max_seqlen, window) : max_seqlen;
    const long long groups = (long long)N * ((Hkv + kWaves - 1) / kWaves) * ((G + 31) / 32);
    const long long want = std::max(1LL, (kTargetWorkgroups + groups - 1) / groups);
    const int max_chunks = std::max(1, (vis + kTileKeys - 1) / kTileKeys);
    const int n = (int)std::min<long long>(want, max_chunks);
    int keys = (vis + n - 1) / n;
    keys = std::max(kTileKeys, (keys + kTileKeys - 1) / kTileKeys * kTileKeys);
    return ChunkPlan{keys, std::max(1, (vis + keys - 1) / keys)};
}

}  // namespace

size_t decode_workspace_bytes(int N, int Hq, int Hkv, int max_seqlen, int window) {
    const ChunkPlan cp = chunk_plan(N, Hkv, Hq / Hkv, max_seqlen, window);
    if (cp.n <= 1) return 0;
    return (size_t)N * Hq * cp.n * kPartStride * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    DecParams p;
    p.q = a.q;
    p.kc = a.k_cache;
    p.vc = a.v_cache;
    p.cu = a.cu_seqlens;
    p.sinks = a.sinks;
    p.out = a.out;
    p.lse = a.lse;
    p.part = static_cast<float*>(a.workspace);
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.window = a.window;
    p.max_seqlen = a.max_seqlen;
    const ChunkPlan cp = chunk_plan(a.N, a.Hkv, p.G, a.max_seqlen, a.window);
    p.n_splits = cp.n;
    p.chunk_keys = cp.keys;
    p.n_hblk = (p.G + 31) / 32;
    p.c = a.scale * kLog2e;
    p.bt = a.block_table;
    p.lens = a.seq_lens;
    p.rope = a.rope;
    p.ps_shift = 0;
    while (a.page_size > 0 && (1 << p.ps_shift) < a.page_size) ++p.ps_shift;
    p.ps_mask = a.page_size > 0 ? a.page_size - 1 : 0;
    p.pps = a.pages_per_seq;
    p.ring_mask = a.ring_tokens > 0 ? a.ring_tokens - 1 : 0x7fffffff;
    dim3 grid(p.n_splits, ((a.Hkv + kWaves - 1) / kWaves) * p.n_hblk, a.N);
    if (p.bt != nullptr)
        hipLaunchKernelGGL(decode_split_kernel<true>, grid, dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_split_kernel<false>, grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_splits == 1) return e;  // one chunk per sequence: nothing to merge
    if (p.n_splits <= kFewChunks)
        hipLaunchKernelGGL(decode_merge_few_kernel, dim3((a.Hq + 3) / 4, a.N), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_merge_kernel, dim3(a.Hq, a.N), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gptoss
