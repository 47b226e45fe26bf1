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
//   split kernel : grid (chunk of visible keys, block of 2 KV heads -- 4 for
//     windows of at most 256 keys -- x head block, sequence); chunks are only
//     cut when too few (sequence, block) pairs would fill the chip, and with
//     two-head blocks, one chunk per sequence and at most 256 sequences the
//     workgroups take their items in a length-ranked order (below).  Each wave owns one KV
//     head, so the waves of a workgroup stream adjacent 128-byte rows of the
//     same tokens.  A wave walks its chunk in 64-key tiles: whole K and V
//     rows (8 lanes per 128-byte row, non-temporal loads) go through
//     wave-private LDS tiles, K read back as MFMA A operands and V
//     transposed, S^T = K Q^T and O^T = V^T P^T on 32x32x16 bf16 MFMAs with
//     the G query heads as columns, an online softmax across tiles, and the
//     next tile's loads in flight while the current one is computed.  Waves
//     synchronise only in the ranking prologue.  A sequence that fits in one
//     chunk is finished in place (sink folded in, out and lse written);
//     otherwise the wave writes one partial (unnormalised O, running max m in
//     log2 units, sum l) per head.
//   merge kernels (one wave per (sequence, head) when there are at most 16
//     chunks, one workgroup per (sequence, head) otherwise):
//     m = max(sink, m_s), l = 2^(sink - m) + sum l_s 2^(m_s - m),
//     out = sum O_s 2^(m_s - m) / l, lse = ln2 (m + log2 l).  The sink enters
//     here exactly once.
#include "common.h"
#include "launch.h"

#include <algorithm>
#include <mutex>

namespace gptoss {
namespace {

constexpr int kTileKeys = kDecodeKeyTile;  // keys per wave step
constexpr int kPartStride = kDecodePartStride;

}  // namespace

// (Named, not file-local: this file and the paged-cache unit that includes
// it pass it to each other.)
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
    uint32_t page_bytes;  // paged cache: bytes per page (page_size * Hkv * 128; below 2^32 where used)
    int ranked;       // one chunk per sequence, N <= kDecodeRankMaxSeqs: items in ranked order
    float c;          // scale * log2(e)
};

// The paged-cache instantiations of the split kernel (kPaged = 1, 2, 3) are
// compiled in a unit of their own (decode_paged.hip, which includes this
// file with GPTOSS_DECODE_PAGED_UNIT defined), so that the build can give
// the packed-cache kernel and them different instruction schedulers.
hipError_t launch_decode_split_paged(const DecParams& p, int mode, int kv_per_block, dim3 grid,
                                     hipStream_t stream);

namespace {

// K/V rows are read once per call: non-temporal loads (the hint that lets
// the caches evict them first) stream 10-12% faster than plain ones, both
// where one CU's outstanding loads bound the rate and where HBM does.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

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
// workgroups per CU, and so did two waves per KV head taking alternate
// tiles; two waves per KV head taking contiguous halves, merged through LDS,
// ran 34.2 against 32.6 us on the 128 x U{1..1024} workload.)
// kPaged != 0: K/V rows are found through the block table (slot = position &
// ring_mask, page = bt[n][slot >> ps_shift], row = slot & ps_mask); the page
// indices of a tile are loaded one tile ahead of its K/V rows.
//   kPaged == 1 (pages of 1-4 tokens, or of 2^32 bytes or more): every lane
//     loads the page of each of its 8 rows (8 vector loads per tile).
//   kPaged == 2 (pages of 8 or more tokens, page bytes below 2^32, a
//     window): the rows a lane group reads in step j are 8 consecutive
//     positions, which cross at most one page boundary (the ring, a multiple
//     of the page size, wraps only at one), so the wave needs two page
//     indices per step, both wave-uniform: scalar loads, which leave the
//     vector memory path to the K/V rows; each lane picks its page and forms
//     its 64-bit row address.
//   kPaged == 3 (the same pages, no window): every chunk starts on an 8-row
//     boundary, so a step never crosses a page: one page index per step and
//     a uniform page base plus a 32-bit offset within the page.  (A kernel
//     holding both this path and the per-lane one ran 13% slower on the full
//     layer than this path alone, even where it never took the other.)
template <int kPaged, int kWaves>
__global__ void __launch_bounds__(64 * kWaves, 2)
decode_split_kernel(DecParams p) {
    constexpr int kThreads = 64 * kWaves;  // kWaves KV heads per workgroup, one per wave
    __shared__ uint4 ksm[kWaves][kTileUnits];  // one row-major K tile per wave
    __shared__ uint4 vsm[kWaves][kTileUnits];  // one row-major V tile per wave

    const int chunk = blockIdx.x;
    int item_y = blockIdx.y, n = blockIdx.z;
    int base, L, vis_lo;
    if (p.ranked) {
        // One CU streams a few tens of GB/s at most, so the workgroups that
        // hold the longest sequences set the time unless every CU gets an
        // even share.  Workgroups start in id order and the first half of the
        // ids fills the CUs once, so the items (sequence, head block) go out
        // longest first over the first half and shortest first over the
        // second: each CU pairs a long item with a short one.  The workgroup
        // ranks the sequences itself, all workgroups alike, by a unique key:
        // visible tiles (capped at 2^23), then lower index first.
        static_assert(kDecodeRankMaxSeqs <= 2 * kThreads && kDecodeRankMaxSeqs <= 256, "two candidates a thread");
        __shared__ uint4 s_key[kDecodeRankMaxSeqs / 4];
        __shared__ int s_pick[4];  // sequence, base, L, vis_lo
        const int N = gridDim.z, N4 = (N + 3) / 4;
        const int Y = gridDim.y, ni = Y * N, id = blockIdx.y + Y * blockIdx.z, half = ni / 2;
        const int r = id < half ? id : ni - 1 - (id - half);
        const int want = r / Y;  // rank of this item's sequence
        item_y = r % Y;
        uint32_t key[2];
        int b_c[2], L_c[2], lo_c[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int i = threadIdx.x + kThreads * c;
            key[c] = 0;  // below every real key (pads the last uint4)
            if (i < N) {
                seq_range(p, i, b_c[c], L_c[c], lo_c[c]);
                const uint32_t tiles = min((uint32_t)(L_c[c] - lo_c[c] + kTileKeys - 1) / kTileKeys, 1u << 23);
                key[c] = ((tiles + 1) << 8) | (uint32_t)(255 - i);
            }
            if (i < 4 * N4) reinterpret_cast<uint32_t*>(s_key)[i] = key[c];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int i = threadIdx.x + kThreads * c;
            if (i < N) {
                int rank = 0;
#pragma unroll 4
                for (int j = 0; j < N4; ++j) {
                    const uint4 u = s_key[j];
                    rank += (u.x > key[c]) + (u.y > key[c]) + (u.z > key[c]) + (u.w > key[c]);
                }
                if (rank == want) {
                    s_pick[0] = i;
                    s_pick[1] = b_c[c];
                    s_pick[2] = L_c[c];
                    s_pick[3] = lo_c[c];
                }
            }
        }
        __syncthreads();
        n = s_pick[0];
        base = s_pick[1];
        L = s_pick[2];
        vis_lo = s_pick[3];
    } else {
        seq_range(p, n, base, L, vis_lo);
    }
    const int kvg = item_y / p.n_hblk;
    const int hb = item_y % p.n_hblk;
    const int n_vis = L - vis_lo;
    const int n_act = (n_vis + p.chunk_keys - 1) / p.chunk_keys;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int* bt_row = kPaged != 0 ? p.bt + (size_t)n * p.pps : nullptr;

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
    int pid[8];  // kPaged == 1: page of each of this lane's 8 rows of the next tile to load
    // kPaged >= 2 (wave-uniform): page indices of step j's first and (mode 2)
    // last rows, and (mode 2) how many of its 8 rows lie in the first one
    int pg_first[8], pg_last[8], cut[8];
    auto tile_key = [&](int t, int j) { return min(c0 + t * kTileKeys + (lane >> 3) + 8 * j, c1 - 1); };
    // packed cache: one uniform base address per tile (scalar arithmetic) and
    // 32-bit per-lane offsets, so a row pair's loads need one clamp (the row
    // offsets of a tile stay below 2^32: the entry points bound Hkv through
    // the grid size); the paged path's 32-bit offsets are bounded where taken
    const uint32_t row_bytes = (uint32_t)p.Hkv * kHeadDim * 2;
    const uint32_t unit_off = 16u * (lane & 7);
    const uint32_t lane_off = (uint32_t)(lane >> 3) * row_bytes + unit_off;
    auto load_pids = [&](int t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (kPaged == 3) {
                // steps start on 8-row boundaries: one page per step
                const __attribute__((address_space(4))) int* btc =
                    (const __attribute__((address_space(4))) int*)bt_row;
                const int k0 = __builtin_amdgcn_readfirstlane(min(c0 + t * kTileKeys + 8 * j, c1 - 1));
                pg_first[j] = btc[(k0 & p.ring_mask) >> p.ps_shift];
            } else if (kPaged == 2) {
                // the table through the constant address space: scalar loads
                const __attribute__((address_space(4))) int* btc =
                    (const __attribute__((address_space(4))) int*)bt_row;
                const int kb0 = __builtin_amdgcn_readfirstlane(c0 + t * kTileKeys + 8 * j);
                const int k0 = min(kb0, c1 - 1), k7 = min(kb0 + 7, c1 - 1);
                pg_first[j] = btc[(k0 & p.ring_mask) >> p.ps_shift];
                pg_last[j] = btc[(k7 & p.ring_mask) >> p.ps_shift];
                // rows past the chunk end repeat row c1 - 1, which lies in
                // the page of k7
                cut[j] = kb0 > c1 - 1 ? 8 : min(8, (p.ps_mask + 1) - (kb0 & p.ps_mask));
            } else {
                pid[j] = bt_row[(tile_key(t, j) & p.ring_mask) >> p.ps_shift];
            }
        }
    };
    auto load_tile = [&](int t) {
        if (kPaged == 0) {
            const int t0 = c0 + t * kTileKeys;
            const char* kt = reinterpret_cast<const char*>(kb) + (size_t)t0 * row_bytes;
            const char* vt = reinterpret_cast<const char*>(vb) + (size_t)t0 * row_bytes;
            const uint32_t lim = (uint32_t)(c1 - 1 - t0) * row_bytes + unit_off;  // the chunk's last row
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t off = min(lane_off + (uint32_t)(8 * j) * row_bytes, lim);
                kr[j] = ld16_stream(kt + off);
                vr[j] = ld16_stream(vt + off);
            }
            return;
        }
        if (kPaged == 3) {
            // every step within one page: a uniform page base per step
            // (scalar arithmetic) plus a 32-bit offset within the page (a
            // slot is below 2^16 and a row below 2^24 bytes: the entry points
            // bound Hkv, so the 24-bit multiply is exact; the launcher takes
            // this path only for pages below 2^32 bytes)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const size_t page_off = (size_t)(uint32_t)pg_first[j] * p.page_bytes;
                const uint32_t in_page = __umul24((uint32_t)(tile_key(t, j) & p.ring_mask & p.ps_mask), row_bytes) + unit_off;
                kr[j] = ld16_stream(reinterpret_cast<const char*>(kb) + page_off + in_page);
                vr[j] = ld16_stream(reinterpret_cast<const char*>(vb) + page_off + in_page);
            }
            return;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = tile_key(t, j);
            int page;
            if (kPaged == 1) page = pid[j];
            else page = (lane >> 3) < cut[j] ? pg_first[j] : pg_last[j];
            const size_t row = ((size_t)page << p.ps_shift) + (size_t)(key & p.ring_mask & p.ps_mask);
            kr[j] = ld16_stream(kb + row * row_stride + 8 * (lane & 7));
            vr[j] = ld16_stream(vb + row * row_stride + 8 * (lane & 7));
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 oacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;

    if (kPaged != 0) {
        load_pids(0);
        load_tile(0);
        if (n_tiles > 1) load_pids(1);
    } else {
        load_tile(0);  // n_tiles >= 1 here
    }
    if (p.rope != nullptr) {
        bool mid = false;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) mid = rope8(qraw[ks], qraw[ks + 2], rcs[ks]) || mid;
        if (__any(mid) && col_ok) {
            // (rare) an fp64 sum on a bf16 midpoint: reload q and its table
            // entries and rotate with exact remainders
            const uint16_t* qrow = p.q + ((size_t)n * p.Hq + head) * kHeadDim;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint4 x0 = ld16(qrow + 16 * ks + 8 * g), x1 = ld16(qrow + 16 * (ks + 2) + 8 * g);
                float4 cs[4];
                load_rope8(p.rope, L - 1, 16 * ks + 8 * g, cs);
                rope8_exact(x0, x1, cs);
                qraw[ks] = x0;
                qraw[ks + 2] = x1;
            }
        }
    }
    bf16x8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(qraw[ks]);
    for (int t = 0; t < n_tiles; ++t) {
        // kPaged >= 2: the next tile's page indices (scalar loads issued at
        // the end of the previous iteration) share the LDS counter; waiting
        // for them here, before this tile's LDS writes, keeps the wait that
        // their use needs from also waiting for those writes
        if (kPaged >= 2) __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
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
            if (kPaged == 1 && t + 2 < n_tiles) load_pids(t + 2);
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
        // kPaged >= 2: the page indices of tile t + 2 are loaded after this
        // tile's last LDS read, so that they arrive while the next iteration
        // waits for the K/V loads of tile t + 1 (scalar loads count with the
        // LDS operations, and every LDS wait issued while they are in flight
        // would wait for them too)
        if (kPaged >= 2) {
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (t + 2 < n_tiles) load_pids(t + 2);
        }
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

#ifndef GPTOSS_DECODE_PAGED_UNIT
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

// Many chunks: one workgroup per (sequence, head) with more than one chunk.
// Wave w merges chunks w, w + 4, ... online (lane = d; running maximum and
// rescale, so the loads of several chunks are in flight at once and the
// partials are read in one pass), then wave 0 merges the four waves' (m, l,
// O) with the sink.
__global__ void __launch_bounds__(256)
decode_merge_kernel(DecParams p) {
    __shared__ float red_o[4][64];
    __shared__ float red_m[4], red_l[4];
    const int head = blockIdx.x, n = blockIdx.y;
    int base, L, vis_lo;
    seq_range(p, n, base, L, vis_lo);
    const int n_act = (L - vis_lo + p.chunk_keys - 1) / p.chunk_keys;
    if (n_act <= 1) return;  // finished by the split kernel (uniform exit)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* src = p.part + ((size_t)n * p.Hq + head) * p.n_splits * kPartStride;
    const float sink = p.sinks[head];
    // every chunk holds a visible key, so its m is finite; a wave without
    // chunks keeps m = -inf, l = 0, O = 0 and adds nothing below
    float m = -INFINITY, l = 0.0f, o = 0.0f;
#pragma unroll 8
    for (int s = wave; s < n_act; s += 4) {
        const float* c = src + s * kPartStride;
        const float ms = c[64], ls = c[65], os = c[lane];
        const float mn = fmaxf(m, ms);
        const float a = fast_exp2(m - mn), b = fast_exp2(ms - mn);
        l = fmaf(l, a, ls * b);
        o = fmaf(o, a, os * b);
        m = mn;
    }
    red_o[wave][lane] = o;
    if (lane == 0) {
        red_m[wave] = m;
        red_l[wave] = l;
    }
    __syncthreads();
    if (wave != 0) return;
    const float s2 = sink * kLog2e;
    const float mtot = fmaxf(fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3])), s2);
    float lt = sink == -INFINITY ? 0.0f : fast_exp2(s2 - mtot), ot = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float a = fast_exp2(red_m[w] - mtot);
        lt = fmaf(red_l[w], a, lt);
        ot = fmaf(red_o[w][lane], a, ot);
    }
    const __bf16 rb = (__bf16)(ot / lt);
    p.out[((size_t)n * p.Hq + head) * kHeadDim + lane] = __builtin_bit_cast(uint16_t, rb);
    if (lane == 0) p.lse[(size_t)n * p.Hq + head] = (mtot + fast_log2(lt)) * kLn2;
}
#endif  // GPTOSS_DECODE_PAGED_UNIT

}  // namespace

#ifdef GPTOSS_DECODE_PAGED_UNIT
hipError_t launch_decode_split_paged(const DecParams& p, int mode, int kv_per_block, dim3 grid,
                                     hipStream_t stream) {
    if (kv_per_block == 2) {
        const dim3 block(128);
        if (mode == 3) hipLaunchKernelGGL((decode_split_kernel<3, 2>), grid, block, 0, stream, p);
        else if (mode == 2) hipLaunchKernelGGL((decode_split_kernel<2, 2>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<1, 2>), grid, block, 0, stream, p);
    } else {
        const dim3 block(256);
        if (mode == 3) hipLaunchKernelGGL((decode_split_kernel<3, 4>), grid, block, 0, stream, p);
        else if (mode == 2) hipLaunchKernelGGL((decode_split_kernel<2, 4>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<1, 4>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}
#else
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
    const DecodePlan cp = decode_plan(a.N, a.Hq, a.Hkv, a.max_seqlen, a.window);
    // every visible key of the longest allowed sequence lies in some chunk
    const long long vis = a.window > 0 ? std::min(a.max_seqlen, a.window) : a.max_seqlen;
    if (cp.chunk_keys < kTileKeys || (long long)cp.chunk_keys * cp.n_splits < vis) return hipErrorInvalidValue;
    if (cp.n_splits > 1 && a.workspace == nullptr) return hipErrorInvalidValue;
    p.n_splits = cp.n_splits;
    p.chunk_keys = cp.chunk_keys;
    p.n_hblk = (p.G + 31) / 32;
    p.ranked = decode_kv_per_block(a.window) == 2 && cp.n_splits == 1 && a.N <= kDecodeRankMaxSeqs;
    p.c = a.scale * kLog2e;
    p.bt = a.block_table;
    p.lens = a.seq_lens;
    p.rope = a.rope;
    p.ps_shift = 0;
    while (a.page_size > 0 && (1 << p.ps_shift) < a.page_size) ++p.ps_shift;
    p.ps_mask = a.page_size > 0 ? a.page_size - 1 : 0;
    p.pps = a.pages_per_seq;
    p.ring_mask = a.ring_tokens > 0 ? a.ring_tokens - 1 : 0x7fffffff;

    const int kvpb = decode_kv_per_block(a.window);
    dim3 grid(p.n_splits, ((a.Hkv + kvpb - 1) / kvpb) * p.n_hblk, a.N);
    // pages of 8+ tokens whose byte size fits 32 bits take the wave-uniform
    // page paths; without a window every chunk starts on an 8-row boundary,
    // so no load step crosses a page (mode 3)
    const long long page_bytes = (long long)a.page_size * a.Hkv * kHeadDim * 2;
    const bool uniform_pages = p.ps_shift >= 3 && page_bytes < (1LL << 32);
    p.page_bytes = uniform_pages ? (uint32_t)page_bytes : 0u;
    const int mode = p.bt == nullptr ? 0 : !uniform_pages ? 1 : p.window == 0 ? 3 : 2;
    hipError_t e;
    if (mode != 0) {
        e = launch_decode_split_paged(p, mode, kvpb, grid, stream);
    } else {
        if (kvpb == 2) hipLaunchKernelGGL((decode_split_kernel<0, 2>), grid, dim3(128), 0, stream, p);
        else hipLaunchKernelGGL((decode_split_kernel<0, 4>), grid, dim3(256), 0, stream, p);
        e = hipGetLastError();
    }
    if (e != hipSuccess || p.n_splits == 1) return e;  // one chunk per sequence: nothing to merge
    if (p.n_splits <= kFewChunks)
        hipLaunchKernelGGL(decode_merge_few_kernel, dim3((a.Hq + 3) / 4, a.N), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(decode_merge_kernel, dim3(a.Hq, a.N), dim3(256), 0, stream, p);
    return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops).  The split
// partials live in this file-scope array instead: every GPU holds its own
// copy for the life of the process, and every call on that GPU shares it
// (calls that may overlap on one GPU race on it).  The kernels overwrite
// every partial they read in the same call, so nothing needs clearing.
namespace {

static __device__ __align__(256) float scratch[kDecodeNoAllocScratchBytes / sizeof(float)];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of this GPU's scratch array, looked up once per device
// with that device current (the array's name in host code is only a
// stand-in for the symbol, not an address a kernel may use).
hipError_t scratch_for_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode_noalloc(const DecodeArgs& args, hipStream_t stream) {
    const DecodePlan cp = decode_plan(args.N, args.Hq, args.Hkv, args.max_seqlen, args.window);
    if (cp.workspace_bytes > kDecodeNoAllocScratchBytes) return hipErrorInvalidValue;  // checked by the caller
    DecodeArgs a = args;
    a.workspace = nullptr;
    if (cp.workspace_bytes > 0) {
        const hipError_t e = scratch_for_current_device(&a.workspace);
        if (e != hipSuccess) return e;
    }
    return launch_decode(a, stream);
}

#endif  // GPTOSS_DECODE_PAGED_UNIT

}  // namespace gptoss
