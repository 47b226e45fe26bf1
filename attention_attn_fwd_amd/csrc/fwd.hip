// Prefill forward of causal / sliding-window grouped-query attention with a
// per-head sink logit (gfx950).
//
// Method (Megatron-LM issue "gpt-oss implementation": "Attention Sinks",
// "Alternating Sliding-Window Attention Pattern"; HF blog "Tricks from OpenAI
// gpt-oss YOU can use with transformers": one fused kernel keeps the scores
// on chip; Flash Attention 3 with sinks): for each query row the softmax runs
// over the visible keys plus one sink logit that has no value vector.  The
// running max starts at the sink (in log2 units) and the running denominator
// at exp(0) = 1, so the sink enters exactly once and no score matrix ever
// reaches HBM.
//
// Work decomposition
//   One workgroup = 256 "columns".  A column is one (query position, query
//   head) pair; the G = Hq / Hkv heads of one KV head are packed next to each
//   other, so every K/V tile staged in LDS serves all G heads (GQA sharing)
//   and the workgroup covers floor(256 / G) positions.  Full-causal layers:
//   4 waves of 64 columns (kNb = 2 32-column MFMA N-blocks), two workgroups
//   per CU.  Sliding-window layers: 8 waves of 32 columns (at most 128
//   registers), two workgroups per CU, 4-5% faster there and the same on the
//   full-causal layer.  (4 waves of 32 columns at three workgroups per CU
//   ran 8% slower on the full-causal layer.)
//   Key tiles of 64 rows are staged HBM -> LDS with 16-byte coalesced loads,
//   double buffered, K and V both row-major (144-byte padded rows); the P.V
//   contraction over keys reads V^T through transposing LDS reads
//   (ds_read_b64_tr_b16), 8 consecutive keys per lane and MFMA slot group.
//   Only tiles that intersect the causal/window band are visited; inside a
//   wave, tiles fully outside its rows' band are skipped and tiles fully
//   inside it skip the mask (32-column waves decide that per 32-key half).
//
// Per key tile and wave (scores transposed, S^T = K Q^T, so that each lane
// holds one column's scores and the row reductions are in-lane):
//   S^T  : 2 (key blocks) x kNb (column blocks) x 4 (d steps) 32x32x16 bf16 MFMAs
//   mask, row max (in-lane + one permlane32 swap), lazy rescale of the output
//   accumulator (only when some row max grew), p = exp2(s * c - m) with
//   c = scale * log2(e), row sums kept per lane-half until the epilogue
//   O^T += V^T P^T : 2 (d blocks) x kNb (column blocks) x 4 (key steps) MFMAs;
//   the fp32 score accumulator converts in-register into the bf16 B operand.
// The key rows fed to the S^T MFMA are permuted (bits 2 and 3 of the row
// index swapped) so that accumulator registers 8h..8h+7 of lane half g hold
// the 8 consecutive keys 16 * (2 * block + h) + 8 g + 0..7 that the P.V MFMA
// expects in its B-operand slots.
#include "common.h"
#include "launch.h"

namespace gptoss {
namespace {

constexpr int kCols = 256;  // columns per workgroup (both layouts)
constexpr int kBk = 64;     // keys per LDS tile

struct FwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* sinks;
    uint16_t* out;
    float* lse;
    const int* cu;      // packed documents: sequence b = rows cu[b] .. cu[b+1]-1; nullptr = dense batch
    const float2* rope; // (cos, sin) table [position][32]: q rotated at load (k arrives rotated); nullptr = none
    int S, Hq, Hkv, G, window;  // S = sequence length (dense) or the longest document (packed)
    int T;              // total token rows (B * S when dense)
    int pos_per_block;  // positions per workgroup = floor(kCols / G)
    int n_qtiles;       // ceil(S / pos_per_block)
    int n_groups;       // B * Hkv
    int B;              // sequences (dense batch or packed documents)
    float c;            // softmax scale * log2(e)
};


// Lazy rescaling bound: a tile's probabilities are exponentiated against the
// running max m as long as every lane's tile sum stays below this bound
// (so every p <= 2^12); otherwise the tile is redone against its true max.
constexpr float kRescaleBound = 4096.0f;

// p = exp2(s * c - m) for the 32 scores of one column held by this lane
// (two 32-key blocks), packed into the bf16 B operands of the four 16-key
// P.V steps; returns the fp32 sum of the unrounded values (summing the bf16
// values would cost lse up to 2^-8 relative when one key dominates).
__device__ __forceinline__ float exp_pack(const f32x16& s0, const f32x16& s1, float c, float m, bf16x8* pb,
                                          int stride) {
    float la = 0.0f, lb = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const f32x16& sv = kk < 2 ? s0 : s1;
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 8 * (kk & 1) + 2 * j;
            const float e0 = fast_exp2(fmaf(sv[r], c, -m));
            const float e1 = fast_exp2(fmaf(sv[r + 1], c, -m));
            w[j] = pack_bf16x2(e0, e1);
            la += e0;
            lb += e1;
        }
        pb[kk * stride] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
    return la + lb;
}

// Workgroup -> (KV group, query tile).  Workgroups are dispatched round-robin
// over the 8 XCDs, so when the groups split evenly each XCD walks its own
// groups and their K/V stay in that XCD's L2.  Groups are numbered
// KV-head-major (group = kv_head * B + sequence), so with 8 KV heads each
// XCD takes one KV head of every sequence, which keeps the XCDs' work equal
// when packed documents differ in length.  Query tiles run heaviest (latest
// positions, most keys) first.
__device__ __forceinline__ void block_coords(const FwdParams& p, int bid, int& grp, int& qt) {
    const int nq = p.n_qtiles;
    if ((p.n_groups & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        const int gpx = p.n_groups >> 3;  // tile-major: heaviest tiles of all groups first
        grp = xcd * gpx + slot % gpx;
        qt = slot / gpx;
    } else {
        grp = bid % p.n_groups;
        qt = bid / p.n_groups;
    }
    qt = nq - 1 - qt;
}

// kWaves waves of kNb 32-column MFMA N-blocks each (kWaves * 32 * kNb =
// kCols); 64-column waves need up to 256 registers (two waves per SIMD),
// 32-column waves at most 128 (four).
template <int kWaves, int kNb>
__global__ void __launch_bounds__(64 * kWaves, kNb == 1 ? 4 : 2)
fwd_kernel(FwdParams p) {
    static_assert(kWaves * 32 * kNb == kCols, "a workgroup holds kCols columns");
    constexpr int kWaveCols = 32 * kNb;           // columns per wave
    constexpr int kThreads = 64 * kWaves;
    constexpr int kStRows = kThreads / 8;         // key rows staged per pass (8 threads per 128-byte row)
    constexpr int kStPasses = kBk / kStRows;      // passes per tile
    __shared__ uint4 smem[2][2][kTileUnits];  // [buffer][K | V][unit], both row-major

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the wave's tile tests are scalar
    const int g = lane >> 5;     // slot group / lane half
    const int l32 = lane & 31;

    int grp, qt;
    block_coords(p, blockIdx.x, grp, qt);
    const int kvh = grp / p.B, b = grp % p.B;  // KV-head-major groups
    const int G = p.G;
    const SeqRows sr = seq_rows(p.cu, p.S, p.Hq, p.T, b);
    const int S = sr.len;  // positions of this sequence
    const int W = p.window;
    const unsigned Weff = W > 0 ? (unsigned)W : 0x7fffffffu;
    const int p0 = qt * p.pos_per_block;
    if (p0 >= S) return;  // a document shorter than the longest one
    const int used_cols = p.pos_per_block * G;
    const int P1 = min(p0 + p.pos_per_block, S) - 1;

    // ---- this lane's two columns (one per N-block)
    int col_pos[kNb], col_head[kNb];
    bool col_ok[kNb];
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) {
        const int cw = wave * kWaveCols + nb * 32 + l32;
        col_pos[nb] = p0 + cw / G;
        col_head[nb] = kvh * G + cw % G;
        col_ok[nb] = cw < used_cols && col_pos[nb] < S;
    }
    // positions covered by this wave (for tile classification)
    const int wc0 = wave * kWaveCols;
    const bool wave_active = wc0 < used_cols && p0 + wc0 / G < S;
    const int wpmin = p0 + wc0 / G;
    const int wpmax = min(p0 + (min(wc0 + kWaveCols - 1, used_cols - 1)) / G, S - 1);

    // ---- Q fragments (B operand of S^T = K Q^T): column n, d = 16ks + 8g + 0..7
    uint4 qraw[kNb][4];
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) {
        const uint16_t* qrow = p.q + ((size_t)(sr.row0 + col_pos[nb]) * p.Hq + col_head[nb]) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            qraw[nb][ks] = make_uint4(0, 0, 0, 0);
            if (col_ok[nb]) qraw[nb][ks] = ld16(qrow + 16 * ks + 8 * g);
        }
    }
    // rotary table entries of this lane's q elements (pairs d, d + 32 are
    // fragments ks and ks + 2), loaded before the first K/V tile so that the
    // rotation waits only for them and the q loads
    float4 rcs[kNb][2][4];
    const bool rope = p.rope != nullptr;
    if (rope) {
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (col_ok[nb]) {
                    load_rope8(p.rope, col_pos[nb], 16 * ks + 8 * g, rcs[nb][ks]);
                } else {
#pragma unroll
                    for (int u = 0; u < 4; ++u) rcs[nb][ks][u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                }
            }
    }

    // ---- softmax state, seeded by the sink: m = sink * log2(e), l = 1
    float m_run[kNb], l_run[kNb];
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) {
        // (a padding column -- no query row -- starts at m = 0: its scores are
        // finite and its results are never stored)
        const float sink = col_ok[nb] ? p.sinks[col_head[nb]] : 0.0f;
        const bool has_sink = sink != -INFINITY;
        m_run[nb] = has_sink ? sink * kLog2e : -INFINITY;
        l_run[nb] = (has_sink && g == 0 && col_ok[nb]) ? 1.0f : 0.0f;
    }
    f32x16 oacc[2][kNb];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][nb][r] = 0.0f;

    // ---- key tile range of the workgroup
    const int key_lo = W > 0 ? max(0, p0 - W + 1) : 0;
    const int t_begin = key_lo / kBk;
    const int t_end = P1 / kBk;  // inclusive

    // global -> register staging of one K/V tile
    const uint32_t kv_row_stride = (uint32_t)p.Hkv * kHeadDim;
    const uint16_t* kbase = p.k + ((size_t)sr.row0 * p.Hkv + kvh) * kHeadDim;
    const uint16_t* vbase = p.v + ((size_t)sr.row0 * p.Hkv + kvh) * kHeadDim;
    const int st_key = tid >> 3, st_unit = tid & 7;  // rows st_key + kStRows j; 16-byte unit
    uint4 kreg[kStPasses], vreg[kStPasses];

    // Rows past the sequence end re-read its last row: no valid query row can
    // see them (they lie past every position), and the tile that holds them
    // is an edge tile, whose scores are masked.
    auto load_tile = [&](int t) {
        const int kt0 = t * kBk;
#pragma unroll
        for (int j = 0; j < kStPasses; ++j) {
            const int key = min(kt0 + st_key + kStRows * j, S - 1);
            kreg[j] = ld16(kbase + row_off(key, kv_row_stride) + 8 * st_unit);
            vreg[j] = ld16(vbase + row_off(key, kv_row_stride) + 8 * st_unit);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kStPasses; ++j) {
            smem[buf][0][tile_unit(st_key + kStRows * j, st_unit)] = kreg[j];
            smem[buf][1][tile_unit(st_key + kStRows * j, st_unit)] = vreg[j];
        }
    };

    if (t_begin <= t_end) load_tile(t_begin);
    if (rope) {
        bool mid = false;
#pragma unroll
        for (int nb = 0; nb < kNb; ++nb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) mid = rope8(qraw[nb][ks], qraw[nb][ks + 2], rcs[nb][ks]) || mid;
        if (__any(mid)) {
            // (rare) an fp64 sum on a bf16 midpoint: reload q and its table
            // entries and rotate with exact remainders
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) {
                if (!col_ok[nb]) continue;
                const uint16_t* qrow = p.q + ((size_t)(sr.row0 + col_pos[nb]) * p.Hq + col_head[nb]) * kHeadDim;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint4 x0 = ld16(qrow + 16 * ks + 8 * g), x1 = ld16(qrow + 16 * (ks + 2) + 8 * g);
                    float4 cs[4];
                    load_rope8(p.rope, col_pos[nb], 16 * ks + 8 * g, cs);
                    rope8_exact(x0, x1, cs);
                    qraw[nb][ks] = x0;
                    qraw[nb][ks + 2] = x1;
                }
            }
        }
    }
    bf16x8 qf[kNb][4];
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qf[nb][ks] = as_bf16x8(qraw[nb][ks]);
    if (t_begin <= t_end) store_tile(0);
    __syncthreads();

    // The tile in which each of this lane's rows first sees a key (with W = 0
    // every row sees key 0, in tile t_begin = 0), and whether any row of the
    // wave can still sit at m = -inf (a sink of -inf) before that tile.
    int first_tile[kNb];
    bool ninf = false;
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) {
        first_tile[nb] = W > 0 ? max(0, col_pos[nb] - W + 1) / kBk : 0;
        ninf = ninf || m_run[nb] == -INFINITY;
    }
    const bool any_ninf = __any(ninf);
    for (int t = t_begin; t <= t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        const bool has_next = t < t_end;
        if (has_next) load_tile(t + 1);

        const int kt0 = t * kBk;
        const bool skip = !wave_active || kt0 > wpmax || (W > 0 && wpmin - (kt0 + kBk - 1) >= W);
        if (!skip) {
            const bool need_mask = !(kt0 + kBk - 1 <= wpmin && (W == 0 || wpmax - kt0 < W));
            // Within an edge tile, 32-column waves skip the mask of a 32-key
            // block that every row of the wave sees whole (about 1% faster on
            // the sliding layer); 64-column waves mask whole tiles (the per-block
            // branch changed how the compiler interleaves the two blocks and
            // cost the full-causal layer 2%).
            bool block_mask[2];
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                const int kb0 = kt0 + 32 * mb;
                block_mask[mb] = !(kb0 + 31 <= wpmin && (W == 0 || wpmax - kb0 < W));
            }
            const uint4* ks = smem[buf][0];
            const uint4* vs = smem[buf][1];

            // S^T = K Q^T for the tile, masked on edge tiles.  Register r of
            // key block mb holds key kt0 + 32 mb + 16 (r / 8) + 8 g + r % 8;
            // it is visible iff 0 <= pos - key < Weff (one unsigned compare).
            auto scores = [&](f32x16 (&sacc)[2][kNb]) {
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < kNb; ++nb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) sacc[mb][nb][r] = 0.0f;
#pragma unroll
                for (int ks_ = 0; ks_ < 4; ++ks_) {
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb) {
                        const int key = 32 * mb + perm_row(l32);
                        const bf16x8 a = as_bf16x8(ks[tile_unit(key, 2 * ks_ + g)]);
#pragma unroll
                        for (int nb = 0; nb < kNb; ++nb) sacc[mb][nb] = mfma32(a, qf[nb][ks_], sacc[mb][nb]);
                    }
                }
                if (need_mask) {
#pragma unroll
                    for (int nb = 0; nb < kNb; ++nb) {
                        const int dd = col_pos[nb] - kt0 - 8 * g;
#pragma unroll
                        for (int mb = 0; mb < 2; ++mb) {
                            if constexpr (kNb == 1) {
                                if (!block_mask[mb]) continue;  // wave-uniform
                            }
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const int cr = 32 * mb + 16 * (r >> 3) + (r & 7);
                                const bool vis = (unsigned)(dd - cr) < Weff;
                                sacc[mb][nb][r] = vis ? sacc[mb][nb][r] : -INFINITY;
                            }
                        }
                    }
                }
            };

            // Online softmax (log2 domain), one column per lane pair.  Fast
            // path: exponentiate against the running max.  Slow path (the
            // first tile in which some row sees keys, a row still at -inf, or
            // a tile sum above the bound): scores against the true row max,
            // rescale.  A row's first tile always takes the exact path so the
            // dominant key of a short row gets p = 1 exactly (no bf16
            // rounding on it).
            bf16x8 pb[4][kNb];
            float lt[kNb];
            bool first = false, at_ninf = false;
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) {
                lt[nb] = 0.0f;
                first = first || first_tile[nb] == t;
                at_ninf = at_ninf || m_run[nb] == -INFINITY;
            }
            bool slow = W > 0 ? __any(first) : t == t_begin;
            if (any_ninf) slow = slow || __any(at_ninf);
            if (!slow) {
                f32x16 sacc[2][kNb];
                scores(sacc);
                bool big = false;
#pragma unroll
                for (int nb = 0; nb < kNb; ++nb) {
                    lt[nb] = exp_pack(sacc[0][nb], sacc[1][nb], p.c, m_run[nb], &pb[0][nb], kNb);
                    big = big || lt[nb] > kRescaleBound;
                }
                slow = __any(big);
            }
            if (slow) {
                f32x16 sacc[2][kNb];
                scores(sacc);
                float alpha[kNb];
                bool grow = false;
#pragma unroll
                for (int nb = 0; nb < kNb; ++nb) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[mb][nb][r]);
                    mx = max_across_halves(mx);
                    const float m_new = fmaxf(m_run[nb], mx * p.c);
                    alpha[nb] = m_new > m_run[nb] ? fast_exp2(m_run[nb] - m_new) : 1.0f;
                    grow |= m_new > m_run[nb];
                    m_run[nb] = m_new;
                }
                if (__any(grow)) {
#pragma unroll
                    for (int nb = 0; nb < kNb; ++nb) {
                        l_run[nb] *= alpha[nb];
#pragma unroll
                        for (int db = 0; db < 2; ++db)
#pragma unroll
                            for (int r = 0; r < 16; ++r) oacc[db][nb][r] *= alpha[nb];
                    }
                }
#pragma unroll
                for (int nb = 0; nb < kNb; ++nb) {
                    const float m_use = m_run[nb] == -INFINITY ? 0.0f : m_run[nb];
                    lt[nb] = exp_pack(sacc[0][nb], sacc[1][nb], p.c, m_use, &pb[0][nb], kNb);
                }
            }
#pragma unroll
            for (int nb = 0; nb < kNb; ++nb) l_run[nb] += lt[nb];

            // O^T += V^T P^T
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    // V^T rows d = 32 db + l32, keys 16 kk + 8 g + 0..7 (transposing read)
                    const bf16x8 a = tile_read_tr8(vs, 16 * kk + 8 * g, 32 * db + 16 * (l32 >> 4), l32 & 15);
#pragma unroll
                    for (int nb = 0; nb < kNb; ++nb) oacc[db][nb] = mfma32(a, pb[kk][nb], oacc[db][nb]);
                }
            }
        }

        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = acc / l (bf16, RNE); lse = ln2 * (m + log2 l)
#pragma unroll
    for (int nb = 0; nb < kNb; ++nb) {
        const float l_tot = sum_across_halves(l_run[nb]);
        if (!col_ok[nb]) continue;
        const float inv = 1.0f / l_tot;
        uint16_t* orow = p.out + ((size_t)(sr.row0 + col_pos[nb]) * p.Hq + col_head[nb]) * kHeadDim;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d0 = 32 * db + 8 * r4 + 4 * g;
                uint2 w;
                w.x = pack_bf16x2(oacc[db][nb][4 * r4 + 0] * inv, oacc[db][nb][4 * r4 + 1] * inv);
                w.y = pack_bf16x2(oacc[db][nb][4 * r4 + 2] * inv, oacc[db][nb][4 * r4 + 3] * inv);
                *reinterpret_cast<uint2*>(orow + d0) = w;
            }
        if (g == 0)
            p.lse[sr.lse_base + col_head[nb] * sr.lse_hstride + col_pos[nb]] = (m_run[nb] + fast_log2(l_tot)) * kLn2;
    }
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
    FwdParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.sinks = a.sinks;
    p.out = a.out;
    p.lse = a.lse;
    p.cu = a.cu;
    p.rope = a.rope;
    p.S = a.S;
    p.T = a.T;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.window = a.window >= a.S ? 0 : a.window;
    static_assert(kCols >= 128, "a workgroup holds at least one position of the largest group (128 heads)");
    p.pos_per_block = kCols / p.G;
    p.n_qtiles = (a.S + p.pos_per_block - 1) / p.pos_per_block;
    p.n_groups = a.B * a.Hkv;
    p.B = a.B;
    p.c = a.scale * kLog2e;
    const long long blocks = (long long)p.n_groups * p.n_qtiles;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // the sliding layer (three key tiles per workgroup, mostly edge tiles)
    // runs 4-5% faster with 32-column waves; the full-causal layer runs the
    // same with either and takes the 64-column layout
    if (p.window > 0)
        hipLaunchKernelGGL((fwd_kernel<8, 1>), dim3((unsigned)blocks), dim3(512), 0, stream, p);
    else
        hipLaunchKernelGGL((fwd_kernel<4, 2>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gptoss
