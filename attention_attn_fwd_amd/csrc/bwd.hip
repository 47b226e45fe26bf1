// Training backward of grouped-query sink attention (gfx950).
//
// Loss L = sum(dout * out).  With P_ij = exp(s_ij - lse_i) (lse includes the
// sink, so P is the exact softmax probability) and Dvec_i = <dout_i, out_i>:
//   dS_ij   = P_ij (<dout_i, v_j> - Dvec_i)
//   dq_i    = scale sum_j dS_ij k_j
//   dk_j    = scale sum_{h in group} sum_i dS_ij q_i
//   dv_j    = sum_{h in group} sum_i P_ij dout_i
//   dsink_h = -sum_{b,i} exp(sink_h - lse_i) Dvec_i
// (the sink's value vector is zero, so its score gradient is
// P_sink (0 - Dvec); Megatron-LM issue "gpt-oss implementation", "Attention
// Sinks", names the feature; the pages give no formula.)
//
// Three launches on the caller's stream (dq, dkdv, dsink), no atomics,
// deterministic:
//   dq     : query-outer, like the forward: S^T = K Q^T and dP^T = V dO^T
//            put one column per lane, which is the operand layout of
//            dQ^T += K^T dS^T (K^T through transposing LDS reads).  Each
//            row's Dvec = <dout, out> is formed in its prologue and stored
//            with lse*log2(e) in the workspace for dkdv.
//   dkdv   : key-outer.  A workgroup owns 128 keys of one KV head (32 per
//            wave) and walks the query columns (position, head-of-group) that
//            can see them, 128 columns per step (four 32-column blocks, each
//            skipped when none of its columns sees the wave's keys).  S = Q K^T and dP = dO V^T
//            put one key per lane and the columns in the accumulator
//            registers, which is the operand layout of the two products
//            that contract over columns: dV^T += dO^T P and dK^T += Q^T dS.
//            Q^T and dO^T come from the row-major LDS tiles through
//            transposing LDS reads.
//   dsink  : one workgroup per head reduces the per-row terms the dq kernel
//            left in the workspace ([head][token row], contiguous).
// P and dP are recomputed in both the key-outer and query-outer kernels.
// dsink does not use Dvec = <dout, out> alone, whose bf16 `out` carries
// rounding that a cancelling sum over all rows would amplify: the dq kernel
// forms r_i = sum_j P_ij dP_ij (= <dout_i, sum_j P_ij v_j>, the same quantity)
// in fp32 as sum_j dS_ij + Dvec_i (1 - P_sink,i) while it sweeps row i's keys
// (the visible probabilities sum to 1 - P_sink,i, so Dvec's rounding cancels
// to within the rounding of P) and stores exp(sink - lse_i) r_i.
#include "common.h"
#include "launch.h"


namespace gptoss {
namespace {

#ifndef GPTOSS_DKDV_WAVES
#define GPTOSS_DKDV_WAVES 4
#endif
#ifndef GPTOSS_DQ_WAVES
#define GPTOSS_DQ_WAVES 4
#endif
#ifndef GPTOSS_DKDV_COLS
#define GPTOSS_DKDV_COLS 128
#endif

struct BwdParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const uint16_t* out;
    const uint16_t* dout;
    const float* lse;
    const float* sinks;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* dsinks;
    float2* ld;      // [T][Hq] {lse * log2(e), Dvec} per token row and head
    float* dsterm;   // [Hq][T] exp(sink - lse) * sum_j P dP per row
    const int* cu;   // packed documents: sequence b = rows cu[b] .. cu[b+1]-1; nullptr = dense batch
    const float2* rope;  // (cos, sin) [position][32]: q rotated by dq (into q_rot), dq/dk through R^T; or nullptr
    uint16_t* q_rot;     // rotated q written by the dq kernel, read by dkdv (rope only)
    int B, S, Hq, Hkv, G, window;  // S = sequence length (dense) or the longest document (packed)
    int T;           // total token rows (B * S when dense)
    float scale;
    float c;  // scale * log2(e)
};

// dsink: one workgroup of 1024 threads per head sums the rows'
// exp(sink - lse) r terms (contiguous per head and sequence).  Each thread
// keeps 16 loads in flight (16 partial sums), so the 16384 rows of a head
// take one round trip instead of one per 1024 rows.
constexpr int kDsinkThreads = 1024;
constexpr int kDsinkUnroll = 16;
__global__ void __launch_bounds__(kDsinkThreads)
bwd_dsink_kernel(BwdParams p) {
    __shared__ float red[kDsinkThreads / 64];
    const int h = blockIdx.x;
    const float* src = p.dsterm + (size_t)h * p.T;
    float a[kDsinkUnroll];
#pragma unroll
    for (int k = 0; k < kDsinkUnroll; ++k) a[k] = 0.0f;
    // the rows of each sequence (for packed documents, only rows inside a
    // document hold a term: the dq kernel wrote those)
    for (int b = 0; b < p.B; ++b) {
        const SeqRows sr = seq_rows(p.cu, p.S, p.Hq, p.T, b);
        const float* seg = src + sr.row0;
        for (int i = threadIdx.x; i < sr.len; i += kDsinkUnroll * kDsinkThreads) {
#pragma unroll
            for (int k = 0; k < kDsinkUnroll; ++k) {
                const int j = i + k * kDsinkThreads;
                const float x = seg[min(j, sr.len - 1)];  // in range; past the end counts 0
                a[k] += j < sr.len ? x : 0.0f;
            }
        }
    }
#pragma unroll
    for (int w = kDsinkUnroll / 2; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) a[k] += a[k + w];
    float acc = a[0];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
        for (int w = 0; w < kDsinkThreads / 64; ++w) t += red[w];
        p.dsinks[h] = -t;
    }
}

// ---------------------------------------------------------------------------
// dkdv: key-outer.
constexpr int kKvWaves = GPTOSS_DKDV_WAVES;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKeysPerBlock = 32 * kKvWaves;  // 32 keys per wave
constexpr int kColsPerStep = GPTOSS_DKDV_COLS;  // 64 or 128
constexpr int kKvBlocks = kColsPerStep / 32;    // 32-column blocks per step
constexpr int kKvStRows = kKvThreads / 8;            // columns staged per pass
constexpr int kKvStPasses = kColsPerStep / kKvStRows;

__device__ __forceinline__ void dkdv_coords(const BwdParams& p, int n_kt, int bid, int& grp, int& kt) {
    const int n_groups = p.B * p.Hkv;
    if ((n_groups & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        // tile-major within the XCD: the heaviest key tiles (lowest, seen by
        // the most queries) of all the XCD's groups are dispatched first.
        // Groups are KV-head-major, so with 8 KV heads each XCD takes one KV
        // head of every sequence: equal work per XCD even when packed
        // documents differ in length.
        const int gpx = n_groups >> 3;
        grp = xcd * gpx + slot % gpx;
        kt = slot / gpx;
    } else {
        grp = bid % n_groups;
        kt = bid / n_groups;
    }
}

__global__ void __launch_bounds__(kKvThreads, 2)
bwd_dkdv_kernel(BwdParams p, int n_kt) {
    __shared__ uint4 sQ[2][kColsPerStep / 64 * kTileUnits];
    __shared__ uint4 sO[2][kColsPerStep / 64 * kTileUnits];
    __shared__ float4 sL[2][kColsPerStep / 4];  // lse * log2(e) per column
    __shared__ float4 sD[2][kColsPerStep / 4];  // Dvec per column
    __shared__ int4 sP[2][kColsPerStep / 4];    // position per column

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31, i16 = lane & 15;
    int grp, kt;
    dkdv_coords(p, n_kt, blockIdx.x, grp, kt);
    const int kvh = grp / p.B, b = grp % p.B;  // KV-head-major groups
    const SeqRows sr = seq_rows(p.cu, p.S, p.Hq, p.T, b);
    const int S = sr.len, W = p.window, G = p.G, Hq = p.Hq;
    const unsigned Weff = W > 0 ? (unsigned)W : 0x7fffffffu;
    const int k0 = kt * kKeysPerBlock;
    if (k0 >= S) return;  // a document shorter than the longest one
    const int kw0 = k0 + 32 * wave;          // this wave's keys kw0 .. kw0+31
    const int kw1 = min(kw0 + 31, S - 1);
    const bool wave_active = kw0 < S;
    const int my_key = kw0 + l32;

    // K and V rows of this lane's key as B operands (d = 16 ks + 8 g + 0..7).
    // K is multiplied by c = scale * log2(e) once here (and rounded to bf16),
    // so that S' = Q (c K)^T is the score in log2 units; with the
    // accumulator started at -lse * log2(e), P = exp2(S') needs no further
    // arithmetic.  (The rounding of c K perturbs P by up to 2^-8 relative, far
    // inside the gradients' tolerance; dK uses Q and dS, not K.)
    const size_t kv_stride = (size_t)p.Hkv * kHeadDim;
    bf16x8 kb[4], vb[4];
    {
        const size_t off = ((size_t)sr.row0 + my_key) * kv_stride + (size_t)kvh * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
            if (my_key < S) {
                x = ld16(p.k + off + 16 * ks + 8 * g);
                y = ld16(p.v + off + 16 * ks + 8 * g);
            }
            const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
            uint32_t kw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) kw[i] = pack_bf16x2(bf16_lo(xw[i]) * p.c, bf16_hi(xw[i]) * p.c);
            kb[ks] = as_bf16x8(make_uint4(kw[0], kw[1], kw[2], kw[3]));
            vb[ks] = as_bf16x8(y);
        }
    }

    // query columns (position, head of the group; head fastest) that can see
    // keys [k0, k0 + 127]
    const int pos_lo = k0;
    const int pos_hi = W > 0 ? min(S - 1, k0 + kKeysPerBlock - 1 + W - 1) : S - 1;
    const int n_cols = (pos_hi - pos_lo + 1) * G;
    const int n_steps = (n_cols + kColsPerStep - 1) / kColsPerStep;

    f32x16 dkacc[2], dvacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkacc[db][r] = dvacc[db][r] = 0.0f;

    // staging: thread stages rows (columns) st_row + kKvStRows j (unit
    // st_unit) of each step, and threads 0 .. kColsPerStep - 1 the
    // per-column scalars.  A column c maps to (pos_lo + c / G, kvh * G + c % G); when G
    // divides the step's columns a step advances every staged column by
    // kColsPerStep / G positions.
    const int st_row = tid >> 3, st_unit = tid & 7;
    const bool g_div = (kColsPerStep % G) == 0;
    const size_t pos_stride = (size_t)Hq * kHeadDim;  // elements per position
    const uint16_t* qsrc = p.rope != nullptr ? p.q_rot : p.q;  // with RoPE: q as the dq kernel rotated it
    const uint16_t* qcol_base = qsrc + ((size_t)sr.row0 * Hq + (size_t)kvh * G) * kHeadDim + 8 * st_unit;
    const uint16_t* ocol_base = p.dout + ((size_t)sr.row0 * Hq + (size_t)kvh * G) * kHeadDim + 8 * st_unit;
    const float2* ld_base = p.ld + (size_t)sr.row0 * Hq + (size_t)kvh * G;
    uint4 rq[kKvStPasses], ro[kKvStPasses];
    float2 rld = make_float2(INFINITY, 0.0f);
    int rpos = 0x3fffffff;
    // per-thread column offsets within a step (constant across steps when G divides kColsPerStep)
    int st_pos[kKvStPasses], st_head[kKvStPasses];
#pragma unroll
    for (int j = 0; j < kKvStPasses; ++j) {
        st_pos[j] = (st_row + kKvStRows * j) / G;
        st_head[j] = (st_row + kKvStRows * j) % G;
    }
    const int ld_pos = tid / G, ld_head = tid % G;
    const int pos_per_step = kColsPerStep / G;
    // position offsets of the 32-column blocks within a whole step
    int blk_lo[kKvBlocks], blk_hi[kKvBlocks];
#pragma unroll
    for (int mb = 0; mb < kKvBlocks; ++mb) {
        blk_lo[mb] = (32 * mb) / G;
        blk_hi[mb] = (32 * mb + 31) / G;
    }
    // Whole steps with G dividing kColsPerStep (all but possibly the first one
    // processed): the rows a thread stages in step st lie st * pos_per_step
    // positions above its rows of step 0, so their addresses are one
    // multiply-add from these step-0 addresses.
    const char* q_row0[kKvStPasses];
    const char* o_row0[kKvStPasses];
#pragma unroll
    for (int j = 0; j < kKvStPasses; ++j) {
        const size_t off = (size_t)(pos_lo + st_pos[j]) * pos_stride + (size_t)st_head[j] * kHeadDim;
        q_row0[j] = reinterpret_cast<const char*>(qcol_base + off);
        o_row0[j] = reinterpret_cast<const char*>(ocol_base + off);
    }
    const char* ld_row0 = reinterpret_cast<const char*>(ld_base + (size_t)(pos_lo + ld_pos) * Hq + ld_head);
    // (64-bit: with G = 1 a step spans 128 positions of Hq heads, and only
    // the row count T * Hq is bounded)
    const uint64_t step_bytes = (uint64_t)pos_per_step * pos_stride * sizeof(uint16_t);
    const uint64_t ld_step_bytes = (uint64_t)pos_per_step * Hq * sizeof(float2);
    auto load_step = [&](int st) {
        const int c0 = st * kColsPerStep;
        if (g_div && c0 + kColsPerStep <= n_cols) {  // wave-uniform
            const uint64_t dq = (uint64_t)(uint32_t)st * step_bytes;
#pragma unroll
            for (int j = 0; j < kKvStPasses; ++j) {
                rq[j] = ld16(q_row0[j] + dq);
                ro[j] = ld16(o_row0[j] + dq);
            }
            if (tid < kColsPerStep) {
                rld = *reinterpret_cast<const float2*>(ld_row0 + (uint64_t)(uint32_t)st * ld_step_bytes);
                rpos = pos_lo + st * pos_per_step + ld_pos;
            }
            return;
        }
        // columns past the last one re-read the last column's rows: their
        // lse is staged as +inf below, so P = dS = 0 for them
#pragma unroll
        for (int j = 0; j < kKvStPasses; ++j) {
            const int c = min(c0 + st_row + kKvStRows * j, n_cols - 1);
            const size_t off = (size_t)(pos_lo + c / G) * pos_stride + (size_t)(c % G) * kHeadDim;
            rq[j] = ld16(qcol_base + off);
            ro[j] = ld16(ocol_base + off);
        }
        if (tid < kColsPerStep) {
            const int c = c0 + tid;
            rld = make_float2(INFINITY, 0.0f);
            rpos = 0x3fffffff;
            if (c < n_cols) {
                const int pos = pos_lo + c / G;
                rld = ld_base[(size_t)pos * Hq + c % G];
                rpos = pos;
            }
        }
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kKvStPasses; ++j) {
            const int row = st_row + kKvStRows * j;
            sQ[buf][tile_unit(row, st_unit)] = rq[j];
            sO[buf][tile_unit(row, st_unit)] = ro[j];
        }
        if (tid < kColsPerStep) {
            // negated: they seed the S' and dP accumulators
            reinterpret_cast<float*>(sL[buf])[tid] = -rld.x;
            reinterpret_cast<float*>(sD[buf])[tid] = -rld.y;
            reinterpret_cast<int*>(sP[buf])[tid] = rpos;
        }
    };

    // One 32-column block: S' - lse' = Q (c K)^T - lse * log2(e) and
    // dP - Dvec = dO V^T - Dvec (one key per lane, register 8h + s = column
    // 32 mb + 16 h + 8 g + s; the accumulators start at the staged -lse' and
    // -Dvec); on edge steps the invisible scores are set to -inf (so P = dS =
    // 0); then P = exp2(.), dS = P (dP - Dvec), and dV^T += dO^T P,
    // dK^T += Q^T dS over those 32 columns.
    auto block = [&](const uint4* tq, const uint4* to, const float4* tl, const float4* td, const int4* tp, int mb,
                     bool need_mask) {
        f32x16 sacc, dpacc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int q4 = (32 * mb + 16 * h + 8 * g) >> 2;  // float4 index of the 8 columns
            const float4 la = tl[q4], lb = tl[q4 + 1];
            const float4 da = td[q4], dbv = td[q4 + 1];
            sacc[8 * h + 0] = la.x; sacc[8 * h + 1] = la.y; sacc[8 * h + 2] = la.z; sacc[8 * h + 3] = la.w;
            sacc[8 * h + 4] = lb.x; sacc[8 * h + 5] = lb.y; sacc[8 * h + 6] = lb.z; sacc[8 * h + 7] = lb.w;
            dpacc[8 * h + 0] = da.x; dpacc[8 * h + 1] = da.y; dpacc[8 * h + 2] = da.z; dpacc[8 * h + 3] = da.w;
            dpacc[8 * h + 4] = dbv.x; dpacc[8 * h + 5] = dbv.y; dpacc[8 * h + 6] = dbv.z; dpacc[8 * h + 7] = dbv.w;
        }
        const int arow = 32 * mb + perm_row(l32);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            sacc = mfma32(as_bf16x8(tq[tile_unit(arow, 2 * ks + g)]), kb[ks], sacc);
            dpacc = mfma32(as_bf16x8(to[tile_unit(arow, 2 * ks + g)]), vb[ks], dpacc);
        }
        if (need_mask) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q4 = (32 * mb + 16 * h + 8 * g) >> 2;
                const int4 pa = tp[q4], pbp = tp[q4 + 1];
                const int pv[8] = {pa.x, pa.y, pa.z, pa.w, pbp.x, pbp.y, pbp.z, pbp.w};
#pragma unroll
                for (int s = 0; s < 8; ++s)
                    sacc[8 * h + s] = (unsigned)(pv[s] - my_key) < Weff ? sacc[8 * h + s] : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t wp[4], wd[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float pr[2], ds[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int s = 2 * j + e;
                    pr[e] = fast_exp2(sacc[8 * h + s]);
                    ds[e] = pr[e] * dpacc[8 * h + s];
                }
                wp[j] = pack_bf16x2(pr[0], pr[1]);
                wd[j] = pack_bf16x2(ds[0], ds[1]);
            }
            const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(wp[0], wp[1], wp[2], wp[3]));
            const bf16x8 dsb = __builtin_bit_cast(bf16x8, make_uint4(wd[0], wd[1], wd[2], wd[3]));
            // dV^T += dO^T P and dK^T += Q^T dS over these 16 columns
            const int r0 = 32 * mb + 16 * h + 8 * g;
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const int cbase = 32 * db + 16 * (l32 >> 4);
                dvacc[db] = mfma32(tile_read_tr8(to, r0, cbase, i16), pb, dvacc[db]);
                dkacc[db] = mfma32(tile_read_tr8(tq, r0, cbase, i16), dsb, dkacc[db]);
            }
        }
    };

    // Steps run from the last columns down: the workgroups of one KV group
    // (dispatched together on one XCD) all start at the sequence end and move
    // down in near lockstep, so each Q/dO tile comes from HBM once and from
    // L2 for the others.
    if (n_steps > 0) {
        load_step(n_steps - 1);
        store_step(0);
    }
    __syncthreads();

    for (int it = 0; it < n_steps; ++it) {
        const int st = n_steps - 1 - it;
        const int buf = it & 1;
        const bool has_next = st > 0;
        if (has_next) load_step(st - 1);

        const int c0 = st * kColsPerStep;
        const bool whole = g_div && c0 + kColsPerStep <= n_cols;  // no scalar divisions by G then
        const int tp_min = pos_lo + (whole ? st * pos_per_step : c0 / G);
        const int tp_max = min(whole ? tp_min + pos_per_step - 1 : pos_lo + (min(c0 + kColsPerStep, n_cols) - 1) / G,
                               S - 1);
        const bool skip = !wave_active || tp_max < kw0 || (W > 0 && tp_min - kw1 >= W);
        if (!skip) {
            // Per 32-column block: its position range; live if one of its
            // columns sees one of the wave's keys, masked unless every column
            // sees all of them (a block none sees contributes exactly nothing).
            bool live[kKvBlocks], need_mask[kKvBlocks];
#pragma unroll
            for (int mb = 0; mb < kKvBlocks; ++mb) {
                int bmin, bmax;
                bool any = true;
                if (whole) {
                    bmin = tp_min + blk_lo[mb];
                    bmax = tp_min + blk_hi[mb];
                } else {
                    const int cb = c0 + 32 * mb;
                    any = cb < n_cols;
                    bmin = pos_lo + cb / G;
                    bmax = pos_lo + (min(cb + 31, n_cols - 1)) / G;
                }
                live[mb] = any && bmax >= kw0 && (W == 0 || bmin - kw1 < W);
                need_mask[mb] = !(bmin >= kw1 && (W == 0 || bmax - kw0 < W));
            }
#pragma unroll
            for (int mb = 0; mb < kKvBlocks; ++mb) {
                if (live[mb]) block(sQ[buf], sO[buf], sL[buf], sD[buf], sP[buf], mb, need_mask[mb]);
                __builtin_amdgcn_sched_barrier(0);  // keep the blocks' live ranges apart
            }
        }

        if (has_next) store_step(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane = key, registers = d rows (acc_row); 4 contiguous d per
    // store.  Element d of db = 0 and d + 32 of db = 1 sit in the same
    // register index, so with RoPE the adjoint rotation of dk is in-lane.
    if (my_key < S) {
        const size_t off = ((size_t)sr.row0 + my_key) * kv_stride + (size_t)kvh * kHeadDim;
        float4 et[8];  // table entries of pairs 8 r4 + 4 g + 0..3, loaded before any store
        if (p.rope != nullptr) {
            const float4* t = reinterpret_cast<const float4*>(p.rope + (size_t)my_key * 32);
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                et[2 * r4] = t[4 * r4 + 2 * g];
                et[2 * r4 + 1] = t[4 * r4 + 2 * g + 1];
            }
        }
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float ka[4], kb2[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ka[j] = dkacc[0][4 * r4 + j] * p.scale;
                kb2[j] = dkacc[1][4 * r4 + j] * p.scale;
            }
            if (p.rope != nullptr) rope4_adjoint_f32(ka, kb2, et[2 * r4], et[2 * r4 + 1]);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const int d0 = 32 * db + 8 * r4 + 4 * g;
                const float* kx = db == 0 ? ka : kb2;
                uint2 wk, wv;
                wk.x = pack_bf16x2(kx[0], kx[1]);
                wk.y = pack_bf16x2(kx[2], kx[3]);
                wv.x = pack_bf16x2(dvacc[db][4 * r4 + 0], dvacc[db][4 * r4 + 1]);
                wv.y = pack_bf16x2(dvacc[db][4 * r4 + 2], dvacc[db][4 * r4 + 3]);
                *reinterpret_cast<uint2*>(p.dk + off + d0) = wk;
                *reinterpret_cast<uint2*>(p.dv + off + d0) = wv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dq: query-outer; 4 waves x 32 columns per workgroup, 64-key tiles.
constexpr int kDqWaves = GPTOSS_DQ_WAVES;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqCols = 32 * kDqWaves;  // 32 columns per wave
constexpr int kBk = 64;
constexpr int kDqStRows = kDqThreads / 8;   // key rows staged per pass
constexpr int kDqStPasses = kBk / kDqStRows;

__device__ __forceinline__ void dq_coords(const BwdParams& p, int n_qt, int bid, int& grp, int& qt) {
    const int n_groups = p.B * p.Hkv;
    if ((n_groups & 7) == 0) {
        const int xcd = bid & 7, slot = bid >> 3;
        const int gpx = n_groups >> 3;  // tile-major: heaviest tiles of all groups first
        grp = xcd * gpx + slot % gpx;
        qt = slot / gpx;
    } else {
        grp = bid % n_groups;
        qt = bid / n_groups;
    }
    qt = n_qt - 1 - qt;  // latest positions (most keys) first
}

__global__ void __launch_bounds__(kDqThreads, 2)
bwd_dq_kernel(BwdParams p, int n_qt, int pos_per_block) {
    __shared__ uint4 sK[2][kTileUnits];
    __shared__ uint4 sV[2][kTileUnits];

    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, l32 = lane & 31, i16 = lane & 15;
    int grp, qt;
    dq_coords(p, n_qt, blockIdx.x, grp, qt);
    const int kvh = grp / p.B, b = grp % p.B;  // KV-head-major groups
    const SeqRows sr = seq_rows(p.cu, p.S, p.Hq, p.T, b);
    const int S = sr.len, W = p.window, G = p.G, Hq = p.Hq;
    const unsigned Weff = W > 0 ? (unsigned)W : 0x7fffffffu;
    const int p0 = qt * pos_per_block;
    if (p0 >= S) return;  // a document shorter than the longest one
    const int used_cols = pos_per_block * G;
    const int P1 = min(p0 + pos_per_block, S) - 1;

    const int cw = wave * 32 + l32;
    const int col_pos = p0 + cw / G;
    const int col_head = kvh * G + cw % G;
    const bool col_ok = cw < used_cols && col_pos < S;
    const int wc0 = wave * 32;
    const bool wave_active = wc0 < used_cols && p0 + wc0 / G < S;
    const int wpmin = p0 + wc0 / G;
    const int wpmax = min(p0 + min(wc0 + 31, used_cols - 1) / G, S - 1);

    // K/V tiles of 64 keys, staged through LDS; the first tile's loads are
    // issued ahead of the row prologue below so the two round trips overlap
    const int key_lo = W > 0 ? max(0, p0 - W + 1) : 0;
    const int t_begin = key_lo / kBk;
    const int t_end = P1 / kBk;

    const size_t kv_stride = (size_t)p.Hkv * kHeadDim;
    const uint16_t* kbase = p.k + ((size_t)sr.row0 * p.Hkv + kvh) * kHeadDim;
    const uint16_t* vbase = p.v + ((size_t)sr.row0 * p.Hkv + kvh) * kHeadDim;
    const int st_row = tid >> 3, st_unit = tid & 7;
    uint4 rk[kDqStPasses], rv[kDqStPasses];
    // rows past the sequence end re-read its last row: no query row sees
    // them, and the tile holding them is an edge tile, whose scores are masked
    auto load_tile = [&](int t) {
        const int kt0 = t * kBk;
#pragma unroll
        for (int j = 0; j < kDqStPasses; ++j) {
            const int key = min(kt0 + st_row + kDqStRows * j, S - 1);
            rk[j] = ld16(kbase + row_off(key, (uint32_t)kv_stride) + 8 * st_unit);
            rv[j] = ld16(vbase + row_off(key, (uint32_t)kv_stride) + 8 * st_unit);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int j = 0; j < kDqStPasses; ++j) {
            const int row = st_row + kDqStRows * j;
            sK[buf][tile_unit(row, st_unit)] = rk[j];
            sV[buf][tile_unit(row, st_unit)] = rv[j];
        }
    };

    if (t_begin <= t_end) load_tile(t_begin);

    // This column's q and dO rows as B operands (d = 16 ks + 8 g + 0..7).
    // The dP accumulator starts at -Dvec, so the MFMAs deliver dP - Dvec and
    // dS = P acc.  (q is not pre-scaled by c here: P must sum, with the
    // sink, to 1 within fp32 rounding for the dsink term below, and a
    // bf16-rounded c q would perturb it by ~1e-3.)
    //
    // The row's Dvec = <dout, out> is formed here from the same dO fragments
    // (the two lane halves hold d = 16 ks + 8 g + 0..7), and {lse log2(e),
    // Dvec} is stored for the key-outer kernel, which runs after this one.
    //
    // With RoPE the q fragments ks and ks + 2 hold the pairs (d, d + 32) of
    // this lane's d, so q is rotated in-lane and written to q_rot for dkdv
    // (each column belongs to exactly one workgroup and lane pair).
    bf16x8 qf[4], of[4];
    float lse2 = INFINITY, dvec = 0.0f, dsum = 0.0f;
    const bool rope = p.rope != nullptr;
    {
        const size_t row = ((size_t)sr.row0 + col_pos) * Hq + col_head;
        const size_t off = row * kHeadDim;
        float4 rcs[2][4];
        if (rope && col_ok) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) load_rope8(p.rope, col_pos, 16 * ks + 8 * g, rcs[ks]);
        }
        // every load is issued before the q_rot store (which the compiler
        // must assume may alias them)
        uint4 xq[4], yq[4], oq[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            xq[ks] = yq[ks] = oq[ks] = make_uint4(0, 0, 0, 0);
            if (col_ok) {
                xq[ks] = ld16(p.q + off + 16 * ks + 8 * g);
                yq[ks] = ld16(p.dout + off + 16 * ks + 8 * g);
                oq[ks] = ld16(p.out + off + 16 * ks + 8 * g);
            }
        }
        if (col_ok) lse2 = p.lse[sr.lse_base + col_head * sr.lse_hstride + col_pos] * kLog2e;
        if (rope) {
            bool mid = false;
            if (col_ok) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) mid = rope8(xq[ks], xq[ks + 2], rcs[ks]) || mid;
            }
            if (__any(mid) && col_ok) {
                // (rare) an fp64 sum on a bf16 midpoint: reload q (the loads
                // above are complete, q_rot not yet written) and rotate with
                // exact remainders
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint4 x0 = ld16(p.q + off + 16 * ks + 8 * g), x1 = ld16(p.q + off + 16 * (ks + 2) + 8 * g);
                    rope8_exact(x0, x1, rcs[ks]);
                    xq[ks] = x0;
                    xq[ks + 2] = x1;
                }
            }
            if (col_ok) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<uint4*>(p.q_rot + off + 16 * ks + 8 * g) = xq[ks];
            }
        }
        float dot = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const uint4 y = yq[ks], o = oq[ks];
            qf[ks] = as_bf16x8(xq[ks]);
            of[ks] = as_bf16x8(y);
            const uint32_t ow[4] = {o.x, o.y, o.z, o.w}, dw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dot = fmaf(bf16_lo(ow[i]), bf16_lo(dw[i]), dot);
                dot = fmaf(bf16_hi(ow[i]), bf16_hi(dw[i]), dot);
            }
        }
        dvec = sum_across_halves(dot);
        if (col_ok && g == 0) p.ld[row] = make_float2(lse2, dvec);
    }

    f32x16 dqacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.0f;

    if (t_begin <= t_end) store_tile(0);
    __syncthreads();

    for (int t = t_begin; t <= t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        const bool has_next = t < t_end;
        if (has_next) load_tile(t + 1);
        const int kt0 = t * kBk;
        const bool skip = !wave_active || kt0 > wpmax || (W > 0 && wpmin - (kt0 + kBk - 1) >= W);
        if (!skip) {
            const bool need_mask = !(kt0 + kBk - 1 <= wpmin && (W == 0 || wpmax - kt0 < W));
            const uint4* tk = sK[buf];
            const uint4* tv = sV[buf];
            // S^T = K Q^T and dP^T = V dO^T (one column per lane; register
            // 8h + s of key block mb = key kt0 + 32 mb + 16 h + 8 g + s); on edge
            // tiles invisible scores become -inf (P = dS = 0); then P, dS and
            // this row's sum_j P dP
            bf16x8 dsb[4];
            const int dd = col_pos - kt0 - 8 * g;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
                f32x16 sacc, dpacc;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    sacc[r] = 0.0f;
                    dpacc[r] = -dvec;
                }
                const int arow = 32 * mb + perm_row(l32);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    sacc = mfma32(as_bf16x8(tk[tile_unit(arow, 2 * ks + g)]), qf[ks], sacc);
                    dpacc = mfma32(as_bf16x8(tv[tile_unit(arow, 2 * ks + g)]), of[ks], dpacc);
                }
                if (need_mask) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int cr = 32 * mb + 16 * (r >> 3) + (r & 7);
                        sacc[r] = (unsigned)(dd - cr) < Weff ? sacc[r] : -INFINITY;
                    }
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t w[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float ds[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int r = 8 * h + 2 * j + e;
                            ds[e] = fast_exp2(fmaf(sacc[r], p.c, -lse2)) * dpacc[r];
                            dsum += ds[e];
                        }
                        w[j] = pack_bf16x2(ds[0], ds[1]);
                    }
                    dsb[2 * mb + h] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
                }
            }
            // dQ^T += K^T dS^T over the 64 keys (16 per step)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int db = 0; db < 2; ++db) {
                    const bf16x8 kT = tile_read_tr8(tk, 16 * kk + 8 * g, 32 * db + 16 * (l32 >> 4), i16);
                    dqacc[db] = mfma32(kT, dsb[kk], dqacc[db]);
                }
            }
        }
        if (has_next) store_tile(buf ^ 1);
        __syncthreads();
    }

    dsum = sum_across_halves(dsum);
    // RoPE table entries of this lane's dq pairs d = 8 r4 + 4 g + 0..3, all
    // loaded before the stores below
    float4 et[8];
    if (rope && col_ok) {
        const float4* t = reinterpret_cast<const float4*>(p.rope + (size_t)col_pos * 32);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            et[2 * r4] = t[4 * r4 + 2 * g];
            et[2 * r4 + 1] = t[4 * r4 + 2 * g + 1];
        }
    }
    if (col_ok) {
        if (g == 0) {
            // this row's dsink term exp(sink - lse) r with
            // r = sum_j P dP = sum_j dS + Dvec (1 - P_sink): the row's
            // probabilities sum to 1 - P_sink, so Dvec (and the bf16
            // rounding of `out` it carries) cancels to within the fp32
            // rounding of P
            const float psink = fast_exp2(p.sinks[col_head] * kLog2e - lse2);
            p.dsterm[(size_t)col_head * p.T + sr.row0 + col_pos] = psink * fmaf(dvec, 1.0f - psink, dsum);
        }
        // d and d + 32 share a register index (db = 0, 1): RoPE's adjoint
        // is in-lane, applied to the fp32 values before the one rounding
        uint16_t* row = p.dq + (((size_t)sr.row0 + col_pos) * Hq + col_head) * kHeadDim;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            float qa[4], qb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qa[j] = dqacc[0][4 * r4 + j] * p.scale;
                qb[j] = dqacc[1][4 * r4 + j] * p.scale;
            }
            if (rope) rope4_adjoint_f32(qa, qb, et[2 * r4], et[2 * r4 + 1]);
#pragma unroll
            for (int db = 0; db < 2; ++db) {
                const float* x = db == 0 ? qa : qb;
                uint2 w;
                w.x = pack_bf16x2(x[0], x[1]);
                w.y = pack_bf16x2(x[2], x[3]);
                *reinterpret_cast<uint2*>(row + 32 * db + 8 * r4 + 4 * g) = w;
            }
        }
    }
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream) {
    BwdParams p;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.out = a.out;
    p.dout = a.dout;
    p.lse = a.lse;
    p.sinks = a.sinks;
    p.dq = a.dq;
    p.dk = a.dk;
    p.dv = a.dv;
    p.dsinks = a.dsinks;
    p.ld = static_cast<float2*>(a.workspace);
    p.dsterm = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + bwd_ld_region_bytes(a.T, a.Hq));
    p.cu = a.cu;
    p.rope = a.rope;
    p.q_rot = a.q_rot;
    p.B = a.B;
    p.S = a.S;
    p.T = a.T;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.G = a.Hq / a.Hkv;
    p.window = a.window >= a.S ? 0 : a.window;
    p.scale = a.scale;
    p.c = a.scale * kLog2e;

    const int n_kt = (a.S + kKeysPerBlock - 1) / kKeysPerBlock;
    const int ppb = kDqCols / p.G >= 1 ? kDqCols / p.G : 1;
    const int n_qt = (a.S + ppb - 1) / ppb;
    if ((long long)n_qt * a.B * a.Hkv > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // dq first: it also stores {lse log2(e), Dvec} per row for dkdv
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)(n_qt * a.B * a.Hkv)), dim3(kDqThreads), 0, stream, p, n_qt,
                       ppb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(n_kt * a.B * a.Hkv)), dim3(kKvThreads), 0, stream, p, n_kt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dsink_kernel, dim3(a.Hq), dim3(kDsinkThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gptoss
