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
//   split kernel : grid (split, KV head x head block, sequence).  A split is
//     256 visible keys; each of the 4 waves takes 64 of them.  A wave reads
//     its K rows straight into MFMA A-operand registers, stages its V rows
//     in LDS (read back transposed), and computes S^T = K Q^T and O^T = V^T P^T with
//     32x32x16 bf16 MFMAs (columns = the query heads of the group).  The 4
//     waves merge through LDS and the workgroup writes one partial
//     (unnormalised O, running max m in log2 units, sum l) per head.  A
//     sequence that fits in one split is finished in place (sink folded in,
//     out and lse written) and never touches the partial buffer.
//   merge kernel : one wave per (sequence, head) with more than one split:
//     m = max(sink, m_s), l = 2^(sink - m) + sum l_s 2^(m_s - m),
//     out = sum O_s 2^(m_s - m) / l, lse = ln2 (m + log2 l).  The sink enters
//     here exactly once.
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace gptoss {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kSplitKeys = 256;   // visible keys per split (64 per wave)
constexpr int kPartStride = 68;   // floats per partial: O[64], m, l, pad

struct DecParams {
    const uint16_t* q;
    const uint16_t* kc;
    const uint16_t* vc;
    const int* cu;
    const float* sinks;
    uint16_t* out;
    float* lse;
    float* part;      // [N][Hq][n_splits][kPartStride]
    int Hq, Hkv, G, window, n_splits, n_hblk, max_seqlen;
    float c;          // scale * log2(e)
};

__device__ __forceinline__ void seq_range(const DecParams& p, int n, int& base, int& L, int& vis_lo) {
    base = p.cu[n];
    L = min(p.cu[n + 1] - base, p.max_seqlen);
    vis_lo = p.window > 0 ? max(0, L - p.window) : 0;
}

__global__ void __launch_bounds__(kThreads)
decode_split_kernel(DecParams p) {
    // per wave: one row-major V tile (64 keys x 64 d, 144-byte rows); the
    // space is reused for the cross-wave merge
    __shared__ uint4 vsm[kWaves][kTileUnits];
    __shared__ float wm[kWaves][32], wl[kWaves][32];

    const int split = blockIdx.x;
    const int kvh = blockIdx.y / p.n_hblk;
    const int hb = blockIdx.y % p.n_hblk;
    const int n = blockIdx.z;
    int base, L, vis_lo;
    seq_range(p, n, base, L, vis_lo);
    const int n_vis = L - vis_lo;
    const int n_act = (n_vis + kSplitKeys - 1) / kSplitKeys;
    if (split >= n_act) return;  // uniform over the workgroup

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, l32 = lane & 31;
    const int G = p.G;
    const int hcol = hb * 32 + l32;             // head within the group
    const bool col_ok = hcol < G;
    const int head = kvh * G + hcol;

    const int t0 = vis_lo + split * kSplitKeys + wave * 64;  // this wave's first key
    const int t_end = min(t0 + 64, L);                       // exclusive
    const bool wave_active = t0 < L;

    const size_t row_stride = (size_t)p.Hkv * kHeadDim;
    const uint16_t* kb = p.kc + ((size_t)base * p.Hkv + kvh) * kHeadDim;
    const uint16_t* vb = p.vc + ((size_t)base * p.Hkv + kvh) * kHeadDim;

    // K A-operand rows (permuted as in the forward) and V rows for staging
    bf16x8 ka[2][4];
    uint4 vr[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int key = t0 + 32 * mb + perm_row(l32);
        const bool ok = wave_active && key < t_end;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (ok) x = ld16(kb + key * row_stride + 16 * ks + 8 * g);
            ka[mb][ks] = as_bf16x8(x);
        }
    }
    // V rows: lane loads 16-byte unit (lane % 8) of rows lane / 8 + 8 j
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int key = t0 + (lane >> 3) + 8 * j;
        uint4 x = make_uint4(0, 0, 0, 0);
        if (wave_active && key < t_end) x = ld16(vb + key * row_stride + 8 * (lane & 7));
        vr[j] = x;
    }
    bf16x8 qf[4];
    {
        const uint16_t* qrow = p.q + ((size_t)n * p.Hq + head) * kHeadDim;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            uint4 x = make_uint4(0, 0, 0, 0);
            if (col_ok) x = ld16(qrow + 16 * ks + 8 * g);
            qf[ks] = as_bf16x8(x);
        }
    }

    // V into this wave's LDS tile (row-major; read transposed for P.V)
#pragma unroll
    for (int j = 0; j < 8; ++j) vsm[wave][tile_unit((lane >> 3) + 8 * j, lane & 7)] = vr[j];

    // S^T = K Q^T  (one 32-column block of heads)
    f32x16 sacc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[mb][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) sacc[mb] = mfma32(ka[mb][ks], qf[ks], sacc[mb]);
    }
    // mask keys outside [t0, t_end)
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = t0 + 32 * mb + perm_row(acc_row(r, g));
            sacc[mb][r] = key < t_end ? sacc[mb][r] : -INFINITY;
            mx = fmaxf(mx, sacc[mb][r]);
        }
    mx = max_across_halves(mx);
    const float m = mx * p.c;                       // -inf only for an idle wave
    const float m_use = m == -INFINITY ? 0.0f : m;
    float lsum = 0.0f;
    bf16x8 pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 v8;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const float e = fast_exp2(fmaf(sacc[mb][8 * h + s], p.c, -m_use));
                lsum += e;
                v8[s] = (__bf16)e;
            }
            pb[2 * mb + h] = v8;
        }
    lsum = sum_across_halves(lsum);

    __syncthreads();  // V tiles written by every lane of each wave
    f32x16 oacc[2];
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            // V^T rows d = 32 db + l32, keys 16 kk + 8 g + 0..7
            const bf16x8 a = tile_read_tr8(vsm[wave], 16 * kk + 8 * g, 32 * db + 16 * (l32 >> 4), l32 & 15);
            oacc[db] = mfma32(a, pb[kk], oacc[db]);
        }
    }

    // ---- merge the 4 waves through LDS: O^T partials as [wave][col][d] fp32
    if (g == 0) {
        wm[wave][l32] = m;
        wl[wave][l32] = lsum;
    }
    __syncthreads();  // all V reads done before the tiles are overwritten
    float* ow = reinterpret_cast<float*>(vsm);  // 4 x 32 x 64 floats = 32 KB
    float msum = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) msum = fmaxf(msum, wm[w][l32]);
    const float mref = msum == -INFINITY ? 0.0f : msum;
    const float myscale = m == -INFINITY ? 0.0f : fast_exp2(m - mref);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = 32 * db + acc_row(r, g);
            ow[(wave * 32 + l32) * 64 + d] = oacc[db][r] * myscale;
        }
    __syncthreads();

    // 256 threads: column c = tid / 8, d chunk (8 floats) = tid % 8
    const int c = tid >> 3, dch = tid & 7;
    const int ghead = hb * 32 + c;
    if (ghead >= G) return;
    const int head_c = kvh * G + ghead;
    float mtot = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mtot = fmaxf(mtot, wm[w][c]);
    const float mref_c = mtot == -INFINITY ? 0.0f : mtot;
    float ltot = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
        if (wm[w][c] != -INFINITY) ltot += wl[w][c] * fast_exp2(wm[w][c] - mref_c);
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] += ow[(w * 32 + c) * 64 + 8 * dch + i];

    if (n_act == 1) {
        // finish in place: fold in the sink
        const float sink = p.sinks[head_c];
        const float s2 = sink * kLog2e;
        const float mf = fmaxf(s2, mtot);
        const float a = fast_exp2(mtot - mf);  // mtot is finite: >= 1 visible key
        const float lfin = (sink == -INFINITY ? 0.0f : fast_exp2(s2 - mf)) + ltot * a;
        const float inv = a / lfin;
        uint4 w4;
        w4.x = pack_bf16x2(o[0] * inv, o[1] * inv);
        w4.y = pack_bf16x2(o[2] * inv, o[3] * inv);
        w4.z = pack_bf16x2(o[4] * inv, o[5] * inv);
        w4.w = pack_bf16x2(o[6] * inv, o[7] * inv);
        st16(p.out + ((size_t)n * p.Hq + head_c) * kHeadDim + 8 * dch, w4);
        if (dch == 0) p.lse[(size_t)n * p.Hq + head_c] = (mf + fast_log2(lfin)) * kLn2;
        return;
    }
    float* dst = p.part + (((size_t)n * p.Hq + head_c) * p.n_splits + split) * kPartStride;
    st16(dst + 8 * dch, *reinterpret_cast<uint4*>(&o[0]));
    st16(dst + 8 * dch + 4, *reinterpret_cast<uint4*>(&o[4]));
    if (dch == 0) {
        dst[64] = mtot;
        dst[65] = ltot;
    }
}

// One wave per (sequence, head); lane = d.
__global__ void __launch_bounds__(256)
decode_merge_kernel(DecParams p, int total) {
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= total) return;
    const int lane = threadIdx.x & 63;
    const int n = wid / p.Hq, head = wid % p.Hq;
    int base, L, vis_lo;
    seq_range(p, n, base, L, vis_lo);
    const int n_act = (L - vis_lo + kSplitKeys - 1) / kSplitKeys;
    const float sink = p.sinks[head];
    uint16_t* orow = p.out + ((size_t)n * p.Hq + head) * kHeadDim;
    if (n_act == 1) return;  // finished by the split kernel
    if (n_act == 0) {        // empty sequence: only the sink
        orow[lane] = 0;
        if (lane == 0) p.lse[(size_t)n * p.Hq + head] = sink;
        return;
    }
    const float* src = p.part + ((size_t)n * p.Hq + head) * p.n_splits * kPartStride;
    float mtot = sink * kLog2e;
    for (int s = 0; s < n_act; ++s) mtot = fmaxf(mtot, src[s * kPartStride + 64]);
    float l = sink == -INFINITY ? 0.0f : fast_exp2(sink * kLog2e - mtot);
    float o = 0.0f;
    for (int s = 0; s < n_act; ++s) {
        const float a = fast_exp2(src[s * kPartStride + 64] - mtot);
        l += src[s * kPartStride + 65] * a;
        o += src[s * kPartStride + lane] * a;
    }
    const float r = o / l;
    const __bf16 rb = (__bf16)r;
    orow[lane] = __builtin_bit_cast(uint16_t, rb);
    if (lane == 0) p.lse[(size_t)n * p.Hq + head] = (mtot + fast_log2(l)) * kLn2;
}

int splits_for(int max_seqlen, int window) {
    const int vis = window > 0 ? std::min(max_seqlen, window) : max_seqlen;
    return std::max(1, (vis + kSplitKeys - 1) / kSplitKeys);
}

}  // namespace

size_t decode_workspace_bytes(int N, int Hq, int Hkv, int max_seqlen, int window) {
    (void)Hkv;
    const int ns = splits_for(max_seqlen, window);
    if (ns <= 1) return 0;
    return (size_t)N * Hq * ns * kPartStride * sizeof(float);
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
    p.n_splits = splits_for(a.max_seqlen, a.window);
    p.n_hblk = (p.G + 31) / 32;
    p.c = a.scale * kLog2e;
    dim3 grid(p.n_splits, a.Hkv * p.n_hblk, a.N);
    hipLaunchKernelGGL(decode_split_kernel, grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int total = a.N * a.Hq;
    hipLaunchKernelGGL(decode_merge_kernel, dim3((total + 3) / 4), dim3(256), 0, stream, p, total);
    return hipGetLastError();
}

}  // namespace gptoss
