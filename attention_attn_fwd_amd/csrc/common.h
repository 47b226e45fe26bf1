// Device helpers shared by the gfx950 sink-attention kernels.
//
// MFMA lane layouts used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand (32 x 16, M x K): lane l supplies row m = l % 32 and the eight
//     K elements of slot group g = l / 32.
//   B operand (16 x 32, K x N): lane l supplies column n = l % 32 and the
//     eight K elements of slot group g = l / 32.
//   C/D (32 x 32): lane l holds column n = l % 32; accumulator register r
//     (0..15) holds row m = 8 * (r / 4) + 4 * g + (r % 4).
// A and B assign K elements to (slot group, slot) the same way, so a kernel
// may use any fixed map between its logical contraction index and
// (g, slot) as long as both operands use it.  Only the C/D row map is relied
// on as stated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gptoss {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kHeadDim = 64;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global load / store through uint4 (8 bf16).
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Round-to-nearest-even fp32 -> bf16 pairs (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// Sum of the two bf16 halves of w added to acc (v_dot2c_f32_bf16 against 1.0).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), ones, acc, false);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Value held by the lane 32 positions away (l ^ 32), via v_permlane32_swap.
// Returns (own, partner) combined by the caller through a symmetric op.
struct Pair { float a, b; };
__device__ __forceinline__ Pair swap32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return Pair{__int_as_float(r[0]), __int_as_float(r[1])};
}
__device__ __forceinline__ float max_across_halves(float x) {
    Pair p = swap32(x);
    return fmaxf(p.a, p.b);
}
__device__ __forceinline__ float sum_across_halves(float x) {
    Pair p = swap32(x);
    return p.a + p.b;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Row of the 32x32 accumulator held in register r by slot group g.
__device__ __forceinline__ constexpr int acc_row(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

// Swap bits 2 and 3 of a 0..31 row index (an involution).  An A operand whose
// lane m supplies row perm_row(m) leaves, in accumulator registers 8h..8h+7
// of slot group g, the 8 consecutive rows 16h + 8g + 0..7 -- exactly the
// K-slot order of a following MFMA that contracts over those rows.
__device__ __forceinline__ int perm_row(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// LDS tiles hold 64 rows x 64 bf16 with a row pitch of 144 bytes (9
// sixteen-byte units: 8 of data, 1 of padding).  gfx950 LDS has 64 four-byte
// banks; a 144-byte pitch puts consecutive rows 36 banks apart, so the 16
// rows read by one 16-lane ds_read_b128 phase (any 16 consecutive rows, in
// any order) land on distinct 4-bank groups, and two rows 8 apart fall in
// opposite bank halves.  Every address a lane uses is then its own base plus
// a compile-time offset.
constexpr int kTilePitch = 144;                 // bytes per row
constexpr int kTilePitchUnits = kTilePitch / 16;
constexpr int kTileUnits = 64 * kTilePitchUnits;  // uint4 per tile
__device__ __forceinline__ int tile_unit(int row, int unit) { return row * kTilePitchUnits + unit; }

// ds_read_b64_tr_b16: within each 16-lane block, lane i receives element
// (i % 4) of the 8-byte chunk addressed by block lane 4 j + i / 4, for
// j = 0..3.  If block lane s addresses tile[r0 + s / 4][c0 + 4 (s % 4)], lane
// i receives tile[r0 + j][c0 + i] for j = 0..3: a 4 x 16 transpose.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const void* lds_ptr) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
    return __builtin_bit_cast(uint2, r);
}

// Transposed 8-slot operand from a row-major tile: lane (block position
// i = lane % 16) receives tile[r0 + 0..7][c0 + i] where c0 is the first
// column of its 16-lane block.  Rows r0..r0+3 come from the first read,
// r0+4..r0+7 from the second.
__device__ __forceinline__ bf16x8 tile_read_tr8(const uint4* tile, int r0, int c0, int i) {
    const char* p = reinterpret_cast<const char*>(tile) + (r0 + (i >> 2)) * kTilePitch + (c0 + 4 * (i & 3)) * 2;
    const uint2 lo = lds_read_tr16(p);
    const uint2 hi = lds_read_tr16(p + 4 * kTilePitch);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// Element offset of row `row` (>= 0) of a tensor with `stride` elements per
// row, as one 32 x 32 -> 64-bit multiply (v_mad_u64_u32).  (A 64-bit stride
// makes the compiler add a high-half product whose don't-care addend
// register can alias a load still in flight, which costs a full wait.)
__device__ __forceinline__ size_t row_off(int row, uint32_t stride) { return (size_t)(uint32_t)row * stride; }

// Nearest bf16 (8 significant bits, ties to even) of the exact value
// hi + lo, as the 16-bit pattern, where lo is the exact remainder of an fp64
// sum hi (|lo| at most half an ulp of hi).  The fp64 significand is rounded
// at its 8th bit by integer addition on the bit pattern (a carry moves into
// the exponent as it should); when hi sits exactly on a bf16 midpoint, the
// sign of lo says on which side the exact value lies.
__device__ __forceinline__ uint32_t bf16_bits_of(double hi, double lo) {
    uint64_t b = (uint64_t)__double_as_longlong(hi);
    if ((b & ((1ull << 45) - 1)) == (1ull << 44) && lo != 0.0)
        b += ((lo > 0.0) == (hi > 0.0)) ? 1 : ~0ull;  // off the midpoint, towards the exact value
    b += ((1ull << 44) - 1) + ((b >> 45) & 1);
    b &= ~((1ull << 45) - 1);
    return __float_as_uint((float)__longlong_as_double((long long)b)) >> 16;
}

// x + y as an fp64 value and its exact remainder (Knuth's two-sum).
__device__ __forceinline__ void two_sum(double x, double y, double& hi, double& lo) {
#pragma clang fp contract(off)
    hi = x + y;
    const double yv = hi - x;
    lo = (x - (hi - yv)) + (y - yv);
}

// Rotary embedding of 8 element pairs: a holds elements i .. i+7 and b their
// partners i+32 .. i+39 (half-split pairing of a 64-wide head), cs the
// (cos, sin) pairs of i .. i+7 as four float4 {c_i, s_i, c_{i+1}, s_{i+1}}.
//   a' = a c - b s,  b' = b c + a s            (the rotation R)
// or, with transpose, the adjoint R^T that carries gradients back:
//   a' = a c + b s,  b' = b c - a s
// Each result is the exact value rounded once to bf16 (nearest even).  With
// bf16 a, b (8 significant bits) and fp32 c, s (24 bits) every product is
// exact in fp64 (32 bits); rope8 rounds their sum once to fp64 (a fused
// multiply-add) and that value to bf16, which is the exact value's rounding
// unless the fp64 value sits exactly on a bf16 midpoint.  rope8 returns
// true if that happened for some element; the caller then reloads a, b and
// cs and calls rope8_exact, which carries the sum with its exact remainder
// (two-sum) so that the remainder decides.  (The remainder is not formed
// always: its fp64 additions cost more than the rest of the rotation.)
__device__ __forceinline__ void rope_elem(const uint32_t (&aw)[4], const uint32_t (&bw)[4], const float4 (&cs)[4],
                                          bool transpose, int k, double& x0, double& x1, double& c, double& s) {
    const int u = k >> 1, e = k & 1;
    x0 = e ? bf16_hi(aw[u]) : bf16_lo(aw[u]);
    x1 = e ? bf16_hi(bw[u]) : bf16_lo(bw[u]);
    c = e ? cs[u].z : cs[u].x;
    const double sn = e ? cs[u].w : cs[u].y;
    s = transpose ? -sn : sn;
}

__device__ __forceinline__ bool rope8(uint4& a, uint4& b, const float4 (&cs)[4], bool transpose = false) {
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t w[2][4] = {};
    bool mid = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        double x0, x1, c, s;
        rope_elem(aw, bw, cs, transpose, k, x0, x1, c, s);
        const double h0 = fma(x0, c, -(x1 * s)), h1 = fma(x1, c, x0 * s);
        mid = mid || ((uint64_t)__double_as_longlong(h0) & ((1ull << 45) - 1)) == (1ull << 44) ||
              ((uint64_t)__double_as_longlong(h1) & ((1ull << 45) - 1)) == (1ull << 44);
        w[0][k >> 1] |= bf16_bits_of(h0, 0.0) << (16 * (k & 1));
        w[1][k >> 1] |= bf16_bits_of(h1, 0.0) << (16 * (k & 1));
    }
    a = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
    b = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
    return mid;
}

__device__ __forceinline__ void rope8_exact(uint4& a, uint4& b, const float4 (&cs)[4], bool transpose = false) {
#pragma clang fp contract(off)
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t w[2][4] = {};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        double x0, x1, c, s, h, lo;
        rope_elem(aw, bw, cs, transpose, k, x0, x1, c, s);
        two_sum(x0 * c, -(x1 * s), h, lo);
        w[0][k >> 1] |= bf16_bits_of(h, lo) << (16 * (k & 1));
        two_sum(x1 * c, x0 * s, h, lo);
        w[1][k >> 1] |= bf16_bits_of(h, lo) << (16 * (k & 1));
    }
    a = make_uint4(w[0][0], w[0][1], w[0][2], w[0][3]);
    b = make_uint4(w[1][0], w[1][1], w[1][2], w[1][3]);
}

// The adjoint rotation R^T on fp32 values: a[j] holds element i + j and b[j]
// its partner i + 32 + j (j = 0..3, i even), t0, t1 the (cos, sin) pairs of
// i .. i+3.  Products and sums rounded once to fp32, as in rope8.
__device__ __forceinline__ void rope4_adjoint_f32(float (&a)[4], float (&b)[4], const float4& t0,
                                                  const float4& t1) {
#pragma clang fp contract(off)
    const float c[4] = {t0.x, t0.z, t1.x, t1.z}, s[4] = {t0.y, t0.w, t1.y, t1.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float ya = a[j] * c[j] + b[j] * s[j];
        const float yb = b[j] * c[j] - a[j] * s[j];
        a[j] = ya;
        b[j] = yb;
    }
}

// The four (cos, sin) float4 of pairs i .. i+7 (i even) at `position` of a
// table of 32 pairs per position.
__device__ __forceinline__ void load_rope8(const float2* tab, int position, int i, float4 (&cs)[4]) {
    const float4* t = reinterpret_cast<const float4*>(tab + (size_t)position * 32 + i);
#pragma unroll
    for (int u = 0; u < 4; ++u) cs[u] = t[u];
}

// Rows of sequence b in a [token, head, d] tensor.  A dense batch
// (cu == nullptr) puts sequence b at rows b * S .. b * S + S - 1; a packed
// batch of variable-length documents puts it at rows cu[b] .. cu[b + 1] - 1,
// with the length capped at S (the longest document the grid covers).
// lse is [B][H][S] for a dense batch and [H][total rows] for a packed one:
// entry (b, h, pos) sits at lse_base + h * lse_hstride + pos.
struct SeqRows {
    int row0, len;
    size_t lse_base, lse_hstride;
};
__device__ __forceinline__ SeqRows seq_rows(const int* cu, int S, int H, int total_rows, int b) {
    SeqRows r;
    if (cu == nullptr) {
        r.row0 = b * S;
        r.len = S;
        r.lse_base = (size_t)b * H * S;
        r.lse_hstride = (size_t)S;
    } else {
        // clamped to [0, total_rows] so that offsets that break the contract
        // (negative, decreasing or past the end) cannot reach outside the
        // tensors; valid offsets pass unchanged
        r.row0 = min(max(cu[b], 0), total_rows);
        r.len = min(min(max(cu[b + 1], r.row0), total_rows) - r.row0, S);
        r.lse_base = (size_t)r.row0;
        r.lse_hstride = (size_t)total_rows;
    }
    return r;
}

}  // namespace gptoss
