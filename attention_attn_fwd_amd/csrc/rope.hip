// Rotary position embedding with YaRN frequency scaling (gfx950): the table
// kernel and a row-rotation kernel.  The forward and decode kernels rotate q
// in their prologue with the same table (rope8 in common.h).
//
// Megatron-LM issue "gpt-oss implementation", "Positional Encodings / YaRN
// RoPE Scaling", names YaRN and cites the YaRN paper (arXiv:2309.00071),
// whose definitions are used: pair i of a 64-wide head has base frequency
// theta_i = base^(-2i/64); it turns r_i = L theta_i / (2 pi) times over the
// original context L; with gamma = clamp((r - alpha) / (beta - alpha), 0, 1)
// its frequency becomes h_i = (1 - gamma) theta_i / s + gamma theta_i, and
// both q and k are multiplied by the temperature m = 0.1 ln s + 1 (1 for
// s = 1).  Pairs are (i, i + 32).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace gptoss {
namespace {

constexpr int kPairs = kHeadDim / 2;

// tab[p][i] = (m cos(p h_i), m sin(p h_i)), evaluated in fp64 and rounded to
// fp32; one thread per (position, pair).
__global__ void __launch_bounds__(256) rope_table_kernel(float2* tab, long long n, double base, double factor,
                                                          double orig_ctx, double alpha, double beta,
                                                          double mscale) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n) return;
    const int p = (int)(idx / kPairs), i = (int)(idx % kPairs);
    const double th = pow(base, -2.0 * i / kHeadDim);
    double h = th;
    if (factor != 1.0) {
        const double r = orig_ctx * th / (2.0 * M_PI);
        double g = (r - alpha) / (beta - alpha);
        g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
        h = (1.0 - g) * th / factor + g * th;
    }
    const double a = (double)p * h;
    tab[idx] = make_float2((float)(mscale * cos(a)), (float)(mscale * sin(a)));
}

// Rotates rows [T, H, 64] (bf16) by their token's position: positions[t]
// (clamped into the table) or, when positions is null, t mod S (a dense
// [B, S, H, 64] tensor); transpose applies R^T (gradients).  One thread per
// (row, 8-pair octet); y may be x.
__global__ void __launch_bounds__(256) rope_rows_kernel(const uint16_t* x, uint16_t* y, const int* positions,
                                                         const float2* tab, int tab_len, long long rows, int H,
                                                         int S, int transpose) {
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= rows * 4) return;
    const long long row = idx >> 2;
    const int o = (int)(idx & 3);
    const long long tok = row / H;
    int pos = positions != nullptr ? positions[tok] : (int)(tok % S);
    pos = pos < 0 ? 0 : (pos >= tab_len ? tab_len - 1 : pos);
    const uint16_t* src = x + row * kHeadDim + 8 * o;
    uint4 a = ld16(src), b = ld16(src + kPairs);
    float4 cs[4];
    load_rope8(tab, pos, 8 * o, cs);
    if (__any(rope8(a, b, cs, transpose != 0))) {
        // (rare) an fp64 sum on a bf16 midpoint: rotate again from the
        // inputs with exact remainders (before any store: y may be x)
        a = ld16(src);
        b = ld16(src + kPairs);
        rope8_exact(a, b, cs, transpose != 0);
    }
    uint16_t* dst = y + row * kHeadDim + 8 * o;
    st16(dst, a);
    st16(dst + kPairs, b);
}

}  // namespace

hipError_t launch_rope_table(float2* tab, int P, double base, double factor, double orig_ctx, double alpha,
                             double beta, hipStream_t stream) {
    const long long n = (long long)P * kPairs;
    const double mscale = factor > 1.0 ? 0.1 * log(factor) + 1.0 : 1.0;
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, tab, n, base, factor,
                       orig_ctx, alpha, beta, mscale);
    return hipGetLastError();
}

hipError_t launch_rope_rows(const uint16_t* x, uint16_t* y, const int* positions, const float2* tab, int tab_len,
                            long long rows, int H, int S, bool transpose, hipStream_t stream) {
    const long long blocks = (rows * 4 + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, y, positions, tab, tab_len,
                       rows, H, S, transpose ? 1 : 0);
    return hipGetLastError();
}

}  // namespace gptoss
