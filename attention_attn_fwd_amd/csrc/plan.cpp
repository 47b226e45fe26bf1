// Host-side planning shared by the C ABI and the launchers: workspace sizes
// and the decode split plan.  No device code and no HIP calls, so the host
// layer (this file and api.cpp) also builds with a plain C++ compiler.
#include <algorithm>

#include "launch.h"

namespace gptoss {

namespace {
constexpr size_t align256(size_t n) { return (n + 255) / 256 * 256; }
// Decode split workgroups the plan aims for: two per CU (a workgroup is two
// waves).  A sequence is cut into chunks only when there are too few
// (sequence, KV-head block) pairs to fill the chip; every chunk but the last
// per sequence costs a partial write and read plus the merge launch, which
// on the 128 x U{1..1024} workload cost more than they gain.
constexpr long long kDecodeTargetWorkgroups = 512;
// Shortest chunk the plan cuts (a multiple of the key tile).  Two tiles:
// a one-tile chunk saves less than the merge launch it brings (a sliding
// layer's 128 visible keys decode fastest unsplit).
constexpr long long kDecodeMinChunkKeys = 2 * kDecodeKeyTile;
static_assert(kDecodeMinChunkKeys % kDecodeKeyTile == 0, "chunks hold whole key tiles");
}  // namespace

size_t bwd_ld_region_bytes(long long total_rows, int Hq) {
    return align256((size_t)total_rows * Hq * 2 * sizeof(float));
}

size_t bwd_workspace_bytes(long long total_rows, int Hq) {
    return bwd_ld_region_bytes(total_rows, Hq) + (size_t)total_rows * Hq * sizeof(float);
}

DecodePlan decode_plan(int N, int Hq, int Hkv, int max_seqlen, int window) {
    // 64-bit throughout: max_seqlen may be up to 2^30 (the entry points
    // refuse more), and none of the roundings below may wrap
    const int G = Hq / Hkv;
    const long long vis = window > 0 ? std::min<long long>(max_seqlen, window) : (long long)max_seqlen;
    const long long groups =
        (long long)N * ((Hkv + decode_kv_per_block(window) - 1) / decode_kv_per_block(window)) * ((G + 31) / 32);
    const long long want = std::max(1LL, (kDecodeTargetWorkgroups + groups - 1) / std::max(1LL, groups));
    const long long max_chunks = std::max(1LL, (vis + kDecodeMinChunkKeys - 1) / kDecodeMinChunkKeys);
    const long long n = std::min(want, max_chunks);
    long long keys = (vis + n - 1) / n;
    keys = std::max<long long>(kDecodeMinChunkKeys, (keys + kDecodeKeyTile - 1) / kDecodeKeyTile * kDecodeKeyTile);
    const long long chunks = std::max(1LL, (vis + keys - 1) / keys);
    DecodePlan p;
    p.chunk_keys = (int)keys;
    p.n_splits = (int)chunks;
    p.workspace_bytes = chunks > 1 ? (size_t)N * Hq * (size_t)chunks * kDecodePartStride * sizeof(float) : 0;
    return p;
}

size_t decode_workspace_bytes(int N, int Hq, int Hkv, int max_seqlen, int window) {
    return decode_plan(N, Hq, Hkv, max_seqlen, window).workspace_bytes;
}

}  // namespace gptoss
