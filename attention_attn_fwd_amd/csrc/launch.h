// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments are validated by the caller; launchers only plan grids and launch.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace gptoss {

struct FwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* sinks;
    uint16_t* out;
    float* lse;
    const int* cu;  // packed documents (sequence b = rows cu[b] .. cu[b+1]-1), nullptr = dense [B, S]
    const float2* rope;  // (cos, sin) table [positions][32]: q rotated at load; nullptr = no rotation
    int B, S, Hq, Hkv, window;  // packed: B = documents, S = longest document
    int T;                      // total token rows (B * S when dense)
    float scale;
};

struct BwdArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* sinks;
    const uint16_t* out;
    const float* lse;
    const uint16_t* dout;
    uint16_t* dq;
    uint16_t* dk;
    uint16_t* dv;
    float* dsinks;
    void* workspace;
    const int* cu;  // as in FwdArgs
    // RoPE (dense batches): q arrives unrotated and k rotated; the dq kernel
    // rotates q with this (cos, sin) table [position][32] and writes it to
    // q_rot (B*S*Hq*64 bf16) for dkdv, and dq, dk leave through the adjoint
    // rotation.  nullptr = no rotation.
    const float2* rope = nullptr;
    uint16_t* q_rot = nullptr;
    int B, S, Hq, Hkv, window;
    int T;
    float scale;
};

struct DecodeArgs {
    const uint16_t* q;
    const uint16_t* k_cache;      // contiguous cache, or the K pages when paged
    const uint16_t* v_cache;      // contiguous cache, or the V pages when paged
    const int* cu_seqlens;        // contiguous cache only
    const int* block_table;       // paged only: [N, pages_per_seq]
    const int* seq_lens;          // paged only: [N]
    const float* sinks;
    uint16_t* out;
    float* lse;
    void* workspace;
    int N, Hq, Hkv, max_seqlen, window;
    int page_size, pages_per_seq, ring_tokens;  // paged only (ring_tokens 0 = linear)
    const float2* rope;  // (cos, sin) table: q rotated at position L_n - 1; nullptr = no rotation
    float scale;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);

// Backward workspace: {lse * log2(e), Dvec} per (token row, head) as float2,
// then (256-byte aligned) one fp32 dsink term per (head, token row).
size_t bwd_ld_region_bytes(long long total_rows, int Hq);
size_t bwd_workspace_bytes(long long total_rows, int Hq);
hipError_t launch_bwd(const BwdArgs& a, hipStream_t stream);

// Decode split plan (host side, no device access).  A split workgroup
// covers kv_per_block KV heads (one wave each) of one sequence's chunk of
// chunk_keys visible keys (a multiple of kDecodeKeyTile); a sequence has at
// most n_splits chunks.  With more than one chunk the workspace holds one
// partial of kDecodePartStride floats per (sequence, query head, chunk).
// Windows of at most kDecodeSmallWindow keys (a sliding layer: visible
// lengths differ little) take 4 KV heads per workgroup; otherwise 2, and
// with one chunk per sequence and at most kDecodeRankMaxSeqs sequences the
// workgroups take the (sequence, head block) items in an order ranked by
// visible length (the split kernel ranks them itself).
constexpr int kDecodeSmallWindow = 256;
constexpr int kDecodeMinKvPerBlock = 2;  // the most workgroup rows a launch can have
constexpr int kDecodeRankMaxSeqs = 256;
constexpr int decode_kv_per_block(int window) { return window > 0 && window <= kDecodeSmallWindow ? 4 : 2; }
constexpr int kDecodeKeyTile = 64;
constexpr int kDecodePartStride = 68;  // O[64], m, l, pad
struct DecodePlan {
    int chunk_keys, n_splits;
    size_t workspace_bytes;
};
DecodePlan decode_plan(int N, int Hq, int Hkv, int max_seqlen, int window);
size_t decode_workspace_bytes(int N, int Hq, int Hkv, int max_seqlen, int window);

hipError_t launch_rope_table(float2* tab, int P, double base, double factor, double orig_ctx, double alpha,
                             double beta, hipStream_t stream);
hipError_t launch_rope_rows(const uint16_t* x, uint16_t* y, const int* positions, const float2* tab, int tab_len,
                            long long rows, int H, int S, bool transpose, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Decode with the split partials in a library-owned device array of
// kDecodeNoAllocScratchBytes per GPU instead of a.workspace (ignored);
// plans needing more must be refused by the caller.
constexpr size_t kDecodeNoAllocScratchBytes = 4u << 20;
hipError_t launch_decode_noalloc(const DecodeArgs& a, hipStream_t stream);

}  // namespace gptoss
