// C ABI of the sink-attention library: argument validation, device check,
// workspace sizing and dispatch to the gfx950 kernels.  Every argument error
// is caught here, before any HIP call, and reported through a status code
// plus a per-thread message.
#include "gptoss_attn.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

gptoss_status fail(gptoss_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

gptoss_status ok() {
    g_last_error.clear();
    return GPTOSS_OK;
}

// Kernels index token rows in int32 and round row counts up to whole tiles
// (at most 256 rows), so row counts stay 2^16 below 2^31.
constexpr long long kIndexLimit = (1LL << 31) - (1LL << 16);
// Decode: the longest sequence a call may name (2^30 tokens; one KV head of
// it alone is 256 GB of bf16 K and V), so that chunk arithmetic fits int32.
constexpr int kMaxDecodeSeqlen = 1 << 30;

gptoss_status check_decode_seqlen(int max_seqlen) {
    if (max_seqlen < 1) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "max_seqlen (%d) must be >= 1", max_seqlen);
    if (max_seqlen > kMaxDecodeSeqlen)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "max_seqlen (%d) exceeds 2^30", max_seqlen);
    return GPTOSS_OK;
}

// Decode launches ceil(Hkv / 2) * ceil(G / 32) workgroup rows per sequence
// chunk, at most 65535; the bound also keeps a K/V tile's row offsets (64
// rows of Hkv * 128 bytes) below 2^32, which the split kernel relies on.
gptoss_status check_decode_heads(int Hq, int Hkv) {
    const long long rows = (long long)((Hkv + gptoss::kDecodeMinKvPerBlock - 1) / gptoss::kDecodeMinKvPerBlock) *
                           ((Hq / Hkv + 31) / 32);
    if (rows > 65535)
        return fail(GPTOSS_ERR_UNSUPPORTED, "decode of %d KV heads needs %lld workgroup rows, more than 65535",
                    Hkv, rows);
    return GPTOSS_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

#define CHECK_PTR(p, align)                                                                  \
    do {                                                                                     \
        if ((p) == nullptr) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "%s is NULL", #p);      \
        if (!aligned((p), (align)))                                                          \
            return fail(GPTOSS_ERR_INVALID_ARGUMENT, "%s is not %d-byte aligned", #p, (int)(align)); \
    } while (0)

// Heads / dims / window / scale checks shared by the three entry points.
gptoss_status check_common(int Hq, int Hkv, int D, int window, float scale) {
    if (Hq < 1 || Hkv < 1)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "Hq (%d) and Hkv (%d) must be >= 1", Hq, Hkv);
    if (Hq % Hkv != 0)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "Hq (%d) is not a multiple of Hkv (%d)", Hq, Hkv);
    if (window < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "window (%d) must be >= 0", window);
    if (!std::isfinite(scale) || !(scale > 0.0f))
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "softmax_scale (%g) must be finite and > 0", (double)scale);
    if (D != 64) return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", D);
    if (Hq / Hkv > 128)
        return fail(GPTOSS_ERR_UNSUPPORTED, "group size Hq/Hkv = %d exceeds 128", Hq / Hkv);
    return GPTOSS_OK;
}

// gfx950 check, cached per device (0 = unknown, 1 = ok, 2 = not gfx950) in a
// table sized once, from the process's device count, on first use (every
// index hipGetDevice can return has an entry; if the count cannot be read
// the table is empty and every call asks the runtime again).
std::once_flag g_dev_once;
std::unique_ptr<std::atomic<int>[]> g_dev_ok;
int g_dev_count = 0;

gptoss_status check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(GPTOSS_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    std::call_once(g_dev_once, [] {
        int n = 0;
        if (hipGetDeviceCount(&n) != hipSuccess || n < 0) n = 0;
        g_dev_ok.reset(new std::atomic<int>[n > 0 ? n : 1]);
        for (int i = 0; i < (n > 0 ? n : 1); ++i) g_dev_ok[i].store(0, std::memory_order_relaxed);
        g_dev_count = n;
    });
    const bool cached = dev >= 0 && dev < g_dev_count;
    if (cached && g_dev_ok[dev].load(std::memory_order_relaxed) == 1) return GPTOSS_OK;
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(GPTOSS_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (cached) g_dev_ok[dev].store(is950 ? 1 : 2, std::memory_order_relaxed);
    if (!is950)
        return fail(GPTOSS_ERR_UNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                    prop.gcnArchName);
    return GPTOSS_OK;
}

gptoss_status launched(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(GPTOSS_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

int gptoss_attn_abi_version(void) { return GPTOSS_ATTN_ABI_VERSION; }

const char* gptoss_attn_last_error(void) { return g_last_error.c_str(); }

gptoss_status gptoss_attn_fwd(const void* q, const void* k, const void* v, const float* sinks, int B, int S,
                              int Hq, int Hkv, int D, int window, float softmax_scale, void* out, float* lse,
                              void* stream) {
    if (B < 0 || S < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B (%d) and S (%d) must be >= 0", B, S);
    gptoss_status st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    if (B == 0 || S == 0) return ok();
    if ((long long)B * S > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B*S = %lld exceeds 2^31 - 2^16", (long long)B * S);
    CHECK_PTR(q, 16);
    CHECK_PTR(k, 16);
    CHECK_PTR(v, 16);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::FwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.sinks = sinks;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.cu = nullptr;
    a.rope = nullptr;
    a.B = B;
    a.S = S;
    a.T = B * S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.scale = softmax_scale;
    return launched(gptoss::launch_fwd(a, static_cast<hipStream_t>(stream)), "forward");
}

size_t gptoss_attn_bwd_workspace_size(int B, int S, int Hq, int Hkv, int D, int window) {
    if (B <= 0 || S <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D != 64 || window < 0) return 0;
    return gptoss::bwd_workspace_bytes((long long)B * S, Hq);
}

gptoss_status gptoss_attn_bwd(const void* q, const void* k, const void* v, const float* sinks, const void* out,
                              const float* lse, const void* dout, int B, int S, int Hq, int Hkv, int D,
                              int window, float softmax_scale, void* dq, void* dk, void* dv, float* dsinks,
                              void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || S < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B (%d) and S (%d) must be >= 0", B, S);
    gptoss_status st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    if (B == 0 || S == 0) return ok();
    if ((long long)B * S > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B*S = %lld exceeds 2^31 - 2^16", (long long)B * S);
    CHECK_PTR(q, 16);
    CHECK_PTR(k, 16);
    CHECK_PTR(v, 16);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    CHECK_PTR(dout, 16);
    CHECK_PTR(dq, 16);
    CHECK_PTR(dk, 16);
    CHECK_PTR(dv, 16);
    CHECK_PTR(dsinks, 4);
    const size_t need = gptoss::bwd_workspace_bytes((long long)B * S, Hq);
    if (workspace_bytes < need)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "workspace_bytes %zu < required %zu", workspace_bytes, need);
    if (need > 0) CHECK_PTR(workspace, 256);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::BwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.sinks = sinks;
    a.out = static_cast<const uint16_t*>(out);
    a.lse = lse;
    a.dout = static_cast<const uint16_t*>(dout);
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.dsinks = dsinks;
    a.workspace = workspace;
    a.cu = nullptr;
    a.B = B;
    a.S = S;
    a.T = B * S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.scale = softmax_scale;
    return launched(gptoss::launch_bwd(a, static_cast<hipStream_t>(stream)), "backward");
}

// Packed variable-length batches: shape checks shared by the two entry points.
static gptoss_status check_varlen(int N, int T, int max_seqlen) {
    if (N < 0 || T < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) and T (%d) must be >= 0", N, T);
    if (max_seqlen < 1) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "max_seqlen (%d) must be >= 1", max_seqlen);
    if (N > 65535) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) exceeds 65535 documents per call", N);
    if ((long long)T > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "T = %d exceeds 2^31 - 2^16", T);
    return GPTOSS_OK;
}

gptoss_status gptoss_attn_fwd_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens,
                                     const float* sinks, int N, int T, int Hq, int Hkv, int D, int max_seqlen,
                                     int window, float softmax_scale, void* out, float* lse, void* stream) {
    gptoss_status st = check_varlen(N, T, max_seqlen);
    if (st != GPTOSS_OK) return st;
    st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    if (N == 0 || T == 0) return ok();
    CHECK_PTR(q, 16);
    CHECK_PTR(k, 16);
    CHECK_PTR(v, 16);
    CHECK_PTR(cu_seqlens, 4);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::FwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.sinks = sinks;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.cu = cu_seqlens;
    a.rope = nullptr;
    a.B = N;
    a.S = max_seqlen < T ? max_seqlen : T;  // no document is longer than the T rows
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.scale = softmax_scale;
    return launched(gptoss::launch_fwd(a, static_cast<hipStream_t>(stream)), "varlen forward");
}

size_t gptoss_attn_bwd_varlen_workspace_size(int T, int Hq, int Hkv, int D) {
    if (T <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D != 64) return 0;
    return gptoss::bwd_workspace_bytes(T, Hq);
}

gptoss_status gptoss_attn_bwd_varlen(const void* q, const void* k, const void* v, const int* cu_seqlens,
                                     const float* sinks, const void* out, const float* lse, const void* dout, int N,
                                     int T, int Hq, int Hkv, int D, int max_seqlen, int window, float softmax_scale,
                                     void* dq, void* dk, void* dv, float* dsinks, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    gptoss_status st = check_varlen(N, T, max_seqlen);
    if (st != GPTOSS_OK) return st;
    st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    if (N == 0 || T == 0) return ok();
    CHECK_PTR(q, 16);
    CHECK_PTR(k, 16);
    CHECK_PTR(v, 16);
    CHECK_PTR(cu_seqlens, 4);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    CHECK_PTR(dout, 16);
    CHECK_PTR(dq, 16);
    CHECK_PTR(dk, 16);
    CHECK_PTR(dv, 16);
    CHECK_PTR(dsinks, 4);
    const size_t need = gptoss::bwd_workspace_bytes(T, Hq);
    if (workspace_bytes < need)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "workspace_bytes %zu < required %zu", workspace_bytes, need);
    CHECK_PTR(workspace, 256);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::BwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.sinks = sinks;
    a.out = static_cast<const uint16_t*>(out);
    a.lse = lse;
    a.dout = static_cast<const uint16_t*>(dout);
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.dsinks = dsinks;
    a.workspace = workspace;
    a.cu = cu_seqlens;
    a.B = N;
    a.S = max_seqlen < T ? max_seqlen : T;  // no document is longer than the T rows
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.scale = softmax_scale;
    return launched(gptoss::launch_bwd(a, static_cast<hipStream_t>(stream)), "varlen backward");
}

size_t gptoss_attn_decode_workspace_size(int N, int Hq, int Hkv, int D, int max_seqlen, int window) {
    if (N <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D != 64 || max_seqlen < 1 || window < 0) return 0;
    if (max_seqlen > kMaxDecodeSeqlen) return 0;
    return gptoss::decode_workspace_bytes(N, Hq, Hkv, max_seqlen, window);
}

// The packed-cache decode, with the caller's workspace or (noalloc) the
// library's per-GPU scratch array.
static gptoss_status decode_entry(const void* q, const void* k_cache, const void* v_cache, const int* cu_seqlens,
                                  const float* sinks, int N, int Hq, int Hkv, int D, int max_seqlen, int window,
                                  float softmax_scale, void* out, float* lse, bool noalloc, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (N < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) must be >= 0", N);
    gptoss_status st = check_decode_seqlen(max_seqlen);
    if (st != GPTOSS_OK) return st;
    st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    st = check_decode_heads(Hq, Hkv);
    if (st != GPTOSS_OK) return st;
    if (N == 0) return ok();
    if ((long long)N > 65535)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) exceeds 65535 sequences per call", N);
    CHECK_PTR(q, 16);
    CHECK_PTR(k_cache, 16);
    CHECK_PTR(v_cache, 16);
    CHECK_PTR(cu_seqlens, 4);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    const size_t need = gptoss::decode_workspace_bytes(N, Hq, Hkv, max_seqlen, window);
    if (noalloc) {
        if (need > gptoss::kDecodeNoAllocScratchBytes)
            return fail(GPTOSS_ERR_INVALID_ARGUMENT,
                        "this decode needs %zu bytes of split partials; the no-allocation entry point holds %zu "
                        "(use gptoss_attn_decode with a workspace)",
                        need, gptoss::kDecodeNoAllocScratchBytes);
    } else {
        if (workspace_bytes < need)
            return fail(GPTOSS_ERR_INVALID_ARGUMENT, "workspace_bytes %zu < required %zu", workspace_bytes, need);
        if (need > 0) CHECK_PTR(workspace, 256);
    }
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint16_t*>(k_cache);
    a.v_cache = static_cast<const uint16_t*>(v_cache);
    a.cu_seqlens = cu_seqlens;
    a.block_table = nullptr;
    a.seq_lens = nullptr;
    a.sinks = sinks;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.workspace = noalloc ? nullptr : workspace;
    a.N = N;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.max_seqlen = max_seqlen;
    a.window = window;
    a.page_size = 0;
    a.pages_per_seq = 0;
    a.ring_tokens = 0;
    a.rope = nullptr;
    a.scale = softmax_scale;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (noalloc) return launched(gptoss::launch_decode_noalloc(a, s), "decode (no allocation)");
    return launched(gptoss::launch_decode(a, s), "decode");
}

gptoss_status gptoss_attn_decode(const void* q, const void* k_cache, const void* v_cache, const int* cu_seqlens,
                                 const float* sinks, int N, int Hq, int Hkv, int D, int max_seqlen, int window,
                                 float softmax_scale, void* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
    return decode_entry(q, k_cache, v_cache, cu_seqlens, sinks, N, Hq, Hkv, D, max_seqlen, window, softmax_scale,
                        out, lse, false, workspace, workspace_bytes, stream);
}

gptoss_status gptoss_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                         const int* cu_seqlens, const float* sinks, int N, int Hq, int Hkv, int D,
                                         int max_seqlen, int window, float softmax_scale, void* out, float* lse,
                                         void* stream) {
    return decode_entry(q, k_cache, v_cache, cu_seqlens, sinks, N, Hq, Hkv, D, max_seqlen, window, softmax_scale,
                        out, lse, true, nullptr, 0, stream);
}

static bool is_pow2(long long x) { return x > 0 && (x & (x - 1)) == 0; }

gptoss_status gptoss_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                       const int* block_table, const int* seq_lens, const float* sinks, int N,
                                       int Hq, int Hkv, int D, int page_size, int pages_per_seq, int ring_tokens,
                                       int max_seqlen, int window, float softmax_scale, void* out, float* lse,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (N < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) must be >= 0", N);
    gptoss_status st = check_decode_seqlen(max_seqlen);
    if (st != GPTOSS_OK) return st;
    st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    st = check_decode_heads(Hq, Hkv);
    if (st != GPTOSS_OK) return st;
    if (!is_pow2(page_size) || page_size > 65536)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "page_size (%d) must be a power of two in [1, 65536]", page_size);
    if (pages_per_seq < 1) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "pages_per_seq (%d) must be >= 1", pages_per_seq);
    if (ring_tokens < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "ring_tokens (%d) must be >= 0", ring_tokens);
    if (ring_tokens == 0) {
        if ((long long)max_seqlen > (long long)pages_per_seq * page_size)
            return fail(GPTOSS_ERR_INVALID_ARGUMENT,
                        "linear cache: max_seqlen (%d) exceeds pages_per_seq * page_size (%lld)", max_seqlen,
                        (long long)pages_per_seq * page_size);
    } else {
        if (window < 1 || window > ring_tokens)
            return fail(GPTOSS_ERR_INVALID_ARGUMENT,
                        "ring cache of %d tokens needs a window in [1, %d] (got %d)", ring_tokens, ring_tokens,
                        window);
        if (!is_pow2(ring_tokens) || ring_tokens % page_size != 0)
            return fail(GPTOSS_ERR_INVALID_ARGUMENT,
                        "ring_tokens (%d) must be a power of two and a multiple of page_size (%d)", ring_tokens,
                        page_size);
        if (ring_tokens / page_size > pages_per_seq)
            return fail(GPTOSS_ERR_INVALID_ARGUMENT, "ring of %d tokens needs %d pages, pages_per_seq is %d",
                        ring_tokens, ring_tokens / page_size, pages_per_seq);
    }
    if (N == 0) return ok();
    if ((long long)N > 65535)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) exceeds 65535 sequences per call", N);
    if ((long long)N * pages_per_seq > 0x7fffffffLL)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "block table of %d x %d entries is too large", N, pages_per_seq);
    CHECK_PTR(q, 16);
    CHECK_PTR(k_pages, 16);
    CHECK_PTR(v_pages, 16);
    CHECK_PTR(block_table, 4);
    CHECK_PTR(seq_lens, 4);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    const size_t need = gptoss::decode_workspace_bytes(N, Hq, Hkv, max_seqlen, window);
    if (workspace_bytes < need)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "workspace_bytes %zu < required %zu", workspace_bytes, need);
    if (need > 0) CHECK_PTR(workspace, 256);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint16_t*>(k_pages);
    a.v_cache = static_cast<const uint16_t*>(v_pages);
    a.cu_seqlens = nullptr;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.sinks = sinks;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.workspace = workspace;
    a.N = N;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.max_seqlen = max_seqlen;
    a.window = window;
    a.page_size = page_size;
    a.pages_per_seq = pages_per_seq;
    a.ring_tokens = ring_tokens;
    a.rope = nullptr;
    a.scale = softmax_scale;
    return launched(gptoss::launch_decode(a, static_cast<hipStream_t>(stream)), "paged decode");
}

// ---------------------------------------------------------------------------
// Rotary embedding with YaRN scaling.

static gptoss_status check_rope_params(int P, int D, double base, double factor, double orig_ctx, double alpha,
                                       double beta) {
    if (D != 64) return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", D);
    if (P < 1) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "table positions (%d) must be >= 1", P);
    if (!std::isfinite(base) || !(base > 1.0))
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "rope base (%g) must be finite and > 1", base);
    if (!std::isfinite(factor) || !(factor >= 1.0))
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "YaRN factor (%g) must be finite and >= 1", factor);
    if (factor > 1.0) {
        if (!std::isfinite(orig_ctx) || !(orig_ctx >= 1.0))
            return fail(GPTOSS_ERR_INVALID_ARGUMENT, "original context (%g) must be >= 1", orig_ctx);
        if (!std::isfinite(alpha) || !std::isfinite(beta) || !(beta > alpha))
            return fail(GPTOSS_ERR_INVALID_ARGUMENT, "YaRN ramp needs finite alpha < beta (got %g, %g)", alpha, beta);
    }
    return GPTOSS_OK;
}

gptoss_status gptoss_attn_rope_table(float* table, int positions, int D, double base, double factor,
                                     double orig_ctx, double alpha, double beta, void* stream) {
    gptoss_status st = check_rope_params(positions, D, base, factor, orig_ctx, alpha, beta);
    if (st != GPTOSS_OK) return st;
    if ((long long)positions * (D / 2) > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "table of %d positions is too large", positions);
    CHECK_PTR(table, 16);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    return launched(gptoss::launch_rope_table(reinterpret_cast<float2*>(table), positions, base, factor, orig_ctx,
                                              alpha, beta, static_cast<hipStream_t>(stream)),
                    "rope table");
}

gptoss_status gptoss_attn_rope_rows(const void* x, void* y, const int* positions, int T, int H, int D,
                                    const float* table, int table_positions, int transpose, void* stream) {
    if (T < 0 || H < 1) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "T (%d) must be >= 0 and H (%d) >= 1", T, H);
    if (D != 64) return fail(GPTOSS_ERR_UNSUPPORTED, "head_dim %d is not supported (only 64)", D);
    if (table_positions < 1)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "table_positions (%d) must be >= 1", table_positions);
    if (T == 0) return ok();
    if ((long long)T * H > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "T*H = %lld rows exceeds 2^31-1", (long long)T * H);
    CHECK_PTR(x, 16);
    CHECK_PTR(y, 16);
    CHECK_PTR(positions, 4);
    CHECK_PTR(table, 16);
    gptoss_status st = check_device();
    if (st != GPTOSS_OK) return st;
    return launched(gptoss::launch_rope_rows(static_cast<const uint16_t*>(x), static_cast<uint16_t*>(y), positions,
                                             reinterpret_cast<const float2*>(table), table_positions,
                                             (long long)T * H, H, 1, transpose != 0,
                                             static_cast<hipStream_t>(stream)),
                    "rope rows");
}

gptoss_status gptoss_attn_fwd_rope(const void* q, const void* k, const void* v, const float* sinks,
                                   const float* table, int table_positions, int B, int S, int Hq, int Hkv, int D,
                                   int window, float softmax_scale, void* out, float* lse, void* k_rot,
                                   void* stream) {
    if (B < 0 || S < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B (%d) and S (%d) must be >= 0", B, S);
    gptoss_status st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    if (B == 0 || S == 0) return ok();
    if ((long long)B * S > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B*S = %lld exceeds 2^31 - 2^16", (long long)B * S);
    if (table_positions < S)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "rope table holds %d positions, S is %d", table_positions, S);
    CHECK_PTR(q, 16);
    CHECK_PTR(k, 16);
    CHECK_PTR(v, 16);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(table, 16);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    CHECK_PTR(k_rot, 16);
    if (k_rot == k) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "k_rot must not alias k");
    st = check_device();
    if (st != GPTOSS_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float2* tab = reinterpret_cast<const float2*>(table);
    hipError_t e = gptoss::launch_rope_rows(static_cast<const uint16_t*>(k), static_cast<uint16_t*>(k_rot), nullptr,
                                            tab, table_positions, (long long)B * S * Hkv, Hkv, S, false, s);
    if (e != hipSuccess) return launched(e, "rope on k");
    gptoss::FwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_rot);
    a.v = static_cast<const uint16_t*>(v);
    a.sinks = sinks;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.cu = nullptr;
    a.rope = tab;
    a.B = B;
    a.S = S;
    a.T = B * S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.scale = softmax_scale;
    return launched(gptoss::launch_fwd(a, s), "forward with rope");
}

gptoss_status gptoss_attn_decode_rope(const void* q, const void* k_cache, const void* v_cache, const int* cu_seqlens,
                                      const float* sinks, const float* table, int table_positions, int N, int Hq,
                                      int Hkv, int D, int max_seqlen, int window, float softmax_scale, void* out,
                                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    if (N < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) must be >= 0", N);
    gptoss_status st = check_decode_seqlen(max_seqlen);
    if (st != GPTOSS_OK) return st;
    st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    st = check_decode_heads(Hq, Hkv);
    if (st != GPTOSS_OK) return st;
    if (table_positions < max_seqlen)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "rope table holds %d positions, max_seqlen is %d", table_positions,
                    max_seqlen);
    if (N == 0) return ok();
    if ((long long)N > 65535)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "N (%d) exceeds 65535 sequences per call", N);
    CHECK_PTR(q, 16);
    CHECK_PTR(k_cache, 16);
    CHECK_PTR(v_cache, 16);
    CHECK_PTR(cu_seqlens, 4);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(table, 16);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    const size_t need = gptoss::decode_workspace_bytes(N, Hq, Hkv, max_seqlen, window);
    if (workspace_bytes < need)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "workspace_bytes %zu < required %zu", workspace_bytes, need);
    if (need > 0) CHECK_PTR(workspace, 256);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    gptoss::DecodeArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const uint16_t*>(k_cache);
    a.v_cache = static_cast<const uint16_t*>(v_cache);
    a.cu_seqlens = cu_seqlens;
    a.block_table = nullptr;
    a.seq_lens = nullptr;
    a.sinks = sinks;
    a.out = static_cast<uint16_t*>(out);
    a.lse = lse;
    a.workspace = workspace;
    a.N = N;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.max_seqlen = max_seqlen;
    a.window = window;
    a.page_size = 0;
    a.pages_per_seq = 0;
    a.ring_tokens = 0;
    a.rope = reinterpret_cast<const float2*>(table);
    a.scale = softmax_scale;
    return launched(gptoss::launch_decode(a, static_cast<hipStream_t>(stream)), "decode with rope");
}

// Backward through the rotation: q is rotated into the workspace, the
// backward runs on the rotated q and k, and dq, dk are carried back through
// R^T in place.
static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t gptoss_attn_bwd_rope_workspace_size(int B, int S, int Hq, int Hkv, int D) {
    if (B <= 0 || S <= 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || D != 64) return 0;
    return align256((size_t)B * S * Hq * D * 2) + gptoss::bwd_workspace_bytes((long long)B * S, Hq);
}

gptoss_status gptoss_attn_bwd_rope(const void* q, const void* k_rot, const void* v, const float* sinks,
                                   const float* table, int table_positions, const void* out, const float* lse,
                                   const void* dout, int B, int S, int Hq, int Hkv, int D, int window,
                                   float softmax_scale, void* dq, void* dk, void* dv, float* dsinks,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    if (B < 0 || S < 0) return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B (%d) and S (%d) must be >= 0", B, S);
    gptoss_status st = check_common(Hq, Hkv, D, window, softmax_scale);
    if (st != GPTOSS_OK) return st;
    if (B == 0 || S == 0) return ok();
    if ((long long)B * S > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B*S = %lld exceeds 2^31 - 2^16", (long long)B * S);
    if ((long long)B * S * Hq > kIndexLimit)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "B*S*Hq = %lld rows exceeds 2^31-1", (long long)B * S * Hq);
    if (table_positions < S)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "rope table holds %d positions, S is %d", table_positions, S);
    CHECK_PTR(q, 16);
    CHECK_PTR(k_rot, 16);
    CHECK_PTR(v, 16);
    CHECK_PTR(sinks, 4);
    CHECK_PTR(table, 16);
    CHECK_PTR(out, 16);
    CHECK_PTR(lse, 4);
    CHECK_PTR(dout, 16);
    CHECK_PTR(dq, 16);
    CHECK_PTR(dk, 16);
    CHECK_PTR(dv, 16);
    CHECK_PTR(dsinks, 4);
    const size_t need = gptoss_attn_bwd_rope_workspace_size(B, S, Hq, Hkv, D);
    if (workspace_bytes < need)
        return fail(GPTOSS_ERR_INVALID_ARGUMENT, "workspace_bytes %zu < required %zu", workspace_bytes, need);
    CHECK_PTR(workspace, 256);
    st = check_device();
    if (st != GPTOSS_OK) return st;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const float2* tab = reinterpret_cast<const float2*>(table);
    uint16_t* q_rot = static_cast<uint16_t*>(workspace);
    void* bwd_ws = static_cast<char*>(workspace) + align256((size_t)B * S * Hq * D * 2);
    gptoss::BwdArgs a;
    a.q = static_cast<const uint16_t*>(q);
    a.k = static_cast<const uint16_t*>(k_rot);
    a.v = static_cast<const uint16_t*>(v);
    a.sinks = sinks;
    a.out = static_cast<const uint16_t*>(out);
    a.lse = lse;
    a.dout = static_cast<const uint16_t*>(dout);
    a.dq = static_cast<uint16_t*>(dq);
    a.dk = static_cast<uint16_t*>(dk);
    a.dv = static_cast<uint16_t*>(dv);
    a.dsinks = dsinks;
    a.workspace = bwd_ws;
    a.cu = nullptr;
    a.rope = tab;
    a.q_rot = q_rot;
    a.B = B;
    a.S = S;
    a.T = B * S;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.window = window;
    a.scale = softmax_scale;
    return launched(gptoss::launch_bwd(a, s), "backward with rope");
}

}  // extern "C"
