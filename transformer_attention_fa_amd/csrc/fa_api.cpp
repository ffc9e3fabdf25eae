// fa_api.cpp -- the C ABI declared in include/fa.h: argument validation on the
// host, then kernel launches on the caller's stream.  No allocation, no host
// synchronisation, no exceptions across the boundary.
#include "fa.h"
#include "fa_internal.h"
#include "fa_testing.h"

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

namespace {

thread_local char g_last_error[512] = "";

fa_status_t fail(fa_status_t s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

bool aligned(const void* p, std::uintptr_t n) { return (reinterpret_cast<std::uintptr_t>(p) % n) == 0; }

// Element counts are capped at 2^40 (the kernels index with 64-bit offsets).
// Each partial product is checked before it is formed, so no product of
// positive sizes can overflow.
bool too_large(long long a, long long b, long long c, long long d)
{
    const long long lim = 1LL << 40;
    long long prod = a;
    for (long long x : {b, c, d}) {
        if (x > 0 && prod > lim / x) return true;
        prod *= x;
    }
    return prod > lim;
}

fa_status_t check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         int B, int H, int H_kv, int N_q, int N_k, int d, float scale)
{
    if (!q || !k || !v || !o)
        return fail(FA_ERR_INVALID_ARGUMENT, "null q, k, v or o pointer");
    if (B < 1 || H < 1 || H_kv < 1 || N_q < 1 || N_k < 1 || d < 1)
        return fail(FA_ERR_INVALID_ARGUMENT, "sizes must be >= 1 (B=%d H=%d H_kv=%d N_q=%d N_k=%d d=%d)",
                    B, H, H_kv, N_q, N_k, d);
    if (H % H_kv != 0)
        return fail(FA_ERR_INVALID_ARGUMENT, "H=%d is not a multiple of H_kv=%d", H, H_kv);
    if (d != 64 && d != 128)
        return fail(FA_ERR_UNSUPPORTED, "head dimension d=%d not supported (64 or 128)", d);
    if (!std::isfinite(scale))
        return fail(FA_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (scale < 0.0f)
        return fail(FA_ERR_UNSUPPORTED, "negative scale not supported");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
        return fail(FA_ERR_INVALID_ARGUMENT, "q, k, v and o must be 16-byte aligned");
    if (lse && !aligned(lse, 4))
        return fail(FA_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
    if (too_large(B, H, N_q, d) || too_large(B, H_kv, N_k, d))
        return fail(FA_ERR_UNSUPPORTED, "problem too large");
    return FA_OK;
}

// Grid limits of the prefill kernels: one work item (bf16) or workgroup (fp32)
// per block of query rows of each (batch, head); HIP's grid holds at most
// 2^31 - 1 workgroups in x.
fa_status_t check_fwd_grid(int B, int H, int N_q, int rows_per_block, const char* name)
{
    const long long blocks = ((long long)N_q + rows_per_block - 1) / rows_per_block * (long long)H * (long long)B;
    if (blocks > fa::kMaxGridX)
        return fail(FA_ERR_UNSUPPORTED, "%s: %lld query blocks of %d rows (B*H*ceil(N_q/%d)) exceed the %lld "
                    "workgroups of a launch", name, blocks, rows_per_block, rows_per_block, fa::kMaxGridX);
    return FA_OK;
}

fa_status_t from_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) return FA_OK;
    return fail(FA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Workspace layout: the split kernel's chunk queue (one 64-bit word) at the
// front, on 256 bytes of its own, so it sits in the same place whatever the
// shape of the call; then fp32 partial outputs [B,H,S,d] and 256-byte aligned
// fp32 partial log-sum-exps [B,H,S].
constexpr size_t kQueueBytes = 256;

size_t workspace_lse_offset(int B, int H, int d, int num_splits)
{
    const size_t rows = (size_t)B * (size_t)H * (size_t)num_splits;
    return kQueueBytes + (rows * (size_t)d * sizeof(float) + 255) / 256 * 256;
}

size_t workspace_bytes_for(int B, int H, int d, int num_splits)
{
    if (B < 1 || H < 1 || d < 1 || num_splits < 1 || num_splits > 256) return 0;
    if (too_large(B, H, num_splits, d + 1)) return 0;
    const size_t rows = (size_t)B * (size_t)H * (size_t)num_splits;
    return workspace_lse_offset(B, H, d, num_splits) + rows * sizeof(float);
}

fa_status_t decode_common(const void* q, const void* k_cache, const void* v_cache,
                          const int* seq_lens, void* o, float* lse,
                          int B, int H, int H_kv, int N_max, int d, float scale,
                          int num_splits, void* workspace, size_t workspace_bytes, int window,
                          hipStream_t stream, const char* name,
                          const int* block_table = nullptr, int max_blocks = 0, int page_size = 0,
                          int num_pages = 0, int kv_fp8 = 0, float k_scale = 1.f, float v_scale = 1.f,
                          bool use_scratch = false)
{
    fa_status_t s = check_common(q, k_cache, v_cache, o, lse, B, H, H_kv, 1, N_max, d, scale);
    if (s != FA_OK) return s;
    // grid limits: the split kernel takes num_splits * H_kv * ceil(rep / 16)
    // * B chunks (a one-dimensional grid of up to that many workgroups), the
    // merge one workgroup per 4 (b, h) rows
    const long long head_groups = (long long)H_kv * ((H / H_kv + fa::kDecodeHeadGroup - 1) / fa::kDecodeHeadGroup);
    if (B > fa::kMaxGridYZ)
        return fail(FA_ERR_UNSUPPORTED, "%s: B=%d sequences exceed the %lld a launch can take", name, B,
                    fa::kMaxGridYZ);
    if (head_groups > fa::kMaxGridYZ)
        return fail(FA_ERR_UNSUPPORTED, "%s: H_kv * ceil((H/H_kv)/%d) = %lld head groups exceed the %lld a launch "
                    "can take", name, fa::kDecodeHeadGroup, head_groups, fa::kMaxGridYZ);
    if ((long long)B * H > fa::kMaxGridX - 3)
        return fail(FA_ERR_UNSUPPORTED, "%s: B*H = %lld query rows exceed %lld", name, (long long)B * H,
                    fa::kMaxGridX - 3);
    if (num_splits >= 1 && num_splits <= 256 && (long long)num_splits * head_groups * B > fa::kMaxGridX)
        return fail(FA_ERR_UNSUPPORTED, "%s: num_splits * B * head groups = %lld chunks exceed %lld", name,
                    (long long)num_splits * head_groups * B, fa::kMaxGridX);
    if (!seq_lens)
        return fail(FA_ERR_INVALID_ARGUMENT, "null seq_lens");
    if (!aligned(seq_lens, 4))
        return fail(FA_ERR_INVALID_ARGUMENT, "seq_lens must be 4-byte aligned");
    if (num_splits < 1 || num_splits > 256)
        return fail(FA_ERR_INVALID_ARGUMENT, "num_splits=%d outside 1..256", num_splits);
    size_t need = workspace_bytes_for(B, H, d, num_splits);
    if (use_scratch) {
        // the library's scratch array instead of a caller workspace: checked
        // against its size, and its address looked up only once every
        // argument has passed
        if (need == 0 || need > fa::kDecodeScratchBytes)
            return fail(FA_ERR_UNSUPPORTED, "%s: B*H*num_splits*(d+1)*4 = %zu bytes of partials exceed the "
                        "library's %zu-byte scratch array (fa_decode takes a caller workspace)", name, need,
                        fa::kDecodeScratchBytes);
        s = from_hip(fa::decode_scratch(&workspace), "scratch lookup");
        if (s != FA_OK) return s;
        workspace_bytes = fa::kDecodeScratchBytes;
    }
    if (!workspace || !aligned(workspace, 16))
        return fail(FA_ERR_INVALID_ARGUMENT, "workspace must be non-null and 16-byte aligned");
    if (need == 0 || workspace_bytes < need)
        return fail(FA_ERR_INVALID_ARGUMENT, "workspace too small: %zu bytes given, %zu needed",
                    workspace_bytes, need);
    char* ws = static_cast<char*>(workspace);
    fa::DecodeArgs a{q, k_cache, v_cache, seq_lens, o, lse,
                     reinterpret_cast<float*>(ws + kQueueBytes),
                     reinterpret_cast<float*>(ws + workspace_lse_offset(B, H, d, num_splits)),
                     reinterpret_cast<unsigned long long*>(ws),
                     B, H, H_kv, N_max, d, num_splits, scale, window,
                     block_table, max_blocks, page_size, num_pages, kv_fp8, k_scale, v_scale};
    char what[64];
    snprintf(what, sizeof what, "%s launch", name);
    return from_hip(fa::launch_decode(a, stream), what);
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t s)
{
    switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED";
    case FA_ERR_HIP: return "FA_ERR_HIP";
    }
    return "FA_ERR_UNKNOWN";
}

const char* fa_last_error(void) { return g_last_error; }

fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N_q, int N_k, int d,
                   float scale, int causal, hipStream_t stream)
{
    fa_status_t s = check_common(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale);
    if (s == FA_OK) s = check_fwd_grid(B, H, N_q, fa::kFwdBf16Rows, "fa_fwd");
    if (s != FA_OK) return s;
    fa::FwdArgs a{q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale, causal != 0, 0};
    return from_hip(fa::launch_fwd_bf16(a, stream), "fa_fwd launch");
}

fa_status_t fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int H_kv, int N_q, int N_k, int d,
                          float scale, int window, hipStream_t stream)
{
    fa_status_t s = check_common(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale);
    if (s == FA_OK) s = check_fwd_grid(B, H, N_q, fa::kFwdBf16Rows, "fa_fwd_window");
    if (s != FA_OK) return s;
    if (window < 1)
        return fail(FA_ERR_INVALID_ARGUMENT, "window=%d must be at least 1", window);
    fa::FwdArgs a{q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale, 1, window};
    return from_hip(fa::launch_fwd_bf16(a, stream), "fa_fwd_window launch");
}

fa_status_t fa_testing_fwd_capped(const void* q, const void* k, const void* v, void* o, float* lse,
                                  int B, int H, int H_kv, int N_q, int N_k, int d, float scale, int causal,
                                  int window, int max_workgroups, unsigned long long* clock_stamps,
                                  hipStream_t stream)
{
    fa_status_t s = check_common(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale);
    if (s == FA_OK) s = check_fwd_grid(B, H, N_q, fa::kFwdBf16Rows, "fa_testing_fwd_capped");
    if (s != FA_OK) return s;
    if (window < 0 || (window > 0 && !causal))
        return fail(FA_ERR_INVALID_ARGUMENT, "window=%d: 0 (none) or >= 1 with causal", window);
    if (max_workgroups < 0)
        return fail(FA_ERR_INVALID_ARGUMENT, "max_workgroups=%d must be >= 0", max_workgroups);
    fa::FwdArgs a{q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale, causal != 0, window};
    a.max_workgroups = max_workgroups;
    if (clock_stamps && !aligned(clock_stamps, 8))
        return fail(FA_ERR_INVALID_ARGUMENT, "clock_stamps must be 8-byte aligned");
    a.clock_stamps = clock_stamps;
    return from_hip(fa::launch_fwd_bf16(a, stream), "fa_testing_fwd_capped launch");
}

fa_status_t fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                       int B, int H, int H_kv, int N_q, int N_k, int d,
                       float scale, int causal, hipStream_t stream)
{
    fa_status_t s = check_common(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale);
    if (s == FA_OK) s = check_fwd_grid(B, H, N_q, fa::fwd_f32_rows(d), "fa_fwd_f32");
    if (s != FA_OK) return s;
    fa::FwdArgs a{q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, scale, causal != 0, 0};
    return from_hip(fa::launch_fwd_f32(a, stream), "fa_fwd_f32 launch");
}

size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits)
{
    return workspace_bytes_for(B, H, d, num_splits);
}

fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int* seq_lens, void* o, float* lse,
                      int B, int H, int H_kv, int N_max, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      hipStream_t stream)
{
    return decode_common(q, k_cache, v_cache, seq_lens, o, lse, B, H, H_kv, N_max, d, scale, num_splits,
                         workspace, workspace_bytes, 0, stream, "fa_decode");
}

fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seq_lens, void* o, float* lse,
                              int B, int H, int H_kv, int N_max, int d, float scale,
                              int num_splits, hipStream_t stream)
{
    return decode_common(q, k_cache, v_cache, seq_lens, o, lse, B, H, H_kv, N_max, d, scale, num_splits, nullptr,
                         0, 0, stream, "fa_decode_noalloc", nullptr, 0, 0, 0, 0, 1.f, 1.f, true);
}

fa_status_t fa_decode_window(const void* q, const void* k_cache, const void* v_cache,
                             const int* seq_lens, void* o, float* lse,
                             int B, int H, int H_kv, int N_max, int d, float scale,
                             int window, int num_splits, void* workspace, size_t workspace_bytes,
                             hipStream_t stream)
{
    if (window < 1)
        return fail(FA_ERR_INVALID_ARGUMENT, "window=%d must be at least 1", window);
    return decode_common(q, k_cache, v_cache, seq_lens, o, lse, B, H, H_kv, N_max, d, scale, num_splits,
                         workspace, workspace_bytes, window, stream, "fa_decode_window");
}

fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int* block_table, int max_blocks, const int* seq_lens,
                            void* o, float* lse, int B, int H, int H_kv, int num_pages, int page_size,
                            int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                            hipStream_t stream)
{
    if (!block_table)
        return fail(FA_ERR_INVALID_ARGUMENT, "null block_table");
    if (!aligned(block_table, 4))
        return fail(FA_ERR_INVALID_ARGUMENT, "block_table must be 4-byte aligned");
    if (max_blocks < 1 || num_pages < 1)
        return fail(FA_ERR_INVALID_ARGUMENT, "max_blocks=%d and num_pages=%d must be at least 1",
                    max_blocks, num_pages);
    if (page_size < 1)
        return fail(FA_ERR_INVALID_ARGUMENT, "page_size=%d must be at least 1", page_size);
    if (page_size % 16 != 0)
        return fail(FA_ERR_UNSUPPORTED, "page_size=%d: pages must hold a multiple of 16 rows", page_size);
    if ((long long)max_blocks * page_size > 0x7fffffffLL || too_large(num_pages, H_kv, page_size, d))
        return fail(FA_ERR_UNSUPPORTED, "page pool or block table too large");
    return decode_common(q, k_pages, v_pages, seq_lens, o, lse, B, H, H_kv, max_blocks * page_size, d, scale,
                         num_splits, workspace, workspace_bytes, 0, stream, "fa_decode_paged", block_table,
                         max_blocks, page_size, num_pages);
}

fa_status_t fa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                          const int* seq_lens, void* o, float* lse, int B, int H, int H_kv, int N_max, int d,
                          float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          hipStream_t stream)
{
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || k_scale <= 0.f || v_scale <= 0.f)
        return fail(FA_ERR_INVALID_ARGUMENT, "k_scale=%g and v_scale=%g must be finite and positive",
                    (double)k_scale, (double)v_scale);
    return decode_common(q, k_cache, v_cache, seq_lens, o, lse, B, H, H_kv, N_max, d, scale, num_splits,
                         workspace, workspace_bytes, 0, stream, "fa_decode_fp8", nullptr, 0, 0, 0, 1, k_scale,
                         v_scale);
}

}  // extern "C"
