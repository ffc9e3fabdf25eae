// fa_internal.h -- launch interface between the C-ABI layer (fa_api.cpp) and
// the gfx950 kernels.  Arguments reaching these functions are already
// validated; each returns the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {

// Launch geometry the host checks before any launch (the kernels assert that
// they match): query rows per work item of the bf16 prefill, query rows per
// workgroup of the fp32 prefill (by head size), query heads per decode
// workgroup, and HIP's limits on grid sizes.
constexpr int kFwdBf16Rows = 256;
constexpr int fwd_f32_rows(int d) { return d == 128 ? 64 : 128; }
constexpr int kDecodeHeadGroup = 16;
constexpr long long kMaxGridX = 0x7fffffffLL;
constexpr long long kMaxGridYZ = 65535;

// One prefill problem, as validated by fa_fwd / fa_fwd_f32.
struct FwdArgs {
    const void* q;       // [B,H,N_q,d]
    const void* k;       // [B,H_kv,N_k,d]
    const void* v;       // [B,H_kv,N_k,d]
    void* o;             // [B,H,N_q,d]
    float* lse;          // [B,H,N_q] or nullptr
    int B, H, H_kv, N_q, N_k, d;
    float scale;         // softmax scale on q.k
    int causal;
    int window;          // sliding window in keys (causal only), 0 = none
    int max_workgroups = 0;   // cap on the persistent grid, 0 = none (a test hook)
    unsigned long long* clock_stamps = nullptr;   // bf16 prefill clock record (a test hook)
};

// One decode step, as validated by fa_decode.
struct DecodeArgs {
    const void* q;       // [B,H,d]
    const void* k;       // [B,H_kv,N_max,d]
    const void* v;       // [B,H_kv,N_max,d]
    const int* seq_lens; // [B], device
    void* o;             // [B,H,d]
    float* lse;          // [B,H] or nullptr
    float* part_o;       // [B,H,S,d]  workspace
    float* part_lse;     // [B,H,S]    workspace
    unsigned long long* queue;   // chunk queue word, workspace
    int B, H, H_kv, N_max, d, num_splits;
    float scale;
    int window;          // the query sees the last `window` rows, 0 = all
    // paged cache (block_table != nullptr): k and v are page pools
    // [num_pages, H_kv, page_size, d]; N_max = max_blocks * page_size
    const int* block_table = nullptr;   // [B, max_blocks], device
    int max_blocks = 0, page_size = 0, num_pages = 0;
    // FP8 E4M3 cache (kv_fp8 != 0): k and v hold codes; keys are k_scale * code,
    // values v_scale * code
    int kv_fp8 = 0;
    float k_scale = 1.f, v_scale = 1.f;
};

// Size of the decode scratch array the allocation-free decode entry point
// uses for its split partials (one array per GPU, in decode.hip).
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;

// Device address of that array on the current device: looked up once per
// device (hipGetSymbolAddress with the device current) and kept.
hipError_t decode_scratch(void** ptr);

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace fa
