// decode.hip -- one decode step against a KV cache: split-KV partials, then an
// LSE merge.
//
// The operation: each sequence b has one new query per head and attends,
// unmasked, to the first seq_lens[b] rows of its key/value cache ("Attention
// mechanism evolution" (toolsku.com), KV-cache code: the cache grows along the
// sequence axis; "Attention variants: GQA/MQA/FlashAttention" (youngju.dev)
// §7: a decode step is a thin matrix-vector product that must re-read the whole
// cache, so it is bound by memory bandwidth, and §2: a KV head serves
// H/H_kv query heads).
//
// Split pass: chunk (c, KV head and head group, b) holds keys
// [f + c*L, min(f + (c+1)*L, len)) with L = ceil((len - f) / num_splits), where
// f = 0, or f = max(0, len - W) with a sliding window of W keys ("Attention
// variants" §4: the newest token sees the W most recent rows), and serves up to 16
// query heads that share one KV head, so each K/V byte of the chunk crosses HBM
// once for all of them.  A workgroup computes one chunk at a time.  When the
// chunks outnumber the workgroups that fit on the device, the grid is one
// resident set that takes chunks, longest sequence first, from a counter in
// the workspace: the 8 XCDs stream at rates up to ~12 % apart, and chunks
// dealt round robin (as the hardware deals workgroups) leave the fast XCDs
// idle while the slow ones finish.  The next chunk's first loads go out while
// the current one's waves merge.  The chunk is cut into 16-key tiles (32 for
// FP8) dealt round robin to the 4 waves; each wave streams its tiles into its
// own slice of LDS with buffer_load_dwordx4 ... lds (two tiles in flight, no
// workgroup barrier) and computes on the matrix cores:
//   S^T (16 keys x 16 heads) = K Q^T     v_mfma_f32_16x16x32_bf16, K from LDS
//   O^T (d x 16 heads)     += V^T P^T    v_mfma_f32_16x16x16_bf16, V^T from LDS
//                                         through transposing reads
// In the 16x16 accumulator layout lane l holds head l%16 and keys 4*(l/16)..+3
// of the tile, which is exactly the B operand the 16x16x16 P V product needs,
// so P goes from the score registers to the matrix core with one conversion.
// An FP8 E4M3 cache (1 byte a value) streams 32-key tiles, the same bytes per
// tile: K codes are read 8 at a time and converted to bf16 in registers (exact)
// for two 16-key S products; V^T comes from the FP8 tile itself through the
// transposing 8-bit read ds_read_b64_tr_b8 (each lane gets one d column of 8
// keys), converted in registers and multiplied with v_mfma_f32_16x16x32_bf16,
// whose B operand -- 8 keys per lane -- is the lane's scores of both 16-key
// blocks (the V rows are read in that key order).
// Padding heads (past the group) have zero queries and are discarded.  The
// online softmax of "Attention variants" §3 runs per wave (running max raised
// only when a tile max exceeds it by more than 8, so p <= 256); the 4 waves
// are merged at the end (through an LDS area of their own, 4 heads a round)
// with the same rescale rule and the chunk writes
// o_c = O/l (fp32) and lse_c = m + ln l; an empty chunk writes lse_c = -inf,
// o_c = 0.
//
// Merge pass (not on the pages; the online-softmax rescale applied to whole
// chunk summaries): M = max_c lse_c, lse = M + ln sum_c exp(lse_c - M),
// o = sum_c exp(lse_c - lse) o_c, rounded to bf16.
#include "fa_internal.h"

#include <hip/hip_runtime.h>
#include <atomic>
#include <mutex>
#include <cstdint>

typedef int fa_dec_i32x4 __attribute__((ext_vector_type(4)));

// Global -> LDS direct load: each lane's 16 bytes land at lds + 16 * lane.
__device__ void fa_dec_buffer_load_lds(fa_dec_i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size,
                                       int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace fa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.0f;   // log2 units
// cache policy of the K/V stream: non-temporal (each byte is used once; the
// hint lets the memory system stream it rather than keep it cached)
constexpr int kStreamPolicy = 2;

struct SplitParams {
    const uint16_t* q;
    const char* k;          // cache (or page pool) bytes: bf16, or FP8 E4M3 codes
    const char* v;
    const int* seq_lens;
    float* part_o;
    float* part_lse;
    int B, H, H_kv, N_max, S, rep, ngrp;
    int window;   // keys seen: the last `window` rows of the cache, 0 = all
    // paged cache: k and v are page pools [num_pages, H_kv, page_size, D];
    // row r of sequence b is row r % page_size of page block_table[b, r / page_size]
    const int* block_table;
    int max_blocks, page_size, num_pages;
    float c;      // scale * log2(e) (times k_scale for an FP8 cache), > 0
    float v_scale;          // FP8 cache: values are v_scale * e4m3 code; 1 otherwise
    // one chunk per sequence (S == 1): the chunk result is the answer, written
    // straight to o (bf16) and lse, and the merge kernel is not launched
    uint16_t* o;
    float* lse;
    // chunks, in order: index = (rank of the sequence * H_kv * ngrp + head
    // group) * S + chunk, longest sequences first.  Workgroup i takes chunk i;
    // with a queue it then claims chunks grid, grid + 1, ... until none is
    // left; without one grid == items.
    int items, grid;
    unsigned long long* queue;
};

// The chunk queue: one 64-bit word, tag in the high half and the number of
// chunks claimed so far in the low half.  The merge kernel puts it back to
// (kQueueTag, 0) after each launch that used it.  A word with another tag is
// a workspace this library did not leave that way (its first use, or other
// data): the first claim finds that and starts the queue afresh.
constexpr unsigned long long kQueueTag = 0x46416451ull;   // "QdAF"
constexpr unsigned long long kQueueIdle = kQueueTag << 32;

// A claim is an add of 1 to the word, issued early; settle_claim(queue, old)
// takes the word it returned and gives the index (0, 1, ...) of the claimed
// chunk past the grid's first ones.
__device__ __forceinline__ unsigned settle_claim(unsigned long long* queue, unsigned long long old)
{
    while ((old >> 32) != kQueueTag) {
        // not a queue of this library: install (tag, 1), taking index 0.  Adds
        // made to the stale word meanwhile are discarded with it; a workgroup
        // that loses the race finds the tag and claims as usual.
        const unsigned long long seen = old + 1;
        const unsigned long long prev = atomicCAS(queue, seen, kQueueIdle | 1ull);
        if (prev == seen) return 0;
        if ((prev >> 32) == kQueueTag) old = atomicAdd(queue, 1ull);
        else old = prev - 1;       // another stale add: retry against the word as it is
    }
    return (unsigned)old;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ i32x4 make_rsrc(const void* p, unsigned bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

// Position of 16-byte chunk c of row r (0..15) of a 16-key tile.  Conflict
// free for the K fragment reads (16 rows, one chunk) and for the transposing
// V reads (8 rows, two adjacent chunks) on the 64-bank LDS.
template <int D>
__device__ __forceinline__ int dswz(int r, int c)
{
    if constexpr (D == 128) return c ^ (2 * (r & 7) + ((r >> 3) & 1));
    else return c ^ (2 * ((r >> 1) & 3) + ((r >> 3) & 1));
}

// Position of 16-byte chunk c of row r (0..15) of a 16-key bf16 K tile (and
// of the staged Q rows, read the same way).  The K fragment read -- 16 rows,
// one chunk per row for each 16 lanes -- measures 2-way bank conflicts on
// gfx950 with dswz's layout and none with chunk XOR row at d = 128 (the
// transposing V reads show the opposite), so the K and V tiles are laid out
// differently.
template <int D>
__device__ __forceinline__ int kswz(int r, int c)
{
    if constexpr (D == 128) return c ^ (r & 15);
    else return dswz<D>(r, c);
}

// Position of 16-byte chunk c of row r (0..15) of a 16-key FP8 tile (rows of D
// bytes).  Conflict free for the 8-byte K fragment reads (16 rows, the two
// halves of one chunk per row pair of lanes) on the 64-bank LDS.
template <int D>
__device__ __forceinline__ int fswz(int r, int c)
{
    if constexpr (D == 128) return c ^ ((r >> 1) & 7);
    else return c ^ ((r >> 2) & 3);
}

// Position of 16-byte chunk c of row r (0..31) of a 32-key FP8 V tile.  The
// transposing 8-bit reads of a d block take one chunk of 8 rows per 16 lanes
// (rows 4g..4g+3 and 16+4g..16+4g+3 for lane group g); this layout spreads the
// 16 rows of each half wave over all 64 banks.
template <int D>
__device__ __forceinline__ int vswz8(int r, int c)
{
    if constexpr (D == 128) return c ^ (((r >> 1) & 3) | (((r >> 4) & 1) << 2));
    else return c ^ (((r >> 2) & 1) | (((r >> 4) & 1) << 1));
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes
// complete, then s_barrier.  Unlike __syncthreads it does not wait for global
// memory operations in flight (the partial stores, the chunk claim), which no
// other wave of the workgroup reads.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// An int from LDS, waiting for this read alone: a plain load there would make
// the compiler wait for every vector memory operation in flight (it cannot
// tell a global->LDS load, which could write the word, from the chunk claim).
__device__ __forceinline__ int lds_read_int(const int* p)
{
    int v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                 : "=v"(v)
                 : "v"((unsigned)(uintptr_t)(const LDS_AS int*)p)
                 : "memory");
    return v;
}

// LDS traffic of the cross-wave merge, which runs while the next chunk's
// global->LDS loads are in flight: plain accesses would make the compiler wait
// for those loads first.  Reads wait for their own results in the same block.
__device__ __forceinline__ void lds_read_f32_4(float (&a)[4], const unsigned (&p)[4])
{
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
                 : "memory");
}
__device__ __forceinline__ void lds_read_f32x4_4(f32x4 (&a)[4], const unsigned (&p)[4])
{
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
                 : "memory");
}
// a 16-byte LDS write; the barrier that follows waits for it
__device__ __forceinline__ void lds_write_f32x4(unsigned p, f32x4 v)
{
    asm volatile("ds_write_b128 %0, %1" : : "v"(p), "v"(v) : "memory");
}

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ float swap32_max(float x)
{
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float swap16_max(float x)
{
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float swap32_sum(float x)
{
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float swap16_sum(float x)
{
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// LDS reads of one tile.  They are written as asm blocks that wait for their
// own results: the compiler treats any LDS read that follows a global->LDS
// load as possibly reading its destination and would wait for every load in
// flight, which would serialise the two-stage pipeline; the stage discipline
// (explicit vmcnt waits below) is what orders these reads after their tile.
__device__ __forceinline__ void lds_read_k4(bf16x8 (&a)[4], unsigned p0, unsigned p1, unsigned p2, unsigned p3)
{
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                 : "v"(p0), "v"(p1), "v"(p2), "v"(p3)
                 : "memory");
}
__device__ __forceinline__ void lds_read_k2(bf16x8 (&a)[2], unsigned p0, unsigned p1)
{
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1])
                 : "v"(p0), "v"(p1)
                 : "memory");
}
// transposing 4x16-bit reads: result lane i of each 16-lane group holds
// column i of the 4 rows addressed by lanes i/4, i/4+4, i/4+8, i/4+12
__device__ __forceinline__ void lds_read_vt8(i16x4 (&a)[8], const unsigned (&p)[8])
{
    asm volatile("ds_read_b64_tr_b16 %0, %8\n\tds_read_b64_tr_b16 %1, %9\n\t"
                 "ds_read_b64_tr_b16 %2, %10\n\tds_read_b64_tr_b16 %3, %11\n\t"
                 "ds_read_b64_tr_b16 %4, %12\n\tds_read_b64_tr_b16 %5, %13\n\t"
                 "ds_read_b64_tr_b16 %6, %14\n\tds_read_b64_tr_b16 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]),
                   "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]), "=&v"(a[7])
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
                 : "memory");
}
__device__ __forceinline__ void lds_read_vt4(i16x4 (&a)[4], const unsigned (&p)[4])
{
    asm volatile("ds_read_b64_tr_b16 %0, %4\n\tds_read_b64_tr_b16 %1, %5\n\t"
                 "ds_read_b64_tr_b16 %2, %6\n\tds_read_b64_tr_b16 %3, %7\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
                 : "memory");
}

__device__ __forceinline__ int clamped_len(const SplitParams& p, int b)
{
    return min(max(p.seq_lens[b], 0), p.N_max);   // never outside the cache
}

// keys read for a sequence of length len: all of them, or the last `window`
__device__ __forceinline__ int key_start(const SplitParams& p, int len)
{
    return p.window > 0 ? max(0, len - p.window) : 0;
}

// Sequences are ranked by the keys they read (descending, then index), so
// chunk indices run from the longest sequence to the shortest: the largest
// chunks start first and the grid drains on the shortest ones.  Each lane
// ranks sequence `lane` (ranks are a permutation of 0..B-1) from the
// clamped lengths the lanes hold (lane_len); batches of more than 64
// sequences keep index order.
__device__ __forceinline__ int lane_rank(const SplitParams& p, int lane_len)
{
    if (p.B > 64) return 0;
    const int lane = threadIdx.x & 63;
    const int mine = lane < p.B ? lane_len - key_start(p, lane_len) : -1;
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
        const int lj = __builtin_amdgcn_readlane(mine, j);
        rank += (lj > mine) || (lj == mine && j < lane);
    }
    return rank;
}

// the sequence of rank z
__device__ __forceinline__ int sequence_of_rank(const SplitParams& p, int rank, int z)
{
    if (p.B > 64) return z;
    const uint64_t hit = __builtin_amdgcn_ballot_w64((int)(threadIdx.x & 63) < p.B && rank == z);
    return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// N 8-byte LDS reads (FP8 K fragments, FP8 V codes), waiting for their own results
template <int N>
__device__ __forceinline__ void lds_read_b64n(u32x2 (&a)[N], const unsigned (&p)[N])
{
    if constexpr (N == 4)
        asm volatile("ds_read_b64 %0, %4\n\tds_read_b64 %1, %5\n\tds_read_b64 %2, %6\n\tds_read_b64 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                     : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
                     : "memory");
    else
        asm volatile("ds_read_b64 %0, %2\n\tds_read_b64 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(a[0]), "=&v"(a[1])
                     : "v"(p[0]), "v"(p[1])
                     : "memory");
}
// eight 8-byte LDS reads (the FP8 K fragments of a 32-key tile)
__device__ __forceinline__ void lds_read_b64x8(u32x2 (&a)[8], const unsigned (&p)[8])
{
    asm volatile("ds_read_b64 %0, %8\n\tds_read_b64 %1, %9\n\tds_read_b64 %2, %10\n\tds_read_b64 %3, %11\n\t"
                 "ds_read_b64 %4, %12\n\tds_read_b64 %5, %13\n\tds_read_b64 %6, %14\n\tds_read_b64 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]),
                   "=&v"(a[7])
                 : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
                 : "memory");
}
// transposing 8 x 8-bit reads: in each 16-lane group, lane 2k+h reads 8
// bytes (row k, columns 8h..8h+7 of an 8 x 16 byte block) and lane i
// receives column i of the 8 rows (byte k from row k)
template <int N>
__device__ __forceinline__ void lds_read_tr8(u32x2 (&a)[N], const unsigned (&p)[N])
{
    if constexpr (N == 8)
        asm volatile("ds_read_b64_tr_b8 %0, %8\n\tds_read_b64_tr_b8 %1, %9\n\t"
                     "ds_read_b64_tr_b8 %2, %10\n\tds_read_b64_tr_b8 %3, %11\n\t"
                     "ds_read_b64_tr_b8 %4, %12\n\tds_read_b64_tr_b8 %5, %13\n\t"
                     "ds_read_b64_tr_b8 %6, %14\n\tds_read_b64_tr_b8 %7, %15\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(a[4]), "=&v"(a[5]), "=&v"(a[6]),
                       "=&v"(a[7])
                     : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5]), "v"(p[6]), "v"(p[7])
                     : "memory");
    else
        asm volatile("ds_read_b64_tr_b8 %0, %4\n\tds_read_b64_tr_b8 %1, %5\n\t"
                     "ds_read_b64_tr_b8 %2, %6\n\tds_read_b64_tr_b8 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
                     : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3])
                     : "memory");
}
// N 16-byte LDS writes, complete before the block ends
template <int N>
__device__ __forceinline__ void lds_write_b128n(const unsigned (&p)[N], const u32x4 (&a)[N])
{
    if constexpr (N == 4)
        asm volatile("ds_write_b128 %0, %4\n\tds_write_b128 %1, %5\n\tds_write_b128 %2, %6\n\tds_write_b128 %3, %7\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     :
                     : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
                     : "memory");
    else
        asm volatile("ds_write_b128 %0, %2\n\tds_write_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     :
                     : "v"(p[0]), "v"(p[1]), "v"(a[0]), "v"(a[1])
                     : "memory");
}

// four FP8 E4M3 codes -> four bf16 (exact: every E4M3 value is a bf16 value),
// two codes per instruction (scale 1)
__device__ __forceinline__ unsigned long long e4m3x4_to_bf16x4(unsigned w)
{
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, true);
    return (unsigned long long)__builtin_bit_cast(unsigned, lo) | ((unsigned long long)__builtin_bit_cast(unsigned, hi) << 32);
}

template <int D, bool PAGED, bool KV8>
__global__ __launch_bounds__(256) void decode_split_kernel(SplitParams p)
{
    constexpr int NW = 4;
    constexpr int TK = KV8 ? 32 : 16;        // keys per tile
    constexpr int ROWB = KV8 ? D : D * 2;    // bytes per cache row
    constexpr int QROWB = D * 2;             // bytes per query row (bf16)
    constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
    constexpr int TILEB = TK * ROWB;         // bytes per K (or V) tile
    constexpr int LOADS = TILEB / (64 * 16); // wave load instructions per tensor per tile
    constexpr int KS = D / 32;               // 16x16x32 k-steps over d
    constexpr int DB = D / 16;               // 16-row blocks of d for O^T
    constexpr int WAVE_LDS = 2 * 2 * TILEB;  // two stages of a K and a V tile
    static_assert(TILEB % (64 * 16) == 0, "tile shape");
    static_assert(kDecodeHeadGroup == 16, "a workgroup serves up to 16 query heads (the 16x16 MFMA columns)");

    constexpr int QB = 16 * 256;             // Q rows of the head group (16 x 256 B at most)
    constexpr int MH = 4;                    // heads per round of the cross-wave merge
    constexpr int MB = NW * MH * D * 4;      // merge area: fp32 rows of MH heads from each wave
    // the tile stages, the Q block and the merge area are disjoint, so the next
    // chunk's Q block and first tiles can load while this chunk's merge runs
    __shared__ __attribute__((aligned(1024))) char lds[NW * WAVE_LDS + QB + MB];
    __shared__ float sh_m[NW * 16], sh_l[NW * 16];   // each wave's running max and sum per head
    __shared__ int next_item;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;
    // clamped length of sequence `lane`: read once, then taken from the lane
    // that holds it (batches of at most 64 sequences)
    const int lane_len = lane < min(p.B, 64) ? clamped_len(p, lane) : 0;
    const int rank = lane_rank(p, lane_len);
    const int gy = p.H_kv * p.ngrp;          // head groups per sequence

    char* const wl = lds + w * WAVE_LDS;
    char* const qs = lds + NW * WAVE_LDS;
    float* const sh_o = reinterpret_cast<float*>(lds + NW * WAVE_LDS + QB);
    const unsigned wl_addr = (unsigned)(uintptr_t)(LDS_AS char*)wl;

    // per-lane offsets of the tile loads inside a stage
    int ld_k[LOADS], ld_v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int pos = i * 64 + lane;
        const int r = pos / CPR, cp = pos % CPR;
        ld_k[i] = r * ROWB + (KV8 ? fswz<D>(r, cp) : kswz<D>(r, cp)) * 16;
        ld_v[i] = r * ROWB + (KV8 ? vswz8<D>(r, cp) : dswz<D>(r, cp)) * 16;
    }
    // per-lane LDS read offsets inside a stage
    int k_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KV8)     // 8 bytes: d = 32*ks + 8*g4 .. +8 = half (g4 & 1) of chunk 2*ks + g4/2
            k_off[ks] = l16 * ROWB + fswz<D>(l16, 2 * ks + (g4 >> 1)) * 16 + (g4 & 1) * 8;
        else
            k_off[ks] = l16 * ROWB + kswz<D>(l16, 4 * ks + g4) * 16;
    }
    // V^T fragments through transposing reads.  bf16: rows 4*g4 + l16/4 of
    // the tile, two adjacent chunks of d block dm.  FP8 (32-key tiles): lane
    // 16g + 2k + h reads 8 codes of row r_k (r_k = 4g + k for k < 4, 16 + 4g
    // + k - 4 after), d = 16*dm + 8h .. +8; lane 16g + i then holds the codes
    // of d = 16*dm + i for keys r_0..r_7, which are the keys this lane holds
    // in P (4g..4g+3 of the first 16-key block of scores, 4g..4g+3 of the
    // second)
    int v_off[DB];
    if constexpr (KV8) {
        const int kk = (lane & 15) >> 1;
        const int r = kk < 4 ? 4 * g4 + kk : 16 + 4 * g4 + (kk - 4);
#pragma unroll
        for (int dm = 0; dm < DB; ++dm) v_off[dm] = TILEB + r * ROWB + vswz8<D>(r, dm) * 16 + (lane & 1) * 8;
    } else {
        const int r = 4 * g4 + (l16 >> 2);
#pragma unroll
        for (int dm = 0; dm < DB; ++dm)
            v_off[dm] = TILEB + r * QROWB + dswz<D>(r, 2 * dm + ((l16 & 3) >> 1)) * 16 + (l16 & 1) * 8;
    }

    // A chunk: the keys [j0, j0 + nkeys) of sequence b for the nh query heads
    // from h0 that share KV head g; this wave streams its tiles w, w+4, ...
    struct Chunk {
        int g, b, h0, nh, j0, nkeys, nt_w;
        int pages;                  // paged cache: lane l holds the page of this wave's tile l
        const char* kbase;
        const char* vbase;
    };
    // paged cache: the block-table entry of tile t of chunk ch, clamped into the pool
    auto table_page = [&](const Chunk& ch, int t) __attribute__((always_inline)) {
        const int page = p.block_table[(size_t)ch.b * p.max_blocks + (ch.j0 + t * TK) / p.page_size];
        return min(max(page, 0), p.num_pages - 1);           // never outside the pool
    };
    auto describe = [&](int item) __attribute__((always_inline)) {
        Chunk ch;
        const int c = item % p.S;
        const int y = (item / p.S) % gy;
        const int hg = y % p.ngrp;
        ch.g = y / p.ngrp;
        ch.b = sequence_of_rank(p, rank, item / (p.S * gy));
        ch.h0 = ch.g * p.rep + hg * 16;          // first query head of the group
        ch.nh = min(16, p.rep - hg * 16);        // heads in the group
        const int len = p.B <= 64 ? __builtin_amdgcn_readlane(lane_len, ch.b) : clamped_len(p, ch.b);
        const int kfirst = key_start(p, len);
        int L = (len - kfirst + p.S - 1) / p.S;
        if (PAGED) L = (L + TK - 1) / TK * TK;   // chunks and tiles start on page-aligned rows
        ch.j0 = kfirst + c * L;
        ch.nkeys = max(0, min(ch.j0 + L, len) - ch.j0);
        const int ntiles = (ch.nkeys + TK - 1) / TK;
        ch.nt_w = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;
        const size_t kv_row0 = PAGED ? 0 : ((size_t)ch.b * p.H_kv + ch.g) * (size_t)p.N_max + (size_t)ch.j0;
        ch.kbase = p.k + kv_row0 * ROWB;
        ch.vbase = p.v + kv_row0 * ROWB;
        // One block-table read per lane and chunk: the entry of this wave's
        // tile `lane`.  Read per tile instead, the entry would be a vector
        // load whose use waits for every tile load in flight before it.
        ch.pages = 0;
        if (PAGED && lane < ch.nt_w) ch.pages = table_page(ch, w + lane * NW);
        return ch;
    };
    // this wave's tile i of chunk ch into stage s: rows past the chunk read as 0
    auto issue = [&](const Chunk& ch, int i, int s) __attribute__((always_inline)) {
        const int t = w + i * NW;
        const int key0 = t * TK;
        const unsigned bytes = (unsigned)min(TK, ch.nkeys - key0) * ROWB;
        size_t off = (size_t)key0 * ROWB;
        if constexpr (PAGED) {
            // the tile's 16 rows lie in one page (page_size % 16 == 0, aligned chunks)
            const int row = ch.j0 + key0;
            const int page = i < 64 ? __builtin_amdgcn_readlane(ch.pages, i)
                                    : __builtin_amdgcn_readfirstlane(table_page(ch, t));
            off = (((size_t)page * p.H_kv + ch.g) * p.page_size + (row % p.page_size)) * ROWB;
        }
        const i32x4 rk = make_rsrc(ch.kbase + off, bytes);
        const i32x4 rv = make_rsrc(ch.vbase + off, bytes);
        char* dst = wl + s * 2 * TILEB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            fa_dec_buffer_load_lds(rk, (LDS_AS void*)(dst + i * 1024), 16, ld_k[i], 0, 0, kStreamPolicy);
            fa_dec_buffer_load_lds(rv, (LDS_AS void*)(dst + TILEB + i * 1024), 16, ld_v[i], 0, 0, kStreamPolicy);
        }
    };
    // A chunk's loads: this wave's 1 KB slice of the group's Q rows into the
    // Q block (rows past the group read as 0; 16-byte chunks placed like a K
    // tile row, whose fragment reads they repeat), then its first two tiles.
    auto start_loads = [&](const Chunk& ch) __attribute__((always_inline)) {
        const int pos = w * 64 + lane;                  // 16-byte chunk position in the Q block
        const int qr = pos / (QROWB / 16), qc = pos % (QROWB / 16);
        const i32x4 rq = make_rsrc(p.q + ((size_t)ch.b * p.H + ch.h0) * D, (unsigned)ch.nh * QROWB);
        fa_dec_buffer_load_lds(rq, (LDS_AS void*)(qs + w * 1024), 16, qr * QROWB + kswz<D>(qr, qc) * 16, 0, 0, 0);
        if (ch.nt_w > 0) issue(ch, 0, 0);
        if (ch.nt_w > 1) issue(ch, 1, 1);
    };

    int item = blockIdx.x;                   // < p.items: the grid is never larger
    Chunk cur = describe(item);
    start_loads(cur);
    bool prefetched = false;                 // cur's loads were issued during the previous chunk's merge
    for (;;) {
        // this wave's Q slice has landed (then the block, after the barrier).
        // Loads issued in one go land in order: the tiles may still fly.  After
        // a prefetch the previous chunk's partial stores follow them: wait for all.
        if (prefetched) wait_vmcnt<0>();
        else if (cur.nt_w > 1) wait_vmcnt<4 * LOADS>();
        else if (cur.nt_w > 0) wait_vmcnt<2 * LOADS>();
        else wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();               // every wave waited for its own slice
        // Q^T fragments (B of S^T): head l16, d = 32*ks + 8*g4 .. +8 (chunk 4*ks + g4)
        bf16x8 qf[KS];
        {
            const unsigned qa = (unsigned)(uintptr_t)(LDS_AS char*)qs + l16 * QROWB;
            if constexpr (KS == 4)
                lds_read_k4(qf, qa + kswz<D>(l16, g4) * 16, qa + kswz<D>(l16, 4 + g4) * 16, qa + kswz<D>(l16, 8 + g4) * 16,
                            qa + kswz<D>(l16, 12 + g4) * 16);
            else lds_read_k2(qf, qa + kswz<D>(l16, g4) * 16, qa + kswz<D>(l16, 4 + g4) * 16);
        }

        f32x4 oacc[DB];
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] = f32x4{};
        float m_run = kNegInf, nbase = 0.f, l_run = 0.f;

        // online softmax of a lane's scores; returns their weights
        auto online = [&](auto& sc) __attribute__((always_inline)) {
            constexpr int N = sizeof(sc) / sizeof(float);
            float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
            if constexpr (N == 8) mx = fmaxf(mx, fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
            mx = swap16_max(swap32_max(mx));
            const float m_blk = mx * p.c;
            if (__builtin_amdgcn_ballot_w64(m_blk > m_run + kRescaleSlack)) {
                const float m_new = fmaxf(m_run, m_blk);
                const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int dm = 0; dm < DB; ++dm) oacc[dm] *= alpha;
                m_run = m_new;
                nbase = (m_new == kNegInf) ? 0.f : -m_new;
            }
        };
        auto compute = [&](int t, int s) __attribute__((always_inline)) {
            const unsigned st = wl_addr + s * 2 * TILEB;
            if constexpr (KV8) {
                // S^T of the two 16-key blocks of the tile; K codes -> bf16 (exact)
                constexpr int NK = 2 * KS;
                unsigned ka[NK];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) ka[kb * KS + ks] = st + k_off[ks] + kb * 16 * ROWB;
                u32x2 k8[NK];
                if constexpr (NK == 8) lds_read_b64x8(k8, ka);
                else lds_read_b64n<4>(k8, ka);
                unsigned vaddr[DB];
#pragma unroll
                for (int dm = 0; dm < DB; ++dm) vaddr[dm] = st + v_off[dm];
                u32x2 v8[DB];
                lds_read_tr8<DB>(v8, vaddr);
                f32x4 sc2[2] = {f32x4{}, f32x4{}};
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const u32x2 w8 = k8[kb * KS + ks];
                        const unsigned long long lo = e4m3x4_to_bf16x4(w8[0]), hi = e4m3x4_to_bf16x4(w8[1]);
                        const bf16x8 kf = __builtin_bit_cast(bf16x8, (u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi,
                                                                             (unsigned)(hi >> 32)}));
                        sc2[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], sc2[kb], 0, 0, 0);
                    }
                // keys past the chunk end: key 16*kb + 4*g4 + r of the tile
                float sc[8];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    const int lim = cur.nkeys - t * TK - 16 * kb - 4 * g4;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sc[4 * kb + r] = (r < lim) ? sc2[kb][r] : kNegInf;
                }
                online(sc);
                float e[8];
#pragma unroll
                for (int r = 0; r < 8; ++r) e[r] = fast_exp2(__builtin_fmaf(sc[r], p.c, nbase));
                l_run += ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
                const bf16x8 pf = __builtin_convertvector((f32x8{e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]}), bf16x8);
#pragma unroll
                for (int dm = 0; dm < DB; ++dm) {
                    const unsigned long long lo = e4m3x4_to_bf16x4(v8[dm][0]), hi = e4m3x4_to_bf16x4(v8[dm][1]);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, (u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi,
                                                                         (unsigned)(hi >> 32)}));
                    oacc[dm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[dm], 0, 0, 0);
                }
            } else {
                bf16x8 kf[KS];
                if constexpr (KS == 4) lds_read_k4(kf, st + k_off[0], st + k_off[1], st + k_off[2], st + k_off[3]);
                else lds_read_k2(kf, st + k_off[0], st + k_off[1]);
                f32x4 sc = {};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], sc, 0, 0, 0);
                unsigned vaddr[DB];
#pragma unroll
                for (int dm = 0; dm < DB; ++dm) vaddr[dm] = st + v_off[dm];
                i16x4 vf[DB];
                if constexpr (DB == 8) lds_read_vt8(vf, vaddr);
                else lds_read_vt4(vf, vaddr);
                // keys past the chunk end
                const int lim = cur.nkeys - t * TK - 4 * g4;
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[r] = (r < lim) ? sc[r] : kNegInf;
                online(sc);
                f32x4 e;
#pragma unroll
                for (int r = 0; r < 4; ++r) e[r] = fast_exp2(__builtin_fmaf(sc[r], p.c, nbase));
                l_run += (e[0] + e[1]) + (e[2] + e[3]);
                const bf16x4 pf = __builtin_convertvector(e, bf16x4);
#pragma unroll
                for (int dm = 0; dm < DB; ++dm)
                    oacc[dm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vf[dm]), pf, oacc[dm], 0, 0, 0);
            }
        };

        // ---- stream this wave's tiles: two in flight, no workgroup barrier.
        // Wave 0 claims the chunk after this one just behind its last tile's
        // loads: late enough that the chunk it takes is not held back from
        // other workgroups for long, early enough that the atomic's round trip
        // overlaps the last tile.  The wait for the tile before the last
        // allows for it (one more operation in flight).
        const int nt_w = cur.nt_w;
        const bool claiming = p.queue && w == 0;
        unsigned long long claim = 0;
        for (int i = 0; i < nt_w; ++i) {
            if (i + 1 < nt_w) {                           // tile i landed, tile i+1 may still fly
                if (claiming && i + 2 == nt_w && nt_w >= 3) wait_vmcnt<2 * LOADS + 1>();   // and the claim
                else wait_vmcnt<2 * LOADS>();
            } else {
                wait_vmcnt<0>();
            }
            compute(w + i * NW, i & 1);
            if (i + 2 < nt_w) issue(cur, i + 2, i & 1);   // this stage's reads are complete
            if (claiming && i + 3 == nt_w && lane == 0) claim = atomicAdd(p.queue, 1ull);
        }
        if (claiming && nt_w < 3 && lane == 0) claim = atomicAdd(p.queue, 1ull);

        // ---- merge the 4 waves through the merge area and write the chunk's
        // partial result, in rounds of MH heads.  Row (w, head h - MH*r) holds
        // the 4 accumulator values of d-block dm as 16-byte chunk 4*dm + g4,
        // with the d-block XORed with the head so the MH heads of one write
        // cover all banks.
        const float l_head = swap16_sum(swap32_sum(l_run));      // sum over the 4 key groups
        if (g4 == 0) {
            sh_m[w * 16 + l16] = m_run;
            sh_l[w * 16 + l16] = l_head;
        }
        const unsigned o_addr = (unsigned)(uintptr_t)(LDS_AS float*)sh_o;
        auto put_rows = [&](int r) __attribute__((always_inline)) {
            const int hl = l16 - MH * r;
            if (hl >= 0 && hl < MH) {
#pragma unroll
                for (int dm = 0; dm < DB; ++dm)
                    lds_write_f32x4(o_addr + ((w * MH + hl) * D + ((4 * (dm ^ hl) + g4) << 2)) * 4, oacc[dm]);
            }
        };
        put_rows(0);
        if (tid == 0)
            next_item = p.queue ? (int)min((long long)p.grid + settle_claim(p.queue, claim), (long long)p.items)
                                : p.items;
        lds_barrier();               // every wave's tiles are done and its round-0 rows written
        const int nxt = __builtin_amdgcn_readfirstlane(lds_read_int(&next_item));
        // The next chunk's Q block and first tiles load while this merge runs:
        // every wave has read this chunk's Q fragments and finished its tiles.
        Chunk nch;
        if (nxt < p.items) {
            nch = describe(nxt);
            start_loads(nch);
        }
        const int rounds = (cur.nh + MH - 1) / MH;
        for (int r = 0; r < rounds; ++r) {
            if (r > 0) {
                lds_barrier();       // the previous round's rows are read
                put_rows(r);
                lds_barrier();
            }
            // wave 0, thread (head h = MH*r + tid/16, part q = tid%16): the
            // 4-float chunks q and q+16 of the head's row (q alone at d = 64).
            // The head's 4 wave weights are computed once per thread, each
            // chunk is one 16-byte read per wave, and the 16 parts of a head
            // store whole runs of the row.
            constexpr int CH = D / 64;               // chunks per thread
            const int hl = tid >> 4, q = tid & 15, hh = MH * r + hl;
            if (tid < 16 * MH && hh < cur.nh) {
                static_assert(NW == 4, "the merge reads one value per wave, four at a time");
                float mw[NW], lw[NW], mm = kNegInf;
                {
                    const unsigned ma = (unsigned)(uintptr_t)(LDS_AS float*)sh_m + hh * 4;
                    const unsigned la = (unsigned)(uintptr_t)(LDS_AS float*)sh_l + hh * 4;
                    const unsigned pm[NW] = {ma, ma + 64, ma + 128, ma + 192};
                    const unsigned pl[NW] = {la, la + 64, la + 128, la + 192};
                    lds_read_f32_4(mw, pm);
                    lds_read_f32_4(lw, pl);
                }
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, mw[ww]);
                const float base = (mm == kNegInf) ? 0.f : mm;
                float a[NW], ll = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    a[ww] = (mw[ww] == kNegInf) ? 0.f : fast_exp2(mw[ww] - base);
                    ll += a[ww] * lw[ww];
                }
                const float scale_out = ll > 0.f ? p.v_scale / ll : 0.f;
                const size_t row = ((size_t)cur.b * p.H + cur.h0 + hh) * p.S + (size_t)(item % p.S);
#pragma unroll
                for (int k = 0; k < CH; ++k) {
                    const int c4 = q + 16 * k;       // chunk of the row: d = 4*c4 .. 4*c4+3
                    f32x4 ow[NW];
                    {
                        const unsigned oa = o_addr + ((hl * D) + ((c4 ^ (hl << 2)) << 2)) * 4;
                        const unsigned po[NW] = {oa, oa + MH * D * 4, oa + 2 * MH * D * 4, oa + 3 * MH * D * 4};
                        lds_read_f32x4_4(ow, po);
                    }
                    f32x4 oo = {};
#pragma unroll
                    for (int ww = 0; ww < NW; ++ww) oo += a[ww] * ow[ww];
                    const f32x4 val = oo * scale_out;
                    if (p.o) {
                        // S == 1 (row indexes (b, h)): the merge of one chunk has weight
                        // exactly 1, so this is the value it would write
                        *reinterpret_cast<bf16x4*>(p.o + row * D + 4 * c4) = __builtin_convertvector(val, bf16x4);
                    } else {
                        *reinterpret_cast<f32x4*>(p.part_o + row * D + 4 * c4) = val;
                    }
                }
                if (q == 0) {
                    const float lse_c = ll > 0.f ? (mm + __builtin_log2f(ll)) * kLn2 : kNegInf;
                    if (p.o) {
                        if (p.lse) p.lse[row] = lse_c;
                    } else {
                        p.part_lse[row] = lse_c;
                    }
                }
            }
        }
        if (nxt >= p.items) break;
        item = nxt;
        cur = nch;
        prefetched = true;
    }
}

struct CombineParams {
    const float* part_o;
    const float* part_lse;
    uint16_t* o;
    float* lse;
    int rows;     // B*H
    int S;
    unsigned long long* queue;   // the split launch's chunk queue, or null
};

// One wave per (b, h) row: merge the S chunk summaries by their log-sum-exp.
// Lane l owns output elements PER*l .. PER*l+PER-1 and holds the log-sum-exps
// (then the weights) of chunks l, l+64, l+128, l+192; the chunk partials are
// read in batches of 8 independent loads, the first batch in flight while the
// log-sum-exps are reduced, so a row costs a few memory round trips rather than
// one per chunk.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineParams p)
{
    constexpr int PER = D / 64;          // output elements per lane
    constexpr int BATCH = 8;
    constexpr int KMAX = 4;              // S <= 256 = 4 x 64
    typedef float vecP __attribute__((ext_vector_type(PER)));
    const int row = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    // the split kernel has finished: leave its queue ready for the next launch
    if (p.queue && blockIdx.x == 0 && threadIdx.x == 0) atomicExch(p.queue, kQueueIdle);
    if (row >= p.rows) return;
    const int S = p.S;                   // 1..256; chunk indices past S are clamped and weigh 0
    const float* lse_c = p.part_lse + (size_t)row * S;
    const vecP* oc = reinterpret_cast<const vecP*>(p.part_o + (size_t)row * S * D) + lane;   // chunk c at oc[c * 64]

    vecP first[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) first[u] = oc[(size_t)min(u, S - 1) * 64];

    float lv[KMAX];
    float mx = kNegInf;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int c = 64 * k + lane;
        lv[k] = (64 * k < S) ? lse_c[min(c, S - 1)] : kNegInf;
        lv[k] = c < S ? lv[k] : kNegInf;
        mx = fmaxf(mx, lv[k]);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
    float sum = 0.f;
    if (mx != kNegInf) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) sum += lv[k] == kNegInf ? 0.f : exp2f((lv[k] - mx) * kLog2e);
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) sum += __shfl_xor(sum, x);
    const float lse = (mx == kNegInf || sum <= 0.f) ? kNegInf : mx + logf(sum);

    vecP acc = {};
    if (lse != kNegInf) {
        // chunk weights exp(lse_c - lse); an empty chunk (lse_c = -inf) weighs 0
        float wt[KMAX];
#pragma unroll
        for (int k = 0; k < KMAX; ++k) wt[k] = lv[k] == kNegInf ? 0.f : exp2f((lv[k] - lse) * kLog2e);
        auto weight = [&](int c) __attribute__((always_inline)) {   // c uniform, < S
            float r = 0.f;
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if ((c >> 6) == k) r = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wt[k]), c & 63));
            return r;
        };
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
            if (u < S) acc += weight(u) * first[u];
        for (int c0 = BATCH; c0 < S; c0 += BATCH) {
            vecP v[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) v[u] = oc[(size_t)min(c0 + u, S - 1) * 64];
#pragma unroll
            for (int u = 0; u < BATCH; ++u)
                if (c0 + u < S) acc += weight(c0 + u) * v[u];
        }
    }
    uint16_t* dst = p.o + (size_t)row * D + lane * PER;
    if constexpr (PER == 2) {
        const bf16x2 t = __builtin_convertvector((f32x2{acc[0], acc[1]}), bf16x2);
        *reinterpret_cast<bf16x2*>(dst) = t;
    } else {
        const bf16x2 t = __builtin_convertvector((f32x2{acc[0], 0.f}), bf16x2);
        dst[0] = __builtin_bit_cast(uint16_t, t[0]);
    }
    if (p.lse && lane == 0) p.lse[row] = lse;
}

// Workgroups of a kernel that fit on the current device at once.  Cached per
// device and kernel (host threads may race to fill an entry; they store the
// same value); 0 if the runtime cannot say.
template <auto Kernel>
int resident_blocks(int threads)
{
    static std::atomic<int> cache[64];    // one per instantiation, i.e. per kernel
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    const int known = cache[dev].load(std::memory_order_relaxed);
    if (known > 0) return known;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, Kernel, threads, 0) != hipSuccess) return 0;
    const int n = cus * (per_cu > 0 ? per_cu : 1);
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

template <int D, bool PAGED, bool KV8>
hipError_t launch_all(const DecodeArgs& a, hipStream_t stream)
{
    SplitParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const char*>(a.k);
    p.v = static_cast<const char*>(a.v);
    p.seq_lens = a.seq_lens;
    p.part_o = a.part_o;
    p.part_lse = a.part_lse;
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.N_max = a.N_max;
    p.S = a.num_splits;
    p.window = a.window;
    p.block_table = a.block_table;
    p.max_blocks = a.max_blocks;
    p.page_size = a.page_size;
    p.num_pages = a.num_pages;
    p.rep = a.H / a.H_kv;
    p.ngrp = (p.rep + kDecodeHeadGroup - 1) / kDecodeHeadGroup;   // groups of up to 16 query heads per KV head
    const float sc = KV8 ? a.scale * a.k_scale : a.scale;   // FP8: keys are k_scale * code
    p.c = sc > 0.f ? sc * kLog2e : 1e-30f;
    p.v_scale = KV8 ? a.v_scale : 1.f;
    p.o = a.num_splits == 1 ? static_cast<uint16_t*>(a.o) : nullptr;
    p.lse = a.lse;
    // chunks (at most 2^31 - 1: checked on the host)
    p.items = (int)((long long)a.num_splits * a.H_kv * p.ngrp * a.B);
    // With several chunks per sequence and more chunks than fit on the device
    // at once, the grid is one resident set of workgroups that take chunks from
    // a queue in the workspace: the XCDs stream at different rates, and the
    // fixed round-robin spread of a one-chunk-a-workgroup grid leaves the fast
    // ones idle at the end.  Otherwise every chunk is a workgroup of its own.
    const int resident = resident_blocks<decode_split_kernel<D, PAGED, KV8>>(256);
    if (a.num_splits > 1 && a.queue && resident > 0 && p.items > resident) {
        p.grid = resident;
        p.queue = a.queue;
    } else {
        p.grid = p.items;
        p.queue = nullptr;
    }
    hipLaunchKernelGGL((decode_split_kernel<D, PAGED, KV8>), dim3(p.grid), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1) return e;
    CombineParams cp{a.part_o, a.part_lse, static_cast<uint16_t*>(a.o), a.lse, a.B * a.H, a.num_splits, p.queue};
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((cp.rows + 3) / 4), dim3(256), 0, stream, cp);
    return hipGetLastError();
}

}  // namespace

// Split partials of fa_decode_noalloc: a file-scope device array, so that
// entry point needs no caller workspace and allocates nothing.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code the
// name `scratch` is a host-side stand-in, not a device address: host code uses
// only the per-device address decode_scratch() looks up.
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));   // with device `dev` current
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    const bool paged = a.block_table != nullptr;
    if (a.kv_fp8) {
        if (paged) return hipErrorInvalidValue;        // not offered
        if (a.d == 128) return launch_all<128, false, true>(a, stream);
        if (a.d == 64) return launch_all<64, false, true>(a, stream);
        return hipErrorInvalidValue;
    }
    if (a.d == 128) return paged ? launch_all<128, true, false>(a, stream) : launch_all<128, false, false>(a, stream);
    if (a.d == 64) return paged ? launch_all<64, true, false>(a, stream) : launch_all<64, false, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
