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
// Split pass: workgroup (c, KV head and head group, b) takes keys
// [f + c*L, min(f + (c+1)*L, len)) with L = ceil((len - f) / num_splits), where
// f = 0, or f = max(0, len - W) with a sliding window of W keys ("Attention
// variants" §4: the newest token sees the W most recent rows), and serves up to 16
// query heads that share one KV head, so each K/V byte of the chunk crosses HBM
// once for all of them.  The chunk is cut into 16-key tiles dealt round robin
// to the 4 waves; each wave streams its tiles into its own slice of LDS with
// buffer_load_dwordx4 ... lds (two tiles in flight, no workgroup barrier) and
// computes on the matrix cores:
//   S^T (16 keys x 16 heads) = K Q^T     v_mfma_f32_16x16x32_bf16, K from LDS
//   O^T (d x 16 heads)     += V^T P^T    v_mfma_f32_16x16x16_bf16, V^T from LDS
//                                         through transposing reads
// In the 16x16 accumulator layout lane l holds head l%16 and keys 4*(l/16)..+3
// of the tile, which is exactly the B operand the 16x16x16 P V product needs,
// so P goes from the score registers to the matrix core with one conversion.
// Padding heads (past the group) have zero queries and are discarded.  The
// online softmax of "Attention variants" §3 runs per wave (running max raised
// only when a tile max exceeds it by more than 8, so p <= 256); the 4 waves
// are merged at the end with the same rescale rule and the chunk writes
// o_c = O/l (fp32) and lse_c = m + ln l; an empty chunk writes lse_c = -inf,
// o_c = 0.
//
// Merge pass (not on the pages; the online-softmax rescale applied to whole
// chunk summaries): M = max_c lse_c, lse = M + ln sum_c exp(lse_c - M),
// o = sum_c exp(lse_c - lse) o_c, rounded to bf16.
#include "fa_internal.h"

#include <hip/hip_runtime.h>
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
};

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

// Workgroups are dispatched in index order with blockIdx.z slowest, so z picks
// the sequence by rank of length, longest first: the largest chunks start
// first and the grid drains on the shortest ones.  Ranks order by length
// (descending), then index, so they are a permutation of 0..B-1.  Batches of
// more than 64 sequences keep index order.
__device__ __forceinline__ int sequence_for(const SplitParams& p, int z)
{
    if (p.B > 64) return z;
    const int lane = threadIdx.x & 63;
    auto work = [&](int b) __attribute__((always_inline)) {   // keys the sequence reads
        const int len = clamped_len(p, b);
        return len - key_start(p, len);
    };
    const int mine = lane < p.B ? work(lane) : -1;
    int rank = 0;
    for (int j = 0; j < p.B; ++j) {
        const int lj = work(j);
        rank += (lj > mine) || (lj == mine && j < lane);
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < p.B && rank == z);
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

// four FP8 E4M3 codes -> four bf16 (exact: every E4M3 value is a bf16 value)
__device__ __forceinline__ unsigned long long e4m3x4_to_bf16x4(unsigned w)
{
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    const bf16x4 r = __builtin_convertvector((f32x4{lo[0], lo[1], hi[0], hi[1]}), bf16x4);
    return __builtin_bit_cast(unsigned long long, r);
}

template <int D, bool PAGED, bool KV8>
__global__ __launch_bounds__(256) void decode_split_kernel(SplitParams p)
{
    constexpr int NW = 4;
    constexpr int TK = 16;                   // keys per tile
    constexpr int ROWB = KV8 ? D : D * 2;    // bytes per cache row
    constexpr int QROWB = D * 2;             // bytes per query row (bf16)
    constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
    constexpr int TILEB = TK * ROWB;         // bytes per K (or V) tile
    constexpr int LOADS = TILEB / (64 * 16); // wave load instructions per tensor per tile
    constexpr int KS = D / 32;               // 16x16x32 k-steps over d
    constexpr int DB = D / 16;               // 16-row blocks of d for O^T
    constexpr int VSTAGE = 2 * 2 * TILEB;    // FP8: bf16 copy of the V tile, after the two stages
    constexpr int WAVE_LDS = 2 * 2 * TILEB + (KV8 ? TK * D * 2 : 0);
    static_assert(TILEB % (64 * 16) == 0, "tile shape");

    constexpr int QB = 16 * 256;             // Q rows of the head group (16 x 256 B at most)
    __shared__ __attribute__((aligned(1024))) char lds[NW * WAVE_LDS + QB];

    const int c = blockIdx.x;
    const int g = blockIdx.y / p.ngrp;
    const int hg = blockIdx.y % p.ngrp;
    const int b = sequence_for(p, blockIdx.z);
    const int h0 = g * p.rep + hg * 16;      // first query head of the group
    const int nh = min(16, p.rep - hg * 16); // heads in the group
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int l16 = lane & 15, g4 = lane >> 4;

    const int len = clamped_len(p, b);
    const int kfirst = key_start(p, len);
    int L = (len - kfirst + p.S - 1) / p.S;
    if (PAGED) L = (L + TK - 1) / TK * TK;   // chunks and tiles start on page-aligned rows
    const int j0 = kfirst + c * L;
    const int nkeys = max(0, min(j0 + L, len) - j0);
    const int ntiles = (nkeys + TK - 1) / TK;
    const int nt_w = ntiles > w ? (ntiles - w + NW - 1) / NW : 0;   // tiles w, w+4, ...

    const size_t kv_row0 = PAGED ? 0 : ((size_t)b * p.H_kv + g) * (size_t)p.N_max + (size_t)j0;
    const char* kbase = p.k + kv_row0 * ROWB;
    const char* vbase = p.v + kv_row0 * ROWB;
    char* wl = lds + w * WAVE_LDS;

    int ld_k[LOADS], ld_v[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int pos = i * 64 + lane;
        const int r = pos / CPR, cp = pos % CPR;
        ld_k[i] = r * ROWB + (KV8 ? fswz<D>(r, cp) : kswz<D>(r, cp)) * 16;
        ld_v[i] = r * ROWB + (KV8 ? fswz<D>(r, cp) : dswz<D>(r, cp)) * 16;
    }
    // tile t of the chunk into stage s: rows past the chunk read as 0
    auto issue = [&](int t, int s) __attribute__((always_inline)) {
        const int key0 = t * TK;
        const unsigned bytes = (unsigned)min(TK, nkeys - key0) * ROWB;
        size_t off = (size_t)key0 * ROWB;
        if constexpr (PAGED) {
            // the tile's 16 rows lie in one page (page_size % 16 == 0, aligned chunks)
            const int row = j0 + key0;
            const int blk = row / p.page_size;
            int page = p.block_table[(size_t)b * p.max_blocks + blk];
            page = min(max(page, 0), p.num_pages - 1);           // never outside the pool
            off = (((size_t)page * p.H_kv + g) * p.page_size + (row - blk * p.page_size)) * ROWB;
        }
        const i32x4 rk = make_rsrc(kbase + off, bytes);
        const i32x4 rv = make_rsrc(vbase + off, bytes);
        char* dst = wl + s * 2 * TILEB;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            fa_dec_buffer_load_lds(rk, (LDS_AS void*)(dst + i * 1024), 16, ld_k[i], 0, 0, kStreamPolicy);
            fa_dec_buffer_load_lds(rv, (LDS_AS void*)(dst + TILEB + i * 1024), 16, ld_v[i], 0, 0, kStreamPolicy);
        }
    };

    // per-lane LDS read offsets inside a stage
    int k_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        if constexpr (KV8)     // 8 bytes: d = 32*ks + 8*g4 .. +8 = half (g4 & 1) of chunk 2*ks + g4/2
            k_off[ks] = l16 * ROWB + fswz<D>(l16, 2 * ks + (g4 >> 1)) * 16 + (g4 & 1) * 8;
        else
            k_off[ks] = l16 * ROWB + kswz<D>(l16, 4 * ks + g4) * 16;
    }
    // V^T fragments through transposing reads of a bf16 tile: the V tile of the
    // stage, or (FP8) the wave's bf16 copy of it
    int v_off[DB];
    {
        const int r = 4 * g4 + (l16 >> 2);
#pragma unroll
        for (int dm = 0; dm < DB; ++dm)
            v_off[dm] = (KV8 ? VSTAGE : TILEB) + r * QROWB + dswz<D>(r, 2 * dm + ((l16 & 3) >> 1)) * 16 +
                        (l16 & 1) * 8;
    }
    // FP8: write i of lane l fills bytes 1024*i + 16*l of the wave's bf16 copy
    // of the V tile (a linear write, free of bank conflicts); that position
    // holds bf16 chunk dswz(row, position) of its row, whose 8 FP8 codes the
    // lane reads first (one 8-byte read)
    constexpr int NCV = TK * D * 2 / 1024;   // 16-byte writes per lane per tile
    unsigned cv_src[NCV], cv_dst[NCV];
    if constexpr (KV8) {
#pragma unroll
        for (int i = 0; i < NCV; ++i) {
            const int byte = i * 1024 + lane * 16;
            const int r = byte / QROWB, cc = dswz<D>(r, (byte % QROWB) / 16);
            cv_dst[i] = VSTAGE + byte;
            cv_src[i] = TILEB + r * ROWB + fswz<D>(r, cc >> 1) * 16 + (cc & 1) * 8;
        }
    }

    f32x4 oacc[DB];
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[i] = f32x4{};
    float m_run = kNegInf, nbase = 0.f, l_run = 0.f;

    // ---- Q rows of the group into LDS (one 1 KB slice per wave; rows past the
    // group read as 0; 16-byte chunks placed like a K tile row, whose fragment
    // reads they repeat), then the first two tiles of this wave
    char* qs = lds + NW * WAVE_LDS;
    {
        const int pos = w * 64 + lane;                  // 16-byte chunk position in the Q block
        const int qr = pos / (QROWB / 16), qc = pos % (QROWB / 16);
        const i32x4 rq = make_rsrc(p.q + ((size_t)b * p.H + h0) * D, (unsigned)nh * QROWB);
        fa_dec_buffer_load_lds(rq, (LDS_AS void*)(qs + w * 1024), 16, qr * QROWB + kswz<D>(qr, qc) * 16, 0, 0, 0);
    }
    if (nt_w > 0) issue(w, 0);
    if (nt_w > 1) issue(w + NW, 1);
    if (nt_w > 1) wait_vmcnt<4 * LOADS>();      // the Q slice (older than both tiles) landed
    else if (nt_w > 0) wait_vmcnt<2 * LOADS>();
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

    const unsigned wl_addr = (unsigned)(uintptr_t)(LDS_AS char*)wl;
    auto compute = [&](int t, int s) __attribute__((always_inline)) {
        const unsigned st = wl_addr + s * 2 * TILEB;
        bf16x8 kf[KS];
        if constexpr (KV8) {
            unsigned ka[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ka[ks] = st + k_off[ks];
            u32x2 k8[KS];
            lds_read_b64n<KS>(k8, ka);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const unsigned long long lo = e4m3x4_to_bf16x4(k8[ks][0]), hi = e4m3x4_to_bf16x4(k8[ks][1]);
                kf[ks] = __builtin_bit_cast(bf16x8, (u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi,
                                                           (unsigned)(hi >> 32)}));
            }
            // V tile: FP8 codes -> the wave's bf16 copy, laid out like a bf16 tile
            unsigned va[NCV], wa[NCV];
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                va[i] = st + cv_src[i];
                wa[i] = wl_addr + cv_dst[i];
            }
            u32x2 v8[NCV];
            u32x4 vb[NCV];
            lds_read_b64n<NCV>(v8, va);
#pragma unroll
            for (int i = 0; i < NCV; ++i) {
                const unsigned long long a = e4m3x4_to_bf16x4(v8[i][0]), c2 = e4m3x4_to_bf16x4(v8[i][1]);
                vb[i] = u32x4{(unsigned)a, (unsigned)(a >> 32), (unsigned)c2, (unsigned)(c2 >> 32)};
            }
            lds_write_b128n<NCV>(wa, vb);
        } else {
            if constexpr (KS == 4) lds_read_k4(kf, st + k_off[0], st + k_off[1], st + k_off[2], st + k_off[3]);
            else lds_read_k2(kf, st + k_off[0], st + k_off[1]);
        }
        f32x4 sc = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[ks], qf[ks], sc, 0, 0, 0);
        unsigned vaddr[DB];
#pragma unroll
        for (int dm = 0; dm < DB; ++dm) vaddr[dm] = (KV8 ? wl_addr : st) + v_off[dm];
        i16x4 vf[DB];
        if constexpr (DB == 8) lds_read_vt8(vf, vaddr);
        else lds_read_vt4(vf, vaddr);
        // keys past the chunk end
        const int lim = nkeys - t * TK - 4 * g4;
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = (r < lim) ? sc[r] : kNegInf;
        float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
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
        f32x4 e;
#pragma unroll
        for (int r = 0; r < 4; ++r) e[r] = fast_exp2(__builtin_fmaf(sc[r], p.c, nbase));
        l_run += (e[0] + e[1]) + (e[2] + e[3]);
        const bf16x4 pf = __builtin_convertvector(e, bf16x4);
#pragma unroll
        for (int dm = 0; dm < DB; ++dm)
            oacc[dm] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vf[dm]), pf, oacc[dm], 0, 0, 0);
    };

    // ---- stream this wave's tiles: two in flight, no workgroup barrier
    for (int i = 0; i < nt_w; ++i) {
        if (i + 1 < nt_w) wait_vmcnt<2 * LOADS>();     // tile i landed, tile i+1 may still fly
        else wait_vmcnt<0>();
        compute(w + i * NW, i & 1);
        if (i + 2 < nt_w) issue(w + (i + 2) * NW, i & 1);   // this stage's reads are complete
    }

    // ---- merge the 4 waves through LDS and write the chunk's partial result
    const float l_head = swap16_sum(swap32_sum(l_run));      // sum over the 4 key groups
    __syncthreads();                                          // tile slices are free
    float* sh_m = reinterpret_cast<float*>(lds);             // [NW][16]
    float* sh_l = sh_m + NW * 16;                             // [NW][16]
    float* sh_o = sh_l + NW * 16;                             // [NW][16][D]
    if (g4 == 0) {
        sh_m[w * 16 + l16] = m_run;
        sh_l[w * 16 + l16] = l_head;
    }
    // row (w, head l16): the 4 accumulator values of d-block dm are 16
    // contiguous bytes, chunk 4*dm + g4 of the row; the chunk index is XORed
    // with the head so the 16 heads of one write land in different banks
#pragma unroll
    for (int dm = 0; dm < DB; ++dm)
        *reinterpret_cast<f32x4*>(sh_o + (w * 16 + l16) * D + (((4 * dm + g4) ^ l16) << 2)) = oacc[dm];
    __syncthreads();
    for (int e = tid; e < nh * D; e += 256) {
        const int hh = e / D, d = e % D;
        float mm = kNegInf;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, sh_m[ww * 16 + hh]);
        const float base = (mm == kNegInf) ? 0.f : mm;
        float ll = 0.f, oo = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            const float mw = sh_m[ww * 16 + hh];
            const float a = (mw == kNegInf) ? 0.f : fast_exp2(mw - base);
            ll += a * sh_l[ww * 16 + hh];
            oo += a * sh_o[(ww * 16 + hh) * D + ((((d >> 2) ^ hh)) << 2) + (d & 3)];
        }
        const size_t row = ((size_t)b * p.H + h0 + hh) * p.S + c;
        const float val = ll > 0.f ? oo / ll * p.v_scale : 0.f;
        const float lse_c = ll > 0.f ? (mm + __builtin_log2f(ll)) * kLn2 : kNegInf;
        if (p.o) {
            // S == 1 (row indexes (b, h)): the merge of one chunk has weight
            // exactly 1, so this is the value it would write
            p.o[row * D + d] = __builtin_bit_cast(uint16_t, __builtin_convertvector((f32x2{val, 0.f}), bf16x2)[0]);
            if (d == 0 && p.lse) p.lse[row] = lse_c;
        } else {
            p.part_o[row * D + d] = val;
            if (d == 0) p.part_lse[row] = lse_c;
        }
    }
}

struct CombineParams {
    const float* part_o;
    const float* part_lse;
    uint16_t* o;
    float* lse;
    int rows;     // B*H
    int S;
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
    p.ngrp = (p.rep + 15) / 16;               // groups of up to 16 query heads per KV head
    const float sc = KV8 ? a.scale * a.k_scale : a.scale;   // FP8: keys are k_scale * code
    p.c = sc > 0.f ? sc * kLog2e : 1e-30f;
    p.v_scale = KV8 ? a.v_scale : 1.f;
    p.o = a.num_splits == 1 ? static_cast<uint16_t*>(a.o) : nullptr;
    p.lse = a.lse;
    const long long gy = (long long)a.H_kv * p.ngrp;
    if (gy > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_split_kernel<D, PAGED, KV8>), dim3(a.num_splits, (unsigned)gy, a.B), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.num_splits == 1) return e;
    CombineParams cp{a.part_o, a.part_lse, static_cast<uint16_t*>(a.o), a.lse, a.B * a.H, a.num_splits};
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((cp.rows + 3) / 4), dim3(256), 0, stream, cp);
    return hipGetLastError();
}

}  // namespace

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
