// fwd_bf16.hip -- tiled exact attention forward on gfx950 bf16 MFMA.
//
// Method ("Attention variants: GQA/MQA/FlashAttention" (youngju.dev) §3):
// cut Q into blocks (one per work item) and K/V into blocks streamed through
// LDS; per query row keep a running maximum m and running sum l; for each key
// block compute the block scores, bring the accumulator and l to a new m when
// needed, add the block's exp(S - m) V; divide by l at the end.  Causal
// problems never load key blocks wholly in the future and mask inside the
// diagonal blocks (§5.5 of the same page).  Query head h reads KV head
// h / (H / H_kv) (§2 of the same page; "Attention mechanism evolution"
// (toolsku.com) GQA code).
//
// gfx950 mapping (not from the pages, whose kernel targets other GPUs):
//  * work item = (query block of BM = 256 rows, head, batch); workgroup = 8
//    waves, each wave owns 32 rows of the block; two waves share each SIMD.
//    Causal launches whose GQA ratio is even pair heads instead: an item is
//    128 rows of two heads that share a KV head, waves 0-3 on one and 4-7 on
//    the other, so the causal diagonal spans two K/V tiles instead of four;
//    At d = 128 the grid is persistent: one workgroup per resident slot
//    (256 CUs x 1 on MI355X), each working through a list of items; d = 64
//    fits two workgroups per CU and runs one item per workgroup;
//  * scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    (A = K fragment from LDS, B = Q fragment held in VGPRs for the whole
//    item).  In the 32x32 accumulator layout lane l holds column l%32 -- one
//    query row -- and 16 of the 32 keys, so row max and row sum are in-lane
//    plus one exchange with lane l^32 (v_permlane32_swap);
//  * the output is accumulated transposed too, O^T += V^T P^T, so it shares
//    the one-row-per-lane layout; P (fp32 -> bf16, round to nearest even) is the
//    B operand straight from the score registers, and the V^T A operand is read
//    from the row-major V tile with the transposing LDS read ds_read_b64_tr_b16
//    (two per MFMA: keys 4h..4h+3 and 8+4h..8+4h+3 of a 16-key step, which is
//    the key order of the score accumulator);
//  * K and V tiles (64 keys) go from global memory straight into LDS with
//    buffer_load_dwordx4 ... lds (no VGPR staging); rows past N_k read as 0
//    through the buffer descriptor's range check and are masked.  16-byte
//    chunks of a row are XOR-swizzled so that both the K fragment reads and the
//    transposing V reads are bank-conflict free on the 64-bank LDS;
//  * the key loop runs in periods, one barrier each: in period j every wave
//    reads K tile j and V tile j-1 while K tile j+1 and V tile j load into the
//    other slots.  A wave's period has a matrix-core phase (O^T += V^T P^T of
//    tile j-1, S^T of tile j) and a softmax phase (tile j's P).  Waves 0-3 run
//    MFMA then softmax, waves 4-7 softmax then MFMA, so on each SIMD one wave's
//    exponentials overlap the other wave's matrix-core work.  Waves 0-3 also
//    load the two tiles, one load after every other MFMA of their matrix-core
//    phase (issued by all waves at the barrier, the loads queue up and stall
//    every wave);
//  * the matrix-core phase is a two-deep pipeline of steps of four MFMAs: the
//    next step's LDS fragments are read before this step's MFMAs issue;
//  * softmax in base 2 (scores scaled by scale*log2(e), v_exp_f32); the
//    running max is only raised -- and O and l rescaled -- when a row's block
//    maximum exceeds it by more than 8 (so every exp2 argument stays <= 8 and
//    p <= 256); the result is the same quantity, O = sum p v / sum p, with the
//    common factor chosen differently; lse = ln2 * (m + log2 l);
//  * item order: workgroups sit on the 8 XCDs round robin; each XCD works
//    through a contiguous range of heads (shared K/V stays in that XCD's L2),
//    longest causal query blocks first within a group of `group` heads, and
//    its workgroups take the list in rounds that alternate direction (a long
//    causal block in one round pairs with a short one in the next);
//  * item switch without a cold start: while an item runs, the next item's Q
//    block streams into its own LDS area (spread over the item's periods,
//    one slice per period when the item is long enough, all of it before the
//    last period) and its first K tile into the K slot the last period
//    leaves free.  The item's last period (PV of its last tile) and the next
//    item's first (S of its first tile) are one switch period: each wave
//    takes its next Q fragments from that area, stages its finished 32 x d
//    output tile in the same rows and stores it as whole rows, then starts
//    the next item;
//  * with single-head items, waves 0-3 take the block's later rows: on the
//    causal diagonal those run longest, and the early-row waves finish before
//    the switch period (with paired items both wave groups take the same rows).
#include "fa_internal.h"

#include <hip/hip_runtime.h>
#include <atomic>
#include <cstddef>
#include <cstdint>
#include <type_traits>

typedef int fa_i32x4 __attribute__((ext_vector_type(4)));

// Global -> LDS direct load: each lane's 16 bytes land at lds + 16 * lane.
__device__ void fa_raw_buffer_load_lds(fa_i32x4 rsrc, __attribute__((address_space(3))) void* lds, int size,
                                       int voffset, int soffset, int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))


constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kRescaleSlack = 8.0f;   // log2 units
constexpr int kStreamOnce = 2;          // buffer load cache policy: non-temporal

// n / d for 0 <= n < 2^31 as a multiply (high half) and a shift, for
// launch-constant divisors (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994, the round-up method with N = 31):
// m = ceil(2^(31+l) / d), l = ceil(log2 d), q = (n * m) >> (31 + l).  m = 0
// marks d = 1.
struct DivConst {
    unsigned m;
    unsigned s;   // l - 1
};

__host__ DivConst div_const(unsigned d)
{
    if (d <= 1) return {0u, 0u};
    unsigned l = 0;
    while ((1ull << l) < d) ++l;
    const unsigned long long m = ((1ull << (31 + l)) + d - 1) / d;
    return {(unsigned)m, l - 1};
}

__device__ __forceinline__ int div_by(int n, DivConst c)
{
    return c.m == 0 ? n : (int)(__umulhi((unsigned)n, c.m) >> c.s);
}

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, H, H_kv, N_q, N_k;
    int rep;      // H / H_kv
    int nqb;      // query blocks per head
    int window;   // sliding window in keys (causal only); 0 = none
    int group;    // heads per longest-first group of the item order
    int items;    // work items (query blocks x heads x batch)
    int grid;     // workgroups of the persistent grid
    int xcd;      // 1: the item list and the grid split per XCD (both multiples of 8)
    float c;      // scale * log2(e), > 0
    // optional clock record (test hook; nullptr otherwise): workgroups 0-7,
    // one per XCD, write {shader cycles, 100 MHz ticks, XCC id} at their start
    // and {shader cycles, ticks} at their end to stamps[8 * g .. 8 * g + 4]
    unsigned long long* stamps;
    // the item decomposition's constants: the head list splits 8 ways
    // (split8), nheads heads a list, groups of gsz heads (the last one glast,
    // at index last_grp), and the divisors gsz * nqb, gsz, glast, H, rep
    int split8, nheads, gsz, glast, last_grp;
    DivConst div_gn, div_gsz, div_glast, div_h, div_rep;
    int hpb;      // heads per batch in the item list: H, or H / 2 when items pair heads
};

// Race-hunting build (-DFA_DEBUG_BARRIERS): one more barrier in the middle
// of every period, between the two phases of each wave, after every memory
// operation of the wave has completed.  Every wave passes it once per period,
// whatever its role, so the barrier counts stay equal; the arithmetic is
// unchanged, so the output must be bit-identical to the normal build's.
__device__ __forceinline__ void debug_barrier()
{
#ifdef FA_DEBUG_BARRIERS
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#endif
}

// Clock record of workgroup g < 8: s_memtime counts shader cycles and
// s_memrealtime the constant 100 MHz clock, so the two spans give the clock
// the kernel ran at.  One lane stores; nothing is kept in registers between
// the two records.
__device__ __forceinline__ void clock_stamp(unsigned long long* stamps, bool at_end)
{
    if (!stamps || blockIdx.x >= 8) return;
    const unsigned long long t = __builtin_amdgcn_s_memtime();
    const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
    if (threadIdx.x != 0) return;
    unsigned long long* rec = stamps + 8 * blockIdx.x;
    if (at_end) {
        rec[3] = t;
        rec[4] = rt;
    } else {
        rec[0] = t;
        rec[1] = rt;
        rec[2] = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 0xf;    // HW_REG_XCC_ID, bits 3:0
    }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt with vmcnt = n and the other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// f(integral_constant<int, I>) for I = FIRST .. LAST-1, unrolled at compile time
template <int FIRST, int LAST, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (FIRST < LAST) {
        f(std::integral_constant<int, FIRST>{});
        static_for<FIRST + 1, LAST>(f);
    }
}

// Buffer descriptor over `bytes` bytes at p (reads past the range return 0).
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

// Position of 16-byte chunk c of tile row r inside the row (XOR swizzle).
template <int D>
__device__ __forceinline__ int swz(int r, int c)
{
    if constexpr (D == 128) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else return c ^ ((r >> 1) & 7);
}

// Order of workgroups: id -> (query block, head, batch); with paired items the
// "head" is a pair of heads, hpb of them per batch.  Workgroups are
// dispatched to the 8 XCDs round robin (id % 8).  When the head count divides
// by 8, XCD x owns the contiguous heads [x*HB/8, (x+1)*HB/8) -- heads that
// share a KV head land on the same XCD and its L2 -- and walks them in groups
// of `group` heads, longest causal query blocks first inside a group.
__device__ __forceinline__ void decompose(int id, const Params& p, bool causal, int& qb, int& h, int& b)
{
    int head0 = 0, slot = id;
    if (p.split8) {
        head0 = (id & 7) * p.nheads;
        slot = id >> 3;
    }
    const int grp = div_by(slot, p.div_gn);
    const int rem = slot - grp * p.gsz * p.nqb;
    const int g0 = grp * p.gsz;
    const bool last = grp == p.last_grp;          // the last group may be smaller
    const int gcount = last ? p.glast : p.gsz;
    const int j = div_by(rem, last ? p.div_glast : p.div_gsz);
    const int bh = head0 + g0 + rem - j * gcount;
    qb = causal ? p.nqb - 1 - j : j;
    b = div_by(bh, p.div_h);
    h = bh - b * p.hpb;
}

// PAIR: an item is BM/2 query rows of two heads that share a KV head (head
// 2i for waves 0-3, head 2i+1 for waves 4-7, the same rows), so both halves
// read the same K/V tiles and a causal item's diagonal spans two tiles, not four
template <int D, int NW, bool CAUSAL, bool PERSIST, bool STAMPS, bool PAIR = false>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(Params p)
{
    static_assert(NW == 8, "the two wave groups pair up on the four SIMDs");
    static_assert(!PAIR || (CAUSAL && PERSIST), "paired items are a causal, persistent form");
    constexpr int BM = NW * 32;              // query rows per work item (all heads)
    constexpr int BMI = PAIR ? BM / 2 : BM;  // query rows of one head per item
    constexpr int NTHR = NW * 64;
    constexpr int BN = 64;                   // keys per LDS tile
    constexpr int KSTEPS = D / 16;           // MFMA k-steps over d for S^T
    constexpr int DBLK = D / 32;             // 32-row blocks of d for O^T
    constexpr int NT = BN / 32;              // 32-key sub-tiles per tile
    constexpr int ROWB = D * 2;              // bytes per K/V row
    constexpr int CPR = D / 8;               // 16-byte chunks per row
    constexpr int TILE = BN * ROWB;          // bytes per K (or V) tile
    constexpr int LOADS = TILE / (NTHR * 16);
    constexpr int QTILE = BM * ROWB;         // bytes of a Q block (the Q area)
    constexpr int QPARTS = QTILE / (NTHR * 16);
    static_assert(TILE % (NTHR * 16) == 0 && QTILE % (NTHR * 16) == 0, "tiles must be whole workgroup loads");
    static_assert(D % 32 == 0, "tile shape");

    // [K slot 0, K slot 1, V slot 0, V slot 1, Q area]
    __shared__ __attribute__((aligned(1024))) char lds[4 * TILE + QTILE];
    char* const qarea = lds + 4 * TILE;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;
    const int role = w >> 2;                 // waves w and w+4 share a SIMD
    // Row groups of single-head items: waves 0-3 take rows 128-255 of the
    // block, waves 4-7 rows 0-127.  On the causal diagonal the later rows run
    // longest, and a matrix-core-first wave ends its last tile with a PV phase
    // alone (its softmax of that tile ran in the period before), so the item's
    // last period is short.  wr is also the wave's 32-row slot in the Q area,
    // which paired items fill with the second head's rows first.
    const int wr = w ^ 4;
    const int off = p.N_k - p.N_q;           // causal diagonal offset

    // ---- tile loads: chunk position -> (row, global chunk).  A workgroup-wide
    //      load covers NTHR*16/ROWB rows; the swizzle repeats every 16 rows, so
    //      load i of a tile (or part i of the Q block) is load 0 moved by
    //      i*NTHR*16 bytes on both sides.
    int ld_voff;
    {
        const int r = tid / CPR, cp = tid % CPR;
        ld_voff = r * ROWB + swz<D>(r, cp) * 16;
    }
    auto issue = [&](const char* base, int kb, char* dst) __attribute__((always_inline)) {
        const int key0 = kb * BN;
        const unsigned bytes = (unsigned)max(0, min(BN, p.N_k - key0)) * ROWB;
        const i32x4 rs = make_rsrc(base + (size_t)key0 * ROWB, bytes);
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            fa_raw_buffer_load_lds(rs, (LDS_AS void*)(dst + (i * NTHR + w * 64) * 16), 16, ld_voff + i * NTHR * 16, 0,
                                   0, 0);
    };
    // the same tile loaded by waves 0-3 alone: 2*LOADS loads each, load i at
    // chunk i*NTHR/2 + (w&3)*64 + lane (NTHR/2 chunks are a whole number of
    // 16-row swizzle periods, so load i is load 0 moved on both sides)
    constexpr int LOADS0 = 2 * LOADS;
    int ld_voff0;
    {
        const int t = (w & 3) * 64 + lane, r = t / CPR, cp = t % CPR;
        ld_voff0 = r * ROWB + swz<D>(r, cp) * 16;
    }
    auto tile_rsrc = [&](const char* base, int kb) __attribute__((always_inline)) {
        const int key0 = kb * BN;
        return make_rsrc(base + (size_t)key0 * ROWB, (unsigned)max(0, min(BN, p.N_k - key0)) * ROWB);
    };
    auto issue0 = [&](const i32x4& rs, char* dst, int i) __attribute__((always_inline)) {
        fa_raw_buffer_load_lds(rs, (LDS_AS void*)(dst + (i * (NTHR / 2) + (w & 3) * 64) * 16), 16,
                               ld_voff0 + i * (NTHR / 2) * 16, 0, 0, 0);
    };

    // ---- work items.  Item (query block, head, batch) covers query rows
    //      q0 .. q0+BMI-1 (of two heads with paired items); the per-wave
    //      quantities below are set per item.
    struct Item {
        unsigned bh;     // b * H + h: Q, O and the LSE rows start at bh * N_q (waves 0-3's head)
        unsigned bh2;    // waves 4-7's head: bh + 1 with paired items, else bh
        unsigned bg;     // b * H_kv + h / rep: K and V rows start at bg * N_k
        int q0;          // first query row of the block
        int nkb;         // key tiles the block reads: kb_lo .. nkb-1
        int kb_lo;
    };
    auto item_at = [&](int id) __attribute__((always_inline)) {
        int qb, hh, b;
        decompose(id, p, CAUSAL, qb, hh, b);
        const int h = PAIR ? 2 * hh : hh;
        Item it;
        it.bh = (unsigned)(b * p.H + h);
        it.bh2 = it.bh + (PAIR ? 1u : 0u);
        it.bg = (unsigned)(b * p.H_kv + div_by(h, p.div_rep));
        it.q0 = qb * BMI;
        int kend = p.N_k;
        if (CAUSAL) kend = min(p.N_k, it.q0 + BMI + off);
        it.nkb = kend > 0 ? (kend + BN - 1) / BN : 0;
        it.kb_lo = 0;
        // with a sliding window ("Attention variants" §4: each row sees the W
        // keys ending at its last causally visible key) the block's first row
        // sees nothing before its window
        if (CAUSAL && p.window > 0) it.kb_lo = min(it.nkb, max(0, it.q0 + off - p.window + 1) / BN);
        // at least two tiles (one for an item alone in its workgroup): the
        // padding lies past N_k or past every row's causal limit, is loaded
        // as zeros or as keys no row sees, and is masked
        it.nkb = max(it.nkb, it.kb_lo + (PERSIST ? 2 : 1));
        return it;
    };
    // Q block of an item into the Q area (16-byte chunks swizzled like a K
    // tile); rows past N_q read as 0.  Q is read once, so the load is
    // non-temporal and leaves L2 to the K/V tiles other items re-read.
    // Paired items: the Q area's first half holds waves 4-7's head, the second
    // half waves 0-3's, each the item's BM/2 rows.
    auto issue_q = [&](const Item& it, int part) __attribute__((always_inline)) {
        const bool hi = part >= QPARTS / 2;
        const unsigned hq = PAIR && !hi ? it.bh2 : it.bh;
        const int prow = PAIR && hi ? part - QPARTS / 2 : part;    // the part within the head's rows
        const unsigned bytes = (unsigned)max(0, min(BMI, p.N_q - it.q0)) * ROWB;
        const i32x4 rs = make_rsrc(p.q + ((size_t)hq * (size_t)p.N_q + (size_t)it.q0) * D, bytes);
        fa_raw_buffer_load_lds(rs, (LDS_AS void*)(qarea + (part * NTHR + w * 64) * 16), 16,
                               ld_voff + prow * NTHR * 16, 0, 0, kStreamOnce);
    };

    Item cur, nxt;
    bool has_next;
    i32x4 rq_nxt;            // the next item's Q block (descriptor), for the steady periods' Q slices;
                             // with paired items its first half, waves 4-7's head
    i32x4 rq_nxt2;           // paired items: its second half, waves 0-3's head
    int q_lim;               // steady periods j < q_lim load Q slice j - kb_lo of the next item
    int sb;                  // slot parity: tile t of the current item lives in slot (t + sb) % 2
    int j_knext;             // period that loads the next item's first K tile
    int qpp;                 // parts of the next item's Q block loaded per period
    int q_first;             // first period of the item that may load the next item's Q block
    const char* kbase;
    const char* vbase;
    int qw0, qi, last_vis, first_vis, nkb_w, a_w;
    bool windowed;
    auto set_wave = [&]() __attribute__((always_inline)) {
        kbase = reinterpret_cast<const char*>(p.k + (size_t)cur.bg * (size_t)p.N_k * D);
        vbase = reinterpret_cast<const char*>(p.v + (size_t)cur.bg * (size_t)p.N_k * D);
        qw0 = cur.q0 + (PAIR ? (w & 3) : wr) * 32;   // first row of this wave
        qi = qw0 + l32;                      // this lane's query row
        last_vis = CAUSAL ? min(qi + off, p.N_k - 1) : p.N_k - 1;
        // tiles this wave computes: a_w .. nkb_w-1.  Later tiles lie after its
        // last row; with a window, earlier tiles lie before its first row's window
        nkb_w = cur.nkb;
        if (CAUSAL) nkb_w = max(0, min(cur.nkb, (qw0 + 31 + off) / BN + 1));
        windowed = CAUSAL && p.window > 0;
        first_vis = windowed ? qi + off - p.window + 1 : 0;   // first visible key of this lane's row
        a_w = windowed ? min(nkb_w, max(0, qw0 + off - p.window + 1) / BN) : 0;
    };

    // ---- Q fragments (B operand of S^T = K Q^T), held for a whole item
    bf16x8 qf[KSTEPS];

    // ---- per-lane LDS read offsets inside a tile, computed once.  The
    //      swizzle only depends on the row modulo 16, so moving by 16 or 32 rows
    //      is a constant added to these (an instruction immediate).
    // K fragment (A of S^T): row l32, chunk 2*ks + half
    int k_off[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) k_off[ks] = l32 * ROWB + swz<D>(l32, 2 * ks + half) * 16;
    // V^T fragment (A of O^T) through transposing reads: source row
    // 4*half + (lane%16)/4 (+8 for keys 8..15 of the 16-key step), column
    // chunk 4*dm + 2*((lane/16)%2) + (lane/2)%2, 8-byte half (lane%2)
    int v_off[2][DBLK];
    {
        const int j16 = lane & 15;
        const int vra = 4 * half + (j16 >> 2);
        const int vch = 2 * ((lane >> 4) & 1) + ((j16 >> 1) & 1);
#pragma unroll
        for (int ab = 0; ab < 2; ++ab)
#pragma unroll
            for (int dm = 0; dm < DBLK; ++dm) {
                const int r = vra + 8 * ab;
                v_off[ab][dm] = r * ROWB + swz<D>(r, dm * 4 + vch) * 16 + (j16 & 1) * 8;
            }
    }

    f32x16 oacc[DBLK];
    float m_run;                // running max (log2 units of the scaled scores)
    float nbase;                // -m_run, or 0 while the row has seen no key
    float l_a, l_b;             // this lane's part of the running sum (two chains)
    f32x16 s[NT];               // S^T of the latest tile
    bf16x8 pf[NT][2];           // P of the latest softmax-ed tile (bf16)

    // matrix-core phase of period j: O^T += V^T P^T for tile j-1 (steps
    // 0 .. NPV-1) and S^T = K Q^T for tile j (steps NPV .. NSTEP-1).  Steps of
    // up to 4 MFMAs run as a two-deep pipeline -- the LDS fragments of step
    // i+1 are read while step i's MFMAs issue -- and scheduling fences between
    // steps keep the compiler from hoisting every read (and its registers) to
    // the top.
    constexpr int NPV = NT * 2;              // 16-key steps of the PV product
    constexpr int NS = KSTEPS / 2;           // pairs of d k-steps of the S product
    constexpr int NSTEP = NPV + NS;
    static_assert(DBLK <= 4, "four fragments per step");
    struct Frags {
        bf16x8 f[4];
    };
    // step st has nmma(st) MFMAs; part k of its fragments is fragment k
    auto nmma = [](int st) constexpr { return st < NPV ? DBLK : 4; };
    // MFMAs of steps FIRST .. st-1
    auto mma_index = [](int first, int st) constexpr {
        int n = 0;
        for (int i = first; i < st; ++i) n += i < NPV ? DBLK : 4;
        return n;
    };
    auto load_part = [&](auto stc, auto kc, Frags& r, const char* kt_lds, const char* vt_lds) __attribute__((always_inline)) {
        constexpr int st = decltype(stc)::value, k = decltype(kc)::value;
        if constexpr (st < NPV) {
            const char* vp = vt_lds + ((st >> 1) * 32 + (st & 1) * 16) * ROWB;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp + v_off[0][k]));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vp + v_off[1][k]));
            r.f[k] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
            constexpr int q = st - NPV;
            r.f[k] = *reinterpret_cast<const bf16x8*>(kt_lds + (k & 1) * 32 * ROWB + k_off[2 * q + (k >> 1)]);
        }
    };
    auto mma_part = [&](auto stc, auto kc, const Frags& r) __attribute__((always_inline)) {
        constexpr int st = decltype(stc)::value, k = decltype(kc)::value;
        if constexpr (st < NPV) {
            oacc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.f[k], pf[st >> 1][st & 1], oacc[k], 0, 0, 0);
        } else {
            constexpr int q = st - NPV;
            if constexpr (q == 0 && k < 2) s[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.f[k], qf[0], f32x16{}, 0, 0, 0);
            else s[k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.f[k], qf[2 * q + (k >> 1)], s[k & 1], 0, 0, 0);
        }
    };
    // Steps FIRST .. LAST-1 as a pipeline: the fragments of step st+1 are read
    // while step st's MFMAs run, one part after each MFMA, so the reads issue
    // in the gaps while the wave waits for the matrix core; scheduling fences
    // keep that order (left alone, the compiler groups the reads and sinks
    // them below the MFMAs to reuse their registers, and the read latency or
    // issue time lands on every step).
    auto run_steps = [&](auto firstc, auto lastc, const char* kt_lds, const char* vt_lds, auto&& after_mma) __attribute__((always_inline)) {
        constexpr int FIRST = decltype(firstc)::value, LAST = decltype(lastc)::value;
        Frags cur;
        static_for<0, nmma(FIRST)>([&](auto kc) __attribute__((always_inline)) {
            load_part(firstc, kc, cur, kt_lds, vt_lds);
        });
        __builtin_amdgcn_sched_barrier(0);
        static_for<FIRST, LAST>([&](auto stc) __attribute__((always_inline)) {
            constexpr int st = decltype(stc)::value;
            constexpr int NM = nmma(st);
            constexpr int NL = st + 1 < LAST ? nmma(st + 1) : 0;
            Frags nxt;
            static_for<0, (NM > NL ? NM : NL)>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                if constexpr (k < NM) {
                    mma_part(stc, kc, cur);
                    after_mma(std::integral_constant<int, mma_index(FIRST, st) + k>{});
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (k < NL) {
                    load_part(std::integral_constant<int, st + 1>{}, kc, nxt, kt_lds, vt_lds);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            if constexpr (NL > 0) cur = nxt;
        });
    };
    // vector phase: mask, online softmax and P for tile j (held in s).
    // NOMASK: the tile is known to be whole for every row of the wave.
    auto softmax_phase = [&](int j, auto nomaskc) __attribute__((always_inline)) {
        constexpr bool NOMASK = decltype(nomaskc)::value;
        const int key0 = j * BN;
        const bool need_mask = (key0 + BN > p.N_k) || (CAUSAL && key0 + BN - 1 > qw0 + off);
        // Element masks.  Lane (l32, half) holds keys kt*32 + 8*(r/4) + r%4 +
        // 4*half of sub-tile kt.  A 32-key sub-tile that every row of the wave
        // sees whole, or that none of them sees, is settled per wave.  Inside
        // a straddling one the lane builds a 32-bit word with bit k set when
        // key k of the sub-tile is visible, and each score tests its own bit,
        // so the tests are independent.  Written as compares against a key
        // limit, the compiler sees that the conditions are monotone and
        // chains them through the scalar unit, one dependent step per score.
        auto apply_mask = [&](int kt, unsigned vis) __attribute__((always_inline)) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (!((vis >> (8 * (r >> 2) + (r & 3))) & 1u)) s[kt][r] = kNegInf;
        };
        // bits 0 .. n-1 set (n clamped to 0 .. 32)
        auto low_bits = [](int n) __attribute__((always_inline)) {
            return n >= 32 ? 0xffffffffu : n <= 0 ? 0u : (1u << n) - 1u;
        };
        if (!NOMASK && need_mask) {
            const int lim = last_vis - key0 - 4 * half;
            const int vis_lo = (CAUSAL ? min(qw0 + off, p.N_k - 1) : p.N_k - 1) - key0;   // over the wave's rows
            const int vis_hi = (CAUSAL ? min(qw0 + 31 + off, p.N_k - 1) : p.N_k - 1) - key0;
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                if (kt * 32 + 31 <= vis_lo) continue;
                if (kt * 32 > vis_hi) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kt][r] = kNegInf;
                } else {
                    apply_mask(kt, low_bits(lim - kt * 32 + 1));      // keys <= lim
                }
            }
        }
        // keys before the window of some row of this wave
        if (!NOMASK && windowed && key0 < qw0 + 31 + off - p.window + 1) {
            const int lo = first_vis - key0 - 4 * half;
            const int win_lo = qw0 + off - p.window + 1 - key0;      // over the wave's rows
            const int win_hi = qw0 + 31 + off - p.window + 1 - key0;
#pragma unroll
            for (int kt = 0; kt < NT; ++kt) {
                if (kt * 32 >= win_hi) continue;
                if (kt * 32 + 31 < win_lo) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kt][r] = kNegInf;
                } else {
                    apply_mask(kt, ~low_bits(lo - kt * 32));           // keys >= lo
                }
            }
        }
        // row max of the tile; the running max is raised only when it grows by
        // more than the slack (then O and l are rescaled)
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float m_blk = mx * p.c;
        if (__builtin_amdgcn_ballot_w64(m_blk > m_run + kRescaleSlack)) {
            const float m_new = fmaxf(m_run, m_blk);
            const float alpha = (m_run == kNegInf) ? 0.f : fast_exp2(m_run - m_new);
            l_a *= alpha;
            l_b *= alpha;
            // O is still the zero it started at until some row of the wave
            // has seen a key (the item's first tile always lands here)
            if (__builtin_amdgcn_ballot_w64(m_run != kNegInf)) {
#pragma unroll
                for (int dm = 0; dm < DBLK; ++dm) oacc[dm] *= alpha;
            }
            m_run = m_new;
            nbase = (m_new == kNegInf) ? 0.f : -m_new;
        }
        // P = exp2(c*s - m): summed in fp32 (the lse needs the unrounded
        // weights), rounded to bf16 as the B operand of O^T += V^T P^T
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                f32x8 t;
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = fast_exp2(__builtin_fmaf(s[kt][s2 * 8 + i], p.c, nbase));
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    l_a += t[i];
                    l_b += t[i + 1];
                }
                pf[kt][s2] = __builtin_convertvector(t, bf16x8);
            }
        // the phase's results exist here: without this the compiler sinks the
        // exponentials past the next barrier, next to the MFMAs that use them
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) asm volatile("" : "+v"(pf[kt][s2]));
        asm volatile("" : "+v"(l_a), "+v"(l_b));
        __builtin_amdgcn_sched_barrier(0);
    };

    // Q fragments of an item from the Q area (this wave's 32 rows)
    char* const qw_lds = qarea + wr * 32 * ROWB;
    auto read_q = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qw_lds + k_off[ks]);
    };

    // ---- periods j = kb_lo .. nkb of an item.  In period j every wave reads
    //      K tile j and V tile j-1 only, while K tile j+1 and V tile j load
    //      into the other slots.  The two waves that share a SIMD run the two
    //      phases in opposite order, so one wave's softmax overlaps the other's
    //      matrix-core work:
    //        waves 0-3:  MFMA(PV j-1, S j), softmax(j)
    //        waves 4-7:  softmax(j-1), MFMA(PV j-1, S j)
    //      A wave computes tiles a_w .. nkb_w-1: period a_w has no PV, period
    //      nkb_w no S, and the periods outside only keep the barriers and
    //      loads.  Periods kb_lo and nkb are switch periods (below), shared with
    //      the item before and after.  Each role has its own loop (straight-line
    //      phases keep the register allocation tight); all waves pass the same
    //      barriers.  Loads for the next item ride along: qpp slices of its Q
    //      block per period from period kb_lo+1 on, and its first K tile into
    //      the K slot that period nkb-1 leaves free.
    // One period: the barrier, this period's loads into the free slots, then
    // the role's phases (SM: 1 = softmax of tile j-1 before the MFMAs, 2 =
    // softmax of tile j after them).  The slot pointers are restrict
    // qualified: within a period the loads and the LDS reads touch different
    // slots, and saying so keeps the compiler from waiting for the loads
    // before the first read (their order across periods comes from the
    // explicit wait and the barrier).
    auto period = [&](int j, auto firstc, auto lastc, auto smc, auto rolec, auto steadyc, const i32x4& rk_in,
                      const i32x4& rv_in, char* __restrict__ kdst, char* __restrict__ vdst, const char* __restrict__ kt,
                      const char* __restrict__ vt) __attribute__((always_inline)) {
        constexpr int FIRST = decltype(firstc)::value, LAST = decltype(lastc)::value, SM = decltype(smc)::value;
        constexpr int ROLE = decltype(rolec)::value;     // 0, 1, or 2 = either (no matrix-core phase)
        // STEADY: K tile j+1 and V tile j belong to this item and K tile j+1
        // is whole, no Q slice of the next item loads in this period, and the
        // tile the softmax works on needs no mask
        constexpr bool STEADY = decltype(steadyc)::value;
        // this wave's loads of the previous period landed (waves 4-7 issued
        // nothing but output stores in the switch period before the item's
        // second period)
        if (STEADY || !(role == 1 && j == q_first)) __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        // K tile j+1 (or the next item's first) and V tile j.  Waves 0-3 load
        // them, one load after every other MFMA of their matrix-core phase:
        // those waves wait for the matrix core there anyway, while eight waves
        // issuing 32 loads at the barrier stall on the shared issue queue.
        // Without a matrix-core phase in this period they load at once.
        const bool ldk = STEADY || j + 1 < cur.nkb || (has_next && j == j_knext);
        const bool ldv = STEADY || j < cur.nkb;
        const i32x4 rk = STEADY ? rk_in
                       : j + 1 < cur.nkb ? tile_rsrc(kbase, j + 1)
                                         : tile_rsrc(reinterpret_cast<const char*>(p.k + (size_t)nxt.bg * (size_t)p.N_k * D), nxt.kb_lo);
        const i32x4 rv = STEADY ? rv_in : tile_rsrc(vbase, j);
        auto spread = [&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i % 2 == 0 && i / 2 < LOADS0) {
                if (ldk) issue0(rk, kdst, i / 2);
            } else if constexpr (i % 2 == 0 && i / 2 < 2 * LOADS0) {
                if (ldv) issue0(rv, vdst, i / 2 - LOADS0);
            }
        };
        constexpr bool has_mma = FIRST < LAST;
        static_assert(has_mma == (ROLE != 2), "a role with a matrix-core phase");
        static_assert(!has_mma || 2 * (2 * LOADS0) <= mma_index(FIRST, LAST), "every load fits in the phase");
        if (!has_mma && role == 0) {
#pragma unroll
            for (int i = 0; i < LOADS0; ++i) {
                if (ldk) issue0(rk, kdst, i);
                if (ldv) issue0(rv, vdst, i);
            }
        }
        // The next item's Q block: qpp parts per period over periods q_first
        // .. nkb-1, so that it has landed when the last period starts; qpp is
        // the smallest power of two that fits them in (1 for items of QPARTS
        // tiles or more: a short item does not load it all in one burst).  An
        // item with no period before its last loads it all in the last.
        if (!STEADY && has_next) {
            const int part_lo = min(QPARTS, (j - q_first) * qpp);
            const int part_hi = min(QPARTS, (j - q_first + 1) * qpp);
            for (int part = part_lo; part < part_hi; ++part) issue_q(nxt, part);
        }
        if (STEADY && j < q_lim) {
            // one slice a period (items of QPARTS tiles or more), its
            // descriptor made once per item
            const int part = j - q_first;
            if constexpr (PAIR) {
                const bool hi = part >= QPARTS / 2;
                fa_raw_buffer_load_lds(hi ? rq_nxt2 : rq_nxt, (LDS_AS void*)(qarea + (part * NTHR + w * 64) * 16), 16,
                                       ld_voff + (hi ? part - QPARTS / 2 : part) * NTHR * 16, 0, 0, kStreamOnce);
            } else {
                fa_raw_buffer_load_lds(rq_nxt, (LDS_AS void*)(qarea + (part * NTHR + w * 64) * 16), 16,
                                       ld_voff + part * NTHR * 16, 0, 0, kStreamOnce);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SM == 1) softmax_phase(j - 1, steadyc);
        if constexpr (ROLE != 0) debug_barrier();
        if constexpr (FIRST < LAST) {
            __builtin_amdgcn_s_setprio(1);           // matrix-core phase first when both waves are ready
            if constexpr (ROLE == 0) run_steps(firstc, lastc, kt, vt, spread);
            else run_steps(firstc, lastc, kt, vt, [](auto) {});
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ROLE == 0) debug_barrier();
        if constexpr (SM == 2) softmax_phase(j, steadyc);
    };
    // slots of period j: K tile j+1 and V tile j load, K tile j and V tile j-1
    // are read
    auto run_period = [&](int j, auto firstc, auto lastc, auto smc, auto rolec, auto steadyc,
                          const i32x4& rk_in = i32x4{}, const i32x4& rv_in = i32x4{}) __attribute__((always_inline)) {
        const int b = (j + sb) & 1;
        period(j, firstc, lastc, smc, rolec, steadyc, rk_in, rv_in, lds + (b ^ 1) * TILE, lds + (2 + b) * TILE,
               lds + b * TILE, lds + (2 + (b ^ 1)) * TILE);
    };
    // steady periods j .. hi-1 with the tile descriptors carried from period
    // to period (advanced by a tile, a 48-bit add), not rebuilt
    auto advance = [](i32x4 r) __attribute__((always_inline)) {
        const uint64_t a = ((uint64_t)(uint32_t)r[1] << 32 | (uint32_t)r[0]) + (uint64_t)TILE;
        r[0] = (int)(uint32_t)a;
        r[1] = (int)(uint32_t)(a >> 32);
        return r;
    };
    auto run_steady = [&](int& j, int hi, auto smc, auto rolec) __attribute__((always_inline)) {
        if (j >= hi) return;
        i32x4 rk = make_rsrc(kbase + (size_t)(j + 1) * TILE, TILE);
        i32x4 rv = make_rsrc(vbase + (size_t)j * TILE, TILE);
        for (; j < hi; ++j) {
            run_period(j, std::integral_constant<int, 0>{}, std::integral_constant<int, NSTEP>{}, smc, rolec,
                       std::true_type{}, rk, rv);
            rk = advance(rk);
            rv = advance(rv);
        }
    };
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using CNPV = std::integral_constant<int, NPV>;
    using CNSTEP = std::integral_constant<int, NSTEP>;
    using CF = std::false_type;       // a general period


    // ---- the workgroup's items: round r of a persistent grid of p.grid
    //      workgroups.  The list splits per XCD when the head count divides by
    //      8 (list index k*8 + x is on XCD x, which runs workgroups g with
    //      g % 8 == x); rounds walk it in alternating directions, so that a
    //      workgroup that took a long causal block in one round takes a short
    //      one in the next.
    auto item_id = [&](int r) __attribute__((always_inline)) {
        const int g = blockIdx.x;
        if constexpr (!PERSIST) return r == 0 ? g : -1;    // one item per workgroup
        if (p.xcd) {
            const int S = p.grid >> 3, sl = g >> 3, x = g & 7;
            const int k = r * S + ((r & 1) ? S - 1 - sl : sl);
            return k < (p.items >> 3) ? k * 8 + x : -1;
        }
        const int k = r * p.grid + ((r & 1) ? p.grid - 1 - g : g);
        return k < p.items ? k : -1;
    };

    // ---- output of a finished item.  O = O_acc / l (bf16), lse = ln2 * (m +
    //      log2 l).  A lane holds 4-element pieces of one row, so storing
    //      straight from the accumulators would write 32 rows x 8 bytes per
    //      instruction.  Each wave stages its 32 x D tile in LDS (16-byte
    //      chunks XOR-swizzled by row) and reads it back row-major: every
    //      global store is then 4 (or 8) whole rows, 1 KB contiguous, and
    //      non-temporal (O is written once).
    constexpr int RPI = 64 / CPR;                  // rows per wave-wide 16-byte read
    u32x4 pend[32 / RPI];                          // this wave's output rows, row-major
    // row sums, the LSE of rows qw0_ .. qw0_+31 of head bh, and the output
    // rows staged at ow and read back into pend
    auto finish = [&](char* ow, unsigned bh, int qw0_) __attribute__((always_inline)) {
        float l_tot;
        {
            const float l_run = l_a + l_b;
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
            l_tot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (p.lse && half == 0 && qw0_ + l32 < p.N_q)
            p.lse[(size_t)bh * (size_t)p.N_q + qw0_ + l32] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
#pragma unroll
        for (int dm = 0; dm < DBLK; ++dm)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 t;
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = oacc[dm][gq * 4 + i] * inv;
                const int c = 4 * dm + gq;         // 16-byte chunk of the row (elements 8c .. 8c+7)
                *reinterpret_cast<bf16x4*>(ow + l32 * ROWB + ((c ^ (l32 & (CPR - 1))) * 16) + half * 8) =
                    __builtin_convertvector(t, bf16x4);
            }
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int rr = k * RPI + lane / CPR, c = lane % CPR;
            pend[k] = *reinterpret_cast<const u32x4*>(ow + rr * ROWB + ((c ^ (rr & (CPR - 1))) * 16));
        }
    };
    auto store_pend = [&](unsigned bh, int qw0_) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 32 / RPI; ++k) {
            const int rr = k * RPI + lane / CPR, c = lane % CPR;
            if (qw0_ + rr < p.N_q)
                __builtin_nontemporal_store(pend[k], reinterpret_cast<u32x4*>(p.o + ((size_t)bh * (size_t)p.N_q + qw0_ + rr) * D + c * 8));
        }
    };
    auto reset_rows = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
        m_run = kNegInf;
        nbase = 0.f;
        l_a = 0.f;
        l_b = 0.f;
    };

    int r = 0;
    int id = item_id(0);
    if (id < 0) return;
    if constexpr (STAMPS) clock_stamp(p.stamps, false);
    cur = item_at(id);
    sb = 0;
    // the item after the current one (round r + 1)
    auto look_ahead = [&]() __attribute__((always_inline)) {
        const int nid = item_id(r + 1);
        has_next = PERSIST && nid >= 0;
        nxt = has_next ? item_at(nid) : cur;
    };
    look_ahead();

    // ---- switch periods.  Period nkb of an item (PV of its last tile) and
    //      period kb_lo of the next (S of its first tile) are one period, with
    //      one barrier; the first item's first period and the last item's last
    //      are such periods too, with no item before or after.  In it every
    //      wave, for the item it leaves (if it computes that item's last tile):
    //      softmax of that tile (waves 4-7), its PV product; then takes its Q
    //      fragments of the item it enters, writes the finished rows out
    //      (staged in its own rows of the Q area, which hold the entered
    //      item's Q block until those fragments are read and the next Q block
    //      only from the next period on), and, for the entered item (if it
    //      computes that item's first tile): the S product, softmax (waves
    //      0-3).  Waves 0-3 load the entered item's tiles of the period (K
    //      tile kb_lo+1, V tile kb_lo) during its S product, or at once.
    //      Between switch periods an item runs periods kb_lo+1 .. nkb-1; items
    //      have at least two key tiles (padding tiles lie past N_k or past
    //      every row's causal limit and are masked), so the next item's Q
    //      block always has a period to load in.
    // (the slot pointers are restrict-qualified parameters, as in period())
    auto switch_body = [&](auto rolec, bool has_prev, bool has_cur, bool do_pv, int j_last, unsigned prev_bh,
                           int prev_qw0, char* __restrict__ kdst, char* __restrict__ vdst, const char* __restrict__ kt,
                           const char* __restrict__ vt) __attribute__((always_inline)) {
        constexpr int RL = decltype(rolec)::value;
        static_assert(2 * (2 * LOADS0) <= mma_index(NPV, NSTEP), "the tile loads fit in the S product");
        // the first switch period needs only the prologue's Q block and first
        // K tile: waves 0-3 let their loads of the item's next tiles fly on
        if (RL == 0 && !has_prev) wait_vmcnt<2 * LOADS0>();
        else __builtin_amdgcn_s_waitcnt(0x0f70);
        __syncthreads();
        if constexpr (RL == 1) {
            if (do_pv) softmax_phase(j_last, CF{});      // with the finished item's rows
        }
        __builtin_amdgcn_sched_barrier(0);
        if (do_pv) {
            __builtin_amdgcn_s_setprio(1);
            run_steps(C0{}, CNPV{}, kt, vt, [](auto) {});
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (has_cur) {
            set_wave();
            read_q();
        }
        if (has_prev) {
            finish(qw_lds, prev_bh, prev_qw0);
            store_pend(prev_bh, prev_qw0);
        }
        reset_rows();
        if (!has_cur) return;
        const bool do_s = nkb_w > a_w && a_w == cur.kb_lo;
        const int j = cur.kb_lo;
        // (the first item's were issued in the prologue)
        const bool ldv = has_prev;
        const bool ldk = ldv && (j + 1 < cur.nkb || (has_next && j == j_knext));
        const i32x4 rk = j + 1 < cur.nkb ? tile_rsrc(kbase, j + 1)
                                        : tile_rsrc(reinterpret_cast<const char*>(p.k + (size_t)nxt.bg * (size_t)p.N_k * D), nxt.kb_lo);
        const i32x4 rv = tile_rsrc(vbase, j);
        auto spread = [&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (i % 2 == 0 && i / 2 < LOADS0) {
                if (ldk) issue0(rk, kdst, i / 2);
            } else if constexpr (i % 2 == 0 && i / 2 < 2 * LOADS0) {
                if (ldv) issue0(rv, vdst, i / 2 - LOADS0);
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        if (do_s) {
            __builtin_amdgcn_s_setprio(1);
            if constexpr (RL == 0) run_steps(CNPV{}, CNSTEP{}, kt, vt, spread);
            else run_steps(CNPV{}, CNSTEP{}, kt, vt, [](auto) {});
            __builtin_amdgcn_s_setprio(0);
            __builtin_amdgcn_sched_barrier(0);
        } else if (RL == 0) {
#pragma unroll
            for (int i = 0; i < LOADS0; ++i) {
                if (ldk) issue0(rk, kdst, i);
                if (ldv) issue0(rv, vdst, i);
            }
        }
        if constexpr (RL == 0) {
            if (do_s) softmax_phase(j, CF{});
        }
    };
    // the switch period; mb: the K slot of the entered item's first tile
    auto switch_period = [&](auto rolec, bool has_prev, bool has_cur, bool do_pv, int j_last, unsigned prev_bh,
                             int prev_qw0, int mb) __attribute__((always_inline)) {
        switch_body(rolec, has_prev, has_cur, do_pv, j_last, prev_bh, prev_qw0, lds + (mb ^ 1) * TILE,
                    lds + (2 + mb) * TILE, lds + mb * TILE, lds + (2 + (mb ^ 1)) * TILE);
    };

    // prologue: the first item's Q block and first K tile (every wave), then
    // its K tile kb_lo+1 and V tile kb_lo (waves 0-3, the loads of its first
    // switch period, which waits for the first two only).  A K tile past the
    // item (an item alone in its workgroup with one tile) loads as zeros or
    // unused keys.
#pragma unroll
    for (int part = 0; part < QPARTS; ++part) issue_q(cur, part);
    issue(reinterpret_cast<const char*>(p.k + (size_t)cur.bg * (size_t)p.N_k * D), cur.kb_lo, lds + (cur.kb_lo & 1) * TILE);
    if (role == 0) {
        const int mb0 = cur.kb_lo & 1;
        const i32x4 rk = tile_rsrc(reinterpret_cast<const char*>(p.k + (size_t)cur.bg * (size_t)p.N_k * D), cur.kb_lo + 1);
        const i32x4 rv = tile_rsrc(reinterpret_cast<const char*>(p.v + (size_t)cur.bg * (size_t)p.N_k * D), cur.kb_lo);
#pragma unroll
        for (int i = 0; i < LOADS0; ++i) {
            issue0(rk, lds + (mb0 ^ 1) * TILE, i);
            issue0(rv, lds + (2 + mb0) * TILE, i);
        }
    }

    // The item loop, compiled once per wave role (the two roles carry
    // different registers from period to period)
    auto item_loop = [&](auto rolec) __attribute__((always_inline)) {
        constexpr int RL = decltype(rolec)::value;
        bool has_prev = false, has_cur = true, do_pv = false;
        int j_last = 0, prev_qw0 = 0;
        unsigned prev_bh = 0;
        int mb = cur.kb_lo & 1;                  // K slot of the entered item's first tile
        j_knext = max(cur.kb_lo, cur.nkb - 1);
        for (;;) {
            switch_period(rolec, has_prev, has_cur, do_pv, j_last, prev_bh, prev_qw0, mb);
            if (!has_cur) break;
            // the next item's Q block loads in periods q_first .. nkb-1
            q_first = cur.kb_lo + 1;
            const int qcount = cur.nkb - q_first;
            qpp = 1;
            while (qpp < QPARTS && qpp * qcount < QPARTS) qpp *= 2;
            q_lim = has_next && qpp == 1 ? q_first + QPARTS : q_first;
            if (has_next) {
                const unsigned qbytes = (unsigned)max(0, min(BMI, p.N_q - nxt.q0)) * ROWB;
                rq_nxt = make_rsrc(p.q + ((size_t)(PAIR ? nxt.bh2 : nxt.bh) * (size_t)p.N_q + (size_t)nxt.q0) * D,
                                   qbytes);
                if constexpr (PAIR)
                    rq_nxt2 = make_rsrc(p.q + ((size_t)nxt.bh * (size_t)p.N_q + (size_t)nxt.q0) * D, qbytes);
            }
            // this wave's first period (S of tile a_w) ran in the switch period
            // when the wave starts at the item's first tile; its last (PV of
            // tile nkb-1) runs in the next one when it ends at the item's last
            const bool started = a_w == cur.kb_lo;
            const bool ends = nkb_w == cur.nkb;
            int j = q_first;
            for (; j < a_w; ++j) run_period(j, C0{}, C0{}, C0{}, C2{}, CF{});    // tiles before this wave's window
            if (nkb_w > a_w) {
                // Steady periods (see period()) j, lo <= j < hi:
                //  * after the first period after the switch period and the
                //    periods that load the next item's Q slices (unless they
                //    load one slice each);
                //  * K tile j+1 and V tile j whole (j + 1 < full, the whole
                //    tiles) and of this item (j + 1 < nkb, so not the next
                //    item's first K tile either);
                //  * the tile the softmax works on (j for waves 0-3, j-1 for
                //    waves 4-7) whole for every row of the wave: t_lo <= t <
                //    t_hi, where t_hi is the first tile reaching past N_k or
                //    past the wave's first row's last visible key, and t_lo
                //    (window) the first tile inside the window of the wave's
                //    last row;
                //  * within the wave's matrix-core periods (j < nkb_w).
                const int qperiods = has_next ? (QPARTS + qpp - 1) / qpp : 0;
                const int full = p.N_k / BN;
                int t_hi = full;
                if (CAUSAL) t_hi = min(t_hi, max(0, qw0 + off + 1) / BN);
                int t_lo = 0;
                if (windowed) t_lo = max(0, qw0 + 31 + off - p.window + 1 + BN - 1) / BN;
                const int s_lo = q_first + max(1, qpp == 1 ? 0 : qperiods);
                const int s_hi = min(min(nkb_w, cur.nkb - 1), full - 1);
                if constexpr (RL == 0) {
                    if (!started) run_period(j++, CNPV{}, CNSTEP{}, C2{}, C0{}, CF{});
                    const int lo = min(max(j, max(s_lo, t_lo)), nkb_w);           // softmax of tile j
                    const int hi = max(lo, min(s_hi, t_hi));
                    for (; j < lo; ++j) run_period(j, C0{}, CNSTEP{}, C2{}, C0{}, CF{});
                    run_steady(j, hi, C2{}, C0{});
                    for (; j < nkb_w; ++j) run_period(j, C0{}, CNSTEP{}, C2{}, C0{}, CF{});
                    if (!ends) run_period(j++, C0{}, CNPV{}, C0{}, C0{}, CF{});   // j == nkb_w: PV of the last tile
                } else {
                    if (!started) run_period(j++, CNPV{}, CNSTEP{}, C0{}, C1{}, CF{});
                    const int lo = min(max(j, max(s_lo, t_lo + 1)), nkb_w);       // softmax of tile j-1
                    const int hi = max(lo, min(s_hi, t_hi + 1));
                    for (; j < lo; ++j) run_period(j, C0{}, CNSTEP{}, C1{}, C1{}, CF{});
                    run_steady(j, hi, C1{}, C1{});
                    for (; j < nkb_w; ++j) run_period(j, C0{}, CNSTEP{}, C1{}, C1{}, CF{});
                    if (!ends) run_period(j++, C0{}, CNPV{}, C1{}, C1{}, CF{});
                }
            }
            for (; j < cur.nkb; ++j) run_period(j, C0{}, C0{}, C0{}, C2{}, CF{});  // tiles after this wave's rows
            // the next switch period leaves this item
            has_prev = true;
            do_pv = nkb_w > a_w && nkb_w == cur.nkb;
            j_last = cur.nkb - 1;
            prev_bh = PAIR && RL == 1 ? cur.bh2 : cur.bh;    // this wave's head
            prev_qw0 = qw0;
            mb = (cur.nkb + sb) & 1;
            has_cur = has_next;
            if (has_next) {
                sb = (j_knext + 1 + sb - nxt.kb_lo) & 1;   // the next item's first K tile sits in slot (j_knext + 1 + sb) % 2
                cur = nxt;
                ++r;
                look_ahead();
                j_knext = max(cur.kb_lo, cur.nkb - 1);
            }
        }
    };
    if (role == 0) item_loop(C0{});
    else item_loop(C1{});
    if constexpr (STAMPS) {
        // the record pointer is read again from the kernel arguments here
        // rather than kept in registers through the item loop
        const char* kernarg = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
        clock_stamp(*reinterpret_cast<unsigned long long* const volatile*>(kernarg + offsetof(Params, stamps)), true);
    }
}

// Workgroups that fit on the current device at once: the grid of the
// persistent kernel.  Cached per device and kernel (host threads may race to
// fill an entry; they store the same value).
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

template <int D, int NW, bool CAUSAL, bool PERSIST, bool STAMPS = false, bool PAIR = false>
hipError_t launch(const FwdArgs& a, int group, hipStream_t stream)
{
    constexpr int BM = NW * 32;
    static_assert(BM == kFwdBf16Rows, "the host checks item counts with this block size");
    // paired items: half the rows of twice the heads, so no more items than
    // BM-row blocks of single heads (the host's count bounds both)
    constexpr int BMI = PAIR ? BM / 2 : BM;
    Params p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.o = static_cast<uint16_t*>(a.o);
    p.lse = a.lse;
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.N_q = a.N_q;
    p.N_k = a.N_k;
    p.rep = a.H / a.H_kv;
    p.hpb = PAIR ? a.H / 2 : a.H;
    p.nqb = (a.N_q + BMI - 1) / BMI;
    // a group of the item order spans `group` heads either way (pairs of heads
    // with paired items), so that its K/V stays within one XCD's L2
    p.group = PAIR ? group / 2 : group;
    if (p.group < 1) p.group = 1;
    {
        const int HB = p.hpb * a.B;
        p.split8 = (HB & 7) == 0;
        p.nheads = p.split8 ? HB >> 3 : HB;
        p.gsz = p.group < p.nheads ? p.group : p.nheads;
        p.last_grp = (p.nheads - 1) / p.gsz;
        p.glast = p.nheads - p.last_grp * p.gsz;
        p.div_gn = div_const((unsigned)(p.gsz * p.nqb));
        p.div_gsz = div_const((unsigned)p.gsz);
        p.div_glast = div_const((unsigned)p.glast);
        p.div_h = div_const((unsigned)p.hpb);
        p.div_rep = div_const((unsigned)p.rep);
    }
    p.window = CAUSAL ? a.window : 0;
    // scale 0 runs as a tiny positive scale: every exp2 argument then rounds to
    // 0 exactly as with scale 0, and masked scores stay -inf instead of NaN
    p.c = a.scale > 0.f ? a.scale * kLog2e : 1e-30f;
    p.stamps = a.clock_stamps;
    const long long items = (long long)p.nqb * p.hpb * a.B;   // at most 2^31 - 1: checked on the host
    if (items == 0) return hipSuccess;
    long long grid = items;
    int xcd = 0;
    if (PERSIST) {
        const int resident = resident_blocks<fwd_bf16_kernel<D, NW, CAUSAL, PERSIST, STAMPS, PAIR>>(NW * 64);
        if (resident <= 0) return hipErrorInvalidDevice;
        if (resident < grid) grid = resident;
        if (a.max_workgroups > 0 && a.max_workgroups < grid) grid = a.max_workgroups;
        // the per-XCD split needs whole rows of 8 workgroups (items is then a
        // multiple of 8 too); otherwise the rounds walk the whole list
        if (((p.hpb * a.B) & 7) == 0 && grid >= 8) {
            grid = grid / 8 * 8;
            xcd = 1;
        }
    }
    p.xcd = xcd;
    p.items = (int)items;
    p.grid = (int)grid;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL, PERSIST, STAMPS, PAIR>), dim3((unsigned)grid), dim3(NW * 64), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

#ifndef FA_FWD_GROUP
#define FA_FWD_GROUP 4
#endif

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream)
{
    const int group = FA_FWD_GROUP;
    // d = 128 runs persistent (one workgroup per CU, item switches hidden
    // behind the next item's loads); d = 64 fits two workgroups per CU, which
    // hide each other's start and end, and runs one item per workgroup
    // Causal items pair two heads that share a KV head when the GQA ratio is
    // even: the same K/V tiles serve both, and the diagonal, where only the
    // waves whose rows reach a tile work, spans two tiles instead of four
    const bool pair = a.causal && (a.H / a.H_kv) % 2 == 0;
    if (a.d == 128 && a.clock_stamps) {   // the test hook's clock record: its own instantiation
        if (pair) return launch<128, 8, true, true, true, true>(a, group, stream);
        return a.causal ? launch<128, 8, true, true, true>(a, group, stream)
                        : launch<128, 8, false, true, true>(a, group, stream);
    }
    if (a.d == 128) {
        if (pair) return launch<128, 8, true, true, false, true>(a, group, stream);
        return a.causal ? launch<128, 8, true, true>(a, group, stream) : launch<128, 8, false, true>(a, group, stream);
    }
    if (a.d == 64)
        return a.causal ? launch<64, 8, true, false>(a, group, stream) : launch<64, 8, false, false>(a, group, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
