// fwd_bf16.hip -- tiled exact attention forward on gfx950 bf16 MFMA.
//
// Method ("Attention variants: GQA/MQA/FlashAttention" (youngju.dev) §3):
// cut Q into blocks (one per workgroup) and K/V into blocks streamed through
// LDS; per query row keep a running maximum m and running sum l; for each key
// block compute the block scores, raise m, bring the accumulator and l to the
// new m, add the block's exp(S - m) V; divide by l at the end.  Causal
// problems skip key blocks wholly in the future and mask inside the diagonal
// blocks (§5.5 of the same page).  Query head h reads KV head h / (H / H_kv)
// (§2 of the same page; "Attention mechanism evolution" (toolsku.com) GQA code).
//
// gfx950 mapping (not from the pages; the pages' kernel targets other GPUs):
//  * workgroup = NW waves, BM = 32*NW query rows; each wave owns 32 rows;
//  * scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = K fragment from LDS, B = Q fragment held in
//    VGPRs for the whole kernel.  In the 32x32 accumulator layout lane l holds
//    column l%32, i.e. one query row, and 16 of the 32 keys, so the row max
//    and row sum are in-lane plus one exchange with lane l^32;
//  * the output is accumulated transposed too, O^T += V^T P^T, so it shares
//    the one-query-per-lane layout and the rescale by exp(m_old - m_new) is a
//    per-lane scalar;  P (fp32 -> bf16, round to nearest even) feeds the B
//    operand straight from the score registers;
//  * V is stored transposed in LDS (d rows, key columns) with bits 2 and 3 of
//    the key index swapped inside each 16-key group, which puts the 8 keys a
//    lane contributes to one MFMA next to each other: one 16-byte LDS read;
//  * softmax in base 2: scores are scaled by scale*log2(e) once, exp2 is the
//    hardware v_exp_f32;  lse = ln2 * (m + log2 l) at the end;
//  * the next K/V tile is fetched into registers while the current one is
//    being computed; LDS rows are padded so MFMA fragment reads are
//    bank-conflict free.
#include "fa_internal.h"

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

struct Params {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    uint16_t* o;
    float* lse;
    int B, H, H_kv, N_q, N_k;
    int rep;      // H / H_kv
    int nqb;      // query blocks per head
    float c;      // scale * log2(e)
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swap bits 2 and 3 of a key index (inside each 16-key group).
__device__ __forceinline__ int key_swizzle(int key)
{
    int t = ((key >> 2) ^ (key >> 3)) & 1;
    return key ^ (t * 0xC);
}

template <int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(Params p)
{
    constexpr int BM = NW * 32;          // query rows per workgroup
    constexpr int NTHR = NW * 64;
    constexpr int KSTEPS = D / 16;       // MFMA k-steps over d for S^T
    constexpr int DBLK = D / 32;         // 32-row blocks of d for O^T
    constexpr int NT = BN / 32;          // 32-key sub-tiles per key block
    constexpr int KROW = D + 8;          // padded K row in LDS (elements)
    constexpr int VROW = BN + 8;         // padded V^T row in LDS (elements)
    constexpr int KCH = BN * D / 8;      // 16-byte chunks in a K tile
    constexpr int KPT = (KCH + NTHR - 1) / NTHR;
    constexpr int VPAIRS = (BN / 4) * (D / 8);   // (4-key quad, 8-d chunk) pairs
    constexpr int VPT = (VPAIRS + NTHR - 1) / NTHR;
    static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t k_lds[BN * KROW];
    __shared__ __attribute__((aligned(16))) uint16_t vt_lds[D * VROW];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // ---- work decomposition: one workgroup per (query block, head, batch);
    //      causal problems run the longest query blocks first
    const int HB = p.H * p.B;
    int qb = blockIdx.x / HB;
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int bh = blockIdx.x % HB;
    const int h = bh % p.H;
    const int b = bh / p.H;
    const int g = h / p.rep;
    const int q0 = qb * BM;
    const int off = p.N_k - p.N_q;                 // causal diagonal offset
    const int qw0 = q0 + w * 32;                   // first row of this wave
    const int qi = qw0 + l32;                      // this lane's query row

    const size_t q_row0 = (size_t)(b * p.H + h) * (size_t)p.N_q;
    const size_t kv_row0 = (size_t)(b * p.H_kv + g) * (size_t)p.N_k;

    int kend = p.N_k;
    if (CAUSAL) kend = min(p.N_k, q0 + BM + off);
    const int nkb = kend > 0 ? (kend + BN - 1) / BN : 0;

    // ---- Q fragments (B operand of S^T = K Q^T), resident for the whole kernel
    bf16x8 qf[KSTEPS];
    {
        const bool ok = qi < p.N_q;
        const u32x4* src = reinterpret_cast<const u32x4*>(p.q + (q_row0 + (size_t)(ok ? qi : 0)) * D);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            u32x4 t = ok ? src[2 * ks + half] : u32x4{0, 0, 0, 0};
            qf[ks] = __builtin_bit_cast(bf16x8, t);
        }
    }

    f32x16 oacc[DBLK];
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf;      // running max, log2 units of the scaled scores
    float l_run = 0.f;          // this lane's part of the running sum

    // ---- register prefetch of one K/V tile
    u32x4 kreg[KPT];
    u32x4 vreg[VPT][4];
    auto fetch = [&](int kb) {
        const int key0 = kb * BN;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * NTHR;
            const int row = c / (D / 8), col = c % (D / 8);
            const bool ok = c < KCH && key0 + row < p.N_k;
            kreg[i] = ok ? reinterpret_cast<const u32x4*>(p.k + (kv_row0 + key0 + row) * D)[col]
                         : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = tid + i * NTHR;
            const int quad = c % (BN / 4), dch = c / (BN / 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int key = key0 + quad * 4 + j;
                const bool ok = c < VPAIRS && key < p.N_k;
                vreg[i][j] = ok ? reinterpret_cast<const u32x4*>(p.v + (kv_row0 + key) * D)[dch]
                                : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * NTHR;
            if (c < KCH) {
                const int row = c / (D / 8), col = c % (D / 8);
                *reinterpret_cast<u32x4*>(&k_lds[row * KROW + col * 8]) = kreg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int c = tid + i * NTHR;
            if (c < VPAIRS) {
                const int quad = c % (BN / 4), dch = c / (BN / 4);
                const int kcol = key_swizzle(quad * 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // d = 8*dch + e: gather that element from the four key rows
                    const int wd = e >> 1;
                    u32x2 pk;
                    if (e & 1) {      // odd d: high halves of the four rows
                        pk[0] = (vreg[i][0][wd] >> 16) | (vreg[i][1][wd] & 0xffff0000u);
                        pk[1] = (vreg[i][2][wd] >> 16) | (vreg[i][3][wd] & 0xffff0000u);
                    } else {          // even d: low halves
                        pk[0] = (vreg[i][0][wd] & 0xffffu) | (vreg[i][1][wd] << 16);
                        pk[1] = (vreg[i][2][wd] & 0xffffu) | (vreg[i][3][wd] << 16);
                    }
                    *reinterpret_cast<u32x2*>(&vt_lds[(dch * 8 + e) * VROW + kcol]) = pk;
                }
            }
        }
    };

    if (nkb > 0) fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
        __syncthreads();
        stage();
        __syncthreads();
        if (kb + 1 < nkb) fetch(kb + 1);

        const int key0 = kb * BN;
        // wave-level causal skip: the whole block lies after this wave's last row
        if (CAUSAL && key0 > qw0 + 31 + off) continue;
        const bool need_mask = (key0 + BN > p.N_k) || (CAUSAL && key0 + BN - 1 > qw0 + off);

        // ---- S^T = K Q^T for the BN keys of the block (fp32 accumulate)
        f32x16 s[NT];
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            s[kt] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                    &k_lds[(kt * 32 + l32) * KROW + ks * 16 + half * 8]);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kt], 0, 0, 0);
            }
        }

        // ---- mask: keys past N_k, and (causal) keys after this row's diagonal
        if (need_mask) {
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = key0 + kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                    const bool vis = key < p.N_k && (!CAUSAL || key <= qi + off);
                    if (!vis) s[kt][r] = kNegInf;
                }
        }

        // ---- online softmax update of this row
        float mx = kNegInf;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mx2 = (mx == kNegInf) ? kNegInf : mx * p.c;
        const float m_new = fmaxf(m_run, mx2);
        const float base = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - base);
        float lsum = 0.f;
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float e = fast_exp2(__builtin_fmaf(s[kt][r], p.c, -base));
                if (need_mask && s[kt][r] == kNegInf) e = 0.f;
                s[kt][r] = e;
                lsum += e;
            }
        l_run = alpha * l_run + lsum;
        m_run = m_new;
#pragma unroll
        for (int dm = 0; dm < DBLK; ++dm) oacc[dm] *= alpha;

        // ---- P^T fragments: bf16, 8 keys per MFMA k-step
        bf16x8 pf[NT][2];
#pragma unroll
        for (int kt = 0; kt < NT; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                f32x8 t;
#pragma unroll
                for (int i = 0; i < 8; ++i) t[i] = s[kt][s2 * 8 + i];
                pf[kt][s2] = __builtin_convertvector(t, bf16x8);
            }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int dm = 0; dm < DBLK; ++dm)
#pragma unroll
            for (int kt = 0; kt < NT; ++kt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                        &vt_lds[(dm * 32 + l32) * VROW + kt * 32 + s2 * 16 + half * 8]);
                    oacc[dm] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kt][s2], oacc[dm], 0, 0, 0);
                }
    }

    // ---- epilogue: O = O_acc / l (bf16), lse = ln2 * (m + log2 l)
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qi < p.N_q) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* dst = p.o + (q_row0 + qi) * D;
#pragma unroll
        for (int dm = 0; dm < DBLK; ++dm)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
                f32x4 t;
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = oacc[dm][gq * 4 + i] * inv;
                const bf16x4 ob = __builtin_convertvector(t, bf16x4);
                *reinterpret_cast<bf16x4*>(dst + dm * 32 + gq * 8 + half * 4) = ob;
            }
        if (p.lse && half == 0)
            p.lse[q_row0 + qi] = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : kNegInf;
    }
}

template <int D, int NW, int BN, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream)
{
    constexpr int BM = NW * 32;
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
    p.nqb = (a.N_q + BM - 1) / BM;
    p.c = a.scale * kLog2e;
    const long long blocks = (long long)p.nqb * a.H * a.B;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, CAUSAL>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream)
{
    if (a.d == 128)
        return a.causal ? launch<128, 4, 64, true>(a, stream) : launch<128, 4, 64, false>(a, stream);
    if (a.d == 64)
        return a.causal ? launch<64, 4, 64, true>(a, stream) : launch<64, 4, 64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
