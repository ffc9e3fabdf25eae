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
// Split pass: workgroup (c, head group, b) takes keys
// [c*L, min((c+1)*L, len)) with L = ceil(len / num_splits) and serves HG query
// heads that share one KV head, so each K/V byte of the chunk is read from HBM
// once for all of them.  Rows are streamed with 16-byte loads, D/8 lanes per
// row, several rows in flight per lane.  Each row slot of a wave keeps its own
// running max / running sum / output (the online softmax of "Attention
// variants" §3); row slots and waves are merged at the end with the same
// rescale rule.  The chunk result is written as o_c = O/l (fp32) and
// lse_c = m + ln l; an empty chunk writes lse_c = -inf, o_c = 0.
//
// Merge pass (not on the pages; the online-softmax rescale applied to whole
// chunk summaries): M = max_c lse_c, lse = M + ln sum_c exp(lse_c - M),
// o = sum_c exp(lse_c - lse) o_c, rounded to bf16.
#include "fa_internal.h"

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

struct SplitParams {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const int* seq_lens;
    float* part_o;
    float* part_lse;
    int H, H_kv, N_max, S, rep;
    float c;      // scale * log2(e)
};

__device__ __forceinline__ float bf_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over the LPR consecutive lanes that hold one cache row (DPP within a row of 16).
template <int LPR>
__device__ __forceinline__ float row_sum(float x)
{
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)); // mirror in 8
    if (LPR == 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)); // mirror in 16
    return x;
}

// Merge running state (m, l, o) with another one (all in log2 units).
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float* o, float m2, float l2, const float* o2)
{
    const float mn = fmaxf(m, m2);
    const float base = (mn == kNegInf) ? 0.f : mn;
    const float a1 = fast_exp2(m - base), a2 = fast_exp2(m2 - base);
    l = a1 * l + a2 * l2;
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = a1 * o[i] + a2 * o2[i];
    m = mn;
}

template <int D, int HG>
__global__ __launch_bounds__(256) void decode_split_kernel(SplitParams p)
{
    constexpr int NW = 4;
    constexpr int LPR = D / 8;           // lanes per cache row
    constexpr int RPW = 64 / LPR;        // rows per wave per load
    constexpr int U = 4;                 // loads in flight per lane (per K and per V)
    constexpr int ROWS_WAVE = RPW * U;   // rows per wave per iteration
    constexpr int ROWS_ITER = NW * ROWS_WAVE;

    __shared__ float sh_m[NW][HG];
    __shared__ float sh_l[NW][HG];
    __shared__ float sh_o[NW][HG][D];

    const int c = blockIdx.x;
    const int h0 = blockIdx.y * HG;
    const int b = blockIdx.z;
    const int g = h0 / p.rep;
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63;
    const int slot = lane / LPR;         // which row of a load this lane serves
    const int dl = lane % LPR;           // 8 elements d = 8*dl .. 8*dl+7

    const int len = p.seq_lens[b];
    const int L = (len + p.S - 1) / p.S;
    const int j0 = c * L;
    const int j1 = min(j0 + L, len);

    // queries of the HG heads, pre-scaled by scale*log2(e): scores come out in log2 units
    float q[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        const u32x4 t = reinterpret_cast<const u32x4*>(p.q + ((size_t)b * p.H + h0 + hh) * D)[dl];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            q[hh][2 * i] = bf_lo(t[i]) * p.c;
            q[hh][2 * i + 1] = bf_hi(t[i]) * p.c;
        }
    }

    float m[HG], l[HG], o[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        m[hh] = kNegInf;
        l[hh] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[hh][i] = 0.f;
    }

    const size_t kv_row0 = ((size_t)b * p.H_kv + g) * (size_t)p.N_max;
    const u32x4* kbase = reinterpret_cast<const u32x4*>(p.k + kv_row0 * D) + dl;
    const u32x4* vbase = reinterpret_cast<const u32x4*>(p.v + kv_row0 * D) + dl;

    for (int r0 = j0; r0 < j1; r0 += ROWS_ITER) {
        u32x4 kr[U], vr[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = r0 + w * ROWS_WAVE + u * RPW + slot;
            ok[u] = j < j1;
            kr[u] = ok[u] ? kbase[(size_t)j * (D / 8)] : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = r0 + w * ROWS_WAVE + u * RPW + slot;
            vr[u] = ok[u] ? vbase[(size_t)j * (D / 8)] : u32x4{0, 0, 0, 0};
        }
        // scores of the U rows for the HG heads
        float s[U][HG];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float kf[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                kf[2 * i] = bf_lo(kr[u][i]);
                kf[2 * i + 1] = bf_hi(kr[u][i]);
            }
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(q[hh][i], kf[i], acc);
                s[u][hh] = row_sum<LPR>(acc);
            }
        }
        // online softmax over the U rows of this slot
        float vf[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vf[u][2 * i] = bf_lo(vr[u][i]);
                vf[u][2 * i + 1] = bf_hi(vr[u][i]);
            }
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            float mx = kNegInf;
#pragma unroll
            for (int u = 0; u < U; ++u) mx = fmaxf(mx, ok[u] ? s[u][hh] : kNegInf);
            const float mn = fmaxf(m[hh], mx);
            const float base = (mn == kNegInf) ? 0.f : mn;
            const float alpha = fast_exp2(m[hh] - base);
            float pr[U];
            float ps = 0.f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                pr[u] = ok[u] ? fast_exp2(s[u][hh] - base) : 0.f;
                ps += pr[u];
            }
            l[hh] = alpha * l[hh] + ps;
            m[hh] = mn;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float acc = o[hh][i] * alpha;
#pragma unroll
                for (int u = 0; u < U; ++u) acc = __builtin_fmaf(pr[u], vf[u][i], acc);
                o[hh][i] = acc;
            }
        }
    }

    // merge the row slots of this wave (lanes with equal dl)
#pragma unroll
    for (int x = LPR; x < 64; x <<= 1) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            const float m2 = __shfl_xor(m[hh], x);
            const float l2 = __shfl_xor(l[hh], x);
            float o2[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) o2[i] = __shfl_xor(o[hh][i], x);
            merge_state<8>(m[hh], l[hh], o[hh], m2, l2, o2);
        }
    }
    if (slot == 0) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            if (dl == 0) {
                sh_m[w][hh] = m[hh];
                sh_l[w][hh] = l[hh];
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) sh_o[w][hh][dl * 8 + i] = o[hh][i];
        }
    }
    __syncthreads();
    // merge the waves and write the chunk's partial result
    for (int e = tid; e < HG * D; e += 256) {
        const int hh = e / D, d = e % D;
        float mm = sh_m[0][hh], ll = sh_l[0][hh], oo = sh_o[0][hh][d];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) merge_state<1>(mm, ll, &oo, sh_m[ww][hh], sh_l[ww][hh], &sh_o[ww][hh][d]);
        const size_t row = ((size_t)b * p.H + h0 + hh) * p.S + c;
        p.part_o[row * D + d] = ll > 0.f ? oo / ll : 0.f;
        if (d == 0) p.part_lse[row] = ll > 0.f ? (mm + __builtin_log2f(ll)) * kLn2 : kNegInf;
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
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(CombineParams p)
{
    constexpr int PER = D / 64;          // output elements per lane
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= p.rows) return;
    const float* lse_c = p.part_lse + (size_t)row * p.S;
    float mx = kNegInf;
    for (int c = lane; c < p.S; c += 64) mx = fmaxf(mx, lse_c[c]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
    float sum = 0.f;
    if (mx != kNegInf)
        for (int c = lane; c < p.S; c += 64) sum += exp2f((lse_c[c] - mx) * kLog2e);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) sum += __shfl_xor(sum, x);
    const float lse = (mx == kNegInf || sum <= 0.f) ? kNegInf : mx + logf(sum);
    float acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] = 0.f;
    if (lse != kNegInf) {
        const float* oc = p.part_o + (size_t)row * p.S * D + lane * PER;
        for (int c = 0; c < p.S; ++c) {
            const float wgt = exp2f((lse_c[c] - lse) * kLog2e);
#pragma unroll
            for (int i = 0; i < PER; ++i) acc[i] = __builtin_fmaf(wgt, oc[(size_t)c * D + i], acc[i]);
        }
    }
    uint16_t* dst = p.o + (size_t)row * D + lane * PER;
    if (PER == 2) {
        const bf16x2 t = __builtin_convertvector((f32x2{acc[0], acc[PER - 1]}), bf16x2);
        *reinterpret_cast<bf16x2*>(dst) = t;
    } else {
        const bf16x2 t = __builtin_convertvector((f32x2{acc[0], 0.f}), bf16x2);
        dst[0] = __builtin_bit_cast(uint16_t, t[0]);
    }
    if (p.lse && lane == 0) p.lse[row] = lse;
}

template <int D, int HG>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream)
{
    SplitParams p;
    p.q = static_cast<const uint16_t*>(a.q);
    p.k = static_cast<const uint16_t*>(a.k);
    p.v = static_cast<const uint16_t*>(a.v);
    p.seq_lens = a.seq_lens;
    p.part_o = a.part_o;
    p.part_lse = a.part_lse;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.N_max = a.N_max;
    p.S = a.num_splits;
    p.rep = a.H / a.H_kv;
    p.c = a.scale * kLog2e;
    if ((long long)a.H / HG > 65535 || a.B > 65535) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((decode_split_kernel<D, HG>), dim3(a.num_splits, a.H / HG, a.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_all(const DecodeArgs& a, hipStream_t stream)
{
    const int rep = a.H / a.H_kv;
    // heads per workgroup: the largest of 8, 4, 2, 1 dividing H/H_kv
    hipError_t e;
    if (rep % 8 == 0) e = launch_split<D, 8>(a, stream);
    else if (rep % 4 == 0) e = launch_split<D, 4>(a, stream);
    else if (rep % 2 == 0) e = launch_split<D, 2>(a, stream);
    else e = launch_split<D, 1>(a, stream);
    if (e != hipSuccess) return e;
    CombineParams cp{a.part_o, a.part_lse, static_cast<uint16_t*>(a.o), a.lse, a.B * a.H, a.num_splits};
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((cp.rows + 3) / 4), dim3(256), 0, stream, cp);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream)
{
    if (a.d == 128) return launch_all<128>(a, stream);
    if (a.d == 64) return launch_all<64>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
