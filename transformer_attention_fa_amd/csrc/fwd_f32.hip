// fwd_f32.hip -- tiled exact attention forward in fp32 (fp32 in, fp32 out).
//
// Same method as the bf16 kernel ("Attention variants: GQA/MQA/FlashAttention"
// (youngju.dev) §3 tiling with a running max and running sum per row, §5.5
// causal block skip, §2 head sharing), with fp32 arithmetic throughout: this
// path exists for callers that need fp32 results, not for speed, so it uses
// plain fp32 FMAs rather than the matrix cores.
//
// Layout of the work: each query row is owned by D/32 consecutive lanes, each
// holding 32 elements of q and of the output accumulator in registers; a
// workgroup of 256 lanes owns 256/(D/32) rows.  Key and value tiles of 32 rows
// go through LDS, where every lane of a row group reads the same address (an
// LDS broadcast).  Partial dot products are summed over the D/32 lanes with
// cross-lane shuffles.
#include "fa_internal.h"

#include <hip/hip_runtime.h>
#include <cstdint>

namespace fa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

struct Params {
    const float* q;
    const float* k;
    const float* v;
    float* o;
    float* lse;
    int B, H, H_kv, N_q, N_k;
    int rep;
    int nqb;
    float c;      // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(Params p)
{
    constexpr int SPLIT = D / 32;        // lanes per query row
    constexpr int BM = 256 / SPLIT;      // query rows per workgroup
    constexpr int BK = 32;               // keys per tile
    constexpr int CST = 36;              // padded 32-float chunk stride in LDS
    constexpr int ROW = SPLIT * CST;     // one key row in LDS (floats)
    constexpr int CHUNKS = BK * D / 4;   // float4 chunks per tile

    __shared__ __attribute__((aligned(16))) float k_lds[BK * ROW];
    __shared__ __attribute__((aligned(16))) float v_lds[BK * ROW];

    const int tid = threadIdx.x;
    const int sub = tid % SPLIT;         // which 32 of the d elements
    const int row_in_block = tid / SPLIT;

    const int HB = p.H * p.B;
    int qb = blockIdx.x / HB;
    if (CAUSAL) qb = p.nqb - 1 - qb;
    const int bh = blockIdx.x % HB;
    const int h = bh % p.H;
    const int b = bh / p.H;
    const int g = h / p.rep;
    const int q0 = qb * BM;
    const int qi = q0 + row_in_block;
    const int off = p.N_k - p.N_q;

    const size_t q_row0 = (size_t)(b * p.H + h) * (size_t)p.N_q;
    const size_t kv_row0 = (size_t)(b * p.H_kv + g) * (size_t)p.N_k;

    float q[32], o[32];
    {
        const bool ok = qi < p.N_q;
        const f32x4* src = reinterpret_cast<const f32x4*>(p.q + (q_row0 + (ok ? qi : 0)) * D + sub * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f32x4 t = ok ? src[i] : f32x4{0.f, 0.f, 0.f, 0.f};
            q[4 * i + 0] = t[0];
            q[4 * i + 1] = t[1];
            q[4 * i + 2] = t[2];
            q[4 * i + 3] = t[3];
        }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    int kend = p.N_k;
    if (CAUSAL) kend = min(p.N_k, q0 + BM + off);
    const int nkb = kend > 0 ? (kend + BK - 1) / BK : 0;

    for (int kb = 0; kb < nkb; ++kb) {
        const int key0 = kb * BK;
        __syncthreads();
        for (int c = tid; c < CHUNKS; c += 256) {
            const int r = c / (D / 4), col = c % (D / 4);
            const int dst = r * ROW + (col / 8) * CST + (col % 8) * 4;
            const bool ok = key0 + r < p.N_k;
            const size_t src = (kv_row0 + key0 + r) * D + col * 4;
            *reinterpret_cast<f32x4*>(&k_lds[dst]) =
                ok ? *reinterpret_cast<const f32x4*>(p.k + src) : f32x4{0.f, 0.f, 0.f, 0.f};
            *reinterpret_cast<f32x4*>(&v_lds[dst]) =
                ok ? *reinterpret_cast<const f32x4*>(p.v + src) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        __syncthreads();

        float s[BK];
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            const float* kr = &k_lds[j * ROW + sub * CST];
            float acc = 0.f;
#pragma unroll
            for (int t = 0; t < 32; ++t) acc = __builtin_fmaf(q[t], kr[t], acc);
#pragma unroll
            for (int x = 1; x < SPLIT; x <<= 1) acc += __shfl_xor(acc, x);
            const int key = key0 + j;
            const bool vis = key < p.N_k && (!CAUSAL || key <= qi + off);
            s[j] = vis ? acc : kNegInf;
            mx = fmaxf(mx, s[j]);
        }
        const float mx2 = (mx == kNegInf) ? kNegInf : mx * p.c;
        const float m_new = fmaxf(m_run, mx2);
        const float base = (m_new == kNegInf) ? 0.f : m_new;
        const float alpha = exp2f(m_run - base);
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            const float e = (s[j] == kNegInf) ? 0.f : exp2f(__builtin_fmaf(s[j], p.c, -base));
            s[j] = e;
            lsum += e;
        }
        l_run = alpha * l_run + lsum;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < 32; ++t) o[t] *= alpha;
#pragma unroll
        for (int j = 0; j < BK; ++j) {
            const float* vr = &v_lds[j * ROW + sub * CST];
#pragma unroll
            for (int t = 0; t < 32; ++t) o[t] = __builtin_fmaf(s[j], vr[t], o[t]);
        }
    }

    if (qi < p.N_q) {
        const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
        f32x4* dst = reinterpret_cast<f32x4*>(p.o + (q_row0 + qi) * D + sub * 32);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dst[i] = f32x4{o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv};
        if (p.lse && sub == 0)
            p.lse[q_row0 + qi] = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream)
{
    constexpr int BM = 256 / (D / 32);
    static_assert(BM == fwd_f32_rows(D), "the host checks workgroup counts with this block size");
    Params p;
    p.q = static_cast<const float*>(a.q);
    p.k = static_cast<const float*>(a.k);
    p.v = static_cast<const float*>(a.v);
    p.o = static_cast<float*>(a.o);
    p.lse = a.lse;
    p.B = a.B;
    p.H = a.H;
    p.H_kv = a.H_kv;
    p.N_q = a.N_q;
    p.N_k = a.N_k;
    p.rep = a.H / a.H_kv;
    p.nqb = (a.N_q + BM - 1) / BM;
    p.c = a.scale * kLog2e;
    const long long blocks = (long long)p.nqb * a.H * a.B;   // at most 2^31 - 1: checked on the host
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream)
{
    if (a.d == 128) return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
    if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace fa
