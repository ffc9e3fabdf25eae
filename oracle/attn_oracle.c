/*
 * attn_oracle.c -- plain, slow, fp64 CPU oracle for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library; the two meet only through the seeded input generators.
 *
 * What it computes is the plain three-step definition of attention, one
 * query row at a time, in double precision:
 *
 *   s_j  = scale * <q, k_j>                      for every key j of the row
 *   mask: a key j is visible to query row i unless causal and j > i + (N_k - N_q),
 *         or, with a sliding window of W keys, j < i + (N_k - N_q) - W + 1
 *   p_j  = exp(s_j - m) / sum_visible exp(s_t - m),   m = max_visible s_t
 *          (masked keys get p_j = 0, exactly as a -inf fill would give)
 *   o    = sum_j p_j v_j
 *   lse  = m + ln(sum_visible exp(s_t - m))
 *
 * Sources (the web pages this repository follows):
 *  - "Attention variants: GQA/MQA/FlashAttention" (youngju.dev), §3: the
 *    standard attention is S = Q K^T, P = softmax(S), O = P V, and the tiled
 *    method reaches the very same numbers; §2 gqa_attention snippet: scores
 *    divided by sqrt(d_k), key/value head shared by rep = H/G consecutive query
 *    heads (repeat_interleave on the head axis); §5.5: causal structure; §4:
 *    sliding-window attention, where each token looks only at the W most
 *    recent tokens (itself included: with W = 3, query 5 sees keys 3, 4, 5).
 *  - "Attention mechanism evolution: MHA -> MLA, Flash Attention" (toolsku.com),
 *    MHA and GQA module code: scale = head_dim^-0.5 applied to QK^T, masked
 *    entries filled with -inf before the softmax, _repeat_kv expands each KV
 *    head over n_rep contiguous query heads.
 *  - "Flash Attention: principles and practice" (holysheep.ai), the
 *    conventional three-step computation.
 *
 * Readings where the pages are silent:
 *  - causal alignment when N_q != N_k is bottom-right: query row i sees keys
 *    j <= i + (N_k - N_q); with N_q == N_k this is j <= i;
 *  - a row with no visible key returns o = 0 and lse = -inf;
 *  - a sliding window is causal: row i sees the W keys ending at its last
 *    causally visible key i + (N_k - N_q); in a decode step the query sees the
 *    last W cached rows;
 *  - lse is natural-log, in units of the scaled scores;
 *  - query head h reads key/value head g = h / (H / H_kv).
 *
 * Inputs are read in the precision they are stored in (fp32, bf16 bit
 * patterns, or fp64) and widened exactly to double; all arithmetic is double.
 *
 * Parity pins: every function here is pinned by the CPU tests (closed forms,
 * special cases, library cross-checks, invariants); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1, ORACLE_F64 = 2 };

/* Exact widening of one stored element to double. */
static double load(const void* base, int dtype, size_t idx)
{
    if (dtype == ORACLE_F64) return ((const double*)base)[idx];
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    /* bf16: the 16 stored bits are the high half of an fp32 pattern */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * One query row against n_keys keys of one KV head.
 *   q_off       element offset of the query row (d contiguous elements)
 *   kv_off      element offset of key/value row 0 of the head (rows of d)
 *   n_keys      number of key rows in the head
 *   first       keys first .. n_visible-1 are visible (causal mask and
 *   n_visible   sliding window); the rest are masked
 *   s           scratch of n_keys doubles (the materialised score row)
 *   o_row       d doubles out;  *lse_out one double out
 */
static void attend_row(const void* q, const void* k, const void* v, int dtype,
                       size_t q_off, size_t kv_off, long n_keys, long first,
                       long n_visible, long d, double scale, double* s,
                       double* o_row, double* lse_out)
{
    long j, t;
    if (n_visible > n_keys) n_visible = n_keys;
    if (first < 0) first = 0;
    for (t = 0; t < d; ++t) o_row[t] = 0.0;
    if (n_visible <= first) {       /* every key masked: empty softmax */
        *lse_out = -INFINITY;
        return;
    }
    /* step 1: scores S = scale * q k^T for the visible keys */
    for (j = first; j < n_visible; ++j) {
        double acc = 0.0;
        for (t = 0; t < d; ++t)
            acc += load(q, dtype, q_off + (size_t)t) *
                   load(k, dtype, kv_off + (size_t)j * (size_t)d + (size_t)t);
        s[j] = scale * acc;
    }
    /* step 2: softmax over the visible keys (masked keys contribute 0) */
    double m = s[first];
    for (j = first + 1; j < n_visible; ++j)
        if (s[j] > m) m = s[j];
    double z = 0.0;
    for (j = first; j < n_visible; ++j) {
        s[j] = exp(s[j] - m);
        z += s[j];
    }
    for (j = first; j < n_visible; ++j) s[j] /= z;
    /* step 3: O = P V */
    for (j = first; j < n_visible; ++j) {
        double p = s[j];
        size_t row = kv_off + (size_t)j * (size_t)d;
        for (t = 0; t < d; ++t) o_row[t] += p * load(v, dtype, row + (size_t)t);
    }
    *lse_out = m + log(z);
}

/* Keys visible to query row i: j <= i + (n_k - n_q) when causal, all otherwise. */
static long visible_keys(long i, long n_q, long n_k, int causal)
{
    if (!causal) return n_k;
    long last = i + (n_k - n_q);    /* last visible key index */
    if (last < 0) return 0;
    return last + 1 < n_k ? last + 1 : n_k;
}

/* First visible key of row i: with a sliding window of w keys (w > 0) the
 * window ends at the row's last causally visible key, i + (n_k - n_q). */
static long first_key(long i, long n_q, long n_k, long w)
{
    if (w <= 0) return 0;
    long f = i + (n_k - n_q) - w + 1;
    return f > 0 ? f : 0;
}

static int check_shape(long B, long H, long H_kv, long N_q, long N_k, long d)
{
    if (B <= 0 || H <= 0 || H_kv <= 0 || N_q <= 0 || N_k <= 0 || d <= 0) return 1;
    if (H % H_kv != 0) return 1;    /* every KV head serves H/H_kv query heads */
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full attention forward.
 *   q [B,H,N_q,d], k and v [B,H_kv,N_k,d] (row-major, d fastest), dtype as above
 *   o [B,H,N_q,d] fp64 out, lse [B,H,N_q] fp64 out
 * Returns 0 on success, 1 on a bad shape, 2 on allocation failure.
 */
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     double* o, double* lse, long B, long H, long H_kv,
                     long N_q, long N_k, long d, double scale, int causal,
                     long window)
{
    if (check_shape(B, H, H_kv, N_q, N_k, d)) return 1;
    if (window > 0 && !causal) return 1;    /* a sliding window is causal */
    long rep = H / H_kv;
    long n_rows = B * H * N_q;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N_k);
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 16)
            for (r = 0; r < n_rows; ++r) {
                long i = r % N_q;
                long h = (r / N_q) % H;
                long b = r / (N_q * H);
                long g = h / rep;
                size_t q_off = (size_t)r * (size_t)d;
                size_t kv_off = ((size_t)(b * H_kv + g) * (size_t)N_k) * (size_t)d;
                attend_row(q, k, v, dtype, q_off, kv_off, N_k,
                           first_key(i, N_q, N_k, window),
                           visible_keys(i, N_q, N_k, causal), d, scale, s,
                           o + (size_t)r * (size_t)d, lse + r);
            }
            free(s);
        }
    }
    return failed ? 2 : 0;
}

/*
 * Selected query rows only (for spot checks of large problems).
 *   rows[3*n]: (b, h, i) triples;  o_rows [n,d], lse_rows [n] fp64 out.
 * Same arguments and semantics as oracle_attention otherwise; returns 1 when a
 * triple is out of range.
 */
int oracle_attention_rows(const void* q, const void* k, const void* v, int dtype,
                          const long* rows, long n, double* o_rows,
                          double* lse_rows, long B, long H, long H_kv, long N_q,
                          long N_k, long d, double scale, int causal, long window)
{
    if (check_shape(B, H, H_kv, N_q, N_k, d)) return 1;
    if (window > 0 && !causal) return 1;
    for (long r = 0; r < n; ++r) {
        long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= H || i < 0 || i >= N_q) return 1;
    }
    long rep = H / H_kv;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N_k);
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < n; ++r) {
                long b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
                long g = h / rep;
                size_t q_off = ((size_t)(b * H + h) * (size_t)N_q + (size_t)i) * (size_t)d;
                size_t kv_off = ((size_t)(b * H_kv + g) * (size_t)N_k) * (size_t)d;
                attend_row(q, k, v, dtype, q_off, kv_off, N_k,
                           first_key(i, N_q, N_k, window),
                           visible_keys(i, N_q, N_k, causal), d, scale, s,
                           o_rows + (size_t)r * (size_t)d, lse_rows + r);
            }
            free(s);
        }
    }
    return failed ? 2 : 0;
}

/*
 * One decode step against a KV cache: each sequence b has one new query per
 * head and attends, without a mask, to the first seq_lens[b] cached rows
 * (the cache of "Attention mechanism evolution" grows by concatenation on the
 * sequence axis, and decoding re-reads all of it: "Attention variants" §7).
 *   q [B,H,d];  k_cache, v_cache [B,H_kv,N_max,d];  seq_lens [B] (host)
 *   o [B,H,d] fp64 out;  lse [B,H] fp64 out
 * Rows at or beyond seq_lens[b] are never read.  With a sliding window of
 * w > 0 keys the query sees only the last w cached rows ("Attention variants"
 * §4).  Returns 1 on a bad shape or a length outside 1..N_max.
 */
int oracle_decode(const void* q, const void* k_cache, const void* v_cache,
                  int dtype, const int* seq_lens, double* o, double* lse,
                  long B, long H, long H_kv, long N_max, long d, double scale,
                  long window)
{
    if (check_shape(B, H, H_kv, 1, N_max, d)) return 1;
    for (long b = 0; b < B; ++b)
        if (seq_lens[b] < 1 || seq_lens[b] > N_max) return 1;
    long rep = H / H_kv;
    int failed = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)N_max);
        if (!s) {
#pragma omp atomic write
            failed = 1;
        } else {
            long r;
#pragma omp for schedule(dynamic, 1)
            for (r = 0; r < B * H; ++r) {
                long b = r / H, h = r % H, g = h / rep;
                size_t kv_off = ((size_t)(b * H_kv + g) * (size_t)N_max) * (size_t)d;
                long len = seq_lens[b];
                long first = window > 0 && len > window ? len - window : 0;
                attend_row(q, k_cache, v_cache, dtype, (size_t)r * (size_t)d,
                           kv_off, len, first, len, d, scale, s,
                           o + (size_t)r * (size_t)d, lse + r);
            }
            free(s);
        }
    }
    return failed ? 2 : 0;
}
