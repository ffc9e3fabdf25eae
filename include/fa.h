/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The library computes attention forward, O = softmax(scale * Q K^T + mask) V,
 * and the per-row log-sum-exp, without ever storing the N_q x N_k score
 * matrix: keys and values are streamed through on-chip memory in tiles and the
 * softmax is carried as a running maximum and running sum per query row.  It
 * also runs one decode step (one new query per head) against a KV cache, with
 * the keys of each sequence split into chunks whose partial results are merged
 * by their log-sum-exp.
 *
 * Sources, by web page title and section:
 *  [AV] "Attention variants: GQA/MQA/FlashAttention" (youngju.dev)
 *       §1 cost model (B, H, N, d_k; the (B,H,N,N) score tensor),
 *       §2 MQA/GQA and the gqa_attention snippet (q [B,H,N,d_k], k/v [B,G,N,d_k],
 *          rep = H/G, repeat_interleave on the head axis, scores / sqrt(d_k)),
 *       §3 FlashAttention tiling and online softmax (exact, not approximate),
 *       §4 sliding-window attention (each token sees the W most recent tokens),
 *       §5 serving memory: paged KV cache (fixed-size blocks managed like
 *          virtual-memory pages), KV quantisation,
 *       §5.5 causal block skip, §7 decode is memory-bandwidth bound,
 *       troubleshooting list: H must be a multiple of G.
 *  [ME] "Attention mechanism evolution: MHA -> MLA, Flash Attention" (toolsku.com)
 *       MHA/GQA module code (head_dim^-0.5 scale, -inf mask fill, KV cache
 *       concatenated on the sequence axis, _repeat_kv over contiguous heads),
 *       Flash Attention usage box (flash_attn_func(q, k, v, causal,
 *       softmax_scale=None) with None meaning 1/sqrt(d)).
 *
 * Conventions shared by every entry point
 *  - Layout: row-major, head dimension fastest.  q [B,H,N_q,d];
 *    k, v [B,H_kv,N_k,d]; o [B,H,N_q,d]; lse [B,H,N_q] (fp32).  Decode:
 *    q [B,H,d]; k_cache, v_cache [B,H_kv,N_max,d]; o [B,H,d]; lse [B,H].
 *  - Head sharing [AV §2, ME GQA code]: query head h reads key/value head
 *    g = h / (H / H_kv).  H_kv == H is MHA, H_kv == 1 is MQA.  H must be a
 *    multiple of H_kv.
 *  - Causal mask (causal != 0) [AV §5.5, ME MHA code]: query row i sees key j
 *    iff j <= i + (N_k - N_q) (aligned to the bottom-right corner, so a block
 *    of new queries after a cache sees the whole cache; with N_q == N_k this is
 *    j <= i).  A row that sees no key gets o = 0 and lse = -inf.
 *  - lse = ln(sum_visible exp(s_ij)) with s_ij = scale * <q_i, k_j>: natural
 *    log, in units of the scaled scores.
 *  - scale must be finite and >= 0 (the pages use 1/sqrt(d)); a negative scale
 *    returns FA_ERR_UNSUPPORTED.
 *  - Supported head dimensions: d = 64 and d = 128 (others: FA_ERR_UNSUPPORTED).
 *  - Pointers are device pointers (HIP), 16-byte aligned (lse: 4-byte aligned),
 *    owned by the caller; the library never allocates, frees or keeps them.
 *    Inputs and outputs must not overlap.
 *  - Calls are asynchronous: they validate on the host, enqueue kernels on
 *    `stream` and return.  No host synchronisation; results are visible after
 *    the stream is synchronised.  Calls on different streams may run at once.
 *  - Errors: invalid arguments are rejected on the host before any launch
 *    (FA_ERR_INVALID_ARGUMENT / FA_ERR_UNSUPPORTED) and nothing is written.
 *    A failed launch returns FA_ERR_HIP.  fa_last_error() gives a message for
 *    the calling thread's last failure.  Nothing throws across the ABI.
 *  - Sizes: each tensor may hold up to 2^40 elements; the kernels address
 *    memory with 64-bit offsets, so a tensor may span more than 4 GiB.  The
 *    launch grids bound a few counts further.  Each limit is checked on the
 *    host and returns FA_ERR_UNSUPPORTED before any launch:
 *      fa_fwd, fa_fwd_window:  B * H * ceil(N_q / 256) <= 2^31 - 1;
 *      fa_fwd_f32:             B * H * ceil(N_q / 64)  <= 2^31 - 1 at d = 128,
 *                              B * H * ceil(N_q / 128) <= 2^31 - 1 at d = 64;
 *      decode entry points:    B <= 65535, H_kv * ceil((H / H_kv) / 16) <= 65535,
 *                              B * H <= 2^31 - 4,
 *                              num_splits * B * H_kv * ceil((H / H_kv) / 16) <= 2^31 - 1.
 *  - Thread safety: calls may come from any thread and keep no setting
 *    between calls.  The only process-wide state is the per-thread error
 *    message and per-device caches of how many prefill and decode workgroups
 *    fit on the device (filled once, the same value by every thread).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARGUMENT = 1,
    FA_ERR_UNSUPPORTED = 2,
    FA_ERR_HIP = 3
} fa_status_t;

/*
 * fa_fwd -- attention forward, bf16 in / bf16 out, fp32 accumulation.
 * [AV §3 tiling + online softmax; AV §2 / ME GQA head sharing; AV §5.5 causal]
 *   q      [B,H,N_q,d]   bf16, device
 *   k, v   [B,H_kv,N_k,d] bf16, device
 *   o      [B,H,N_q,d]   bf16, device, written (rounded to nearest even)
 *   lse    [B,H,N_q]     fp32, device, written; may be NULL (not written)
 *   B, H, H_kv, N_q, N_k >= 1; H % H_kv == 0; d in {64, 128}
 *   scale  softmax scale applied to q.k (e.g. 1/sqrt(d)); finite, >= 0
 *   causal 0 = no mask, non-zero = bottom-right causal mask
 *   stream HIP stream to enqueue on (0 = the null stream)
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int H_kv, int N_q, int N_k, int d,
                   float scale, int causal, hipStream_t stream);

/*
 * fa_fwd_window -- fa_fwd with a sliding-window causal mask [AV §4: each token
 * looks only at the W most recent tokens, itself included].  Query row i sees
 * key j iff  i + (N_k - N_q) - window + 1 <= j <= i + (N_k - N_q): the window
 * ends at the row's last causally visible key.  Key tiles wholly outside every
 * row's window are neither loaded nor computed, so the cost grows with
 * N_q * window rather than N_q * N_k.
 *   window >= 1 (keys); a window of at least N_k + max(0, N_q - N_k) equals
 *          fa_fwd with causal = 1.  window < 1: FA_ERR_INVALID_ARGUMENT.
 *   Other arguments, layouts and errors as fa_fwd (the mask is always causal).
 */
fa_status_t fa_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int H_kv, int N_q, int N_k, int d,
                          float scale, int window, hipStream_t stream);

/*
 * fa_fwd_f32 -- the same operation as fa_fwd with fp32 inputs and fp32
 * output, fp32 arithmetic throughout [AV §3: tiles of Q, K and V with a
 * running max and running sum per row give exactly the standard attention;
 * AV §2 head sharing; AV §5.5 causal].  The path exists for precision, not
 * speed: scores, exponentials and the output accumulate in fp32 from the
 * stored fp32 values.
 *   q      [B,H,N_q,d]    fp32, device
 *   k, v   [B,H_kv,N_k,d] fp32, device
 *   o      [B,H,N_q,d]    fp32, device, written
 *   lse    [B,H,N_q]      fp32, device, written; may be NULL
 * Other arguments, limits and errors as fa_fwd.
 */
fa_status_t fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                       int B, int H, int H_kv, int N_q, int N_k, int d,
                       float scale, int causal, hipStream_t stream);

/*
 * fa_decode_workspace_bytes -- size of the workspace fa_decode needs: 256
 * bytes holding the split kernel's chunk queue (an 8-byte word at the front),
 * fp32 partial outputs [B,H,num_splits,d], then fp32 partial log-sum-exps
 * [B,H,num_splits] (256-byte aligned).  Returns 0 for invalid arguments.
 */
size_t fa_decode_workspace_bytes(int B, int H, int d, int num_splits);

/*
 * fa_decode -- one decode step: each sequence b has one new query per head,
 * attending without a mask to the first seq_lens[b] rows of its cache
 * [ME KV-cache code: the cache grows along the sequence axis; AV §7 decode
 * re-reads the cache].  The keys of sequence b are cut into num_splits chunks
 * of ceil(seq_lens[b] / num_splits) rows; one kernel computes each chunk's
 * partial output and log-sum-exp, a second merges them:
 *   M = max_c lse_c;  lse = M + ln sum_c exp(lse_c - M);
 *   o = sum_c exp(lse_c - lse) o_c.
 * (The merge is not on the pages; it is the online-softmax rescale of AV §3
 * applied to whole-chunk summaries.)  Empty chunks contribute nothing.  With
 * num_splits = 1 the single chunk is the answer: the first kernel writes o
 * and lse itself (the same values the merge would give) and the workspace is
 * not touched.
 *   q         [B,H,d]          bf16, device
 *   k_cache   [B,H_kv,N_max,d] bf16, device; rows >= seq_lens[b] are never read
 *   v_cache   [B,H_kv,N_max,d] bf16, device; same
 *   seq_lens  [B] int32, device; each value should lie in 0..N_max.  The
 *             library does not read device memory on the host, so it cannot
 *             report a bad value; the kernels clamp each one into 0..N_max,
 *             so the cache is never read outside its rows.  A length of 0
 *             gives o = 0 and lse = -inf for that sequence.
 *   o         [B,H,d] bf16, device, written
 *   lse       [B,H]   fp32, device, written; may be NULL
 *   B, H, H_kv, N_max >= 1; H % H_kv == 0; d in {64, 128}
 *   scale     finite, >= 0
 *   num_splits 1 .. 256
 *   workspace device buffer of at least fa_decode_workspace_bytes(B,H,d,num_splits)
 *             bytes, 16-byte aligned, owned by the caller; its contents on
 *             entry are ignored and on return are unspecified, with one
 *             exception: when num_splits > 1 and the chunks outnumber the
 *             split workgroups that fit on the device, those workgroups take
 *             chunks from a queue word at the front (a tag and a count).  The
 *             merge kernel leaves it holding the tag and a zero count, and a
 *             call that finds any other value starts the queue afresh; only
 *             the tag with a nonzero count, which a call stopped between its
 *             two kernels leaves, would be taken for a queue in progress
 *   stream    HIP stream; both kernels are enqueued on it, in order
 */
fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache,
                      const int* seq_lens, void* o, float* lse,
                      int B, int H, int H_kv, int N_max, int d, float scale,
                      int num_splits, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * fa_decode_noalloc -- fa_decode without a caller workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It allocates nothing and calls no
 * allocating routine.  The split partials go to a scratch array inside the
 * library instead: 16 MiB (16777216 bytes) per GPU, one array per GPU the
 * library runs on, held until the process ends.  Its address on a device is
 * looked up on the first call with that device current.
 *   The call needs fa_decode_workspace_bytes(B, H, d, num_splits) <= 16 MiB
 *   (at d = 128 and 16 splits: B * H <= 2032); larger calls return
 *   FA_ERR_UNSUPPORTED before any launch.
 *   Every call on one GPU shares that GPU's array, and the array keeps the
 *   last call's contents.  Each call writes every partial it reads before
 *   reading it and leaves the chunk queue word ready for the next (the
 *   array starts zeroed, which the first call takes for a fresh queue), so
 *   nothing needs clearing between calls.  Calls that overlap
 *   on one GPU (on different streams, or from several threads) race on the
 *   array: serialise them, or use fa_decode with a workspace per stream.
 *   Other arguments, results and errors as fa_decode.
 */
fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int* seq_lens, void* o, float* lse,
                              int B, int H, int H_kv, int N_max, int d, float scale,
                              int num_splits, hipStream_t stream);

/*
 * fa_decode_window -- fa_decode where the query sees only the last `window`
 * cached rows of its sequence, keys [max(0, seq_lens[b] - window),
 * seq_lens[b]) [AV §4 sliding window; for the newest token the window ends
 * at the cache's last row].  Those keys are cut into num_splits chunks as in
 * fa_decode; nothing before them is read.
 *   window >= 1; window < 1: FA_ERR_INVALID_ARGUMENT.  Other arguments,
 *   workspace and errors as fa_decode (same workspace size).
 */
fa_status_t fa_decode_window(const void* q, const void* k_cache, const void* v_cache,
                             const int* seq_lens, void* o, float* lse,
                             int B, int H, int H_kv, int N_max, int d, float scale,
                             int window, int num_splits, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * fa_decode_paged -- fa_decode on a paged KV cache [AV §5: the cache is cut
 * into fixed-size blocks managed like virtual-memory pages, so sequences need
 * no contiguous allocation].  Row r of sequence b, KV head g lives at
 *   k_pages[block_table[b * max_blocks + r / page_size], g, r % page_size, :]
 * and likewise in v_pages.  Results equal fa_decode on the gathered cache up
 * to rounding order.
 *   k_pages, v_pages [num_pages, H_kv, page_size, d] bf16, device (the pools)
 *   block_table [B, max_blocks] int32, device: physical page of each logical
 *               block; entries are trusted device data -- the kernel clamps
 *               each one into 0..num_pages-1, so a bad entry can never read
 *               outside the pools; only blocks holding rows < seq_lens[b] are read
 *   seq_lens    [B] int32, device; clamped into 0..max_blocks*page_size
 *   page_size   rows per page, a multiple of 16 (others: FA_ERR_UNSUPPORTED)
 *   max_blocks, num_pages >= 1
 *   The keys of each sequence are cut into num_splits chunks of
 *   16 * ceil(ceil(seq_lens[b] / num_splits) / 16) rows (chunk edges on
 *   16-row boundaries, so a tile never crosses a page).
 *   Other arguments, workspace (same size as fa_decode) and errors as fa_decode.
 */
fa_status_t fa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int* block_table, int max_blocks, const int* seq_lens,
                            void* o, float* lse, int B, int H, int H_kv, int num_pages, int page_size,
                            int d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * fa_decode_fp8 -- fa_decode on a KV cache stored in FP8 [AV §5 KV
 * quantisation: the cache held in FP8 halves the bytes a memory-bound decode
 * step reads].  The pages name no FP8 variant or scaling; this library takes
 * OCP FP8 E4M3 (4 exponent bits, bias 7, 3 mantissa bits, no infinities, NaN
 * = S.1111.111) -- the variant gfx950 converts in hardware -- with one scale per
 * tensor: key row j is k_scale * e4m3(k_cache[..., j, :]) and value row j is
 * v_scale * e4m3(v_cache[..., j, :]).  Scores and outputs are computed as in
 * fa_decode on those dequantised values (the FP8 values convert to bf16
 * exactly; k_scale folds into the softmax scale and v_scale into the output).
 *   k_cache, v_cache [B,H_kv,N_max,d] uint8 (E4M3 codes), device, 16-byte aligned
 *   k_scale, v_scale finite, > 0 (else FA_ERR_INVALID_ARGUMENT)
 *   q bf16, o bf16, lse fp32, seq_lens, num_splits, workspace: as fa_decode.
 */
fa_status_t fa_decode_fp8(const void* q, const void* k_cache, const void* v_cache, float k_scale, float v_scale,
                          const int* seq_lens, void* o, float* lse, int B, int H, int H_kv, int N_max, int d,
                          float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Static text for a status code. */
const char* fa_status_string(fa_status_t s);

/* Message describing the calling thread's last failed call ("" if none). */
const char* fa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
