/*
 * paged_kv.h -- C ABI of libpagedkv.so: the decode step over a paged BF16 KV
 * cache on an AMD Instinct MI355X (gfx950).
 *
 * Passages this library implements:
 *   [HN-pool]   "Hours of YouTube and 85 handtyped pages of notes on LLM
 *               Inference - Start here" (hackernews.jp translation of the
 *               project README), section "これまでの進捗" (progress so far),
 *               bullet on the shared BF16 KV page pool: one block table per
 *               sequence and layer, each physical page holds K and V of 16
 *               tokens, decode adds one new token at its absolute RoPE
 *               position.
 *   [HN-attn]   same page and section, bullet on paged decode attention with
 *               an FP32 online softmax: every query head streams its own
 *               sequence's cached pages and accumulates weighted V, without
 *               gathering a contiguous prefix and without storing scores.
 *   [HN-batch]  same page and section, bullet on batch decode: runtime-sized
 *               buffers, packed projections, a separate page mapping and
 *               attention length per sequence; the request count does not
 *               grow the pool.
 *   [HN-scope]  same page, section "現在のスコープ" (current scope): model
 *               dimensions and the 2,048-token context are fixed; a request
 *               that cannot fit is refused with a clear error.
 *   [TV-decode] "Tiny-vLLMでゼロから構築する高性能LLM推論エンジン"
 *               (agentlenshq.com), section "Prefill vs. Decode": decode is
 *               bound by memory bandwidth; section "GPUメモリ管理": allocate
 *               big buffers up front and reuse them.
 *
 * Geometry is fixed to the Llama-3.2-1B attention shape the pages use
 * ([HN-scope]): 32 query heads, 8 KV heads (query head h reads KV head h/4),
 * head dimension 64, 16 tokens per page, contexts of at most 2,048 tokens.
 *
 * Conventions for every call:
 *   - BF16 values travel as raw uint16_t bit patterns.
 *   - Pointers marked (device) are device memory of the current HIP device;
 *     (host) pointers are host memory.  All buffers belong to the caller;
 *     no call allocates or frees memory, and the library keeps no state
 *     besides a per-thread copy of the last HIP error text and the fixed
 *     scratch array of paged_kv_append_decode_attn_noalloc.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; calls that share
 *     buffers must be ordered by the caller (same stream, or events).
 *   - Element strides count elements of the buffer's own type.
 *   - Every argument check happens on the host before any HIP call, so a
 *     non-zero status means nothing was enqueued.  Values that live in
 *     device memory (context lengths, table entries) are preconditions the
 *     library does not check; breaking one is undefined behaviour.
 *   - The calls are reentrant and thread-safe.
 */
#ifndef PAGED_KV_H_
#define PAGED_KV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_NUM_Q_HEADS 32
#define PKV_NUM_KV_HEADS 8
#define PKV_HEAD_DIM 64
#define PKV_PAGE_TOKENS 16
#define PKV_MAX_CONTEXT 2048

/* Status codes. */
#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1)   /* null pointer, negative count or stride, range error */
#define PKV_ERR_ALIGNMENT (-2)     /* pointer not 16-byte aligned or stride not a multiple of 16 bytes */
#define PKV_ERR_WORKSPACE (-3)     /* workspace smaller than paged_decode_attn_workspace_size() */
#define PKV_ERR_UNSUPPORTED (-4)   /* reserved for geometries other than the fixed one */
#define PKV_ERR_HIP (-5)           /* a HIP launch failed; text via paged_kv_status_string */

/*
 * The shared page pool ([HN-pool]).  Element (page p, KV head g, slot t,
 * dim d) of K lives at k_pool[p*page_stride + g*head_stride + t*slot_stride + d],
 * and of V at the same offset from v_pool.  Dims of one slot are contiguous.
 * Default layout: page = [K | V][8 heads][16 slots][64 dims] BF16 = 32 KiB,
 * i.e. page_stride 16384, head_stride 1024, slot_stride 64 and
 * v_pool = k_pool + 8192.  k_pool and v_pool: (device), 16-byte aligned;
 * the three strides must be positive multiples of 8 elements, slot_stride at
 * least 64, and the 16 slots of one head must span less than 2^30 elements
 * (15*slot_stride + 64 < 2^30); num_pages must fit in int32.  Pools outside
 * these bounds are refused with INVALID_ARG (ALIGNMENT for the multiples).
 */
typedef struct paged_kv_pool {
    uint16_t* k_pool;
    uint16_t* v_pool;
    int64_t num_pages;
    int64_t page_stride;
    int64_t head_stride;
    int64_t slot_stride;
} paged_kv_pool;

/*
 * RoPE table for the append ([HN-pool]: the new token is rotated at its
 * absolute position).  Fills cos_out/sin_out (host, [max_pos][32] FP32,
 * row-major) with cos and sin of pos * theta^(-2i/64), computed in FP64 and
 * rounded once to FP32.  Llama 3.2 uses theta = 500000.  Upload the table
 * once and pass it to every paged_kv_append call.
 * Errors: INVALID_ARG for null outputs, max_pos < 1 or theta <= 0.
 */
int paged_kv_rope_table(double theta, int32_t max_pos, float* cos_out, float* sin_out);

/*
 * Decode append ([HN-pool], [HN-batch]).  For each sequence s < num_seqs with
 * n = context_lens[s] >= 1 (the length AFTER this append), the new token sits
 * at position pos = n-1:
 *   - the 32 heads of q[s] and the 8 heads of k_new[s] are rotated by the
 *     table row pos (pairs (i, i+32), i < 32: x_i c - x_{i+32} s and
 *     x_{i+32} c + x_i s); each result is the FP64 value of that expression
 *     (both products are exact in FP64) rounded once to BF16, ties to even;
 *     q[s] is overwritten in place;
 *   - rotated K and unchanged V of KV head g go to page
 *     block_table[s*bt_stride + pos/16], slot pos%16.
 * Sequences with n <= 0 are skipped (nothing written).  A sequence whose
 * position pos is outside the table (pos >= max_pos) is skipped too (q not
 * rotated, nothing written); one whose page index pos/16 is at or past
 * bt_stride, or whose table entry is not a page in [0, num_pages), gets q
 * rotated but no K/V write.
 *   pool          (host struct, device arrays) the page pool
 *   block_table   (device) int32 [num_seqs][bt_stride], this layer's tables
 *   context_lens  (device) int32 [num_seqs]
 *   q             (device) BF16 [num_seqs][q_stride], heads at h*64, >= 2048 per row
 *   k_new, v_new  (device) BF16 [num_seqs][k_stride / v_stride], heads at g*64
 *   rope_cos/sin  (device) FP32 [max_pos][32] from paged_kv_rope_table
 * q, k_new and v_new may be slices of one packed QKV buffer.
 * Precondition (unchecked): no two sequences write the same (page, slot).
 * Errors: INVALID_ARG (null pointer, num_seqs < 0, bt_stride < 1, a stride
 * below its row width, max_pos < 1), ALIGNMENT, HIP.  num_seqs == 0: no-op.
 */
int paged_kv_append(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                    const int32_t* context_lens, int32_t num_seqs, uint16_t* q, int64_t q_stride,
                    const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                    int64_t v_stride, const float* rope_cos, const float* rope_sin,
                    int32_t max_pos, void* stream);

/*
 * Prefill page fill ([HN-pool]: the prefill fills the prompt's pages, which
 * decode then extends one token at a time).  Prompt rows are packed: the
 * rows of sequence s are cu_tokens[s] .. cu_tokens[s+1]-1, and its row i is
 * the token at position start_pos[s] + i (start_pos[s] = tokens it already
 * holds, 0 for a fresh prompt; several sequences and chunked prompts share
 * one call).  Each row is handled exactly as paged_kv_append handles a
 * sequence with context length position + 1: its q (if q is not NULL) and k
 * are rotated at its position and rounded once to BF16, q in place, and K'
 * and V go to page block_table[s*bt_stride + position/16], slot position%16.
 * The result equals the appends of the rows one after another, bit for bit.
 * The same guards apply per row: a position outside the RoPE table skips the
 * row, a page index at or past bt_stride or a table entry outside
 * [0, num_pages) skips its K/V write.
 *   start_pos   (device) int32 [num_seqs]
 *   cu_tokens   (device) int32 [num_seqs + 1], non-decreasing, cu_tokens[0] = 0
 *               and cu_tokens[num_seqs] = total_tokens
 *   total_tokens host copy of cu_tokens[num_seqs] (sizes the launch)
 *   q           (device) BF16 [total_tokens][q_stride] or NULL
 *   k_new, v_new (device) BF16 [total_tokens][k_stride / v_stride]
 * Preconditions (unchecked): the offsets are as stated, and no two rows write
 * the same (page, slot).
 * Errors: INVALID_ARG (null pointer other than q, negative counts,
 * total_tokens > 2^30, bt_stride < 1, a stride below its row width,
 * max_pos < 1), ALIGNMENT, HIP.  num_seqs == 0 or total_tokens == 0: no-op.
 */
int paged_kv_prefill(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                     const int32_t* start_pos, const int32_t* cu_tokens, int32_t num_seqs,
                     int32_t total_tokens, uint16_t* q, int64_t q_stride, const uint16_t* k_new,
                     int64_t k_stride, const uint16_t* v_new, int64_t v_stride,
                     const float* rope_cos, const float* rope_sin, int32_t max_pos,
                     void* stream);

/*
 * Whole-page copies: page dst[i] receives all of page src[i] (K and V, every
 * KV head, slot and dim), for i < num_pairs, in one launch.  This is the
 * device half of copy-on-write for pages shared between sequences that
 * start with the same prompt ("【ITニュース解説】From a Rust Inference Engine
 * to Heterogeneous Serving", the paragraph on the prefix cache): the host
 * pager (paged_kv_pager.h) hands out the pairs, and they are copied before
 * the next token is written.  Pairs naming a page outside [0, num_pages) are
 * skipped.
 *   src, dst  (device) int32 [num_pairs]
 * Preconditions (unchecked): no dst is another pair's src or dst.
 * Errors: INVALID_ARG (null pointer, num_pairs < 0), ALIGNMENT, HIP.
 * num_pairs == 0: no-op.
 */
int paged_kv_copy_pages(const paged_kv_pool* pool, const int32_t* src, const int32_t* dst,
                        int32_t num_pairs, void* stream);

/*
 * Split plan of the decode attention.  Each (sequence, KV head) is served by
 * S workgroups of 4 wavefronts.  A sequence whose context fills np pages is
 * cut into 4*S chunks of ceil(np / (4*S)) whole pages, in logical order; each
 * wavefront streams one chunk, the 4 chunks of a workgroup are merged on
 * chip, and when S > 1 the S workgroup partials are merged by the combine
 * phase.  S depends only on (num_seqs, max_context_len) and the chunk
 * boundaries only on each sequence's own length, so results are bitwise
 * reproducible and independent of where pages sit in the pool.  Returns
 * S >= 1, or 0 for arguments outside num_seqs >= 1, 1 <= max_context_len <= 2048.
 */
int32_t paged_decode_attn_num_splits(int32_t num_seqs, int32_t max_context_len);

/*
 * The round length R that paged_decode_attn_order uses on the current
 * device: the sequences whose attention workgroups (one per KV head, single
 * split) the device holds at once.  0 when it cannot be determined (the
 * order is then the plain sorted order).
 */
int32_t paged_decode_attn_order_round(void);

/*
 * The same start order computed on the host, for callers that lay out the
 * batch themselves (a serving host knows its lengths): placing sequence
 * seq_order[p] at batch row p gives the attention calls that order with no
 * seq_order argument, so their workgroups need not look it up.  Pass
 * round_len = paged_decode_attn_order_round() for the current device (0
 * gives the plain sorted order).  Equal, entry for entry, to what
 * paged_decode_attn_order writes for the same lengths on a device whose
 * round length is round_len.
 *   context_lens  (host) int32 [num_seqs]
 *   seq_order     (host) int32 [num_seqs], written
 * Errors: INVALID_ARG (null pointer, num_seqs < 0, round_len < 0,
 * max_context_len outside [1, 2048]).  num_seqs == 0: no-op.  No HIP call.
 */
int paged_decode_attn_order_host(const int32_t* context_lens, int32_t num_seqs,
                                 int32_t max_context_len, int32_t round_len, int32_t* seq_order);

/*
 * Start order of a decode batch whose lengths differ ([HN-batch]: each
 * sequence has its own attention length).  When a launch has more
 * workgroups than the GPU holds at once, they start in rank order, and a
 * long sequence that starts late sets the end of the launch; started
 * longest first, the long ones overlap the short ones.  The sequences are
 * sorted by descending page count ceil(min(context_lens[s],
 * max_context_len) / 16), ties in batch order; sorted rank r (0 = most
 * pages) then starts at position p(r), and seq_order[p(r)] = that sequence.
 * With R = paged_decode_attn_order_round() (the sequences whose workgroups
 * start together), P = R/4 and B = num_seqs >= 4P >= 4:
 *   r < 3P:          p = P + (2P - 1 - r) for P <= r < 2P, else p = r
 *                    (the 3P longest, the middle quarter reversed);
 *   r >= B - P:      p = 3P + (B - 1 - r)  (the P shortest, shortest first);
 *   otherwise:       p = r + P              (the rest, longest first).
 * Else p(r) = r.  The CUs that take the longest sequences in one slot round
 * take shorter ones in the next, and the shortest sequences finish within
 * the first round and hand their slots on.  A permutation of
 * [0, num_seqs), computed on the device by one small launch.  Lengths are
 * the same for every layer of a decode step, so one call per step serves
 * all its layers' attention calls (pass seq_order to them).  The attention
 * follows the order only when its workgroups exceed what the GPU holds at
 * once; the order never changes a result bit.
 *   context_lens  (device) int32 [num_seqs]
 *   seq_order     (device) int32 [num_seqs], written
 * Errors: INVALID_ARG (null pointer, num_seqs < 0, max_context_len outside
 * [1, 2048]), HIP.  num_seqs == 0: no-op.
 */
int paged_decode_attn_order(const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t* seq_order, void* stream);

/*
 * Bytes of device workspace paged_decode_attn needs for this plan: 0 when
 * S == 1, else 2048 + S * num_seqs * 32 * 66 * 4.  The first 2048 bytes are
 * 512 int32 counters, one per (sequence, KV head) for up to 64 sequences
 * (the plan only asks for S > 1 below 64 sequences); then come the partials,
 * per workgroup and query head 64 accumulator values, a maximum and a sum,
 * FP32.  Returns 0 for arguments outside the ranges above.
 */
size_t paged_decode_attn_workspace_size(int32_t num_seqs, int32_t max_context_len);

/*
 * Makes a workspace ready for use: zeroes its counter block (the first
 * min(workspace_bytes, 2048) bytes), asynchronously on `stream`.  Call it
 * once after allocating a workspace (zeroing the whole allocation instead
 * does the same); paged_decode_attn and paged_kv_append_decode_attn leave
 * the counters zero again when they finish, so a workspace serves any
 * number of calls, of any num_seqs and max_context_len, without it.  A
 * workspace whose counters are not zero makes those calls produce wrong
 * output rows (they never wait, so nothing hangs).  The counter block is a
 * plain fill; it is not meant for a captured graph (make the workspace
 * ready before capture).
 *   workspace  (device) 16-byte aligned, or NULL when workspace_bytes is 0
 * Errors: INVALID_ARG (NULL with workspace_bytes > 0), ALIGNMENT, HIP.
 */
int paged_decode_attn_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged decode attention ([HN-attn], [HN-batch], [TV-decode]).  For each
 * sequence s, query head h and n = context_lens[s]:
 *   out[s][h*64 + d] = sum_{t<n} softmax_t(scale * q[s][h].K[t][h/4]) V[t][h/4][d]
 * over the logical token order t, where token t is read from page
 * block_table[s*bt_stride + t/16], slot t%16.  FP32 online softmax over BF16
 * inputs; the context is cut into chunks (paged_decode_attn_num_splits)
 * whose partial results are merged with the log-sum-exp rule.  One launch:
 * when S > 1, the last of a (sequence, KV head)'s S workgroups to finish
 * merges their partials into the output (the combine phase's arithmetic,
 * in the same order, so the result equals split + combine bit for bit),
 * counting finished workgroups in the workspace's counters.  Rows with
 * n <= 0 are written as zeros; a length above max_context_len is clamped to
 * it.  K/V of tokens at or past n, and pages that no table entry below
 * ceil(n/16) names, are never read.  Each row's first min(bt_stride, 128)
 * table entries are loaded together when the row's work starts, whatever n
 * is (so the table must be readable as [num_seqs][bt_stride]); entries at or
 * past ceil(n/16) may hold any value, which is never used.  A table entry
 * below ceil(n/16) that is not a page in [0, num_pages) is not dereferenced;
 * that sequence's rows come out NaN.
 *   seq_order        (device) int32 [num_seqs] from paged_decode_attn_order, or
 *                    NULL: the order in which sequences are started (see there).
 *                    It changes no result bit; an entry outside [0, num_seqs)
 *                    counts as its own rank.
 *   max_context_len  host-known upper bound of every context_lens[s] (drives the plan)
 *   q                (device) BF16 [num_seqs][q_stride], already rotated
 *   out              (device) FP32 [num_seqs][out_stride], >= 2048 per row
 *   workspace        (device) >= paged_decode_attn_workspace_size() bytes,
 *                    16-byte aligned, made ready once with
 *                    paged_decode_attn_workspace_init (counters zero); may
 *                    be NULL when that size is 0.  Calls running
 *                    concurrently need separate workspaces.
 * Errors: INVALID_ARG (null pointer, num_seqs < 0, max_context_len outside
 * [1, min(2048, 16*bt_stride)], non-finite scale, a stride below its row
 * width), ALIGNMENT (out_stride must be a multiple of 4), WORKSPACE, HIP.
 * num_seqs == 0: no-op.
 */
int paged_decode_attn(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                      const int32_t* context_lens, const int32_t* seq_order, int32_t num_seqs,
                      int32_t max_context_len,
                      const uint16_t* q, int64_t q_stride, float scale, float* out,
                      int64_t out_stride, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two phases of paged_decode_attn as separate calls, for callers that
 * time or schedule them apart.  Enqueuing paged_decode_attn_split then
 * paged_decode_attn_combine on one stream with the same arguments gives
 * exactly paged_decode_attn's output bits.  The split phase streams the
 * pages and writes one partial (maximum, sum, accumulator) per workgroup
 * into the workspace -- or, when S == 1, the final rows into out; it does
 * not use the counters.  The combine phase merges the partials into out in
 * a launch of its own; when S == 1 it enqueues nothing.  The split phase
 * takes the arguments, checks and errors of paged_decode_attn; the combine
 * phase checks its own arguments the same way (INVALID_ARG, ALIGNMENT,
 * WORKSPACE).
 */
int paged_decode_attn_split(const paged_kv_pool* pool, const int32_t* block_table,
                            int64_t bt_stride, const int32_t* context_lens,
                            const int32_t* seq_order, int32_t num_seqs,
                            int32_t max_context_len, const uint16_t* q, int64_t q_stride,
                            float scale, float* out, int64_t out_stride, void* workspace,
                            size_t workspace_bytes, void* stream);
int paged_decode_attn_combine(const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, float* out, int64_t out_stride,
                              const void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused decode step of one layer: the append and the attention in one
 * launch ([HN-pool], [HN-attn], [HN-batch]; [TV-decode]: the step is bound
 * by memory bandwidth, and the append's own launch, with its start-up and
 * drain, is a visible share of it).  Same result, bit for bit in out (NaN
 * rows aside: NaN in both, payload unspecified) and in the pool, as
 *     paged_kv_append(pool, block_table, bt_stride, context_lens, num_seqs,
 *                     q, q_stride, k_new, k_stride, v_new, v_stride,
 *                     rope_cos, rope_sin, max_pos, stream);
 *     paged_decode_attn(pool, block_table, bt_stride, context_lens, seq_order,
 *                       num_seqs, max_context_len, q, q_stride, scale, out,
 *                       out_stride, workspace, workspace_bytes, stream);
 * except that q is only read: the rotated q is used but not written back.
 * A new token past max_context_len is still written to its page and, as in
 * the two calls, not attended.  Arguments, preconditions and errors are
 * those of the two calls together (the attention's checks come first).
 * num_seqs == 0: no-op.
 */
int paged_kv_append_decode_attn(const paged_kv_pool* pool, const int32_t* block_table,
                                int64_t bt_stride, const int32_t* context_lens,
                                const int32_t* seq_order, int32_t num_seqs,
                                int32_t max_context_len, const uint16_t* q, int64_t q_stride,
                                const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                                int64_t v_stride, const float* rope_cos, const float* rope_sin,
                                int32_t max_pos, float scale, float* out, int64_t out_stride,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_kv_append_decode_attn without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It allocates nothing: when the
 * plan needs partials (S > 1, which the plan only asks for below 64
 * sequences), they and the merge counters live in a fixed device array of
 * the library, 2,048 + 8 * 63 * 32 * 66 * 4 = 4,259,840 bytes, which holds
 * the largest such plan.  Each GPU the library runs on holds its own copy
 * until the process ends.  The first call on a device looks the array's
 * address up and clears its counters with a small kernel on `stream`; every
 * call leaves the counters zero again.  All calls on one GPU share that
 * array: calls that overlap in time on one GPU (different streams, or
 * threads) race and give wrong output rows; order them.  Arguments, results
 * (bit for bit), preconditions and errors are those of
 * paged_kv_append_decode_attn; WORKSPACE is returned only for a plan larger
 * than the array, which valid arguments never produce.
 */
int paged_kv_append_decode_attn_noalloc(const paged_kv_pool* pool, const int32_t* block_table,
                                        int64_t bt_stride, const int32_t* context_lens,
                                        const int32_t* seq_order, int32_t num_seqs,
                                        int32_t max_context_len,
                                        const uint16_t* q, int64_t q_stride,
                                        const uint16_t* k_new, int64_t k_stride,
                                        const uint16_t* v_new, int64_t v_stride,
                                        const float* rope_cos, const float* rope_sin,
                                        int32_t max_pos, float scale, float* out,
                                        int64_t out_stride, void* stream);

/* Text for a status code; for PKV_ERR_HIP it includes the last HIP error
 * text seen by this thread.  The pointer stays valid until the next call
 * from the same thread. */
const char* paged_kv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H_ */
