/*
 * paged_kv_pager.h -- host-side page management for the paged KV cache of
 * libpagedkv.so: a FIFO free list of physical pages, the lazy page step of a
 * decode batch, and a request pager with admission credits and prefix
 * sharing.  Host memory only; no HIP call is made by any function here.
 *
 * Passages this implements (see paged_kv.h for the full citations):
 *   [HN-scope]  "Hours of YouTube and 85 handtyped pages of notes on LLM
 *               Inference - Start here", section "現在のスコープ":
 *               - admission reserves room for the largest prefix a request can
 *                 process, prompt + allowed new tokens - 1, rounded up to
 *                 16-token pages, for every layer; the allowed output budget is
 *                 clamped to the context limit and the last predicted token is
 *                 never processed;
 *               - these admission credits are separate from physical pages,
 *                 which are allocated lazily; finishing early frees both;
 *               - requests wait in FIFO order while their budget does not fit
 *                 beside the active ones; a budget above the whole pool is
 *                 refused with a clear error; nothing is preempted;
 *               - the statistics: pool size, peak active requests, largest
 *                 decode batch, peak allocated pages, admission wait time,
 *                 final free pages.
 *   [HN-batch]  same page, section "これまでの進捗", the static and continuous
 *               schedulers that admit queued prompts by the page budget and
 *               return pages and budget on completion.
 *   [RS-prefix] "【ITニュース解説】From a Rust Inference Engine to
 *               Heterogeneous Serving" (engr-sng.com), the paragraph on the
 *               prefix cache: a shared prompt prefix skips work but makes it
 *               harder to know when a page may be reused or freed.
 *
 * Conventions: handles are opaque and owned by the caller (create/destroy);
 * every call on one handle is serialised by a lock inside it, so handles may
 * be shared between threads.  Status codes are those of paged_kv.h plus the
 * ones below; paged_kv_status_string() gives their text.
 */
#ifndef PAGED_KV_PAGER_H_
#define PAGED_KV_PAGER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_ERR_EXHAUSTED (-6)     /* no free page left */
#define PKV_ERR_REJECTED (-7)      /* the request's budget exceeds the whole pool */
#define PKV_ERR_BUDGET (-8)        /* a length beyond the request's admitted budget */
#define PKV_ERR_STATE (-9)         /* unknown request, or a request in the wrong state */

/* ------------------------------------------------------------ free list -- */

typedef struct paged_kv_free_list paged_kv_free_list;

/*
 * A FIFO free list over a pool of pool_pages page ids ([HN-scope]: physical
 * pages are handed out lazily and returned on completion).  pages (host,
 * num_free ids in [0, pool_pages), distinct) are the free pages in the order
 * they will be handed out; the other ids count as allocated.
 * Errors: INVALID_ARG (null out, pool_pages < 1 or > 2^31 - 1, num_free
 * outside [0, pool_pages], an id out of range or repeated).
 */
int paged_kv_free_list_create(const int32_t* pages, int64_t num_free, int64_t pool_pages,
                              paged_kv_free_list** out);
void paged_kv_free_list_destroy(paged_kv_free_list* fl);
/* Takes the oldest free page.  EXHAUSTED when none is left. */
int paged_kv_free_list_pop(paged_kv_free_list* fl, int32_t* page);
/* Returns a page to the back of the list.  INVALID_ARG for an id out of
 * range or one that is already free. */
int paged_kv_free_list_push(paged_kv_free_list* fl, int32_t page);
/* Pool size, peak number of allocated pages since creation, free pages now. */
int paged_kv_free_list_stats(const paged_kv_free_list* fl, int64_t* pool_pages,
                             int64_t* peak_allocated, int64_t* free_pages);

/*
 * The lazy page step of one decode step ([HN-scope]).  For every sequence s
 * with n = context_lens[s] >= 1 (the length after this step's append) whose
 * new token, at position n-1, falls in a logical page j = (n-1)/16 it does
 * not hold yet (table entry < 0), one page per layer is taken from fl and
 * written to block_tables[(l*num_seqs + s)*bt_stride + j].  All or nothing:
 * when fewer pages are free than the step needs, EXHAUSTED is returned and
 * nothing changes.  changed (host, >= num_seqs entries, may be NULL) receives
 * the sequences whose rows changed, in increasing order, and num_changed
 * their number.
 *   block_tables  (host) int32 [num_layers][num_seqs][bt_stride]
 * Errors: INVALID_ARG (null pointer, negative counts, bt_stride < 1, a
 * position past the table width), EXHAUSTED.
 */
int paged_kv_lazy_page_step(paged_kv_free_list* fl, int32_t* block_tables, int32_t num_layers,
                            int32_t num_seqs, int64_t bt_stride, const int32_t* context_lens,
                            int32_t* changed, int32_t* num_changed);

/* ---------------------------------------------------------------- pager -- */

typedef struct paged_kv_pager paged_kv_pager;

typedef struct paged_kv_pager_stats {
    int64_t pool_pages;            /* pages the pager manages */
    int64_t free_pages;            /* free now */
    int64_t live_pages;            /* held by at least one request now */
    int64_t peak_live_pages;       /* peak allocated pages */
    int64_t credit_pages;          /* credits held by active requests now */
    int64_t shared_refs;           /* references beyond the first, over all live pages */
    int64_t copies;                /* copy-on-write page copies handed out so far */
    int32_t active_requests;
    int32_t peak_active_requests;
    int32_t waiting_requests;
    int32_t largest_decode_batch;
    int64_t submitted, admitted, rejected, finished;
    double wait_max_us;            /* longest admission wait (submit -> admit), microseconds */
    double wait_total_us;          /* sum of admission waits of admitted requests */
} paged_kv_pager_stats;

/*
 * A pager over pages 0 .. num_pages-1 (all free, handed out in id order) of a
 * model with num_layers layers and a context of max_context tokens.
 * Errors: INVALID_ARG (null out, num_pages < 1, num_layers < 1,
 * max_context < 1).
 */
int paged_kv_pager_create(int32_t num_pages, int32_t num_layers, int32_t max_context,
                          paged_kv_pager** out);
void paged_kv_pager_destroy(paged_kv_pager* pg);

/*
 * Queues a request ([HN-scope] admission): allowed_new = min(max_new_tokens,
 * max_context + 1 - prompt_tokens) new tokens, and a budget of
 * ceil((prompt_tokens + allowed_new - 1) / 16) pages per layer, times
 * num_layers, in credits.  A budget above the whole pool is refused
 * (REJECTED, nothing queued); otherwise the request waits in FIFO order.
 * Writes its id and allowed_new (either may be NULL).
 * Errors: INVALID_ARG (prompt_tokens outside [1, max_context],
 * max_new_tokens < 1), REJECTED.
 */
int paged_kv_pager_submit(paged_kv_pager* pg, int32_t prompt_tokens, int32_t max_new_tokens,
                          int64_t* request_id, int32_t* allowed_new);

/*
 * Admits waiting requests in FIFO order while the head's credits fit beside
 * the active requests' credits, up to capacity of them; stops at the first
 * that does not fit (no overtaking).  ids (host, capacity entries) receive
 * the admitted ids in order and num_admitted their number.
 */
int paged_kv_pager_admit(paged_kv_pager* pg, int64_t* ids, int32_t capacity,
                         int32_t* num_admitted);

/*
 * Makes an active request hold the pages of tokens [0, length) in every
 * layer, taking pages lazily, one per layer per new logical page.  Before a
 * token is written into a page that another request also holds (a shared
 * prefix page), the request gets a private page instead; each such
 * copy-on-write is reported as a (src, dst) page pair whose contents the
 * caller copies on the device before writing.  The request's table row is
 * written in full: table[l*layer_stride + j] for j < ceil(length/16).
 *   table        (host) int32, this request's [num_layers][layer_stride] row
 *   copy_src/dst (host) >= num_layers entries each; may be NULL when no
 *                copy is needed (INVALID_ARG, and nothing changes, when one is)
 * Length never shrinks: a length at or below what the request holds changes
 * nothing.  Admission guarantees that the pages are there.
 * Errors: INVALID_ARG (null table, length < 0, layer_stride too small),
 * STATE (unknown or not active), BUDGET (length above prompt + allowed_new
 * - 1).
 */
int paged_kv_pager_reserve(paged_kv_pager* pg, int64_t request_id, int32_t length,
                           int32_t* table, int64_t layer_stride, int32_t* copy_src,
                           int32_t* copy_dst, int32_t* num_copies);

/*
 * paged_kv_pager_reserve for the requests of one decode batch (ids[i] grows
 * to lengths[i]; its table row is tables + i*seq_stride), recording the batch
 * size for the statistics.  All lengths, and the pages the whole batch
 * needs, are checked before any page moves.  Copies are counted per physical
 * page: a shared page held by r requests and written by w of them in this
 * step costs min(w, r-1) copies (the last holder left writes in place), the
 * same as reserving the requests one by one.
 * copy_src/copy_dst need room for n * num_layers pairs.
 * Errors: those of reserve; EXHAUSTED (nothing changed) only if a broken
 * invariant leaves fewer free pages than the batch needs.
 */
int paged_kv_pager_decode_step(paged_kv_pager* pg, const int64_t* ids, const int32_t* lengths,
                               int32_t n, int32_t* tables, int64_t seq_stride,
                               int64_t layer_stride, int32_t* copy_src, int32_t* copy_dst,
                               int32_t* num_copies);

/*
 * Prefix sharing ([RS-prefix]): an active request dst that holds nothing yet
 * takes references to the pages of the first `tokens` tokens of the active
 * request src (which holds at least that many), in every layer, and holds
 * `tokens` tokens.  A partial last page is shared too; whichever request
 * writes into it first gets its own copy (see reserve).  dst's credits are
 * not reduced: sharing saves pages, admission stays as conservative as
 * without it.  dst's table row is written as in reserve.
 * Errors: INVALID_ARG (tokens < 1, tokens above dst's prompt, null table),
 * STATE (unknown or inactive requests, dst already holding pages, src
 * holding fewer tokens, src == dst).
 */
int paged_kv_pager_share_prefix(paged_kv_pager* pg, int64_t src_id, int64_t dst_id,
                                int32_t tokens, int32_t* table, int64_t layer_stride);

/*
 * Ends a request (done, stopped early, or cancelled while waiting): its page
 * references are dropped (a page no request holds goes back to the free
 * list) and its credits are released.  Errors: STATE (unknown id).
 */
int paged_kv_pager_finish(paged_kv_pager* pg, int64_t request_id);

int paged_kv_pager_get_stats(const paged_kv_pager* pg, paged_kv_pager_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_PAGER_H_ */
