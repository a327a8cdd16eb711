// C ABI of libpagedkv.so (declared in include/paged_kv.h): host-side argument
// checks, the split planner, and the kernel launches.  Every check runs
// before any HIP call, so a rejected call enqueues nothing; invalid requests
// get a clear status instead of undefined device behaviour ("Hours of YouTube
// and 85 handtyped pages of notes on LLM Inference - Start here", section
// "現在のスコープ": a request that cannot fit is refused with a clear error).
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "internal.h"
#include "paged_kv.h"
#include "paged_kv_pager.h"

namespace pkv {

// Split planner.  A decode batch has num_seqs * 8 (sequence, KV head)
// units; each outer chunk of a unit is one workgroup of kChunkWaves
// wavefronts.  The plan aims for about kTargetWaves wavefronts (two per SIMD
// of a 256-CU part) so that small batches still fill the chip, and never cuts
// chunks of a full-length context below kMinPagesPerSplit pages.  It depends
// only on (num_seqs, max_context_len).
#ifndef PKV_MIN_PAGES_PER_SPLIT
#define PKV_MIN_PAGES_PER_SPLIT 4
#endif
constexpr int64_t kTargetWaves = kPlanTargetWaves;
constexpr int32_t kMinPagesPerSplit = PKV_MIN_PAGES_PER_SPLIT;

static bool plan_args_ok(int32_t num_seqs, int32_t max_context_len) {
    return num_seqs >= 1 && max_context_len >= 1 && max_context_len <= kMaxContext;
}

Plan make_plan(int32_t num_seqs, int32_t max_context_len) {
    const int32_t max_pages = (max_context_len + kPageTokens - 1) / kPageTokens;
    const int64_t waves_per_split = (int64_t)num_seqs * kKVHeads * kChunkWaves;
    int64_t s = (kTargetWaves + waves_per_split - 1) / waves_per_split;
    const int64_t s_cap = max_pages / ((int64_t)kChunkWaves * kMinPagesPerSplit);
    if (s > s_cap) s = s_cap;
    if (s > kMaxSplits) s = kMaxSplits;
    if (num_seqs >= kMergeSeqs) s = 1;   // already implied; the merge counters rely on it
    if (s < 1) s = 1;
    return Plan{(int32_t)s};
}

// Workspace when S > 1: [counters: kCounterBytes][acc [B][32][S][64] FP32]
// [(max, sum) [B][32][S] float2].
size_t workspace_bytes(int32_t num_seqs, int32_t max_context_len) {
    const Plan plan = make_plan(num_seqs, max_context_len);
    if (plan.splits <= 1) return 0;
    return kCounterBytes +
           (size_t)plan.splits * (size_t)num_seqs * kQHeads * kPartialFloats * sizeof(float);
}

}  // namespace pkv

namespace {

thread_local char g_status_text[256];

int hip_status(hipError_t e) {
    if (e == hipSuccess) return PKV_OK;
    snprintf(g_status_text, sizeof g_status_text, "HIP error: %s", hipGetErrorString(e));
    return PKV_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_pool(const paged_kv_pool* pool) {
    if (!pool || !pool->k_pool || !pool->v_pool) return PKV_ERR_INVALID_ARG;
    if (pool->num_pages < 1 || pool->page_stride < 1 || pool->head_stride < 1 ||
        pool->slot_stride < pkv::kHeadDim)
        return PKV_ERR_INVALID_ARG;
    if (pool->num_pages > INT32_MAX) return PKV_ERR_INVALID_ARG;  // page ids are int32
    // The attention reads each (page, KV head) tile through a buffer
    // descriptor whose byte range and lane offsets are 32-bit: the 16 slots
    // of a head must span less than 2^30 elements.
    if ((pkv::kPageTokens - 1) * pool->slot_stride + pkv::kHeadDim >= ((int64_t)1 << 30))
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(pool->k_pool) || !aligned16(pool->v_pool)) return PKV_ERR_ALIGNMENT;
    if (pool->page_stride % 8 || pool->head_stride % 8 || pool->slot_stride % 8)
        return PKV_ERR_ALIGNMENT;
    return PKV_OK;
}

// Checks of the append's own arguments (num_seqs >= 1 checked by the caller).
int check_append(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                 const int32_t* context_lens, const uint16_t* q, int64_t q_stride,
                 const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                 int64_t v_stride, const float* rope_cos, const float* rope_sin,
                 int32_t max_pos) {
    const int st = check_pool(pool);
    if (st != PKV_OK) return st;
    if (!block_table || !context_lens || !q || !k_new || !v_new || !rope_cos || !rope_sin)
        return PKV_ERR_INVALID_ARG;
    if (bt_stride < 1 || max_pos < 1) return PKV_ERR_INVALID_ARG;
    if (q_stride < pkv::kQHeads * pkv::kHeadDim || k_stride < pkv::kKVHeads * pkv::kHeadDim ||
        v_stride < pkv::kKVHeads * pkv::kHeadDim)
        return PKV_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(rope_cos) ||
        !aligned16(rope_sin) || q_stride % 8 || k_stride % 8 || v_stride % 8)
        return PKV_ERR_ALIGNMENT;
    return PKV_OK;
}

// Points the partial and counter arrays of p (plan and num_seqs set) into a
// workspace laid out as workspace_bytes() describes.
void set_workspace(pkv::AttnParams& p, void* workspace) {
    char* base = static_cast<char*>(workspace);
    const size_t acc_bytes =
        (size_t)p.plan.splits * p.num_seqs * pkv::kQHeads * pkv::kHeadDim * sizeof(float);
    p.ws_cnt = reinterpret_cast<int32_t*>(base);
    p.ws_acc = reinterpret_cast<float*>(base + pkv::kCounterBytes);
    p.ws_ml = reinterpret_cast<float2*>(base + pkv::kCounterBytes + acc_bytes);
}

// Whether an attention launch follows the caller's sequence order: only
// when its workgroups do not all fit on the device at once (the order then
// decides which ones start first; otherwise every workgroup starts at once
// and reading the order would only delay each start).  The resident count
// is the occupancy of the attention kernel times the compute units, looked
// up once per device.
bool use_order(const int32_t* seq_order, int32_t num_seqs, const pkv::Plan& plan) {
    if (!seq_order) return false;
    const int64_t grid = (int64_t)num_seqs * pkv::kKVHeads * plan.splits;
    return grid > pkv::resident_workgroups();
}

// Priority by pages left pays while the launch is at most two rounds of
// resident workgroups: the critical path and the two workgroups that share a
// CU then set its end.  Over many rounds of like workgroups the hardware's
// oldest-first issue frees slots soonest, and it is left alone.
bool priority_by_pages_left(int32_t num_seqs, const pkv::Plan& plan) {
    const int64_t grid = (int64_t)num_seqs * pkv::kKVHeads * plan.splits;
    return (grid + 1) / 2 <= pkv::resident_workgroups();
}

struct AttnCheck {
    int status;
    pkv::AttnParams params;
};

AttnCheck check_attn(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                     const int32_t* context_lens, const int32_t* seq_order, int32_t num_seqs,
                     int32_t max_context_len,
                     const uint16_t* q, int64_t q_stride, float scale, float* out,
                     int64_t out_stride, void* workspace, size_t workspace_bytes) {
    AttnCheck r{};
    r.status = PKV_ERR_INVALID_ARG;
    if (num_seqs < 0) return r;
    if (num_seqs == 0) {
        r.status = PKV_OK;
        return r;
    }
    int st = check_pool(pool);
    if (st != PKV_OK) {
        r.status = st;
        return r;
    }
    if (!block_table || !context_lens || !q || !out) return r;
    if (bt_stride < 1 || max_context_len < 1 || max_context_len > pkv::kMaxContext) return r;
    if ((int64_t)max_context_len > bt_stride * pkv::kPageTokens) return r;
    if (!isfinite(scale)) return r;
    if (q_stride < pkv::kQHeads * pkv::kHeadDim || out_stride < pkv::kQHeads * pkv::kHeadDim)
        return r;
    if (!aligned16(q) || !aligned16(out) || q_stride % 8 || out_stride % 4) {
        r.status = PKV_ERR_ALIGNMENT;
        return r;
    }
    const size_t need = pkv::workspace_bytes(num_seqs, max_context_len);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) {
            r.status = PKV_ERR_WORKSPACE;
            return r;
        }
        if (!aligned16(workspace)) {
            r.status = PKV_ERR_ALIGNMENT;
            return r;
        }
    }
    pkv::AttnParams& p = r.params;
    p.plan = pkv::make_plan(num_seqs, max_context_len);
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.num_pages = pool->num_pages;
    p.page_stride = pool->page_stride;
    p.head_stride = pool->head_stride;
    p.slot_stride = pool->slot_stride;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.max_context_len = max_context_len;
    p.seq_order = use_order(seq_order, num_seqs, p.plan) ? seq_order : nullptr;
    p.priority_by_pages_left = priority_by_pages_left(num_seqs, p.plan) ? 1 : 0;
    p.q = q;
    p.q_stride = q_stride;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634);  // scale / ln 2
    p.out = out;
    p.out_stride = out_stride;
    if (need > 0) set_workspace(p, workspace);
    r.status = PKV_OK;
    return r;
}

}  // namespace

extern "C" {

int paged_kv_rope_table(double theta, int32_t max_pos, float* cos_out, float* sin_out) {
    if (!cos_out || !sin_out || max_pos < 1 || !(theta > 0.0) || !isfinite(theta))
        return PKV_ERR_INVALID_ARG;
    for (int32_t pos = 0; pos < max_pos; ++pos) {
        for (int i = 0; i < pkv::kHeadDim / 2; ++i) {
            // angle = pos * theta^(-2i/64), FP64, then one rounding to FP32
            const double freq = pow(theta, -(double)(2 * i) / (double)pkv::kHeadDim);
            const double angle = (double)pos * freq;
            cos_out[(int64_t)pos * 32 + i] = (float)cos(angle);
            sin_out[(int64_t)pos * 32 + i] = (float)sin(angle);
        }
    }
    return PKV_OK;
}

int paged_kv_append(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                    const int32_t* context_lens, int32_t num_seqs, uint16_t* q, int64_t q_stride,
                    const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                    int64_t v_stride, const float* rope_cos, const float* rope_sin,
                    int32_t max_pos, void* stream) {
    if (num_seqs < 0) return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0) return PKV_OK;
    const int st = check_append(pool, block_table, bt_stride, context_lens, q, q_stride, k_new,
                                k_stride, v_new, v_stride, rope_cos, rope_sin, max_pos);
    if (st != PKV_OK) return st;
    pkv::AppendParams p;
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.num_pages = pool->num_pages;
    p.page_stride = pool->page_stride;
    p.head_stride = pool->head_stride;
    p.slot_stride = pool->slot_stride;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.q = q;
    p.q_stride = q_stride;
    p.k_new = k_new;
    p.k_stride = k_stride;
    p.v_new = v_new;
    p.v_stride = v_stride;
    p.rope_cos = rope_cos;
    p.rope_sin = rope_sin;
    p.max_pos = max_pos;
    return hip_status(pkv::launch_append(p, static_cast<hipStream_t>(stream)));
}

int paged_kv_prefill(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                     const int32_t* start_pos, const int32_t* cu_tokens, int32_t num_seqs,
                     int32_t total_tokens, uint16_t* q, int64_t q_stride, const uint16_t* k_new,
                     int64_t k_stride, const uint16_t* v_new, int64_t v_stride,
                     const float* rope_cos, const float* rope_sin, int32_t max_pos,
                     void* stream) {
    if (num_seqs < 0 || total_tokens < 0 || total_tokens > (1 << 30)) return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0 || total_tokens == 0) return PKV_OK;
    if (!start_pos || !cu_tokens) return PKV_ERR_INVALID_ARG;
    // q is optional here: with NULL only K/V are written.  Its stride is
    // checked only when it is given.
    static const uint16_t kNoQ[8] __attribute__((aligned(16))) = {};
    const int st = check_append(pool, block_table, bt_stride, start_pos, q ? q : kNoQ,
                                q ? q_stride : pkv::kQHeads * pkv::kHeadDim, k_new, k_stride,
                                v_new, v_stride, rope_cos, rope_sin, max_pos);
    if (st != PKV_OK) return st;
    pkv::PrefillParams p;
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.num_pages = pool->num_pages;
    p.page_stride = pool->page_stride;
    p.head_stride = pool->head_stride;
    p.slot_stride = pool->slot_stride;
    p.block_table = block_table;
    p.bt_stride = bt_stride;
    p.start_pos = start_pos;
    p.cu_tokens = cu_tokens;
    p.num_seqs = num_seqs;
    p.total_tokens = total_tokens;
    p.q = q;
    p.q_stride = q_stride;
    p.k_new = k_new;
    p.k_stride = k_stride;
    p.v_new = v_new;
    p.v_stride = v_stride;
    p.rope_cos = rope_cos;
    p.rope_sin = rope_sin;
    p.max_pos = max_pos;
    return hip_status(pkv::launch_prefill(p, static_cast<hipStream_t>(stream)));
}

int paged_kv_copy_pages(const paged_kv_pool* pool, const int32_t* src, const int32_t* dst,
                        int32_t num_pairs, void* stream) {
    if (num_pairs < 0) return PKV_ERR_INVALID_ARG;
    if (num_pairs == 0) return PKV_OK;
    const int st = check_pool(pool);
    if (st != PKV_OK) return st;
    if (!src || !dst) return PKV_ERR_INVALID_ARG;
    pkv::CopyParams p;
    p.k_pool = pool->k_pool;
    p.v_pool = pool->v_pool;
    p.num_pages = pool->num_pages;
    p.page_stride = pool->page_stride;
    p.head_stride = pool->head_stride;
    p.slot_stride = pool->slot_stride;
    p.src = src;
    p.dst = dst;
    p.n = num_pairs;
    return hip_status(pkv::launch_copy_pages(p, static_cast<hipStream_t>(stream)));
}

int32_t paged_decode_attn_num_splits(int32_t num_seqs, int32_t max_context_len) {
    if (!pkv::plan_args_ok(num_seqs, max_context_len)) return 0;
    return pkv::make_plan(num_seqs, max_context_len).splits;
}

size_t paged_decode_attn_workspace_size(int32_t num_seqs, int32_t max_context_len) {
    if (!pkv::plan_args_ok(num_seqs, max_context_len)) return 0;
    return pkv::workspace_bytes(num_seqs, max_context_len);
}

int paged_decode_attn_order(const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int32_t* seq_order, void* stream) {
    if (num_seqs < 0) return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0) return PKV_OK;
    if (!context_lens || !seq_order || max_context_len < 1 || max_context_len > pkv::kMaxContext)
        return PKV_ERR_INVALID_ARG;
    return hip_status(pkv::launch_order(context_lens, num_seqs, max_context_len, seq_order,
                                        static_cast<hipStream_t>(stream)));
}

int32_t paged_decode_attn_order_round(void) { return pkv::resident_seqs(); }

int paged_decode_attn_order_host(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                                 int32_t round_len, int32_t* seq_order) {
    if (num_seqs < 0 || round_len < 0) return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0) return PKV_OK;
    if (!context_lens || !seq_order || max_context_len < 1 || max_context_len > pkv::kMaxContext)
        return PKV_ERR_INVALID_ARG;
    // The same order as order_kernel: a stable counting sort by descending
    // page count, then each sorted rank written at its start position.
    constexpr int kBins = pkv::kMaxContext / pkv::kPageTokens + 1;
    int64_t start[kBins + 1] = {};
    for (int32_t s = 0; s < num_seqs; ++s)
        ++start[kBins - 1 - pkv::order_page_count(context_lens[s], max_context_len) + 1];
    for (int b = 1; b <= kBins; ++b) start[b] += start[b - 1];   // start[kBins-1-count]: first rank of count
    for (int32_t s = 0; s < num_seqs; ++s) {
        const int bin = kBins - 1 - pkv::order_page_count(context_lens[s], max_context_len);
        const int r = (int)start[bin]++;
        seq_order[pkv::order_position(r, num_seqs, round_len)] = s;
    }
    return PKV_OK;
}

int paged_decode_attn_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (workspace_bytes == 0) return PKV_OK;
    if (!workspace) return PKV_ERR_INVALID_ARG;
    if (!aligned16(workspace)) return PKV_ERR_ALIGNMENT;
    const size_t n = workspace_bytes < pkv::kCounterBytes ? workspace_bytes : pkv::kCounterBytes;
    return hip_status(hipMemsetAsync(workspace, 0, n, static_cast<hipStream_t>(stream)));
}

int paged_decode_attn_split(const paged_kv_pool* pool, const int32_t* block_table,
                            int64_t bt_stride, const int32_t* context_lens,
                            const int32_t* seq_order, int32_t num_seqs,
                            int32_t max_context_len, const uint16_t* q, int64_t q_stride,
                            float scale, float* out, int64_t out_stride, void* workspace,
                            size_t workspace_bytes, void* stream) {
    AttnCheck c = check_attn(pool, block_table, bt_stride, context_lens, seq_order, num_seqs,
                             max_context_len, q, q_stride, scale, out, out_stride, workspace,
                             workspace_bytes);
    if (c.status != PKV_OK || num_seqs == 0) return c.status;
    return hip_status(pkv::launch_attn_split(c.params, false, static_cast<hipStream_t>(stream)));
}

int paged_decode_attn_combine(const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, float* out, int64_t out_stride,
                              const void* workspace, size_t workspace_bytes, void* stream) {
    if (num_seqs < 0) return PKV_ERR_INVALID_ARG;
    if (num_seqs == 0) return PKV_OK;
    if (!context_lens || !out || max_context_len < 1 || max_context_len > pkv::kMaxContext)
        return PKV_ERR_INVALID_ARG;
    if (out_stride < pkv::kQHeads * pkv::kHeadDim) return PKV_ERR_INVALID_ARG;
    if (!aligned16(out) || out_stride % 4) return PKV_ERR_ALIGNMENT;
    const pkv::Plan plan = pkv::make_plan(num_seqs, max_context_len);
    if (plan.splits <= 1) return PKV_OK;
    const size_t need = pkv::workspace_bytes(num_seqs, max_context_len);
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PKV_ERR_ALIGNMENT;
    pkv::AttnParams p{};
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.max_context_len = max_context_len;
    p.plan = plan;
    p.out = out;
    p.out_stride = out_stride;
    set_workspace(p, const_cast<void*>(workspace));
    return hip_status(pkv::launch_attn_combine(p, static_cast<hipStream_t>(stream)));
}

int paged_decode_attn(const paged_kv_pool* pool, const int32_t* block_table, int64_t bt_stride,
                      const int32_t* context_lens, const int32_t* seq_order, int32_t num_seqs,
                      int32_t max_context_len,
                      const uint16_t* q, int64_t q_stride, float scale, float* out,
                      int64_t out_stride, void* workspace, size_t workspace_bytes, void* stream) {
    AttnCheck c = check_attn(pool, block_table, bt_stride, context_lens, seq_order, num_seqs,
                             max_context_len, q, q_stride, scale, out, out_stride, workspace,
                             workspace_bytes);
    if (c.status != PKV_OK || num_seqs == 0) return c.status;
    return hip_status(pkv::launch_attn_split(c.params, true, static_cast<hipStream_t>(stream)));
}

int paged_kv_append_decode_attn(const paged_kv_pool* pool, const int32_t* block_table,
                                int64_t bt_stride, const int32_t* context_lens,
                                const int32_t* seq_order, int32_t num_seqs,
                                int32_t max_context_len, const uint16_t* q, int64_t q_stride,
                                const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                                int64_t v_stride, const float* rope_cos, const float* rope_sin,
                                int32_t max_pos, float scale, float* out, int64_t out_stride,
                                void* workspace, size_t workspace_bytes, void* stream) {
    AttnCheck c = check_attn(pool, block_table, bt_stride, context_lens, seq_order, num_seqs,
                             max_context_len, q, q_stride, scale, out, out_stride, workspace,
                             workspace_bytes);
    if (c.status != PKV_OK || num_seqs == 0) return c.status;
    const int st = check_append(pool, block_table, bt_stride, context_lens, q, q_stride, k_new,
                                k_stride, v_new, v_stride, rope_cos, rope_sin, max_pos);
    if (st != PKV_OK) return st;
    pkv::AttnParams& p = c.params;
    p.k_pool_w = pool->k_pool;
    p.v_pool_w = pool->v_pool;
    p.k_new = k_new;
    p.k_stride = k_stride;
    p.v_new = v_new;
    p.v_stride = v_stride;
    p.rope_cos = rope_cos;
    p.rope_sin = rope_sin;
    p.max_pos = max_pos;
    return hip_status(pkv::launch_append_attn_split(p, static_cast<hipStream_t>(stream)));
}

int paged_kv_append_decode_attn_noalloc(const paged_kv_pool* pool, const int32_t* block_table,
                                        int64_t bt_stride, const int32_t* context_lens,
                                        const int32_t* seq_order, int32_t num_seqs,
                                        int32_t max_context_len,
                                        const uint16_t* q, int64_t q_stride,
                                        const uint16_t* k_new, int64_t k_stride,
                                        const uint16_t* v_new, int64_t v_stride,
                                        const float* rope_cos, const float* rope_sin,
                                        int32_t max_pos, float scale, float* out,
                                        int64_t out_stride, void* stream) {
    // Every argument is checked before any HIP call; the workspace check is
    // against the fixed scratch (a stand-in pointer: only its size and
    // alignment are looked at here).
    const size_t need = num_seqs > 0 && pkv::plan_args_ok(num_seqs, max_context_len)
                            ? pkv::workspace_bytes(num_seqs, max_context_len)
                            : 0;
    if (need > pkv::scratch_bytes()) return PKV_ERR_WORKSPACE;
    static char stand_in alignas(16);
    AttnCheck c = check_attn(pool, block_table, bt_stride, context_lens, seq_order, num_seqs,
                             max_context_len, q, q_stride, scale, out, out_stride,
                             need ? &stand_in : nullptr, need);
    if (c.status != PKV_OK || num_seqs == 0) return c.status;
    const int st = check_append(pool, block_table, bt_stride, context_lens, q, q_stride, k_new,
                                k_stride, v_new, v_stride, rope_cos, rope_sin, max_pos);
    if (st != PKV_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    pkv::AttnParams& p = c.params;
    if (need > 0) {
        void* ws = nullptr;
        const int hs = hip_status(pkv::scratch_buffer(&ws, s));
        if (hs != PKV_OK) return hs;
        set_workspace(p, ws);
    }
    p.k_pool_w = pool->k_pool;
    p.v_pool_w = pool->v_pool;
    p.k_new = k_new;
    p.k_stride = k_stride;
    p.v_new = v_new;
    p.v_stride = v_stride;
    p.rope_cos = rope_cos;
    p.rope_sin = rope_sin;
    p.max_pos = max_pos;
    return hip_status(pkv::launch_append_attn_split(p, s));
}

const char* paged_kv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_INVALID_ARG: return "invalid argument";
        case PKV_ERR_ALIGNMENT: return "pointer or stride not 16-byte aligned";
        case PKV_ERR_WORKSPACE: return "workspace smaller than paged_decode_attn_workspace_size()";
        case PKV_ERR_UNSUPPORTED: return "unsupported geometry";
        case PKV_ERR_HIP: return g_status_text[0] ? g_status_text : "HIP error";
        case PKV_ERR_EXHAUSTED: return "KV page pool exhausted: no free page left";
        case PKV_ERR_REJECTED:
            return "request rejected: its page budget exceeds the whole KV page pool";
        case PKV_ERR_BUDGET: return "length beyond the request's admitted budget";
        case PKV_ERR_STATE: return "unknown request, or request in the wrong state";
        default: return "unknown status";
    }
}

}  // extern "C"
