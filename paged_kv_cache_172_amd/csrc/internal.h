// Internal interface between the C ABI layer (api.cpp) and the HIP kernels
// (kernels.hip).  Not installed; the public ABI is include/paged_kv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kQHeads = 32;
constexpr int kKVHeads = 8;
constexpr int kGroup = kQHeads / kKVHeads;  // query heads per KV head
constexpr int kHeadDim = 64;
constexpr int kPageTokens = 16;
constexpr int kMaxContext = 2048;
constexpr int kPartialFloats = kHeadDim + 2;  // accumulator row + (max, sum)

struct AppendParams {
    uint16_t* k_pool;
    uint16_t* v_pool;
    int64_t num_pages, page_stride, head_stride, slot_stride;
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* context_lens;
    int32_t num_seqs;
    uint16_t* q;
    int64_t q_stride;
    const uint16_t* k_new;
    int64_t k_stride;
    const uint16_t* v_new;
    int64_t v_stride;
    const float* rope_cos;
    const float* rope_sin;
    int32_t max_pos;
};

// Prefill page fill: packed prompt rows; row t of sequence s (cu_tokens[s] <=
// t < cu_tokens[s+1]) is the token at position start_pos[s] + t - cu_tokens[s].
struct PrefillParams {
    uint16_t* k_pool;
    uint16_t* v_pool;
    int64_t num_pages, page_stride, head_stride, slot_stride;
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* start_pos;
    const int32_t* cu_tokens;
    int32_t num_seqs;
    int32_t total_tokens;
    uint16_t* q;  // may be null: K/V only
    int64_t q_stride;
    const uint16_t* k_new;
    int64_t k_stride;
    const uint16_t* v_new;
    int64_t v_stride;
    const float* rope_cos;
    const float* rope_sin;
    int32_t max_pos;
};

// Whole-page copies (copy-on-write of shared prefix pages).
struct CopyParams {
    uint16_t* k_pool;
    uint16_t* v_pool;
    int64_t num_pages, page_stride, head_stride, slot_stride;
    const int32_t* src;
    const int32_t* dst;
    int32_t n;
};

// The split plan: S outer chunks per (sequence, KV head), each one workgroup
// of kChunkWaves waves; a sequence of np pages is cut into kChunkWaves * S
// chunks of ceil(np / (kChunkWaves * S)) pages.
constexpr int kChunkWaves = 4;
// Outer chunks per sequence at most (the plan caps S here; with contexts of
// at most 2,048 tokens and 4 pages per wave at least, S <= 8 anyway).
constexpr int kMaxSplits = 8;
struct Plan {
    int32_t splits;
};

// The plan asks for S > 1 only while num_seqs * 8 * kChunkWaves wavefronts
// fall short of its target of kPlanTargetWaves, i.e. for fewer than
// kMergeSeqs sequences.  The in-kernel merge of those S partials counts the
// finished workgroups of each (sequence, KV head) in a fixed block of
// kMergeSeqs * 8 int32 counters at the start of the workspace, whatever
// num_seqs is, so that every call finds its counters at the same place.
#ifndef PKV_TARGET_WAVES
#define PKV_TARGET_WAVES 2048
#endif
constexpr int64_t kPlanTargetWaves = PKV_TARGET_WAVES;
constexpr int kMergeSeqs = (int)(kPlanTargetWaves / (kKVHeads * kChunkWaves));
constexpr size_t kCounterBytes = (size_t)kMergeSeqs * kKVHeads * sizeof(int32_t);
static_assert(kCounterBytes % 256 == 0, "partials start 256-byte aligned");

struct AttnParams {
    const uint16_t* k_pool;
    const uint16_t* v_pool;
    int64_t num_pages, page_stride, head_stride, slot_stride;
    const int32_t* block_table;
    int64_t bt_stride;
    const int32_t* context_lens;
    const int32_t* seq_order;   // rank -> sequence, or null (batch order)
    int32_t num_seqs;
    int32_t max_context_len;
    const uint16_t* q;
    int64_t q_stride;
    float scale_log2;  // scale * log2(e): logits are kept in base-2 units
    Plan plan;
    // Waves take their issue priority from the pages they have left (the
    // most first); set when the grid is at most two rounds of what the GPU
    // holds at once.
    int32_t priority_by_pages_left;
    float* out;
    int64_t out_stride;
    float* ws_acc;     // [num_seqs][32][S][64]
    float2* ws_ml;     // [num_seqs][32][S] (maximum in base-2 units, sum)
    int32_t* ws_cnt;   // [kMergeSeqs][8] finished workgroups per (sequence, KV head)
    // Fused append only (launch_append_attn_split): the same pool, writable,
    // the new token's k/v rows and the RoPE table.
    uint16_t* k_pool_w;
    uint16_t* v_pool_w;
    const uint16_t* k_new;
    int64_t k_stride;
    const uint16_t* v_new;
    int64_t v_stride;
    const float* rope_cos;
    const float* rope_sin;
    int32_t max_pos;
};

Plan make_plan(int32_t num_seqs, int32_t max_context_len);
size_t workspace_bytes(int32_t num_seqs, int32_t max_context_len);

hipError_t launch_append(const AppendParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);
hipError_t launch_copy_pages(const CopyParams& p, hipStream_t stream);
// merge: when S > 1, the last workgroup of each (sequence, KV head) to
// finish merges the S partials into out (no combine launch needed).
hipError_t launch_attn_split(const AttnParams& p, bool merge, hipStream_t stream);
hipError_t launch_append_attn_split(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_combine(const AttnParams& p, hipStream_t stream);

// Ranks the sequences of a batch for the attention launches: seq_order[r]
// is the sequence of rank r, by descending page count (of the length clamped
// to max_context_len), ties by index.  One workgroup.
hipError_t launch_order(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                        int32_t* seq_order, hipStream_t stream);
// Attention workgroups the current device holds at once (looked up once per
// device); INT64_MAX when the query fails.
// The position at which sorted rank r (0 = most pages) starts.  The first
// `round_len` = R positions start together, one round of resident
// workgroups; the dispatcher deals them to the CUs in R/4-position slot
// rounds (one position per CU of an XCD).  With P = R/4: positions [0, 3P)
// take the 3P longest sequences, the middle slot round reversed, so that the
// CUs which take the longest in one round take the shorter in the next;
// positions [3P, 4P) take the P shortest, shortest first, which finish within
// the launch's ramp and hand their slots on; the rest follow, longest first.
// Identity when R < 4 or the batch is smaller than a round.
__host__ __device__ inline int order_position(int r, int num_seqs, int round_len) {
    const int P = round_len / 4;
    if (P < 1 || num_seqs < 4 * P) return r;
    if (r < 3 * P) {
        const int slot = r / P, k = r - slot * P;
        return slot == 1 ? P + (P - 1 - k) : r;
    }
    if (r >= num_seqs - P) return 3 * P + (num_seqs - 1 - r);
    return r + P;
}
// The page count the start order ranks by: ceil(min(ctx, max_context_len) / 16), 0 when ctx <= 0.
__host__ __device__ inline int order_page_count(int32_t ctx, int32_t max_context_len) {
    const int n = ctx < max_context_len ? ctx : max_context_len;
    return n > 0 ? (n + kPageTokens - 1) / kPageTokens : 0;
}

int64_t resident_workgroups();
// Sequences whose single-split workgroups (one per KV head) the current
// device holds at once: resident_workgroups() / 8, or 0 when unknown.
int32_t resident_seqs();

// The library's fixed device scratch (for callers that cannot allocate):
// its size, and its address on the current device (looked up, and its
// counters cleared on `stream`, on the first call per device).
size_t scratch_bytes();
hipError_t scratch_buffer(void** out, hipStream_t stream);

}  // namespace pkv
