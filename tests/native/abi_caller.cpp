// A native caller of libpagedkv.so through its C ABI (include/paged_kv.h),
// for the GPU tests: no Python in the call path.
//
// 1. Parity.  A mixed batch of 8 sequences (1 to 2,048 tokens), one layer:
//    the fused call (paged_kv_append_decode_attn) against the FP64 oracle
//    (oracle/pkv_oracle.c, test infrastructure, linked as its own library):
//    the pool bytes and the BF16 rows the append writes must be equal bit for
//    bit, the attention output within 2e-3 absolute and 1e-2 relative (to
//    max(|oracle|, 1e-3)); the two-call path (paged_kv_append then
//    paged_decode_attn) must equal the fused call bit for bit.  The library's
//    RoPE table must equal the oracle's bit for bit.
// 2. Latency.  One sequence of 37 tokens (the fused call and the attention
//    alone, planned from 2,048 and from 37 tokens): back-to-back calls from
//    C on one stream between two HIP events, and the host's own time per
//    call.
//
// Prints one JSON line; exits 0 when every check passes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "paged_kv.h"

extern "C" {
// oracle/pkv_oracle.c (FP64 reference, test infrastructure)
int pkv_oracle_rope_table(double theta, int32_t max_pos, float* cos_out, float* sin_out);
int pkv_oracle_append(uint16_t* k_pool, uint16_t* v_pool, int64_t num_pages, int64_t page_stride,
                      int64_t head_stride, int64_t slot_stride, const int32_t* block_table,
                      int64_t bt_stride, const int32_t* ctx, int32_t num_seqs, uint16_t* q,
                      int64_t q_stride, const uint16_t* k, int64_t k_stride, const uint16_t* v,
                      int64_t v_stride, const float* rope_cos, const float* rope_sin,
                      int32_t max_pos);
int pkv_oracle_attn(const uint16_t* k_pool, const uint16_t* v_pool, int64_t num_pages,
                    int64_t page_stride, int64_t head_stride, int64_t slot_stride,
                    const int32_t* block_table, int64_t bt_stride, const int32_t* ctx,
                    int32_t num_seqs, const uint16_t* q, int64_t q_stride, double scale,
                    double* out64, int64_t out64_stride, float* out32, int64_t out32_stride);
}

namespace {

constexpr int kQRow = 32 * 64;       // q and output row: 32 heads x 64 dims
constexpr int kKVRow = 8 * 64;       // new k / v row: 8 KV heads x 64 dims
constexpr int kPageElems = 2 * 8 * 16 * 64;
constexpr int kHalfPage = 8 * 16 * 64;
constexpr int kMaxPos = 2048;
constexpr int kTableWidth = 128;
constexpr uint16_t kBf16Nan = 0x7FC0;
constexpr float kScale = 0.125f;

int g_failures = 0;

void fail(const char* what) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    ++g_failures;
}

#define HIP_OK(call)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (call);                                                               \
        if (e_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, \
                         __LINE__);                                                           \
            std::exit(2);                                                                     \
        }                                                                                     \
    } while (0)

#define PKV_OK_OR_DIE(call)                                                                   \
    do {                                                                                      \
        int st_ = (call);                                                                     \
        if (st_ != PKV_OK) {                                                                  \
            std::fprintf(stderr, "libpagedkv error %d (%s) at %s:%d\n", st_,                 \
                         paged_kv_status_string(st_), __FILE__, __LINE__);                   \
            std::exit(3);                                                                     \
        }                                                                                     \
    } while (0)

// Seeded inputs (xorshift64*; no part of the method): BF16 bit patterns of
// values in [-2, 2), and a permutation for page placement.
struct Rng {
    uint64_t s;
    explicit Rng(uint64_t seed) : s(seed * 0x9E3779B97F4A7C15ull + 1) {}
    uint64_t next() {
        s ^= s >> 12;
        s ^= s << 25;
        s ^= s >> 27;
        return s * 0x2545F4914F6CDD1Dull;
    }
    uint16_t bf16() {
        const float x = (float)((next() >> 40) * (1.0 / 16777216.0)) * 4.0f - 2.0f;
        uint32_t b;
        std::memcpy(&b, &x, 4);
        return (uint16_t)(b >> 16);
    }
};

template <typename T>
T* to_device(const std::vector<T>& h) {
    T* d = nullptr;
    HIP_OK(hipMalloc(&d, h.size() * sizeof(T)));
    HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

template <typename T>
std::vector<T> to_host(const T* d, size_t n) {
    std::vector<T> h(n);
    HIP_OK(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

// One host batch: pool [P][2][8][16][64], table [B][128], lengths, new rows.
struct Batch {
    std::vector<int32_t> ctx;
    int32_t num_pages = 0;
    std::vector<uint16_t> pool;
    std::vector<int32_t> table;
    std::vector<uint16_t> q, k, v;
};

Batch make_batch(const std::vector<int32_t>& lengths, uint64_t seed) {
    Rng rng(seed);
    Batch b;
    b.ctx = lengths;
    const int B = (int)lengths.size();
    int held = 0;
    for (int n : lengths) held += (n + 15) / 16;
    b.num_pages = held + 16;   // spare pages: never referenced, NaN
    std::vector<int32_t> perm(b.num_pages);
    for (int i = 0; i < b.num_pages; ++i) perm[i] = i;
    for (int i = b.num_pages - 1; i > 0; --i) std::swap(perm[i], perm[rng.next() % (uint64_t)(i + 1)]);
    b.pool.assign((size_t)b.num_pages * kPageElems, kBf16Nan);
    b.table.assign((size_t)B * kTableWidth, -1);
    int next = 0;
    for (int s = 0; s < B; ++s) {
        const int n = lengths[s];
        for (int j = 0; j < (n + 15) / 16; ++j) {
            const int page = perm[next++];
            b.table[(size_t)s * kTableWidth + j] = page;
            for (int t = 0; t < 16; ++t) {
                if (j * 16 + t >= n - 1) break;   // the new token's slot and later stay NaN
                for (int g = 0; g < 8; ++g)
                    for (int d = 0; d < 64; ++d) {
                        const size_t off = (size_t)page * kPageElems + (size_t)g * 1024 + t * 64 + d;
                        b.pool[off] = rng.bf16();                  // K
                        b.pool[off + kHalfPage] = rng.bf16();      // V
                    }
            }
        }
    }
    b.q.resize((size_t)B * kQRow);
    b.k.resize((size_t)B * kKVRow);
    b.v.resize((size_t)B * kKVRow);
    for (auto& x : b.q) x = rng.bf16();
    for (auto& x : b.k) x = rng.bf16();
    for (auto& x : b.v) x = rng.bf16();
    return b;
}

// Device copy of a batch, with its output rows and workspace.
struct DevBatch {
    uint16_t* pool = nullptr;
    int32_t* table = nullptr;
    int32_t* ctx = nullptr;
    uint16_t *q = nullptr, *k = nullptr, *v = nullptr;
    float* out = nullptr;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    paged_kv_pool p{};
    int B = 0;
    int max_context_len = 0;
};

DevBatch upload(const Batch& b, int max_context_len, hipStream_t stream) {
    DevBatch d;
    d.B = (int)b.ctx.size();
    d.max_context_len = max_context_len;
    d.pool = to_device(b.pool);
    d.table = to_device(b.table);
    d.ctx = to_device(b.ctx);
    d.q = to_device(b.q);
    d.k = to_device(b.k);
    d.v = to_device(b.v);
    HIP_OK(hipMalloc(&d.out, (size_t)d.B * kQRow * sizeof(float)));
    d.ws_bytes = paged_decode_attn_workspace_size(d.B, max_context_len);
    if (d.ws_bytes) {
        HIP_OK(hipMalloc(&d.ws, d.ws_bytes));
        PKV_OK_OR_DIE(paged_decode_attn_workspace_init(d.ws, d.ws_bytes, stream));
    }
    d.p = paged_kv_pool{d.pool, d.pool + kHalfPage, b.num_pages, kPageElems, 16 * 64, 64};
    return d;
}

void release(DevBatch& d) {
    for (void* x : {(void*)d.pool, (void*)d.table, (void*)d.ctx, (void*)d.q, (void*)d.k, (void*)d.v,
                    (void*)d.out, d.ws})
        if (x) HIP_OK(hipFree(x));
    d = DevBatch{};
}

int fused(DevBatch& d, const float* cos, const float* sin, hipStream_t stream) {
    return paged_kv_append_decode_attn(&d.p, d.table, kTableWidth, d.ctx, nullptr, d.B, d.max_context_len,
                                       d.q, kQRow, d.k, kKVRow, d.v, kKVRow, cos, sin, kMaxPos, kScale,
                                       d.out, kQRow, d.ws, d.ws_bytes, stream);
}

int attn(DevBatch& d, hipStream_t stream) {
    return paged_decode_attn(&d.p, d.table, kTableWidth, d.ctx, nullptr, d.B, d.max_context_len, d.q, kQRow,
                             kScale, d.out, kQRow, d.ws, d.ws_bytes, stream);
}

}  // namespace

int main() {
    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));

    // RoPE tables: the library's, checked against the oracle's bit for bit.
    std::vector<float> cos_h((size_t)kMaxPos * 32), sin_h((size_t)kMaxPos * 32);
    std::vector<float> cos_o((size_t)kMaxPos * 32), sin_o((size_t)kMaxPos * 32);
    PKV_OK_OR_DIE(paged_kv_rope_table(500000.0, kMaxPos, cos_h.data(), sin_h.data()));
    if (pkv_oracle_rope_table(500000.0, kMaxPos, cos_o.data(), sin_o.data()) != 0) fail("oracle rope table");
    if (std::memcmp(cos_h.data(), cos_o.data(), cos_h.size() * 4) ||
        std::memcmp(sin_h.data(), sin_o.data(), sin_h.size() * 4))
        fail("RoPE table differs from the oracle's");
    float* cos_d = to_device(cos_h);
    float* sin_d = to_device(sin_h);

    // ---- parity: a mixed batch ----
    const std::vector<int32_t> lengths = {37, 1, 16, 17, 300, 1000, 2048, 129};
    const int B = (int)lengths.size();
    Batch hb = make_batch(lengths, 1720);
    DevBatch fz = upload(hb, 2048, stream);
    PKV_OK_OR_DIE(fused(fz, cos_d, sin_d, stream));
    HIP_OK(hipStreamSynchronize(stream));
    const auto pool_gpu = to_host(fz.pool, hb.pool.size());
    const auto out_gpu = to_host(fz.out, (size_t)B * kQRow);

    // the two-call path on a second copy
    DevBatch tc = upload(hb, 2048, stream);
    PKV_OK_OR_DIE(paged_kv_append(&tc.p, tc.table, kTableWidth, tc.ctx, B, tc.q, kQRow, tc.k, kKVRow, tc.v,
                                  kKVRow, cos_d, sin_d, kMaxPos, stream));
    PKV_OK_OR_DIE(attn(tc, stream));
    HIP_OK(hipStreamSynchronize(stream));
    const auto pool_two = to_host(tc.pool, hb.pool.size());
    const auto out_two = to_host(tc.out, (size_t)B * kQRow);
    const auto q_two = to_host(tc.q, hb.q.size());

    // the oracle on host copies
    std::vector<uint16_t> pool_o = hb.pool, q_o = hb.q;
    if (pkv_oracle_append(pool_o.data(), pool_o.data() + kHalfPage, hb.num_pages, kPageElems, 16 * 64, 64,
                          hb.table.data(), kTableWidth, hb.ctx.data(), B, q_o.data(), kQRow, hb.k.data(),
                          kKVRow, hb.v.data(), kKVRow, cos_o.data(), sin_o.data(), kMaxPos) != 0)
        fail("oracle append");
    std::vector<double> ref((size_t)B * kQRow);
    if (pkv_oracle_attn(pool_o.data(), pool_o.data() + kHalfPage, hb.num_pages, kPageElems, 16 * 64, 64,
                        hb.table.data(), kTableWidth, hb.ctx.data(), B, q_o.data(), kQRow, kScale, ref.data(),
                        kQRow, nullptr, 0) != 0)
        fail("oracle attention");

    if (pool_gpu != pool_o) fail("fused call: pool differs from the oracle");
    if (q_two != q_o) fail("paged_kv_append: rotated q differs from the oracle");
    if (pool_two != pool_gpu) fail("two calls: pool differs from the fused call");
    if (std::memcmp(out_two.data(), out_gpu.data(), out_gpu.size() * 4)) fail("two calls: output differs from the fused call");
    double max_abs = 0.0, max_rel = 0.0;
    bool finite = true;
    for (size_t i = 0; i < out_gpu.size(); ++i) {
        if (!std::isfinite(out_gpu[i])) finite = false;
        const double e = std::fabs((double)out_gpu[i] - ref[i]);
        max_abs = std::fmax(max_abs, e);
        max_rel = std::fmax(max_rel, e / std::fmax(std::fabs(ref[i]), 1e-3));
    }
    if (!finite) fail("fused call: non-finite output");
    if (!(max_abs <= 2e-3 && max_rel <= 1e-2)) fail("fused call: output outside 2e-3 / 1e-2 of the oracle");
    release(fz);
    release(tc);

    // ---- latency: one sequence of 37 tokens, back-to-back calls from C ----
    Batch one = make_batch({37}, 1721);
    struct Leg {
        const char* name;
        int max_context_len;
        bool fused;
        double device_us, host_us;
        int splits;
    } legs[] = {{"fused_plan_2048", 2048, true, 0, 0, 0}, {"attn_plan_2048", 2048, false, 0, 0, 0},
                {"fused_plan_37", 37, true, 0, 0, 0}, {"attn_plan_37", 37, false, 0, 0, 0}};
    constexpr int kReps = 500;
    hipEvent_t e0, e1;
    HIP_OK(hipEventCreate(&e0));
    HIP_OK(hipEventCreate(&e1));
    for (auto& leg : legs) {
        DevBatch d = upload(one, leg.max_context_len, stream);
        leg.splits = paged_decode_attn_num_splits(1, leg.max_context_len);
        PKV_OK_OR_DIE(fused(d, cos_d, sin_d, stream));   // writes the new token's rows
        for (int i = 0; i < 20; ++i) PKV_OK_OR_DIE(leg.fused ? fused(d, cos_d, sin_d, stream) : attn(d, stream));
        HIP_OK(hipStreamSynchronize(stream));
        HIP_OK(hipEventRecord(e0, stream));
        const auto t0 = std::chrono::steady_clock::now();
        for (int i = 0; i < kReps; ++i) PKV_OK_OR_DIE(leg.fused ? fused(d, cos_d, sin_d, stream) : attn(d, stream));
        const auto t1 = std::chrono::steady_clock::now();
        HIP_OK(hipEventRecord(e1, stream));
        HIP_OK(hipEventSynchronize(e1));
        float ms = 0.0f;
        HIP_OK(hipEventElapsedTime(&ms, e0, e1));
        leg.device_us = ms * 1e3 / kReps;
        leg.host_us = std::chrono::duration<double, std::micro>(t1 - t0).count() / kReps;
        const auto out = to_host(d.out, kQRow);
        for (float x : out)
            if (!std::isfinite(x)) {
                fail("latency leg: non-finite output");
                break;
            }
        release(d);
    }

    std::printf("{\"parity\": {\"num_seqs\": %d, \"max_abs\": %.3g, \"max_rel\": %.3g, \"pool_bit_exact\": %s, "
                "\"two_calls_bit_exact\": %s}, \"latency_us_per_call\": {",
                B, max_abs, max_rel, pool_gpu == pool_o ? "true" : "false",
                (pool_two == pool_gpu && !std::memcmp(out_two.data(), out_gpu.data(), out_gpu.size() * 4))
                    ? "true"
                    : "false");
    for (size_t i = 0; i < sizeof(legs) / sizeof(legs[0]); ++i)
        std::printf("%s\"%s\": {\"splits\": %d, \"device\": %.2f, \"host\": %.2f}", i ? ", " : "", legs[i].name,
                    legs[i].splits, legs[i].device_us, legs[i].host_us);
    std::printf("}, \"failures\": %d}\n", g_failures);
    HIP_OK(hipFree(cos_d));
    HIP_OK(hipFree(sin_d));
    HIP_OK(hipEventDestroy(e0));
    HIP_OK(hipEventDestroy(e1));
    HIP_OK(hipStreamDestroy(stream));
    return g_failures ? 1 : 0;
}
