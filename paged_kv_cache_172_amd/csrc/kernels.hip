// HIP kernels for gfx950 (CDNA4, wave64): decode append and paged decode
// attention over a shared BF16 page pool.
//
// Passages implemented ("Hours of YouTube and 85 handtyped pages of notes on
// LLM Inference - Start here", section "これまでの進捗"):
//   - the bullet on the shared BF16 KV page pool: one block table per
//     sequence and layer, 16 tokens of K and V per physical page, decode
//     adds one token at its absolute RoPE position (append_kernel);
//   - the bullet on paged decode attention: every query head streams its
//     sequence's cached pages with an FP32 online softmax and accumulates
//     weighted V, with no gathered prefix and no stored scores
//     (attn_split_kernel + attn_combine_kernel).
// Decode is bound by memory bandwidth ("Tiny-vLLMでゼロから構築する高性能LLM推論
// エンジン", section "Prefill vs. Decode"), so the attention kernel is shaped
// around HBM reads: 16-byte loads, a prefetch distance of two pages, and no
// matrix cores.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ helpers --

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP lane movement inside 16-lane rows.
constexpr int kDppQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Sum of the four lanes of each quad, on every lane of the quad.
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    return x;
}

// Exchange across 32-lane halves / odd-even rows (v_permlane32_swap /
// v_permlane16_swap).  Returns {new a, new b}.
struct Pair {
    float a, b;
};
__device__ __forceinline__ Pair swap32(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ Pair swap16(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// Max over lanes {i, i^4, i^8, ...}: all 16 quads of the wave (lane bits 2..5).
__device__ __forceinline__ float max_over_quads(float x) {
    x = fmaxf(x, dpp<kDppRowRor4>(x));
    x = fmaxf(x, dpp<kDppRowRor8>(x));
    Pair p = swap16(x, x);
    x = fmaxf(p.a, p.b);
    p = swap32(x, x);
    return fmaxf(p.a, p.b);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T uniform(T x) {
    return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ uint4 load16(const char* base, uint32_t byte_off) {
    return *reinterpret_cast<const uint4*>(base + byte_off);
}

// ------------------------------------------------------------- append --

// Round an FP64 value to the nearest BF16 bit pattern, ties to even, in one
// step from the FP64 bits (no intermediate FP32 rounding).
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double y) {
    const uint64_t u = __double_as_longlong(y);
    const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
    const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
    if (mag > 0x7FF0000000000000ull) return sign | 0x7FC0u;  // NaN
    const int e = (int)(mag >> 52);                          // biased FP64 exponent
    if (e >= 1023 + 128) return sign | 0x7F80u;              // |y| >= 2^128 (or inf)
    const uint64_t sig = (mag & 0x000FFFFFFFFFFFFFull) | (e ? (1ull << 52) : 0ull);
    // Keep `shift` low bits out: 45 for a normal BF16 result (8 significant
    // bits of 53), more below 2^-126 where the BF16 grid step is 2^-133.
    int shift = 45;
    int eb = e - 1023 + 127;                                 // BF16 biased exponent
    if (eb < 1) {
        shift = 45 + (1 - eb);
        eb = 0;
    }
    if (shift >= 54) return sign;                            // below half the smallest subnormal
    uint64_t kept = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    if (rem > half || (rem == half && (kept & 1))) ++kept;
    if (eb == 0) return sign | (uint32_t)kept;               // subnormal (or carried into 0x0080)
    if (kept == 0x100) {                                     // carried into the next binade
        kept = 0x80;
        ++eb;
        if (eb >= 255) return sign | 0x7F80u;
    }
    return sign | ((uint32_t)eb << 7) | ((uint32_t)kept & 0x7Fu);
}

// Rotate 8 pairs (i0+e, i0+e+32), e < 8, of one head vector at table row pos,
// in FP64, and round each result once to BF16.  x1 holds dims i0..i0+7 and x2
// dims i0+32..i0+39 as packed BF16 pairs.
__device__ __forceinline__ void rope8(uint4& x1, uint4& x2, const float* crow, const float* srow) {
    const float4 c0 = *reinterpret_cast<const float4*>(crow);
    const float4 c1 = *reinterpret_cast<const float4*>(crow + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(srow);
    const float4 s1 = *reinterpret_cast<const float4*>(srow + 4);
    const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    uint32_t a[4] = {x1.x, x1.y, x1.z, x1.w};
    uint32_t b[4] = {x2.x, x2.y, x2.z, x2.w};
    uint32_t ya[4], yb[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        uint32_t lo_a = 0, lo_b = 0;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int e = 2 * w + half;
            const double u1 = (double)(half ? bf16_hi(a[w]) : bf16_lo(a[w]));
            const double u2 = (double)(half ? bf16_hi(b[w]) : bf16_lo(b[w]));
            const double c = (double)cs[e];
            const double s = (double)sn[e];
            // Both products are exact in FP64 (8 x 24 significant bits), so
            // each line rounds once, whatever the compiler contracts.
            const uint32_t r1 = f64_to_bf16_rne(u1 * c - u2 * s);
            const uint32_t r2 = f64_to_bf16_rne(u2 * c + u1 * s);
            lo_a |= r1 << (16 * half);
            lo_b |= r2 << (16 * half);
        }
        ya[w] = lo_a;
        yb[w] = lo_b;
    }
    x1 = make_uint4(ya[0], ya[1], ya[2], ya[3]);
    x2 = make_uint4(yb[0], yb[1], yb[2], yb[3]);
}

// One block per sequence, 256 threads:
//   threads   0..127  rotate q: head tid/4, pairs (tid%4)*8 .. +7
//   threads 128..159  rotate k: head (tid-128)/4, written to the page slot
//   threads 160..223  copy v: 16 bytes each, written to the page slot
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int s = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = p.context_lens[s];
    if (n < 1) return;
    const int pos = n - 1;
    if (pos >= p.max_pos) return;                 // outside the RoPE table: not dereferenced
    const int64_t j = pos >> 4;
    const int slot = pos & 15;
    if (j >= p.bt_stride) return;
    const int64_t page = p.block_table[(int64_t)s * p.bt_stride + j];
    const bool page_ok = page >= 0 && page < p.num_pages;
    const float* crow = p.rope_cos + (int64_t)pos * 32;
    const float* srow = p.rope_sin + (int64_t)pos * 32;
    if (tid < 128) {
        const int h = tid >> 2, i0 = (tid & 3) * 8;
        uint16_t* base = p.q + (int64_t)s * p.q_stride + h * kHeadDim;
        uint4 x1 = *reinterpret_cast<const uint4*>(base + i0);
        uint4 x2 = *reinterpret_cast<const uint4*>(base + i0 + 32);
        rope8(x1, x2, crow + i0, srow + i0);
        *reinterpret_cast<uint4*>(base + i0) = x1;
        *reinterpret_cast<uint4*>(base + i0 + 32) = x2;
    } else if (tid < 160) {
        if (!page_ok) return;
        const int g = (tid - 128) >> 2, i0 = ((tid - 128) & 3) * 8;
        const uint16_t* src = p.k_new + (int64_t)s * p.k_stride + g * kHeadDim;
        uint4 x1 = *reinterpret_cast<const uint4*>(src + i0);
        uint4 x2 = *reinterpret_cast<const uint4*>(src + i0 + 32);
        rope8(x1, x2, crow + i0, srow + i0);
        uint16_t* dst = p.k_pool + page * p.page_stride + g * p.head_stride + slot * p.slot_stride;
        *reinterpret_cast<uint4*>(dst + i0) = x1;
        *reinterpret_cast<uint4*>(dst + i0 + 32) = x2;
    } else if (tid < 224) {
        if (!page_ok) return;
        const int chunk = tid - 160, g = chunk >> 3, d0 = (chunk & 7) * 8;
        const uint4 v = *reinterpret_cast<const uint4*>(p.v_new + (int64_t)s * p.v_stride +
                                                        g * kHeadDim + d0);
        uint16_t* dst = p.v_pool + page * p.page_stride + g * p.head_stride + slot * p.slot_stride;
        *reinterpret_cast<uint4*>(dst + d0) = v;
    }
}

// ---------------------------------------------------------- attention --
//
// One wavefront per work unit (sequence s, KV head g, chunk c); it serves the
// 4 query heads 4g..4g+3.  Inside a page the 64 lanes are 16 quads: quad t
// (lanes 4t..4t+3) owns token slot t, and lane quarter c4 = lane%4 owns dims
// [8*c4, 8*c4+8) and [32+8*c4, 32+8*c4+8) of that token's K and V row (two
// 16-byte loads each; four consecutive lanes read 64 contiguous bytes).
//
// Per page: QK^T is 8 v_dot2_f32_bf16 per head per lane plus a 2-step DPP
// quad sum; every quad then runs its own FP32 online softmax over the tokens
// it owns (slot t of every page of the chunk), with a running maximum that is
// raised only when a logit exceeds it by more than kRescaleSlack (base-2
// units; values p = 2^(x - m) stay below 2^kRescaleSlack, so nothing
// overflows).  At the end of the chunk the 16 quads are merged with the
// log-sum-exp rule through permlane swaps and DPP, and the wave writes one
// partial (max, sum, 64-wide accumulator) per query head, or the normalised
// output when the plan has a single chunk.

constexpr float kRescaleSlack = 8.0f;
constexpr int kWavesPerBlock = 4;
#ifndef PKV_SPLIT_WAVES_PER_EU
#define PKV_SPLIT_WAVES_PER_EU 3
#endif

struct PageRegs {
    uint4 ka, kb, va, vb;
};

struct SoftmaxState {
    float m[kGroup];
    float l[kGroup];
    float acc[kGroup][16];
};

__device__ __forceinline__ PageRegs load_page(const char* kbase, const char* vbase,
                                              uint32_t off_a, uint32_t off_b) {
    PageRegs r;
    r.ka = load16(kbase, off_a);
    r.kb = load16(kbase, off_b);
    r.va = load16(vbase, off_a);
    r.vb = load16(vbase, off_b);
    return r;
}

template <bool kMasked>
__device__ __forceinline__ void consume_page(PageRegs pg, const uint4 (&qa)[kGroup],
                                             const uint4 (&qb)[kGroup], float scale_log2,
                                             bool valid, SoftmaxState& st) {
    float x[kGroup];
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
        float s0 = dot2_bf16(qa[r].x, pg.ka.x, 0.0f);
        float s1 = dot2_bf16(qb[r].x, pg.kb.x, 0.0f);
        s0 = dot2_bf16(qa[r].y, pg.ka.y, s0);
        s1 = dot2_bf16(qb[r].y, pg.kb.y, s1);
        s0 = dot2_bf16(qa[r].z, pg.ka.z, s0);
        s1 = dot2_bf16(qb[r].z, pg.kb.z, s1);
        s0 = dot2_bf16(qa[r].w, pg.ka.w, s0);
        s1 = dot2_bf16(qb[r].w, pg.kb.w, s1);
        x[r] = s0 + s1;
    }
#pragma unroll
    for (int r = 0; r < kGroup; ++r) x[r] = quad_sum(x[r]) * scale_log2;
    if (kMasked) {
#pragma unroll
        for (int r = 0; r < kGroup; ++r) x[r] = valid ? x[r] : -INFINITY;
        pg.va = valid ? pg.va : make_uint4(0, 0, 0, 0);
        pg.vb = valid ? pg.vb : make_uint4(0, 0, 0, 0);
    }
    // Largest excess of a new logit over its running maximum (NaN-free: a
    // masked logit is -inf and m is finite or -inf, and -inf - -inf only
    // occurs for a masked slot whose quad has seen nothing, which excess
    // ignores because fmaxf drops the NaN).
    float excess = x[0] - st.m[0];
#pragma unroll
    for (int r = 1; r < kGroup; ++r) excess = fmaxf(excess, x[r] - st.m[r]);
    if (__builtin_amdgcn_ballot_w64(excess > kRescaleSlack)) {
#pragma unroll
        for (int r = 0; r < kGroup; ++r) {
            // Only heads whose logit jumped rescale; the others keep alpha = 1
            // (their m may still be -inf, and -inf - -inf must not be formed).
            const bool up = x[r] > st.m[r] + kRescaleSlack;  // x finite here
            const float alpha = up ? exp2_fast(st.m[r] - x[r]) : 1.0f;  // 0 when m was -inf
            st.l[r] *= alpha;
#pragma unroll
            for (int k = 0; k < 16; ++k) st.acc[r][k] *= alpha;
            st.m[r] = up ? x[r] : st.m[r];
        }
    }
    const uint32_t vw[8] = {pg.va.x, pg.va.y, pg.va.z, pg.va.w, pg.vb.x, pg.vb.y, pg.vb.z, pg.vb.w};
    float vf[16];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        vf[2 * w] = bf16_lo(vw[w]);
        vf[2 * w + 1] = bf16_hi(vw[w]);
    }
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
        float pr = exp2_fast(x[r] - st.m[r]);
        if (kMasked) pr = valid ? pr : 0.0f;
        st.l[r] += pr;
#pragma unroll
        for (int k = 0; k < 16; ++k) st.acc[r][k] = fmaf(pr, vf[k], st.acc[r][k]);
    }
}

__global__ __launch_bounds__(kWavesPerBlock * 64) __attribute__((amdgpu_waves_per_eu(PKV_SPLIT_WAVES_PER_EU)))
void attn_split_kernel(AttnParams p) {
    const int lane = threadIdx.x & 63;
    const int wave = uniform((int)(threadIdx.x >> 6));
    const int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + wave;  // g fastest, then s, then c
    const int g = (int)(unit % kKVHeads);
    const int64_t sc = unit / kKVHeads;
    const int s = (int)(sc % p.num_seqs);
    const int c = (int)(sc / p.num_seqs);
    if (c >= p.plan.splits) return;

    int n = uniform(p.context_lens[s]);
    n = n < p.max_context_len ? n : p.max_context_len;
    const int np = n > 0 ? (n + kPageTokens - 1) / kPageTokens : 0;
    const int pb = c * p.plan.pages_per_split;
    const int pe = min(pb + p.plan.pages_per_split, np);

    const int t = lane >> 2;   // token slot owned by this lane's quad
    const int c4 = lane & 3;   // dim quarter owned inside the quad
    const bool single = p.plan.splits == 1;

    if (pb >= pe) {            // empty chunk: only a zero-length context needs a write
        if (single) {
            float* orow = p.out + (int64_t)s * p.out_stride + (kGroup * g) * kHeadDim;
            *reinterpret_cast<float4*>(orow + lane * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }

    // This chunk's table entries, one per lane (at most 128 pages per chunk).
    const int32_t* bt_row = p.block_table + (int64_t)s * p.bt_stride + pb;
    const int cnt = pe - pb;
    const int32_t tbl0 = lane < cnt ? bt_row[lane] : 0;
    const int32_t tbl1 = lane + 64 < cnt ? bt_row[lane + 64] : 0;

    // q of the 4 query heads, this lane's 16 dims, as packed BF16 pairs.
    uint4 qa[kGroup], qb[kGroup];
    const uint16_t* qrow = p.q + (int64_t)s * p.q_stride + (kGroup * g) * kHeadDim;
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
        qa[r] = *reinterpret_cast<const uint4*>(qrow + r * kHeadDim + c4 * 8);
        qb[r] = *reinterpret_cast<const uint4*>(qrow + r * kHeadDim + 32 + c4 * 8);
    }

    const uint32_t off_a = (uint32_t)((t * p.slot_stride + c4 * 8) * 2);
    const uint32_t off_b = off_a + 64;
    const char* kpool = reinterpret_cast<const char*>(p.k_pool) + (int64_t)g * p.head_stride * 2;
    const char* vpool = reinterpret_cast<const char*>(p.v_pool) + (int64_t)g * p.head_stride * 2;
    const int64_t page_bytes = p.page_stride * 2;
    bool bad_page = false;

    auto page_base = [&](int j, const char*& kb, const char*& vb) {
        const int idx = j - pb;
        int32_t phys = idx < 64 ? __builtin_amdgcn_readlane(tbl0, idx)
                                : __builtin_amdgcn_readlane(tbl1, idx - 64);
        if (phys < 0 || phys >= p.num_pages) {  // never dereference a bad entry
            bad_page = true;
            phys = 0;
        }
        kb = kpool + (int64_t)phys * page_bytes;
        vb = vpool + (int64_t)phys * page_bytes;
    };

    SoftmaxState st;
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
        st.m[r] = -INFINITY;
        st.l[r] = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k) st.acc[r][k] = 0.0f;
    }
    const float sl2 = p.scale_log2;

    // Pages pb .. pe-1 with two pages in flight ahead of the one consumed.
    const char *kb, *vb;
    page_base(pb, kb, vb);
    PageRegs cur = load_page(kb, vb, off_a, off_b);
    PageRegs nxt = cur;
    if (pb + 1 < pe) {
        page_base(pb + 1, kb, vb);
        nxt = load_page(kb, vb, off_a, off_b);
    }
    int j = pb;
    for (; j + 2 < pe; ++j) {
        page_base(j + 2, kb, vb);
        PageRegs nn = load_page(kb, vb, off_a, off_b);
        consume_page<false>(cur, qa, qb, sl2, true, st);
        cur = nxt;
        nxt = nn;
    }
    if (j + 1 < pe) {
        consume_page<false>(cur, qa, qb, sl2, true, st);
        cur = nxt;
        ++j;
    }
    // Last page of the chunk: the only one that can hold slots past n.
    const int valid_tokens = n - j * kPageTokens;
    consume_page<true>(cur, qa, qb, sl2, t < valid_tokens, st);

    // ---- merge the 16 quads of the wave (log-sum-exp rule) ----
    float M[kGroup];
#pragma unroll
    for (int r = 0; r < kGroup; ++r) M[r] = max_over_quads(st.m[r]);  // finite: slot 0 is valid
#pragma unroll
    for (int r = 0; r < kGroup; ++r) {
        const float alpha = st.m[r] == -INFINITY ? 0.0f : exp2_fast(st.m[r] - M[r]);
        st.l[r] *= alpha;
#pragma unroll
        for (int k = 0; k < 16; ++k) st.acc[r][k] *= alpha;
    }
    // Sum over lane bit 5 (permlane32 swap): lanes 0..31 keep heads 0/1, 32..63 heads 2/3;
    // then over lane bit 4 (permlane16 swap): row R (lanes 16R..16R+15) keeps head R.
    float u[16];
    float lsum;
    {
        float t0[16], t1[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            Pair a = swap32(st.acc[0][k], st.acc[2][k]);
            t0[k] = a.a + a.b;
            Pair b = swap32(st.acc[1][k], st.acc[3][k]);
            t1[k] = b.a + b.b;
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            Pair a = swap16(t0[k], t1[k]);
            u[k] = a.a + a.b;
        }
        Pair la = swap32(st.l[0], st.l[2]);
        Pair lb = swap32(st.l[1], st.l[3]);
        Pair lc = swap16(la.a + la.b, lb.a + lb.b);
        lsum = lc.a + lc.b;
    }
    // Sum over lane bits 2..3 (the 4 quads of a row) with DPP row rotations.
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        u[k] += dpp<kDppRowRor4>(u[k]);
        u[k] += dpp<kDppRowRor8>(u[k]);
    }
    lsum += dpp<kDppRowRor4>(lsum);
    lsum += dpp<kDppRowRor8>(lsum);

    const int row = lane >> 4;              // query head 4g + row
    const int qd = (lane >> 2) & 3;         // which 4 of the lane's 16 values it stores
    float mrow = M[0];
    mrow = row == 1 ? M[1] : mrow;
    mrow = row == 2 ? M[2] : mrow;
    mrow = row == 3 ? M[3] : mrow;
    float4 v4;
    v4.x = qd == 0 ? u[0] : qd == 1 ? u[4] : qd == 2 ? u[8] : u[12];
    v4.y = qd == 0 ? u[1] : qd == 1 ? u[5] : qd == 2 ? u[9] : u[13];
    v4.z = qd == 0 ? u[2] : qd == 1 ? u[6] : qd == 2 ? u[10] : u[14];
    v4.w = qd == 0 ? u[3] : qd == 1 ? u[7] : qd == 2 ? u[11] : u[15];
    const int dim0 = c4 * 8 + (qd & 1) * 4 + (qd >> 1) * 32;
    const int h = kGroup * g + row;
    if (bad_page) lsum = NAN;
    if (single) {
        const float inv = 1.0f / lsum;
        float* orow = p.out + (int64_t)s * p.out_stride + h * kHeadDim;
        *reinterpret_cast<float4*>(orow + dim0) =
            make_float4(v4.x * inv, v4.y * inv, v4.z * inv, v4.w * inv);
    } else {
        const int64_t slot_idx = ((int64_t)s * kQHeads + h) * p.plan.splits + c;
        *reinterpret_cast<float4*>(p.ws_acc + slot_idx * kHeadDim + dim0) = v4;
        if ((lane & 15) == 0) p.ws_ml[slot_idx] = make_float2(mrow, lsum);
    }
}

// One thread per (sequence, query head, 4 output dims).
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int d4 = (int)(tid & 15);
    const int h = (int)((tid >> 4) & 31);
    const int64_t s = tid >> 9;
    if (s >= p.num_seqs) return;
    int n = p.context_lens[s];
    n = n < p.max_context_len ? n : p.max_context_len;
    const int np = n > 0 ? (n + kPageTokens - 1) / kPageTokens : 0;
    const int S = p.plan.splits;
    const int nc = (np + p.plan.pages_per_split - 1) / p.plan.pages_per_split;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (nc > 0) {
        const int64_t base = ((int64_t)s * kQHeads + h) * S;
        float M = -INFINITY;
        for (int c = 0; c < nc; ++c) M = fmaxf(M, p.ws_ml[base + c].x);
        float L = 0.0f;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int c = 0; c < nc; ++c) {
            const float2 ml = p.ws_ml[base + c];
            const float w = ml.x == -INFINITY ? 0.0f : exp2_fast(ml.x - M);
            const float4 v = *reinterpret_cast<const float4*>(p.ws_acc + (base + c) * kHeadDim + d4 * 4);
            L = fmaf(w, ml.y, L);
            a.x = fmaf(w, v.x, a.x);
            a.y = fmaf(w, v.y, a.y);
            a.z = fmaf(w, v.z, a.z);
            a.w = fmaf(w, v.w, a.w);
        }
        const float inv = 1.0f / L;
        o = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    }
    *reinterpret_cast<float4*>(p.out + s * p.out_stride + h * kHeadDim + d4 * 4) = o;
}

}  // namespace

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(append_kernel, dim3(p.num_seqs), dim3(256), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_split(const AttnParams& p, hipStream_t stream) {
    const int64_t units = (int64_t)p.num_seqs * kKVHeads * p.plan.splits;
    const int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(attn_split_kernel, dim3((unsigned)blocks), dim3(kWavesPerBlock * 64), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnParams& p, hipStream_t stream) {
    const int64_t threads = (int64_t)p.num_seqs * kQHeads * 16;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
