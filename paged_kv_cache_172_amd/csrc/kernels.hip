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
// around HBM reads: 16-byte loads and a prefetch distance of two pages.  The
// two contractions of a page, Q K^T of the 4 query heads and the weighted
// sum of V over its 16 tokens, run on the matrix cores to take work off the
// vector ALUs; the softmax is FP32, its weights enter the V product as two
// BF16 terms each, and every sum is FP32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

namespace pkv {
namespace {


// ------------------------------------------------------------ helpers --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// DPP lane movement inside 16-lane rows.
constexpr int kDppRowRor4 = 0x124;
constexpr int kDppRowRor8 = 0x128;
constexpr int kDppQuadBcast0 = 0x00;  // quad_perm [0,0,0,0]: lane 0 of each quad to all 4
constexpr int kDppQuadBcast1 = 0x55;  // quad_perm [1,1,1,1]
constexpr int kDppQuadBcast2 = 0xAA;  // quad_perm [2,2,2,2]
constexpr int kDppQuadBcast3 = 0xFF;  // quad_perm [3,3,3,3]
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}

// Max / sum across the 4 rows of 16 lanes (lane bits 4 and 5), with
// v_permlane16_swap and v_permlane32_swap.
__device__ __forceinline__ float cross_rows_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float cross_rows_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ T uniform(T x) {
    return __builtin_amdgcn_readfirstlane(x);
}

// ------------------------------------------------------------- append --

// Round an FP64 value to the nearest BF16 bit pattern, ties to even, without
// branches.  Step 1 rounds to FP32 "to odd": the FP32 value toward zero,
// with its last bit set when anything was cut off.  Step 2 rounds that to
// BF16 to nearest, ties to even.  FP32 carries 24 significant bits, more than
// BF16's 8 + 2, so the two steps give the single rounding's result (Boldo and
// Melquiond, "When double rounding is odd", 2005); the same holds on the
// subnormal grids (2^-149 against 2^-133) and for overflow (FP32 max rounds
// to infinity).  NaN gives the sign with the quiet pattern 0x7FC0.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double y) {
    const float f = (float)y;                         // nearest FP32 (FP32 denormals kept)
    const double back = (double)f;
    uint32_t b = __float_as_uint(f);
    b -= fabs(back) > fabs(y) ? 1u : 0u;              // rounded away from zero: step back
    b |= back != y ? 1u : 0u;                         // sticky bit
    const uint32_t r = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    const uint32_t sign = (uint32_t)(__double_as_longlong(y) >> 48) & 0x8000u;
    return y != y ? sign | 0x7FC0u : r;
}

// The BF16 bits of the nearest value to y, ties to even, for |y| in
// [2^-126, (2 - 2^-8) 2^127): results that are normal BF16 numbers.  It works
// on the high word of y's FP64 bits with the low word folded into its last
// bit (only "nonzero" matters below the rounding bit): add the half-way bias
// below the 7 kept mantissa bits, and rebias the exponent from 1023 to 127
// (896 << 20, a multiple of the 2^13 cut, is subtracted before the shift).
// ok is cleared when y lies outside that range.
__device__ __forceinline__ uint32_t f64_to_bf16_normal(double y, bool& ok) {
    const uint64_t u = __double_as_longlong(y);
    const uint32_t hi = (uint32_t)(u >> 32);
    const uint32_t mag = (hi & 0x7FFFFFFFu) | min((uint32_t)u, 1u);
    ok = ok && mag - 0x38100000u < 0x47EFF000u - 0x38100000u;
    const uint32_t r = (mag + (0xFFFu - 0x38000000u) + ((mag >> 13) & 1u)) >> 13;
    return r | ((hi >> 16) & 0x8000u);
}

// One rotated element in FP32, u*c - v*s: p = v*s rounded and its exact
// error e (an FMA); r = u*c - p rounded; y = r - e rounded.  Then
// |y - (u c - v s)| <= ulp(r)/2 + ulp(y)/2 + 2^-150 (the last term if e
// underflowed; FP32 denormals are kept, as these kernels are compiled), at
// most 2 ulp(y) when |r| <= 2|y| and y is normal.  y then
// rounds to BF16 as the exact value (and its FP64 rounding) does when y lies
// at least 3 FP32 ulps from every BF16 half-way point: its low 16 bits
// outside 0x8000 +- 2 (points across a binade edge lie 2^15 ulps away or
// more).  The caller folds the three conditions over its elements:
//   margin: the minimum of (bits(y) << 16) + 0x80020000 is >= 5 << 16;
//   slack:  the minimum of 2|y| - |r| is >= 0 (its sign is exact: both are
//           on the 2^-149 grid, so a nonzero difference never rounds to 0);
//   normal: every y is a normal number.
struct RotCheck {
    uint32_t margin = 0xFFFFFFFFu;
    float slack = INFINITY;
    bool normal = true;
};
__device__ __forceinline__ float rot_f32(float u, float c, float v, float s, RotCheck& k) {
#pragma clang fp contract(off)
    const float p = v * s;
    const float e = __builtin_fmaf(v, s, -p);
    const float r = __builtin_fmaf(u, c, -p);
    const float y = r - e;
    k.margin = min(k.margin, (__float_as_uint(y) << 16) + 0x80020000u);
    k.slack = fminf(k.slack, __builtin_fmaf(2.0f, fabsf(y), -fabsf(r)));
    k.normal = k.normal && __builtin_isnormal(y);
    return y;
}

// Rotate the 4 pairs (i0+e, i0+e+32), e < 4, of one head vector with the
// table row of the new token's position, and round each result once to BF16
// as from its FP64 value.  x1 holds dims i0..i0+3 and x2 dims i0+32..i0+35
// as BF16 pairs.  Three paths, chosen for the whole wave: FP32 with a
// certainty test (rot_f32); FP64 with the normal-range rounding;
// FP64 with the general rounding.  Where more than one applies they give
// the same bits.
__device__ __forceinline__ void rope4(uint2& x1, uint2& x2, float4 c, float4 sn) {
    const uint32_t a[2] = {x1.x, x1.y};
    const uint32_t b[2] = {x2.x, x2.y};
    const float cs[4] = {c.x, c.y, c.z, c.w};
    const float ss[4] = {sn.x, sn.y, sn.z, sn.w};
    float u1[4], u2[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        u1[e] = (e & 1) ? bf16_hi(a[e >> 1]) : bf16_lo(a[e >> 1]);
        u2[e] = (e & 1) ? bf16_hi(b[e >> 1]) : bf16_lo(b[e >> 1]);
    }
    RotCheck k;
    f32x4_t fa, fb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        fa[e] = rot_f32(u1[e], cs[e], u2[e], ss[e], k);      // u1 c - u2 s
        fb[e] = rot_f32(u2[e], cs[e], -u1[e], ss[e], k);     // u2 c + u1 s
    }
    const bool certain = k.normal && k.margin >= 0x50000u && k.slack >= 0.0f;
    if (__builtin_amdgcn_ballot_w64(!certain) == 0) {   // wave-uniform
        const uint2 ba = __builtin_bit_cast(uint2, __builtin_convertvector(fa, bf16x4_t));
        const uint2 bb = __builtin_bit_cast(uint2, __builtin_convertvector(fb, bf16x4_t));
        x1 = ba;
        x2 = bb;
        return;
    }
    double ya[4], yb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double d1 = (double)u1[e], d2 = (double)u2[e];
        const double cc = (double)cs[e], s = (double)ss[e];
        // Both products are exact in FP64 (8 x 24 significant bits), so
        // each line rounds once, whatever the compiler contracts.
        ya[e] = d1 * cc - d2 * s;
        yb[e] = d2 * cc + d1 * s;
    }
    uint32_t ra[4], rb[4];
    bool ok = true;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ra[e] = f64_to_bf16_normal(ya[e], ok);
        rb[e] = f64_to_bf16_normal(yb[e], ok);
    }
    if (__builtin_amdgcn_ballot_w64(!ok) != 0) {   // wave-uniform
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ra[e] = f64_to_bf16_rne(ya[e]);
            rb[e] = f64_to_bf16_rne(yb[e]);
        }
    }
    x1 = make_uint2(ra[0] | (ra[1] << 16), ra[2] | (ra[3] << 16));
    x2 = make_uint2(rb[0] | (rb[1] << 16), rb[2] | (rb[3] << 16));
}

// Three 128-thread blocks per group of appended rows; a task is 4 rotation
// pairs of one head (or 16 bytes of V), the same task for every row of the
// group:
//   blocks 0, 1: q tasks 0..255 (head task/8, pairs (task%8)*4 .. +3)
//   block 2:     threads 0..63 k tasks (head t/8), threads 64..127 copy V.
// A prefill without q runs only block 2 of each group.  A block takes kRows
// consecutive rows: it finds their sequences and positions once (one
// binary search, then a walk), requests the inputs of all of them, and then
// rotates and stores row by row, so the latency of those lookups and loads
// is paid once per group.
constexpr int kAppendThreads = 128;
constexpr int kAppendBlocksPerToken = 3;
#ifndef PKV_PREFILL_ROWS
#define PKV_PREFILL_ROWS 2
#endif
constexpr int kPrefillRows = PKV_PREFILL_ROWS;

// Where one appended row comes from and goes to.
struct TokenSite {
    int seq;   // sequence (block-table row)
    int row;   // row of q / k / v
    int pos;   // absolute position; < 0: nothing to do
};

// Decode: sequence s appends its token at position context_lens[s] - 1.
template <int kRows>
__device__ __forceinline__ void find_sites(const AppendParams& p, int first, TokenSite (&site)[kRows]) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int t = first + r;
        site[r] = t < p.num_seqs ? TokenSite{t, t, p.context_lens[t] - 1} : TokenSite{0, 0, -1};
    }
}

// Prefill: packed row t belongs to the sequence s with cu_tokens[s] <= t <
// cu_tokens[s+1] and sits at position start_pos[s] + t - cu_tokens[s].  The
// first row's sequence comes from a binary search over the num_seqs + 1
// offsets, the next rows' from walking forward (skipping empty sequences).
template <int kRows>
__device__ __forceinline__ void find_sites(const PrefillParams& p, int first, TokenSite (&site)[kRows]) {
    int lo = 0, hi = p.num_seqs;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_tokens[mid + 1] <= first) lo = mid + 1;
        else hi = mid;
    }
    int s = lo;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int t = first + r;
        while (s < p.num_seqs && p.cu_tokens[s + 1] <= t) ++s;
        const bool ok = t < p.total_tokens && s < p.num_seqs && p.cu_tokens[s] <= t;
        site[r] = ok ? TokenSite{s, t, p.start_pos[s] + (t - p.cu_tokens[s])} : TokenSite{0, 0, -1};
    }
}

template <int kRows, typename Params>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(Params p) {
    const int parts = p.q ? kAppendBlocksPerToken : 1;
    const int group = (int)(blockIdx.x / (unsigned)parts);
    const int part = p.q ? (int)(blockIdx.x % (unsigned)parts) : 2;
    const int tid = threadIdx.x;
    const bool is_v = part == 2 && tid >= 64;
    TokenSite site[kRows];
    find_sites<kRows>(p, group * kRows, site);
    // head-vector base and pair offset of this thread's task
    int head, i0;
    const uint16_t* base;
    int64_t stride;
    if (part < 2) {
        const int task = part * kAppendThreads + tid;
        head = task >> 3;
        i0 = (task & 7) * 4;
        base = p.q + head * kHeadDim;
        stride = p.q_stride;
    } else if (!is_v) {
        head = tid >> 3;
        i0 = (tid & 7) * 4;
        base = p.k_new + head * kHeadDim;
        stride = p.k_stride;
    } else {
        head = (tid - 64) >> 3;
        i0 = ((tid - 64) & 7) * 8;
        base = p.v_new + head * kHeadDim;
        stride = p.v_stride;
    }
    // Requests first: the row inputs, the table rows and the page ids.
    uint2 x1[kRows], x2[kRows];
    uint4 vrow[kRows];
    float4 c[kRows], sn[kRows];
    int64_t page[kRows];
    bool go[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int pos = site[r].pos;
        // outside the RoPE table, or no row: nothing is read or written
        go[r] = pos >= 0 && pos < p.max_pos;
        x1[r] = x2[r] = make_uint2(0, 0);
        vrow[r] = make_uint4(0, 0, 0, 0);
        c[r] = sn[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        page[r] = -1;
        if (!go[r]) continue;
        const uint16_t* src = base + (int64_t)site[r].row * stride;
        if (is_v) {
            vrow[r] = *reinterpret_cast<const uint4*>(src + i0);
        } else {
            x1[r] = *reinterpret_cast<const uint2*>(src + i0);
            x2[r] = *reinterpret_cast<const uint2*>(src + i0 + 32);
            c[r] = *reinterpret_cast<const float4*>(p.rope_cos + (int64_t)pos * 32 + i0);
            sn[r] = *reinterpret_cast<const float4*>(p.rope_sin + (int64_t)pos * 32 + i0);
        }
        if (part == 2) {
            const int64_t j = pos >> 4;
            if (j < p.bt_stride) page[r] = p.block_table[(int64_t)site[r].seq * p.bt_stride + j];
        }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        if (!go[r]) continue;
        const int slot = site[r].pos & 15;
        // never write through a bad entry (q is still rotated)
        const bool to_page = page[r] >= 0 && page[r] < p.num_pages;
        const int64_t dst_off = page[r] * p.page_stride + head * p.head_stride + slot * p.slot_stride;
        if (is_v) {
            if (to_page) *reinterpret_cast<uint4*>(p.v_pool + dst_off + i0) = vrow[r];
            continue;
        }
        uint2 y1 = x1[r], y2 = x2[r];
        rope4(y1, y2, c[r], sn[r]);
        uint16_t* dst;
        if (part < 2) {
            dst = const_cast<uint16_t*>(base) + (int64_t)site[r].row * stride;
        } else {
            if (!to_page) continue;
            dst = p.k_pool + dst_off;
        }
        *reinterpret_cast<uint2*>(dst + i0) = y1;
        *reinterpret_cast<uint2*>(dst + i0 + 32) = y2;
    }
}

// --------------------------------------------------------- page copy --
//
// Copy-on-write of shared prefix pages: block i copies all of page src[i]
// (K and V, every head, slot and dim, through the pool strides) to page
// dst[i], 16 bytes per thread-step.  Pairs with an id outside the pool are
// skipped.
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_pages_kernel(CopyParams p) {
    const int i = blockIdx.x;
    const int64_t src = p.src[i];
    const int64_t dst = p.dst[i];
    if (src < 0 || src >= p.num_pages || dst < 0 || dst >= p.num_pages) return;
    // 8 heads x 16 slots x 8 chunks of 8 BF16, for K then V
    constexpr int kChunks = kKVHeads * kPageTokens * (kHeadDim / 8);
    for (int c = threadIdx.x; c < 2 * kChunks; c += kCopyThreads) {
        const int half = c / kChunks;
        const int r = c % kChunks;
        const int g = r / (kPageTokens * 8);
        const int t = (r / 8) % kPageTokens;
        const int d = (r % 8) * 8;
        const int64_t off = g * p.head_stride + t * p.slot_stride + d;
        uint16_t* base = half ? p.v_pool : p.k_pool;
        *reinterpret_cast<uint4*>(base + dst * p.page_stride + off) =
            *reinterpret_cast<const uint4*>(base + src * p.page_stride + off);
    }
}

// ---------------------------------------------------------- attention --
//
// One workgroup of 4 wavefronts per (sequence s, KV head g, outer chunk ci);
// it serves the 4 query heads 4g..4g+3.  The sequence's np pages are cut into
// 4*S chunks of ceil(np / (4*S)) pages and wave w takes chunk 4*ci + w, so the
// chunk boundaries follow each sequence's own length.  Inside a page, lane l
// loads the dims [8*c4, 8*c4+8) and [32+8*c4, 32+8*c4+8), c4 = l >> 4, of
// token slot l & 15's K row, the layout of the matrix-core operand below, and
// the same dims, c4 = l & 3, of token slot l >> 2's V row, so that 4
// consecutive lanes read 64 contiguous bytes (V passes through LDS anyway;
// for pages in cache that halves the time).
//
// Per page (consume_page): S^T = K Q^T is two v_mfma_f32_16x16x32_bf16, the
// page's K being the A operand as loaded, which leaves lane l with head
// l & 3's logits of tokens 4*c4 .. 4*c4+3.  The FP32 online softmax keeps one
// running maximum per head for the whole wave, raised only when a logit
// exceeds it by more than kRescaleSlack (base-2 units; values p = 2^(x - m)
// stay below 2^kRescaleSlack, so nothing overflows).  The lane's 4 weights
// are exactly the A operand of a v_mfma_f32_16x16x16_bf16 over the page's 16
// tokens; V reaches the B operand through the wave's LDS tile and the
// transposing read ds_read_b64_tr_b16, and the product sums over the tokens
// inside the matrix core.  So at the end of a chunk only the 4 lane rows'
// weight sums need adding; the 4 waves of the workgroup are merged with the
// log-sum-exp rule through LDS, and the workgroup writes the normalised
// output (S = 1) or one partial (max, sum, 64-wide accumulator) per query
// head for the combine kernel (S > 1).

constexpr float kRescaleSlack = 8.0f;
#ifndef PKV_RING
#define PKV_RING 3
#endif
constexpr int kRing = PKV_RING;  // page buffers per wave: kRing-1 pages in flight
static_assert(kRing >= 2 && kRing <= 8, "ring size");
#ifndef PKV_SPLIT_WAVES_PER_EU
#define PKV_SPLIT_WAVES_PER_EU 3
#endif

struct PageRegs {
    uint4 ka, kb, va, vb;
};

// A wave's running state.  Lane l serves query head l & 3 for the logits
// and the weights (tokens 4c..4c+3 of each page, c = l >> 4), and holds the
// weighted V sums of all 4 heads for dims 16T + (l & 15) (the same on the 4
// lane groups c).
struct WaveState {
    float m;          // running maximum (base 2) of head l & 3, the same on all its lanes
    float l;          // sum of this lane's weights (its 4 tokens of every page so far)
    f32x4_t o[4];     // o[T][i]: head i, dim 16T + (l & 15)
};

// Buffer descriptor for one (page, KV head) tile: 48-bit base, raw
// (stride 0), `bytes` of range.  A descriptor with 0 bytes turns the load
// into a no-op that returns zeros without touching memory, which is how
// prefetches past the end of a chunk are issued without branches.
constexpr int32_t kBufferWord3 = 0x00020000;  // gfx9-family raw buffer format
constexpr int kStoreNonTemporal = 2;          // cache policy bit "nt" of a buffer store

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kBufferWord3);
}

#ifndef PKV_LOAD_POLICY
#define PKV_LOAD_POLICY 0
#endif
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, PKV_LOAD_POLICY);
    return __builtin_bit_cast(uint4, v);
}

__device__ __forceinline__ PageRegs load_page(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                              uint32_t k_off, uint32_t v_off) {
    PageRegs r;
    r.ka = buffer_load16(kr, k_off);
    r.kb = buffer_load16(kr, k_off + 64);
    r.va = buffer_load16(vr, v_off);
    r.vb = buffer_load16(vr, v_off + 64);
    return r;
}

// Up to 8 page buffers addressed only by compile-time indices, so they live
// in VGPRs (an array indexed in a loop with an early exit can end up in
// scratch memory).
struct PageRing {
    PageRegs s0, s1, s2, s3, s4, s5, s6, s7;
    template <int I>
    __device__ __forceinline__ PageRegs& at() {
        static_assert(I >= 0 && I < 8, "ring slot");
        if constexpr (I == 0) return s0;
        else if constexpr (I == 1) return s1;
        else if constexpr (I == 2) return s2;
        else if constexpr (I == 3) return s3;
        else if constexpr (I == 4) return s4;
        else if constexpr (I == 5) return s5;
        else if constexpr (I == 6) return s6;
        else return s7;
    }
};

struct QRegs {
    bf16x8_t a, b;   // B operands: query head (lane & 3), dims 8c..8c+7 / 32+8c..32+8c+7
};

// Where a wave keeps the page it consumes in LDS (BF16 rows padded to
// kTileRow, so that the 64 lanes of a store or a transposing read spread
// over the banks), and the lane's offsets into it.
constexpr int kTileRow = kHeadDim + 8;
struct PageCtx {
    uint16_t* vt;        // this wave's V tile [16 tokens][kTileRow]
    uint16_t* kt;        // this wave's K tile (fused kernel only)
    int w_off;           // V as loaded: row l >> 2, dims 8(l & 3).. (+32 for the second half)
    int k_off;           // K as the MFMA takes it: row l & 15, dims 8c.. (+32)
    int tr_off;          // row 4c + j/4, dims 4(j%4).. (+16T for tile T): the transposing read
    int lane;
    int c;               // lane >> 4: this lane's tokens 4c..4c+3
    int slot;            // fused: the appended token's slot in its page
    const uint32_t* new_k;   // fused: its rotated K row in LDS (BF16 pairs)
    const uint32_t* new_v;   // fused: its V row in LDS
};

__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }
// Hides where a value came from: the K rows read back from LDS stay in
// registers instead of the compiler merging them with the ring's slots.
__device__ __forceinline__ void opaque(uint4& v) { asm("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w)); }

// Max over the lanes that serve the same query head (lane bits 2..5).
__device__ __forceinline__ float head_max(float x) {
    x = fmaxf(x, dpp<kDppRowRor4>(x));
    x = fmaxf(x, dpp<kDppRowRor8>(x));
    return cross_rows_max(x);
}

// One page: the logits of the 4 query heads for its 16 tokens on the matrix
// cores (S^T = K Q^T: A = the page's K, column k = the lane's 8 dims; B = the
// 4 query heads repeated over the 16 columns), so lane l receives head
// l & 3's logits of tokens 4c..4c+3; the FP32 online softmax with one
// running maximum per head for the whole wave; the weights p, each split
// into two BF16 terms hi + lo (p - (hi + lo) is below 2^-17 p), times V on
// the matrix cores, which sums over the page's tokens (A = the weights,
// B = V transposed through LDS); products exact, sums in FP32.
//   kMasked: tokens 4c+i >= valid are left out (their V rows are zeroed in
//   LDS, so that a NaN-poisoned slot adds nothing); patch (fused kernel):
//   this page holds the token appended in this launch, whose K and V rows
//   are taken from LDS (what the page held when it was loaded may predate
//   the append).  That page is the sequence's last, so only the masked tail
//   sees it, and only that one page goes through the K tile in LDS.
template <bool kMasked, bool kFused>
__device__ __forceinline__ void consume_page(PageRegs pg, const QRegs& q, float scale_log2, int valid,
                                             bool patch, const PageCtx& cx, WaveState& st) {
    if (kMasked && (cx.lane >> 2) >= valid) {
        pg.va = make_uint4(0, 0, 0, 0);
        pg.vb = make_uint4(0, 0, 0, 0);
    }
    *reinterpret_cast<uint4*>(cx.vt + cx.w_off) = pg.va;
    *reinterpret_cast<uint4*>(cx.vt + cx.w_off + 32) = pg.vb;
    uint4 ka = pg.ka, kb = pg.kb;
    if constexpr (kFused && kMasked) {
        if (patch) {   // wave-uniform: the page of the token appended in this launch
            *reinterpret_cast<uint4*>(cx.kt + cx.k_off) = pg.ka;
            *reinterpret_cast<uint4*>(cx.kt + cx.k_off + 32) = pg.kb;
            if (cx.lane < 16) {
                const int i8 = (cx.lane & 7) * 8;
                const uint4 val = *reinterpret_cast<const uint4*>((cx.lane < 8 ? cx.new_k : cx.new_v) + i8 / 2);
                *reinterpret_cast<uint4*>((cx.lane < 8 ? cx.kt : cx.vt) + cx.slot * kTileRow + i8) = val;
            }
            compiler_fence();   // LDS operations of one wave complete in order
            ka = *reinterpret_cast<const uint4*>(cx.kt + cx.k_off);
            kb = *reinterpret_cast<const uint4*>(cx.kt + cx.k_off + 32);
            opaque(ka);
            opaque(kb);
        }
    }
    f32x4_t s4 = {0.0f, 0.0f, 0.0f, 0.0f};
    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, ka), q.a, s4, 0, 0, 0);
    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kb), q.b, s4, 0, 0, 0);
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = s4[i] * scale_log2;
        if (kMasked) x[i] = 4 * cx.c + i < valid ? x[i] : -INFINITY;
    }
    // Largest excess of a logit over the running maximum (NaN-free: m is
    // finite or -inf, and -inf - -inf only occurs for a masked token before
    // any valid one, which fmaxf drops).
    const float excess = fmaxf(fmaxf(x[0] - st.m, x[1] - st.m), fmaxf(x[2] - st.m, x[3] - st.m));
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(excess > kRescaleSlack) != 0, 0)) {
        const float pm = head_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
        const bool up = pm > st.m + kRescaleSlack;
        const float alpha = up ? exp2_fast(st.m - pm) : 1.0f;   // 0 when m was -inf
        st.l *= alpha;
        st.m = up ? pm : st.m;
        // o[T][i] belongs to head i, whose factor sits on lane i of each quad.
        const float a0 = dpp<kDppQuadBcast0>(alpha), a1 = dpp<kDppQuadBcast1>(alpha);
        const float a2 = dpp<kDppQuadBcast2>(alpha), a3 = dpp<kDppQuadBcast3>(alpha);
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            st.o[T][0] *= a0;
            st.o[T][1] *= a1;
            st.o[T][2] *= a2;
            st.o[T][3] *= a3;
        }
    }
    f32x4_t p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = exp2_fast(x[i] - st.m);
        if (kMasked) p[i] = 4 * cx.c + i < valid ? p[i] : 0.0f;
    }
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    const bf16x4_t hi = __builtin_convertvector(p, bf16x4_t);
    const f32x4_t rest = p - __builtin_convertvector(hi, f32x4_t);
    const bf16x4_t lo = __builtin_convertvector(rest, bf16x4_t);
    const s16x4_t ahi = __builtin_bit_cast(s16x4_t, hi), alo = __builtin_bit_cast(s16x4_t, lo);
    compiler_fence();
#pragma unroll
    for (int T = 0; T < 4; ++T) {
        const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4_t*)(cx.vt + cx.tr_off + 16 * T));
        st.o[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ahi, v, st.o[T], 0, 0, 0);
        st.o[T] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(alo, v, st.o[T], 0, 0, 0);
    }
    compiler_fence();   // the next page's tile stores come after these reads
}

// A round is kRing straight-line steps (unrolled by template recursion, so
// every ring slot index is a compile-time constant).  Invariant at the start
// of a round: slots 0..kRing-2 hold pages j..j+kRing-2 (issued), slot
// kRing-1 is free.  Step I issues page j+kRing-1 into the slot freed by the
// previous step, then consumes slot I.
template <bool kFused, int I, typename Issue>
__device__ __forceinline__ void ring_round(PageRing& ring, int& j, const QRegs& q, float sl2,
                                           const PageCtx& cx, WaveState& st, Issue& issue) {
    if constexpr (I < kRing) {
        ring.template at<(I + kRing - 1) % kRing>() = issue(j + kRing - 1);
        consume_page<false, kFused>(ring.template at<I>(), q, sl2, kPageTokens, false, cx, st);
        ++j;
        ring_round<kFused, I + 1>(ring, j, q, sl2, cx, st, issue);
    }
}

// The last 1..kRing pages of a chunk sit in slots 0..left-1; they are
// consumed with the token mask (only the chunk's last page can be partial).
// tok_page: the page that holds the token appended by a fused call (-1:
// none).
template <bool kFused, int I>
__device__ __forceinline__ void ring_tail(PageRing& ring, int j, int left, int n, const QRegs& q,
                                          float sl2, int tok_page, const PageCtx& cx, WaveState& st) {
    if constexpr (I < kRing) {
        if (I < left) {
            consume_page<true, kFused>(ring.template at<I>(), q, sl2, n - (j + I) * kPageTokens,
                                       j + I == tok_page, cx, st);
            ring_tail<kFused, I + 1>(ring, j, left, n, q, sl2, tok_page, cx, st);
        }
    }
}

template <int I, typename Issue>
__device__ __forceinline__ void ring_fill(PageRing& ring, int pb, Issue& issue) {
    if constexpr (I < kRing - 1) {
        ring.template at<I>() = issue(pb + I);
        ring_fill<I + 1>(ring, pb, issue);
    }
}

// The log-sum-exp merge of the S outer-chunk partials of one query head:
// with M = max_c m_c (base 2), out = sum_c 2^(m_c - M) acc_c / sum_c
// 2^(m_c - M) l_c; an empty chunk (m_c = -inf) weighs 0.  The partials
// arrive in kMaxSplits slots whose slots past S hold a reread partial; their
// terms are selected exact zeros (never a product with the reread values,
// which may be NaN), so the sums are those over the S.  The separate combine
// kernel and the in-kernel merge both use these two steps, in the same
// order, so the two paths give the same bits.
struct MergeWeights {
    float w[kMaxSplits];
    float inv;   // 1 / sum of the weighted sums (0 when that sum is 0)
};
__device__ __forceinline__ MergeWeights merge_weights(const float2 (&ml)[kMaxSplits], int S) {
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) M = fmaxf(M, c < S ? ml[c].x : -INFINITY);
    MergeWeights r;
    float L = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) {
        const bool in = c < S && ml[c].x != -INFINITY;
        r.w[c] = in ? exp2_fast(ml[c].x - M) : 0.0f;
        L = fmaf(r.w[c], c < S ? ml[c].y : 0.0f, L);
    }
    r.inv = L == 0.0f ? 0.0f : 1.0f / L;
    return r;
}
__device__ __forceinline__ float merge_dim(const MergeWeights& mw, const float (&x)[kMaxSplits], int S) {
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) a = fmaf(mw.w[c], c < S ? x[c] : 0.0f, a);
    return a * mw.inv;
}

// Partials are exchanged between workgroups that may run on different XCDs,
// whose L2 caches are not coherent with each other: they are written and
// read with device-scope (agent) accesses, which the gfx950 memory model
// makes coherent across the XCDs (write-through stores, loads that do not
// take another XCD's stale line), so no L2 write-back or invalidation of
// the whole cache is needed.
__device__ __forceinline__ void store_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(float2* p, float2 v) {
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_agent(const float2* p) {
    return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float2*>(p)),
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
// Waits until this wave's stores have completed (on gfx9 the vector memory
// counter covers stores), and keeps the compiler from moving memory
// operations across it.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Row tasks of the fused append: 6 rows (query heads 4g..4g+3 and the new
// K of head g, rotated; the new V of head g, copied) x 8 groups of 4 pairs
// (dims i0..i0+3 and i0+32..i0+35).  Every wave that has pages runs all 48
// in its lanes 0..47 and passes the rows to its other lanes through its own
// LDS rows, so no wave waits for another.
constexpr int kRotRows = kGroup + 2;
constexpr int kRotTasks = kRotRows * 8;
static_assert(kRotTasks <= 64, "one task per lane");

// kFused = false: paged decode attention over the cache as it is (q already
// rotated by the append).  kFused = true: the same, with the append of the
// new token done in the same launch: q and the new K are rotated here (the
// same rotation and rounding as append_kernel, rope4), q is used without being
// written back, the K/V row is written into its page by the workgroup of
// outer chunk 0, and the attention reads the new token from registers.
//
// kMerge (S > 1 only): after writing its partials, each workgroup counts
// itself in its (sequence, KV head)'s counter; the one that finds the other
// S - 1 already counted merges the S partials into the output row (the
// combine kernel's arithmetic, in the same order) and sets the counter back
// to 0 for the next call.  No workgroup waits for another.
// A wave's instruction-issue priority follows the pages it still has to
// stream, the most first (set again before every ring round), in launches of
// at most two rounds of resident workgroups.  Without it a CU's issue
// arbitration favours the older of its workgroups at every tie: the older
// finishes long before the younger, which then streams alone with half the
// loads in flight, and short chunks compete with the long ones that set the
// end of the launch.
__device__ __forceinline__ void issue_priority(int pages_left) {
    if (pages_left > 24) __builtin_amdgcn_s_setprio(3);
    else if (pages_left > 16) __builtin_amdgcn_s_setprio(2);
    else if (pages_left > 8) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
}

template <bool kFused, bool kMerge>
__global__ __launch_bounds__(kChunkWaves * 64) __attribute__((amdgpu_waves_per_eu(PKV_SPLIT_WAVES_PER_EU)))
void attn_split_kernel(AttnParams p) {
    // Partials of the workgroup's 4 waves: [wave][head][64 dims] and (max, sum).
    __shared__ float lds_acc[kChunkWaves][kGroup][kHeadDim];
    __shared__ float2 lds_ml[kChunkWaves][kGroup];
    // Fused append: each wave's new rows (BF16 pairs) [q head 0..3, K, V].
    __shared__ __align__(16) uint32_t lds_rot[kFused ? kChunkWaves : 1][kRotRows * kHeadDim / 2];
    // Each wave's current page: V (and, fused, K) rows of its 16 tokens.
    __shared__ __align__(16) uint16_t lds_vt[kChunkWaves][kPageTokens * kTileRow];
    __shared__ __align__(16) uint16_t lds_kt[kFused ? kChunkWaves : 1][kPageTokens * kTileRow];
    __shared__ int lds_last;   // kMerge: this workgroup is the last of its (sequence, KV head)

    const int lane = threadIdx.x & 63;
    const int w = uniform((int)(threadIdx.x >> 6));
    const uint32_t wg = blockIdx.x;                    // g fastest, then rank, then outer chunk
    const int g = (int)(wg % kKVHeads);
    const uint32_t rest = wg / kKVHeads;
    const int rank = (int)(rest % (uint32_t)p.num_seqs);
    const int ci = (int)(rest / (uint32_t)p.num_seqs);
    // The sequence started at this position: the caller's order when given
    // (paged_decode_attn_order: the longest sequences do not start last, and
    // each CU's first workgroups carry about the same pages), else batch
    // order.  An entry outside [0, num_seqs) falls back to the position itself.
    int s = rank;
    if (p.seq_order) {
        const int o = uniform(p.seq_order[rank]);
        s = o >= 0 && o < p.num_seqs ? o : rank;
    }
    const int t = lane & 15;   // token slot of this lane (the MFMA column)
    const int c4 = lane >> 4;  // dims 8*c4..8*c4+7 and 32+8*c4..32+8*c4+7 (the MFMA k slice)

    if constexpr (kFused) {
        // The arguments the fused prologue reads, held in scalar registers
        // from here: their loads join the first batch instead of following
        // one another after the length arrives.
        asm volatile("" ::"s"(p.q), "s"(p.q_stride), "s"(p.k_new), "s"(p.k_stride), "s"(p.v_new),
                     "s"(p.v_stride), "s"(p.rope_cos), "s"(p.rope_sin), "s"(p.max_pos));
    }
    // Independent loads first: the table row (first 128 entries, one per
    // lane in two registers), q of the 4 query heads, and the length.
    const int32_t* bt_row = p.block_table + (int64_t)s * p.bt_stride;
    const int bt_w = p.bt_stride < kMaxContext / kPageTokens ? (int)p.bt_stride
                                                              : kMaxContext / kPageTokens;
    const int32_t tbl0 = lane < bt_w ? bt_row[lane] : 0;
    const int32_t tbl1 = lane + 64 < bt_w ? bt_row[lane + 64] : 0;
    QRegs q;
    const uint16_t* qrow = p.q + (int64_t)s * p.q_stride + (kGroup * g) * kHeadDim;
    // Fused: the new rows of the append's 48 row tasks, one per lane (lanes
    // past 47 repeat the last one): 4 q heads, the new K and V of KV head g.
    // They do not depend on the length, so they are requested with q's.
    const int task = kFused ? min(lane, kRotTasks - 1) : 0;
    const int row = task >> 3;
    const int i0 = (task & 7) * 4;
    uint2 x1 = make_uint2(0, 0), x2 = make_uint2(0, 0);
    if constexpr (kFused) {
        const uint16_t* src = row < kGroup ? qrow + row * kHeadDim
                            : row == kGroup ? p.k_new + (int64_t)s * p.k_stride + g * kHeadDim
                                            : p.v_new + (int64_t)s * p.v_stride + g * kHeadDim;
        x1 = *reinterpret_cast<const uint2*>(src + i0);
        x2 = *reinterpret_cast<const uint2*>(src + i0 + 32);
    } else {
        const uint16_t* qh = qrow + (lane & 3) * kHeadDim + c4 * 8;
        q.a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qh));
        q.b = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qh + 32));
    }
    const int ctx = uniform(p.context_lens[s]);
    const int n = ctx < p.max_context_len ? ctx : p.max_context_len;
    const int np = n > 0 ? (n + kPageTokens - 1) / kPageTokens : 0;

    // This wave's chunk: the sequence's np pages are cut into 4*S chunks of
    // ceil(np / (4*S)) pages; wave w of outer chunk ci takes chunk 4*ci + w.
    const int nchunks = kChunkWaves * p.plan.splits;
    const int cs = (np + nchunks - 1) / nchunks;
    const int pb = (kChunkWaves * ci + w) * cs;
    const int pe = min(pb + cs, np);
    if (p.priority_by_pages_left) issue_priority(pe - pb);

    // The fused append rotates only where append_kernel would (a token
    // position inside the RoPE table); otherwise q is used as given.
    const int pos = ctx - 1;
    const bool rotate = kFused && ctx >= 1 && pos < p.max_pos;
    // The chunk's result: o[T][i] = head i, dim 16T + (lane & 15); and head
    // lane & 3's (max, sum).
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int T = 0; T < 4; ++T) st.o[T] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    bool bad_page = false;

    // K lands in the MFMA operand layout (row l & 15); V, which passes
    // through LDS, is loaded 4 lanes per 64 contiguous bytes of a row.
    const uint32_t k_off = (uint32_t)((t * p.slot_stride + c4 * 8) * 2);
    const uint32_t v_off = (uint32_t)(((lane >> 2) * p.slot_stride + (lane & 3) * 8) * 2);
    const int32_t tile_bytes = (int32_t)((15 * p.slot_stride + kHeadDim) * 2);
    // The sequence's last page holds 1..16 valid slots: its range ends after
    // the last valid row, so the loads of the rows past it return zeros
    // without reading memory (the mask leaves those slots out anyway).
    const int last_rows = np > 0 ? n - (np - 1) * kPageTokens : kPageTokens;
    const int32_t last_tile_bytes = (int32_t)(((last_rows - 1) * p.slot_stride + kHeadDim) * 2);
    const char* kpool = reinterpret_cast<const char*>(p.k_pool) + (int64_t)g * p.head_stride * 2;
    const char* vpool = reinterpret_cast<const char*>(p.v_pool) + (int64_t)g * p.head_stride * 2;
    const int64_t page_bytes = p.page_stride * 2;

    // Issue the loads of logical page j (a no-op load when j >= pe).
    auto issue = [&](int j) {
        const bool live = j < pe;
        const int idx = j < pe - 1 ? j : pe - 1;
        int32_t phys = idx < 64 ? __builtin_amdgcn_readlane(tbl0, idx)
                                : __builtin_amdgcn_readlane(tbl1, idx - 64);
        if (phys < 0 || phys >= p.num_pages) {  // never dereference a bad entry
            bad_page |= live;
            phys = 0;
        }
        const int32_t bytes = live ? (j == np - 1 ? last_tile_bytes : tile_bytes) : 0;
        const int64_t off = (int64_t)phys * page_bytes;
        return load_page(tile_rsrc(kpool + off, bytes), tile_rsrc(vpool + off, bytes), k_off,
                         v_off);
    };

    // Ring of kRing page buffers: while page j is consumed, pages j+1 ..
    // j+kRing-1 are in flight.  The last page of the chunk is the only
    // one that can hold slots past n, so it is consumed with the mask.
    PageRing ring;
    int tok_page = -1;   // fused: the page of the token appended in this launch, when attended
    uint32_t* rot = lds_rot[kFused ? w : 0];
    PageCtx cx;
    cx.vt = lds_vt[w];
    cx.kt = lds_kt[kFused ? w : 0];
    cx.w_off = (lane >> 2) * kTileRow + (lane & 3) * 8;
    cx.k_off = t * kTileRow + c4 * 8;
    cx.tr_off = (4 * c4 + ((lane & 15) >> 2)) * kTileRow + 4 * (lane & 3);
    cx.lane = lane;
    cx.c = c4;
    cx.slot = pos & (kPageTokens - 1);
    cx.new_k = rot + kGroup * 32;
    cx.new_v = rot + (kGroup + 1) * 32;
    if (pb < pe) {
        if constexpr (kFused) {
            // Fused append, part 1: the row tasks' RoPE rows (at the token's
            // position) are requested before the first pages, and the rotation
            // runs while those are in flight.  A wave with an empty chunk
            // skips all of it (it never uses q, and wave 0 of outer chunk 0,
            // which stores the K/V row, always has pages when the token is
            // rotated): in a batch of short sequences its loads and rotation
            // would only compete with the waves that stream.
            const int64_t trow = (int64_t)(rotate ? pos : 0) * 32 + i0;
            const float4 c = *reinterpret_cast<const float4*>(p.rope_cos + trow);
            const float4 sn = *reinterpret_cast<const float4*>(p.rope_sin + trow);
            ring_fill<0>(ring, pb, issue);
            if (rotate && row <= kGroup) rope4(x1, x2, c, sn);
            if (lane < kRotTasks) {
                *reinterpret_cast<uint2*>(&rot[row * 32 + i0 / 2]) = x1;
                *reinterpret_cast<uint2*>(&rot[row * 32 + 16 + i0 / 2]) = x2;
            }

            // Fused append, part 2: the wave's lanes take the rotated q rows
            // (LDS ops of one wave complete in order; the fences keep the
            // compiler from moving the reads above the writes).  When the new
            // token lies inside the attended length, the page that holds it
            // takes the token's K and V rows from LDS (consume_page).
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            q.a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&rot[(lane & 3) * 32 + c4 * 4]));
            q.b = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(&rot[(lane & 3) * 32 + 16 + c4 * 4]));
            if (rotate && ctx == n) tok_page = np - 1;
        }
        if constexpr (!kFused) ring_fill<0>(ring, pb, issue);
        const float sl2 = p.scale_log2;
        int j = pb;
        const int rounds = (pe - 1 - pb) / kRing;   // whole rounds of unmasked pages
        for (int r = 0; r < rounds; ++r) {
            if (p.priority_by_pages_left) issue_priority(pe - j);
            ring_round<kFused, 0>(ring, j, q, sl2, cx, st, issue);
        }
        if (p.priority_by_pages_left) issue_priority(pe - j);
        ring.template at<kRing - 1>() = issue(j + kRing - 1);
        ring_tail<kFused, 0>(ring, j, pe - j, n, q, sl2, tok_page, cx, st);
        // The sum of head lane & 3 over the 4 lane rows (their tokens differ).
        st.l = cross_rows_sum(st.l);
        if (bad_page) st.l = NAN;
    }

    if constexpr (kFused) {
        // Fused append, part 3: wave 0 of outer chunk 0 stores the new K/V
        // row where append_kernel would.  After the page loop: a store counts
        // against the same in-order memory counter as the page loads, so an
        // earlier one would hold back this wave's waits for its pages; here
        // none are left, and the write overlaps the merge below.
        if (rotate && ci == 0 && w == 0 && lane < 16) {
            const int64_t jpage = pos >> 4;
            if (jpage < p.bt_stride) {
                // From the table registers when the entry is among the first 128.
                const int64_t page = jpage < bt_w ? (jpage < 64 ? __builtin_amdgcn_readlane(tbl0, (int)jpage)
                                                                : __builtin_amdgcn_readlane(tbl1, (int)jpage - 64))
                                                  : bt_row[jpage];
                if (page >= 0 && page < p.num_pages) {   // never write through a bad entry
                    const int64_t dst = page * p.page_stride + g * p.head_stride +
                                        (int64_t)(pos & (kPageTokens - 1)) * p.slot_stride;
                    const int i8 = (lane & 7) * 8;
                    const uint4 val = *reinterpret_cast<const uint4*>(
                        &rot[(lane < 8 ? kGroup : kGroup + 1) * 32 + i8 / 2]);
                    *reinterpret_cast<uint4*>((lane < 8 ? p.k_pool_w : p.v_pool_w) + dst + i8) = val;
                }
            }
        }
    }

    // ---- merge the 4 chunks of the workgroup through LDS ----
    {
        // Lane row c4 stores head c4 (every row holds all 4 heads).
#pragma unroll
        for (int T = 0; T < 4; ++T) {
            const float v = c4 == 0 ? st.o[T][0] : c4 == 1 ? st.o[T][1] : c4 == 2 ? st.o[T][2] : st.o[T][3];
            lds_acc[w][c4][16 * T + (lane & 15)] = v;
        }
        if (lane < kGroup) lds_ml[w][lane] = make_float2(st.m, st.l);
    }
    __syncthreads();
    // Wave w finishes query head 4g + w; lane = output dim.
    const int r = w;
    float Mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kChunkWaves; ++i) Mx = fmaxf(Mx, lds_ml[i][r].x);
    float L = 0.0f, o = 0.0f;
#pragma unroll
    for (int i = 0; i < kChunkWaves; ++i) {
        const float2 ml = lds_ml[i][r];
        const float wt = ml.x == -INFINITY ? 0.0f : exp2_fast(ml.x - Mx);
        L = fmaf(wt, ml.y, L);
        o = fmaf(wt, lds_acc[i][r][lane], o);
    }
    const int h = kGroup * g + r;
    if (p.plan.splits == 1) {
        const float ov = L == 0.0f ? 0.0f : o / L;
        const char* ob = reinterpret_cast<const char*>(p.out + (int64_t)s * p.out_stride + h * kHeadDim);
        // Non-temporal: nothing in this launch reads the output again.
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), tile_rsrc(ob, kHeadDim * 4), lane * 4, 0,
                                              kStoreNonTemporal);
    } else {
        const int S = p.plan.splits;
        const int64_t slot_idx = ((int64_t)s * kQHeads + h) * S + ci;
        store_agent(&p.ws_acc[slot_idx * kHeadDim + lane], o);
        if (lane == 0) store_agent(&p.ws_ml[slot_idx], make_float2(Mx, L));
        if constexpr (kMerge) {
            // Count this workgroup once all 4 waves' partials are stored.
            wait_stores();
            __syncthreads();
            if (threadIdx.x == 0) {
                const int done = __hip_atomic_fetch_add(&p.ws_cnt[s * kKVHeads + g], 1, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
                lds_last = done == S - 1;
            }
            __syncthreads();
            if (lds_last) {
                // Wave w merges query head h = 4g + w; lane = output dim.
                const int64_t base = ((int64_t)s * kQHeads + h) * S;
                float2 ml[kMaxSplits];
                float x[kMaxSplits];
#pragma unroll
                for (int c = 0; c < kMaxSplits; ++c) {
                    const int64_t slot = base + (c < S ? c : S - 1);
                    ml[c] = load_agent(&p.ws_ml[slot]);
                    x[c] = load_agent(&p.ws_acc[slot * kHeadDim + lane]);
                }
                const float ov = merge_dim(merge_weights(ml, S), x, S);
                const char* ob = reinterpret_cast<const char*>(p.out + (int64_t)s * p.out_stride + h * kHeadDim);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), tile_rsrc(ob, kHeadDim * 4), lane * 4,
                                                      0, kStoreNonTemporal);
                if (threadIdx.x == 0)
                    __hip_atomic_store(&p.ws_cnt[s * kKVHeads + g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// One thread per (sequence, query head, 4 output dims): merges the S
// outer-chunk partials with the log-sum-exp rule (merge_weights, merge_dim).
// All S (max, sum) pairs and accumulator quads are requested at once (an
// index past S rereads the last partial and is then ignored), so the thread
// waits for one round trip, not one per partial.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnParams p) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int d4 = (int)(tid & 15);
    const int h = (int)((tid >> 4) & 31);
    const int64_t s = tid >> 9;
    if (s >= p.num_seqs) return;
    const int S = p.plan.splits;
    const int64_t base = ((int64_t)s * kQHeads + h) * S;
    float2 ml[kMaxSplits];
    float4 v[kMaxSplits];
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) {
        const int64_t slot = base + (c < S ? c : S - 1);
        ml[c] = p.ws_ml[slot];
        v[c] = *reinterpret_cast<const float4*>(p.ws_acc + slot * kHeadDim + d4 * 4);
    }
    const MergeWeights mw = merge_weights(ml, S);
    float xs[4][kMaxSplits];
#pragma unroll
    for (int c = 0; c < kMaxSplits; ++c) {
        xs[0][c] = v[c].x;
        xs[1][c] = v[c].y;
        xs[2][c] = v[c].z;
        xs[3][c] = v[c].w;
    }
    *reinterpret_cast<float4*>(p.out + s * p.out_stride + h * kHeadDim + d4 * 4) =
        make_float4(merge_dim(mw, xs[0], S), merge_dim(mw, xs[1], S), merge_dim(mw, xs[2], S),
                    merge_dim(mw, xs[3], S));
}

// ----------------------------------------------------------- ordering --
//
// One workgroup ranks the num_seqs sequences by descending page count
// (stable: ties keep batch order), a counting sort over the 129 possible
// counts: a histogram in LDS, its exclusive prefix (longest first) scanned
// by one wave, then rounds of 1,024 sequences, one per thread: a thread's place is
// the start of its count's range, plus its count's members in earlier
// rounds, in earlier waves of this round, and in lower lanes of its own wave
// (lanes with the same count found with one ballot per bit of the count).
// The sorted rank then maps to the position the sequence starts at
// (order_position: the first round of resident workgroups balanced across
// CUs).
constexpr int kOrderThreads = 1024;
constexpr int kOrderWaves = kOrderThreads / 64;
constexpr int kOrderBins = kMaxContext / kPageTokens + 1;   // page counts 0..128
static_assert(kOrderBins <= 255, "counts fit 8 bits; 255 marks no sequence");

__device__ __forceinline__ int page_bin(const int32_t* ctx, int s, int max_context_len) {
    return order_page_count(ctx[s], max_context_len);
}

__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t* ctx, int num_seqs, int max_context_len,
                                                              int round_len, int32_t* order) {
    __shared__ int start[kOrderBins];                 // first rank of each count, this round
    __shared__ int wave_count[kOrderWaves][kOrderBins];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    for (int b = tid; b < kOrderBins; b += kOrderThreads) start[b] = 0;
    for (int i = tid; i < kOrderWaves * kOrderBins; i += kOrderThreads) (&wave_count[0][0])[i] = 0;
    // The first round's counts stay in registers for the ranking below.
    const int key0 = tid < num_seqs ? page_bin(ctx, tid, max_context_len) : 255;
    __syncthreads();
    // histogram (start[] doubles as the count of each bin)
    if (key0 != 255) atomicAdd(&start[key0], 1);
    for (int s = tid + kOrderThreads; s < num_seqs; s += kOrderThreads)
        atomicAdd(&start[page_bin(ctx, s, max_context_len)], 1);
    __syncthreads();   // every count is in
    // Exclusive prefix over the counts, longest first, in one wave: lane l
    // holds scan positions 4l..4l+3 (position t is the count 128 - t).
    static_assert(kOrderBins <= 256, "four scan positions per lane");
    if (wv == 0) {
        int v[4], sum = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lane + i;
            v[i] = t < kOrderBins ? start[kOrderBins - 1 - t] : 0;
            sum += v[i];
        }
        int incl = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        int run = incl - sum;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * lane + i;
            if (t < kOrderBins) start[kOrderBins - 1 - t] = run;
            run += v[i];
        }
    }
    __syncthreads();
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int r0 = 0; r0 < num_seqs; r0 += kOrderThreads) {
        const int s = r0 + tid;
        const bool valid = s < num_seqs;
        const int key = r0 == 0 ? key0 : valid ? page_bin(ctx, s, max_context_len) : 255;
        uint64_t same = ~0ull;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const bool bit = (key >> k) & 1;
            const uint64_t b = __builtin_amdgcn_ballot_w64(bit);
            same &= bit ? b : ~b;
        }
        const int lower = __builtin_popcountll(same & below);
        if (valid && lower == 0) wave_count[wv][key] = __builtin_popcountll(same);
        __syncthreads();
        if (valid) {
            int pre = 0;
            for (int v = 0; v < wv; ++v) pre += wave_count[v][key];
            order[order_position(start[key] + pre + lower, num_seqs, round_len)] = s;
        }
        __syncthreads();
        for (int b = tid; b < kOrderBins; b += kOrderThreads) {
            int c = 0;
            for (int v = 0; v < kOrderWaves; ++v) {
                c += wave_count[v][b];
                wave_count[v][b] = 0;
            }
            start[b] += c;
        }
        __syncthreads();
    }
}

// Zeroes n 32-bit words (the merge counters of the fixed scratch array).
__global__ __launch_bounds__(256) void zero_words_kernel(int32_t* p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0;
}

// The fixed scratch of paged_kv_append_decode_attn_noalloc: the workspace of
// the largest plan that uses one (S = kMaxSplits partials of kMergeSeqs - 1
// sequences after the counter block), laid out as workspace_bytes()
// describes.  Each device holds its own copy until the process ends.
constexpr size_t kScratchBytes =
    kCounterBytes + (size_t)kMaxSplits * (kMergeSeqs - 1) * kQHeads * kPartialFloats * sizeof(float);
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

hipError_t launch_order(const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                        int32_t* seq_order, hipStream_t stream) {
    hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, context_lens, num_seqs,
                       max_context_len, resident_seqs(), seq_order);
    return hipGetLastError();
}

int32_t resident_seqs() {
    const int64_t wgs = resident_workgroups();
    if (wgs == INT64_MAX) return 0;
    const int64_t seqs = wgs / kKVHeads;
    return seqs > INT32_MAX ? 0 : (int32_t)seqs;
}

int64_t resident_workgroups() {
    static std::mutex mu;
    static int64_t cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return INT64_MAX;
    std::lock_guard<std::mutex> g(mu);
    if (!cached[dev]) {
        int per_cu = 0, cus = 0;
        // the fused kernel holds the most resources of the attention variants
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_split_kernel<true, true>,
                                                         kChunkWaves * 64, 0) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            per_cu < 1 || cus < 1)
            return INT64_MAX;
        cached[dev] = (int64_t)per_cu * cus;
    }
    return cached[dev];
}

// The device address of this device's scratch array.  In host code the
// array's name is only a stand-in for it, so the address is looked up once
// per device (with that device current) and kept; on that first call the
// counter block is cleared by a fill kernel on the caller's stream.
hipError_t scratch_buffer(void** out, hipStream_t stream) {
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> g(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        const int words = (int)(kCounterBytes / sizeof(int32_t));
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream,
                           static_cast<int32_t*>(p), words);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return hipSuccess;
}

hipError_t launch_append(const AppendParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((append_kernel<1, AppendParams>),
                       dim3((unsigned)p.num_seqs * kAppendBlocksPerToken), dim3(kAppendThreads), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_copy_pages(const CopyParams& p, hipStream_t stream) {
    hipLaunchKernelGGL(copy_pages_kernel, dim3((unsigned)p.n), dim3(kCopyThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
    const int64_t groups = ((int64_t)p.total_tokens + kPrefillRows - 1) / kPrefillRows;
    const int64_t blocks = groups * (p.q ? kAppendBlocksPerToken : 1);
    hipLaunchKernelGGL((append_kernel<kPrefillRows, PrefillParams>), dim3((unsigned)blocks),
                       dim3(kAppendThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_split(const AttnParams& p, bool merge, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.num_seqs * kKVHeads * p.plan.splits;
    if (merge && p.plan.splits > 1) {
        if (p.num_seqs > kMergeSeqs) return hipErrorInvalidValue;   // the plan never asks for it
        hipLaunchKernelGGL((attn_split_kernel<false, true>), dim3((unsigned)blocks), dim3(kChunkWaves * 64),
                           0, stream, p);
    } else {
        hipLaunchKernelGGL((attn_split_kernel<false, false>), dim3((unsigned)blocks), dim3(kChunkWaves * 64),
                           0, stream, p);
    }
    return hipGetLastError();
}

hipError_t launch_append_attn_split(const AttnParams& p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.num_seqs * kKVHeads * p.plan.splits;
    if (p.plan.splits > 1 && p.num_seqs > kMergeSeqs) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_split_kernel<true, true>), dim3((unsigned)blocks), dim3(kChunkWaves * 64), 0,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_attn_combine(const AttnParams& p, hipStream_t stream) {
    if (p.plan.splits < 1 || p.plan.splits > kMaxSplits) return hipErrorInvalidValue;   // the plan caps S
    const int64_t threads = (int64_t)p.num_seqs * kQHeads * 16;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace pkv
