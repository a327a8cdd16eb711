/*
 * pkv_oracle.c -- plain, slow, single-threaded FP64 CPU oracle for the decode
 * step over a paged BF16 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library and its Python binding) never calls it and shares no code,
 * header, table or constant with it.
 *
 * Sources (all prose; none of them prints code or a worked example):
 *   [TV]  "Tiny-vLLMでゼロから構築する高性能LLM推論エンジン" (agentlenshq.com),
 *         sections "Bfloat16の選択" and "KV Cache".
 *   [HN]  "Hours of YouTube and 85 handtyped pages of notes on LLM Inference -
 *         Start here" (hackernews.jp translation of the project README),
 *         sections "これまでの進捗" (progress so far) and "現在のスコープ"
 *         (current scope).
 *
 * What is computed is the plain definition, written out in FP64:
 *   - BF16 rounding: nearest representable BF16 value, ties to an even
 *     mantissa ([TV] "Bfloat16の選択": 8 exponent bits like FP32, 7 mantissa
 *     bits).
 *   - RoPE table: angle = pos * theta^(-2i/64), cos/sin in FP64, each rounded
 *     once to FP32.  theta = 500000 is passed in by the caller.
 *   - Append ([HN] progress, the bullet on the shared BF16 KV page pool: one
 *     table per sequence and layer, 16 tokens of K and V per physical page,
 *     decode appends one token at its absolute RoPE position): rotate q and k
 *     of the new token at pos = ctx-1 (half-split pairs (i, i+32)), round once
 *     to BF16, store K' and V into page bt[(ctx-1)/16], slot (ctx-1)%16.
 *   - Attention ([HN] progress, the bullet on paged decode attention: every
 *     query head reads its own sequence's cached pages, softmax in FP32 or
 *     better, weighted sum of V): for query head h and KV head h/4,
 *     o = sum_t softmax_t(scale * q.k_t) v_t over t = 0..ctx-1 in logical
 *     order, computed as the plain two-pass definition (max, exp, sum) in
 *     FP64.  It is not the online recurrence: that is the method being
 *     checked, and the tests pin this routine against an online recurrence
 *     and against split/merge partitions separately.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - ctx counts tokens after the append; the new token sits at ctx-1.
 *   - slot = pos mod 16, page index = pos div 16.
 *   - query head h reads KV head floor(h/4).
 *   - RoPE pairs (i, i+32); no frequency rescaling.
 *   - ctx <= 0: append writes nothing, attention writes a zero row.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 * No FMA contraction, so each product and sum below is one IEEE FP64 op.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HQ 32      /* query heads                      */
#define HKV 8      /* KV heads                         */
#define HD 64      /* head dimension                   */
#define HALF 32    /* rotation pairs per head          */
#define PTOK 16    /* tokens per physical page         */

/* ---------------------------------------------------------------- BF16 -- */

/* Exact value of a BF16 bit pattern: the upper half of an FP32 pattern. */
double pkv_oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Nearest BF16 value to y, ties to an even mantissa, overflow to infinity.
 * Written from the definition: find the spacing of the BF16 grid at |y|
 * (2^(E-7) for a normal binade E, 2^-133 below 2^-126), round |y|/spacing
 * to the nearest integer with ties to even, and scale back. */
uint16_t pkv_oracle_bf16_round(double y) {
    if (isnan(y)) return (uint16_t)(signbit(y) ? 0xFFC0u : 0x7FC0u);
    uint16_t sign = signbit(y) ? 0x8000u : 0x0000u;
    double a = fabs(y);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    int e2;
    (void)frexp(a, &e2);          /* a = f * 2^e2, f in [0.5, 1) */
    int binade = e2 - 1;          /* floor(log2 a)               */
    if (binade < -126) binade = -126;
    double spacing = ldexp(1.0, binade - 7);
    double units = a / spacing;   /* exact: division by a power of two */
    double r = nearbyint(units) * spacing;   /* round-half-even (default mode) */
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    float f = (float)r;           /* exact: r lies on the BF16 grid */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

/* ---------------------------------------------------------------- RoPE -- */

/* cos/sin table [max_pos][32] in FP32: angle = pos * theta^(-2i/64). */
int pkv_oracle_rope_table(double theta, int32_t max_pos, float* cos_out, float* sin_out) {
    if (max_pos < 0 || !(theta > 0.0) || !cos_out || !sin_out) return -1;
    for (int32_t pos = 0; pos < max_pos; ++pos) {
        for (int i = 0; i < HALF; ++i) {
            double inv_freq = pow(theta, -(2.0 * (double)i) / (double)HD);
            double angle = (double)pos * inv_freq;
            cos_out[(int64_t)pos * HALF + i] = (float)cos(angle);
            sin_out[(int64_t)pos * HALF + i] = (float)sin(angle);
        }
    }
    return 0;
}

/* Rotate one 64-wide head vector at table row `pos`, in FP64, no rounding. */
void pkv_oracle_rope_rotate_f64(const double* x, const float* cos_row, const float* sin_row,
                                double* y) {
    for (int i = 0; i < HALF; ++i) {
        double c = (double)cos_row[i];
        double s = (double)sin_row[i];
        double x1 = x[i];
        double x2 = x[i + HALF];
        y[i] = x1 * c - x2 * s;
        y[i + HALF] = x2 * c + x1 * s;
    }
}

/* Rotate a BF16 head vector and round every element once to BF16. */
static void rotate_bf16(const uint16_t* src, uint16_t* dst, const float* cos_row,
                        const float* sin_row) {
    double x[HD], y[HD];
    for (int d = 0; d < HD; ++d) x[d] = pkv_oracle_bf16_to_f64(src[d]);
    pkv_oracle_rope_rotate_f64(x, cos_row, sin_row, y);
    for (int d = 0; d < HD; ++d) dst[d] = pkv_oracle_bf16_round(y[d]);
}

/* ------------------------------------------------------------ indexing -- */

/* Where the token that makes the context `ctx` long is stored:
 * logical page ctx-1 div 16, slot ctx-1 mod 16.  Returns -1 for ctx < 1. */
int pkv_oracle_locate(int32_t ctx, int32_t* page_index, int32_t* slot) {
    if (ctx < 1) return -1;
    int32_t pos = ctx - 1;
    *page_index = pos / PTOK;
    *slot = pos % PTOK;
    return 0;
}

/* Number of logical pages holding ctx tokens. */
int32_t pkv_oracle_num_pages(int32_t ctx) {
    if (ctx < 1) return 0;
    return (ctx + PTOK - 1) / PTOK;
}

static int64_t elem_offset(int64_t page, int g, int slot, int64_t page_stride,
                           int64_t head_stride, int64_t slot_stride) {
    return page * page_stride + (int64_t)g * head_stride + (int64_t)slot * slot_stride;
}

/* -------------------------------------------------------------- append -- */

/* For every sequence s with ctx[s] >= 1: rotate q[s] (32 heads) in place and
 * k[s] (8 heads), round to BF16, store K' and V at the page/slot of position
 * ctx[s]-1 through block_table row s.  Returns 0, or -1 when a position is
 * outside the RoPE table or a page index is outside the pool. */
int pkv_oracle_append(uint16_t* k_pool, uint16_t* v_pool, int64_t num_pages, int64_t page_stride,
                      int64_t head_stride, int64_t slot_stride, const int32_t* block_table,
                      int64_t bt_stride, const int32_t* ctx, int32_t num_seqs, uint16_t* q,
                      int64_t q_stride, const uint16_t* k, int64_t k_stride, const uint16_t* v,
                      int64_t v_stride, const float* rope_cos, const float* rope_sin,
                      int32_t max_pos) {
    for (int32_t s = 0; s < num_seqs; ++s) {
        int32_t n = ctx[s];
        if (n < 1) continue;
        int32_t pos = n - 1;
        if (pos >= max_pos) return -1;
        int32_t j, t;
        pkv_oracle_locate(n, &j, &t);
        if (j >= bt_stride) return -1;
        int64_t page = block_table[(int64_t)s * bt_stride + j];
        if (page < 0 || page >= num_pages) return -1;
        const float* crow = rope_cos + (int64_t)pos * HALF;
        const float* srow = rope_sin + (int64_t)pos * HALF;
        for (int h = 0; h < HQ; ++h) {
            uint16_t* qh = q + (int64_t)s * q_stride + (int64_t)h * HD;
            uint16_t rotated[HD];
            rotate_bf16(qh, rotated, crow, srow);
            memcpy(qh, rotated, sizeof rotated);
        }
        for (int g = 0; g < HKV; ++g) {
            const uint16_t* kg = k + (int64_t)s * k_stride + (int64_t)g * HD;
            const uint16_t* vg = v + (int64_t)s * v_stride + (int64_t)g * HD;
            int64_t off = elem_offset(page, g, t, page_stride, head_stride, slot_stride);
            rotate_bf16(kg, k_pool + off, crow, srow);
            memcpy(v_pool + off, vg, HD * sizeof(uint16_t));
        }
    }
    return 0;
}

/* Prefill page fill ("Hours of YouTube and 85 handtyped pages of notes on LLM
 * Inference - Start here", section "これまでの進捗", page-pool bullet: the
 * prefill fills the prompt's pages).  The prompt rows are packed: sequence s
 * owns rows cu_tokens[s] .. cu_tokens[s+1]-1, and its row i is the token at
 * position start_pos[s] + i.  The fill is defined as the decode append of
 * each token in turn, with context length = its position + 1.  q may be NULL
 * (then only K/V are written).  Returns 0, or the first append's error. */
int pkv_oracle_prefill(uint16_t* k_pool, uint16_t* v_pool, int64_t num_pages, int64_t page_stride,
                       int64_t head_stride, int64_t slot_stride, const int32_t* block_table,
                       int64_t bt_stride, const int32_t* start_pos, const int32_t* cu_tokens,
                       int32_t num_seqs, uint16_t* q, int64_t q_stride, const uint16_t* k,
                       int64_t k_stride, const uint16_t* v, int64_t v_stride,
                       const float* rope_cos, const float* rope_sin, int32_t max_pos) {
    uint16_t scratch_q[HQ * HD];
    for (int32_t s = 0; s < num_seqs; ++s) {
        for (int32_t row = cu_tokens[s]; row < cu_tokens[s + 1]; ++row) {
            const int32_t n = start_pos[s] + (row - cu_tokens[s]) + 1;
            uint16_t* qrow = scratch_q;
            if (q) {
                qrow = q + (int64_t)row * q_stride;
            } else {
                memset(scratch_q, 0, sizeof scratch_q);
            }
            const int rc = pkv_oracle_append(
                k_pool, v_pool, num_pages, page_stride, head_stride, slot_stride,
                block_table + (int64_t)s * bt_stride, bt_stride, &n, 1, qrow, HQ * HD,
                k + (int64_t)row * k_stride, k_stride, v + (int64_t)row * v_stride, v_stride,
                rope_cos, rope_sin, max_pos);
            if (rc != 0) return rc;
        }
    }
    return 0;
}

/* ----------------------------------------------------------- attention -- */

/* out64 (may be NULL) and out32 (may be NULL) are [num_seqs][32*64] rows with
 * strides out64_stride / out32_stride.  Returns 0, or -1 when a page index
 * needed for a valid token is outside the pool. */
int pkv_oracle_attn(const uint16_t* k_pool, const uint16_t* v_pool, int64_t num_pages,
                    int64_t page_stride, int64_t head_stride, int64_t slot_stride,
                    const int32_t* block_table, int64_t bt_stride, const int32_t* ctx,
                    int32_t num_seqs, const uint16_t* q, int64_t q_stride, double scale,
                    double* out64, int64_t out64_stride, float* out32, int64_t out32_stride) {
    int32_t max_n = 0;
    for (int32_t s = 0; s < num_seqs; ++s)
        if (ctx[s] > max_n) max_n = ctx[s];
    double* z = (double*)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(max_n > 0 ? max_n : 1));
    if (!z || !w) {
        free(z);
        free(w);
        return -2;
    }
    int status = 0;
    for (int32_t s = 0; s < num_seqs && status == 0; ++s) {
        int32_t n = ctx[s];
        if (n > 0 && (n + PTOK - 1) / PTOK > bt_stride) { status = -1; break; }
        for (int h = 0; h < HQ; ++h) {
            int g = h / (HQ / HKV);
            double o[HD];
            for (int d = 0; d < HD; ++d) o[d] = 0.0;
            if (n > 0) {
                double qv[HD];
                for (int d = 0; d < HD; ++d)
                    qv[d] = pkv_oracle_bf16_to_f64(q[(int64_t)s * q_stride + (int64_t)h * HD + d]);
                /* pass 1: logits in logical order, and their maximum */
                double m = -INFINITY;
                for (int32_t tau = 0; tau < n; ++tau) {
                    int64_t page = block_table[(int64_t)s * bt_stride + tau / PTOK];
                    if (page < 0 || page >= num_pages) { status = -1; break; }
                    const uint16_t* kr =
                        k_pool + elem_offset(page, g, tau % PTOK, page_stride, head_stride, slot_stride);
                    double dot = 0.0;
                    for (int d = 0; d < HD; ++d) dot += qv[d] * pkv_oracle_bf16_to_f64(kr[d]);
                    z[tau] = scale * dot;
                    if (z[tau] > m) m = z[tau];
                }
                if (status != 0) break;
                /* pass 2: weights, their sum, and the weighted sum of V */
                double total = 0.0;
                for (int32_t tau = 0; tau < n; ++tau) {
                    w[tau] = exp(z[tau] - m);
                    total += w[tau];
                }
                for (int32_t tau = 0; tau < n; ++tau) {
                    int64_t page = block_table[(int64_t)s * bt_stride + tau / PTOK];
                    const uint16_t* vr =
                        v_pool + elem_offset(page, g, tau % PTOK, page_stride, head_stride, slot_stride);
                    for (int d = 0; d < HD; ++d) o[d] += w[tau] * pkv_oracle_bf16_to_f64(vr[d]);
                }
                for (int d = 0; d < HD; ++d) o[d] /= total;
            }
            for (int d = 0; d < HD; ++d) {
                if (out64) out64[(int64_t)s * out64_stride + (int64_t)h * HD + d] = o[d];
                if (out32) out32[(int64_t)s * out32_stride + (int64_t)h * HD + d] = (float)o[d];
            }
        }
    }
    free(z);
    free(w);
    return status;
}
