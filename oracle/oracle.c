/*
 * Quantized scaled-dot-product attention -- plain CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the reference the HIP library is checked
 * against; it is not part of the product. Only tests, the smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code, header, table or helper
 * with the GPU library, and the GPU library never links or calls it.
 *
 * Every function is a slow, direct statement of the arithmetic the source pages
 * define, in their order:
 *   - IEEE binary32 exactly where the method rounds (norm, rotation, scales, codes,
 *     the softmax exponent), so that INT8 codes, FP32 scales and k means are
 *     bit-exact targets;
 *   - binary64 where the method only accumulates (softmax sums, P.V, merges).
 * Build flags: -O2 -fno-fast-math -ffp-contract=off, so that every float operation
 * is one IEEE operation; fmaf() appears only where the method fuses.
 *
 * Sources (page titles; section / identifier on the page):
 *   [kit]   WanGP shared/attention_kit.py: HeadGroup.mean_squares, KVPrefix, GROUP,
 *           quantize_q8, dequantize_q8_into, _merge_lse_, _attend_with_prefix,
 *           joint_qkv_attention (mean squares by head groups).
 *   [quant] WanGP shared/kernels/qk_quant_triton.py: module docstring (layouts),
 *           _blocks / PADDED_ROWS, _rows, _norm_rope_quant, norm_rope_mean,
 *           norm_rope_quantize.
 *   [impl]  fastkernels L2/attention_impl.py: _repeat_kv_for_heads, _cache_seq,
 *           _sdpa_one, _decode_torch, _prefill_torch_from_cache.
 *   [tq]    vLLM triton_turboquant_unified_attention.py: the 2D kernel's online
 *           softmax (m_j, P, l_j, alpha, acc) and the 3D split-KV kernel.
 *
 * Readings where the pages are silent or disagree are stated at each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------
 * Number formats, from their definitions.
 * ---------------------------------------------------------------------------- */

static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16: the top 16 bits of a binary32. */
static float bf16_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest even (NaN kept quiet). */
static uint16_t f32_bf16(float f) {
    uint32_t u = f32_bits(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static float bf16_round(float f) { return bf16_f32(f32_bf16(f)); }

/* IEEE binary16 -> value. */
static double f16_value(uint16_t h) {
    int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* binary32 -> IEEE binary16, round to nearest even, overflow to infinity. */
static uint16_t f32_f16(float f) {
    uint16_t sign = (uint16_t)(signbit(f) ? 0x8000 : 0);
    double a = fabs((double)f);
    if (isnan(f)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;
    if (a < ldexp(1.0, -14)) {                 /* subnormal: quantum 2^-24 */
        double q = rint(ldexp(a, 24));         /* q == 1024 is the least normal */
        return sign | (uint16_t)q;
    }
    int E; frexp(a, &E);                       /* a = m 2^E, m in [0.5, 1) */
    int e = E - 1;
    double q = rint(ldexp(a, 10 - e));         /* in [1024, 2048] */
    if (q == 2048.0) { q = 1024.0; e += 1; }
    if (e > 15) return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

/* OCP FP8 e4m3fn value (bias 7, no infinities, S.1111.111 is NaN, max 448). */
static double e4m3_value(uint8_t b) {
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* binary32 -> e4m3fn, round to nearest even, saturating at +-448. */
static uint8_t f32_e4m3(float f) {
    uint8_t sign = (uint8_t)(signbit(f) ? 0x80 : 0);
    double a = fabs((double)f);
    if (isnan(f)) return 0x7f;
    if (a >= 448.0) return sign | 0x7e;
    if (a < ldexp(1.0, -6)) {                  /* subnormal: quantum 2^-9 */
        double q = rint(ldexp(a, 9));          /* q == 8 is the least normal */
        return sign | (uint8_t)q;
    }
    int E; frexp(a, &E);
    int e = E - 1;                              /* -6 .. 8 */
    double q = rint(ldexp(a, 3 - e));           /* in [8, 16] */
    if (q == 16.0) { q = 8.0; e += 1; }
    if (e > 8 || (e == 8 && q > 14.0)) return sign | 0x7e;
    return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));
}

/* exported for the format pins */
float orc_bf16_round(float f) { return bf16_round(f); }
uint16_t orc_f32_to_f16(float f) { return f32_f16(f); }
double orc_f16_value(uint16_t h) { return f16_value(h); }
uint8_t orc_f32_to_e4m3(float f) { return f32_e4m3(f); }
double orc_e4m3_value(uint8_t b) { return e4m3_value(b); }

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* threads of the OpenMP loops from now on (timing of the oracle on one core and on all) */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------------
 * Row prologue [quant] _rows: weighted RMSNorm in FP32 rounded to bf16, RoPE in
 * FP32 with one fused multiply-add per channel, minus the head mean, times the
 * softmax scale. Rows at or beyond the token count are zeros.
 * ---------------------------------------------------------------------------- */

enum { NORM_NONE = 0, NORM_HEAD = 1, NORM_ALL_HEADS = 2 };
enum { ROPE_NONE = 0, ROPE_SPLIT_HALF = 1, ROPE_INTERLEAVED = 2 };
enum { LAYOUT_PER_BLOCK = 0, LAYOUT_THREAD_Q = 1, LAYOUT_THREAD_K = 2, LAYOUT_WARP_Q = 3 };

typedef struct {
    int64_t B, T, H, D;
    const uint16_t* x;        /* (B, T, H, D) bf16 */
    int norm;                 /* NORM_* */
    const uint16_t* w;        /* (rows, D) per head, or (rows, H*D) over all heads; bf16 */
    const int32_t* wrows;     /* (T): weight row of each token, or NULL for row 0 */
    float eps;
    int rope;                 /* ROPE_* */
    const float* table;       /* cos at rb*b + rs*t + rp*pair, sin at cos + rc */
    int64_t pairs, rb, rs, rp, rc;
    const float* mean;        /* (B, H, D) FP32 or NULL */
    float sm_scale;
} orc_rows;

/*
 * Sum of squares of one row in the canonical order (reading: the pages fix the
 * order only for their own lane layout). The row splits into n = D/8 partial
 * sums; partial l takes channels 4l .. 4l+3 and then D/2 + 4l .. D/2 + 4l + 3 (each
 * channel with its split-half rotation partner): p = x*x for the first, then
 * p = fma(x, x, p) for the other 7 in that order. An xor butterfly over the n
 * partials (offsets n/2, ..., 1) then adds each partial to its partner; every
 * partial ends equal, and partial 0 is the sum.
 */
static float sumsq_canonical(const float* x, int64_t D) {
    int n = (int)(D / 8);
    float p[64], q[64];
    for (int l = 0; l < n; ++l) {
        int ch[8];
        for (int k = 0; k < 4; ++k) { ch[k] = 4 * l + k; ch[4 + k] = (int)(D / 2) + 4 * l + k; }
        float s = x[ch[0]] * x[ch[0]];
        for (int k = 1; k < 8; ++k) s = fmaf(x[ch[k]], x[ch[k]], s);
        p[l] = s;
    }
    for (int off = n / 2; off >= 1; off /= 2) {
        for (int l = 0; l < n; ++l) q[l] = p[l] + p[l ^ off];
        for (int l = 0; l < n; ++l) p[l] = q[l];
    }
    return p[0];
}

/*
 * Mean of squares of a token over all heads [kit] HeadGroup.mean_squares and the
 * mean squares by head groups in joint_qkv_attention: per head the canonical row
 * sum, heads added in ascending order from zero, divided by H*D. FP32, (B, T).
 */
void orc_mean_sq_all_heads(const uint16_t* x, int64_t B, int64_t T, int64_t H, int64_t D, float* ms) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t) {
            float tot = 0.0f, row[512];
            for (int64_t h = 0; h < H; ++h) {
                const uint16_t* xr = x + ((b * T + t) * H + h) * D;
                for (int64_t c = 0; c < D; ++c) row[c] = bf16_f32(xr[c]);
                tot = tot + sumsq_canonical(row, D);
            }
            ms[b * T + t] = tot / (float)(H * D);
        }
}

/* z = the prologue of row (b, t, h) without mean and scale; ms: the all-heads
 * mean squares of this token when the norm spans all heads. */
static void prologue_rotated(const orc_rows* r, int64_t b, int64_t t, int64_t h, float ms_all, float* z) {
    const int64_t D = r->D;
    float x[512], y[512];
    const uint16_t* xr = r->x + ((b * r->T + t) * r->H + h) * D;
    for (int64_t c = 0; c < D; ++c) x[c] = bf16_f32(xr[c]);
    if (r->norm == NORM_NONE) {
        for (int64_t c = 0; c < D; ++c) y[c] = x[c];
    } else {
        float ms, wd;
        const uint16_t* w;
        int64_t row = r->wrows ? r->wrows[t] : 0;
        if (r->norm == NORM_HEAD) {
            ms = sumsq_canonical(x, D) / (float)D;
            w = r->w + row * D;
        } else {
            ms = ms_all;
            w = r->w + row * (r->H * D) + h * D;
        }
        float inv = 1.0f / sqrtf(ms + r->eps);
        for (int64_t c = 0; c < D; ++c) {
            wd = bf16_f32(w[c]);
            y[c] = bf16_round((x[c] * inv) * wd);   /* norm output in the activation dtype */
        }
    }
    if (r->rope == ROPE_NONE) {
        for (int64_t c = 0; c < D; ++c) z[c] = y[c];
        return;
    }
    const int64_t P = r->pairs;
    for (int64_t c = 0; c < D; ++c) {
        if (c >= 2 * P) { z[c] = y[c]; continue; }
        int64_t partner, pair;
        int leading;
        if (r->rope == ROPE_INTERLEAVED) {          /* channel 2p with 2p + 1 */
            leading = (c % 2) == 0;
            partner = c ^ 1;
            pair = c / 2;
        } else {                                     /* channel p with p + P */
            leading = c < P;
            partner = leading ? c + P : c - P;
            pair = leading ? c : c - P;
        }
        const float* a = r->table + r->rb * b + r->rs * t + r->rp * pair;
        float cs = a[0], sn = a[r->rc];
        if (leading) z[c] = fmaf(cs, y[c], (-sn) * y[partner]);
        else z[c] = fmaf(sn, y[partner], cs * y[c]);
    }
}

/* v = the full prologue: rotated row, minus the head mean, times sm_scale. */
static void prologue(const orc_rows* r, int64_t b, int64_t t, int64_t h, float ms_all, float* v) {
    const int64_t D = r->D;
    if (t >= r->T) { for (int64_t c = 0; c < D; ++c) v[c] = 0.0f; return; }
    prologue_rotated(r, b, t, h, ms_all, v);
    if (r->mean) {
        const float* mu = r->mean + (b * r->H + h) * D;
        for (int64_t c = 0; c < D; ++c) v[c] = v[c] - mu[c];
    }
    for (int64_t c = 0; c < D; ++c) v[c] = v[c] * r->sm_scale;
}

static float* all_heads_ms(const orc_rows* r) {
    if (r->norm != NORM_ALL_HEADS) return NULL;
    float* ms = (float*)malloc(sizeof(float) * (size_t)(r->B * r->T));
    orc_mean_sq_all_heads(r->x, r->B, r->T, r->H, r->D, ms);
    return ms;
}

/* The rotated rows of (b, h) for all tokens, without mean and scale; used by the
 * k mean. Exported so that the tests can check the norm and rotation alone. */
void orc_prologue_rows(const orc_rows* r, float* out /* (B, T, H, D) */) {
    float* ms = all_heads_ms(r);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < r->B; ++b)
        for (int64_t t = 0; t < r->T; ++t)
            for (int64_t h = 0; h < r->H; ++h)
                prologue(r, b, t, h, ms ? ms[b * r->T + t] : 0.0f, out + ((b * r->T + t) * r->H + h) * r->D);
    free(ms);
}

/* ------------------------------------------------------------------------------
 * k mean [quant] norm_rope_mean: the mean over tokens of the normalized, rotated
 * rows per (batch, head), from FP32 partial sums per block of 64 rows.
 * Canonical order (reading; the pages fix only "FP32 partials per block, then a
 * sum over blocks, divided by the token count"): in a block, row t = 4i + r
 * (i = 0..15) joins partial S_r in ascending i, from zero; the block's partial is
 * (S_0 + S_1) + (S_2 + S_3); the blocks are added in chunks of 16 consecutive
 * blocks (ascending within a chunk, from zero), the chunk sums in ascending order
 * from zero; the total is divided by T. Rows at or beyond T add zero.
 * ---------------------------------------------------------------------------- */
void orc_kmean(const orc_rows* rin, float* mean /* (B, H, D) */) {
    orc_rows r = *rin;
    r.mean = NULL;
    r.sm_scale = 1.0f;
    float* ms = all_heads_ms(&r);
    const int64_t D = r.D, nblk = (r.T + 63) / 64;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < r.B; ++b)
        for (int64_t h = 0; h < r.H; ++h) {
            float total[512], chunk[512], S[4][512], z[512];
            for (int64_t c = 0; c < D; ++c) total[c] = chunk[c] = 0.0f;
            for (int64_t blk = 0; blk < nblk; ++blk) {
                for (int k = 0; k < 4; ++k)
                    for (int64_t c = 0; c < D; ++c) S[k][c] = 0.0f;
                for (int i = 0; i < 16; ++i)
                    for (int k = 0; k < 4; ++k) {
                        int64_t t = blk * 64 + 4 * i + k;
                        prologue(&r, b, t, h, (ms && t < r.T) ? ms[b * r.T + t] : 0.0f, z);
                        for (int64_t c = 0; c < D; ++c) S[k][c] = S[k][c] + z[c];
                    }
                for (int64_t c = 0; c < D; ++c) chunk[c] = chunk[c] + ((S[0][c] + S[1][c]) + (S[2][c] + S[3][c]));
                if (blk % 16 == 15 || blk == nblk - 1)
                    for (int64_t c = 0; c < D; ++c) { total[c] = total[c] + chunk[c]; chunk[c] = 0.0f; }
            }
            for (int64_t c = 0; c < D; ++c) mean[(b * r.H + h) * D + c] = total[c] / (float)r.T;
        }
    free(ms);
}

/* ------------------------------------------------------------------------------
 * Row groups of the scale layouts [quant] module docstring, SCALES_PER_BLOCK,
 * PADDED_ROWS and _blocks; scale index of token t.
 * ---------------------------------------------------------------------------- */
int64_t orc_scale_count(int64_t T, int layout, int block) {
    switch (layout) {
    case LAYOUT_PER_BLOCK: return (T + block - 1) / block;
    case LAYOUT_THREAD_Q: return ((T + 127) / 128) * 4 * 8;   /* 32-row blocks padded to 128 rows */
    case LAYOUT_THREAD_K: return ((T + 63) / 64) * 4;
    case LAYOUT_WARP_Q: return ((T + 127) / 128) * 4;
    }
    return -1;
}

int64_t orc_scale_index(int64_t t, int layout, int block) {
    switch (layout) {
    case LAYOUT_PER_BLOCK: return t / block;
    case LAYOUT_THREAD_Q: return 8 * (t / 32) + t % 8;          /* rows r, r+8, r+16, r+24 */
    case LAYOUT_THREAD_K: return 4 * (t / 64) + (t % 8) / 2;    /* row pairs */
    case LAYOUT_WARP_Q: return 4 * (t / 128) + (t % 128) / 32;  /* 32 consecutive rows */
    }
    return -1;
}

/*
 * q/k quantization [quant] _norm_rope_quant: per group the largest |v| over its
 * rows and channels; scale = amax / 127 + scale_eps (two FP32 roundings; the
 * division correctly rounded -- reading: the pages' approximate division is the
 * hardware of the pages, not the method); code r = v / scale, then r + 0.5 or
 * r - 0.5 by the sign of r (r >= 0 counts as positive), then truncation toward
 * zero. Every group up to the scale count is written (tail groups of the padded
 * THREAD_Q rows get scale_eps). A group whose scale is zero (all-zero rows with
 * scale_eps = 0) gets codes 0 (reading: the pages leave 0/0 undefined).
 */
void orc_quant_qk(const orc_rows* r, int layout, int block, float scale_eps,
                  int8_t* codes /* (B, T, H, D) */, float* scales /* (B, H, nscale) */) {
    float* ms = all_heads_ms(r);
    const int64_t D = r->D, T = r->T, nscale = orc_scale_count(T, layout, block);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < r->B; ++b)
        for (int64_t h = 0; h < r->H; ++h) {
            float* v = (float*)malloc(sizeof(float) * (size_t)(T * D));
            float* amax = (float*)calloc((size_t)nscale, sizeof(float));
            float* sc = scales + (b * r->H + h) * nscale;
            for (int64_t t = 0; t < T; ++t) {
                prologue(r, b, t, h, ms ? ms[b * T + t] : 0.0f, v + t * D);
                int64_t g = orc_scale_index(t, layout, block);
                for (int64_t c = 0; c < D; ++c) amax[g] = fmaxf(amax[g], fabsf(v[t * D + c]));
            }
            for (int64_t g = 0; g < nscale; ++g) sc[g] = amax[g] / 127.0f + scale_eps;
            for (int64_t t = 0; t < T; ++t) {
                float s = sc[orc_scale_index(t, layout, block)];
                int8_t* out = codes + ((b * T + t) * r->H + h) * D;
                for (int64_t c = 0; c < D; ++c) {
                    float q = v[t * D + c] / s;
                    q = (q >= 0.0f) ? q + 0.5f : q - 0.5f;
                    out[c] = isnan(q) ? (int8_t)0 : (int8_t)truncf(q);
                }
            }
            free(v);
            free(amax);
        }
    free(ms);
}

/* ------------------------------------------------------------------------------
 * V to FP8 (reading of "P.V FP8 e4m3 with per-channel v scales"): per (batch,
 * head, channel) vs = max(amax over tokens / 448, 1e-8); codes e4m3fn(v / vs),
 * round to nearest even, saturating at 448. Codes (B, T, H, D), scales (B, H, D).
 * ---------------------------------------------------------------------------- */
void orc_quant_v_fp8(const uint16_t* v, int64_t B, int64_t T, int64_t H, int64_t D,
                     uint8_t* codes, float* vs) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t c = 0; c < D; ++c) {
                float amax = 0.0f;
                for (int64_t t = 0; t < T; ++t) amax = fmaxf(amax, fabsf(bf16_f32(v[((b * T + t) * H + h) * D + c])));
                float s = fmaxf(amax / 448.0f, 1e-8f);
                vs[(b * H + h) * D + c] = s;
                for (int64_t t = 0; t < T; ++t) {
                    int64_t i = ((b * T + t) * H + h) * D + c;
                    codes[i] = f32_e4m3(bf16_f32(v[i]) / s);
                }
            }
}

/* ------------------------------------------------------------------------------
 * Attention core, quantized mode. For query row i of head h (kv head
 * h / (H / Hk), [impl] _repeat_kv_for_heads), walk the keys in tiles of kv_tile
 * ([tq] online softmax):
 *   a = integer dot of the q and k codes (exact);
 *   c = RN(qs * ks), times score_scale when it is not 1 (log2 units: the q rows
 *       carry log2(e)/sqrt(D));
 *   s = RN(a * c);  m' = max(m, max over the tile of s);
 *   p = RN(2^fma(a, c, -m'))  (the correctly rounded exp2 of the FP32 exponent);
 *   alpha = RN(2^RN(m - m')), 0 while m is -inf;
 *   l = l * alpha + sum p  (l from the unrounded p, as the [tq] kernel sums P
 *       before converting it for the dot);
 *   acc = acc * alpha + sum Pt * Vt, with Pt = bf16(p), Vt = v (bf16 P.V), or
 *       Pt = e4m3(256 p), Vt = the e4m3 v codes (FP8 P.V; reading: a power-of-two
 *       P scale keeps the scaling exact, and e4m3 precision is relative);
 *   out = acc / l (bf16), acc * vs / (256 l) (FP8); lse = m + log2 l (base 2).
 * Sums and products after p are binary64 (their order is not part of the method).
 *
 * allow: for each (i, j), if p moved by a relative flip_rel (the exp2 of the
 * hardware is within a few ulps, not correctly rounded) changes Pt, the largest
 * change |dPt| * |Vt_jc| joins a flip allowance, rescaled and normalized like
 * acc. The GPU result may differ from out by at most tolerance + allow.
 * FP8 P.V adds a second allowance for the reduced-precision sum of an FP8 dot
 * product (reading: an FP8 matrix unit may add a run of 8 consecutive products
 * aligned to the largest of them, keeping 13 bits below its leading bit, as the
 * 8-bit products carry at most 8 significant bits). Keys j = 8m .. 8m+7 form a
 * run; with E the exponent of the run's largest |Pt Vt| and u = 2^(E - 13), a
 * product that is not a multiple of u may lose up to min(|Pt Vt|, u).
 * ---------------------------------------------------------------------------- */
typedef struct {
    int64_t B, S, H, D;       /* codes (B, S, H, D) */
    const int8_t* codes;
    const float* scales;      /* (B, H, nscale) */
    int layout, block;
} orc_qk;

static double pt_value(double p, int fp8) {
    float pf = (float)p;
    return fp8 ? e4m3_value(f32_e4m3(pf * 256.0f)) : (double)bf16_round(pf);
}

/* Bound of what a run of products loses when it is summed on a grid of 2^(E - 13),
 * E the exponent of the run's largest magnitude (see the FP8 allowance above). */
static double run_truncation_bound(const double* prod, int64_t n) {
    double mx = 0.0, lost = 0.0;
    for (int64_t j = 0; j < n; ++j) mx = fmax(mx, fabs(prod[j]));
    if (mx == 0.0) return 0.0;
    int E;
    frexp(mx, &E);                          /* mx = f 2^E, f in [0.5, 1): leading bit 2^(E-1) */
    const double u = ldexp(1.0, E - 1 - 13);
    for (int64_t j = 0; j < n; ++j) {
        double a = fabs(prod[j]);
        if (fmod(a, u) != 0.0) lost += fmin(a, u);
    }
    return lost;
}

/* exported for the pin of the FP8 dot-product reading (a run of products given directly) */
double orc_run_truncation_bound(const double* prod, int64_t n) { return run_truncation_bound(prod, n); }

static double pt_flip(float p, int fp8, double flip_rel) {
    double base = pt_value(p, fp8);
    double lo = pt_value((double)p * (1.0 - flip_rel), fp8);
    double hi = pt_value((double)p * (1.0 + flip_rel), fp8);
    return fmax(fabs(lo - base), fabs(hi - base));
}

void orc_attn(const orc_qk* q, const orc_qk* k,
              const void* v, int fp8, const float* vs,
              float score_scale, int kv_tile, double flip_rel,
              int causal, const float* sinks /* (H,) natural-log logits or NULL */,
              const int64_t* rows, int64_t nrows,
              double* out /* (B, nrows, H, D) */, double* lse /* (B, H, nrows) */,
              double* allow /* (B, nrows, H, D) or NULL */,
              double* allow_run /* (B, nrows, H, D) or NULL: the FP8 run part of allow alone */) {
    const int64_t B = q->B, H = q->H, D = q->D, Sk = k->S, Hk = k->H, G = H / Hk;
    const int64_t off = Sk - q->S;   /* causal: query i sees keys 0 .. i + Sk - Sq */
    const int64_t nq = orc_scale_count(q->S, q->layout, q->block);
    const int64_t nk = orc_scale_count(Sk, k->layout, k->block);
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t ri = 0; ri < nrows; ++ri) {
                const int64_t i = rows[ri], hk = h / G;
                const int8_t* qc = q->codes + ((b * q->S + i) * H + h) * D;
                const float qs = q->scales[(b * H + h) * nq + orc_scale_index(i, q->layout, q->block)];
                double acc[512], al[512], ar[512];
                float* a = (float*)malloc(sizeof(float) * (size_t)kv_tile);
                float* c = (float*)malloc(sizeof(float) * (size_t)kv_tile);
                double* ptv = (double*)malloc(sizeof(double) * (size_t)kv_tile);
                for (int64_t d = 0; d < D; ++d) acc[d] = al[d] = ar[d] = 0.0;
                /* [tq] sinks: the softmax starts from M = the head's sink logit (base 2 here:
                 * RN(s_h * log2 e) in FP32), L = 1, so the sink joins the denominator only */
                float m = sinks ? sinks[h] * 1.44269504f : -INFINITY;
                double l = sinks ? 1.0 : 0.0;
                const int64_t kend = causal ? (i + off + 1 < Sk ? i + off + 1 : Sk) : Sk;
                for (int64_t j0 = 0; j0 < kend; j0 += kv_tile) {
                    int64_t n = kend - j0 < kv_tile ? kend - j0 : kv_tile;
                    float mt = -INFINITY;
                    for (int64_t jj = 0; jj < n; ++jj) {
                        int64_t j = j0 + jj;
                        const int8_t* kc = k->codes + ((b * Sk + j) * Hk + hk) * D;
                        int64_t dot = 0;
                        for (int64_t d = 0; d < D; ++d) dot += (int64_t)qc[d] * (int64_t)kc[d];
                        float ks = k->scales[(b * Hk + hk) * nk + orc_scale_index(j, k->layout, k->block)];
                        float cc = qs * ks;
                        if (score_scale != 1.0f) cc = cc * score_scale;
                        a[jj] = (float)dot;     /* |dot| <= 127^2 * 512 < 2^24: exact */
                        c[jj] = cc;
                        float s = a[jj] * cc;
                        mt = fmaxf(mt, s);
                    }
                    float mn = fmaxf(m, mt);
                    double alpha = (m == -INFINITY) ? 0.0 : (double)(float)exp2((double)(m - mn));
                    for (int64_t d = 0; d < D; ++d) { acc[d] *= alpha; al[d] *= alpha; ar[d] *= alpha; }
                    l *= alpha;
                    for (int64_t jj = 0; jj < n; ++jj) {
                        int64_t j = j0 + jj;
                        float p = (float)exp2((double)fmaf(a[jj], c[jj], -mn));
                        l += (double)p;
                        double pt = pt_value(p, fp8);
                        double fl = allow ? pt_flip(p, fp8, flip_rel) : 0.0;
                        ptv[jj] = pt;
                        for (int64_t d = 0; d < D; ++d) {
                            int64_t vi = ((b * Sk + j) * Hk + hk) * D + d;
                            double vt = fp8 ? e4m3_value(((const uint8_t*)v)[vi]) : (double)bf16_f32(((const uint16_t*)v)[vi]);
                            acc[d] += pt * vt;
                            al[d] += fl * fabs(vt);
                        }
                    }
                    if (allow && fp8) {
                        /* runs of 8 keys from key indices 8m (tiles start at multiples of 8) */
                        for (int64_t d = 0; d < D; ++d)
                            for (int64_t r0 = 0; r0 < n; r0 += 8) {
                                double prod[8];
                                int64_t rn = n - r0 < 8 ? n - r0 : 8;
                                for (int64_t u = 0; u < rn; ++u) {
                                    int64_t vi = ((b * Sk + j0 + r0 + u) * Hk + hk) * D + d;
                                    prod[u] = ptv[r0 + u] * e4m3_value(((const uint8_t*)v)[vi]);
                                }
                                const double lost = run_truncation_bound(prod, rn);
                                al[d] += lost;
                                ar[d] += lost;
                            }
                    }
                    m = mn;
                }
                for (int64_t d = 0; d < D; ++d) {
                    double f = fp8 ? (double)vs[(b * Hk + hk) * D + d] / (256.0 * l) : 1.0 / l;
                    out[((b * nrows + ri) * H + h) * D + d] = acc[d] * f;
                    if (allow) allow[((b * nrows + ri) * H + h) * D + d] = al[d] * f;
                    if (allow_run) allow_run[((b * nrows + ri) * H + h) * D + d] = ar[d] * f;
                }
                lse[(b * H + h) * nrows + ri] = (double)m + log2(l);
                free(a);
                free(c);
                free(ptv);
            }
}

/* ------------------------------------------------------------------------------
 * Cached q8 prefix pass and log-sum-exp merge [kit] KVPrefix, dequantize_q8_into,
 * _attend_with_prefix, _merge_lse_. The prefix keys are attended in a pass of
 * their own with the same query codes; their scores share the projected keys'
 * offset (reading of the native-prefix rule "the keys attended with it subtract
 * the prefix mean too"): s = qh . (kh - mu), qh = qc * qs, kh = kc * ks16 per
 * 32-channel group, evaluated in binary64 with no rounding points. Softmax tiles
 * as the core; Vt = bf16(vc * vs16) (16-bit dequantization), Pt = bf16(p).
 * Merge in binary64: top = max(a, b); wa = 2^(a - top); wb = 2^(b - top);
 * out = out_a wa / (wa + wb) + out_b wb / (wa + wb); lse = top + log2(wa + wb).
 * Both -inf: out 0, lse -inf (reading: the pages never meet it).
 * ---------------------------------------------------------------------------- */
typedef struct {
    int64_t B, P, H, D;                 /* codes (B or 1, P, H, D) */
    const int8_t* k; const uint16_t* ks;   /* ks (B or 1, P, H, D/32) FP16 */
    const int8_t* v; const uint16_t* vs;
} orc_q8prefix;

void orc_prefix_merge(const orc_qk* q, const orc_q8prefix* pf, const float* mu /* (B, Hk, D) or NULL */,
                      float score_scale, int kv_tile, double flip_rel,
                      const float* out_in /* (B, Sq, H, D) */, const float* lse_in /* (B, H, Sq) */,
                      const int64_t* rows, int64_t nrows,
                      double* out, double* lse, double* allow,
                      double* prefix_out /* (B, nrows, H, D) or NULL */, double* prefix_lse /* or NULL */) {
    const int64_t B = q->B, H = q->H, D = q->D, Hk = pf->H, G = H / Hk, P = pf->P, NG = D / 32;
    const int64_t nq = orc_scale_count(q->S, q->layout, q->block);
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t ri = 0; ri < nrows; ++ri) {
                const int64_t i = rows[ri], hk = h / G, bp = pf->B == 1 ? 0 : b;
                const int8_t* qc = q->codes + ((b * q->S + i) * H + h) * D;
                const double qs = q->scales[(b * H + h) * nq + orc_scale_index(i, q->layout, q->block)];
                double delta = 0.0, acc[512], al[512];
                if (mu)
                    for (int64_t d = 0; d < D; ++d) delta += (double)qc[d] * qs * (double)mu[(b * Hk + hk) * D + d];
                double* s = (double*)malloc(sizeof(double) * (size_t)kv_tile);
                for (int64_t d = 0; d < D; ++d) acc[d] = al[d] = 0.0;
                double m = -INFINITY, l = 0.0;
                for (int64_t j0 = 0; j0 < P; j0 += kv_tile) {
                    int64_t n = P - j0 < kv_tile ? P - j0 : kv_tile;
                    double mt = -INFINITY;
                    for (int64_t jj = 0; jj < n; ++jj) {
                        int64_t j = j0 + jj;
                        const int8_t* kc = pf->k + ((bp * P + j) * Hk + hk) * D;
                        const uint16_t* ks = pf->ks + ((bp * P + j) * Hk + hk) * NG;
                        double sum = 0.0;
                        for (int64_t g = 0; g < NG; ++g) {
                            int64_t dot = 0;
                            for (int64_t d = 32 * g; d < 32 * g + 32; ++d) dot += (int64_t)qc[d] * (int64_t)kc[d];
                            sum += f16_value(ks[g]) * (double)dot;
                        }
                        s[jj] = (qs * sum - delta) * (double)score_scale;
                        mt = fmax(mt, s[jj]);
                    }
                    double mn = fmax(m, mt);
                    double alpha = (m == -INFINITY) ? 0.0 : exp2(m - mn);
                    for (int64_t d = 0; d < D; ++d) { acc[d] *= alpha; al[d] *= alpha; }
                    l *= alpha;
                    for (int64_t jj = 0; jj < n; ++jj) {
                        int64_t j = j0 + jj;
                        float p = (float)exp2(s[jj] - mn);
                        l += (double)p;
                        double pt = pt_value(p, 0), fl = pt_flip(p, 0, flip_rel);
                        const int8_t* vc = pf->v + ((bp * P + j) * Hk + hk) * D;
                        const uint16_t* vsc = pf->vs + ((bp * P + j) * Hk + hk) * NG;
                        for (int64_t d = 0; d < D; ++d) {
                            double vt = (double)bf16_round((float)vc[d] * (float)f16_value(vsc[d / 32]));
                            acc[d] += pt * vt;
                            al[d] += fl * fabs(vt);
                        }
                    }
                    m = mn;
                }
                double pl = m + log2(l);
                double a = lse_in[(b * H + h) * q->S + i];
                double top = fmax(a, pl);
                double wa, wb;
                if (top == -INFINITY) { wa = 0.0; wb = 0.0; }
                else { wa = exp2(a - top); wb = exp2(pl - top); }
                double tot = wa + wb;
                for (int64_t d = 0; d < D; ++d) {
                    int64_t o = ((b * nrows + ri) * H + h) * D + d;
                    double po = acc[d] / l;
                    if (prefix_out) prefix_out[o] = po;
                    if (tot == 0.0) { out[o] = 0.0; if (allow) allow[o] = 0.0; continue; }
                    out[o] = (double)out_in[((b * q->S + i) * H + h) * D + d] * (wa / tot) + po * (wb / tot);
                    if (allow) allow[o] = al[d] / l * (wb / tot);
                }
                if (prefix_lse) prefix_lse[(b * H + h) * nrows + ri] = pl;
                lse[(b * H + h) * nrows + ri] = tot == 0.0 ? -INFINITY : top + log2(tot);
                free(s);
            }
}

/* ------------------------------------------------------------------------------
 * q8 format [kit] quantize_q8: per 32 channels scale = max(amax / 127, 1e-8) in
 * FP32; codes clamp(round-half-even(x / scale), -127, 127) from the FP32 scale;
 * the scale is stored FP16. x (rows, D) FP32.
 * ---------------------------------------------------------------------------- */
void orc_q8_quantize(const float* x, int64_t rows, int64_t D, int8_t* codes, uint16_t* scales) {
    const int64_t NG = D / 32;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t g = 0; g < NG; ++g) {
            const float* xs = x + r * D + 32 * g;
            float amax = 0.0f;
            for (int c = 0; c < 32; ++c) amax = fmaxf(amax, fabsf(xs[c]));
            float s = fmaxf(amax / 127.0f, 1e-8f);
            for (int c = 0; c < 32; ++c) {
                float q = rintf(xs[c] / s);
                if (q > 127.0f) q = 127.0f;
                if (q < -127.0f) q = -127.0f;
                codes[r * D + 32 * g + c] = (int8_t)q;
            }
            scales[r * NG + g] = f32_f16(s);
        }
}

/* ------------------------------------------------------------------------------
 * Paged decode over a q8 cache [impl] _cache_seq, _sdpa_one, _decode_torch,
 * _repeat_kv_for_heads; [tq] block-table addressing. Sequence n of length L
 * attends positions 0..L-1 (its one query sits at L - 1, so the causal mask
 * keeps them all). Position pos lives in physical block block_table[n][pos / bs],
 * slot pos % bs. Keys and values are the exact q8 values code * fp16 scale;
 * binary64 softmax of (q . k) * scale. Caches [NB, bs, Hk, D], scales
 * [NB, bs, Hk, D/32]; q (N, Hq, D) bf16, or binary16 when q_f16; out (N, Hq, D).
 * ---------------------------------------------------------------------------- */
/* A query element: bf16, or IEEE binary16 when q_f16 (both exact in binary64). */
static double q_value(const uint16_t* q, int64_t i, int q_f16) {
    return q_f16 ? f16_value(q[i]) : (double)bf16_f32(q[i]);
}

void orc_paged_decode(const uint16_t* q, int q_f16, const int8_t* kc, const uint16_t* ks,
                      const int8_t* vc, const uint16_t* vsc, int64_t bs, int64_t Hk,
                      const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                      int64_t N, int64_t Hq, int64_t D, double scale,
                      const float* sinks /* (Hq,) natural-log logits or NULL */, double* out) {
    const int64_t G = Hq / Hk, NG = D / 32;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t hk = h / G, L = seq_lens[n];
            double* s = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
            double m = -INFINITY, l = 0.0, acc[512];
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t pos = 0; pos < L; ++pos) {
                int64_t phys = block_table[n * bt_stride + pos / bs], slot = pos % bs;
                int64_t base = (phys * bs + slot) * Hk + hk;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += q_value(q, (n * Hq + h) * D + d, q_f16) * ((double)kc[base * D + d] * f16_value(ks[base * NG + d / 32]));
                s[pos] = dot * scale;
                m = fmax(m, s[pos]);
            }
            /* [tq] sinks: exp(s_h) joins the denominator only */
            if (sinks) m = fmax(m, (double)sinks[h]);
            if (sinks) l = exp((double)sinks[h] - m);
            for (int64_t pos = 0; pos < L; ++pos) {
                int64_t phys = block_table[n * bt_stride + pos / bs], slot = pos % bs;
                int64_t base = (phys * bs + slot) * Hk + hk;
                double p = exp(s[pos] - m);
                l += p;
                for (int64_t d = 0; d < D; ++d) acc[d] += p * ((double)vc[base * D + d] * f16_value(vsc[base * NG + d / 32]));
            }
            for (int64_t d = 0; d < D; ++d) out[(n * Hq + h) * D + d] = L > 0 ? acc[d] / l : 0.0;
            free(s);
        }
}

/* ------------------------------------------------------------------------------
 * Paged (chunked) causal prefill over a q8 cache [impl] _prefill_torch_from_cache,
 * _cache_seq, _sdpa_one, _repeat_kv_for_heads; [tq] unified 2D kernel (varlen queries
 * by query_start_len, seq_lens = context + query length, sinks). Sequence n owns the
 * query tokens [query_start[n], query_start[n+1]) (q_len of them) and the keys at
 * positions 0..seq_lens[n]-1 of its paged cache; its query j sits at position
 * key_offset + j, key_offset = seq_lens[n] - q_len, and attends the keys at positions
 * 0..key_offset + j (the mask k_pos <= key_offset + q_pos). Keys and values are the exact
 * q8 values code * fp16 scale; binary64 softmax of (q . k) * scale; a sink adds exp(sink)
 * to the denominator only. rows: the query tokens to compute (NULL: all T of them);
 * out (nrows, Hq, D). q (T, Hq, D) bf16 (binary16 when q_f16) contiguous.
 * ---------------------------------------------------------------------------- */
void orc_paged_prefill(const uint16_t* q, int q_f16, const int8_t* kc, const uint16_t* ks,
                       const int8_t* vc, const uint16_t* vsc, int64_t bs, int64_t Hk,
                       const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                       const int32_t* query_start, int64_t N, int64_t Hq, int64_t D, double scale,
                       const float* sinks, const int64_t* rows, int64_t nrows, double* out) {
    const int64_t G = Hq / Hk, NG = D / 32;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t r = 0; r < nrows; ++r)
        for (int64_t h = 0; h < Hq; ++h) {
            const int64_t t = rows ? rows[r] : r;
            int64_t n = 0;
            while (n + 1 < N && query_start[n + 1] <= t) ++n;     /* the sequence that owns token t */
            const int64_t q_len = query_start[n + 1] - query_start[n];
            const int64_t k_len = seq_lens[n];
            const int64_t key_offset = k_len - q_len;
            const int64_t j = t - query_start[n];
            const int64_t last = key_offset + j;                  /* keys 0..last are visible */
            const int64_t hk = h / G;
            double* s = (double*)malloc(sizeof(double) * (size_t)(last + 1));
            double m = -INFINITY, l = 0.0, acc[512];
            for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t pos = 0; pos <= last; ++pos) {
                int64_t phys = block_table[n * bt_stride + pos / bs], slot = pos % bs;
                int64_t base = (phys * bs + slot) * Hk + hk;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += q_value(q, (t * Hq + h) * D + d, q_f16) * ((double)kc[base * D + d] * f16_value(ks[base * NG + d / 32]));
                s[pos] = dot * scale;
                m = fmax(m, s[pos]);
            }
            if (sinks) m = fmax(m, (double)sinks[h]);
            if (sinks) l = exp((double)sinks[h] - m);
            for (int64_t pos = 0; pos <= last; ++pos) {
                int64_t phys = block_table[n * bt_stride + pos / bs], slot = pos % bs;
                int64_t base = (phys * bs + slot) * Hk + hk;
                double p = exp(s[pos] - m);
                l += p;
                for (int64_t d = 0; d < D; ++d) acc[d] += p * ((double)vc[base * D + d] * f16_value(vsc[base * NG + d / 32]));
            }
            for (int64_t d = 0; d < D; ++d) out[(r * Hq + h) * D + d] = acc[d] / l;
            free(s);
        }
}

/* ------------------------------------------------------------------------------
 * Unquantized attention in binary64 (the accuracy target): the same bf16 q, k, v;
 * norm and rotation in binary64 without the bf16 rounding; no mean; natural-base
 * softmax of q . k / sqrt(D) ([impl] _sdpa_one without mask); optionally a q8
 * prefix put before the keys ([kit] joint attention "keys and values computed
 * beforehand ... put before the projected ones"), at its exact q8 values.
 * ---------------------------------------------------------------------------- */
static void prologue_f64(const orc_rows* r, int64_t b, int64_t t, int64_t h, double ms_all, double* z) {
    const int64_t D = r->D;
    double x[512], y[512];
    const uint16_t* xr = r->x + ((b * r->T + t) * r->H + h) * D;
    for (int64_t c = 0; c < D; ++c) x[c] = bf16_f32(xr[c]);
    if (r->norm == NORM_NONE) {
        for (int64_t c = 0; c < D; ++c) y[c] = x[c];
    } else {
        int64_t row = r->wrows ? r->wrows[t] : 0;
        double ms = 0.0;
        const uint16_t* w;
        if (r->norm == NORM_HEAD) {
            for (int64_t c = 0; c < D; ++c) ms += x[c] * x[c];
            ms /= (double)D;
            w = r->w + row * D;
        } else {
            ms = ms_all;
            w = r->w + row * (r->H * D) + h * D;
        }
        double inv = 1.0 / sqrt(ms + (double)r->eps);
        for (int64_t c = 0; c < D; ++c) y[c] = x[c] * inv * (double)bf16_f32(w[c]);
    }
    for (int64_t c = 0; c < D; ++c) z[c] = y[c];
    if (r->rope == ROPE_NONE) return;
    for (int64_t c = 0; c < 2 * r->pairs; ++c) {
        int64_t partner, pair;
        int leading;
        if (r->rope == ROPE_INTERLEAVED) { leading = (c % 2) == 0; partner = c ^ 1; pair = c / 2; }
        else { leading = c < r->pairs; partner = leading ? c + r->pairs : c - r->pairs; pair = leading ? c : c - r->pairs; }
        const float* a = r->table + r->rb * b + r->rs * t + r->rp * pair;
        double cs = a[0], sn = a[r->rc];
        z[c] = leading ? cs * y[c] - sn * y[partner] : sn * y[partner] + cs * y[c];
    }
}

static double* all_heads_ms_f64(const orc_rows* r) {
    if (r->norm != NORM_ALL_HEADS) return NULL;
    double* ms = (double*)malloc(sizeof(double) * (size_t)(r->B * r->T));
    for (int64_t b = 0; b < r->B; ++b)
        for (int64_t t = 0; t < r->T; ++t) {
            double tot = 0.0;
            for (int64_t h = 0; h < r->H; ++h)
                for (int64_t c = 0; c < r->D; ++c) {
                    double xv = bf16_f32(r->x[((b * r->T + t) * r->H + h) * r->D + c]);
                    tot += xv * xv;
                }
            ms[b * r->T + t] = tot / (double)(r->H * r->D);
        }
    return ms;
}

void orc_attn_exact(const orc_rows* qr, const orc_rows* kr, const uint16_t* v /* (B, Sk, Hk, D) bf16 */,
                    const orc_q8prefix* pf /* or NULL */,
                    const int64_t* rows, int64_t nrows, double* out /* (B, nrows, H, D) */) {
    const int64_t B = qr->B, H = qr->H, D = qr->D, Sk = kr->T, Hk = kr->H, G = H / Hk;
    const int64_t P = pf ? pf->P : 0, NG = D / 32, Ktot = P + Sk;
    double* msq = all_heads_ms_f64(qr);
    double* msk = all_heads_ms_f64(kr);
    /* keys of every (b, kv head), rotated once */
    double* K = (double*)malloc(sizeof(double) * (size_t)(B * Sk * Hk * D));
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t j = 0; j < Sk; ++j)
            for (int64_t hk = 0; hk < Hk; ++hk)
                prologue_f64(kr, b, j, hk, msk ? msk[b * Sk + j] : 0.0, K + ((b * Sk + j) * Hk + hk) * D);
    const double inv_sqrt_d = 1.0 / sqrt((double)D);
#pragma omp parallel for collapse(3) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t ri = 0; ri < nrows; ++ri) {
                const int64_t i = rows[ri], hk = h / G, bp = (pf && pf->B == 1) ? 0 : b;
                double qv[512], acc[512];
                prologue_f64(qr, b, i, h, msq ? msq[b * qr->T + i] : 0.0, qv);
                double* s = (double*)malloc(sizeof(double) * (size_t)Ktot);
                double m = -INFINITY, l = 0.0;
                for (int64_t j = 0; j < Ktot; ++j) {
                    double dot = 0.0;
                    if (j < P) {
                        const int8_t* kc = pf->k + ((bp * P + j) * Hk + hk) * D;
                        const uint16_t* ks = pf->ks + ((bp * P + j) * Hk + hk) * NG;
                        for (int64_t d = 0; d < D; ++d) dot += qv[d] * (double)kc[d] * f16_value(ks[d / 32]);
                    } else {
                        const double* kk = K + ((b * Sk + (j - P)) * Hk + hk) * D;
                        for (int64_t d = 0; d < D; ++d) dot += qv[d] * kk[d];
                    }
                    s[j] = dot * inv_sqrt_d;
                    m = fmax(m, s[j]);
                }
                for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t j = 0; j < Ktot; ++j) {
                    double p = exp(s[j] - m);
                    l += p;
                    for (int64_t d = 0; d < D; ++d) {
                        double vv;
                        if (j < P) vv = (double)pf->v[((bp * P + j) * Hk + hk) * D + d] * f16_value(pf->vs[((bp * P + j) * Hk + hk) * NG + d / 32]);
                        else vv = bf16_f32(v[((b * Sk + (j - P)) * Hk + hk) * D + d]);
                        acc[d] += p * vv;
                    }
                }
                for (int64_t d = 0; d < D; ++d) out[((b * nrows + ri) * H + h) * D + d] = acc[d] / l;
                free(s);
            }
    free(K);
    free(msq);
    free(msk);
}
