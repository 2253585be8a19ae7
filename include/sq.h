/*
 * sq.h -- quantized scaled-dot-product attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libsq.so. Four stages:
 *   1. a fused q/k prologue -- weighted RMSNorm, RoPE, k mean-smoothing -- that
 *      quantizes rows to INT8 in four row-group scale layouts (sq_norm_stats,
 *      sq_kmean, sq_quant_qk), and V to FP8 (sq_quant_v_fp8);
 *   2. the attention core: INT8 Q.K^T, FP32 online softmax, P.V in bf16 or FP8
 *      (sq_attn);
 *   3. a pass over a cached q8 key/value prefix merged with the projected keys by
 *      log-sum-exp (sq_attn_prefix_lse_merge);
 *   4. paged, GQA-stacked decode over a q8 KV cache (sq_paged_decode), causal
 *      chunked prefill over it (sq_paged_prefill) and its writer (sq_q8_cache_write).
 *
 * Sources, cited by page title and the section or identifier on the page:
 *   [kit]   WanGP shared/attention_kit.py
 *   [quant] WanGP shared/kernels/qk_quant_triton.py
 *   [impl]  fastkernels L2/attention_impl.py (vLLM-aligned paged attention layer)
 *   [tq]    vLLM triton_turboquant_unified_attention.py
 *
 * Conventions (all entry points):
 *  - Memory: every tensor pointer is a DEVICE pointer owned by the caller. The
 *    library never allocates, frees or keeps device memory; scratch memory is a
 *    caller-provided workspace whose size the matching *_workspace_bytes query
 *    returns (0 means no workspace is needed; the pointer may then be NULL). The one
 *    exception is sq_paged_decode_noalloc, whose scratch is a fixed array of the
 *    library's own on each GPU it runs on (SQ_DECODE_SCRATCH_BYTES).
 *  - Strides are in elements. The last (channel) dimension of every row view is
 *    contiguous. Row bases must be 16-byte aligned (SQ_ERR_ALIGN otherwise).
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream). Every call only
 *    enqueues work on it and returns; the host never waits and never reads device
 *    values. Buffers must stay valid until that work has completed.
 *  - Errors: calls return SQ_OK (0) or a negative SQ_ERR_* code. On error nothing
 *    has been enqueued. sq_status_string() names a code; sq_last_error() gives a
 *    detail message for the calling thread's last failed call.
 *  - Thread safety: calls are reentrant; the only library state is the per-thread
 *    last-error message.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raised whenever an argument list changes: 2 added causal masking and sinks (sq_attn,
 * sq_paged_decode) and sq_paged_prefill; 3 added out_dtype (FP32 or bf16 outputs) to
 * sq_attn, sq_paged_decode and sq_paged_prefill; 4 added q_dtype (bf16 or f16 queries) to
 * sq_paged_decode, sq_paged_decode_noalloc and sq_paged_prefill. sq_abi_version() returns it. */
#define SQ_ABI_VERSION 4

enum {
    SQ_OK = 0,
    SQ_ERR_NULL = -1,        /* a required pointer is NULL */
    SQ_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes */
    SQ_ERR_STRIDE = -3,      /* a stride the kernels cannot address */
    SQ_ERR_ALIGN = -4,       /* a row base or stride breaks 16-byte alignment */
    SQ_ERR_UNSUPPORTED = -5, /* a valid but unimplemented combination */
    SQ_ERR_WORKSPACE = -6,   /* workspace missing or too small */
    SQ_ERR_HIP = -7          /* a HIP runtime call failed (message in sq_last_error) */
};

typedef enum { SQ_BF16 = 0, SQ_F16 = 1, SQ_F32 = 2, SQ_I8 = 3, SQ_FP8E4M3 = 4 } sq_dtype;

/* Row-group scale layouts [quant] module docstring, SCALES_PER_BLOCK, PADDED_ROWS:
 * the scale index of token t is
 *   PER_BLOCK(block)  t / block                          (block 32, 64 or 128)
 *   THREAD_Q (32)     8 (t / 32) + t % 8                 rows r, r+8, r+16, r+24 of 32; tokens padded to 128
 *   THREAD_K (64)     4 (t / 64) + (t % 8) / 2           row pairs, repeating every 8 rows
 *   WARP_Q   (128)    4 (t / 128) + (t % 128) / 32       32 consecutive rows
 * Scales are FP32 (B, H, sq_scale_count(T)) per tensor. */
typedef enum { SQ_LAYOUT_PER_BLOCK = 0, SQ_LAYOUT_THREAD_Q = 1, SQ_LAYOUT_THREAD_K = 2, SQ_LAYOUT_WARP_Q = 3 } sq_layout;

typedef enum { SQ_NORM_NONE = 0, SQ_NORM_HEAD = 1, SQ_NORM_ALL_HEADS = 2 } sq_norm_mode;
typedef enum { SQ_ROPE_NONE = 0, SQ_ROPE_SPLIT_HALF = 1, SQ_ROPE_INTERLEAVED = 2 } sq_rope_mode;

/* A bf16 row tensor (B, T, H, D): element (b, t, h, c) at data[b*sb + t*st + h*sh + c].
 * D is 64 or 128. [quant] _launch strides XB / XS / XH. */
typedef struct {
    const void* data;
    int64_t B, T, H, D;
    int64_t sb, st, sh;
} sq_rows;

/* Weighted RMSNorm [quant] _rows (NORM), [kit] HeadGroup.mean_squares.
 *  mode HEAD: per (token, head) mean of squares over the D channels.
 *  mode ALL_HEADS: per token mean of squares over all H*D channels of the tensor.
 *  weight: bf16 (rows, D) for HEAD or (rows, H*D) for ALL_HEADS, rows contiguous.
 *  weight_rows: int32 (T,) weight row of each token (segments of tokens with their
 *    own weights, [quant] weight_rows), or NULL for row 0.
 *  mean_sq: optional FP32 per-token mean squares for ALL_HEADS, element (b, t) at
 *    mean_sq[b*msb + t*mst], as sq_norm_stats writes them; NULL = computed by the
 *    call into its workspace.
 *  The norm output is rounded to bf16 (the activation dtype) before rotation. */
typedef struct {
    sq_norm_mode mode;
    const void* weight;
    const int32_t* weight_rows;
    const float* mean_sq;
    int64_t msb, mst;
    float eps;
} sq_norm;

/* RoPE [quant] _rows (ROTATE), _pairs, _launch rope_args: pair p of token t of batch
 * b rotates by cos = table[rb*b + rs*t + rp*p], sin = table[rb*b + rs*t + rp*p + rc]
 * (FP32). SPLIT_HALF pairs channel p with p + pairs; INTERLEAVED pairs 2p with
 * 2p + 1; channels >= 2*pairs pass through. rb = 0 serves every batch item.
 * A (..., pairs, 2) table has rp = 2, rc = 1; 2x2 matrices [[cos,-sin],[sin,cos]]
 * (..., pairs, 2, 2) have rp = 4, rc = 2. Both modes take any pairs in [1, D/2]. */
typedef struct {
    sq_rope_mode mode;
    const float* table;
    int64_t pairs, rb, rs, rp, rc;
} sq_rope;

/* INT8 codes (B, S, H, D) with their FP32 scales (B, H, n) in one layout, as
 * sq_quant_qk writes them: code (b, s, h, c) at codes[b*sb + s*st + h*sh + c],
 * scale j of (b, h) at scales[b*ssb + h*ssh + j]. */
typedef struct {
    const int8_t* codes;
    int64_t B, S, H, D;
    int64_t sb, st, sh;
    const float* scales;
    int64_t ssb, ssh;
    sq_layout layout;
    int block;
} sq_qk;

/* Values for sq_attn: (B, S, Hk, D); element (b, s, h, c) at
 * data[b*sb + s*st + h*sh + c*sd].
 *  bf16: token-major, sd == 1 (staged channel-major in the workspace by sq_attn).
 *  FP8 e4m3fn: channel-major, st == 1, as sq_quant_v_fp8 writes them, with FP32
 *    per-channel scales (B, Hk, D) at scale[b*vsb + h*vsh + c]. */
typedef struct {
    const void* data;
    sq_dtype dtype;
    int64_t sb, st, sh, sd;
    const float* scale;
    int64_t vsb, vsh;
} sq_values;

/* A cached q8 prefix [kit] KVPrefix (q8 form), GROUP, quantize_q8: keys and values
 * int8 (Bp, P, Hk, D) with FP16 scales (Bp, P, Hk, D/32), one scale per 32 channels;
 * Bp = 1 serves every batch item. Element (b, p, h, c) of k at k[b*kb + p*kt + h*kh + c],
 * its scale at k_scale[b*ksb + p*kst + h*ksh + c/32]; likewise v. Token rows may not
 * overlap (kt, vt >= D; kst, vst >= D/32), and one (b, kv head) slice of each tensor,
 * P + 128 rows long, must span < 2 GiB (SQ_ERR_STRIDE / SQ_ERR_UNSUPPORTED otherwise). */
typedef struct {
    int64_t B, P, Hk, D;
    const int8_t* k;
    int64_t kb, kt, kh;
    const uint16_t* k_scale;
    int64_t ksb, kst, ksh;
    const int8_t* v;
    int64_t vb, vt, vh;
    const uint16_t* v_scale;
    int64_t vsb, vst, vsh;
} sq_q8prefix;

/* Number of scales per (b, h) of a T-token tensor in a layout; -1 if the layout and
 * block do not pair (THREAD_Q:32, THREAD_K:64, WARP_Q:128, PER_BLOCK:32|64|128). */
int64_t sq_scale_count(int64_t T, sq_layout layout, int block);

/* ---- A1. Per-token mean of squares over all heads [kit] HeadGroup.mean_squares,
 * joint_qkv_attention's mean squares by head groups. mean_sq[b*msb + t*mst] =
 * (sum over heads in ascending order of the head's sum of squares) / (H*D), FP32;
 * each head's sum in the canonical order: D/8 partials, partial l over channels
 * 4l .. 4l+3 then D/2 + 4l .. D/2 + 4l + 3 (x*x for the first, then fma per channel),
 * combined by an xor butterfly (offsets D/16 .. 1). */
int sq_norm_stats(const sq_rows* x, float* mean_sq, int64_t msb, int64_t mst, void* stream);

/* ---- A2. k mean [quant] norm_rope_mean: mean over tokens of the normalized,
 * rotated rows per (b, head), FP32, written to mean[b*mb + h*mh + c]. Partial sums
 * per 64-row block in a fixed order (row 4i + r of a block joins partial r in
 * ascending i; the block's sum is (S0 + S1) + (S2 + S3); block sums added in chunks of
 * 16 consecutive blocks, ascending within a chunk, and the chunk sums added in
 * ascending order; divided by T), so the result is bit-reproducible. `norm` may be NULL
 * (no norm); `rope` may be NULL (no rotation). The token strides of x (x->st * 2 bytes),
 * of the rope table (rs * 4) and of mean_sq (mst * 4) must each be under 16 MiB
 * (SQ_ERR_STRIDE otherwise); the same holds for sq_quant_qk, whose code token stride
 * ot must also be under 16 MiB. */
size_t sq_kmean_workspace_bytes(const sq_rows* k, const sq_norm* norm);
int sq_kmean(const sq_rows* k, const sq_norm* norm, const sq_rope* rope, float* mean, int64_t mb, int64_t mh,
             void* ws, size_t ws_bytes, void* stream);

/* ---- A3. Fused q/k quantization [quant] _norm_rope_quant, norm_rope_quantize.
 * Each row: norm (FP32, output rounded to bf16), rotation (FP32, one fused
 * multiply-add per channel), minus mean (b, h) when `mean` is not NULL (k
 * smoothing: mean[b*mb + h*mh + c]), times sm_scale. Per layout group:
 * scale = amax / 127 + scale_eps (correctly rounded FP32); code of r = v / scale
 * (correctly rounded) is trunc(r + 0.5) for r >= 0, trunc(r - 0.5) otherwise.
 * Every scale up to sq_scale_count(T) is written (THREAD_Q tail groups: scale_eps).
 * codes (B, T, H, D) int8 at codes[b*ob + t*ot + h*oh + c]; scales (B, H, n) at
 * scales[b*ssb + h*ssh + j]. */
size_t sq_quant_qk_workspace_bytes(const sq_rows* x, const sq_norm* norm);
int sq_quant_qk(const sq_rows* x, const sq_norm* norm, const sq_rope* rope, const float* mean, int64_t mb,
                int64_t mh, float sm_scale, float scale_eps, sq_layout layout, int block, int8_t* codes, int64_t ob,
                int64_t ot, int64_t oh, float* scales, int64_t ssb, int64_t ssh, void* ws, size_t ws_bytes,
                void* stream);

/* ---- A4. V to FP8 e4m3fn with per-channel scales (reading of "P.V FP8 e4m3 with
 * per-channel v scales"): vs(b, h, c) = max(amax over tokens |v| / 448, 1e-8);
 * code = e4m3fn(v / vs) rounded to nearest even, saturating at 448. Codes are
 * written CHANNEL-MAJOR, the layout sq_attn reads: code (b, t, h, c) at
 * codes[b*ob + h*oh + c*od + t], od >= T rounded up to 16 and a multiple of 16;
 * token columns [T, od) are zero-filled. vs at vs[b*vsb + h*vsh + c]. */
size_t sq_quant_v_fp8_workspace_bytes(const sq_rows* v);
int sq_quant_v_fp8(const sq_rows* v, uint8_t* codes, int64_t ob, int64_t oh, int64_t od, float* vs, int64_t vsb,
                   int64_t vsh, void* ws, size_t ws_bytes, void* stream);

/* ---- B. Quantized attention core (kv head of q head h is h / (H / Hk)
 * [impl] _repeat_kv_for_heads). For each query row, over key tiles of
 * kv_tile keys ([tq] online softmax): a = integer q.k; c = RN(qs * ks) (times
 * score_scale if it is not 1); s = RN(a c); m' = max(m, tile max of s);
 * p = 2^fma(a, c, -m'); alpha = 2^(m - m'); l = l alpha + sum p; acc = acc alpha +
 * sum Pt Vt with Pt = bf16(p) (bf16 v) or e4m3(256 p) (FP8 v); out = acc / l (bf16 v)
 * or acc * vs / (256 l) (FP8 v); lse = m + log2 l (base 2, the scores' log2 units).
 * q rows carry the softmax scale (log2(e)/sqrt(D) through sm_scale). q layouts:
 * PER_BLOCK, THREAD_Q, WARP_Q; k layouts: PER_BLOCK, THREAD_K. kv_tile: 64 or 128.
 * out (B, Sq, H, D) at out[b*ob + i*ot + h*oh + c] in elements of
 * out_dtype: SQ_F32, or SQ_BF16 (the FP32 result rounded to nearest even; an option for
 * callers that keep activations in bf16), aligned to its element size (SQ_ERR_ALIGN;
 * another dtype SQ_ERR_UNSUPPORTED); lse FP32 (B, H, Sq) at lse[b*lb + h*lh + i], or NULL.
 * causal (0 or 1) [impl] _sdpa_one's mask, [tq] unified attention's causal mask:
 * query i sits at key position i + Sk - Sq (its context is the Sk - Sq keys before
 * the queries) and sees keys 0 .. i + Sk - Sq; needs Sk >= Sq (SQ_ERR_SHAPE).
 * sinks: NULL, or FP32 (H,) per-head sink logits in natural-log units [tq] USE_SINKS:
 * the running max starts at m = RN(sink * log2(e)) (FP32) and the sum at l = 1, so
 * the sink joins the denominator (and lse) but adds no value row. When two passes
 * are merged (sq_lse_merge, sq_attn_prefix_lse_merge), give the sinks to one only. */
size_t sq_attn_workspace_bytes(const sq_qk* q, const sq_qk* k, const sq_values* v);
int sq_attn(const sq_qk* q, const sq_qk* k, const sq_values* v, float score_scale, int kv_tile, int causal,
            const float* sinks, void* out, sq_dtype out_dtype, int64_t ob, int64_t ot, int64_t oh, float* lse,
            int64_t lb, int64_t lh, void* ws, size_t ws_bytes, void* stream);

/* ---- C. q8 prefix pass + log-sum-exp merge [kit] _attend_with_prefix,
 * dequantize_q8_into, _merge_lse_. The same q codes attend the prefix keys in a
 * pass of their own with score s = qh . (kh - mu), qh = qc * qs, kh = kc * ks16 per
 * 32 channels, mu = k_mean (b, kv head) (the mean the projected keys subtracted, so
 * both passes share the offset; NULL = 0), times score_scale; softmax as sq_attn
 * over kv_tile keys with Pt = bf16(p) and Vt = bf16(vc * vs16). The pass is merged
 * into (out, lse), which hold the projected pass on entry (lse base 2): top =
 * max(a, b), wa = 2^(a - top), wb = 2^(b - top), out = out wa/(wa+wb) +
 * prefix wb/(wa+wb), lse = top + log2(wa + wb). Both -inf: out 0, lse -inf.
 * Workspace: sq_attn_prefix_lse_merge_workspace_bytes (the prefix's key tiles laid out
 * once per call for the pass: f16 key codes, FP32 key scales, Vt; about 4 D + 16 bytes per
 * prefix key and kv head, for either kv_tile). */
size_t sq_attn_prefix_lse_merge_workspace_bytes(const sq_qk* q, const sq_q8prefix* prefix);
int sq_attn_prefix_lse_merge(const sq_qk* q, const sq_q8prefix* prefix, const float* k_mean, int64_t mb, int64_t mh,
                             float score_scale, int kv_tile, float* out, int64_t ob, int64_t ot, int64_t oh,
                             float* lse, int64_t lb, int64_t lh, void* ws, size_t ws_bytes, void* stream);

/* ---- C2. Log-sum-exp merge of two attentions of the same queries over disjoint key
 * sets [kit] _merge_lse_ (the merge of a native cached prefix's pass, _attend_with_prefix):
 * per (b, i, h): top = max(a, b) of the two base-2 log-sum-exps; wa = 2^(a - top),
 * wb = 2^(b - top); out = out * (wa / (wa + wb)) + other * (wb / (wa + wb)); lse = top +
 * log2(wa + wb) (written so merges chain; the pages' merge leaves it as it was). Both
 * -inf: out 0, lse -inf. out, other FP32 (B, S, H, D) at out[b*ob + i*ot + h*oh + c]
 * (other likewise with pb, pt, ph); lse, other_lse FP32 (B, H, S) at lse[b*lb + h*lh + i]
 * (other_lse with qb, qh): the layouts sq_attn writes. A native prefix: k mean of the
 * prefix keys (sq_kmean), prefix keys quantized with it (sq_quant_qk), prefix values to
 * FP8 (sq_quant_v_fp8), the projected keys quantized with the same mean, one sq_attn pass
 * per key set, then this merge. D 64 or 128; out/other rows 16-byte aligned; B H S below
 * 2^36 (one workgroup per 32 queries of a (b, h) at D 128, 64 at D 64, at most 2^31 of them:
 * SQ_ERR_UNSUPPORTED beyond). */
int sq_lse_merge(float* out, int64_t ob, int64_t ot, int64_t oh, float* lse, int64_t lb, int64_t lh, const float* other,
                 int64_t pb, int64_t pt, int64_t ph, const float* other_lse, int64_t qb, int64_t qh, int64_t B, int64_t S,
                 int64_t H, int64_t D, void* stream);

/* ---- D. Paged GQA decode over a q8 cache [impl] _cache_seq, _sdpa_one,
 * _decode_torch; [tq] block-table addressing and split-KV segments. Sequence n of
 * length L = seq_lens[n] (1 <= L <= max_seq_len) has one query ((N, Hq, D) of q_dtype,
 * SQ_BF16 or SQ_F16, at q[n*qn + h*qh + c]) at position L - 1, which attends positions 0..L-1. Position
 * pos lives in physical block block_table[n*bt_stride + pos / block_size], slot
 * pos % block_size. Caches [num_blocks, block_size, Hk, D] int8 (contiguous), FP16
 * scales [num_blocks, block_size, Hk, D/32]; keys and values are code * scale.
 * Softmax of (q . k) * softmax_scale; out (N, Hq, D) at out[n*on + h*oh + c] in elements
 * of out_dtype (SQ_F32, or SQ_BF16 rounded to nearest even, as sq_attn).
 * max_seq_len is a host bound for the workspace and the grid (no device read).
 * block_size 16; D 64 or 128; Hq / Hk in {1, 2, 4, 8}. q 16-byte aligned rows, caches
 * 16-byte aligned, scale tensors aligned to one row of D/32 FP16 (D/16 bytes).
 * Both products run on f16 matrix units with FP32 accumulation: q is carried as f16
 * after an exact power-of-two rescale per head, and the weight of a value row is
 * f16(p * value scale) (relative rounding <= 2^-11 per weight).
 * sinks: NULL, or FP32 (Hq,) per-query-head sink logits in natural-log units
 * [tq] USE_SINKS (the split kernel's first segment carries it): exp(sink) joins the
 * softmax denominator once per (sequence, head) and adds no value row. */
size_t sq_paged_decode_workspace_bytes(int num_seqs, int Hq, int D, int max_seq_len);
int sq_paged_decode(const void* q, sq_dtype q_dtype, int64_t qn, int64_t qh, const int8_t* k_cache,
                    const uint16_t* k_scale, const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks, int block_size, int Hk,
                    const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens, int num_seqs,
                    int max_seq_len, int Hq, int D, float softmax_scale, const float* sinks, void* out,
                    sq_dtype out_dtype, int64_t on, int64_t oh, void* ws, size_t ws_bytes, void* stream);

/* ---- D, without allocation. For callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Computes exactly what sq_paged_decode computes (the same kernels, the same
 * arguments without ws / ws_bytes), with the segment partials in a file-scope device
 * array of SQ_DECODE_SCRATCH_BYTES that each GPU the library runs on holds until the
 * process ends. Nothing is allocated by the call. Its first call on a device looks the
 * array's address up (hipGetSymbolAddress) with that device current. A call whose
 * partials, sq_paged_decode_workspace_bytes(num_seqs, Hq, D, max_seq_len), exceed the
 * array returns SQ_ERR_WORKSPACE before anything is enqueued (64 MiB holds e.g. 64
 * sequences x 32 query heads up to 16,128 positions). All calls on one GPU share the
 * array: calls whose work may overlap on that GPU (other streams, other threads) race and
 * must be ordered by the caller. No part of the array needs to start at zero. */
#define SQ_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
int sq_paged_decode_noalloc(const void* q, sq_dtype q_dtype, int64_t qn, int64_t qh, const int8_t* k_cache,
                            const uint16_t* k_scale, const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks, int block_size, int Hk,
                            const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens, int num_seqs,
                            int max_seq_len, int Hq, int D, float softmax_scale, const float* sinks, void* out,
                            sq_dtype out_dtype, int64_t on, int64_t oh, void* stream);

/* ---- D3. Paged causal prefill over a q8 cache [impl] _prefill_torch_from_cache,
 * _cache_seq, _sdpa_one (per sequence, mask k_pos <= key_offset + q_pos); [tq] unified
 * 2D kernel (varlen q blocks by query_start_len, context_len = seq_len - query_len,
 * USE_SINKS). Sequence n owns the packed query tokens [query_start[n], query_start[n+1])
 * of q ((num_tokens, Hq, D) of q_dtype, SQ_BF16 or SQ_F16, at q[t*qt + h*qh + c]; query_start
 * int32 (num_seqs + 1,),
 * nondecreasing, query_start[0] = 0, query_start[num_seqs] = num_tokens) and the keys at
 * positions 0 .. L-1 of its paged cache, L = seq_lens[n] (the context plus its own
 * queries, whose keys and values must already be in the cache, e.g. by
 * sq_q8_cache_write; q_len <= L <= max_seq_len). Its query j sits at position L - q_len + j
 * and attends positions 0 .. L - q_len + j. Caches, scales, block table and softmax_scale
 * as sq_paged_decode (block_size 16, D 64 or 128, Hq / Hk in {1, 2, 4, 8}; scales 2-byte
 * aligned); sinks NULL or FP32 (Hq,). out (num_tokens, Hq, D) at out[t*ot + h*oh + c] in
 * elements of out_dtype (SQ_F32, or SQ_BF16 rounded to nearest even, as sq_attn). The
 * products accumulate in FP32 on the matrix units: q as f16 after an exact power-of-two
 * rescale per (token, head); each key code * scale as f16(code * scale) plus the remainder in
 * e4m3 under a power-of-two scale per (key, 32 channels), multiplied by an e4m3 copy of q (a
 * key off by at most 2^-16 of itself); each value code * scale held exactly as a pair of f16
 * (cached values must stay below 65504 in magnitude); P as f16 (relative rounding
 * <= 2^-11), the denominator summed from the same f16 P. A block-table entry outside
 * [0, num_blocks) is read as block 0 (no fault; that sequence's rows are then undefined).
 * No workspace; only enqueues. */
int sq_paged_prefill(const void* q, sq_dtype q_dtype, int64_t qt, int64_t qh, int64_t num_tokens, const int8_t* k_cache,
                     const uint16_t* k_scale, const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks,
                     int block_size, int Hk, const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                     const int32_t* query_start, int num_seqs, int max_seq_len, int Hq, int D, float softmax_scale,
                     const float* sinks, void* out, sq_dtype out_dtype, int64_t ot, int64_t oh, void* stream);

/* ---- D2. q8 paged-cache writer [kit] quantize_q8 (per token, head and group of 32
 * channels: scale = max(amax / 127, 1e-8) in FP32, code = x / scale (correctly
 * rounded FP32 division) rounded half to even and clamped to [-127, 127], the scale
 * stored as FP16 (round to nearest even)) and [impl] _store_kvcache_nhd (token t goes
 * to slot s = slot_mapping[t]: cache block s / block_size, row s % block_size; s < 0
 * skips the token). New rows k, v (n_tokens, Hk, D) of bf16 or FP32 (dtype): element
 * (t, h, c) at k[t*kn + h*kh + c], v likewise with vn, vh; inputs finite. Caches and
 * scales in the layout sq_paged_decode reads: [num_blocks, block_size, Hk, D] int8 and
 * [num_blocks, block_size, Hk, D/32] FP16, contiguous. A slot at or past
 * num_blocks * block_size is skipped as well, so a bad mapping cannot write outside
 * the caches; two tokens mapped to one slot race (either row may land). D 64 or 128;
 * k and v rows 16-byte aligned (strides in elements); caches 16-byte aligned, scales
 * 2-byte aligned. No workspace; only enqueues on `stream`. */
int sq_q8_cache_write(const void* k, const void* v, sq_dtype dtype, int64_t n_tokens, int Hk, int D, int64_t kn,
                      int64_t kh, int64_t vn, int64_t vh, const int64_t* slot_mapping, int8_t* k_cache,
                      uint16_t* k_scale, int8_t* v_cache, uint16_t* v_scale, int64_t num_blocks, int block_size,
                      void* stream);

const char* sq_status_string(int status);
const char* sq_last_error(void);
int sq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
