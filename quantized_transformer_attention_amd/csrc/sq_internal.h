// Internal declarations of libsq: argument blocks handed from the C entry points
// (api.cpp) to the kernel launchers (*.hip). Host-only types; no HIP headers here,
// so the validation layer stays free of the HIP runtime.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/sq.h"

namespace sq {

// Thread-local last error; returns `status` for tail calls.
int fail(int status, const char* fmt, ...);
void clear_error();

// Launch tracing (SQ_TRACE in the environment, read once): one stderr line per kernel launch.
bool trace_enabled();
void trace_launch(const char* kernel, unsigned gx, unsigned gy, unsigned gz, unsigned block, size_t lds,
                  const void* stream);

// ---------------------------------------------------------------- row prologue
// Split-half rotation over pairs < D/2 (channel p with p + pairs): an internal mode next to
// sq_rope_mode's values, since its partner exchange needs LDS.
constexpr int kRopeSplitPart = 3;

struct RowArgs {
    const uint16_t* x;          // bf16 rows
    int64_t B, T, H, D, sb, st, sh;
    int norm;                   // sq_norm_mode
    const uint16_t* w;          // bf16 weight rows (rows, wd)
    int64_t wd;                 // D (per head) or H*D (all heads)
    const int32_t* wrows;       // per-token weight row or nullptr
    const float* ms;            // all-heads mean squares (b, t) or nullptr
    int64_t msb, mst;
    float eps;
    int rope;                   // sq_rope_mode, or kRopeSplitPart
    const float* table;
    int64_t pairs, rb, rs, rp, rc;
    bool rope_contig;           // rp == 2, rc == 1 and 16-byte aligned rows
};

struct QuantArgs {
    RowArgs r;
    const float* mean;          // (b, h) rows of D or nullptr
    int64_t mb, mh;
    float sm_scale, scale_eps;
    int layout, block;
    int8_t* codes;
    int64_t ob, ot, oh;
    float* scales;
    int64_t ssb, ssh;
    int64_t nscale;             // scales per (b, h)
};

struct KmeanArgs {
    RowArgs r;
    float* partial;             // (B, H, nblk, D) workspace
    int64_t nblk;
    float* mean;
    int64_t mb, mh;
};

struct NormStatsArgs {
    const uint16_t* x;
    int64_t B, T, H, D, sb, st, sh;
    float* ms;
    int64_t msb, mst;
};

struct QuantVArgs {
    const uint16_t* v;
    int64_t B, T, H, D, sb, st, sh;
    uint8_t* codes;             // channel-major
    int64_t ob, oh, od;
    float* vs;
    int64_t vsb, vsh;
    uint32_t* amax;             // (B, H, D) workspace
};

// ---------------------------------------------------------------- attention core
struct AttnArgs {
    const int8_t* q;
    int64_t B, Sq, H, D, qsb, qst, qsh;
    const float* qs;
    int64_t qssb, qssh;
    int q_layout, q_block;
    const int8_t* k;
    int64_t Sk, Hk, ksb, kst, ksh;
    const float* ks;
    int64_t kssb, kssh;
    int k_layout, k_block;
    int k_shift, k_nscale;      // PER_BLOCK: log2(k_block); scales per (b, kv head)
    const void* v;              // channel-major bf16 or fp8 (sb, sh, sd; tokens contiguous)
    int v_fp8;
    int64_t vsb, vsh, vsd;
    const float* vscale;
    int64_t vssb, vssh;
    float score_scale;
    int kv_tile;
    int causal;                 // query i sees keys 0 .. i + Sk - Sq
    const float* sinks;         // (H,) sink logits in natural-log units, or NULL
    float* out;                 // FP32 elements, or bf16 ones when out_bf16 (strides count elements)
    int out_bf16;
    int64_t ob, ot, oh;
    float* lse;
    int64_t lb, lh;
};

struct VTransposeArgs {
    const uint16_t* v;          // token-major bf16 (B, S, Hk, D)
    int64_t B, S, H, D, sb, st, sh;
    uint16_t* out;              // channel-major (B, H, D, Spad)
    int64_t Spad;
};

struct PrefixArgs {
    const int8_t* q;
    int64_t B, Sq, H, D, qsb, qst, qsh;
    const float* qs;
    int64_t qssb, qssh;
    int q_layout, q_block;
    int64_t PB, P, Hk;
    const int8_t* k;
    int64_t kb, kt, kh;
    const uint16_t* ks;
    int64_t ksb, kst, ksh;
    const int8_t* v;
    int64_t vb, vt, vh;
    const uint16_t* vs;
    int64_t vsb, vst, vsh;
    const float* mu;
    int64_t mb, mh;
    float score_scale;
    int kv_tile;
    int causal;                 // query i sees keys 0 .. i + Sk - Sq
    const float* sinks;         // (H,) sink logits in natural-log units, or NULL
    float* out;                 // FP32 elements, or bf16 ones when out_bf16 (strides count elements)
    int out_bf16;
    int64_t ob, ot, oh;
    float* lse;
    int64_t lb, lh;
    uint8_t* img;               // workspace: the prefix's key tiles as LDS images (k_prefix_stage)
    int64_t ntiles;             // key tiles per (prefix batch, kv head): ceil(P / kv_tile)
};

// Bytes of one key tile's image in the prefix pass's workspace (head dim D, kv_tile 64 or 128): the
// tile's f16 K rows, its bf16 V^T rows and its keys' FP32 group scales (padded to 1 KB).
constexpr size_t prefix_image_bytes(int64_t D, int kv_tile) {
    return static_cast<size_t>(kv_tile * 2 * D + D * 2 * kv_tile + (D / 32 * kv_tile * 4 + 1023) / 1024 * 1024);
}

// Positions per split-KV segment of the paged decode (one workgroup each).
constexpr int kDecodeSeg = 256;

struct MergeArgs {
    float* out;
    int64_t ob, ot, oh;
    float* lse;
    int64_t lb, lh;
    const float* other;
    int64_t pb, pt, ph;
    const float* other_lse;
    int64_t qb, qh;
    int64_t B, S, H, D;
};

struct CacheWriteArgs {
    const void* k;
    const void* v;
    int64_t n;                  // tokens
    int Hk, D;
    int64_t kn, kh, vn, vh;     // element strides
    const int64_t* slots;
    int8_t* kc;
    uint16_t* ks;
    int8_t* vc;
    uint16_t* vs;
    int64_t nslots;             // num_blocks * block_size
};

struct DecodeArgs {
    const uint16_t* q;          // bf16 or f16 (q_f16) (N, Hq, D) at q[n*qn + h*qh + c]
    int q_f16;
    int64_t qn, qh;
    const int8_t* kc;
    const uint16_t* ks;
    const int8_t* vc;
    const uint16_t* vs;
    int64_t num_blocks;
    int bs, Hk, Hq, D;
    const int32_t* bt;
    int64_t bt_stride;
    const int32_t* lens;
    int N, max_len;
    float scale;
    const float* sinks;         // (Hq,) sink logits in natural-log units, or NULL
    float* out;                 // FP32 elements, or bf16 ones when out_bf16
    int out_bf16;
    int64_t on, oh;
    float* part;                // split-KV partials (N, Hq, segs, D + 2): acc, max, exp-sum
    int segs;                   // segments per sequence: ceil(max_len / kDecodeSeg)
};

struct PrefillArgs {
    const uint16_t* q;          // bf16 or f16 (q_f16) (T, Hq, D) at q[t*qt + h*qh + c]
    int q_f16;
    int64_t qt, qh;
    const int8_t* kc;
    const uint16_t* ks;
    const int8_t* vc;
    const uint16_t* vs;
    int64_t num_blocks;
    int Hk, Hq, D;
    const int32_t* bt;
    int64_t bt_stride;
    const int32_t* lens;        // keys per sequence (context + its queries)
    const int32_t* qstart;      // (N + 1,) first query token of each sequence
    int N, max_len;
    int64_t nqb;                // q blocks: num_tokens / rows-per-block + N (an upper bound)
    int T;                      // num_tokens: rows outside [0, T) are neither read nor written
    float scale;                // softmax_scale * log2 e
    const float* sinks;         // (Hq,) sink logits in natural-log units, or NULL
    float* out;                 // FP32 elements, or bf16 ones when out_bf16
    int out_bf16;
    int64_t ot, oh;
};

// ---------------------------------------------------------------- launchers (*.hip)
int launch_norm_stats(const NormStatsArgs& a, void* stream);
int launch_kmean(const KmeanArgs& a, void* stream);
int launch_quant_qk(const QuantArgs& a, void* stream);
int launch_quant_v_fp8(const QuantVArgs& a, void* stream);
int launch_v_transpose(const VTransposeArgs& a, void* stream);
int launch_attn(const AttnArgs& a, void* stream);
int launch_prefix(const PrefixArgs& a, void* stream);
int launch_lse_merge(const MergeArgs& a, void* stream);
int launch_cache_write(const CacheWriteArgs& a, bool f32, void* stream);
int launch_decode(const DecodeArgs& a, void* stream);
// The device address of the decode's own scratch array on the current device (looked up once per
// device); SQ_OK or an SQ_ERR_* code with the detail set.
int decode_scratch(void** ptr);
int launch_prefill(const PrefillArgs& a, void* stream);
constexpr int kPrefillWaves = 8;            // waves per prefill workgroup (32 rows each)

// ---------------------------------------------------------------- validation (validate.cpp)
int check_rows(const sq_rows* x, const char* what);
int check_norm(const sq_norm* n, const sq_rows* x, const char* what);
int check_rope(const sq_rope* r, const sq_rows* x, const char* what);
int check_layout(int layout, int block, const char* what);
int check_qk(const sq_qk* t, const char* what);
int64_t scale_count(int64_t T, int layout, int block);
RowArgs row_args(const sq_rows* x, const sq_norm* n, const sq_rope* r);

}  // namespace sq
