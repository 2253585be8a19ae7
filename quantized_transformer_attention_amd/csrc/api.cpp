// libsq C entry points: validate on the host (validate.cpp, no HIP call), size the
// workspace, then hand an argument block to the kernel launchers. Nothing is
// enqueued when validation fails.
#include <cmath>
#include <cstring>

#include "sq_internal.h"

using namespace sq;

namespace {

constexpr size_t kAlign = 256;
size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool all_heads_needs_ws(const sq_norm* n) { return n && n->mode == SQ_NORM_ALL_HEADS && !n->mean_sq; }

int check_ws(void* ws, size_t have, size_t need, const char* what) {
    if (need == 0) return SQ_OK;
    if (!ws) return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got NULL", what, need);
    if (have < need) return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes required, got %zu", what, need, have);
    if (reinterpret_cast<uintptr_t>(ws) % kAlign)
        return fail(SQ_ERR_ALIGN, "%s: workspace must be %zu-byte aligned", what, kAlign);
    return SQ_OK;
}

// An attention output is FP32 or bf16 (rounded to nearest even), aligned to its element size.
int check_out(const void* out, sq_dtype dtype, const char* what) {
    if (dtype != SQ_F32 && dtype != SQ_BF16) return fail(SQ_ERR_UNSUPPORTED, "%s: out_dtype must be F32 or BF16", what);
    if (reinterpret_cast<uintptr_t>(out) % (dtype == SQ_F32 ? 4 : 2))
        return fail(SQ_ERR_ALIGN, "%s: out must be aligned to its element size", what);
    return SQ_OK;
}

// Runs A1 into the workspace when the all-heads norm has no precomputed statistics.
int prepare_all_heads(const sq_rows* x, RowArgs& r, void* ws, void* stream) {
    if (r.norm != SQ_NORM_ALL_HEADS || r.ms) return SQ_OK;
    NormStatsArgs s{static_cast<const uint16_t*>(x->data), x->B, x->T, x->H, x->D, x->sb, x->st, x->sh,
                    static_cast<float*>(ws), x->T, 1};
    r.ms = s.ms;
    r.msb = x->T;
    r.mst = 1;
    return launch_norm_stats(s, stream);
}

int check_prologue(const sq_rows* x, const sq_norm* n, const sq_rope* r, const char* what) {
    int st = check_rows(x, what);
    if (!st) st = check_norm(n, x, what);
    if (!st) st = check_rope(r, x, what);
    if (st) return st;
    // rows of a tile are addressed by 24-bit byte offsets from the tile's first token
    constexpr int64_t kMaxTokenBytes = int64_t(1) << 24;
    if (x->st * 2 >= kMaxTokenBytes || (r && r->mode != SQ_ROPE_NONE && r->rs * 4 >= kMaxTokenBytes) ||
        (n && n->mode == SQ_NORM_ALL_HEADS && n->mean_sq && n->mst * 4 >= kMaxTokenBytes))
        return fail(SQ_ERR_STRIDE, "%s: a token stride of x, the rope table or mean_sq spans 16 MiB or more", what);
    return SQ_OK;
}

}  // namespace

extern "C" {

int sq_norm_stats(const sq_rows* x, float* mean_sq, int64_t msb, int64_t mst, void* stream) {
    clear_error();
    int st = check_rows(x, "sq_norm_stats");
    if (st) return st;
    if (x->B * x->T * x->H == 0) return SQ_OK;
    if (!mean_sq) return fail(SQ_ERR_NULL, "sq_norm_stats: mean_sq is NULL");
    if (msb < 0 || mst < 0) return fail(SQ_ERR_STRIDE, "sq_norm_stats: negative stride");
    NormStatsArgs a{static_cast<const uint16_t*>(x->data), x->B, x->T, x->H, x->D, x->sb, x->st, x->sh,
                    mean_sq, msb, mst};
    return launch_norm_stats(a, stream);
}

size_t sq_kmean_workspace_bytes(const sq_rows* k, const sq_norm* norm) {
    if (!k) return 0;
    const int64_t nblk = (k->T + 63) / 64;
    size_t bytes = round_up(sizeof(float) * static_cast<size_t>(k->B * k->H * nblk * k->D));
    if (all_heads_needs_ws(norm)) bytes += round_up(sizeof(float) * static_cast<size_t>(k->B * k->T));
    return bytes;
}

int sq_kmean(const sq_rows* k, const sq_norm* norm, const sq_rope* rope, float* mean, int64_t mb, int64_t mh,
             void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    int st = check_prologue(k, norm, rope, "sq_kmean");
    if (st) return st;
    if (k->B * k->H == 0) return SQ_OK;
    if (k->T == 0) return fail(SQ_ERR_SHAPE, "sq_kmean: the mean of zero tokens is undefined");
    if (!mean) return fail(SQ_ERR_NULL, "sq_kmean: mean is NULL");
    if (mb < 0 || mh < 0) return fail(SQ_ERR_STRIDE, "sq_kmean: negative stride");
    st = check_ws(ws, ws_bytes, sq_kmean_workspace_bytes(k, norm), "sq_kmean");
    if (st) return st;
    KmeanArgs a{};
    a.r = row_args(k, norm, rope);
    a.nblk = (k->T + 63) / 64;
    a.partial = static_cast<float*>(ws);
    a.mean = mean;
    a.mb = mb;
    a.mh = mh;
    void* ms_ws = static_cast<char*>(ws) + round_up(sizeof(float) * static_cast<size_t>(k->B * k->H * a.nblk * k->D));
    st = prepare_all_heads(k, a.r, ms_ws, stream);
    if (st) return st;
    return launch_kmean(a, stream);
}

size_t sq_quant_qk_workspace_bytes(const sq_rows* x, const sq_norm* norm) {
    if (!x || !all_heads_needs_ws(norm)) return 0;
    return round_up(sizeof(float) * static_cast<size_t>(x->B * x->T));
}

int sq_quant_qk(const sq_rows* x, const sq_norm* norm, const sq_rope* rope, const float* mean, int64_t mb,
                int64_t mh, float sm_scale, float scale_eps, sq_layout layout, int block, int8_t* codes, int64_t ob,
                int64_t ot, int64_t oh, float* scales, int64_t ssb, int64_t ssh, void* ws, size_t ws_bytes,
                void* stream) {
    clear_error();
    int st = check_prologue(x, norm, rope, "sq_quant_qk");
    if (!st) st = check_layout(layout, block, "sq_quant_qk");
    if (st) return st;
    if (x->B * x->T * x->H == 0) return SQ_OK;
    if (!codes || !scales) return fail(SQ_ERR_NULL, "sq_quant_qk: codes or scales are NULL");
    if (ob < 0 || ot < 0 || oh < 0 || ssb < 0 || ssh < 0) return fail(SQ_ERR_STRIDE, "sq_quant_qk: negative stride");
    if ((reinterpret_cast<uintptr_t>(codes) & 7) || ob % 8 || ot % 8 || oh % 8)
        return fail(SQ_ERR_ALIGN, "sq_quant_qk: code rows must start on 8-byte boundaries");
    if (ot >= (int64_t(1) << 24)) return fail(SQ_ERR_STRIDE, "sq_quant_qk: the code token stride spans 16 MiB or more");
    if (mean && ((reinterpret_cast<uintptr_t>(mean) & 15) || mb % 4 || mh % 4))
        return fail(SQ_ERR_ALIGN, "sq_quant_qk: mean rows must be 16-byte aligned");
    if (!std::isfinite(sm_scale) || !std::isfinite(scale_eps) || scale_eps < 0.0f)
        return fail(SQ_ERR_SHAPE, "sq_quant_qk: sm_scale and scale_eps must be finite, scale_eps >= 0");
    st = check_ws(ws, ws_bytes, sq_quant_qk_workspace_bytes(x, norm), "sq_quant_qk");
    if (st) return st;
    QuantArgs a{};
    a.r = row_args(x, norm, rope);
    a.mean = mean;
    a.mb = mb;
    a.mh = mh;
    a.sm_scale = sm_scale;
    a.scale_eps = scale_eps;
    a.layout = layout;
    a.block = block;
    a.codes = codes;
    a.ob = ob; a.ot = ot; a.oh = oh;
    a.scales = scales;
    a.ssb = ssb; a.ssh = ssh;
    a.nscale = scale_count(x->T, layout, block);
    st = prepare_all_heads(x, a.r, ws, stream);
    if (st) return st;
    return launch_quant_qk(a, stream);
}

size_t sq_quant_v_fp8_workspace_bytes(const sq_rows* v) {
    if (!v) return 0;
    return round_up(sizeof(uint32_t) * static_cast<size_t>(v->B * v->H * v->D));
}

int sq_quant_v_fp8(const sq_rows* v, uint8_t* codes, int64_t ob, int64_t oh, int64_t od, float* vs, int64_t vsb,
                   int64_t vsh, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    int st = check_rows(v, "sq_quant_v_fp8");
    if (st) return st;
    if (v->B * v->T * v->H == 0) return SQ_OK;
    if (!codes || !vs) return fail(SQ_ERR_NULL, "sq_quant_v_fp8: codes or vs are NULL");
    if (ob < 0 || oh < 0 || vsb < 0 || vsh < 0) return fail(SQ_ERR_STRIDE, "sq_quant_v_fp8: negative stride");
    if (od < (v->T + 15) / 16 * 16 || od % 16)
        return fail(SQ_ERR_STRIDE, "sq_quant_v_fp8: token stride od must be a multiple of 16 and >= T rounded up");
    if ((reinterpret_cast<uintptr_t>(codes) & 15) || ob % 16 || oh % 16)
        return fail(SQ_ERR_ALIGN, "sq_quant_v_fp8: channel rows must start on 16-byte boundaries");
    st = check_ws(ws, ws_bytes, sq_quant_v_fp8_workspace_bytes(v), "sq_quant_v_fp8");
    if (st) return st;
    QuantVArgs a{static_cast<const uint16_t*>(v->data), v->B, v->T, v->H, v->D, v->sb, v->st, v->sh,
                 codes, ob, oh, od, vs, vsb, vsh, static_cast<uint32_t*>(ws)};
    return launch_quant_v_fp8(a, stream);
}

}  // extern "C"

namespace {

int check_pair(const sq_qk* q, const sq_qk* k, const char* what) {
    int st = check_qk(q, what);
    if (!st) st = check_qk(k, what);
    if (st) return st;
    if (q->layout == SQ_LAYOUT_THREAD_K)
        return fail(SQ_ERR_UNSUPPORTED, "%s: q layout THREAD_K is a key layout", what);
    if (k->layout == SQ_LAYOUT_THREAD_Q || k->layout == SQ_LAYOUT_WARP_Q)
        return fail(SQ_ERR_UNSUPPORTED, "%s: k layout must be PER_BLOCK or THREAD_K", what);
    if (q->B != k->B || q->D != k->D) return fail(SQ_ERR_SHAPE, "%s: q and k differ in batch or head dim", what);
    if (k->H < 1 || q->H % k->H) return fail(SQ_ERR_SHAPE, "%s: q heads %lld not a multiple of kv heads %lld", what,
                                             (long long)q->H, (long long)k->H);
    return SQ_OK;
}

int64_t padded_keys(int64_t S) { return (S + 127) / 128 * 128; }

}  // namespace

extern "C" {

size_t sq_attn_workspace_bytes(const sq_qk* q, const sq_qk* k, const sq_values* v) {
    (void)q;
    if (!k || !v || v->dtype != SQ_BF16) return 0;
    return round_up(sizeof(uint16_t) * static_cast<size_t>(k->B * k->H * k->D * padded_keys(k->S)));
}

int sq_attn(const sq_qk* q, const sq_qk* k, const sq_values* v, float score_scale, int kv_tile, int causal,
            const float* sinks, void* out, sq_dtype out_dtype, int64_t ob, int64_t ot, int64_t oh, float* lse,
            int64_t lb, int64_t lh, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    int st = check_pair(q, k, "sq_attn");
    if (st) return st;
    if (q->B * q->S * q->H == 0) return SQ_OK;
    if (k->S < 1) return fail(SQ_ERR_SHAPE, "sq_attn: no keys");
    if (!v || !v->data) return fail(SQ_ERR_NULL, "sq_attn: values are NULL");
    if (!out) return fail(SQ_ERR_NULL, "sq_attn: out is NULL");
    st = check_out(out, out_dtype, "sq_attn");
    if (st) return st;
    if (ob < 0 || ot < 0 || oh < 0 || lb < 0 || lh < 0) return fail(SQ_ERR_STRIDE, "sq_attn: negative stride");
    if (kv_tile != 64 && kv_tile != 128) return fail(SQ_ERR_UNSUPPORTED, "sq_attn: kv_tile must be 64 or 128");
    if (!(score_scale > 0.0f) || !std::isfinite(score_scale))
        return fail(SQ_ERR_SHAPE, "sq_attn: score_scale must be finite and > 0");
    if (causal != 0 && causal != 1) return fail(SQ_ERR_SHAPE, "sq_attn: causal must be 0 or 1");
    if (causal && k->S < q->S)
        return fail(SQ_ERR_SHAPE, "sq_attn: causal needs at least as many keys as queries (Sk %lld < Sq %lld)",
                    (long long)k->S, (long long)q->S);
    AttnArgs a{};
    a.q = q->codes; a.B = q->B; a.Sq = q->S; a.H = q->H; a.D = q->D;
    a.qsb = q->sb; a.qst = q->st; a.qsh = q->sh;
    a.qs = q->scales; a.qssb = q->ssb; a.qssh = q->ssh; a.q_layout = q->layout; a.q_block = q->block;
    a.k = k->codes; a.Sk = k->S; a.Hk = k->H; a.ksb = k->sb; a.kst = k->st; a.ksh = k->sh;
    a.ks = k->scales; a.kssb = k->ssb; a.kssh = k->ssh; a.k_layout = k->layout; a.k_block = k->block;
    a.k_shift = 0;
    while ((1 << a.k_shift) < k->block) ++a.k_shift;
    a.k_nscale = static_cast<int>(sq_scale_count(k->S, k->layout, k->block));
    a.score_scale = score_scale;
    a.kv_tile = kv_tile;
    a.causal = causal;
    a.sinks = sinks;
    a.out = static_cast<float*>(out); a.out_bf16 = out_dtype == SQ_BF16;
    a.ob = ob; a.ot = ot; a.oh = oh;
    a.lse = lse; a.lb = lb; a.lh = lh;
    // the key loop addresses one (b, kv head) slice of K and of V^T with 32-bit byte offsets
    constexpr int64_t kLim = int64_t(1) << 31;
    if ((k->S + 256) * k->st >= kLim)
        return fail(SQ_ERR_UNSUPPORTED, "sq_attn: one kv head's keys span more than 2 GiB (S * st)");
    if (v->dtype == SQ_FP8E4M3 && (k->D * v->sd + 256) >= kLim)
        return fail(SQ_ERR_UNSUPPORTED, "sq_attn: one kv head's FP8 values span more than 2 GiB");
    if (v->dtype == SQ_BF16 && 2 * k->D * (padded_keys(k->S) + 256) >= kLim)
        return fail(SQ_ERR_UNSUPPORTED, "sq_attn: one kv head's values span more than 2 GiB");
    if (v->dtype == SQ_FP8E4M3) {
        if (v->st != 1) return fail(SQ_ERR_STRIDE, "sq_attn: FP8 values must be channel-major (st == 1)");
        if (!v->scale) return fail(SQ_ERR_NULL, "sq_attn: FP8 values need their per-channel scales");
        if (v->sd < (k->S + 15) / 16 * 16 || v->sd % 16 || v->sb < 0 || v->sh < 0 || v->vsb < 0 || v->vsh < 0)
            return fail(SQ_ERR_STRIDE, "sq_attn: FP8 channel stride must be a multiple of 16 >= keys rounded up");
        if ((reinterpret_cast<uintptr_t>(v->data) & 15) || v->sb % 16 || v->sh % 16)
            return fail(SQ_ERR_ALIGN, "sq_attn: FP8 channel rows must start on 16-byte boundaries");
        a.v = v->data; a.v_fp8 = 1;
        a.vsb = v->sb; a.vsh = v->sh; a.vsd = v->sd;
        a.vscale = v->scale; a.vssb = v->vsb; a.vssh = v->vsh;
        return launch_attn(a, stream);
    }
    if (v->dtype != SQ_BF16) return fail(SQ_ERR_UNSUPPORTED, "sq_attn: values must be bf16 or FP8 e4m3");
    if (v->sd != 1) return fail(SQ_ERR_STRIDE, "sq_attn: bf16 values must be token-major (sd == 1)");
    if ((reinterpret_cast<uintptr_t>(v->data) & 15) || v->sb % 8 || v->st % 8 || v->sh % 8 || v->sb < 0 || v->st < 0 ||
        v->sh < 0)
        return fail(SQ_ERR_ALIGN, "sq_attn: bf16 value rows must start on 16-byte boundaries");
    st = check_ws(ws, ws_bytes, sq_attn_workspace_bytes(q, k, v), "sq_attn");
    if (st) return st;
    const int64_t spad = padded_keys(k->S);
    VTransposeArgs t{static_cast<const uint16_t*>(v->data), k->B, k->S, k->H, k->D, v->sb, v->st, v->sh,
                     static_cast<uint16_t*>(ws), spad};
    st = launch_v_transpose(t, stream);
    if (st) return st;
    a.v = ws; a.v_fp8 = 0;
    a.vsb = k->H * k->D * spad; a.vsh = k->D * spad; a.vsd = spad;
    return launch_attn(a, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------- C. q8 prefix pass + merge
extern "C" {

namespace {
// The prefix pass's tile images for one kv_tile: every (prefix batch, kv head) slice in whole tiles.
size_t prefix_ws_bytes(const sq_q8prefix& p, int kv_tile) {
    const int64_t ntiles = (p.P + kv_tile - 1) / kv_tile;
    return static_cast<size_t>(p.B) * static_cast<size_t>(p.Hk) * static_cast<size_t>(ntiles) *
           prefix_image_bytes(p.D, kv_tile);
}
}  // namespace

size_t sq_attn_prefix_lse_merge_workspace_bytes(const sq_qk* q, const sq_q8prefix* prefix) {
    if (!q || !prefix || prefix->B < 1 || prefix->P < 1 || prefix->Hk < 1 || (prefix->D != 64 && prefix->D != 128))
        return 0;
    if (q->B * q->S * q->H == 0) return 0;
    const size_t a = prefix_ws_bytes(*prefix, 64), b = prefix_ws_bytes(*prefix, 128);
    return round_up(a > b ? a : b);
}

int sq_attn_prefix_lse_merge(const sq_qk* q, const sq_q8prefix* prefix, const float* k_mean, int64_t mb, int64_t mh,
                             float score_scale, int kv_tile, float* out, int64_t ob, int64_t ot, int64_t oh,
                             float* lse, int64_t lb, int64_t lh, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* what = "sq_attn_prefix_lse_merge";
    int st = check_qk(q, what);
    if (st) return st;
    if (q->layout == SQ_LAYOUT_THREAD_K) return fail(SQ_ERR_UNSUPPORTED, "%s: q layout THREAD_K is a key layout", what);
    if (!prefix) return fail(SQ_ERR_NULL, "%s: prefix descriptor is NULL", what);
    const sq_q8prefix& p = *prefix;
    if (p.B < 0 || p.P < 0 || p.Hk < 1) return fail(SQ_ERR_SHAPE, "%s: bad prefix sizes", what);
    if (p.D != q->D) return fail(SQ_ERR_SHAPE, "%s: prefix head dim %lld differs from q's %lld", what,
                                 (long long)p.D, (long long)q->D);
    if (q->H % p.Hk) return fail(SQ_ERR_SHAPE, "%s: q heads %lld not a multiple of prefix kv heads %lld", what,
                                 (long long)q->H, (long long)p.Hk);
    if (p.B != 1 && p.B != q->B) return fail(SQ_ERR_SHAPE, "%s: prefix batch must be 1 or q's batch", what);
    if (q->B * q->S * q->H == 0 || p.P == 0) return SQ_OK;
    if (!p.k || !p.v || !p.k_scale || !p.v_scale) return fail(SQ_ERR_NULL, "%s: prefix tensors are NULL", what);
    if (!out || !lse) return fail(SQ_ERR_NULL, "%s: out and lse (the projected pass) are required", what);
    if ((reinterpret_cast<uintptr_t>(p.k) & 15) || (reinterpret_cast<uintptr_t>(p.v) & 15) || p.kb % 16 ||
        p.kt % 16 || p.kh % 16 || p.vb % 16 || p.vt % 16 || p.vh % 16)
        return fail(SQ_ERR_ALIGN, "%s: prefix code rows must start on 16-byte boundaries", what);
    if ((reinterpret_cast<uintptr_t>(p.k_scale) & 1) || (reinterpret_cast<uintptr_t>(p.v_scale) & 1))
        return fail(SQ_ERR_ALIGN, "%s: FP16 scales must be 2-byte aligned", what);
    if (p.kb < 0 || p.kt < 0 || p.kh < 0 || p.vb < 0 || p.vt < 0 || p.vh < 0 || p.ksb < 0 || p.kst < 0 ||
        p.ksh < 0 || p.vsb < 0 || p.vst < 0 || p.vsh < 0 || ob < 0 || ot < 0 || oh < 0 || lb < 0 || lh < 0)
        return fail(SQ_ERR_STRIDE, "%s: negative stride", what);
    if (k_mean && ((reinterpret_cast<uintptr_t>(k_mean) & 15) || mb % 4 || mh % 4 || mb < 0 || mh < 0))
        return fail(SQ_ERR_ALIGN, "%s: k_mean rows must be 16-byte aligned", what);
    if (kv_tile != 64 && kv_tile != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: kv_tile must be 64 or 128", what);
    if (!(score_scale > 0.0f) || !std::isfinite(score_scale))
        return fail(SQ_ERR_SHAPE, "%s: score_scale must be finite and > 0", what);
    {
        // rows may not overlap, and one (b, kv head) slice, read in whole tiles past P,
        // must stay within 32-bit byte offsets
        const int64_t groups = p.D / 32;
        if (p.P > 1 && (p.kt < p.D || p.vt < p.D || p.kst < groups || p.vst < groups))
            return fail(SQ_ERR_STRIDE, "%s: prefix token strides must cover a whole row", what);
        const int64_t rows = p.P + 128, lim = int64_t(1) << 31;
        if (rows * p.kt + p.D >= lim || rows * p.vt + p.D >= lim || 2 * (rows * p.kst + groups) >= lim ||
            2 * (rows * p.vst + groups) >= lim)
            return fail(SQ_ERR_UNSUPPORTED, "%s: one prefix slice spans 2 GiB or more", what);
    }
    {
        // the tile images of one (prefix batch, kv head) are addressed with 32-bit offsets
        const int64_t ntiles = (p.P + kv_tile - 1) / kv_tile;
        if (ntiles * static_cast<int64_t>(prefix_image_bytes(p.D, kv_tile)) >= (int64_t(1) << 31))
            return fail(SQ_ERR_UNSUPPORTED, "%s: %lld prefix keys (the tile images of one head span 2 GiB)", what,
                        (long long)p.P);
        st = check_ws(ws, ws_bytes, prefix_ws_bytes(p, kv_tile), what);
        if (st) return st;
    }
    PrefixArgs a{};
    a.img = static_cast<uint8_t*>(ws);
    a.ntiles = (p.P + kv_tile - 1) / kv_tile;
    a.q = q->codes; a.B = q->B; a.Sq = q->S; a.H = q->H; a.D = q->D;
    a.qsb = q->sb; a.qst = q->st; a.qsh = q->sh;
    a.qs = q->scales; a.qssb = q->ssb; a.qssh = q->ssh; a.q_layout = q->layout; a.q_block = q->block;
    a.PB = p.B; a.P = p.P; a.Hk = p.Hk;
    a.k = p.k; a.kb = p.kb; a.kt = p.kt; a.kh = p.kh;
    a.ks = p.k_scale; a.ksb = p.ksb; a.kst = p.kst; a.ksh = p.ksh;
    a.v = p.v; a.vb = p.vb; a.vt = p.vt; a.vh = p.vh;
    a.vs = p.v_scale; a.vsb = p.vsb; a.vst = p.vst; a.vsh = p.vsh;
    a.mu = k_mean; a.mb = mb; a.mh = mh;
    a.score_scale = score_scale;
    a.kv_tile = kv_tile;
    a.out = out; a.ob = ob; a.ot = ot; a.oh = oh;
    a.lse = lse; a.lb = lb; a.lh = lh;
    return launch_prefix(a, stream);
}

// ---------------------------------------------------------------------------- C2. log-sum-exp merge
int sq_lse_merge(float* out, int64_t ob, int64_t ot, int64_t oh, float* lse, int64_t lb, int64_t lh, const float* other,
                 int64_t pb, int64_t pt, int64_t ph, const float* other_lse, int64_t qb, int64_t qh, int64_t B, int64_t S,
                 int64_t H, int64_t D, void* stream) {
    clear_error();
    const char* what = "sq_lse_merge";
    if (D != 64 && D != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: head dim %lld is not 64 or 128", what, (long long)D);
    if (B < 0 || S < 0 || H < 0) return fail(SQ_ERR_SHAPE, "%s: negative size", what);
    if (B * S * H == 0) return SQ_OK;
    if (!out || !lse || !other || !other_lse) return fail(SQ_ERR_NULL, "%s: an output or log-sum-exp pointer is NULL", what);
    if (ob < 0 || ot < 0 || oh < 0 || lb < 0 || lh < 0 || pb < 0 || pt < 0 || ph < 0 || qb < 0 || qh < 0)
        return fail(SQ_ERR_STRIDE, "%s: negative stride", what);
    if ((reinterpret_cast<uintptr_t>(out) & 15) || (reinterpret_cast<uintptr_t>(other) & 15) || ob % 4 || ot % 4 ||
        oh % 4 || pb % 4 || pt % 4 || ph % 4)
        return fail(SQ_ERR_ALIGN, "%s: out and other rows must start on 16-byte boundaries", what);
    MergeArgs a{out, ob, ot, oh, lse, lb, lh, other, pb, pt, ph, other_lse, qb, qh, B, S, H, D};
    return launch_lse_merge(a, stream);
}

// ---------------------------------------------------------------------------- D2. q8 paged-cache writer
int sq_q8_cache_write(const void* k, const void* v, sq_dtype dtype, int64_t n_tokens, int Hk, int D, int64_t kn,
                      int64_t kh, int64_t vn, int64_t vh, const int64_t* slot_mapping, int8_t* k_cache,
                      uint16_t* k_scale, int8_t* v_cache, uint16_t* v_scale, int64_t num_blocks, int block_size,
                      void* stream) {
    clear_error();
    const char* what = "sq_q8_cache_write";
    if (dtype != SQ_BF16 && dtype != SQ_F32) return fail(SQ_ERR_UNSUPPORTED, "%s: rows must be bf16 or FP32", what);
    if (D != 64 && D != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: head dim %d is not 64 or 128", what, D);
    if (n_tokens < 0 || Hk < 1 || num_blocks < 0 || block_size < 1)
        return fail(SQ_ERR_SHAPE, "%s: n_tokens >= 0, Hk >= 1, num_blocks >= 0 and block_size >= 1 are required", what);
    if (n_tokens == 0) return SQ_OK;
    if (!k || !v || !slot_mapping || !k_cache || !k_scale || !v_cache || !v_scale)
        return fail(SQ_ERR_NULL, "%s: a row, slot-mapping, cache or scale pointer is NULL", what);
    if (kn < 0 || kh < 0 || vn < 0 || vh < 0) return fail(SQ_ERR_STRIDE, "%s: negative stride", what);
    const int64_t per16 = dtype == SQ_BF16 ? 8 : 4;   // elements per 16 bytes
    if ((reinterpret_cast<uintptr_t>(k) & 15) || (reinterpret_cast<uintptr_t>(v) & 15) || kn % per16 || kh % per16 ||
        vn % per16 || vh % per16)
        return fail(SQ_ERR_ALIGN, "%s: k and v rows must start on 16-byte boundaries", what);
    if ((reinterpret_cast<uintptr_t>(k_cache) & 15) || (reinterpret_cast<uintptr_t>(v_cache) & 15) ||
        (reinterpret_cast<uintptr_t>(k_scale) & 1) || (reinterpret_cast<uintptr_t>(v_scale) & 1))
        return fail(SQ_ERR_ALIGN, "%s: caches must be 16-byte and scales 2-byte aligned", what);
    CacheWriteArgs a{};
    a.k = k; a.v = v; a.n = n_tokens; a.Hk = Hk; a.D = D;
    a.kn = kn; a.kh = kh; a.vn = vn; a.vh = vh;
    a.slots = slot_mapping;
    a.kc = k_cache; a.ks = k_scale; a.vc = v_cache; a.vs = v_scale;
    a.nslots = num_blocks * block_size;
    return launch_cache_write(a, dtype == SQ_F32, stream);
}

// ---------------------------------------------------------------------------- D. paged GQA decode
size_t sq_paged_decode_workspace_bytes(int num_seqs, int Hq, int D, int max_seq_len) {
    if (num_seqs <= 0 || Hq <= 0 || D <= 0 || max_seq_len <= 0) return 0;
    const int64_t segs = (max_seq_len + kDecodeSeg - 1) / kDecodeSeg;
    return round_up(sizeof(float) * static_cast<size_t>(num_seqs) * Hq * segs * (D + 2));
}

namespace {
// Validation of the paged decode's arguments (everything but the workspace) into its kernel arguments.
// SQ_OK with *empty set when there is nothing to do; a failure sets the detail under the name what.
int decode_args(const char* what, const void* q, sq_dtype q_dtype, int64_t qn, int64_t qh, const int8_t* k_cache,
                const uint16_t* k_scale, const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks,
                int block_size, int Hk, const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                int num_seqs, int max_seq_len, int Hq, int D, float softmax_scale, const float* sinks, void* out,
                sq_dtype out_dtype, int64_t on, int64_t oh, DecodeArgs& a, bool* empty) {
    *empty = false;
    if (num_seqs < 0 || Hq < 1 || Hk < 1 || num_blocks < 0)
        return fail(SQ_ERR_SHAPE, "%s: bad sizes (num_seqs %d, Hq %d, Hk %d)", what, num_seqs, Hq, Hk);
    if (D != 64 && D != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: head dim %d (64 or 128)", what, D);
    if (q_dtype != SQ_BF16 && q_dtype != SQ_F16)
        return fail(SQ_ERR_UNSUPPORTED, "%s: q dtype %d (bf16 or f16)", what, (int)q_dtype);
    if (block_size != 16) return fail(SQ_ERR_UNSUPPORTED, "%s: block_size %d (only 16)", what, block_size);
    if (Hq % Hk) return fail(SQ_ERR_SHAPE, "%s: Hq %d not a multiple of Hk %d", what, Hq, Hk);
    const int G = Hq / Hk;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(SQ_ERR_UNSUPPORTED, "%s: Hq / Hk = %d (1, 2, 4 or 8)", what, G);
    if (num_seqs == 0) {
        *empty = true;
        return SQ_OK;
    }
    if (max_seq_len < 1) return fail(SQ_ERR_SHAPE, "%s: max_seq_len must be >= 1", what);
    if (!q || !k_cache || !k_scale || !v_cache || !v_scale || !block_table || !seq_lens || !out)
        return fail(SQ_ERR_NULL, "%s: a required pointer is NULL", what);
    if (bt_stride < (max_seq_len + block_size - 1) / block_size)
        return fail(SQ_ERR_STRIDE, "%s: block-table rows (%lld entries) shorter than max_seq_len needs", what,
                    (long long)bt_stride);
    if ((reinterpret_cast<uintptr_t>(q) & 15) || qn % 8 || qh % 8 || qn < 0 || qh < 0)
        return fail(SQ_ERR_ALIGN, "%s: q rows must start on 16-byte boundaries", what);
    if ((reinterpret_cast<uintptr_t>(k_cache) & 15) || (reinterpret_cast<uintptr_t>(v_cache) & 15))
        return fail(SQ_ERR_ALIGN, "%s: caches must be 16-byte aligned", what);
    if (((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & (D / 16 - 1)) != 0)
        return fail(SQ_ERR_ALIGN, "%s: FP16 scale rows must be aligned to their size (%d bytes)", what, D / 16);
    if (on < 0 || oh < 0) return fail(SQ_ERR_STRIDE, "%s: negative output stride", what);
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
        return fail(SQ_ERR_SHAPE, "%s: softmax_scale must be finite and > 0", what);
    {
        const int st = check_out(out, out_dtype, what);
        if (st) return st;
    }
    a = DecodeArgs{};
    a.q = static_cast<const uint16_t*>(q); a.q_f16 = q_dtype == SQ_F16; a.qn = qn; a.qh = qh;
    a.kc = k_cache; a.ks = k_scale; a.vc = v_cache; a.vs = v_scale;
    a.num_blocks = num_blocks; a.bs = block_size; a.Hk = Hk; a.Hq = Hq; a.D = D;
    a.bt = block_table; a.bt_stride = bt_stride; a.lens = seq_lens;
    a.N = num_seqs; a.max_len = max_seq_len;
    a.scale = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);  // log2 units
    a.sinks = sinks;
    a.out = static_cast<float*>(out); a.out_bf16 = out_dtype == SQ_BF16;
    a.on = on; a.oh = oh;
    a.segs = (max_seq_len + kDecodeSeg - 1) / kDecodeSeg;
    return SQ_OK;
}
}  // namespace

int sq_paged_decode(const void* q, sq_dtype q_dtype, int64_t qn, int64_t qh, const int8_t* k_cache, const uint16_t* k_scale,
                    const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks, int block_size, int Hk,
                    const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens, int num_seqs,
                    int max_seq_len, int Hq, int D, float softmax_scale, const float* sinks, void* out,
                    sq_dtype out_dtype, int64_t on, int64_t oh, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    const char* what = "sq_paged_decode";
    DecodeArgs a;
    bool empty = false;
    {
        const int st = decode_args(what, q, q_dtype, qn, qh, k_cache, k_scale, v_cache, v_scale, num_blocks, block_size, Hk,
                                   block_table, bt_stride, seq_lens, num_seqs, max_seq_len, Hq, D, softmax_scale, sinks,
                                   out, out_dtype, on, oh, a, &empty);
        if (st || empty) return st;
    }
    {
        const int st = check_ws(ws, ws_bytes, sq_paged_decode_workspace_bytes(num_seqs, Hq, D, max_seq_len), what);
        if (st) return st;
    }
    a.part = static_cast<float*>(ws);
    return launch_decode(a, stream);
}

int sq_paged_decode_noalloc(const void* q, sq_dtype q_dtype, int64_t qn, int64_t qh, const int8_t* k_cache,
                            const uint16_t* k_scale,
                            const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks, int block_size, int Hk,
                            const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens, int num_seqs,
                            int max_seq_len, int Hq, int D, float softmax_scale, const float* sinks, void* out,
                            sq_dtype out_dtype, int64_t on, int64_t oh, void* stream) {
    clear_error();
    const char* what = "sq_paged_decode_noalloc";
    DecodeArgs a;
    bool empty = false;
    {
        const int st = decode_args(what, q, q_dtype, qn, qh, k_cache, k_scale, v_cache, v_scale, num_blocks, block_size, Hk,
                                   block_table, bt_stride, seq_lens, num_seqs, max_seq_len, Hq, D, softmax_scale, sinks,
                                   out, out_dtype, on, oh, a, &empty);
        if (st || empty) return st;
    }
    const size_t need = sq_paged_decode_workspace_bytes(num_seqs, Hq, D, max_seq_len);
    if (need > SQ_DECODE_SCRATCH_BYTES)
        return fail(SQ_ERR_WORKSPACE,
                    "%s: %d sequences x %d heads up to %d positions need %zu bytes of segment partials, more than the "
                    "library's scratch array (%zu); call sq_paged_decode with a workspace",
                    what, num_seqs, Hq, max_seq_len, need, static_cast<size_t>(SQ_DECODE_SCRATCH_BYTES));
    void* ws = nullptr;
    {
        const int st = decode_scratch(&ws);
        if (st) return st;
    }
    a.part = static_cast<float*>(ws);
    return launch_decode(a, stream);
}


// ---------------------------------------------------------------------------- D3. paged causal prefill
int sq_paged_prefill(const void* q, sq_dtype q_dtype, int64_t qt, int64_t qh, int64_t num_tokens, const int8_t* k_cache,
                     const uint16_t* k_scale, const int8_t* v_cache, const uint16_t* v_scale, int64_t num_blocks,
                     int block_size, int Hk, const int32_t* block_table, int64_t bt_stride, const int32_t* seq_lens,
                     const int32_t* query_start, int num_seqs, int max_seq_len, int Hq, int D, float softmax_scale,
                     const float* sinks, void* out, sq_dtype out_dtype, int64_t ot, int64_t oh, void* stream) {
    clear_error();
    const char* what = "sq_paged_prefill";
    if (num_seqs < 0 || num_tokens < 0 || Hq < 1 || Hk < 1 || num_blocks < 0)
        return fail(SQ_ERR_SHAPE, "%s: bad sizes (num_seqs %d, num_tokens %lld, Hq %d, Hk %d)", what, num_seqs,
                    (long long)num_tokens, Hq, Hk);
    if (D != 64 && D != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: head dim %d (64 or 128)", what, D);
    if (q_dtype != SQ_BF16 && q_dtype != SQ_F16)
        return fail(SQ_ERR_UNSUPPORTED, "%s: q dtype %d (bf16 or f16)", what, (int)q_dtype);
    if (block_size != 16) return fail(SQ_ERR_UNSUPPORTED, "%s: block_size %d (only 16)", what, block_size);
    if (Hq % Hk) return fail(SQ_ERR_SHAPE, "%s: Hq %d not a multiple of Hk %d", what, Hq, Hk);
    const int G = Hq / Hk;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return fail(SQ_ERR_UNSUPPORTED, "%s: Hq / Hk = %d (1, 2, 4 or 8)", what, G);
    if (num_seqs == 0 || num_tokens == 0) return SQ_OK;
    if (max_seq_len < 1) return fail(SQ_ERR_SHAPE, "%s: max_seq_len must be >= 1", what);
    if (num_blocks < 1) return fail(SQ_ERR_SHAPE, "%s: the cache has no blocks", what);
    if (num_tokens >= (int64_t(1) << 31) / 2)
        return fail(SQ_ERR_UNSUPPORTED, "%s: %lld query tokens (fewer than 2^30)", what, (long long)num_tokens);
    if (!q || !k_cache || !k_scale || !v_cache || !v_scale || !block_table || !seq_lens || !query_start || !out)
        return fail(SQ_ERR_NULL, "%s: a required pointer is NULL", what);
    if (bt_stride < (max_seq_len + block_size - 1) / block_size)
        return fail(SQ_ERR_STRIDE, "%s: block-table rows (%lld entries) shorter than max_seq_len needs", what,
                    (long long)bt_stride);
    if ((reinterpret_cast<uintptr_t>(q) & 15) || qt % 8 || qh % 8 || qt < 0 || qh < 0)
        return fail(SQ_ERR_ALIGN, "%s: q rows must start on 16-byte boundaries", what);
    if ((reinterpret_cast<uintptr_t>(k_cache) & 15) || (reinterpret_cast<uintptr_t>(v_cache) & 15))
        return fail(SQ_ERR_ALIGN, "%s: caches must be 16-byte aligned", what);
    if (((reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) & 1) != 0)
        return fail(SQ_ERR_ALIGN, "%s: FP16 scales must be 2-byte aligned", what);
    if (ot < 0 || oh < 0) return fail(SQ_ERR_STRIDE, "%s: negative output stride", what);
    if (!(softmax_scale > 0.0f) || !std::isfinite(softmax_scale))
        return fail(SQ_ERR_SHAPE, "%s: softmax_scale must be finite and > 0", what);
    {
        const int st = check_out(out, out_dtype, what);
        if (st) return st;
    }
    PrefillArgs a{};
    a.q = static_cast<const uint16_t*>(q); a.q_f16 = q_dtype == SQ_F16; a.qt = qt; a.qh = qh;
    a.kc = k_cache; a.ks = k_scale; a.vc = v_cache; a.vs = v_scale;
    a.num_blocks = num_blocks; a.Hk = Hk; a.Hq = Hq; a.D = D;
    a.bt = block_table; a.bt_stride = bt_stride;
    a.lens = seq_lens; a.qstart = query_start;
    a.N = num_seqs; a.max_len = max_seq_len;
    a.nqb = num_tokens / (32 * kPrefillWaves / G) + num_seqs;
    a.T = static_cast<int>(num_tokens);
    a.scale = static_cast<float>(static_cast<double>(softmax_scale) * 1.4426950408889634);  // log2 units
    a.sinks = sinks;
    a.out = static_cast<float*>(out); a.out_bf16 = out_dtype == SQ_BF16;
    a.ot = ot; a.oh = oh;
    if (a.nqb * Hk >= (int64_t(1) << 31)) return fail(SQ_ERR_UNSUPPORTED, "%s: too many query blocks", what);
    return launch_prefill(a, stream);
}

}  // extern "C"
