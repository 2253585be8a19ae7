// Host-side argument validation and error reporting for libsq. This file makes no
// HIP call: every check runs before anything is enqueued, so a rejected call leaves
// the stream untouched, and the checks can be exercised on a machine without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>

#include "sq_internal.h"

namespace sq {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = 0; }

bool trace_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("SQ_TRACE");
        return v != nullptr && v[0] != 0 && !(v[0] == '0' && v[1] == 0);
    }();
    return on;
}

void trace_launch(const char* kernel, unsigned gx, unsigned gy, unsigned gz, unsigned block, size_t lds,
                  const void* stream) {
    std::fprintf(stderr, "sq_trace: %s grid=(%u,%u,%u) block=%u dyn_lds=%zu stream=%p\n", kernel, gx, gy, gz, block,
                 lds, stream);
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int64_t scale_count(int64_t T, int layout, int block) {
    switch (layout) {
    case SQ_LAYOUT_PER_BLOCK:
        if (block != 32 && block != 64 && block != 128) return -1;
        return (T + block - 1) / block;
    case SQ_LAYOUT_THREAD_Q: return block == 32 ? (T + 127) / 128 * 32 : -1;
    case SQ_LAYOUT_THREAD_K: return block == 64 ? (T + 63) / 64 * 4 : -1;
    case SQ_LAYOUT_WARP_Q: return block == 128 ? (T + 127) / 128 * 4 : -1;
    }
    return -1;
}

int check_layout(int layout, int block, const char* what) {
    if (scale_count(1, layout, block) < 0)
        return fail(SQ_ERR_UNSUPPORTED, "%s: layout %d with block %d is not one of THREAD_Q:32, THREAD_K:64, "
                    "WARP_Q:128, PER_BLOCK:32|64|128", what, layout, block);
    return SQ_OK;
}

int check_rows(const sq_rows* x, const char* what) {
    if (!x) return fail(SQ_ERR_NULL, "%s: row descriptor is NULL", what);
    if (x->B < 0 || x->T < 0 || x->H < 0) return fail(SQ_ERR_SHAPE, "%s: negative size", what);
    if (x->D != 64 && x->D != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: head dim %lld is not 64 or 128", what, (long long)x->D);
    if (x->B * x->T * x->H == 0) return SQ_OK;
    if (!x->data) return fail(SQ_ERR_NULL, "%s: data is NULL", what);
    if (x->sb < 0 || x->st < 0 || x->sh < 0) return fail(SQ_ERR_STRIDE, "%s: negative stride", what);
    if (!aligned16(x->data) || x->sb % 8 || x->st % 8 || x->sh % 8)
        return fail(SQ_ERR_ALIGN, "%s: rows must start on 16-byte boundaries (strides multiple of 8 elements)", what);
    return SQ_OK;
}

int check_norm(const sq_norm* n, const sq_rows* x, const char* what) {
    if (!n || n->mode == SQ_NORM_NONE) return SQ_OK;
    if (n->mode != SQ_NORM_HEAD && n->mode != SQ_NORM_ALL_HEADS)
        return fail(SQ_ERR_UNSUPPORTED, "%s: unknown norm mode %d", what, (int)n->mode);
    if (!n->weight) return fail(SQ_ERR_NULL, "%s: norm weight is NULL", what);
    if (!aligned16(n->weight)) return fail(SQ_ERR_ALIGN, "%s: norm weight must be 16-byte aligned", what);
    if (!(n->eps >= 0.0f) || std::isinf(n->eps)) return fail(SQ_ERR_SHAPE, "%s: eps must be finite and >= 0", what);
    if (n->mode == SQ_NORM_HEAD && n->mean_sq)
        return fail(SQ_ERR_UNSUPPORTED, "%s: mean_sq is only read by the all-heads norm", what);
    (void)x;
    return SQ_OK;
}

int check_rope(const sq_rope* r, const sq_rows* x, const char* what) {
    if (!r || r->mode == SQ_ROPE_NONE) return SQ_OK;
    if (r->mode != SQ_ROPE_SPLIT_HALF && r->mode != SQ_ROPE_INTERLEAVED)
        return fail(SQ_ERR_UNSUPPORTED, "%s: unknown rope mode %d", what, (int)r->mode);
    if (!r->table) return fail(SQ_ERR_NULL, "%s: rope table is NULL", what);
    if (r->pairs < 1 || r->pairs > x->D / 2)
        return fail(SQ_ERR_SHAPE, "%s: rope pairs %lld outside [1, D/2]", what, (long long)r->pairs);
    if (r->rb < 0 || r->rs < 0 || r->rp < 0) return fail(SQ_ERR_STRIDE, "%s: negative rope stride", what);
    if ((reinterpret_cast<uintptr_t>(r->table) & 3) != 0) return fail(SQ_ERR_ALIGN, "%s: rope table misaligned", what);
    return SQ_OK;
}

int check_qk(const sq_qk* t, const char* what) {
    if (!t) return fail(SQ_ERR_NULL, "%s: descriptor is NULL", what);
    if (t->B < 0 || t->S < 0 || t->H < 0) return fail(SQ_ERR_SHAPE, "%s: negative size", what);
    if (t->D != 64 && t->D != 128) return fail(SQ_ERR_UNSUPPORTED, "%s: head dim %lld is not 64 or 128", what, (long long)t->D);
    int st = check_layout(t->layout, t->block, what);
    if (st) return st;
    if (t->B * t->S * t->H == 0) return SQ_OK;
    if (!t->codes || !t->scales) return fail(SQ_ERR_NULL, "%s: codes or scales are NULL", what);
    if (!aligned16(t->codes) || t->sb % 16 || t->st % 16 || t->sh % 16)
        return fail(SQ_ERR_ALIGN, "%s: code rows must start on 16-byte boundaries", what);
    if (t->ssb < 0 || t->ssh < 0) return fail(SQ_ERR_STRIDE, "%s: negative scale stride", what);
    return SQ_OK;
}

RowArgs row_args(const sq_rows* x, const sq_norm* n, const sq_rope* r) {
    RowArgs a{};
    a.x = static_cast<const uint16_t*>(x->data);
    a.B = x->B; a.T = x->T; a.H = x->H; a.D = x->D;
    a.sb = x->sb; a.st = x->st; a.sh = x->sh;
    a.norm = n ? n->mode : SQ_NORM_NONE;
    if (a.norm != SQ_NORM_NONE) {
        a.w = static_cast<const uint16_t*>(n->weight);
        a.wd = a.norm == SQ_NORM_ALL_HEADS ? x->H * x->D : x->D;
        a.wrows = n->weight_rows;
        a.ms = n->mean_sq;
        a.msb = n->msb; a.mst = n->mst;
        a.eps = n->eps;
    }
    a.rope = r ? r->mode : SQ_ROPE_NONE;
    if (a.rope != SQ_ROPE_NONE) {
        a.table = r->table;
        a.pairs = r->pairs; a.rb = r->rb; a.rs = r->rs; a.rp = r->rp; a.rc = r->rc;
        a.rope_contig = r->rp == 2 && r->rc == 1 && (reinterpret_cast<uintptr_t>(r->table) & 15) == 0 &&
                        r->rb % 4 == 0 && r->rs % 4 == 0;
        // split half over fewer than D/2 pairs puts a channel's partner outside the lane that holds it
        if (a.rope == SQ_ROPE_SPLIT_HALF && r->pairs != x->D / 2) {
            a.rope = kRopeSplitPart;
            a.rope_contig = false;
        }
    }
    return a;
}

}  // namespace sq

extern "C" {

int64_t sq_scale_count(int64_t T, sq_layout layout, int block) { return sq::scale_count(T, layout, block); }

const char* sq_status_string(int status) {
    switch (status) {
    case SQ_OK: return "SQ_OK";
    case SQ_ERR_NULL: return "SQ_ERR_NULL";
    case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE";
    case SQ_ERR_STRIDE: return "SQ_ERR_STRIDE";
    case SQ_ERR_ALIGN: return "SQ_ERR_ALIGN";
    case SQ_ERR_UNSUPPORTED: return "SQ_ERR_UNSUPPORTED";
    case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE";
    case SQ_ERR_HIP: return "SQ_ERR_HIP";
    }
    return "SQ_ERR_UNKNOWN";
}

const char* sq_last_error(void) { return sq::g_last_error; }

int sq_abi_version(void) { return SQ_ABI_VERSION; }

}  // extern "C"
