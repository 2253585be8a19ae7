#include "sq_internal.h"
namespace sq {
int launch_prefix(const PrefixArgs&, void*) { return fail(SQ_ERR_UNSUPPORTED, "prefix pass not built yet"); }
int launch_decode(const DecodeArgs&, void*) { return fail(SQ_ERR_UNSUPPORTED, "paged decode not built yet"); }
}
extern "C" {
size_t sq_attn_prefix_lse_merge_workspace_bytes(const sq_qk*, const sq_q8prefix*) { return 0; }
int sq_attn_prefix_lse_merge(const sq_qk*, const sq_q8prefix*, const float*, int64_t, int64_t, float, int, float*,
                             int64_t, int64_t, int64_t, float*, int64_t, int64_t, void*, size_t, void*) {
    return sq::fail(SQ_ERR_UNSUPPORTED, "prefix pass not built yet");
}
size_t sq_paged_decode_workspace_bytes(int, int, int, int) { return 0; }
int sq_paged_decode(const void*, int64_t, int64_t, const int8_t*, const uint16_t*, const int8_t*, const uint16_t*,
                    int64_t, int, int, const int32_t*, int64_t, const int32_t*, int, int, int, int, float, float*,
                    int64_t, int64_t, void*, size_t, void*) {
    return sq::fail(SQ_ERR_UNSUPPORTED, "paged decode not built yet");
}
}
