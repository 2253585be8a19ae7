// Launchers for a host-only build of libsq's C entry points (api.cpp, validate.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: the argument checks run as in the library, and a call that passes them
// stops here with SQ_ERR_HIP instead of enqueuing a kernel (the host has no GPU). Test infrastructure only.
#include "../../quantized_transformer_attention_amd/csrc/sq_internal.h"

namespace sq {
namespace {
int no_gpu(const char* what) { return fail(SQ_ERR_HIP, "%s: host-only build, no kernel launched", what); }
}  // namespace
int launch_norm_stats(const NormStatsArgs&, void*) { return no_gpu("norm stats"); }
int launch_kmean(const KmeanArgs&, void*) { return no_gpu("k mean"); }
int launch_quant_qk(const QuantArgs&, void*) { return no_gpu("quantizer"); }
int launch_quant_v_fp8(const QuantVArgs&, void*) { return no_gpu("V to FP8"); }
int launch_v_transpose(const VTransposeArgs&, void*) { return no_gpu("V staging"); }
int launch_attn(const AttnArgs&, void*) { return no_gpu("attention core"); }
int launch_prefix(const PrefixArgs&, void*) { return no_gpu("prefix pass"); }
int launch_lse_merge(const MergeArgs&, void*) { return no_gpu("merge"); }
int launch_cache_write(const CacheWriteArgs&, bool, void*) { return no_gpu("cache writer"); }
int launch_decode(const DecodeArgs&, void*) { return no_gpu("decode"); }
int decode_scratch(void**) { return no_gpu("decode scratch"); }
int launch_prefill(const PrefillArgs&, void*) { return no_gpu("prefill"); }
}  // namespace sq
