// Log-sum-exp merge of two attentions of the same queries over disjoint key sets on gfx950.
//
// Method: [kit] WanGP shared/attention_kit.py _merge_lse_ (top = max of the two base-2
// log-sum-exps, weights 2^(lse - top) normalised by their sum, out blended in FP32) as
// _attend_with_prefix uses it for a native cached prefix.
//
// A row (b, i, h) of D floats is D/4 lanes with one 16-byte load of each input per lane;
// each lane reads its row's two log-sum-exps itself (the same address across the row's
// lanes is one request). Every load of a wave's rows goes out before the arithmetic.
// HBM-bound: 12 D bytes per row plus 12 bytes of log-sum-exps.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

constexpr int kRowSteps = 4;

template <int D>
__global__ __launch_bounds__(256) void k_lse_merge(MergeArgs a) {
    constexpr int LPR = D / 4, RPW = kWave / LPR;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t rows = a.B * a.S * a.H;
    const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * 4 + w) * (kRowSteps * RPW);
    if (r0 >= rows) return;  // wave-uniform
    float4 x[kRowSteps], y[kRowSteps];
    float la[kRowSteps], lb[kRowSteps];
    int64_t obase[kRowSteps], lbase[kRowSteps];
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s) {
        int64_t r = r0 + s * RPW + lr;
        if (r >= rows) r = rows - 1;   // rows past the end recompute the last row and store nothing
        const int64_t h = r % a.H, i = (r / a.H) % a.S, b = r / (a.H * a.S);
        obase[s] = b * a.ob + i * a.ot + h * a.oh;
        lbase[s] = b * a.lb + h * a.lh + i;
        x[s] = *reinterpret_cast<const float4*>(a.out + obase[s] + 4 * lc);
        y[s] = *reinterpret_cast<const float4*>(a.other + b * a.pb + i * a.pt + h * a.ph + 4 * lc);
        la[s] = a.lse[lbase[s]];
        lb[s] = a.other_lse[b * a.qb + h * a.qh + i];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the arithmetic
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s) {
        const float top = fmaxf(la[s], lb[s]);
        float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float l = -__builtin_inff();
        if (top > -__builtin_inff()) {
            const float wa = __builtin_amdgcn_exp2f(la[s] - top), wb = __builtin_amdgcn_exp2f(lb[s] - top);
            const float tot = wa + wb, fa = wa / tot, fb = wb / tot;
            o = make_float4(x[s].x * fa + y[s].x * fb, x[s].y * fa + y[s].y * fb, x[s].z * fa + y[s].z * fb,
                            x[s].w * fa + y[s].w * fb);
            l = top + __builtin_log2f(tot);
        }
        const int64_t r = r0 + s * RPW + lr;
        if (r < rows) {
            *reinterpret_cast<float4*>(a.out + obase[s] + 4 * lc) = o;
            if (lc == 0) a.lse[lbase[s]] = l;
        }
    }
}

}  // namespace

int launch_lse_merge(const MergeArgs& a, void* stream) {
    const int64_t rows = a.B * a.S * a.H;
    if (rows == 0) return SQ_OK;
    const int64_t per_wg = 4 * kRowSteps * (kWave / (a.D / 4));
    dim3 grid(static_cast<unsigned>((rows + per_wg - 1) / per_wg));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 128) SQ_LAUNCH(k_lse_merge<128>, grid, dim3(256), 0, s, a);
    else SQ_LAUNCH(k_lse_merge<64>, grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_lse_merge: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
