// Log-sum-exp merge of two attentions of the same queries over disjoint key sets on gfx950.
//
// Method: [kit] WanGP shared/attention_kit.py _merge_lse_ (top = max of the two base-2
// log-sum-exps, weights 2^(lse - top) normalised by their sum, out blended in FP32) as
// _attend_with_prefix uses it for a native cached prefix.
//
// A row (b, i, h) of D floats is D/4 lanes with one 16-byte load of each input per lane;
// each lane reads its row's two log-sum-exps itself (the same address across the row's
// lanes is one request). A workgroup takes RB consecutive queries i of one (b, h), so the
// log-sum-exps it reads and writes ((B, H, S) arrays) are whole lines; the workgroups go
// head-fastest, so those running together cover whole stretches of out rows (b, i, 0..H-1).
// Every load of a wave's rows goes out before the arithmetic. HBM-bound: 12 D bytes per row
// plus 12 bytes of log-sum-exps.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

constexpr int kRowSteps = 4;

template <int D>
__global__ __launch_bounds__(256) void k_lse_merge(MergeArgs a) {
    constexpr int LPR = D / 4, RPW = kWave / LPR, RB = 4 * kRowSteps * RPW;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t nib = (a.S + RB - 1) / RB;
    const int64_t h = blockIdx.x % a.H, ib = (blockIdx.x / a.H) % nib, b = blockIdx.x / (a.H * nib);
    const int64_t i0 = ib * RB + w * (kRowSteps * RPW);
    if (b >= a.B || i0 >= a.S) return;  // wave-uniform
    float4 x[kRowSteps], y[kRowSteps];
    float la[kRowSteps], lb[kRowSteps];
    int64_t obase[kRowSteps], lbase[kRowSteps];
#pragma unroll
    for (int s = 0; s < kRowSteps; ++s) {
        int64_t i = i0 + s * RPW + lr;
        if (i >= a.S) i = a.S - 1;   // queries past the end recompute the last one and store nothing
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
        if (i0 + s * RPW + lr < a.S) {
            *reinterpret_cast<float4*>(a.out + obase[s] + 4 * lc) = o;
            if (lc == 0) a.lse[lbase[s]] = l;
        }
    }
}

}  // namespace

int launch_lse_merge(const MergeArgs& a, void* stream) {
    if (a.B * a.S * a.H == 0) return SQ_OK;
    const int64_t rb = 4 * kRowSteps * (kWave / (a.D / 4));   // queries per workgroup
    const int64_t wgs = a.B * a.H * ((a.S + rb - 1) / rb);
    if (wgs >= (int64_t(1) << 31)) return fail(SQ_ERR_UNSUPPORTED, "sq_lse_merge: too many rows (%lld workgroups)", (long long)wgs);
    dim3 grid(static_cast<unsigned>(wgs));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 128) SQ_LAUNCH(k_lse_merge<128>, grid, dim3(256), 0, s, a);
    else SQ_LAUNCH(k_lse_merge<64>, grid, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_lse_merge: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
