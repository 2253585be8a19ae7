// Paged, GQA-stacked decode over a q8 KV cache on gfx950.
//
// Method: [impl] fastkernels L2/attention_impl.py (_cache_seq: block-table gather,
// _sdpa_one / _decode_torch: one query at position L - 1 attends positions 0..L-1,
// _repeat_kv_for_heads: q head h reads kv head h / (Hq / Hk)); [tq] vLLM
// triton_turboquant_unified_attention.py (GQA heads stacked on one pass over a kv
// head's pages; the 3D kernel's split over KV segments, merged afterwards by the
// segments' max and exp-sum); [kit] WanGP shared/attention_kit.py (q8: int8 per
// token, head and 32 channels with one FP16 scale).
//
// The path is bound by HBM: per cached token and kv head 2 x 128 code bytes + 2 x 8
// scale bytes. One workgroup (4 waves) owns one segment of kDecodeSeg positions of
// one (sequence, kv head) and serves all Hq / Hk query heads from a single read of
// the segment's K and V:
//  * lane l holds channels 16 (l % 8) .. +15 of token l / 8 of an 8-token step, so a
//    128-byte cache row is one 16-byte load per lane, 8 lanes per row;
//  * pass 1 writes the segment's scores (log2 units: q carries softmax_scale *
//    log2 e) to LDS; per-group dots are scaled by their FP16 key scale before the
//    8-lane butterfly;
//  * pass 2 reads V once, p = 2^(s - M) against the segment max M (no rescaling in
//    the loop), and accumulates p * code * scale in FP32;
//  * the partial (acc, M, l) of each (query head, segment) goes to the workspace;
//    k_decode_reduce merges the segments of a query by their maxima.
// Positions whose block-table entry is outside [0, num_blocks) are skipped (never
// read), so a bad table cannot fault the device.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

constexpr int kD = 128;
constexpr int kSeg = kDecodeSeg;
constexpr int kTpw = kSeg / 4;  // positions per wave

__device__ __forceinline__ void unpack_i8x16(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * k + j] = static_cast<float>(static_cast<int8_t>((w[k] >> (8 * j)) & 0xff));
    }
}

template <int G>
__global__ __launch_bounds__(256) void k_decode_split(DecodeArgs a) {
    constexpr int ST = kTpw / 8;          // 8-position steps per wave
    constexpr int PG = kTpw / 16;         // pages per wave
    __shared__ float sc[kSeg * G];
    __shared__ float red[4 * G * kD];
    __shared__ float wred[4 * G];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lc = l & 7, tr = l >> 3;
    // kv head fastest in the grid: the workgroups of one segment's 8 heads run together, so
    // the rows of every cache slot (all heads side by side in NHD) are read in one window
    const int hk = blockIdx.x, seg = blockIdx.y, n = blockIdx.z;
    const int L = min(a.lens[n], a.max_len);
    const int s0 = seg * kSeg;
    if (s0 >= L) return;  // uniform over the workgroup
    const int s1 = min(L, s0 + kSeg);
    const int wp0 = s0 + w * kTpw;        // first position of this wave (a multiple of 16)
    const int32_t* bt = a.bt + static_cast<int64_t>(n) * a.bt_stride;

    // the physical block of each of the wave's pages (one table read per page; -1 if unused or invalid)
    int myblk = -1;
    if (l < PG && wp0 + 16 * l < s1) {
        const int b = bt[(wp0 >> 4) + l];
        myblk = (b >= 0 && b < a.num_blocks) ? b : -1;
    }
    int64_t rowbase[PG];
#pragma unroll
    for (int pg = 0; pg < PG; ++pg) {
        const int b = __builtin_amdgcn_readlane(myblk, pg);
        rowbase[pg] = b < 0 ? -1 : static_cast<int64_t>(b) * 16 * a.Hk + hk;   // row of slot 0, this kv head
    }

    // the G query heads of this kv head, channels 16 lc .. 16 lc + 15, in log2 units
    float q[G][16];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uint16_t* qp = a.q + static_cast<int64_t>(n) * a.qn + static_cast<int64_t>(hk * G + h) * a.qh + 16 * lc;
        float f[16];
        unpack_bf16x8(*reinterpret_cast<const uint4*>(qp), f);
        unpack_bf16x8(*reinterpret_cast<const uint4*>(qp + 8), f + 8);
#pragma unroll
        for (int c = 0; c < 16; ++c) q[h][c] = f[c] * a.scale;
    }

    // ---- pass 1: every key load of the wave in flight at once, then the scores
    uint4 kraw[ST];
    float ksc[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        const int pos = wp0 + 8 * st + tr;
        const int64_t rb = rowbase[st >> 1];
        const bool ok = rb >= 0 && pos < s1;
        const int64_t row = rb + static_cast<int64_t>(8 * (st & 1) + tr) * a.Hk;
        kraw[st] = ok ? *reinterpret_cast<const uint4*>(a.kc + row * kD + 16 * lc) : make_uint4(0, 0, 0, 0);
        ksc[st] = ok ? f16_to_f32(a.ks[row * (kD / 32) + (lc >> 1)]) : 0.0f;
    }
    // the value loads go out with the key loads: both streams in flight before any math
    uint4 vraw[ST];
    float vsc[ST];
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        const int pos = wp0 + 8 * st + tr;
        const int64_t rb = rowbase[st >> 1];
        const bool ok = rb >= 0 && pos < s1;
        const int64_t row = rb + static_cast<int64_t>(8 * (st & 1) + tr) * a.Hk;
        vraw[st] = ok ? *reinterpret_cast<const uint4*>(a.vc + row * kD + 16 * lc) : make_uint4(0, 0, 0, 0);
        vsc[st] = ok ? f16_to_f32(a.vs[row * (kD / 32) + (lc >> 1)]) : 0.0f;
    }
#pragma unroll
    for (int st = 0; st < ST; ++st) {
        const int pos = wp0 + 8 * st + tr;
        const bool ok = rowbase[st >> 1] >= 0 && pos < s1;
        float kf[16];
        unpack_i8x16(kraw[st], kf);
        float part[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float d = q[h][0] * kf[0];
#pragma unroll
            for (int c = 1; c < 16; ++c) d = __builtin_fmaf(q[h][c], kf[c], d);
            part[h] = d * ksc[st];
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            part[h] += shfl_xor(part[h], 1);
            part[h] += shfl_xor(part[h], 2);
            part[h] += shfl_xor(part[h], 4);
        }
        if (lc == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) sc[(w * kTpw + 8 * st + tr) * G + h] = ok ? part[h] : -__builtin_inff();
        }
    }
    __syncthreads();

    // ---- segment max per query head
    float M[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = -__builtin_inff();
        for (int t = tid; t < kSeg; t += 256) m = fmaxf(m, sc[t * G + h]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, shfl_xor(m, off));
        if (l == 0) wred[w * G + h] = m;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h)
        M[h] = fmaxf(fmaxf(wred[h], wred[G + h]), fmaxf(wred[2 * G + h], wred[3 * G + h]));

    // ---- pass 2: p = 2^(s - M), acc += p * v (missing positions have s = -inf: p = 0, v = 0)
    float acc[G][16], ls[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        ls[h] = 0.0f;
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[h][c] = 0.0f;
    }
    const bool any = M[0] > -__builtin_inff();   // every head's max is finite iff a position exists
    if (any) {
#pragma unroll
        for (int st = 0; st < ST; ++st) {
            const int tl = w * kTpw + 8 * st + tr;
            float vf[16];
            unpack_i8x16(vraw[st], vf);
#pragma unroll
            for (int c = 0; c < 16; ++c) vf[c] = vf[c] * vsc[st];
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = __builtin_amdgcn_exp2f(sc[tl * G + h] - M[h]);
                ls[h] += p;
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[h][c] = __builtin_fmaf(p, vf[c], acc[h][c]);
            }
        }
    }
    // reduce over the 8 token lanes of each channel slice, then over the 4 waves
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int off = 8; off < 64; off <<= 1) {
            ls[h] += shfl_xor(ls[h], off);
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[h][c] += shfl_xor(acc[h][c], off);
        }
    }
    __syncthreads();  // wred reuse
    if (tr == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int c = 0; c < 16; ++c) red[(w * G + h) * kD + 16 * lc + c] = acc[h][c];
        }
    }
    if (l == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) wred[w * G + h] = ls[h];
    }
    __syncthreads();
    const int nseg = a.segs;
    for (int i = tid; i < G * (kD + 2); i += 256) {
        const int h = i / (kD + 2), c = i % (kD + 2);
        float v;
        if (c < kD) v = (red[h * kD + c] + red[(G + h) * kD + c]) + (red[(2 * G + h) * kD + c] + red[(3 * G + h) * kD + c]);
        else if (c == kD) v = M[h];
        else v = (wred[h] + wred[G + h]) + (wred[2 * G + h] + wred[3 * G + h]);
        a.part[((static_cast<int64_t>(n) * a.Hq + hk * G + h) * nseg + seg) * (kD + 2) + c] = v;
    }
}

// Merge the segments of one (sequence, query head): weights 2^(M_s - max M).
__global__ __launch_bounds__(kD) void k_decode_reduce(DecodeArgs a) {
    const int c = threadIdx.x, hq = blockIdx.x, n = blockIdx.y;
    const int L = min(a.lens[n], a.max_len);
    const int nseg = L > 0 ? (L + kSeg - 1) / kSeg : 0;
    const float* p = a.part + (static_cast<int64_t>(n) * a.Hq + hq) * a.segs * (kD + 2);
    float mg = -__builtin_inff();
    for (int s = 0; s < nseg; ++s) mg = fmaxf(mg, p[s * (kD + 2) + kD]);
    float tot = 0.0f, o = 0.0f;
    if (mg > -__builtin_inff()) {
        for (int s = 0; s < nseg; ++s) {
            const float ms = p[s * (kD + 2) + kD];
            const float wgt = ms > -__builtin_inff() ? __builtin_amdgcn_exp2f(ms - mg) : 0.0f;
            tot = __builtin_fmaf(wgt, p[s * (kD + 2) + kD + 1], tot);
            o = __builtin_fmaf(wgt, p[s * (kD + 2) + c], o);
        }
    }
    a.out[static_cast<int64_t>(n) * a.on + static_cast<int64_t>(hq) * a.oh + c] = tot > 0.0f ? o / tot : 0.0f;
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

int launch_decode(const DecodeArgs& a, void* stream) {
    if (a.N == 0) return SQ_OK;
    const int G = a.Hq / a.Hk;
    dim3 g1(static_cast<unsigned>(a.Hk), static_cast<unsigned>(a.segs), static_cast<unsigned>(a.N));
    switch (G) {
    case 1: hipLaunchKernelGGL(k_decode_split<1>, g1, dim3(256), 0, S(stream), a); break;
    case 2: hipLaunchKernelGGL(k_decode_split<2>, g1, dim3(256), 0, S(stream), a); break;
    case 4: hipLaunchKernelGGL(k_decode_split<4>, g1, dim3(256), 0, S(stream), a); break;
    default: hipLaunchKernelGGL(k_decode_split<8>, g1, dim3(256), 0, S(stream), a); break;
    }
    hipLaunchKernelGGL(k_decode_reduce, dim3(static_cast<unsigned>(a.Hq), static_cast<unsigned>(a.N)), dim3(kD), 0,
                       S(stream), a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_paged_decode: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
