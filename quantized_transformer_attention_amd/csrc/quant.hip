// Fused q/k prologue and quantizers on gfx950.
//
// [quant] WanGP shared/kernels/qk_quant_triton.py (_rows, _norm_rope_quant,
// norm_rope_mean, norm_rope_quantize) and [kit] WanGP shared/attention_kit.py
// (HeadGroup.mean_squares).
//
// Row layout in a wavefront: a row of D bf16 channels is D/8 lanes; lane l holds the
// 4 channels [4l, 4l + 4) and their split-half rotation partners [D/2 + 4l, D/2 + 4l + 4)
// (two 8-byte loads), so the full split-half rotation and the interleaved rotation are
// lane-local (no cross-lane exchange) and each lane needs the cos/sin of only 4 pairs.
// D = 128 puts 4 rows in a wave, D = 64 puts 8. Per-row reductions (sum of squares,
// |v| max) are xor butterflies inside the row's lanes.
// The quantizer keeps a whole 128-row tile of one head in registers (32 rows per
// wave), so x is read from HBM once and the norm and rotation run once per element,
// then reduces the layout's group maxima in LDS and writes codes from registers.
// Work items (token tile, b, h) go out head-fastest and XCD-contiguous (workgroup i runs
// on XCD i mod 8), so the heads of a token tile share that tile's RoPE table rows in
// one XCD's L2 instead of fetching them from memory once per head.
#include "device.h"
#include "sq_internal.h"

namespace sq {

namespace {

// x[0..3] = channels 4 lc .. 4 lc + 3, x[4..7] = channels D/2 + 4 lc .. D/2 + 4 lc + 3.
template <int D>
__device__ __forceinline__ void load_row_bf16(const uint16_t* row, int lc, float* x) {
    const uint2 u = *reinterpret_cast<const uint2*>(row + 4 * lc);
    const uint2 v = *reinterpret_cast<const uint2*>(row + D / 2 + 4 * lc);
    x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
    x[4] = bf16_lo(v.x); x[5] = bf16_hi(v.x); x[6] = bf16_lo(v.y); x[7] = bf16_hi(v.y);
}

template <int D>
__device__ __forceinline__ void load_row_f32(const float* row, int lc, float* x) {
    const float4 u = *reinterpret_cast<const float4*>(row + 4 * lc);
    const float4 v = *reinterpret_cast<const float4*>(row + D / 2 + 4 * lc);
    x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
    x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
}

// Canonical sum of squares of a row: per lane p = x0*x0 then fma over the other 7
// channels in the order held (4l .. 4l+3, D/2 + 4l .. D/2 + 4l + 3); xor butterfly
// over the row's LPR lanes (offsets LPR/2 .. 1).
template <int LPR>
__device__ __forceinline__ float row_sumsq(const float* x) {
    float p = x[0] * x[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) p = __builtin_fmaf(x[k], x[k], p);
    return row_sum<LPR>(p);
}

// Row prologue [quant] _rows: z = rotate(bf16(norm(x) * w)) for the 8 channels a lane
// holds of row (b, t, h), in two halves so that a wave can put the loads of all its rows
// in flight before it computes any of them: row_fetch issues the loads (unconditionally,
// so a caller passes a row index clamped into [0, T) and masks the result of a row past
// the end), rows4 computes four steps of rows. Every lane of a row takes part in rows4
// (the norm's butterfly and the shared root). SQ_ROPE_SPLIT_HALF rotates all D/2 pairs,
// lane-locally; kRopeSplitPart (split half over pairs < D/2, channel p with p + pairs) takes
// each partner from the row's lanes through the wave's LDS exchange row.
// PERTOK: a weight row per token (RowArgs::wrows), else one shared row.
template <int NORM, int ROPE, bool PERTOK>
struct RowRaw {
    uint2 xu, xv;     // bf16 channels 4 lc .. 4 lc + 3 and D/2 + 4 lc .. D/2 + 4 lc + 3
    float ms;         // all-heads mean square of the token
    uint2 wu, wv;     // per-token weight row, same channels as x
    // rotation table: cos in tc[0..NT), sin in tc[NT..2 NT); NT = 4 pairs of the lane, or
    // with kRopeSplitPart the pair of each of its 8 channels
    static constexpr int NT = ROPE == kRopeSplitPart ? 8 : 4;
    float tc[2 * NT];
};

// Pair of channel slot k (0..7) of lane lc under kRopeSplitPart, or -1 where the channel
// passes through (c >= 2 pairs).
template <int D>
__device__ __forceinline__ int64_t part_pair(int lc, int k, int64_t pairs) {
    const int64_t c = k < 4 ? 4 * lc + k : D / 2 + 4 * lc + (k - 4);
    return c < pairs ? c : (c < 2 * pairs ? c - pairs : -1);
}

// Where the rows of a token range start (the range's first token t0 at (b, h)): a row
// t0 + rr of a tensor sits rr times its token stride in bytes past the base; the entry
// points keep those strides under 16 MiB, so a 24-bit multiply gives the offset.
struct RowBase {
    const char* x;
    const char* ms;
    const char* tb;
    const int32_t* wr;
    uint32_t xst, mst, tst;

    __device__ __forceinline__ RowBase(const RowArgs& a, int64_t b, int64_t t0, int64_t h) {
        x = reinterpret_cast<const char*>(a.x + b * a.sb + t0 * a.st + h * a.sh);
        ms = a.ms ? reinterpret_cast<const char*>(a.ms + b * a.msb + t0 * a.mst) : nullptr;
        tb = a.table ? reinterpret_cast<const char*>(a.table + a.rb * b + a.rs * t0) : nullptr;
        wr = a.wrows ? a.wrows + t0 : nullptr;
        xst = static_cast<uint32_t>(a.st * 2);
        mst = static_cast<uint32_t>(a.mst * 4);
        tst = static_cast<uint32_t>(a.rs * 4);
    }
};

// Loads of row t0 + rr (rr < T - t0).
template <int D, int NORM, int ROPE, bool CONTIG, bool PERTOK>
__device__ __forceinline__ void row_fetch(const RowArgs& a, const RowBase& rb, uint32_t rr, int64_t h, int lc,
                                          int64_t wrow, RowRaw<NORM, ROPE, PERTOK>& r) {
    const char* xr = rb.x + __umul24(rr, rb.xst);
    r.xu = *reinterpret_cast<const uint2*>(xr + 8 * lc);
    r.xv = *reinterpret_cast<const uint2*>(xr + D + 8 * lc);
    if constexpr (NORM == SQ_NORM_ALL_HEADS) r.ms = *reinterpret_cast<const float*>(rb.ms + __umul24(rr, rb.mst));
    if constexpr (NORM != SQ_NORM_NONE && PERTOK) {
        const uint16_t* wr = a.w + wrow * a.wd + (NORM == SQ_NORM_ALL_HEADS ? h * D : 0);
        r.wu = *reinterpret_cast<const uint2*>(wr + 4 * lc);
        r.wv = *reinterpret_cast<const uint2*>(wr + D / 2 + 4 * lc);
    }
    if constexpr (ROPE != SQ_ROPE_NONE) {
        const float* tb = reinterpret_cast<const float*>(rb.tb + __umul24(rr, rb.tst));
        if constexpr (ROPE == SQ_ROPE_SPLIT_HALF && CONTIG) {
            // pairs 4 lc .. 4 lc + 3, stored (cos, sin) interleaved
            const float4 u = *reinterpret_cast<const float4*>(tb + 8 * lc);
            const float4 v = *reinterpret_cast<const float4*>(tb + 8 * lc + 4);
            r.tc[0] = u.x; r.tc[4] = u.y; r.tc[1] = u.z; r.tc[5] = u.w;
            r.tc[2] = v.x; r.tc[6] = v.y; r.tc[3] = v.z; r.tc[7] = v.w;
        } else if constexpr (ROPE == kRopeSplitPart) {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                int64_t pair = part_pair<D>(lc, k, a.pairs);
                if (pair < 0) pair = 0;  // not applied
                r.tc[k] = tb[a.rp * pair];
                r.tc[8 + k] = tb[a.rp * pair + a.rc];
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // split half: pairs 4 lc + u; interleaved: pairs 2 lc, 2 lc + 1, D/4 + 2 lc, D/4 + 2 lc + 1
                // (a pair past the rotated count reads pair 0 and is not applied)
                int64_t pair = ROPE == SQ_ROPE_SPLIT_HALF ? 4 * lc + u : (u < 2 ? 0 : D / 4) + 2 * lc + (u & 1);
                if (pair >= a.pairs) pair = 0;
                r.tc[u] = tb[a.rp * pair];
                r.tc[4 + u] = tb[a.rp * pair + a.rc];
            }
        }
    }
}

// First half of a row's arithmetic: its 8 channels in x and, with a norm, the value
// ms + eps whose reciprocal square root scales the row.
template <int D, int NORM, int ROPE, bool PERTOK>
__device__ __forceinline__ float row_stats(const RowArgs& a, const RowRaw<NORM, ROPE, PERTOK>& r, float* x) {
    x[0] = bf16_lo(r.xu.x); x[1] = bf16_hi(r.xu.x); x[2] = bf16_lo(r.xu.y); x[3] = bf16_hi(r.xu.y);
    x[4] = bf16_lo(r.xv.x); x[5] = bf16_hi(r.xv.x); x[6] = bf16_lo(r.xv.y); x[7] = bf16_hi(r.xv.y);
    if constexpr (NORM == SQ_NORM_HEAD) return row_sumsq<D / 8>(x) / static_cast<float>(D) + a.eps;
    else if constexpr (NORM == SQ_NORM_ALL_HEADS) return r.ms + a.eps;
    else return 1.0f;
}

// 1 / sqrt(v[j]) (both steps correctly rounded) for the four rows v[0..3] of a lane's
// four consecutive steps: lane lc of a row evaluates step lc mod 4, then each step takes
// its value from that lane of the row, so a wave evaluates the root once per four steps.
template <int LPR>
__device__ __forceinline__ void inv_rms4(const float* v, int lc, float* inv) {
    const float t0 = (lc & 1) ? v[1] : v[0], t1 = (lc & 1) ? v[3] : v[2];
    const float r = 1.0f / sqrtf((lc & 2) ? t1 : t0);
    inv[0] = row_lane<LPR, 0>(r);
    inv[1] = row_lane<LPR, 1>(r);
    inv[2] = row_lane<LPR, 2>(r);
    inv[3] = row_lane<LPR, 3>(r);
}

// Second half: z = rotate(bf16(x * inv * w)). xch: this row's D floats of the wave's
// exchange rows in LDS (kRopeSplitPart only).
template <int D, int NORM, int ROPE, bool PERTOK>
__device__ __forceinline__ void row_apply(const RowArgs& a, const RowRaw<NORM, ROPE, PERTOK>& r, const float* x,
                                          float inv, const float* wsh, int lc, float* xch, float* z) {
    float y[8];
    if constexpr (NORM == SQ_NORM_NONE) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = x[k];
    } else {
        float w[8];
        if constexpr (PERTOK) {
            w[0] = bf16_lo(r.wu.x); w[1] = bf16_hi(r.wu.x); w[2] = bf16_lo(r.wu.y); w[3] = bf16_hi(r.wu.y);
            w[4] = bf16_lo(r.wv.x); w[5] = bf16_hi(r.wv.x); w[6] = bf16_lo(r.wv.y); w[7] = bf16_hi(r.wv.y);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) w[k] = wsh[k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = (x[k] * inv) * w[k];
#pragma unroll
        for (int k = 0; k < 8; k += 2) bf16_round2(y[k], y[k + 1]);
    }
    if constexpr (ROPE == SQ_ROPE_NONE) {
#pragma unroll
        for (int k = 0; k < 8; ++k) z[k] = y[k];
    } else if constexpr (ROPE == SQ_ROPE_SPLIT_HALF) {
        // channel 4 lc + k (leading) with its partner D/2 + 4 lc + k (trailing), pair 4 lc + k
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float cs = r.tc[k], sn = r.tc[4 + k];
            z[k] = __builtin_fmaf(cs, y[k], (-sn) * y[4 + k]);
            z[4 + k] = __builtin_fmaf(sn, y[k], cs * y[4 + k]);
        }
    } else if constexpr (ROPE == kRopeSplitPart) {
        // the row goes to LDS, each rotated channel reads its partner back: leading c < pairs
        // with c + pairs, trailing c in [pairs, 2 pairs) with c - pairs. The fences order the
        // wave's LDS accesses for the compiler (a wave executes its LDS operations in order).
        *reinterpret_cast<float4*>(xch + 4 * lc) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(xch + D / 2 + 4 * lc) = make_float4(y[4], y[5], y[6], y[7]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int64_t P = a.pairs;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int64_t c = k < 4 ? 4 * lc + k : D / 2 + 4 * lc + (k - 4);
            const float cs = r.tc[k], sn = r.tc[8 + k];
            if (c < P) z[k] = __builtin_fmaf(cs, y[k], (-sn) * xch[c + P]);
            else if (c < 2 * P) z[k] = __builtin_fmaf(sn, xch[c - P], cs * y[k]);
            else z[k] = y[k];
        }
        // the next row's stores wait for these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    } else {  // interleaved: channel 2p with 2p + 1
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t pair = (u < 2 ? 0 : D / 4) + 2 * lc + (u & 1);
            const int k = 2 * u;
            const float cs = r.tc[u], sn = r.tc[4 + u];
            const float z0 = __builtin_fmaf(cs, y[k], (-sn) * y[k + 1]);
            const float z1 = __builtin_fmaf(sn, y[k], cs * y[k + 1]);
            const bool rot = pair < a.pairs;
            z[k] = rot ? z0 : y[k];
            z[k + 1] = rot ? z1 : y[k + 1];
        }
    }
}

// Steps s0 .. s0 + 3 of a lane's fetched rows through both halves into z.
template <int D, int NORM, int ROPE, bool PERTOK>
__device__ __forceinline__ void rows4(const RowArgs& a, const RowRaw<NORM, ROPE, PERTOK>* raw, const float* wsh,
                                      int lc, float* xch, float (*z)[8]) {
    float x[4][8], v[4], inv[4] = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = row_stats<D, NORM, ROPE, PERTOK>(a, raw[j], x[j]);
    if constexpr (NORM != SQ_NORM_NONE) inv_rms4<D / 8>(v, lc, inv);
#pragma unroll
    for (int j = 0; j < 4; ++j) row_apply<D, NORM, ROPE, PERTOK>(a, raw[j], x[j], inv[j], wsh, lc, xch, z[j]);
}

// The shared weight row of a head (PERTOK == false); unused without a norm.
template <int D, int NORM>
__device__ __forceinline__ void load_shared_weights(const RowArgs& a, int64_t h, int lc, float* w) {
    if constexpr (NORM != SQ_NORM_NONE)
        load_row_bf16<D>(a.w + (NORM == SQ_NORM_ALL_HEADS ? h * D : 0), lc, w);
}

// Weight rows of N tokens t0 + rr[i] (all 0 without per-token rows), loaded together.
template <int N>
__device__ __forceinline__ void load_wrows(const RowArgs& a, const RowBase& rb, const uint32_t* rr, int64_t* wrow) {
    if (a.wrows) {
#pragma unroll
        for (int i = 0; i < N; ++i) wrow[i] = rb.wr[rr[i]];
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) wrow[i] = 0;
    }
}

// Group of row r (0..127) of a tile: ((r >> sh) << mul) + ((r & mask) >> low), with the
// four layouts' shifts and masks:
//   THREAD_Q 8 (r / 32) + r mod 8;  THREAD_K 4 (r / 64) + (r mod 8) / 2;
//   WARP_Q r / 32;                  PER_BLOCK r / block (block 32, 64 or 128).
struct GroupMap {
    int sh, mul, mask, low;
    __device__ __forceinline__ GroupMap(int layout, int block) {
        switch (layout) {
        case SQ_LAYOUT_THREAD_Q: sh = 5; mul = 3; mask = 7; low = 0; break;
        case SQ_LAYOUT_THREAD_K: sh = 6; mul = 2; mask = 7; low = 1; break;
        case SQ_LAYOUT_WARP_Q: sh = 5; mul = 0; mask = 0; low = 0; break;
        default: sh = block == 32 ? 5 : (block == 64 ? 6 : 7); mul = 0; mask = 0; low = 0; break;
        }
    }
    __device__ __forceinline__ int operator()(int r) const { return ((r >> sh) << mul) + ((r & mask) >> low); }
};

__host__ __device__ __forceinline__ int groups_per_tile(int layout, int block) {
    switch (layout) {
    case SQ_LAYOUT_THREAD_Q: return 32;
    case SQ_LAYOUT_THREAD_K: return 8;
    case SQ_LAYOUT_WARP_Q: return 4;
    default: return 128 / block;
    }
}

// ---------------------------------------------------------------- A1: mean squares over all heads
// One wave per token; the heads go HPI at a time (a row per HPI-lane group), NB such
// steps with their loads in flight together. Heads past H read head H - 1 and add nothing.
template <int D>
__global__ __launch_bounds__(256) void k_norm_stats(NormStatsArgs a) {
    constexpr int LPR = D / 8, HPI = kWave / LPR, NB = 4;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (tok >= a.B * a.T) return;  // wave-uniform
    const int64_t b = tok / a.T, t = tok % a.T;
    const uint16_t* xt = a.x + b * a.sb + t * a.st;
    float tot = 0.0f;
    for (int64_t h0 = 0; h0 < a.H; h0 += HPI * NB) {
        uint2 u[NB], v[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t h = h0 + HPI * j + lr < a.H ? h0 + HPI * j + lr : a.H - 1;
            u[j] = *reinterpret_cast<const uint2*>(xt + h * a.sh + 4 * lc);
            v[j] = *reinterpret_cast<const uint2*>(xt + h * a.sh + D / 2 + 4 * lc);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its arithmetic
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float x[8] = {bf16_lo(u[j].x), bf16_hi(u[j].x), bf16_lo(u[j].y), bf16_hi(u[j].y),
                                bf16_lo(v[j].x), bf16_hi(v[j].x), bf16_lo(v[j].y), bf16_hi(v[j].y)};
            const float p = row_sumsq<LPR>(x);
#pragma unroll
            for (int i = 0; i < HPI; ++i) {
                const float s = __shfl(p, i * LPR, kWave);
                if (h0 + HPI * j + i < a.H) tot = tot + s;
            }
        }
    }
    if (lane == 0) a.ms[b * a.msb + t * a.mst] = tot / static_cast<float>(a.H * D);
}

// ---------------------------------------------------------------- A2: k mean
// A lane's 16 rows in four steps of 4 rows; the loads of a step go out before the
// arithmetic of the step ahead of it, so two steps of loads are in flight at the start
// and one while a step computes.
template <int D, int NORM, int ROPE, bool CONTIG, bool PERTOK>
__device__ __forceinline__ void kmean_block(const KmeanArgs& a, int64_t b, int64_t h, int64_t blk, int lc, int r,
                                            float* xch) {
    constexpr int LPR = D / 8;
    const bool active = r < 4;
    float wsh[8];
    if constexpr (!PERTOK) load_shared_weights<D, NORM>(a.r, h, lc, wsh);
    float S[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const RowBase base(a.r, b, blk * 64, h);
    const uint32_t rlast = static_cast<uint32_t>(a.r.T - blk * 64 < 64 ? a.r.T - blk * 64 - 1 : 63);
    uint32_t rr[16];
    int64_t wrow[16] = {};
#pragma unroll
    for (int i = 0; i < 16; ++i) rr[i] = min(static_cast<uint32_t>(4 * i + r), rlast);
    if constexpr (PERTOK) load_wrows<16>(a.r, base, rr, wrow);
    RowRaw<NORM, ROPE, PERTOK> raw[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) row_fetch<D, NORM, ROPE, CONTIG, PERTOK>(a.r, base, rr[i], h, lc, wrow[i], raw[i]);
#pragma unroll
    for (int j0 = 0; j0 < 16; j0 += 4) {
        __builtin_amdgcn_sched_barrier(0);  // the step's loads stay ahead of the arithmetic below
        float z[4][8];
        rows4<D, NORM, ROPE, PERTOK>(a.r, raw + j0, wsh, lc, xch, z);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool valid = active && blk * 64 + 4 * (j0 + j) + r < a.r.T;
#pragma unroll
            for (int k = 0; k < 8; ++k) S[k] = S[k] + (valid ? z[j][k] : 0.0f);
        }
        if (j0 + 8 < 16) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = j0 + 8; i < j0 + 12; ++i)
                row_fetch<D, NORM, ROPE, CONTIG, PERTOK>(a.r, base, rr[i], h, lc, wrow[i], raw[i]);
        }
    }
    // S + S' over lanes l ^ LPR, then l ^ 2 LPR (a symmetric add either way: the same bits as shuffles)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if constexpr (LPR == 16) {
            S[k] = swap32_add(swap16_add(S[k]));
        } else {
            S[k] = S[k] + row_ror<8>(S[k]);
            S[k] = swap16_add(S[k]);
        }
    }
    if (r == 0) {
        float* dst = a.partial + ((b * a.r.H + h) * a.nblk + blk) * D;
        *reinterpret_cast<float4*>(dst + 4 * lc) = make_float4(S[0], S[1], S[2], S[3]);
        *reinterpret_cast<float4*>(dst + D / 2 + 4 * lc) = make_float4(S[4], S[5], S[6], S[7]);
    }
}

// One wave per 64-row block, 4 blocks per workgroup: row 4i + r (i = 0..15) joins
// partial r; the block's sum is (S0 + S1) + (S2 + S3), written to partial (b, h, blk, :).
template <int D, int NORM, int ROPE, bool CONTIG, bool PERTOK>
__global__ __launch_bounds__(256) void k_kmean_partial(KmeanArgs a) {
    constexpr int LPR = D / 8;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, r = lane / LPR;
    const int64_t nbg = (a.nblk + 3) / 4, items = nbg * a.r.B * a.r.H;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int64_t h = item % a.r.H, b = (item / a.r.H) % a.r.B, blk = (item / (a.r.H * a.r.B)) * 4 + w;
    if (blk >= a.nblk) return;  // wave-uniform
    // kRopeSplitPart: each wave's exchange rows, one per row it holds at a step (512 / D rows of D)
    __shared__ __attribute__((aligned(16))) float xch_s[ROPE == kRopeSplitPart ? 4 * 512 : 4];
    float* xch = ROPE == kRopeSplitPart ? xch_s + w * 512 + r * D : xch_s;
    kmean_block<D, NORM, ROPE, CONTIG, PERTOK>(a, b, h, blk, lc, r, xch);
}

// Block sums are added in chunks of 16 consecutive blocks (ascending within a chunk),
// the chunk sums in ascending order, then divided by T. k_kmean_chunks: one thread per
// (b, h, chunk, channel), the chunk's loads in flight together; the sum replaces the
// chunk's first block sum (only this thread reads that chunk's blocks of this channel).
__global__ __launch_bounds__(256) void k_kmean_chunks(KmeanArgs a) {
    constexpr int CB = 16;
    const int D = static_cast<int>(a.r.D), per = 256 / D;
    const int64_t nchunk = (a.nblk + CB - 1) / CB;
    const int64_t chunk = static_cast<int64_t>(blockIdx.x) * per + threadIdx.x / D, bh = blockIdx.y;
    const int c = threadIdx.x % D;
    if (chunk >= nchunk) return;
    float* part = a.partial + (bh * a.nblk + chunk * CB) * D + c;
    const int nb = static_cast<int>(a.nblk - chunk * CB < CB ? a.nblk - chunk * CB : CB);
    float v[CB];
#pragma unroll
    for (int j = 0; j < CB; ++j) v[j] = part[static_cast<int64_t>(j < nb ? j : 0) * D];
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < CB; ++j)
        if (j < nb) s = s + v[j];
    part[0] = s;
}

// One thread per (b, h, channel): the chunk sums in ascending order, 16 loads at a time.
__global__ __launch_bounds__(256) void k_kmean_final(KmeanArgs a) {
    constexpr int CB = 16, NL = 16;
    const int64_t D = a.r.D, i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i >= a.r.B * a.r.H * D) return;
    const int64_t bh = i / D, c = i % D, b = bh / a.r.H, h = bh % a.r.H;
    const int64_t nchunk = (a.nblk + CB - 1) / CB;
    const float* part = a.partial + bh * a.nblk * D + c;
    float tot = 0.0f;
    for (int64_t g = 0; g < nchunk; g += NL) {
        float v[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) v[j] = part[(g + j < nchunk ? g + j : g) * CB * D];
#pragma unroll
        for (int j = 0; j < NL; ++j)
            if (g + j < nchunk) tot = tot + v[j];
    }
    a.mean[b * a.mb + h * a.mh + c] = tot / static_cast<float>(a.r.T);
}

// ---------------------------------------------------------------- A3: fused q/k quantization
// The 32 rows of a wave (8 per lane at D = 128, 4 at D = 64): every load goes out first,
// then each row is finished, centred and scaled (rows past T become 0) into v, and the
// row |v| maxima join their groups' maxima in LDS.
template <int D, int NORM, int ROPE, bool CONTIG, bool PERTOK>
__device__ __forceinline__ void quant_rows(const QuantArgs& a, int64_t b, int64_t h, int64_t tile, int w, int lc,
                                           int lr, uint32_t* amax_s, float* xch, float (*v)[8]) {
    constexpr int LPR = D / 8, RPI = kWave / LPR, IT = 32 / RPI;
    float mu[8] = {0, 0, 0, 0, 0, 0, 0, 0}, wsh[8];
    if (a.mean) load_row_f32<D>(a.mean + b * a.mb + h * a.mh, lc, mu);
    if constexpr (!PERTOK) load_shared_weights<D, NORM>(a.r, h, lc, wsh);
    const GroupMap gmap(a.layout, a.block);
    const RowBase base(a.r, b, tile * 128, h);
    const uint32_t rlast = static_cast<uint32_t>(a.r.T - tile * 128 < 128 ? a.r.T - tile * 128 - 1 : 127);
    uint32_t rr[IT];
    int64_t wrow[IT] = {};
#pragma unroll
    for (int i = 0; i < IT; ++i) rr[i] = min(static_cast<uint32_t>(32 * w + RPI * i + lr), rlast);
    if constexpr (PERTOK) load_wrows<IT>(a.r, base, rr, wrow);
    RowRaw<NORM, ROPE, PERTOK> raw[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) row_fetch<D, NORM, ROPE, CONTIG, PERTOK>(a.r, base, rr[i], h, lc, wrow[i], raw[i]);
    __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the arithmetic
    // rows past T are computed from a clamped row and never enter a group maximum or a store
    float m[IT];
#pragma unroll
    for (int i0 = 0; i0 < IT; i0 += 4) {
        rows4<D, NORM, ROPE, PERTOK>(a.r, raw + i0, wsh, lc, xch, v + i0);
#pragma unroll
        for (int i = i0; i < i0 + 4; ++i) {
            m[i] = 0.0f;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                v[i][k] = (v[i][k] - mu[k]) * a.sm_scale;  // exact when there is no mean (0) or scale (1)
                m[i] = fmaxf(m[i], fabsf(v[i][k]));
            }
            m[i] = row_max<LPR>(m[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int r = 32 * w + RPI * i + lr;
        if (tile * 128 + r < a.r.T && lc == 0) atomicMax(&amax_s[gmap(r)], __float_as_uint(m[i]));
    }
}

template <int D, int NORM, int ROPE, bool CONTIG, bool PERTOK>
__global__ __launch_bounds__(256) void k_quant_qk(QuantArgs a) {
    constexpr int LPR = D / 8, RPI = kWave / LPR, IT = 32 / RPI;
    const int64_t ntile = (a.r.T + 127) / 128, items = ntile * a.r.B * a.r.H;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int64_t h = item % a.r.H, b = (item / a.r.H) % a.r.B, tile = item / (a.r.H * a.r.B);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lc = lane % LPR, lr = lane / LPR;
    __shared__ uint32_t amax_s[32];
    __shared__ float2 scale_s[32];  // (scale, 1 / scale) of the tile's groups
    __shared__ int slow_s;          // a group whose scale is 0 or whose reciprocal overflows
    if (tid < 32) amax_s[tid] = 0u;
    if (tid == 0) slow_s = 0;
    __syncthreads();
    float v[IT][8];
    const int layout = a.layout, block = a.block;
    __shared__ __attribute__((aligned(16))) float xch_s[ROPE == kRopeSplitPart ? 4 * 512 : 4];  // as in k_kmean_partial
    float* xch = ROPE == kRopeSplitPart ? xch_s + w * 512 + lr * D : xch_s;
    quant_rows<D, NORM, ROPE, CONTIG, PERTOK>(a, b, h, tile, w, lc, lr, amax_s, xch, v);
    __syncthreads();
    const int ng = groups_per_tile(layout, block);
    const GroupMap gmap(layout, block);
    if (tid < ng) {
        const float sc = __uint_as_float(amax_s[tid]) / 127.0f + a.scale_eps;
        const float y = 1.0f / sc;
        scale_s[tid] = make_float2(sc, y);
        if (!(sc > 0.0f && y < __builtin_inff())) slow_s = 1;
        const int64_t gi = tile * ng + tid;
        if (gi < a.nscale) a.scales[b * a.ssb + h * a.ssh + gi] = sc;
    }
    __syncthreads();
    const bool fast = slow_s == 0;
    float2 sy[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) sy[i] = scale_s[gmap(32 * w + RPI * i + lr)];
    int8_t* dst0 = a.codes + b * a.ob + tile * 128 * a.ot + h * a.oh + 4 * lc;
    const uint32_t ot = static_cast<uint32_t>(a.ot);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int r = 32 * w + RPI * i + lr;
        const float s = sy[i].x, y = sy[i].y;
        float q[8];
        if (__builtin_expect(fast, 1)) {
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = div_rn(v[i][k], s, y);
        } else {
            // a zero scale (all-zero group with scale_eps = 0) gives codes 0; a reciprocal that
            // overflows takes the plain division
#pragma unroll
            for (int k = 0; k < 8; ++k) q[k] = s > 0.0f ? (y < __builtin_inff() ? div_rn(v[i][k], s, y) : v[i][k] / s) : 0.0f;
        }
        uint32_t word[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = static_cast<int>(q[k] + copysignf(0.5f, q[k]));
            word[k >> 2] |= (static_cast<uint32_t>(c) & 0xffu) << (8 * (k & 3));
        }
        if (tile * 128 + r < a.r.T) {
            int8_t* dst = dst0 + __umul24(static_cast<uint32_t>(r), ot);
            *reinterpret_cast<uint32_t*>(dst) = word[0];
            *reinterpret_cast<uint32_t*>(dst + D / 2) = word[1];
        }
    }
}

// ---------------------------------------------------------------- A4: V to FP8 (channel-major)
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* p, int64_t n, uint32_t value) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = value;
}

// Per-channel |v| maxima of a 256-token chunk of one (b, h): every row load of a wave first
// (rows past T read row T - 1, which leaves a maximum unchanged), the wave's row groups
// reduced by shuffles, the 4 waves in LDS, then one atomic per channel and workgroup.
template <int D>
__global__ __launch_bounds__(256) void k_v_amax(QuantVArgs a) {
    constexpr int LPR = D / 8, RPI = kWave / LPR, IT = 64 / RPI;
    __shared__ float red[4][D];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const uint16_t* base = a.v + b * a.sb + h * a.sh + lc * 8;
    uint4 raw[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        int64_t t = chunk * 256 + w * 64 + RPI * i + lr;
        if (t >= a.T) t = a.T - 1;
        raw[i] = *reinterpret_cast<const uint4*>(base + t * a.st);
    }
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        float x[8];
        unpack_bf16x8(raw[i], x);
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], fabsf(x[k]));
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        if constexpr (LPR == 8) m[k] = fmaxf(m[k], row_ror<8>(m[k]));
        m[k] = swap32_max(swap16_max(m[k]));
    }
    if (lr == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) red[w][lc * 8 + k] = m[k];
    }
    __syncthreads();
    if (tid < D) {
        const float mx = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
        atomicMax(a.amax + (b * a.H + h) * D + tid, __float_as_uint(mx));
    }
}

// One 128-token tile of one (b, h): codes through LDS into channel-major rows.
template <int D>
__global__ __launch_bounds__(256) void k_v_fp8(QuantVArgs a) {
    constexpr int LPR = D / 8, RPI = kWave / LPR, IT = 32 / RPI, LDS_STRIDE = 128 + 16;
    __shared__ uint8_t tileT[D * LDS_STRIDE];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    float vs[8], y[8];
    const uint32_t* am = a.amax + (b * a.H + h) * D + lc * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        vs[k] = fmaxf(__uint_as_float(am[k]) / 448.0f, 1e-8f);
        y[k] = 1.0f / vs[k];
    }
    if (tile == 0 && lr == 0 && w == 0) {
#pragma unroll
        for (int k = 0; k < 8; ++k) a.vs[b * a.vsb + h * a.vsh + lc * 8 + k] = vs[k];
    }
    // every row load first (rows past T read row T - 1; their codes are then zeroed)
    uint4 raw[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        int64_t t = tile * 128 + 32 * w + RPI * i + lr;
        if (t >= a.T) t = a.T - 1;
        raw[i] = *reinterpret_cast<const uint4*>(a.v + b * a.sb + t * a.st + h * a.sh + lc * 8);
    }
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int r = 32 * w + RPI * i + lr;
        const bool valid = tile * 128 + r < a.T;
        uint8_t code[8];
        float x[8];
        unpack_bf16x8(raw[i], x);
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            // the quotient keeps the sign of x (a -0 input gives the -0 code, 0x80)
            float q0 = fminf(fmaxf(copysignf(div_rn(x[k], vs[k], y[k]), x[k]), -448.0f), 448.0f);
            float q1 = fminf(fmaxf(copysignf(div_rn(x[k + 1], vs[k + 1], y[k + 1]), x[k + 1]), -448.0f), 448.0f);
            const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
            code[k] = valid ? static_cast<uint8_t>(pk & 0xff) : 0;
            code[k + 1] = valid ? static_cast<uint8_t>((pk >> 8) & 0xff) : 0;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) tileT[(lc * 8 + k) * LDS_STRIDE + r] = code[k];
    }
    __syncthreads();
    // D rows of 128 bytes: 8 chunks of 16 bytes per row
    for (int j = tid; j < D * 8; j += 256) {
        const int c = j >> 3, part = (j & 7) * 16;
        const int64_t t0 = tile * 128 + part;
        if (t0 >= a.od) continue;
        const uint4 val = *reinterpret_cast<const uint4*>(&tileT[c * LDS_STRIDE + part]);
        *reinterpret_cast<uint4*>(a.codes + b * a.ob + h * a.oh + c * a.od + t0) = val;
    }
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

inline int check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return SQ_OK;
}

template <int D, int NORM, int ROPE, bool PERTOK>
void launch_quant_w(const QuantArgs& a, dim3 grid, hipStream_t s) {
    if (a.r.rope_contig) SQ_LAUNCH((k_quant_qk<D, NORM, ROPE, true, PERTOK>), grid, dim3(256), 0, s, a);
    else SQ_LAUNCH((k_quant_qk<D, NORM, ROPE, false, PERTOK>), grid, dim3(256), 0, s, a);
}

// per-token weight rows only matter with a norm
template <int D, int NORM, int ROPE>
void launch_quant_c(const QuantArgs& a, dim3 grid, hipStream_t s) {
    if (NORM != SQ_NORM_NONE && a.r.wrows) launch_quant_w<D, NORM, ROPE, NORM != SQ_NORM_NONE>(a, grid, s);
    else launch_quant_w<D, NORM, ROPE, false>(a, grid, s);
}

template <int D, int NORM>
void launch_quant_rope(const QuantArgs& a, dim3 grid, hipStream_t s) {
    switch (a.r.rope) {
    case SQ_ROPE_NONE: launch_quant_c<D, NORM, SQ_ROPE_NONE>(a, grid, s); break;
    case SQ_ROPE_SPLIT_HALF: launch_quant_c<D, NORM, SQ_ROPE_SPLIT_HALF>(a, grid, s); break;
    case kRopeSplitPart: launch_quant_c<D, NORM, kRopeSplitPart>(a, grid, s); break;
    default: launch_quant_c<D, NORM, SQ_ROPE_INTERLEAVED>(a, grid, s); break;
    }
}

template <int D>
void launch_quant_d(const QuantArgs& a, dim3 grid, hipStream_t s) {
    switch (a.r.norm) {
    case SQ_NORM_NONE: launch_quant_rope<D, SQ_NORM_NONE>(a, grid, s); break;
    case SQ_NORM_HEAD: launch_quant_rope<D, SQ_NORM_HEAD>(a, grid, s); break;
    default: launch_quant_rope<D, SQ_NORM_ALL_HEADS>(a, grid, s); break;
    }
}

template <int D, int NORM, int ROPE, bool PERTOK>
void launch_kmean_w(const KmeanArgs& a, dim3 grid, hipStream_t s) {
    if (a.r.rope_contig) SQ_LAUNCH((k_kmean_partial<D, NORM, ROPE, true, PERTOK>), grid, dim3(256), 0, s, a);
    else SQ_LAUNCH((k_kmean_partial<D, NORM, ROPE, false, PERTOK>), grid, dim3(256), 0, s, a);
}

template <int D, int NORM, int ROPE>
void launch_kmean_c(const KmeanArgs& a, dim3 grid, hipStream_t s) {
    if (NORM != SQ_NORM_NONE && a.r.wrows) launch_kmean_w<D, NORM, ROPE, NORM != SQ_NORM_NONE>(a, grid, s);
    else launch_kmean_w<D, NORM, ROPE, false>(a, grid, s);
}

template <int D, int NORM>
void launch_kmean_rope(const KmeanArgs& a, dim3 grid, hipStream_t s) {
    switch (a.r.rope) {
    case SQ_ROPE_NONE: launch_kmean_c<D, NORM, SQ_ROPE_NONE>(a, grid, s); break;
    case SQ_ROPE_SPLIT_HALF: launch_kmean_c<D, NORM, SQ_ROPE_SPLIT_HALF>(a, grid, s); break;
    case kRopeSplitPart: launch_kmean_c<D, NORM, kRopeSplitPart>(a, grid, s); break;
    default: launch_kmean_c<D, NORM, SQ_ROPE_INTERLEAVED>(a, grid, s); break;
    }
}

template <int D>
void launch_kmean_d(const KmeanArgs& a, dim3 grid, hipStream_t s) {
    switch (a.r.norm) {
    case SQ_NORM_NONE: launch_kmean_rope<D, SQ_NORM_NONE>(a, grid, s); break;
    case SQ_NORM_HEAD: launch_kmean_rope<D, SQ_NORM_HEAD>(a, grid, s); break;
    default: launch_kmean_rope<D, SQ_NORM_ALL_HEADS>(a, grid, s); break;
    }
}

}  // namespace

int launch_norm_stats(const NormStatsArgs& a, void* stream) {
    const int64_t tokens = a.B * a.T;
    if (tokens == 0) return SQ_OK;
    dim3 grid(static_cast<unsigned>((tokens + 3) / 4));
    if (a.D == 128) SQ_LAUNCH(k_norm_stats<128>, grid, dim3(256), 0, S(stream), a);
    else SQ_LAUNCH(k_norm_stats<64>, grid, dim3(256), 0, S(stream), a);
    return check_launch("sq_norm_stats");
}

int launch_kmean(const KmeanArgs& a, void* stream) {
    if (a.r.B * a.r.H * a.r.D == 0) return SQ_OK;
    const int64_t items = (a.nblk + 3) / 4 * a.r.B * a.r.H;
    dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
    if (a.nblk > 0) {
        if (a.r.D == 128) launch_kmean_d<128>(a, grid, S(stream));
        else launch_kmean_d<64>(a, grid, S(stream));
    }
    const int64_t nchunk = (a.nblk + 15) / 16, per = 256 / a.r.D;
    if (a.nblk > 0)
        SQ_LAUNCH(k_kmean_chunks, dim3(static_cast<unsigned>((nchunk + per - 1) / per), static_cast<unsigned>(a.r.B * a.r.H)),
                           dim3(256), 0, S(stream), a);
    SQ_LAUNCH(k_kmean_final, dim3(static_cast<unsigned>((a.r.B * a.r.H * a.r.D + 255) / 256)), dim3(256), 0,
                       S(stream), a);
    return check_launch("sq_kmean");
}

int launch_quant_qk(const QuantArgs& a, void* stream) {
    if (a.r.B * a.r.T * a.r.H == 0) return SQ_OK;
    const int64_t items = (a.r.T + 127) / 128 * a.r.B * a.r.H;
    dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
    if (a.r.D == 128) launch_quant_d<128>(a, grid, S(stream));
    else launch_quant_d<64>(a, grid, S(stream));
    return check_launch("sq_quant_qk");
}

int launch_quant_v_fp8(const QuantVArgs& a, void* stream) {
    if (a.B * a.H == 0) return SQ_OK;
    const int64_t n = a.B * a.H * a.D;
    SQ_LAUNCH(k_fill_u32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, S(stream), a.amax, n, 0u);
    if (a.T > 0) {
        dim3 g1(static_cast<unsigned>((a.T + 255) / 256), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
        if (a.D == 128) SQ_LAUNCH(k_v_amax<128>, g1, dim3(256), 0, S(stream), a);
        else SQ_LAUNCH(k_v_amax<64>, g1, dim3(256), 0, S(stream), a);
    }
    dim3 g2(static_cast<unsigned>((a.od + 127) / 128), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    if (a.D == 128) SQ_LAUNCH(k_v_fp8<128>, g2, dim3(256), 0, S(stream), a);
    else SQ_LAUNCH(k_v_fp8<64>, g2, dim3(256), 0, S(stream), a);
    return check_launch("sq_quant_v_fp8");
}

}  // namespace sq
