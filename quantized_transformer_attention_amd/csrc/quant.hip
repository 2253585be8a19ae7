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
#pragma unroll
    for (int off = LPR / 2; off >= 1; off >>= 1) p = p + shfl_xor(p, off);
    return p;
}

// cos and sin of pairs p0 .. p0 + 3 of a table row
template <bool CONTIG>
__device__ __forceinline__ void load_pairs4(const float* tb, const RowArgs& a, int64_t p0, float* cs, float* sn) {
    if constexpr (CONTIG) {
        const float4 u = *reinterpret_cast<const float4*>(tb + 2 * p0);
        const float4 v = *reinterpret_cast<const float4*>(tb + 2 * p0 + 4);
        cs[0] = u.x; sn[0] = u.y; cs[1] = u.z; sn[1] = u.w;
        cs[2] = v.x; sn[2] = v.y; cs[3] = v.z; sn[3] = v.w;
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            cs[k] = tb[a.rp * (p0 + k)];
            sn[k] = tb[a.rp * (p0 + k) + a.rc];
        }
    }
}

// Row prologue [quant] _rows: z = rotate(bf16(norm(x) * w)) for the 8 channels a lane
// holds of row (b, t, h). Every lane of the row must call it (the norm's butterfly);
// rows with valid == false read nothing and their result is unspecified.
// ROPE_SPLIT_HALF here rotates all D/2 pairs (the entry point checks pairs == D/2).
template <int D, int NORM, int ROPE, bool CONTIG>
__device__ __forceinline__ void row_prologue(const RowArgs& a, int64_t b, int64_t t, int64_t h, int lc, bool valid,
                                             float* z) {
    constexpr int LPR = D / 8;
    float x[8], y[8];
    if (valid) load_row_bf16<D>(a.x + b * a.sb + t * a.st + h * a.sh, lc, x);
    else {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = 0.0f;
    }
    if constexpr (NORM == SQ_NORM_NONE) {
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = x[k];
    } else {
        float ms;
        if constexpr (NORM == SQ_NORM_HEAD) {
            ms = row_sumsq<LPR>(x) / static_cast<float>(D);
        } else {
            ms = valid ? a.ms[b * a.msb + t * a.mst] : 1.0f;
        }
        const float inv = 1.0f / sqrtf(ms + a.eps);
        const int64_t wrow = (a.wrows && valid) ? a.wrows[t] : 0;
        float w[8];
        load_row_bf16<D>(a.w + wrow * a.wd + (NORM == SQ_NORM_ALL_HEADS ? h * D : 0), lc, w);
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = bf16_round((x[k] * inv) * w[k]);
    }
    if constexpr (ROPE == SQ_ROPE_NONE) {
#pragma unroll
        for (int k = 0; k < 8; ++k) z[k] = y[k];
    } else if constexpr (ROPE == SQ_ROPE_SPLIT_HALF) {
        // channel 4 lc + k (leading) with its partner D/2 + 4 lc + k (trailing), pair 4 lc + k
        float cs[4], sn[4];
        if (valid) load_pairs4<CONTIG>(a.table + a.rb * b + a.rs * t, a, 4 * lc, cs, sn);
        else {
#pragma unroll
            for (int k = 0; k < 4; ++k) { cs[k] = 1.0f; sn[k] = 0.0f; }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            z[k] = __builtin_fmaf(cs[k], y[k], (-sn[k]) * y[4 + k]);
            z[4 + k] = __builtin_fmaf(sn[k], y[k], cs[k] * y[4 + k]);
        }
    } else {  // interleaved: channel 2p with 2p + 1; pairs 2 lc, 2 lc + 1 and D/4 + 2 lc, D/4 + 2 lc + 1
        const float* tb = a.table + a.rb * b + a.rs * t;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t pair = (u < 2 ? 0 : D / 4) + 2 * lc + (u & 1);
            const int k = 2 * u;
            if (valid && pair < a.pairs) {
                const float cs = tb[a.rp * pair], sn = tb[a.rp * pair + a.rc];
                z[k] = __builtin_fmaf(cs, y[k], (-sn) * y[k + 1]);
                z[k + 1] = __builtin_fmaf(sn, y[k], cs * y[k + 1]);
            } else {
                z[k] = y[k];
                z[k + 1] = y[k + 1];
            }
        }
    }
}

__device__ __forceinline__ int local_group(int r, int layout, int block) {
    switch (layout) {
    case SQ_LAYOUT_THREAD_Q: return 8 * (r >> 5) + (r & 7);
    case SQ_LAYOUT_THREAD_K: return 4 * (r >> 6) + ((r & 7) >> 1);
    case SQ_LAYOUT_WARP_Q: return r >> 5;
    default: return r / block;
    }
}

__host__ __device__ __forceinline__ int groups_per_tile(int layout, int block) {
    switch (layout) {
    case SQ_LAYOUT_THREAD_Q: return 32;
    case SQ_LAYOUT_THREAD_K: return 8;
    case SQ_LAYOUT_WARP_Q: return 4;
    default: return 128 / block;
    }
}

// ---------------------------------------------------------------- A1: mean squares over all heads
template <int D>
__global__ __launch_bounds__(256) void k_norm_stats(NormStatsArgs a) {
    constexpr int LPR = D / 8, HPI = kWave / LPR;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t tok = static_cast<int64_t>(blockIdx.x) * 4 + w;
    if (tok >= a.B * a.T) return;  // wave-uniform
    const int64_t b = tok / a.T, t = tok % a.T;
    float tot = 0.0f;
    for (int64_t h0 = 0; h0 < a.H; h0 += HPI) {
        const int64_t h = h0 + lr;
        float x[8];
        if (h < a.H) load_row_bf16<D>(a.x + b * a.sb + t * a.st + h * a.sh, lc, x);
        else {
#pragma unroll
            for (int k = 0; k < 8; ++k) x[k] = 0.0f;
        }
        const float p = row_sumsq<LPR>(x);
#pragma unroll
        for (int j = 0; j < HPI; ++j) {
            const float s = __shfl(p, j * LPR, kWave);
            if (h0 + j < a.H) tot = tot + s;
        }
    }
    if (lane == 0) a.ms[b * a.msb + t * a.mst] = tot / static_cast<float>(a.H * D);
}

// ---------------------------------------------------------------- A2: k mean
// One wave per 64-row block, 4 blocks per workgroup: row 4i + r (i = 0..15) joins
// partial r; the block's sum is (S0 + S1) + (S2 + S3), written to partial (b, h, blk, :).
template <int D, int NORM, int ROPE, bool CONTIG>
__global__ __launch_bounds__(256) void k_kmean_partial(KmeanArgs a) {
    constexpr int LPR = D / 8;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, r = lane / LPR;
    const int64_t nbg = (a.nblk + 3) / 4, items = nbg * a.r.B * a.r.H;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int64_t h = item % a.r.H, b = (item / a.r.H) % a.r.B, blk = (item / (a.r.H * a.r.B)) * 4 + w;
    if (blk >= a.nblk) return;  // wave-uniform
    const bool active = r < 4;
    float S[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < 16; ++i) {
        const int64_t t = blk * 64 + 4 * i + r;
        const bool valid = active && t < a.r.T;
        float z[8];
        row_prologue<D, NORM, ROPE, CONTIG>(a.r, b, t, h, lc, valid, z);
#pragma unroll
        for (int k = 0; k < 8; ++k) S[k] = S[k] + (valid ? z[k] : 0.0f);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) S[k] = S[k] + shfl_xor(S[k], LPR);
#pragma unroll
    for (int k = 0; k < 8; ++k) S[k] = S[k] + shfl_xor(S[k], 2 * LPR);
    if (r == 0) {
        float* dst = a.partial + ((b * a.r.H + h) * a.nblk + blk) * D;
        *reinterpret_cast<float4*>(dst + 4 * lc) = make_float4(S[0], S[1], S[2], S[3]);
        *reinterpret_cast<float4*>(dst + D / 2 + 4 * lc) = make_float4(S[4], S[5], S[6], S[7]);
    }
}

// One workgroup per (b, h): block sums are added in chunks of 16 consecutive blocks
// (ascending within a chunk), the chunk sums in ascending order, then divided by T.
// The chunks of a group of 32 are summed in parallel, their sums kept in LDS.
__global__ __launch_bounds__(256) void k_kmean_final(KmeanArgs a) {
    constexpr int CG = 32, CB = 16;
    __shared__ float cs[CG * 128];
    const int64_t D = a.r.D, bh = blockIdx.x, b = bh / a.r.H, h = bh % a.r.H;
    const int tid = threadIdx.x, c = tid % D, r = tid / D, rpw = 256 / D;
    const float* part = a.partial + bh * a.nblk * D;
    const int64_t nchunk = (a.nblk + CB - 1) / CB;
    float tot = 0.0f;
    for (int64_t g0 = 0; g0 < nchunk; g0 += CG) {
        const int ng = static_cast<int>(nchunk - g0 < CG ? nchunk - g0 : CG);
        for (int j = r; j < ng; j += rpw) {
            const int64_t blk0 = (g0 + j) * CB, blk1 = blk0 + CB < a.nblk ? blk0 + CB : a.nblk;
            float s = 0.0f;
            for (int64_t blk = blk0; blk < blk1; ++blk) s = s + part[blk * D + c];
            cs[j * D + c] = s;
        }
        __syncthreads();
        if (tid < D)
            for (int j = 0; j < ng; ++j) tot = tot + cs[j * D + c];
        __syncthreads();
    }
    if (tid < D) a.mean[b * a.mb + h * a.mh + c] = tot / static_cast<float>(a.r.T);
}

// ---------------------------------------------------------------- A3: fused q/k quantization
template <int D, int NORM, int ROPE, bool CONTIG>
__global__ __launch_bounds__(256) void k_quant_qk(QuantArgs a) {
    constexpr int LPR = D / 8, RPI = kWave / LPR, IT = 32 / RPI;
    const int64_t ntile = (a.r.T + 127) / 128, items = ntile * a.r.B * a.r.H;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int64_t h = item % a.r.H, b = (item / a.r.H) % a.r.B, tile = item / (a.r.H * a.r.B);
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lc = lane % LPR, lr = lane / LPR;
    __shared__ uint32_t amax_s[32];
    __shared__ float scale_s[32];
    if (tid < 32) amax_s[tid] = 0u;
    __syncthreads();
    const int layout = a.layout, block = a.block;
    const bool has_mean = a.mean != nullptr, has_scale = a.sm_scale != 1.0f;
    float mu[8];
    if (has_mean) load_row_f32<D>(a.mean + b * a.mb + h * a.mh, lc, mu);
    float v[IT][8];
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int r = 32 * w + RPI * i + lr;
        const int64_t t = tile * 128 + r;
        const bool valid = t < a.r.T;
        row_prologue<D, NORM, ROPE, CONTIG>(a.r, b, t, h, lc, valid, v[i]);
        float m = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float z = v[i][k];
            if (has_mean) z = z - mu[k];
            if (has_scale) z = z * a.sm_scale;
            v[i][k] = valid ? z : 0.0f;
            m = fmaxf(m, fabsf(v[i][k]));
        }
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) m = fmaxf(m, shfl_xor(m, off));
        if (valid && lc == 0) atomicMax(&amax_s[local_group(r, layout, block)], __float_as_uint(m));
    }
    __syncthreads();
    const int ng = groups_per_tile(layout, block);
    if (tid < ng) {
        const float sc = __uint_as_float(amax_s[tid]) / 127.0f + a.scale_eps;
        scale_s[tid] = sc;
        const int64_t gi = tile * ng + tid;
        if (gi < a.nscale) a.scales[b * a.ssb + h * a.ssh + gi] = sc;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int r = 32 * w + RPI * i + lr;
        const int64_t t = tile * 128 + r;
        const float s = scale_s[local_group(r, layout, block)];
        const float y = 1.0f / s;
        float q[8];
        if (__builtin_expect(__all(s > 0.0f && y < __builtin_inff()), 1)) {
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
        if (t < a.r.T) {
            int8_t* dst = a.codes + b * a.ob + t * a.ot + h * a.oh;
            *reinterpret_cast<uint32_t*>(dst + 4 * lc) = word[0];
            *reinterpret_cast<uint32_t*>(dst + D / 2 + 4 * lc) = word[1];
        }
    }
}

// ---------------------------------------------------------------- A4: V to FP8 (channel-major)
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* p, int64_t n, uint32_t value) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    if (i < n) p[i] = value;
}

template <int D>
__global__ __launch_bounds__(256) void k_v_amax(QuantVArgs a) {
    constexpr int LPR = D / 8, RPI = kWave / LPR;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < 64 / RPI; ++i) {
        const int64_t t = chunk * 256 + w * 64 + RPI * i + lr;
        if (t >= a.T) break;
        float x[8];
        unpack_bf16x8(*reinterpret_cast<const uint4*>(a.v + b * a.sb + t * a.st + h * a.sh + lc * 8), x);
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], fabsf(x[k]));
    }
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
        for (int k = 0; k < 8; ++k) m[k] = fmaxf(m[k], shfl_xor(m[k], off));
    if (lr == 0) {
        uint32_t* dst = a.amax + (b * a.H + h) * D + lc * 8;
#pragma unroll
        for (int k = 0; k < 8; ++k) atomicMax(dst + k, __float_as_uint(m[k]));
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
#pragma unroll
    for (int i = 0; i < IT; ++i) {
        const int r = 32 * w + RPI * i + lr;
        const int64_t t = tile * 128 + r;
        uint8_t code[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (t < a.T) {
            float x[8];
            unpack_bf16x8(*reinterpret_cast<const uint4*>(a.v + b * a.sb + t * a.st + h * a.sh + lc * 8), x);
#pragma unroll
            for (int k = 0; k < 8; k += 2) {
                // the quotient keeps the sign of x (a -0 input gives the -0 code, 0x80)
                float q0 = fminf(fmaxf(copysignf(div_rn(x[k], vs[k], y[k]), x[k]), -448.0f), 448.0f);
                float q1 = fminf(fmaxf(copysignf(div_rn(x[k + 1], vs[k + 1], y[k + 1]), x[k + 1]), -448.0f), 448.0f);
                const int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
                code[k] = static_cast<uint8_t>(pk & 0xff);
                code[k + 1] = static_cast<uint8_t>((pk >> 8) & 0xff);
            }
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

template <int D, int NORM, int ROPE>
void launch_quant_c(const QuantArgs& a, dim3 grid, hipStream_t s) {
    if (a.r.rope_contig) hipLaunchKernelGGL((k_quant_qk<D, NORM, ROPE, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_quant_qk<D, NORM, ROPE, false>), grid, dim3(256), 0, s, a);
}

template <int D, int NORM>
void launch_quant_rope(const QuantArgs& a, dim3 grid, hipStream_t s) {
    switch (a.r.rope) {
    case SQ_ROPE_NONE: launch_quant_c<D, NORM, SQ_ROPE_NONE>(a, grid, s); break;
    case SQ_ROPE_SPLIT_HALF: launch_quant_c<D, NORM, SQ_ROPE_SPLIT_HALF>(a, grid, s); break;
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

template <int D, int NORM, int ROPE>
void launch_kmean_c(const KmeanArgs& a, dim3 grid, hipStream_t s) {
    if (a.r.rope_contig) hipLaunchKernelGGL((k_kmean_partial<D, NORM, ROPE, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_kmean_partial<D, NORM, ROPE, false>), grid, dim3(256), 0, s, a);
}

template <int D, int NORM>
void launch_kmean_rope(const KmeanArgs& a, dim3 grid, hipStream_t s) {
    switch (a.r.rope) {
    case SQ_ROPE_NONE: launch_kmean_c<D, NORM, SQ_ROPE_NONE>(a, grid, s); break;
    case SQ_ROPE_SPLIT_HALF: launch_kmean_c<D, NORM, SQ_ROPE_SPLIT_HALF>(a, grid, s); break;
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
    if (a.D == 128) hipLaunchKernelGGL(k_norm_stats<128>, grid, dim3(256), 0, S(stream), a);
    else hipLaunchKernelGGL(k_norm_stats<64>, grid, dim3(256), 0, S(stream), a);
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
    hipLaunchKernelGGL(k_kmean_final, dim3(static_cast<unsigned>(a.r.B * a.r.H)), dim3(256), 0, S(stream), a);
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
    hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, S(stream), a.amax, n, 0u);
    if (a.T > 0) {
        dim3 g1(static_cast<unsigned>((a.T + 255) / 256), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
        if (a.D == 128) hipLaunchKernelGGL(k_v_amax<128>, g1, dim3(256), 0, S(stream), a);
        else hipLaunchKernelGGL(k_v_amax<64>, g1, dim3(256), 0, S(stream), a);
    }
    dim3 g2(static_cast<unsigned>((a.od + 127) / 128), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    if (a.D == 128) hipLaunchKernelGGL(k_v_fp8<128>, g2, dim3(256), 0, S(stream), a);
    else hipLaunchKernelGGL(k_v_fp8<64>, g2, dim3(256), 0, S(stream), a);
    return check_launch("sq_quant_v_fp8");
}

}  // namespace sq
