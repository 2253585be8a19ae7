// q8 paged-cache writer on gfx950: new K/V rows quantized to q8 and scattered into the
// paged cache by a slot mapping.
//
// Method: [kit] WanGP shared/attention_kit.py quantize_q8 (int8 per token, head and
// group of 32 channels, FP32 scale max(amax / 127, 1e-8) kept as FP16, codes
// round-half-even of x / scale clamped to +-127) and [impl] fastkernels L2/attention_impl.py
// _store_kvcache_nhd (slot -> cache block slot / block_size, row slot % block_size; a
// negative slot skips the token; NHD rows of Hk * D per slot).
//
// A row (token, head) of D channels is D/8 lanes, 8 consecutive channels per lane, so a
// 32-channel group is 4 adjacent lanes and its |x| maximum two DPP steps. Every row of a
// wave's four steps is loaded before any arithmetic (row indices clamped, results of rows
// past the end dropped), the slot of each row included. HBM-bound: per row 2 D (bf16) or
// 4 D (FP32) bytes read, D code bytes and D/16 scale bytes written.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

constexpr int kSteps = 4;

// max over the 4 lanes of a quad (xor 1, then xor 2 by DPP quad permutations)
__device__ __forceinline__ float quad_max(float m) {
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xf, 0xf, false)));  // [1,0,3,2]
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xf, 0xf, false)));  // [2,3,0,1]
    return m;
}

template <int D, bool F32>
__global__ __launch_bounds__(256) void k_q8_cache_write(CacheWriteArgs a) {
    constexpr int LPR = D / 8, RPW = kWave / LPR;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane % LPR, lr = lane / LPR;
    const int64_t rows_half = a.n * a.Hk, rows = 2 * rows_half;   // K rows, then V rows
    const int64_t r0 = (static_cast<int64_t>(blockIdx.x) * 4 + w) * (kSteps * RPW);
    if (r0 >= rows) return;  // wave-uniform

    // ---- every load of the wave's rows first: the rows and their tokens' slots
    int64_t slot[kSteps];
    uint32_t raw[kSteps][F32 ? 8 : 4];
    int tok[kSteps], head[kSteps];
    bool isv[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        int64_t r = r0 + s * RPW + lr;
        if (r >= rows) r = rows - 1;
        isv[s] = r >= rows_half;
        const int64_t rr = isv[s] ? r - rows_half : r;
        tok[s] = static_cast<int>(rr / a.Hk);
        head[s] = static_cast<int>(rr % a.Hk);
        slot[s] = a.slots[tok[s]];
        const int64_t off = isv[s] ? tok[s] * a.vn + head[s] * a.vh : tok[s] * a.kn + head[s] * a.kh;
        if constexpr (F32) {
            const float* src = static_cast<const float*>(isv[s] ? a.v : a.k) + off + 8 * lc;
            const uint4 u0 = *reinterpret_cast<const uint4*>(src), u1 = *reinterpret_cast<const uint4*>(src + 4);
            raw[s][0] = u0.x; raw[s][1] = u0.y; raw[s][2] = u0.z; raw[s][3] = u0.w;
            raw[s][4] = u1.x; raw[s][5] = u1.y; raw[s][6] = u1.z; raw[s][7] = u1.w;
        } else {
            const uint16_t* src = static_cast<const uint16_t*>(isv[s] ? a.v : a.k) + off + 8 * lc;
            const uint4 u = *reinterpret_cast<const uint4*>(src);
            raw[s][0] = u.x; raw[s][1] = u.y; raw[s][2] = u.z; raw[s][3] = u.w;
        }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the arithmetic

#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        float x[8];
        if constexpr (F32) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(raw[s][e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) { x[2 * e] = bf16_lo(raw[s][e]); x[2 * e + 1] = bf16_hi(raw[s][e]); }
        }
        float m = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
        m = quad_max(m);                                   // the group's |x| maximum (4 lanes)
        const float sc = fmaxf(m / 127.0f, 1e-8f);
        const float y = 1.0f / sc;                         // RN(1 / sc): sc >= 1e-8 keeps it finite
        uint32_t word[2] = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float q = fminf(fmaxf(__builtin_rintf(div_rn(x[e], sc, y)), -127.0f), 127.0f);
            word[e >> 2] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xffu) << (8 * (e & 3));
        }
        const int64_t r = r0 + s * RPW + lr;
        if (r < rows && slot[s] >= 0 && slot[s] < a.nslots) {
            const int64_t row = slot[s] * a.Hk + head[s];   // (block, row in block) flattened, then head
            int8_t* dst = (isv[s] ? a.vc : a.kc) + row * D + 8 * lc;
            *reinterpret_cast<uint2*>(dst) = make_uint2(word[0], word[1]);
            if ((lc & 3) == 0) {
                uint16_t* sd = (isv[s] ? a.vs : a.ks) + row * (D / 32) + (lc >> 2);
                *sd = __builtin_bit_cast(uint16_t, static_cast<_Float16>(sc));
            }
        }
    }
}

}  // namespace

int launch_cache_write(const CacheWriteArgs& a, bool f32, void* stream) {
    const int64_t rows = 2 * a.n * a.Hk;
    if (rows == 0) return SQ_OK;
    const int64_t per_wg = 4 * kSteps * (kWave / (a.D / 8));
    dim3 grid(static_cast<unsigned>((rows + per_wg - 1) / per_wg));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 128) {
        if (f32) SQ_LAUNCH((k_q8_cache_write<128, true>), grid, dim3(256), 0, s, a);
        else SQ_LAUNCH((k_q8_cache_write<128, false>), grid, dim3(256), 0, s, a);
    } else {
        if (f32) SQ_LAUNCH((k_q8_cache_write<64, true>), grid, dim3(256), 0, s, a);
        else SQ_LAUNCH((k_q8_cache_write<64, false>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_q8_cache_write: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
