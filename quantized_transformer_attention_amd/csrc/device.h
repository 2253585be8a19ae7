// Device helpers shared by the libsq kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/sq.h"
#include "sq_internal.h"

namespace sq {

constexpr int kWave = 64;

// Every kernel launch of the library: with SQ_TRACE set in the environment (not "0") it is first
// logged to stderr (kernel, grid, block, stream), then enqueued.
#define SQ_LAUNCH(K, G, B, SH, S, ...)                                                                       \
    do {                                                                                                     \
        const dim3 sq_g_ = (G), sq_b_ = (B);                                                                 \
        if (::sq::trace_enabled()) ::sq::trace_launch(#K, sq_g_.x, sq_g_.y, sq_g_.z, sq_b_.x, (SH), (S));    \
        hipLaunchKernelGGL(K, sq_g_, sq_b_, SH, S, __VA_ARGS__);                                              \
    } while (0)

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 8 bf16 (one 16-byte load) -> 8 floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
    f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
    f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// 8 f16 (one 16-byte load) -> 8 floats (exact).
__device__ __forceinline__ void unpack_f16x8(const uint4& u, float* f) {
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const h2_t h = __builtin_bit_cast(h2_t, w[i]);
        f[2 * i] = static_cast<float>(h[0]);
        f[2 * i + 1] = static_cast<float>(h[1]);
    }
}

// Stores element idx of an output tensor: FP32, or bfloat16 rounded to nearest even when bf16
// (idx counts elements of the stored type).
__device__ __forceinline__ void store_out(float* out, int64_t idx, float v, bool bf16) {
    if (bf16) reinterpret_cast<__bf16*>(out)[idx] = static_cast<__bf16>(v);
    else out[idx] = v;
}

// Round to bfloat16, nearest even (v_cvt_pk_bf16_f32), back to float.
__device__ __forceinline__ float bf16_round(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

// Both of a and b rounded to bf16 (nearest even) by one paired conversion.
__device__ __forceinline__ void bf16_round2(float& a, float& b) {
    typedef float f2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
    const uint32_t u = __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t){a, b}, b2_t));
    a = __uint_as_float(u << 16);
    b = __uint_as_float(u & 0xffff0000u);
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Correctly rounded v / s given y = RN(1 / s): q = RN(v y), r = v - q s exactly (fma),
// q' = RN(q + r y). By Markstein's theorem q' = RN(v / s) when y is the correctly rounded
// reciprocal and nothing overflows or underflows.
__device__ __forceinline__ float div_rn(float v, float s, float y) {
    float q = v * y;
    float r = __builtin_fmaf(-q, s, v);
    return __builtin_fmaf(r, y, q);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Scale index of token t in a row-group layout [quant] module docstring.
__device__ __forceinline__ int64_t scale_idx(int64_t t, int layout, int block) {
    switch (layout) {
    case SQ_LAYOUT_THREAD_Q: return 8 * (t >> 5) + (t & 7);
    case SQ_LAYOUT_THREAD_K: return 4 * (t >> 6) + ((t & 7) >> 1);
    case SQ_LAYOUT_WARP_Q: return 4 * (t >> 7) + ((t & 127) >> 5);
    default: return t / block;
    }
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

// LDS tiles are rows of 16-byte slots; slot s of row r is stored at slot s ^ f(r) so that
// the rows one MFMA operand read touches (consecutive rows, one slot each) land in
// distinct bank groups, whether the LDS serves 8 or 16 such lanes per cycle:
//   8 slots per row (128 B):  f(r) = (r & 7) ^ ((r >> 3) & 1)
//   4 slots per row (64 B):   f(r) = (r >> 1) & 3
//   16 slots per row (256 B): f(r) = r & 15
// Lane (l + n) mod 16 of lane l's 16-lane row (DPP row rotate).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + N, 0xf, 0xf, true));
}

// v op v' with v' the value of lane l ^ 16 (v_permlane16_swap) or l ^ 32 (v_permlane32_swap): the swap
// hands each lane the pair (v_l, v_l') in one order or the other, and op is symmetric, so every lane
// gets the same bits as with an LDS shuffle, without one.
__device__ __forceinline__ float swap16_max(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float swap32_max(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float swap16_add(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float swap32_add(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Reductions over a row of LPR lanes (LPR in {8, 16}); every lane of the row gets the
// result. The sum adds partners at lane offsets LPR/2, .., 2, 1 in that order: rotating a
// 16-lane row by 8, 4, 2, 1 pairs each lane with the same values as xor offsets 8, 4, 2, 1
// (after a step the row repeats with that period), so both give the same bits.
template <int LPR>
__device__ __forceinline__ float row_sum(float p) {
    if constexpr (LPR == 16) {
        p = p + row_ror<8>(p);
        p = p + row_ror<4>(p);
        p = p + row_ror<2>(p);
        p = p + row_ror<1>(p);
    } else {
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) p = p + __shfl_xor(p, off, kWave);
    }
    return p;
}

// Maximum of non-negative, non-NaN values (compared as their bit patterns, which order
// such floats; 0 is then the identity that lets the rotation fold into the max).
template <int LPR>
__device__ __forceinline__ float row_max(float m) {
    if constexpr (LPR == 16) {
        uint32_t u = __float_as_uint(m);
        u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x128, 0xf, 0xf, true)));
        u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x124, 0xf, 0xf, true)));
        u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x122, 0xf, 0xf, true)));
        u = max(u, static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(u), 0x121, 0xf, 0xf, true)));
        m = __uint_as_float(u);
    } else {
#pragma unroll
        for (int off = LPR / 2; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    }
    return m;
}

// Lane J of this lane's LPR-lane row (a swizzle inside the 32-lane half; rows are aligned).
template <int LPR, int J>
__device__ __forceinline__ float row_lane(float v) {
    constexpr int pattern = (0x1f & ~(LPR - 1)) | (J << 5);
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), pattern));
}

// Maximum over the 64 lanes of a wave (every lane gets it): DPP row rotations by 8, 4, 2, 1, then the
// lane swaps across rows and halves.
__device__ __forceinline__ float wave_max(float m) {
    m = fmaxf(m, row_ror<8>(m));
    m = fmaxf(m, row_ror<4>(m));
    m = fmaxf(m, row_ror<2>(m));
    m = fmaxf(m, row_ror<1>(m));
    return swap32_max(swap16_max(m));
}

template <int NS>
__device__ __forceinline__ int swz(int row, int slot) {
    if constexpr (NS == 8) return slot ^ ((row & 7) ^ ((row >> 3) & 1));
    else if constexpr (NS == 4) return slot ^ ((row >> 1) & 3);
    else return slot ^ (row & 15);
}

// 8 int8 (byte k = element k) -> 8 f16, exact: byte b ^ 0x80 = b + 128 goes under the f16
// exponent byte 0x64 (f16 0x64uu = 1024 + uu), then 1152 comes off in packed f16
typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8h_t i8x8_to_f16(uint32_t w0, uint32_t w1) {
    const uint32_t u0 = w0 ^ 0x80808080u, u1 = w1 ^ 0x80808080u;
    const h2_t bias = {static_cast<_Float16>(1152.0f), static_cast<_Float16>(1152.0f)};
    h2_t r[4];
    r[0] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) - bias;
    r[1] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) - bias;
    r[2] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) - bias;
    r[3] = __builtin_bit_cast(h2_t, __builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) - bias;
    return __builtin_bit_cast(v8h_t, r);
}

// Key (within a key tile of the 32x32 attention kernels) held in K's LDS row rho. Row rho = 32 b + r
// of 32-key block b with r = 8 j + 4 h + i is output register 4 j + i of the lanes of half h for
// block b (v_mfma_*_32x32 output layout); the keys are chosen
// so that lane half h holds, in register order, the consecutive keys its P^T operand needs:
//   FP8 (64 keys per product): block b = 2 s + t gives keys 64 s + 32 h + 16 t + 4 j + i;
//   bf16 (16 keys per product): block b gives keys 32 b + 16 (j >> 1) + 8 h + 4 (j & 1) + i.
// Either way 8 consecutive registers (fixed b and j >> 1) hold 8 consecutive keys from a multiple of 8.
template <bool FP8>
__host__ __device__ constexpr int kappa_of_row(int rho) {
    const int b = rho >> 5, r = rho & 31, j = r >> 3, h = (r >> 2) & 1, i = r & 3;
    return FP8 ? 64 * (b >> 1) + 32 * h + 16 * (b & 1) + 4 * j + i
               : 32 * b + 16 * (j >> 1) + 8 * h + 4 * (j & 1) + i;
}

typedef __attribute__((address_space(1))) void gvoid_t;
typedef __attribute__((address_space(3))) void lvoid_t;

// s_waitcnt vmcnt(0): every global load of this wave (the tile copies included) has landed.
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Work items (b, h, query block) are handed out so that the workgroups that run on
// one XCD at the same time (dispatch sends workgroup i to XCD i mod 8) share a head:
// XCD x takes the contiguous item range [x per, (x + 1) per), in order.
__device__ __forceinline__ int64_t xcd_item(int64_t L, int64_t per) { return (L & 7) * per + (L >> 3); }

}  // namespace sq
