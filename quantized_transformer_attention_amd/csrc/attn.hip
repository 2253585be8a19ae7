// Quantized attention core on gfx950: INT8 Q.K^T on MFMA, FP32 online softmax in
// base 2, P.V on FP8 or bf16 MFMA.
//
// Method: the staged quantized core of [kit] WanGP shared/attention_kit.py
// (q/k INT8 with block scales, v FP8 or 16-bit) and the online softmax of [tq] vLLM
// triton_turboquant_unified_attention.py (kernel_tq_unified_attention_2d: m_j, P,
// l_j, alpha, acc). [impl] _repeat_kv_for_heads fixes the GQA head mapping.
//
// Design (one workgroup = 4 waves = 128 queries of one (b, h); K and V^T tiles of
// KT keys staged once in LDS and shared by the 4 waves):
//  * S^T = K Q^T with v_mfma_i32_16x16x64_i8: the 16x16 result puts one query per
//    lane column (lane % 16) and 4 keys per lane, so the row max and sum over keys
//    are in-lane plus two cross-lane steps.
//  * K rows are permuted into LDS so that lane group g (lane / 16) ends up holding
//    the KT/4 consecutive keys [g KT/4, (g+1) KT/4): those registers are then
//    already the A operand (P, queries x keys) of the P.V MFMA, and the B operand
//    (V, keys x channels) is a contiguous run of keys of one channel -- which is why
//    V is read channel-major (sq_quant_v_fp8 writes FP8 V that way; bf16 V is
//    staged channel-major by k_v_transpose).
//  * The softmax max is taken on the int32 dots per k-scale group (c > 0 makes
//    RN(a c) monotonic in a), and p = 2^fma(a, c, -m') uses the hardware exp2.
//  * FP8 P.V: Pt = e4m3(256 p) by a scaled convert (2^-8 scale: exact), one
//    v_mfma_f32_16x16x128_f8f6f4 per 16 channels per 128 keys.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));

// 4 floats -> 4 e4m3 bytes of 256 x (the scaled convert divides by its scale, 2^-8).
__device__ __forceinline__ int pack_fp8x4_256(float a, float b, float c, float d) {
    v2s r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, a, b, 0.00390625f, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c, d, 0.00390625f, true);
    return __builtin_bit_cast(int, r);
}

template <int D, int KT, bool FP8>
struct Cfg {
    static constexpr int NQ = 2;                     // 16-query tiles per wave
    static constexpr int QPB = 4 * NQ * 16;          // queries per workgroup
    static constexpr int NT = KT / 16;               // 16-key sub-tiles
    static constexpr int NC = D / 64;                // 64-channel chunks of Q.K^T
    static constexpr int NCT = D / 16;               // 16-channel tiles of P.V
    static constexpr int KQ = KT / 4;                // keys per lane group
    static constexpr int KSTR = D + 16;              // LDS K row stride, bytes
    static constexpr int VSTR = FP8 ? KT + 16 : 2 * KT + 16;  // LDS V^T row stride, bytes
};

template <int D, int KT, bool FP8>
__global__ __launch_bounds__(256) void k_attn(AttnArgs a) {
    using C = Cfg<D, KT, FP8>;
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[KT * C::KSTR];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * C::VSTR];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 15, g = l >> 4;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int64_t hk = h / (a.H / a.Hk);
    const int64_t q0 = static_cast<int64_t>(blockIdx.x) * C::QPB + w * (C::NQ * 16);

    // Q codes as the B operand of S^T = K Q^T (held for the whole key loop), q scales
    v4i qop[C::NQ][C::NC];
    float qsc[C::NQ];
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        const int64_t qi = q0 + n * 16 + lq;
        const bool ok = qi < a.Sq;
#pragma unroll
        for (int ch = 0; ch < C::NC; ++ch) {
            v4i z = {0, 0, 0, 0};
            qop[n][ch] = ok ? *reinterpret_cast<const v4i*>(a.q + b * a.qsb + qi * a.qst + h * a.qsh + ch * 64 + 16 * g) : z;
        }
        qsc[n] = ok ? a.qs[b * a.qssb + h * a.qssh + scale_idx(qi, a.q_layout, a.q_block)] : 0.0f;
    }

    float m_run[C::NQ], l_run[C::NQ];
    v4f o[C::NQ][C::NCT];
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        m_run[n] = -__builtin_inff();
        l_run[n] = 0.0f;
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) o[n][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int64_t ntiles = (a.Sk + KT - 1) / KT;
    const int8_t* kbase_ptr = a.k + b * a.ksb + hk * a.ksh;
    for (int64_t tile = 0; tile < ntiles; ++tile) {
        const int64_t kbase = tile * KT;
        __syncthreads();
        // ---- stage K (rows permuted: key kappa -> row 16 t + 4 G + ii) and V^T
        for (int j = tid; j < KT * D / 16; j += 256) {
            const int kappa = j / (D / 16), part = j % (D / 16);
            const int64_t key = kbase + kappa;
            v4i val = {0, 0, 0, 0};
            if (key < a.Sk) val = *reinterpret_cast<const v4i*>(kbase_ptr + key * a.kst + part * 16);
            const int G4 = kappa / C::KQ, rem = kappa % C::KQ;
            const int row = 16 * (rem >> 2) + 4 * G4 + (rem & 3);
            *reinterpret_cast<v4i*>(k_lds + row * C::KSTR + part * 16) = val;
        }
        if constexpr (FP8) {
            const uint8_t* vb = static_cast<const uint8_t*>(a.v) + b * a.vsb + hk * a.vsh;
            for (int j = tid; j < D * KT / 16; j += 256) {
                const int c = j / (KT / 16), part = j % (KT / 16);
                const int64_t key = kbase + part * 16;
                v4i val = {0, 0, 0, 0};
                if (key < a.Sk) val = *reinterpret_cast<const v4i*>(vb + c * a.vsd + key);
                *reinterpret_cast<v4i*>(v_lds + c * C::VSTR + part * 16) = val;
            }
        } else {
            const uint16_t* vb = static_cast<const uint16_t*>(a.v) + b * a.vsb + hk * a.vsh;
            for (int j = tid; j < D * KT / 8; j += 256) {
                const int c = j / (KT / 8), part = j % (KT / 8);
                const int64_t key = kbase + part * 8;
                v4i val = {0, 0, 0, 0};
                if (key < a.Sk) val = *reinterpret_cast<const v4i*>(vb + c * a.vsd + key);
                *reinterpret_cast<v4i*>(v_lds + c * C::VSTR + part * 16) = val;
            }
        }
        __syncthreads();

        // ---- c = RN(qs ks) per k-scale group of this lane group's keys
        const int64_t kg0 = kbase + C::KQ * g;
        float cg[C::NQ][4];
        {
            float ks[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (kg0 < a.Sk) {
                const float* kp = a.ks + b * a.kssb + hk * a.kssh;
                if (a.k_layout == SQ_LAYOUT_THREAD_K) {
                    const int64_t base = 4 * (kg0 >> 6);
#pragma unroll
                    for (int q = 0; q < 4; ++q) ks[q] = kp[base + q];
                } else {
                    const float s = kp[kg0 / a.k_block];
#pragma unroll
                    for (int q = 0; q < 4; ++q) ks[q] = s;
                }
            }
#pragma unroll
            for (int n = 0; n < C::NQ; ++n)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float c = qsc[n] * ks[q];
                    if (a.score_scale != 1.0f) c = c * a.score_scale;
                    cg[n][q] = c;
                }
        }

        // ---- S^T = K Q^T (int32)
        v4i s[C::NT][C::NQ];
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
#pragma unroll
            for (int n = 0; n < C::NQ; ++n) s[t][n] = v4i{0, 0, 0, 0};
#pragma unroll
            for (int ch = 0; ch < C::NC; ++ch) {
                const v4i kop = *reinterpret_cast<const v4i*>(k_lds + (16 * t + lq) * C::KSTR + ch * 64 + 16 * g);
#pragma unroll
                for (int n = 0; n < C::NQ; ++n) s[t][n] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, qop[n][ch], s[t][n], 0, 0, 0);
            }
        }

        const bool partial = kbase + KT > a.Sk;
        // ---- online softmax, P operands
        v8i pf8[C::NQ];
        v8bf pbf[C::NQ][KT / 32];
#pragma unroll
        for (int n = 0; n < C::NQ; ++n) {
            int amx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
#pragma unroll
            for (int t = 0; t < C::NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    int av = s[t][n][i];
                    if (partial && kg0 + 4 * t + i >= a.Sk) {
                        av = INT32_MIN;
                        s[t][n][i] = INT32_MIN;
                    }
                    const int q = 2 * (t & 1) + (i >> 1);
                    amx[q] = max(amx[q], av);
                }
            float mt = -__builtin_inff();
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (amx[q] != INT32_MIN) mt = fmaxf(mt, static_cast<float>(amx[q]) * cg[n][q]);
            mt = fmaxf(mt, shfl_xor(mt, 16));
            mt = fmaxf(mt, shfl_xor(mt, 32));
            const float mo = m_run[n];
            const float mn = fmaxf(mo, mt);
            const float alpha = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
            m_run[n] = mn;
            float lsum = 0.0f;
            float p[C::NT][4];
#pragma unroll
            for (int t = 0; t < C::NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int q = 2 * (t & 1) + (i >> 1);
                    const int av = s[t][n][i];
                    float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(av), cg[n][q], -mn));
                    if (partial && av == INT32_MIN) pv = 0.0f;
                    p[t][i] = pv;
                    lsum += pv;
                }
            l_run[n] = l_run[n] * alpha + lsum;
            if constexpr (FP8) {
#pragma unroll
                for (int t = 0; t < C::NT; ++t) pf8[n][t] = pack_fp8x4_256(p[t][0], p[t][1], p[t][2], p[t][3]);
            } else {
#pragma unroll
                for (int u = 0; u < KT / 32; ++u) {
                    v8bf x;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = static_cast<__bf16>(p[2 * u][i]);
                        x[4 + i] = static_cast<__bf16>(p[2 * u + 1][i]);
                    }
                    pbf[n][u] = x;
                }
            }
            // rescale the accumulator rows (query 4 g + i of this n-tile) when a max moved
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
                    for (int ct = 0; ct < C::NCT; ++ct) o[n][ct][i] *= ai;
                }
            }
        }

        // ---- acc += Pt Vt
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) {
            if constexpr (FP8) {
                const v8i vop = *reinterpret_cast<const v8i*>(v_lds + (ct * 16 + lq) * C::VSTR + 32 * g);
#pragma unroll
                for (int n = 0; n < C::NQ; ++n)
                    o[n][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf8[n], vop, o[n][ct], 0, 0, 0, 0, 0, 0);
            } else {
#pragma unroll
                for (int u = 0; u < KT / 32; ++u) {
                    const v8bf vop = *reinterpret_cast<const v8bf*>(v_lds + (ct * 16 + lq) * C::VSTR + 2 * (C::KQ * g + 8 * u));
#pragma unroll
                    for (int n = 0; n < C::NQ; ++n)
                        o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pbf[n][u], vop, o[n][ct], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: l over the 4 lane groups, lse, out = acc / l (x vs / 256)
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        float lt = l_run[n];
        lt = lt + shfl_xor(lt, 16);
        lt = lt + shfl_xor(lt, 32);
        const int64_t qi = q0 + n * 16 + lq;
        if (a.lse && g == 0 && qi < a.Sq) a.lse[b * a.lb + h * a.lh + qi] = m_run[n] + log2f(lt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(lt, 4 * g + i, kWave);
            const float inv = 1.0f / li;
            const int64_t qr = q0 + n * 16 + 4 * g + i;
            if (qr >= a.Sq) continue;
            float* op = a.out + b * a.ob + qr * a.ot + h * a.oh;
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct) {
                const int c = ct * 16 + lq;
                float val = o[n][ct][i] * inv;
                if constexpr (FP8) val = val * (a.vscale[b * a.vssb + hk * a.vssh + c] * 0.00390625f);
                op[c] = val;
            }
        }
    }
}

// Token-major bf16 V (B, S, H, D) -> channel-major (B, H, D, Spad), zero-padded.
template <int D>
__global__ __launch_bounds__(256) void k_v_transpose(VTransposeArgs a) {
    constexpr int STR = 64 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t tileT[D * STR];
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * 64, h = blockIdx.y, b = blockIdx.z;
    for (int j = tid; j < 64 * (D / 8); j += 256) {
        const int row = j / (D / 8), part = j % (D / 8);
        const int64_t t = t0 + row;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (t < a.S) val = *reinterpret_cast<const uint4*>(a.v + b * a.sb + t * a.st + h * a.sh + part * 8);
        const uint32_t wv[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            tileT[(part * 8 + 2 * k) * STR + row] = static_cast<uint16_t>(wv[k] & 0xffff);
            tileT[(part * 8 + 2 * k + 1) * STR + row] = static_cast<uint16_t>(wv[k] >> 16);
        }
    }
    __syncthreads();
    for (int j = tid; j < D * 8; j += 256) {
        const int c = j >> 3, part = (j & 7) * 8;
        const uint4 val = *reinterpret_cast<const uint4*>(&tileT[c * STR + part]);
        *reinterpret_cast<uint4*>(a.out + ((b * a.H + h) * D + c) * a.Spad + t0 + part) = val;
    }
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

int launch_v_transpose(const VTransposeArgs& a, void* stream) {
    dim3 grid(static_cast<unsigned>(a.Spad / 64), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    if (a.D == 128) hipLaunchKernelGGL(k_v_transpose<128>, grid, dim3(256), 0, S(stream), a);
    else hipLaunchKernelGGL(k_v_transpose<64>, grid, dim3(256), 0, S(stream), a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn: V staging launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

int launch_attn(const AttnArgs& a, void* stream) {
    if (a.B * a.Sq * a.H == 0) return SQ_OK;
    dim3 grid(static_cast<unsigned>((a.Sq + 127) / 128), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    hipStream_t s = S(stream);
    if (a.v_fp8) {
        if (a.D == 128) hipLaunchKernelGGL((k_attn<128, 128, true>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_attn<64, 128, true>), grid, dim3(256), 0, s, a);
    } else if (a.kv_tile == 128) {
        if (a.D == 128) hipLaunchKernelGGL((k_attn<128, 128, false>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_attn<64, 128, false>), grid, dim3(256), 0, s, a);
    } else {
        if (a.D == 128) hipLaunchKernelGGL((k_attn<128, 64, false>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_attn<64, 64, false>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
