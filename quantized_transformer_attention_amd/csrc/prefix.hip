// Cached q8 prefix pass merged with the projected-key pass by log-sum-exp, on gfx950.
//
// Method: [kit] WanGP shared/attention_kit.py -- KVPrefix and GROUP (q8: int8 per
// token, head and 32 channels with one FP16 scale), dequantize_q8_into (16-bit value
// = code * scale rounded once), _attend_with_prefix (the prefix attended in a pass of
// its own that returns its log-sum-exp) and _merge_lse_ (base-2 merge of two passes);
// the online softmax of [tq] vLLM triton_turboquant_unified_attention.py.
//
// Scores of the prefix keys share the projected keys' offset: s = qh . (kh - mu) with
// qh = q code * q scale and kh = code * FP16 scale per 32 channels, i.e.
//   s = qs * sum_g ks_g * (qc . kc)_g  -  qs * (qc . mu).
// One workgroup = 4 waves = 128 queries of one (b, h), as the core:
//  * S^T = K Q^T per 32-channel group with v_mfma_i32_16x16x32_i8 (K = one q8 group),
//    so each group's exact int32 dot meets its own key scale in FP32;
//  * V codes are dequantized while staged: bf16(code * scale) channel-major in LDS,
//    the B operand of the bf16 P.V MFMA; P = bf16(p);
//  * the epilogue merges (prefix out, prefix lse) into (out, lse) in place.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int D, int KT>
struct PCfg {
    static constexpr int NQ = 2;                 // 16-query tiles per wave
    static constexpr int QPB = 4 * NQ * 16;      // queries per workgroup
    static constexpr int NT = KT / 16;           // 16-key sub-tiles
    static constexpr int NG = D / 32;            // q8 groups per row
    static constexpr int NCT = D / 16;           // 16-channel tiles of P.V
    static constexpr int KQ = KT / 4;            // keys per lane group
    static constexpr int KSTR = D + 16;          // LDS K row stride, bytes
    static constexpr int VSTR = 2 * KT + 16;     // LDS V^T row stride, bytes
};

template <int D, int KT>
__global__ __launch_bounds__(256) void k_prefix(PrefixArgs a) {
    using C = PCfg<D, KT>;
    __shared__ __attribute__((aligned(16))) uint8_t k_lds[KT * C::KSTR];
    __shared__ __attribute__((aligned(16))) uint8_t v_lds[D * C::VSTR];
    __shared__ __attribute__((aligned(16))) float ks_lds[KT * C::NG];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lq = l & 15, g = l >> 4;
    const int64_t h = blockIdx.y, b = blockIdx.z;
    const int64_t hk = h / (a.H / a.Hk);
    const int64_t q0 = static_cast<int64_t>(blockIdx.x) * C::QPB + w * (C::NQ * 16);
    const int64_t pb = a.PB == 1 ? 0 : b;

    // q codes per group (B operand), q scale and the offset delta = qs (qc . mu)
    long qop[C::NQ][C::NG];
    float qsc[C::NQ], dlt[C::NQ];
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        const int64_t qi = q0 + n * 16 + lq;
        const bool ok = qi < a.Sq;
        const int8_t* qp = a.q + b * a.qsb + qi * a.qst + h * a.qsh;
#pragma unroll
        for (int gg = 0; gg < C::NG; ++gg) qop[n][gg] = ok ? *reinterpret_cast<const long*>(qp + 32 * gg + 8 * g) : 0;
        qsc[n] = ok ? a.qs[b * a.qssb + h * a.qssh + scale_idx(qi, a.q_layout, a.q_block)] : 0.0f;
        float d = 0.0f;
        if (ok && a.mu) {
            const float* mp = a.mu + b * a.mb + hk * a.mh;
            for (int c = 0; c < D; c += 4) {
                const int cw = *reinterpret_cast<const int*>(qp + c);
                const float4 m4 = *reinterpret_cast<const float4*>(mp + c);
                d = __builtin_fmaf(static_cast<float>(static_cast<int8_t>(cw & 0xff)), m4.x, d);
                d = __builtin_fmaf(static_cast<float>(static_cast<int8_t>((cw >> 8) & 0xff)), m4.y, d);
                d = __builtin_fmaf(static_cast<float>(static_cast<int8_t>((cw >> 16) & 0xff)), m4.z, d);
                d = __builtin_fmaf(static_cast<float>(static_cast<int8_t>((cw >> 24) & 0xff)), m4.w, d);
            }
        }
        dlt[n] = qsc[n] * d;
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

    const int8_t* kb = a.k + pb * a.kb + hk * a.kh;
    const uint16_t* ksb = a.ks + pb * a.ksb + hk * a.ksh;
    const int8_t* vb = a.v + pb * a.vb + hk * a.vh;
    const uint16_t* vsb = a.vs + pb * a.vsb + hk * a.vsh;
    const int64_t ntiles = (a.P + KT - 1) / KT;
    for (int64_t tile = 0; tile < ntiles; ++tile) {
        const int64_t kbase = tile * KT;
        __syncthreads();
        // ---- stage K codes (rows permuted as the core: key kappa -> row 16 t + 4 G + i)
        for (int j = tid; j < KT * D / 16; j += 256) {
            const int kappa = j / (D / 16), part = j % (D / 16);
            const int64_t key = kbase + kappa;
            v4i val = {0, 0, 0, 0};
            if (key < a.P) val = *reinterpret_cast<const v4i*>(kb + key * a.kt + part * 16);
            const int G4 = kappa / C::KQ, rem = kappa % C::KQ;
            const int row = 16 * (rem >> 2) + 4 * G4 + (rem & 3);
            *reinterpret_cast<v4i*>(k_lds + row * C::KSTR + part * 16) = val;
        }
        // ---- key scales (natural key order)
        for (int j = tid; j < KT * C::NG; j += 256) {
            const int kappa = j / C::NG, gg = j % C::NG;
            const int64_t key = kbase + kappa;
            ks_lds[j] = key < a.P ? f16_to_f32(ksb[key * a.kst + gg]) : 0.0f;
        }
        // ---- V: bf16(code * scale), channel-major
        for (int j = tid; j < KT * D / 16; j += 256) {
            const int kappa = j / (D / 16), part = j % (D / 16);
            const int64_t key = kbase + kappa;
            uint16_t* dst = reinterpret_cast<uint16_t*>(v_lds) + (part * 16) * (C::VSTR / 2) + kappa;
            if (key < a.P) {
                const uint4 raw = *reinterpret_cast<const uint4*>(vb + key * a.vt + part * 16);
                const float sc = f16_to_f32(vsb[key * a.vst + (part >> 1)]);
                const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const float x = static_cast<float>(static_cast<int8_t>((wv[k >> 2] >> (8 * (k & 3))) & 0xff));
                    dst[k * (C::VSTR / 2)] = bf16_bits(x * sc);
                }
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) dst[k * (C::VSTR / 2)] = 0;
            }
        }
        __syncthreads();

        // ---- S^T = K Q^T per q8 group, scaled by the key scales
        const int64_t kg0 = kbase + C::KQ * g;
        const bool partial = kbase + KT > a.P;
        float s[C::NT][C::NQ][4];
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
            float ksv[4][C::NG];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int gg = 0; gg < C::NG; ++gg) ksv[i][gg] = ks_lds[(C::KQ * g + 4 * t + i) * C::NG + gg];
            v4i dg[C::NQ][C::NG];
#pragma unroll
            for (int gg = 0; gg < C::NG; ++gg) {
                const long kop = *reinterpret_cast<const long*>(k_lds + (16 * t + lq) * C::KSTR + 32 * gg + 8 * g);
#pragma unroll
                for (int n = 0; n < C::NQ; ++n)
                    dg[n][gg] = __builtin_amdgcn_mfma_i32_16x16x32_i8(kop, qop[n][gg], v4i{0, 0, 0, 0}, 0, 0, 0);
            }
#pragma unroll
            for (int n = 0; n < C::NQ; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float acc = ksv[i][0] * static_cast<float>(dg[n][0][i]);
#pragma unroll
                    for (int gg = 1; gg < C::NG; ++gg) acc = __builtin_fmaf(ksv[i][gg], static_cast<float>(dg[n][gg][i]), acc);
                    float sv = __builtin_fmaf(qsc[n], acc, -dlt[n]);
                    if (a.score_scale != 1.0f) sv = sv * a.score_scale;
                    if (partial && kg0 + 4 * t + i >= a.P) sv = -__builtin_inff();
                    s[t][n][i] = sv;
                }
        }

        // ---- online softmax (base 2), P = bf16(p)
        v8bf pbf[C::NQ][KT / 32];
#pragma unroll
        for (int n = 0; n < C::NQ; ++n) {
            float mt = -__builtin_inff();
#pragma unroll
            for (int t = 0; t < C::NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[t][n][i]);
            mt = fmaxf(mt, shfl_xor(mt, 16));
            mt = fmaxf(mt, shfl_xor(mt, 32));
            const float mo = m_run[n];
            const float mn = fmaxf(mo, mt);
            const float alpha = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
            m_run[n] = mn;
            float p[C::NT][4], lsum = 0.0f;
#pragma unroll
            for (int t = 0; t < C::NT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = s[t][n][i] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(s[t][n][i] - mn);
                    p[t][i] = pv;
                    lsum += pv;
                }
            l_run[n] = l_run[n] * alpha + lsum;
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
            if (__any(alpha != 1.0f)) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
                    for (int ct = 0; ct < C::NCT; ++ct) o[n][ct][i] *= ai;
                }
            }
        }

        // ---- acc += P V
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) {
#pragma unroll
            for (int u = 0; u < KT / 32; ++u) {
                const v8bf vop = *reinterpret_cast<const v8bf*>(v_lds + (ct * 16 + lq) * C::VSTR + 2 * (C::KQ * g + 8 * u));
#pragma unroll
                for (int n = 0; n < C::NQ; ++n)
                    o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pbf[n][u], vop, o[n][ct], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: prefix (out, lse) merged into (out, lse) in place
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        float lt = l_run[n];
        lt = lt + shfl_xor(lt, 16);
        lt = lt + shfl_xor(lt, 32);
        const float lse_p = m_run[n] + log2f(lt);     // -inf when no key contributed
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t qr = q0 + n * 16 + 4 * g + i;
            const float li = __shfl(lt, 4 * g + i, kWave);
            const float lp = __shfl(lse_p, 4 * g + i, kWave);
            if (qr >= a.Sq) continue;
            float* lsep = a.lse + b * a.lb + h * a.lh + qr;
            const float la = *lsep;
            const float top = fmaxf(la, lp);
            float wa = 0.0f, wb = 0.0f;
            if (top > -__builtin_inff()) {
                wa = __builtin_amdgcn_exp2f(la - top);
                wb = __builtin_amdgcn_exp2f(lp - top);
            }
            const float tot = wa + wb;
            const float fa = tot > 0.0f ? wa / tot : 0.0f, fb = wb > 0.0f ? wb / (tot * li) : 0.0f;
            float* op = a.out + b * a.ob + qr * a.ot + h * a.oh;
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct) {
                const int c = ct * 16 + lq;
                op[c] = tot > 0.0f ? __builtin_fmaf(op[c], fa, o[n][ct][i] * fb) : 0.0f;
            }
            // every lane of the 16 has read *lsep above: write after the reads of this row
            if (lq == 0) *lsep = tot > 0.0f ? top + log2f(tot) : -__builtin_inff();
        }
    }
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

int launch_prefix(const PrefixArgs& a, void* stream) {
    if (a.B * a.Sq * a.H == 0 || a.P == 0) return SQ_OK;
    dim3 grid(static_cast<unsigned>((a.Sq + 127) / 128), static_cast<unsigned>(a.H), static_cast<unsigned>(a.B));
    hipStream_t s = S(stream);
    if (a.kv_tile == 128) {
        if (a.D == 128) hipLaunchKernelGGL((k_prefix<128, 128>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_prefix<64, 128>), grid, dim3(256), 0, s, a);
    } else {
        if (a.D == 128) hipLaunchKernelGGL((k_prefix<128, 64>), grid, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((k_prefix<64, 64>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn_prefix_lse_merge: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
