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
//
// Two kernels:
//  * k_prefix_stage lays every key tile of the prefix out once, in the workspace, exactly as
//    the main kernel wants it in LDS (one linear image per (prefix batch, kv head, tile)):
//    K codes widened to f16 (exact) in the core's permuted, swizzled row order; the keys'
//    FP16 group scales as FP32, group-major in that row order; V^T = bf16(code * scale)
//    channel-major, swizzled as the core's bf16 V^T. The query blocks of every head then
//    copy those images with LDS DMA instead of each converting the same tiles again.
//  * k_prefix follows the attention core's layout (one workgroup = 4 waves = 128 queries of
//    one (b, h); v_mfma 32x32: one query per lane, 16 keys per lane of each 32-key block):
//    per q8 group two v_mfma_f32_32x32x16_f16 of the integer-valued f16 codes give the
//    group's dot exactly in FP32 (|dot| < 2^24), which meets its key's group scale in one
//    FMA; s and the softmax are FP32 in base 2; O^T = V^T P^T on v_mfma_f32_32x32x16_bf16
//    with P = bf16(p); the rows of a query stay in its lane (no exchange to rescale), and
//    the rescale is skipped when no row max of the wave moved. The epilogue merges
//    (prefix out, prefix lse) into (out, lse) in place.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

template <int D, int KT>
struct PCfg {
    static constexpr int NB = KT / 32;               // 32-key blocks of S^T
    static constexpr int NG = D / 32;                // q8 groups per row (and 32-channel blocks of O^T)
    static constexpr int NST = D / 16;               // 16-channel steps of the f16 products
    static constexpr int KROW = 2 * D;               // bytes of one f16 K row
    static constexpr int KNS = KROW / 16;            // 16-byte slots per K row
    static constexpr int RBV = 2 * KT;               // bytes of one bf16 V^T row (one channel)
    static constexpr int VNS = RBV / 16;
    static constexpr int KBYTES = KT * KROW, VBYTES = D * RBV;
    static constexpr int SBYTES = (NG * KT * 4 + 1023) / 1024 * 1024;   // group scales, padded to 1 KB
    static constexpr int IMG = KBYTES + VBYTES + SBYTES;                  // one tile's image
    static constexpr int PIECES = IMG / 1024;
    static_assert(IMG == prefix_image_bytes(D, KT), "the workspace is sized from the same image layout");
};

// ---------------------------------------------------------------------------- tile images
// One workgroup per (tile, kv head, prefix batch): the tile's codes and scales go to LDS with
// coalesced loads (keys at or past P as zeros), then every 16-byte slot of the image is built
// from there and written once.
template <int D, int KT>
__global__ __launch_bounds__(256) void k_prefix_stage(PrefixArgs a) {
    using C = PCfg<D, KT>;
    __shared__ __attribute__((aligned(16))) int8_t kc_s[KT * D];
    __shared__ __attribute__((aligned(16))) int8_t vc_s[KT * D];
    __shared__ float ks_s[KT * C::NG];
    __shared__ float vs_s[KT * C::NG];
    const int tid = threadIdx.x;
    const int tile = blockIdx.x, hk = blockIdx.y, pb = blockIdx.z;
    const int64_t kbase = static_cast<int64_t>(tile) * KT;
    const int8_t* kb = a.k + pb * a.kb + hk * a.kh;
    const int8_t* vb = a.v + pb * a.vb + hk * a.vh;
    const uint16_t* ksb = a.ks + pb * a.ksb + hk * a.ksh;
    const uint16_t* vsb = a.vs + pb * a.vsb + hk * a.vsh;
    for (int i = tid; i < KT * D / 16; i += 256) {
        const int key = i / (D / 16), part = i % (D / 16);
        const int64_t gk = kbase + key;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (gk < a.P) {
            kv = *reinterpret_cast<const uint4*>(kb + gk * a.kt + 16 * part);
            vv = *reinterpret_cast<const uint4*>(vb + gk * a.vt + 16 * part);
        }
        *reinterpret_cast<uint4*>(kc_s + key * D + 16 * part) = kv;
        *reinterpret_cast<uint4*>(vc_s + key * D + 16 * part) = vv;
    }
    for (int i = tid; i < KT * C::NG; i += 256) {
        const int key = i / C::NG, g = i % C::NG;
        const int64_t gk = kbase + key;
        ks_s[i] = gk < a.P ? f16_to_f32(ksb[gk * a.kst + g]) : 0.0f;
        vs_s[i] = gk < a.P ? f16_to_f32(vsb[gk * a.vst + g]) : 0.0f;
    }
    __syncthreads();
    uint8_t* img = a.img + ((static_cast<int64_t>(pb) * a.Hk + hk) * a.ntiles + tile) * C::IMG;
    // K: row rho holds key kappa_of_row(rho); its physical slot s holds channels 8 L .. 8 L + 7, L = swz(rho, s)
    for (int i = tid; i < KT * C::KNS; i += 256) {
        const int rho = i / C::KNS, s = i % C::KNS, L = swz<C::KNS>(rho, s);
        const uint2 w = *reinterpret_cast<const uint2*>(kc_s + kappa_of_row<false>(rho) * D + 8 * L);
        *reinterpret_cast<v8h*>(img + rho * C::KROW + 16 * s) = i8x8_to_f16(w.x, w.y);
    }
    // V^T: row c, physical slot s holds keys 8 L .. 8 L + 7 of channel c, L = swz(c, s)
    for (int i = tid; i < D * C::VNS; i += 256) {
        const int c = i / C::VNS, s = i % C::VNS, L = swz<C::VNS>(c, s);
        v8bf r;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int key = 8 * L + e;
            r[e] = static_cast<__bf16>(static_cast<float>(vc_s[key * D + c]) * vs_s[key * C::NG + c / 32]);
        }
        *reinterpret_cast<v8bf*>(img + C::KBYTES + c * C::RBV + 16 * s) = r;
    }
    // group scales [g][rho]
    float* sim = reinterpret_cast<float*>(img + C::KBYTES + C::VBYTES);
    for (int i = tid; i < C::NG * KT; i += 256) {
        const int g = i / KT, rho = i % KT;
        sim[i] = ks_s[kappa_of_row<false>(rho) * C::NG + g];
    }
}

// ---------------------------------------------------------------------------- prefix pass
template <int D, int KT>
struct PWave {
    using C = PCfg<D, KT>;
    v8h qop[C::NST];          // B operand: this lane's query, channels 16 st + 8 h .. + 7 as f16
    float c1, c2;             // s = c1 t - c2: c1 = qs score_scale, c2 = qs (qc . mu) score_scale
    float m_run, l_run;
    v16f o[C::NG];            // O^T: this lane's query, channels 32 cb + 8 j + 4 h + i
};

// One key tile from its LDS image. TAIL (the last tile when P is not a whole number of tiles): keys at
// or past nval (this lane half's count, as in the core) are masked; a template argument, so that the
// full tiles carry no masking code.
template <int D, int KT, bool TAIL>
__device__ __forceinline__ void prefix_tile(PWave<D, KT>& st, const uint8_t* img, int ql, int h, int nval) {
    using C = PCfg<D, KT>;
    const uint8_t* k_lds = img;
    const uint8_t* v_lds = img + C::KBYTES;
    const float* s_lds = reinterpret_cast<const float*>(img + C::KBYTES + C::VBYTES);
    // t[b][4 j + i] = sum_g ks_g dot_g for key kappa_of_row(32 b + 8 j + 4 h + i)
    v16f t[C::NB];
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        const int row = 32 * b + ql;
#pragma unroll
        for (int g = 0; g < C::NG; ++g) {
            v16f d = {};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int stp = 2 * g + u;
                const v8h kop = *reinterpret_cast<const v8h*>(k_lds + row * C::KROW + swz<C::KNS>(row, 2 * stp + h) * 16);
                d = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop, st.qop[stp], d, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4f sc = *reinterpret_cast<const v4f*>(s_lds + g * KT + 32 * b + 8 * j + 4 * h);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    t[b][4 * j + i] = g == 0 ? d[4 * j + i] * sc[i] : __builtin_fmaf(d[4 * j + i], sc[i], t[b][4 * j + i]);
            }
        }
    }
    if constexpr (TAIL) {
        asm volatile("" : "+v"(nval));
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kappa_of_row<false>(32 * b + 8 * (r >> 2) + (r & 3)) >= nval) t[b][r] = -__builtin_inff();
    }
    // the tile max of s = c1 t - c2 (c1 >= 0: the max of t maps to it); every query sees the tile's
    // first key, so the max over both lane halves is finite
    float mt = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, t[b][r]);
    mt = swap32_max(mt);
    const float ms = __builtin_fmaf(mt, st.c1, -st.c2);
    const float mo = st.m_run;
    const float mn = fmaxf(mo, ms);
    const float alpha = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
    st.m_run = mn;
    // p = 2^(s - m'), l += p, P^T operands: keys 32 b + 16 (j >> 1) + 8 h + 4 (j & 1) + i are elements
    // 4 (j & 1) + i of step 2 b + (j >> 1)
    const float c0 = -(st.c2 + mn);
    float lsum = 0.0f;
    v8bf pbf[KT / 16];
#pragma unroll
    for (int b = 0; b < C::NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int j = r >> 2, i = r & 3;
            float x = __builtin_fmaf(t[b][r], st.c1, c0);
            if (TAIL && t[b][r] == -__builtin_inff()) x = -__builtin_inff();   // a masked key: p = 0 exactly
            const float pv = __builtin_amdgcn_exp2f(x);
            lsum += pv;
            pbf[2 * b + (j >> 1)][4 * (j & 1) + i] = static_cast<__bf16>(pv);
        }
    st.l_run = st.l_run * alpha + lsum;
    if (__builtin_amdgcn_ballot_w64(mn != mo) != 0) {
#pragma unroll
        for (int cb = 0; cb < C::NG; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(st.o[cb][e]) : "v"(alpha));
    }
    // O^T += V^T P^T
#pragma unroll
    for (int cb = 0; cb < C::NG; ++cb) {
        const int row = 32 * cb + ql;
#pragma unroll
        for (int u = 0; u < KT / 16; ++u) {
            const v8bf vop = *reinterpret_cast<const v8bf*>(v_lds + row * C::RBV + swz<C::VNS>(row, 2 * u + h) * 16);
            st.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pbf[u], st.o[cb], 0, 0, 0);
        }
    }
}

// The image of tile j (contiguous, PIECES KB) straight into LDS: wave w copies pieces w, w + 4, ...
template <int D, int KT>
__device__ __forceinline__ void prefix_dma(__amdgpu_buffer_rsrc_t r, int j, uint8_t* buf, int w, int lane) {
    using C = PCfg<D, KT>;
    asm volatile("" : "+s"(w));
    const int base = j * C::IMG + 16 * lane;
#pragma unroll
    for (int u = 0; u < (C::PIECES + 3) / 4; ++u) {
        const int piece = 4 * u + w;
        if (C::PIECES % 4 == 0 || piece < C::PIECES)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lvoid_t*)(buf + 1024 * piece), 16, base + 1024 * piece, 0, 0, 0);
    }
}

template <int D, int KT>
__global__ __launch_bounds__(256, 2) void k_prefix(PrefixArgs a) {
    using C = PCfg<D, KT>;
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[C::IMG];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[C::IMG];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, ql = l & 31, h = l >> 5;
    const int64_t nqb = (a.Sq + 127) / 128, items = nqb * a.H * a.B;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int64_t qb = item % nqb, hh = (item / nqb) % a.H, b = item / (nqb * a.H);
    const int64_t hk = hh / (a.H / a.Hk);
    const int64_t pb = a.PB == 1 ? 0 : b;
    const int64_t qi = qb * 128 + w * 32 + ql;
    const bool ok = qi < a.Sq;

    PWave<D, KT> st;
    {
        const int8_t* qp = a.q + b * a.qsb + (ok ? qi : 0) * a.qst + hh * a.qsh;
#pragma unroll
        for (int s = 0; s < C::NST; ++s) {
            const uint2 c = ok ? *reinterpret_cast<const uint2*>(qp + 16 * s + 8 * h) : make_uint2(0, 0);
            st.qop[s] = i8x8_to_f16(c.x, c.y);
        }
        const float qsc = ok ? a.qs[b * a.qssb + hh * a.qssh + scale_idx(qi, a.q_layout, a.q_block)] : 0.0f;
        // qc . mu over this lane half's channels, then both halves
        float d = 0.0f;
        if (ok && a.mu) {
            const float* mp = a.mu + b * a.mb + hk * a.mh;
#pragma unroll
            for (int s = 0; s < C::NST; ++s) {
                const uint2 c = *reinterpret_cast<const uint2*>(qp + 16 * s + 8 * h);
                const float4 m0 = *reinterpret_cast<const float4*>(mp + 16 * s + 8 * h);
                const float4 m1 = *reinterpret_cast<const float4*>(mp + 16 * s + 8 * h + 4);
                const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    d = __builtin_fmaf(static_cast<float>(static_cast<int8_t>(((e < 4 ? c.x : c.y) >> (8 * (e & 3))) & 0xff)),
                                       mv[e], d);
            }
        }
        d = swap32_add(d);
        st.c1 = qsc * a.score_scale;
        st.c2 = (qsc * d) * a.score_scale;
        st.m_run = -__builtin_inff();
        st.l_run = 0.0f;
#pragma unroll
        for (int cb = 0; cb < C::NG; ++cb) st.o[cb] = v16f{};
    }

    const int ntiles = static_cast<int>(a.ntiles);
    const uint8_t* imgs = a.img + (pb * a.Hk + hk) * a.ntiles * C::IMG;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(imgs), 0, ntiles * C::IMG, 0x00020000);
    // keys of the last tile this lane half sees (the core's count: a half-h lane's keys sit 8 h above half 0's)
    const int nval_last = static_cast<int>(a.P - static_cast<int64_t>(ntiles - 1) * KT) - 8 * h;
    const bool last_partial = a.P % KT != 0;

    prefix_dma<D, KT>(rs, 0, buf0, w, l);
    wait_vm();
    __syncthreads();
    // full tiles in the loop (the buffer of tile j chosen at run time, wave-uniform), a partial last
    // tile after it
    const int nfull = last_partial ? ntiles - 1 : ntiles;
    for (int j = 0; j < nfull; ++j) {
        const bool odd = (j & 1) != 0;
        uint8_t* cur = odd ? buf1 : buf0;
        uint8_t* nxt = odd ? buf0 : buf1;
        if (j + 1 < ntiles) prefix_dma<D, KT>(rs, j + 1, nxt, w, l);
        prefix_tile<D, KT, false>(st, cur, ql, h, 0);
        wait_vm();
        __syncthreads();
    }
    if (last_partial) prefix_tile<D, KT, true>(st, (nfull & 1) ? buf1 : buf0, ql, h, nval_last);

    // ---- epilogue: prefix (out, lse) merged into (out, lse) in place
    float lt = st.l_run;
    lt = swap32_add(lt);
    const float lse_p = st.m_run + log2f(lt);     // -inf when no key contributed
    if (!ok) return;
    float* lsep = a.lse + b * a.lb + hh * a.lh + qi;
    const float la = *lsep;
    const float top = fmaxf(la, lse_p);
    float wa = 0.0f, wb = 0.0f;
    if (top > -__builtin_inff()) {
        wa = __builtin_amdgcn_exp2f(la - top);
        wb = __builtin_amdgcn_exp2f(lse_p - top);
    }
    const float tot = wa + wb;
    const float fa = tot > 0.0f ? wa / tot : 0.0f, fb = wb > 0.0f ? wb / (tot * lt) : 0.0f;
    float* op = a.out + b * a.ob + qi * a.ot + hh * a.oh;
#pragma unroll
    for (int cb = 0; cb < C::NG; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 32 * cb + 8 * j + 4 * h;
            float4 v = *reinterpret_cast<const float4*>(op + c);
            v.x = tot > 0.0f ? __builtin_fmaf(v.x, fa, st.o[cb][4 * j + 0] * fb) : 0.0f;
            v.y = tot > 0.0f ? __builtin_fmaf(v.y, fa, st.o[cb][4 * j + 1] * fb) : 0.0f;
            v.z = tot > 0.0f ? __builtin_fmaf(v.z, fa, st.o[cb][4 * j + 2] * fb) : 0.0f;
            v.w = tot > 0.0f ? __builtin_fmaf(v.w, fa, st.o[cb][4 * j + 3] * fb) : 0.0f;
            *reinterpret_cast<float4*>(op + c) = v;
        }
    // both halves have read *lsep above (one wave, in order); half 0 writes it
    if (h == 0) *lsep = tot > 0.0f ? top + log2f(tot) : -__builtin_inff();
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

template <int D, int KT>
void launch_prefix_dk(const PrefixArgs& a, hipStream_t s) {
    SQ_LAUNCH((k_prefix_stage<D, KT>), dim3(static_cast<unsigned>(a.ntiles), static_cast<unsigned>(a.Hk),
                                              static_cast<unsigned>(a.PB)), dim3(256), 0, s, a);
    const int64_t items = (a.Sq + 127) / 128 * a.H * a.B;
    SQ_LAUNCH((k_prefix<D, KT>), dim3(static_cast<unsigned>((items + 7) / 8 * 8)), dim3(256), 0, s, a);
}

}  // namespace

int launch_prefix(const PrefixArgs& a, void* stream) {
    if (a.B * a.Sq * a.H == 0 || a.P == 0) return SQ_OK;
    hipStream_t s = S(stream);
    if (a.kv_tile == 128) {
        if (a.D == 128) launch_prefix_dk<128, 128>(a, s);
        else launch_prefix_dk<64, 128>(a, s);
    } else {
        if (a.D == 128) launch_prefix_dk<128, 64>(a, s);
        else launch_prefix_dk<64, 64>(a, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn_prefix_lse_merge: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
