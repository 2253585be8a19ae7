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
    static constexpr int KNS = D / 16;           // 16-byte slots per K row
    static constexpr int RBV = 2 * KT;           // bytes of one bf16 V^T row (one channel)
    static constexpr int VNS = RBV / 16;
    static constexpr int KBYTES = KT * D, VBYTES = D * RBV, SBYTES = KT * NG * 4;
    static constexpr int BUF = KBYTES + VBYTES + SBYTES;
    static constexpr int VITEMS = KT / 2 * (D / 16);        // (key pair, 16 channels) items per tile
    static constexpr int VPT = (VITEMS + 255) / 256;        // items per thread
    static constexpr int SCH = (KT * NG + 255) / 256;       // key scales per thread per tile
};

// The next tile's value codes and scales and its key scales, held in registers while the
// current tile is processed, then written to the other LDS buffer. A value item is 16
// channels of two adjacent keys, so each V^T word written holds both keys of one channel.
// Rows past P come back as zeros from the buffer loads (offsets beyond the record count).
template <int D, int KT>
struct PStage {
    using C = PCfg<D, KT>;
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    v4u v[C::VPT][2];
    uint32_t vs[C::VPT][2];
    uint32_t ks[C::SCH];

    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t vr, __amdgpu_buffer_rsrc_t vsr,
                                         __amdgpu_buffer_rsrc_t ksr, int vt, int vst, int kst, int kbase, int tid) {
#pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
            const int j = tid + 256 * u, part = j / (KT / 2), key = kbase + 2 * (j % (KT / 2));
            if (C::VITEMS % 256 == 0 || j < C::VITEMS) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    v[u][e] = __builtin_amdgcn_raw_buffer_load_b128(vr, (key + e) * vt + part * 16, 0, 0);
                    vs[u][e] = __builtin_amdgcn_raw_buffer_load_b16(vsr, 2 * ((key + e) * vst + (part >> 1)), 0, 0);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < C::SCH; ++u) {
            const int j = tid + 256 * u;
            if ((KT * C::NG) % 256 == 0 || j < KT * C::NG)
                ks[u] = __builtin_amdgcn_raw_buffer_load_b16(ksr, 2 * ((kbase + j / C::NG) * kst + j % C::NG), 0, 0);
        }
    }

    // V^T rows (one per channel) of bf16(code * scale), 16-byte slots swizzled; key scales as FP32
    __device__ __forceinline__ void store(uint8_t* vl, float* ksl, int tid) const {
        asm volatile("" : "+v"(tid));
#pragma unroll
        for (int u = 0; u < C::VPT; ++u) {
            const int j = tid + 256 * u, part = j / (KT / 2), kp = j % (KT / 2);
            if (C::VITEMS % 256 == 0 || j < C::VITEMS) {
                const float s0 = f16_to_f32(static_cast<uint16_t>(vs[u][0]));
                const float s1 = f16_to_f32(static_cast<uint16_t>(vs[u][1]));
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int sh = 8 * (k & 3);
                    const float x0 = static_cast<float>(static_cast<int8_t>((v[u][0][k >> 2] >> sh) & 0xff));
                    const float x1 = static_cast<float>(static_cast<int8_t>((v[u][1][k >> 2] >> sh) & 0xff));
                    const int row = part * 16 + k;
                    const int off = row * C::RBV + swz<C::VNS>(row, kp >> 2) * 16 + 4 * (kp & 3);
                    *reinterpret_cast<uint32_t*>(vl + off) =
                        static_cast<uint32_t>(bf16_bits(x0 * s0)) | (static_cast<uint32_t>(bf16_bits(x1 * s1)) << 16);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < C::SCH; ++u) {
            const int j = tid + 256 * u;
            if ((KT * C::NG) % 256 == 0 || j < KT * C::NG) ksl[j] = f16_to_f32(static_cast<uint16_t>(ks[u]));
        }
    }
};

template <int D, int KT>
struct PWave {
    using C = PCfg<D, KT>;
    long qop[C::NQ][C::NG];
    float qsc[C::NQ], dlt[C::NQ];
    float m_run[C::NQ], l_run[C::NQ];
    v4f o[C::NQ][C::NCT];
};

// One key tile of the prefix pass: S^T per q8 group (int32 dots times the key's FP16 scale
// for that group), online softmax in base 2, acc += bf16(p) V^T. TAIL masks keys >= P.
// Scores and probabilities are formed one 16-query tile at a time; P.V runs for both.
template <int D, int KT, bool TAIL>
__device__ __forceinline__ void prefix_tile(const PrefixArgs& a, PWave<D, KT>& st, const uint8_t* k_lds,
                                            const uint8_t* v_lds, const float* ks_lds, int nval, int lane) {
    using C = PCfg<D, KT>;
    int lq = lane & 15, g = lane >> 4;
    v8bf pbf[C::NQ][KT / 32];
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        // fresh lane offsets per query tile: the K and key-scale reads are not kept from the
        // previous tile (that would hold every sub-tile's operands in registers at once)
        asm volatile("" : "+v"(lane));
        lq = lane & 15;
        g = lane >> 4;
        float s[C::NT][4];
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
            __builtin_amdgcn_sched_barrier(0);   // one sub-tile's group dots live at a time
            float ksv[4][C::NG];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int gg = 0; gg < C::NG; ++gg) ksv[i][gg] = ks_lds[(C::KQ * g + 4 * t + i) * C::NG + gg];
#pragma unroll
            for (int i = 0; i < 4; ++i) s[t][i] = 0.0f;
#pragma unroll
            for (int gg = 0; gg < C::NG; ++gg) {
                const int row = 16 * t + lq;
                const int sl = 2 * gg + (g >> 1);                // 16-byte slot holding channels 32 gg + 8 g .. + 7
                const long kop = *reinterpret_cast<const long*>(k_lds + row * D + swz<C::KNS>(row, sl) * 16 + 8 * (g & 1));
                const v4i dg = __builtin_amdgcn_mfma_i32_16x16x32_i8(kop, st.qop[n][gg], v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
                for (int i = 0; i < 4; ++i) s[t][i] = __builtin_fmaf(ksv[i][gg], static_cast<float>(dg[i]), s[t][i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float sv = __builtin_fmaf(st.qsc[n], s[t][i], -st.dlt[n]);
                if (a.score_scale != 1.0f) sv = sv * a.score_scale;
                if (TAIL && 4 * t + i >= nval) sv = -__builtin_inff();
                s[t][i] = sv;
            }
        }

        __builtin_amdgcn_sched_barrier(0);
        float mt = -__builtin_inff();
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[t][i]);
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const float mo = st.m_run[n];
        const float mn = fmaxf(mo, mt);
        const float alpha = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        st.m_run[n] = mn;
        float lsum = 0.0f;
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // mn is finite: the tile's first key exists, so every lane group's max is real
                const float pv = __builtin_amdgcn_exp2f(s[t][i] - mn);
                lsum += pv;
                pbf[n][t >> 1][4 * (t & 1) + i] = static_cast<__bf16>(pv);
            }
        st.l_run[n] = st.l_run[n] * alpha + lsum;
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
                for (int ct = 0; ct < C::NCT; ++ct) st.o[n][ct][i] *= ai;
            }
        }
    }

    asm volatile("" : "+v"(lane));
    lq = lane & 15;
    g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
        if (ct % 2 == 0) __builtin_amdgcn_sched_barrier(0);
        const int row = ct * 16 + lq;
#pragma unroll
        for (int u = 0; u < KT / 32; ++u) {
            const int ls = (C::KQ * g + 8 * u) / 8;      // 16-byte slot of keys KQ g + 8 u .. + 7
            const v8bf vop = *reinterpret_cast<const v8bf*>(v_lds + row * C::RBV + swz<C::VNS>(row, ls) * 16);
#pragma unroll
            for (int n = 0; n < C::NQ; ++n)
                st.o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pbf[n][u], vop, st.o[n][ct], 0, 0, 0);
        }
    }
}

// K codes of tile [kbase, kbase + KT) straight into LDS (rows permuted as in the core:
// key G KQ + 4 t + i -> row 16 t + 4 G + i; slots swizzled); rows past P read as zeros.
template <int D, int KT>
__device__ __forceinline__ void prefix_dma_k(__amdgpu_buffer_rsrc_t kr, int kst, int kbase, uint8_t* kl, int w, int lane) {
    using C = PCfg<D, KT>;
    constexpr int KCH = C::KBYTES / 1024;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int u = 0; u < (KCH + 3) / 4; ++u) {
        const int piece = 4 * u + w;
        if (KCH % 4 == 0 || piece < KCH) {
            const int o = 1024 * piece + 16 * lane;
            const int row = o / D, ls = swz<C::KNS>(row, (o % D) / 16);
            const int key = kbase + ((row & 15) >> 2) * C::KQ + 4 * (row >> 4) + (row & 3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lvoid_t*)(kl + 1024 * piece), 16, key * kst + ls * 16, 0, 0, 0);
        }
    }
}

template <int D, int KT>
__global__ __launch_bounds__(256, 2) void k_prefix(PrefixArgs a) {
    using C = PCfg<D, KT>;
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[C::BUF];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[C::BUF];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lq = l & 15, g = l >> 4;
    const int64_t nqb = (a.Sq + C::QPB - 1) / C::QPB, items = nqb * a.H * a.B;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int64_t qb = item % nqb, h = (item / nqb) % a.H, b = item / (nqb * a.H);
    const int64_t hk = h / (a.H / a.Hk);
    const int64_t q0 = qb * C::QPB + w * (C::NQ * 16);
    const int64_t pb = a.PB == 1 ? 0 : b;

    // q codes per group (B operand), q scale and the offset delta = qs (qc . mu)
    PWave<D, KT> st;
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        const int64_t qi = q0 + n * 16 + lq;
        const bool ok = qi < a.Sq;
        const int8_t* qp = a.q + b * a.qsb + qi * a.qst + h * a.qsh;
#pragma unroll
        for (int gg = 0; gg < C::NG; ++gg) st.qop[n][gg] = ok ? *reinterpret_cast<const long*>(qp + 32 * gg + 8 * g) : 0;
        st.qsc[n] = ok ? a.qs[b * a.qssb + h * a.qssh + scale_idx(qi, a.q_layout, a.q_block)] : 0.0f;
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
        st.dlt[n] = st.qsc[n] * d;
        st.m_run[n] = -__builtin_inff();
        st.l_run[n] = 0.0f;
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) st.o[n][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    const int8_t* kb = a.k + pb * a.kb + hk * a.kh;
    const uint16_t* ksb = a.ks + pb * a.ksb + hk * a.ksh;
    const int8_t* vb = a.v + pb * a.vb + hk * a.vh;
    const uint16_t* vsb = a.vs + pb * a.vsb + hk * a.vsh;
    // 32-bit offsets: the host checks that (P + 128) rows of every operand span < 2^31 bytes
    const int kst = static_cast<int>(a.kt), vt = static_cast<int>(a.vt);
    const int kss = static_cast<int>(a.kst), vss = static_cast<int>(a.vst);
    const int P = static_cast<int>(a.P);
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(kb), 0, (P - 1) * kst + D, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(vb), 0, (P - 1) * vt + D, 0x00020000);
    const __amdgpu_buffer_rsrc_t vsrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vsb), 0, 2 * ((P - 1) * vss + C::NG), 0x00020000);
    const __amdgpu_buffer_rsrc_t ksrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(ksb), 0, 2 * ((P - 1) * kss + C::NG), 0x00020000);
    const int ntiles = (P + KT - 1) / KT;
    const int last = ntiles - 1;
    // keys of the last tile held by this lane group (all KQ when the tile is full)
    const int nval_last = P - last * KT - C::KQ * g;
    const bool tail = nval_last < C::KQ;

    PStage<D, KT> pre;
    auto copy = [&](int j, uint8_t* buf) {
        prefix_dma_k<D, KT>(krs, kst, j * KT, buf, w, l);
        pre.load(vrs, vsrs, ksrs, vt, vss, kss, j * KT, tid);
    };
    auto place = [&](uint8_t* buf) {
        pre.store(buf + C::KBYTES, reinterpret_cast<float*>(buf + C::KBYTES + C::VBYTES), tid);
    };
    auto step = [&](const uint8_t* buf) {
        prefix_tile<D, KT, false>(a, st, buf, buf + C::KBYTES,
                                  reinterpret_cast<const float*>(buf + C::KBYTES + C::VBYTES), C::KQ, l);
    };

    copy(0, buf0);
    place(buf0);
    wait_vm();
    __syncthreads();
    // full tiles two at a time over the two buffers; the last tile (full or not) after
    const int nbody = last;     // tiles processed inside the loop
    int j = 0;
    for (; j + 1 < nbody; j += 2) {
        copy(j + 1, buf1);
        step(buf0);
        place(buf1);
        wait_vm();
        __syncthreads();
        copy(j + 2, buf0);
        step(buf1);
        place(buf0);
        wait_vm();
        __syncthreads();
    }
    if (j < nbody) {            // one more body tile: it sits in buf0, the last goes to buf1
        copy(j + 1, buf1);
        step(buf0);
        place(buf1);
        wait_vm();
        __syncthreads();
        ++j;
    }
    const uint8_t* lb = (j & 1) ? buf1 : buf0;
    if (__builtin_expect(__any(tail), 0))   // lane groups past P see nval <= 0: every key masked
        prefix_tile<D, KT, true>(a, st, lb, lb + C::KBYTES, reinterpret_cast<const float*>(lb + C::KBYTES + C::VBYTES),
                                 nval_last, l);
    else
        step(lb);

    // ---- epilogue: prefix (out, lse) merged into (out, lse) in place
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        float lt = st.l_run[n];
        lt = lt + shfl_xor(lt, 16);
        lt = lt + shfl_xor(lt, 32);
        const float lse_p = st.m_run[n] + log2f(lt);     // -inf when no key contributed
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
                op[c] = tot > 0.0f ? __builtin_fmaf(op[c], fa, st.o[n][ct][i] * fb) : 0.0f;
            }
            // all 16 lanes of this row read *lsep above, in the same instruction
            if (lq == 0) *lsep = tot > 0.0f ? top + log2f(tot) : -__builtin_inff();
        }
    }
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

int launch_prefix(const PrefixArgs& a, void* stream) {
    if (a.B * a.Sq * a.H == 0 || a.P == 0) return SQ_OK;
    const int64_t items = (a.Sq + 127) / 128 * a.H * a.B;
    dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
    hipStream_t s = S(stream);
    if (a.kv_tile == 128) {
        if (a.D == 128) SQ_LAUNCH((k_prefix<128, 128>), grid, dim3(256), 0, s, a);
        else SQ_LAUNCH((k_prefix<64, 128>), grid, dim3(256), 0, s, a);
    } else {
        if (a.D == 128) SQ_LAUNCH((k_prefix<128, 64>), grid, dim3(256), 0, s, a);
        else SQ_LAUNCH((k_prefix<64, 64>), grid, dim3(256), 0, s, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn_prefix_lse_merge: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
