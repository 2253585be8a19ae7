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
    v2s r;   // both halves are written below: no initial value is needed
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
    static constexpr int VB = FP8 ? 1 : 2;           // bytes per V element
    static constexpr int RBV = KT * VB;              // bytes of one V^T row (one channel)
    static constexpr int KBYTES = KT * D, VBYTES = D * RBV;
    static constexpr int KNS = D / 16, VNS = RBV / 16;   // 16-byte slots per K row and per V^T row
};

// Copies key tile [kbase, kbase + KT) of K (rows permuted: key kappa -> row 16 t + 4 G + i
// with kappa = G KQ + 4 t + i) and of V^T straight from global memory into LDS with
// buffer_load_dwordx4 ... lds: lane i of a wave fills bytes [16 i, 16 i + 16) of a 1 KB
// piece. The buffer resources end at the last valid byte of the (b, kv head) slices, so
// rows past the end read as zeros (their scores are masked) and can never fault.
//
// Wave w fills pieces 4 u + w. Piece 4 u + w starts 4096 u / D rows (K) and 4096 u / RBV
// rows (V^T) after piece w, a whole number of swizzle periods, so a lane's slot is the same
// in every piece and its source offset moves by a wave-uniform amount: the per-lane part
// is computed once (dma_lane_offsets) and a tile costs one add per piece.
template <int D, int KT, bool FP8>
struct DmaOffsets {
    int k, v;   // byte offsets of this lane's 16 bytes of piece w, relative to tile 0
};

template <int D, int KT, bool FP8>
__device__ __forceinline__ DmaOffsets<D, KT, FP8> dma_lane_offsets(int kst, int vrow, int w, int lane) {
    using C = Cfg<D, KT, FP8>;
    static_assert((4096 / D) % 16 == 0, "K pieces must advance by whole swizzle periods");
    static_assert((4096 / C::RBV) % 16 == 0, "V pieces must advance by whole swizzle periods");
    DmaOffsets<D, KT, FP8> r;
    {
        const int o = 1024 * w + 16 * lane;
        const int row = o / D, ls = swz<C::KNS>(row, (o % D) / 16);
        const int key = ((row & 15) >> 2) * C::KQ + 4 * (row >> 4) + (row & 3);
        r.k = key * kst + ls * 16;
    }
    {
        const int o = 1024 * w + 16 * lane;
        const int row = o / C::RBV, ls = swz<C::VNS>(row, (o % C::RBV) / 16);
        r.v = row * vrow + ls * 16;
    }
    return r;
}

template <int D, int KT, bool FP8>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int kst, int vrow,
                                         int kbase, uint8_t* kl, uint8_t* vl, int w, DmaOffsets<D, KT, FP8> off) {
    using C = Cfg<D, KT, FP8>;
    constexpr int KCH = C::KBYTES / 1024, VCH = C::VBYTES / 1024;
    static_assert(KCH % 4 == 0 && VCH % 4 == 0, "every wave fills the same number of pieces");
    // wave-uniform offsets recomputed per tile (scalar adds) rather than hoisted out of the
    // key loop, where they would crowd the scalar registers into spilling
    asm volatile("" : "+s"(w), "+s"(kst), "+s"(vrow));
    // piece 4 u + w of K: keys advance by (4096 u / D rows) / 16 rows per 4 keys
    const int kb = kbase * kst;
#pragma unroll
    for (int u = 0; u < KCH / 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lvoid_t*)(kl + 1024 * (4 * u + w)), 16,
                                                 off.k + kb + (u * (4096 / D) / 4) * kst, 0, 0, 0);
    const int vb = kbase * C::VB;
#pragma unroll
    for (int u = 0; u < VCH / 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lvoid_t*)(vl + 1024 * (4 * u + w)), 16,
                                                 off.v + vb + (u * (4096 / C::RBV)) * vrow, 0, 0, 0);
}


template <int D, int KT, bool FP8>
struct WaveState {
    using C = Cfg<D, KT, FP8>;
    v4i qop[C::NQ][C::NC];
    float qsc[C::NQ];
    float m_run[C::NQ], l_run[C::NQ];
    v4f o[C::NQ][C::NCT];
};

typedef float v4f_t __attribute__((ext_vector_type(4)));

// Key scales of the KQ keys [kg0, kg0 + KQ) of one lane group, by k-scale group q: THREAD_K
// keeps 4 scales per 64 keys, key t in group (t >> 1) & 3; PER_BLOCK one per 32, 64 or 128
// keys (KQ <= 32 keys never straddle a block). Past the last scale the buffer load gives 0.
__device__ __forceinline__ v4f_t load_kscales(__amdgpu_buffer_rsrc_t r, int kg0, int layout, int shift) {
    if (layout == SQ_LAYOUT_THREAD_K) {
        return __builtin_bit_cast(v4f_t, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (kg0 >> 6), 0, 0));
    } else {
        const float s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 4 * (kg0 >> shift), 0, 0));
        return v4f_t{s, s, s, s};
    }
}

// One key tile: S^T = K Q^T on INT8 MFMA, online softmax in base 2, acc += P V.
// ks: this lane group's key scales for the tile (load_kscales).
// TAIL: keys are masked per query, key kappa of query qi kept iff kappa < min(Sk, qend0 + qi - q0)
// with qend0 the key end of the wave's first query (Sk when not causal).
template <int D, int KT, bool FP8, bool TAIL>
__device__ __forceinline__ void tile_step(const AttnArgs& a, WaveState<D, KT, FP8>& st, const uint8_t* k_lds,
                                          const uint8_t* v_lds, int kbase, v4f_t ks, int lq, int g, int qend0) {
    using C = Cfg<D, KT, FP8>;
    // c = RN(qs ks) per k-scale group of this lane group's keys (times score_scale: exact for 1)
    const int kg0 = kbase + C::KQ * g;
    float cg[C::NQ][4];
#pragma unroll
    for (int n = 0; n < C::NQ; ++n)
#pragma unroll
        for (int q = 0; q < 4; ++q) cg[n][q] = (st.qsc[n] * ks[q]) * a.score_scale;

    // per 16-query tile n: S^T = K Q^T (int32), then the online softmax and its P operand.
    // Only one tile's scores are live; K is read from LDS again for the second tile.
    v8i pf8[C::NQ];
    v8bf pbf[C::NQ][KT / 32];
    float alpha[C::NQ];
    int lane = 16 * g + lq;
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        // fresh lane offsets per tile n: without them the first tile's K operand reads would
        // be kept in registers for the second
        asm volatile("" : "+v"(lane));
        const int klq = lane & 15, kg = lane >> 4;
        v4i s[C::NT];
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
#pragma unroll
            for (int ch = 0; ch < C::NC; ++ch) {
                const int row = 16 * t + klq;
                const v4i kop = *reinterpret_cast<const v4i*>(k_lds + row * D + swz<C::KNS>(row, 4 * ch + kg) * 16);
                s[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, st.qop[n][ch], ch == 0 ? v4i{0, 0, 0, 0} : s[t], 0, 0, 0);
            }
        }
        // keys of this lane group in the tile that this lane's query sees (all KQ but in the last
        // tile and, causal, the diagonal ones); opaque so that the masks are not computed once
        // before the key loop and kept (64 scalar registers of lane masks)
        int nval = min(static_cast<int>(a.Sk), qend0 + 16 * n + lq) - kg0;
        if (TAIL) asm volatile("" : "+v"(nval));
        int amx[4] = {INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN};
#pragma unroll
        for (int t = 0; t < C::NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (TAIL && 4 * t + i >= nval) s[t][i] = INT32_MIN;
                const int q = 2 * (t & 1) + (i >> 1);
                amx[q] = max(amx[q], s[t][i]);
            }
        float mt = -__builtin_inff();
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float mq = static_cast<float>(amx[q]) * cg[n][q];
            if (!TAIL || amx[q] != INT32_MIN) mt = fmaxf(mt, mq);
        }
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const float mo = st.m_run[n];
        const float mn = fmaxf(mo, mt);
        alpha[n] = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        st.m_run[n] = mn;
        float lsum = 0.0f;
#pragma unroll
        for (int t = 0; t < C::NT; ++t) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int q = 2 * (t & 1) + (i >> 1);
                const int av = s[t][i];
                float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(static_cast<float>(av), cg[n][q], -mn));
                if (TAIL && av == INT32_MIN) pv = 0.0f;
                p[i] = pv;
                lsum += pv;
            }
            if constexpr (FP8) {
                pf8[n][t] = pack_fp8x4_256(p[0], p[1], p[2], p[3]);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) pbf[n][t >> 1][4 * (t & 1) + i] = static_cast<__bf16>(p[i]);
            }
        }
        st.l_run[n] = st.l_run[n] * alpha[n] + lsum;
    }

    // Rescale the accumulator rows (query 4 g + i of tile n) by alpha. Unconditional: alpha is
    // exactly 1 where no max moved, and a branch around the product makes the compiler keep a
    // second copy of the accumulator (register moves every tile, spills).
#pragma unroll
    for (int n = 0; n < C::NQ; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float ai = __shfl(alpha[n], 4 * g + i, kWave);
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct) st.o[n][ct][i] *= ai;
        }

    // acc += Pt Vt
#pragma unroll
    for (int ct = 0; ct < C::NCT; ++ct) {
        const int row = ct * 16 + lq;
        if constexpr (FP8) {
            const v4i lo = *reinterpret_cast<const v4i*>(v_lds + row * C::RBV + swz<C::VNS>(row, 2 * g) * 16);
            const v4i hi = *reinterpret_cast<const v4i*>(v_lds + row * C::RBV + swz<C::VNS>(row, 2 * g + 1) * 16);
            const v8i vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
            for (int n = 0; n < C::NQ; ++n)
                st.o[n][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pf8[n], vop, st.o[n][ct], 0, 0, 0, 0, 0, 0);
        } else {
#pragma unroll
            for (int u = 0; u < KT / 32; ++u) {
                const int ls = (C::KQ * g + 8 * u) / 8;       // 16-byte slot of keys KQ g + 8 u .. + 7
                const v8bf vop = *reinterpret_cast<const v8bf*>(v_lds + row * C::RBV + swz<C::VNS>(row, ls) * 16);
#pragma unroll
                for (int n = 0; n < C::NQ; ++n)
                    st.o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pbf[n][u], vop, st.o[n][ct], 0, 0, 0);
            }
        }
    }
}


template <int D, int KT, bool FP8>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
    using C = Cfg<D, KT, FP8>;
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[C::KBYTES + C::VBYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[C::KBYTES + C::VBYTES];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lq = l & 15, g = l >> 4;
    const int64_t nqb = (a.Sq + C::QPB - 1) / C::QPB;
    const int64_t items = nqb * a.H * a.B;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    // causal: the last query blocks see the most keys and are dealt first
    const int64_t qb = a.causal ? nqb - 1 - item % nqb : item % nqb, h = (item / nqb) % a.H, b = item / (nqb * a.H);
    const int64_t hk = h / (a.H / a.Hk);
    const int64_t q0 = qb * C::QPB + w * (C::NQ * 16);

    // a sink starts the running max at its logit (base 2) and the sum at 1, counted once: in lane
    // group 0, whose sum the epilogue adds to the other three
    const float m0 = a.sinks ? a.sinks[h] * 1.44269504f : -__builtin_inff();
    const float l0 = (a.sinks && g == 0) ? 1.0f : 0.0f;
    WaveState<D, KT, FP8> st;
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        const int64_t qi = q0 + n * 16 + lq;
        const bool ok = qi < a.Sq;
#pragma unroll
        for (int ch = 0; ch < C::NC; ++ch) {
            v4i z = {0, 0, 0, 0};
            st.qop[n][ch] = ok ? *reinterpret_cast<const v4i*>(a.q + b * a.qsb + qi * a.qst + h * a.qsh + ch * 64 + 16 * g) : z;
        }
        st.qsc[n] = ok ? a.qs[b * a.qssb + h * a.qssh + scale_idx(qi, a.q_layout, a.q_block)] : 0.0f;
        st.m_run[n] = m0;
        st.l_run[n] = l0;
#pragma unroll
        for (int ct = 0; ct < C::NCT; ++ct) st.o[n][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }

    // what the epilogue needs, folded to a few values before the key loop (fewer live scalars)
    const int64_t obase = b * a.ob + h * a.oh;   // element offset of (b, h) in out
    const bool obf = a.out_bf16 != 0;
    const int64_t ot = a.ot;
    float* const lbase = a.lse ? a.lse + b * a.lb + h * a.lh : nullptr;
    const float* const vsbase = FP8 ? a.vscale + b * a.vssb + hk * a.vssh : nullptr;
    const int q0i = static_cast<int>(q0), Sq = static_cast<int>(a.Sq);

    const int8_t* kb = a.k + b * a.ksb + hk * a.ksh;
    const uint8_t* vb = static_cast<const uint8_t*>(a.v) + (b * a.vsb + hk * a.vsh) * C::VB;
    const float* ksp = a.ks + b * a.kssb + hk * a.kssh;
    const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ksp), 0, 4 * a.k_nscale, 0x00020000);
    const int kl_layout = a.k_layout, kl_shift = a.k_shift;
    // Causal: query i sits at key position i + Sk - Sq and sees keys up to it. The workgroup
    // reads the key tiles its last query sees; a wave masks the tiles past its first query's
    // end (lo_end) and skips those past its last query's end (hi_end).
    const int Sk = static_cast<int>(a.Sk), off = Sk - Sq;
    const int kv_end = a.causal ? min(Sk, static_cast<int>(min(a.Sq, qb * C::QPB + C::QPB)) + off) : Sk;
    const int ntiles = (kv_end + KT - 1) / KT;
    const int qend0 = a.causal ? q0i + off + 1 : Sk;
    const int lo_end = min(Sk, qend0), hi_end = a.causal ? min(Sk, q0i + C::NQ * 16 + off) : Sk;
    const int kst = static_cast<int>(a.kst), vrow = static_cast<int>(a.vsd) * C::VB;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(kb), 0, static_cast<int>((a.Sk - 1) * a.kst + D), 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vb), 0, D * vrow, 0x00020000);
    const DmaOffsets<D, KT, FP8> doff = dma_lane_offsets<D, KT, FP8>(kst, vrow, w, l);
    // tile j streams into buffer j % 2 while tile j - 1 is processed from the other one
    auto copy = [&](int j, uint8_t* buf) { dma_tile<D, KT, FP8>(krs, vrs, kst, vrow, j * KT, buf, buf + C::KBYTES, w, doff); };
    // the key scales of tile j + 1 are fetched (before its K/V copy) while tile j is
    // processed, so no wait on them ever waits for a copy in flight
    auto kscales = [&](int j) { return load_kscales(ksr, j * KT + C::KQ * g, kl_layout, kl_shift); };
    auto step = [&](int j, const uint8_t* buf, v4f_t ks) {
        const int kbase = j * KT;
        if (kbase >= hi_end) return;  // no query of the wave sees the tile: its state is unchanged
        if (kbase + KT > lo_end) tile_step<D, KT, FP8, true>(a, st, buf, buf + C::KBYTES, kbase, ks, lq, g, qend0);
        else tile_step<D, KT, FP8, false>(a, st, buf, buf + C::KBYTES, kbase, ks, lq, g, qend0);
    };
    v4f_t ks_next = kscales(0);
    copy(0, buf0);
    wait_vm();
    __syncthreads();
    for (int j = 0; j < ntiles; j += 2) {
        v4f_t ks_cur = ks_next;
        if (j + 1 < ntiles) {
            ks_next = kscales(j + 1);
            copy(j + 1, buf1);
        }
        step(j, buf0, ks_cur);
        wait_vm();
        __syncthreads();
        if (j + 1 >= ntiles) break;
        ks_cur = ks_next;
        if (j + 2 < ntiles) {
            ks_next = kscales(j + 2);
            copy(j + 2, buf0);
        }
        step(j + 1, buf1, ks_cur);
        wait_vm();
        __syncthreads();
    }

    // epilogue: l over the 4 lane groups, lse, out = acc / l (x vs / 256)
#pragma unroll
    for (int n = 0; n < C::NQ; ++n) {
        float lt = st.l_run[n];
        lt = lt + shfl_xor(lt, 16);
        lt = lt + shfl_xor(lt, 32);
        const int qi = q0i + n * 16 + lq;
        if (lbase && g == 0 && qi < Sq) lbase[qi] = st.m_run[n] + log2f(lt);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float li = __shfl(lt, 4 * g + i, kWave);
            const float inv = 1.0f / li;
            const int qr = q0i + n * 16 + 4 * g + i;
            if (qr >= Sq) continue;
            const int64_t orow = obase + qr * ot;
#pragma unroll
            for (int ct = 0; ct < C::NCT; ++ct) {
                const int c = ct * 16 + lq;
                float val = st.o[n][ct][i] * inv;
                if constexpr (FP8) val = val * (vsbase[c] * 0.00390625f);
                store_out(a.out, orow + c, val, obf);
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
    const int64_t items = (a.Sq + 127) / 128 * a.H * a.B;
    dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
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
