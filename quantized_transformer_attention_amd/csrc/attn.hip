// Quantized attention core on gfx950: INT8 Q.K^T on MFMA, FP32 online softmax in
// base 2, P.V on FP8 or bf16 MFMA.
//
// Method: the staged quantized core of [kit] WanGP shared/attention_kit.py
// (q/k INT8 with block scales, v FP8 or 16-bit) and the online softmax of [tq] vLLM
// triton_turboquant_unified_attention.py (kernel_tq_unified_attention_2d: m_j, P,
// l_j, alpha, acc). [impl] _repeat_kv_for_heads fixes the GQA head mapping.
//
// Design (one workgroup = 4 waves = 128 queries of one (b, h), 32 per wave; K and V^T
// tiles of KT keys staged once in LDS by DMA and shared by the 4 waves):
//  * S^T = K Q^T with v_mfma_i32_32x32x32_i8: the 32x32 result puts one query per lane
//    (lane % 32) and 16 keys of each 32-key block per lane, the two halves of the wave
//    (lane / 32) holding different keys, so a row max or sum is in-lane plus one step
//    across the halves.
//  * O^T = V^T P^T (channels x queries) with v_mfma_scale_f32_32x32x64_f8f6f4 (FP8) or
//    v_mfma_f32_32x32x16_bf16: the B operand P^T is, per lane, a run of consecutive keys
//    of that lane's query -- K rows are permuted into LDS so that the S^T registers of a
//    lane are exactly those keys, in order, in runs of 8 consecutive keys -- and the A
//    operand V^T is a run of keys of one channel, which is why V is read channel-major
//    (sq_quant_v_fp8 writes FP8 V that way; bf16 V is staged channel-major by
//    k_v_transpose). The output rows of a query stay in its own lane, so rescaling them
//    needs no exchange, and it is skipped when no row max of the wave moved (alpha = 1).
//  * The softmax max is taken on the int32 dots per k-scale group (c > 0 makes
//    RN(a c) monotonic in a), and p = 2^fma(a, c, -m') uses the hardware exp2.
//  * FP8 P.V: Pt = e4m3(256 p) by a scaled convert (2^-8 scale: exact).
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
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
    static constexpr int QPB = 4 * 32;               // queries per workgroup: 4 waves of 32
    static constexpr int NB = KT / 32;               // 32-key blocks of S^T
    static constexpr int NCS = D / 32;               // 32-channel steps of Q.K^T (and blocks of O^T)
    static constexpr int NCH = KT / 64 > 0 ? KT / 64 : 1;   // 64-key chunks (THREAD_K scale blocks)
    static constexpr int VB = FP8 ? 1 : 2;           // bytes per V element
    static constexpr int RBV = KT * VB;              // bytes of one V^T row (one channel)
    static constexpr int KBYTES = KT * D, VBYTES = D * RBV;
    static constexpr int KNS = D / 16, VNS = RBV / 16;   // 16-byte slots per K row and per V^T row
    // score groups sharing one c: FP8 (64-key chunk, k-scale group q); bf16 (32-key block, q)
    static constexpr int NG = FP8 ? 4 * NCH : 4 * NB;
};

// The k-scale group of output register 4 j + i (any block): THREAD_K group (key mod 8) / 2.
__host__ __device__ constexpr int kgroup(int j, int i) { return 2 * (j & 1) + (i >> 1); }

// Copies key tile [kbase, kbase + KT) of K (rows permuted as kappa_of_row) and of V^T straight
// from global memory into LDS with buffer_load_dwordx4 ... lds: lane i of a wave fills bytes
// [16 i, 16 i + 16) of a 1 KB piece. The buffer resources end at the last valid byte of the
// (b, kv head) slices, so rows past the end read as zeros (their scores are masked) and can
// never fault.
//
// Wave w fills pieces 4 u + w. Piece 4 u + w starts 4096 u / D rows (K) and 4096 u / RBV rows
// (V^T) after piece w, a whole number of swizzle periods and of 32-key blocks, so a lane's slot
// is the same in every piece and its source key moves by kappa_of_row(4096 u / D), a constant:
// the per-lane part is computed once (dma_lane_offsets) and a tile costs one add per piece.
template <int D, int KT, bool FP8>
struct DmaOffsets {
    int k, v;   // byte offsets of this lane's 16 bytes of piece w, relative to tile 0
};

template <int D, int KT, bool FP8>
__device__ __forceinline__ DmaOffsets<D, KT, FP8> dma_lane_offsets(int kst, int vrow, int w, int lane) {
    using C = Cfg<D, KT, FP8>;
    static_assert((4096 / D) % 32 == 0, "K pieces must advance by whole blocks and swizzle periods");
    static_assert((4096 / C::RBV) % 16 == 0, "V pieces must advance by whole swizzle periods");
    DmaOffsets<D, KT, FP8> r;
    {
        const int o = 1024 * w + 16 * lane;
        const int row = o / D, ls = swz<C::KNS>(row, (o % D) / 16);
        r.k = kappa_of_row<FP8>(row) * kst + ls * 16;
    }
    {
        const int o = 1024 * w + 16 * lane;
        const int row = o / C::RBV, ls = swz<C::VNS>(row, (o % C::RBV) / 16);
        r.v = row * vrow + ls * 16;
    }
    return r;
}

// (TK, SS: the kernel's key-scale layout and score-scale flag, unused here; a specialization per kernel
// keeps the host pass from sharing one across kernels, which it rejects)
template <int D, int KT, bool FP8, bool TK, bool SS>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int kst, int vrow,
                                         int kbase, uint8_t* kl, uint8_t* vl, int w, DmaOffsets<D, KT, FP8> off) {
    using C = Cfg<D, KT, FP8>;
    constexpr int KCH = C::KBYTES / 1024, VCH = C::VBYTES / 1024;
    static_assert(KCH % 4 == 0 && VCH % 4 == 0, "every wave fills the same number of pieces");
    // wave-uniform offsets recomputed per tile (scalar adds) rather than hoisted out of the
    // key loop, where they would crowd the scalar registers into spilling
    asm volatile("" : "+s"(w), "+s"(kst), "+s"(vrow));
    const int kb = kbase * kst;
#pragma unroll
    for (int u = 0; u < KCH / 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lvoid_t*)(kl + 1024 * (4 * u + w)), 16,
                                                 off.k + kb + kappa_of_row<FP8>(u * (4096 / D)) * kst, 0, 0, 0);
    const int vb = kbase * C::VB;
#pragma unroll
    for (int u = 0; u < VCH / 4; ++u)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lvoid_t*)(vl + 1024 * (4 * u + w)), 16,
                                                 off.v + vb + (u * (4096 / C::RBV)) * vrow, 0, 0, 0);
}

// The key scales a lane needs for one tile, raw (FP32): THREAD_K (TK) the 4 scales of each 64-key
// chunk (key t in group (t >> 1) & 3); PER_BLOCK the scale of each 32-key block b at [b >> 1][b & 1]
// (its keys never straddle a scale block for this lane half). Past the last scale the buffer
// load gives 0.
template <int D, int KT, bool FP8>
struct KScales {
    v4f c[Cfg<D, KT, FP8>::NCH];
};

// (SS: one specialization per kernel, as for dma_tile)
template <int D, int KT, bool FP8, bool TK, bool SS>
__device__ __forceinline__ KScales<D, KT, FP8> load_kscales(__amdgpu_buffer_rsrc_t r, int kbase, int h, int shift) {
    using C = Cfg<D, KT, FP8>;
    KScales<D, KT, FP8> k;
    if constexpr (TK) {
#pragma unroll
        for (int ch = 0; ch < C::NCH; ++ch)
            k.c[ch] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * ((kbase >> 6) + ch), 0, 0));
    } else {
#pragma unroll
        for (int b = 0; b < C::NB; ++b) {
            // the lowest key of this lane half in block b: its 32-key run lies in one scale block
            const int kmin = kbase + (FP8 ? 64 * (b >> 1) + 32 * h + 16 * (b & 1) : 32 * b + 8 * h);
            k.c[b >> 1][b & 1] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 4 * (kmin >> shift), 0, 0));
        }
    }
    return k;
}

template <int D, int KT, bool FP8>
struct WaveState {
    using C = Cfg<D, KT, FP8>;
    v4i qop[C::NCS];          // B operand of S^T: this lane's query, channels 32 c + 16 h .. + 15
    float qsc;
    float m_run, l_run;
    v16f o[C::NCS];           // O^T: this lane's query, channels 32 cb + 8 j + 4 h + i
};

// One key tile: S^T = K Q^T on INT8 MFMA, online softmax in base 2, O^T += V^T P^T.
// TAIL: keys are masked per query, key kappa of query ql (lane % 32) kept iff kappa < min(Sk, qend0 +
// ql) - kbase with qend0 the key end of the wave's first query (Sk when not causal). It is a template
// argument: the key loop runs the tiles that need no mask and those that do in loops of their own,
// so the unmasked tiles carry no masking code (a run-time flag gets if-converted into per-key selects
// on every tile).
template <bool FP8, int NB, bool TAIL>
__device__ __forceinline__ void exp_pack(const v16i (&s)[NB], const float* cg, float mn, float& lsum,
                                         v8i* pf8, v8bf* pbf) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int gi = FP8 ? 4 * (b >> 1) + kgroup(j, i) : 4 * b + kgroup(j, i);
                const int av = s[b][4 * j + i];
                float x = __builtin_fmaf(static_cast<float>(av), cg[gi], -mn);
                if (TAIL && av == INT32_MIN) x = -__builtin_inff();   // a masked key: p = 0 exactly
                const float pv = __builtin_amdgcn_exp2f(x);
                p[i] = pv;
                if (b == 0 && j == 0 && i == 0) lsum = pv;   // the first term starts the sum (no 0 + p)
                else lsum += pv;
            }
            if constexpr (FP8) {
                // keys 64 (b >> 1) + 32 h + 16 (b & 1) + 4 j + i: dword 4 (b & 1) + j of chunk b >> 1
                pf8[b >> 1][4 * (b & 1) + j] = pack_fp8x4_256(p[0], p[1], p[2], p[3]);
            } else {
                // keys 32 b + 16 (j >> 1) + 8 h + 4 (j & 1) + i: elements 4 (j & 1) + i of step 2 b + (j >> 1)
#pragma unroll
                for (int i = 0; i < 4; ++i) pbf[2 * b + (j >> 1)][4 * (j & 1) + i] = static_cast<__bf16>(p[i]);
            }
        }
}

template <int D, int KT, bool FP8, bool TAIL, bool TK, bool SS>
__device__ __forceinline__ void tile_step(const AttnArgs& a, WaveState<D, KT, FP8>& st, const uint8_t* k_lds,
                                          const uint8_t* v_lds, int kbase, const KScales<D, KT, FP8>& ks, int ql,
                                          int h, int qend0) {
    using C = Cfg<D, KT, FP8>;
    // c = RN(qs ks) per score group, times score_scale when it is not 1 (SS)
    float cg[C::NG];
#pragma unroll
    for (int gi = 0; gi < C::NG; ++gi) {
        const int q = gi & 3, blk = gi >> 2;                  // FP8: blk = 64-key chunk; bf16: 32-key block
        const int ch = FP8 ? blk : blk >> 1;
        const float tk = ks.c[ch][q];
        const float pb = FP8 ? ks.c[ch][0] : ks.c[ch][blk & 1];
        cg[gi] = SS ? (st.qsc * (TK ? tk : pb)) * a.score_scale : st.qsc * (TK ? tk : pb);
    }

    // S^T of the tile: s[b][4 j + i] = dot of this lane's query with key kappa_of_row(32 b + 8 j + 4 h + i)
    v16i s[C::NB];
#pragma unroll
    for (int b = 0; b < C::NB; ++b) {
        const int row = 32 * b + ql;
#pragma unroll
        for (int c = 0; c < C::NCS; ++c) {
            const v4i kop = *reinterpret_cast<const v4i*>(k_lds + row * D + swz<C::KNS>(row, 2 * c + h) * 16);
            s[b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kop, st.qop[c], c == 0 ? v16i{} : s[b], 0, 0, 0);
        }
    }
    if constexpr (TAIL) {
        // keys this lane's query sees: local key < nval (a lane of half h holds the half-0 keys plus 32 h
        // (FP8 permutation) or 8 h (bf16)); opaque so that it is not computed once before the key loop
        int nval = min(static_cast<int>(a.Sk), qend0 + ql) - kbase - (FP8 ? 32 : 8) * h;
        asm volatile("" : "+v"(nval));
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kappa_of_row<FP8>(32 * b + 8 * (r >> 2) + (r & 3)) >= nval) s[b][r] = INT32_MIN;
    }
    // maxima per score group (int32), then scaled; a group with every key masked is left out
    float mt = -__builtin_inff();
#pragma unroll
    for (int gi = 0; gi < C::NG; ++gi) {
        const int q = gi & 3, blk = gi >> 2;
        int amx = INT32_MIN;
#pragma unroll
        for (int b = 0; b < C::NB; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int j = r >> 2, i = r & 3;
                if (kgroup(j, i) == q && (FP8 ? (b >> 1) == blk : b == blk)) amx = max(amx, s[b][r]);
            }
        const float mq = static_cast<float>(amx) * cg[gi];
        // only a masked tile can leave a group with no key (the int8 dots never reach INT32_MIN)
        mt = fmaxf(mt, !TAIL || amx != INT32_MIN ? mq : -__builtin_inff());
    }
    mt = swap32_max(mt);
    const float mo = st.m_run;
    const float mn = fmaxf(mo, mt);
    // alpha = 0 while m is -inf: exp2(-inf - m') is 0 when m' is finite, which every tile without
    // masked keys makes it; only a masked tile can leave m' at -inf (and -inf - -inf undefined)
    const float alpha = (TAIL && mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
    st.m_run = mn;

    // p = 2^(a c - m'), l += p, P^T operands
    float lsum = 0.0f;
    v8i pf8[C::NCH];
    v8bf pbf[KT / 16];
    exp_pack<FP8, C::NB, TAIL>(s, cg, mn, lsum, pf8, pbf);
    st.l_run = __builtin_fmaf(st.l_run, alpha, lsum);

    // Rescale the accumulator of this lane's query by alpha, unless no query of the wave moved its max
    // (alpha is then exactly 1 everywhere and the products would change nothing). The products are
    // written in place (a read-write operand), so both paths leave the accumulator in the same registers.
    if (__builtin_amdgcn_ballot_w64(mn != mo) != 0) {
#pragma unroll
        for (int cb = 0; cb < C::NCS; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) asm volatile("v_mul_f32 %0, %1, %0" : "+v"(st.o[cb][e]) : "v"(alpha));
    }

    // O^T += V^T P^T
#pragma unroll
    for (int cb = 0; cb < C::NCS; ++cb) {
        const int row = 32 * cb + ql;
        if constexpr (FP8) {
#pragma unroll
            for (int ch = 0; ch < C::NCH; ++ch) {
                const v4i lo = *reinterpret_cast<const v4i*>(v_lds + row * C::RBV + swz<C::VNS>(row, 4 * ch + 2 * h) * 16);
                const v4i hi = *reinterpret_cast<const v4i*>(v_lds + row * C::RBV + swz<C::VNS>(row, 4 * ch + 2 * h + 1) * 16);
                const v8i vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                st.o[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pf8[ch], st.o[cb], 0, 0, 0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < KT / 16; ++u) {
                const v8bf vop = *reinterpret_cast<const v8bf*>(v_lds + row * C::RBV + swz<C::VNS>(row, 2 * u + h) * 16);
                st.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pbf[u], st.o[cb], 0, 0, 0);
            }
        }
    }
}


template <int D, int KT, bool FP8, bool TK, bool SS>
__global__ __launch_bounds__(256, 2) void k_attn(AttnArgs a) {
    using C = Cfg<D, KT, FP8>;
    static_assert(!FP8 || KT % 64 == 0, "FP8 P.V takes 64 keys per product");
    __shared__ __attribute__((aligned(1024))) uint8_t buf0[C::KBYTES + C::VBYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t buf1[C::KBYTES + C::VBYTES];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, ql = l & 31, h = l >> 5;
    const int64_t nqb = (a.Sq + C::QPB - 1) / C::QPB;
    const int64_t items = nqb * a.H * a.B;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    // causal: the last query blocks see the most keys and are dealt first
    const int64_t qb = a.causal ? nqb - 1 - item % nqb : item % nqb, hh = (item / nqb) % a.H, b = item / (nqb * a.H);
    const int64_t hk = hh / (a.H / a.Hk);
    const int64_t q0 = qb * C::QPB + w * 32;

    WaveState<D, KT, FP8> st;
    {
        const int64_t qi = q0 + ql;
        const bool ok = qi < a.Sq;
#pragma unroll
        for (int c = 0; c < C::NCS; ++c) {
            const v4i z = {0, 0, 0, 0};
            st.qop[c] = ok ? *reinterpret_cast<const v4i*>(a.q + b * a.qsb + qi * a.qst + hh * a.qsh + 32 * c + 16 * h) : z;
        }
        st.qsc = ok ? a.qs[b * a.qssb + hh * a.qssh + scale_idx(qi, a.q_layout, a.q_block)] : 0.0f;
        // a sink starts the running max at its logit (base 2) and the sum at 1, counted once: in
        // lane half 0, whose sum the epilogue adds to the other half's
        st.m_run = a.sinks ? a.sinks[hh] * 1.44269504f : -__builtin_inff();
        st.l_run = (a.sinks && h == 0) ? 1.0f : 0.0f;
#pragma unroll
        for (int c = 0; c < C::NCS; ++c) st.o[c] = v16f{};
    }

    // what the epilogue needs, folded to a few values before the key loop (fewer live scalars)
    const int64_t obase = b * a.ob + hh * a.oh;   // element offset of (b, h) in out
    const bool obf = a.out_bf16 != 0;
    const int64_t ot = a.ot;
    float* const lbase = a.lse ? a.lse + b * a.lb + hh * a.lh : nullptr;
    const float* const vsbase = FP8 ? a.vscale + b * a.vssb + hk * a.vssh : nullptr;
    const int q0i = static_cast<int>(q0), Sq = static_cast<int>(a.Sq);

    const int8_t* kb = a.k + b * a.ksb + hk * a.ksh;
    const uint8_t* vb = static_cast<const uint8_t*>(a.v) + (b * a.vsb + hk * a.vsh) * C::VB;
    const float* ksp = a.ks + b * a.kssb + hk * a.kssh;
    const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(ksp), 0, 4 * a.k_nscale, 0x00020000);
    const int kl_shift = a.k_shift;
    // Causal: query i sits at key position i + Sk - Sq and sees keys up to it. The workgroup
    // reads the key tiles its last query sees; a wave masks the tiles past its first query's
    // end (lo_end) and skips those past its last query's end (hi_end).
    const int Sk = static_cast<int>(a.Sk), off = Sk - Sq;
    const int kv_end = a.causal ? min(Sk, static_cast<int>(min(a.Sq, qb * C::QPB + C::QPB)) + off) : Sk;
    const int ntiles = (kv_end + KT - 1) / KT;
    const int qend0 = a.causal ? q0i + off + 1 : Sk;
    const int lo_end = min(Sk, qend0), hi_end = a.causal ? min(Sk, q0i + 32 + off) : Sk;
    const int kst = static_cast<int>(a.kst), vrow = static_cast<int>(a.vsd) * C::VB;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(kb), 0, static_cast<int>((a.Sk - 1) * a.kst + D), 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(vb), 0, D * vrow, 0x00020000);
    const DmaOffsets<D, KT, FP8> doff = dma_lane_offsets<D, KT, FP8>(kst, vrow, w, l);
    // tile j streams into buffer j % 2 while tile j - 1 is processed from the other one
    auto copy = [&](int j, uint8_t* buf) { dma_tile<D, KT, FP8, TK, SS>(krs, vrs, kst, vrow, j * KT, buf, buf + C::KBYTES, w, doff); };
    // the key scales of tile j + 1 are fetched (before its K/V copy) while tile j is
    // processed, so no wait on them ever waits for a copy in flight
    auto kscales = [&](int j) { return load_kscales<D, KT, FP8, TK, SS>(ksr, j * KT, h, kl_shift); };
    KScales<D, KT, FP8> ks_next = kscales(0);
    copy(0, buf0);
    wait_vm();
    __syncthreads();
    // one tile per iteration, its buffer chosen at run time (wave-uniform): a loop body unrolled
    // per buffer would hold the accumulator in two register ranges and copy it between them
    auto body = [&](int j, auto tail_tag) {
        constexpr bool TAIL = decltype(tail_tag)::value;
        const bool odd = (j & 1) != 0;
        uint8_t* cur = odd ? buf1 : buf0;
        uint8_t* nxt = odd ? buf0 : buf1;
        const KScales<D, KT, FP8> ks_cur = ks_next;
        if (j + 1 < ntiles) {
            ks_next = kscales(j + 1);
            copy(j + 1, nxt);
        }
        // a tile past the wave's last query's key end leaves its state unchanged
        const int kbase = j * KT;
        if (!TAIL || kbase < hi_end)
            tile_step<D, KT, FP8, TAIL, TK, SS>(a, st, cur, cur + C::KBYTES, kbase, ks_cur, ql, h, qend0);
        wait_vm();
        __syncthreads();
    };
    // tiles [0, jm) end at or below the wave's first query's key end and need no mask; every wave
    // runs ntiles iterations (one barrier each) over the two loops
    const int jm = min(ntiles, lo_end / KT);
    for (int j = 0; j < jm; ++j) body(j, std::integral_constant<bool, false>{});
    for (int j = jm; j < ntiles; ++j) body(j, std::integral_constant<bool, true>{});

    // epilogue: l over the two lane halves, lse, out = acc / l (x vs / 256)
    float lt = st.l_run;
    lt = swap32_add(lt);
    const int qi = q0i + ql;
    if (lbase && h == 0 && qi < Sq) lbase[qi] = st.m_run + log2f(lt);
    if (qi < Sq) {
        const float inv = 1.0f / lt;
        const int64_t orow = obase + qi * ot;
#pragma unroll
        for (int cb = 0; cb < C::NCS; ++cb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = 32 * cb + 8 * j + 4 * h + i;
                    float val = st.o[cb][4 * j + i] * inv;
                    if constexpr (FP8) val = val * (vsbase[c] * 0.00390625f);
                    store_out(a.out, orow + c, val, obf);
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
    if (a.D == 128) SQ_LAUNCH(k_v_transpose<128>, grid, dim3(256), 0, S(stream), a);
    else SQ_LAUNCH(k_v_transpose<64>, grid, dim3(256), 0, S(stream), a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn: V staging launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

// k_attn<D, KT, FP8, TK, SS> for the run-time head dim, key tile, P.V type, key-scale layout and score
// scale (SS: not 1) (written out: a host template around the launches makes the host pass check the
// kernel bodies)
#define SQ_ATTN_LAUNCH_DK(FP8, TK, SS)                                                       \
    do {                                                                                     \
        if (a.kv_tile == 128) {                                                              \
            if (a.D == 128) SQ_LAUNCH((k_attn<128, 128, FP8, TK, SS>), grid, dim3(256), 0, s, a); \
            else SQ_LAUNCH((k_attn<64, 128, FP8, TK, SS>), grid, dim3(256), 0, s, a);        \
        } else {                                                                             \
            if (a.D == 128) SQ_LAUNCH((k_attn<128, 64, FP8, TK, SS>), grid, dim3(256), 0, s, a); \
            else SQ_LAUNCH((k_attn<64, 64, FP8, TK, SS>), grid, dim3(256), 0, s, a);         \
        }                                                                                    \
    } while (0)
#define SQ_ATTN_LAUNCH_SS(FP8, TK)                            \
    do {                                                      \
        if (a.score_scale != 1.0f) SQ_ATTN_LAUNCH_DK(FP8, TK, true); \
        else SQ_ATTN_LAUNCH_DK(FP8, TK, false);               \
    } while (0)

int launch_attn(const AttnArgs& a, void* stream) {
    if (a.B * a.Sq * a.H == 0) return SQ_OK;
    const int64_t items = (a.Sq + 127) / 128 * a.H * a.B;
    dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
    hipStream_t s = S(stream);
    const bool tk = a.k_layout == SQ_LAYOUT_THREAD_K;
    if (a.v_fp8) {
        if (tk) SQ_ATTN_LAUNCH_SS(true, true);
        else SQ_ATTN_LAUNCH_SS(true, false);
    } else {
        if (tk) SQ_ATTN_LAUNCH_SS(false, true);
        else SQ_ATTN_LAUNCH_SS(false, false);
    }
#undef SQ_ATTN_LAUNCH_SS
#undef SQ_ATTN_LAUNCH_DK
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_attn: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
