// Paged, GQA-stacked decode over a q8 KV cache on gfx950.
//
// Method: [impl] fastkernels L2/attention_impl.py (_cache_seq: block-table gather,
// _sdpa_one / _decode_torch: one query at position L - 1 attends positions 0..L-1,
// _repeat_kv_for_heads: q head h reads kv head h / (Hq / Hk)); [tq] vLLM
// triton_turboquant_unified_attention.py (GQA heads stacked on one pass over a kv
// head's pages; the 3D kernel's split over KV segments, merged afterwards by the
// segments' max and exp-sum); [kit] WanGP shared/attention_kit.py (q8: int8 per
// token, head and 32 channels with one FP16 scale).
//
// The path is bound by HBM: per cached token and kv head 2 x D code bytes + 2 x D/16
// scale bytes (D = 64 or 128). One workgroup (4 waves) owns one segment of kDecodeSeg positions of
// one (sequence, kv head) and serves all Hq / Hk query heads from a single read of
// the segment's K and V; each wave takes 64 positions (4 pages). Both contractions run
// on the f16 matrix cores (f32 accumulation), the query heads padded to 16 rows:
//  * Q.K: K rows are read whole (16 bytes a lane), put through the wave's LDS rows into the B
//    operand layout (8 channels of one position per lane) and widened exactly to f16 (byte
//    permute + packed f16 subtract);
//    q (bf16 or f16) is f16 after an exact power-of-two
//    rescale per head (the head's largest |q| lands in [2^14, 2^15), so no bf16 value
//    overflows); one MFMA per 32-channel q8 group, whose dot then meets its FP16 key scale
//    in FP32. Scores (log2 units) go to LDS.
//  * P.V: p = 2^(s - M) against the segment max M (no rescaling in the loop); the value
//    scale is folded into the weight, P' = f16(p * vs * 2^e) per 32-channel group, with 2^e
//    per wave putting the wave's largest value scale in [2^14, 2^15) (small values would
//    otherwise give weights in f16's subnormal range) and undone exactly on the FP32
//    accumulator; V codes are staged in LDS and read back transposed (ds_read_b64_tr_b8:
//    8 positions of one channel per lane), widened exactly to f16.
//  * every load of a wave is issued up front and unconditionally (no per-lane guard, which
//    would make each load wait for the one before).
//  * the partial (acc, M, l) of each (query head, segment) goes to the workspace;
//    k_decode_reduce merges the segments of a query by their maxima.
// Positions whose block-table entry is outside [0, num_blocks) are skipped: their rows are
// read from block 0 instead (never from the bad entry), their scores are -inf and their
// value scales zero, so a bad table cannot fault the device; with no blocks at all nothing
// is read and the output is 0.
#include <atomic>

#include "device.h"
#include "sq_internal.h"

// Segment partials of sq_paged_decode_noalloc: one array on every GPU the library runs on,
// held until the process ends. In host code this name is a host-side stand-in, never a device
// address: host code uses only the address decode_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[SQ_DECODE_SCRATCH_BYTES];

namespace sq {
namespace {

constexpr int kSeg = kDecodeSeg;
constexpr int kTpw = kSeg / 4;  // positions per wave
static_assert(kTpw == 64, "a wave takes 4 pages");

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

// The NG = D / 32 FP16 group scales of one cache row (8 or 4 bytes).
template <int D>
__device__ __forceinline__ uint2 load_scale_row(const uint16_t* p) {
    if constexpr (D == 128) return *reinterpret_cast<const uint2*>(p);
    else return make_uint2(*reinterpret_cast<const uint32_t*>(p), 0u);
}

template <int G, int D>
__global__ __launch_bounds__(256, 3) void k_decode_split(DecodeArgs a) {
    constexpr int NG = D / 32;        // q8 channel groups (and MFMAs per score)
    constexpr int NCT = D / 16;       // 16-channel output tiles of P.V
    constexpr int NV = D / 16;        // 16-byte V loads per lane (64 rows of D bytes per wave)
    constexpr int RPL = 1024 / D;     // V rows per load
    __shared__ __attribute__((aligned(16))) float sc[G][kSeg];             // scores [head][position]
    __shared__ __attribute__((aligned(1024))) uint8_t vst[4][kTpw * D];    // each wave's V rows; then its partial acc
    __shared__ __attribute__((aligned(16))) float4 vsf[4][kTpw];           // their scales as FP32 (NG per row)
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, j = l >> 4, lc = l & 15;
    // The Hk workgroups of one (sequence, segment) run back to back on one XCD (workgroup i
    // goes to XCD i % 8), so each cache slot's rows and scale rows (all heads side by side in
    // NHD) are fetched from HBM once into that XCD's L2; the (sequence, segment) pairs are
    // dealt round-robin over the XCDs, which keeps their loads even.
    const int xcd = blockIdx.x & 7, k = blockIdx.x >> 3;
    const int64_t chunk = 8 * static_cast<int64_t>(k / a.Hk) + xcd;
    if (chunk >= static_cast<int64_t>(a.segs) * a.N) return;  // uniform over the workgroup
    const int hk = k % a.Hk;
    const int seg = static_cast<int>(chunk % a.segs);
    const int n = static_cast<int>(chunk / a.segs);
    const int L = a.num_blocks > 0 ? min(a.lens[n], a.max_len) : 0;   // empty cache: no position is readable
    const int s0 = seg * kSeg;
    if (s0 >= L) return;  // uniform over the workgroup
    const int s1 = min(L, s0 + kSeg);
    const int wp0 = s0 + w * kTpw;        // first position of this wave (a multiple of 16)
    const int32_t* bt = a.bt + static_cast<int64_t>(n) * a.bt_stride;

    // the physical block of each of the wave's 4 pages (one table read per page; -1 if unused or invalid)
    int myblk = -1;
    if (l < 4 && wp0 + 16 * l < s1) {
        const int b = bt[(wp0 >> 4) + l];
        myblk = (b >= 0 && b < a.num_blocks) ? b : -1;
    }
    int64_t rowbase[4];
#pragma unroll
    for (int pg = 0; pg < 4; ++pg) {
        const int b = __builtin_amdgcn_readlane(myblk, pg);
        rowbase[pg] = b < 0 ? -1 : static_cast<int64_t>(b) * 16 * a.Hk + hk;   // row of slot 0, this kv head
    }

    // ---- all loads of the wave go out first, q and K (needed first) before V, so the scores
    // can start while the values are still in flight. Register loads only: a use of a register
    // load while an LDS copy (global_load_lds) is in flight waits for everything outstanding.
    // Like every load here they are unconditional (a lane-dependent guard around each load
    // makes it wait for the one before): a page outside the table reads block 0's rows instead,
    // positions past the end read their page's unused slots; all of them get score -inf and
    // value scale 0.
    uint4 qraw[NG];
    {
        const uint16_t* qp = a.q + static_cast<int64_t>(n) * a.qn + static_cast<int64_t>(hk * G + min(lc, G - 1)) * a.qh;
#pragma unroll
        for (int g = 0; g < NG; ++g) qraw[g] = *reinterpret_cast<const uint4*>(qp + 32 * g + 8 * j);
    }
    // K and V rows, whole rows per load (16 bytes a lane, NV lanes a row: a load touches only full
    // rows, which sustains a higher read rate than the 32-byte pieces of the MFMA operand layout):
    // load r holds rows RPL r .. RPL r + RPL - 1 (lane l: row RPL r + l / NV, bytes 16 (l % NV)). K goes
    // through the wave's LDS rows into the operand layout; V follows it there once the scores are done.
    // The key scales of position 16 t + lc go to lane (j, lc); the value scales of row l to lane l.
    uint4 kraw[NV], vraw[NV];
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const int row = RPL * r + l / NV;           // wave-local row: page row / 16, slot row % 16
        const int64_t rb = rowbase[row >> 4] >= 0 ? rowbase[row >> 4] : hk;
        kraw[r] = *reinterpret_cast<const uint4*>(a.kc + (rb + static_cast<int64_t>(row & 15) * a.Hk) * D + 16 * (l % NV));
    }
    uint2 ksr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t row = (rowbase[t] >= 0 ? rowbase[t] : hk) + static_cast<int64_t>(lc) * a.Hk;
        ksr[t] = load_scale_row<D>(a.ks + row * NG);
    }
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const int row = RPL * r + l / NV;
        const int64_t rb = rowbase[row >> 4] >= 0 ? rowbase[row >> 4] : hk;
        vraw[r] = *reinterpret_cast<const uint4*>(a.vc + (rb + static_cast<int64_t>(row & 15) * a.Hk) * D + 16 * (l % NV));
    }
    uint2 vsr;
    {
        const int64_t rb0 = rowbase[l >> 4];
        const int64_t rb = rb0 >= 0 ? rb0 : hk;
        vsr = load_scale_row<D>(a.vs + (rb + static_cast<int64_t>(l & 15) * a.Hk) * NG);
    }
    // ---- q of head m = lc (zero rows for m >= G): channels 32 g + 8 j .. + 7 as f16, times
    // 2^sh with sh per head putting its largest |q| in [2^14, 2^15)
    v8h qa[NG];
    int sh = 0;
    {
        float f[NG][8];
        float mx = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (a.q_f16) unpack_f16x8(qraw[g], f[g]);
            else unpack_bf16x8(qraw[g], f[g]);
#pragma unroll
            for (int k = 0; k < 8; ++k) mx = fmaxf(mx, fabsf(f[g][k]));
        }
        mx = swap32_max(swap16_max(mx));
        sh = mx > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(mx) + 1 : 0;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int k = 0; k < 8; ++k)
                qa[g][k] = lc < G ? static_cast<_Float16>(__builtin_amdgcn_ldexpf(f[g][k], sh)) : static_cast<_Float16>(0.0f);
    }

    // ---- K rows to this wave's LDS rows: 16-byte chunk c of row rho at slot c ^ (rho mod NV), so that the
    // operand reads below (16 rows, one chunk each) spread over the banks
#pragma unroll
    for (int r = 0; r < NV; ++r) {
        const int row = RPL * r + l / NV;
        *reinterpret_cast<uint4*>(vst[w] + row * D + 16 * ((l % NV) ^ (row & (NV - 1)))) = kraw[r];
    }

    // ---- pass 1: scores of the wave's 64 positions. Lane (j, lc) produces heads 4 j + i; their
    // score scale softmax_scale * log2 e * 2^-sh (a power-of-two change of a float: exact)
    float scl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) scl[i] = __builtin_amdgcn_ldexpf(a.scale, -__shfl(sh, min(4 * j + i, 15), kWave));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // lane (j, lc): position 16 t + lc, channels 32 g + 8 j .. + 7 of each group g (chunk 2 g + j / 2)
        const int krow = 16 * t + lc;
        v4f dg[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint2 kv = *reinterpret_cast<const uint2*>(vst[w] + krow * D + 16 * ((2 * g + (j >> 1)) ^ (krow & (NV - 1))) +
                                                             8 * (j & 1));
            dg[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[g], i8x8_to_f16(kv.x, kv.y), v4f{0.0f, 0.0f, 0.0f, 0.0f},
                                                          0, 0, 0);
        }
        // lane (j, lc) now holds heads 4 j + i of position 16 t + lc
        const int pos = wp0 + 16 * t + lc;
        const bool ok = rowbase[t] >= 0 && pos < s1;
        const float ks[4] = {f16_to_f32(ksr[t].x & 0xffff), f16_to_f32(ksr[t].x >> 16), f16_to_f32(ksr[t].y & 0xffff),
                             f16_to_f32(ksr[t].y >> 16)};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int h = 4 * j + i;
            float sv = dg[0][i] * ks[0];
#pragma unroll
            for (int g = 1; g < NG; ++g) sv = __builtin_fmaf(dg[g][i], ks[g], sv);
            sv = sv * scl[i];
            if (h < G) sc[h][w * kTpw + 16 * t + lc] = ok ? sv : -__builtin_inff();
        }
    }
    // this wave's V rows (over its K rows, which the scores have been read from) and value scales to
    // LDS (scales zero on rows past the end of the sequence or on an unread page)
#pragma unroll
    for (int r = 0; r < NV; ++r) *reinterpret_cast<uint4*>(vst[w] + 1024 * r + 16 * l) = vraw[r];
    // value scales times 2^esh: the wave's largest |scale| lands in [2^14, 2^15), so the f16 weights
    // p vs 2^esh <= 2^15 stay normal for the keys that matter; o is multiplied by 2^-esh after the loop
    int esh = 0;
    {
        const bool okv = rowbase[l >> 4] >= 0 && wp0 + l < s1;
        const h2 s01 = __builtin_bit_cast(h2, vsr.x), s23 = __builtin_bit_cast(h2, vsr.y);
        // (D = 64: two scales; the other two lanes of the float4 are 0 and never read)
        float4 sf = okv ? make_float4(static_cast<float>(s01[0]), static_cast<float>(s01[1]), static_cast<float>(s23[0]),
                                      static_cast<float>(s23[1]))
                        : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float mx = fmaxf(fmaxf(fabsf(sf.x), fabsf(sf.y)), fmaxf(fabsf(sf.z), fabsf(sf.w)));
        mx = wave_max(mx);
        esh = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
        sf.x = __builtin_amdgcn_ldexpf(sf.x, esh);
        sf.y = __builtin_amdgcn_ldexpf(sf.y, esh);
        sf.z = __builtin_amdgcn_ldexpf(sf.z, esh);
        sf.w = __builtin_amdgcn_ldexpf(sf.w, esh);
        vsf[w][l] = sf;
    }
    __syncthreads();

    // ---- segment max per query head, by every wave over all 256 positions (no exchange)
    float M[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = fmaxf(fmaxf(sc[h][l], sc[h][64 + l]), fmaxf(sc[h][128 + l], sc[h][192 + l]));
        m = wave_max(m);
        M[h] = m;
    }

    // ---- pass 2: p = 2^(s - M), acc += f16(p vs) . v
    float Mm = -__builtin_inff();
#pragma unroll
    for (int h = 0; h < G; ++h)
        if (lc == h) Mm = M[h];
    const bool live = lc < G && Mm > -__builtin_inff();
    v4f o[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) o[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float lsum = 0.0f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int r0 = 32 * u + 8 * j;             // first of this lane's 8 positions (wave-local)
        float p[8];
        if (live) {
            const float4 a0 = *reinterpret_cast<const float4*>(&sc[min(lc, G - 1)][w * kTpw + r0]);
            const float4 a1 = *reinterpret_cast<const float4*>(&sc[min(lc, G - 1)][w * kTpw + r0 + 4]);
            const float sv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) p[k] = __builtin_amdgcn_exp2f(sv[k] - Mm);
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) p[k] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) lsum += p[k];
        // weights per group: P'_g[k] = f16(p[k] * vs[k][g])
        v8h pw[NG];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float4 sf = vsf[w][r0 + k];
            pw[0][k] = static_cast<_Float16>(p[k] * sf.x);
            pw[1][k] = static_cast<_Float16>(p[k] * sf.y);
            if constexpr (NG == 4) {
                pw[NG - 2][k] = static_cast<_Float16>(p[k] * sf.z);
                pw[NG - 1][k] = static_cast<_Float16>(p[k] * sf.w);
            }
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            // lanes 2 k and 2 k + 1 of the group give row r0 + k's channels 16 ct .. + 7 and + 8 .. + 15;
            // lane lc receives channel 16 ct + lc of the 8 rows
            typedef __attribute__((address_space(3))) v2i* lv2p;
            const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lv2p)(vst[w] + (r0 + (lc >> 1)) * D + 16 * ct + 8 * (lc & 1)));
            o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pw[ct >> 1], i8x8_to_f16(raw[0], raw[1]), o[ct], 0, 0, 0);
        }
    }
    lsum = swap32_add(swap16_add(lsum));
    // undo the value-scale factor (exact: a power of two on FP32)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ct][i] = __builtin_amdgcn_ldexpf(o[ct][i], -esh);

    // ---- the 4 waves' partials (same max) summed; lane (j, lc) of o[ct] holds heads 4 j + i, channel 16 ct + lc
    float* red = reinterpret_cast<float*>(vst[w]);   // this wave's own rows: read by nobody else
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * j + i < G) red[(4 * j + i) * D + 16 * ct + lc] = o[ct][i];
    // this wave's exp-sums in its own (now unused) scale rows
    float* lred = reinterpret_cast<float*>(vsf[w]);
    if (j == 0 && lc < G) lred[lc] = lsum;
    __syncthreads();
    // partial of head h: acc (D), max, exp-sum at part[((n Hq + hk G + h) segs + seg) (D + 2)]
    const int64_t hstride = static_cast<int64_t>(a.segs) * (D + 2);
    float* prow = a.part + (static_cast<int64_t>(n) * a.Hq + hk * G) * hstride + static_cast<int64_t>(seg) * (D + 2);
    const float* r0 = reinterpret_cast<const float*>(vst[0]);
    const float* r1 = reinterpret_cast<const float*>(vst[1]);
    const float* r2 = reinterpret_cast<const float*>(vst[2]);
    const float* r3 = reinterpret_cast<const float*>(vst[3]);
#pragma unroll
    for (int idx = tid; idx < G * D; idx += 256)   // element h D + c of the wave rows: head h, channel c
        prow[(idx / D) * hstride + idx % D] = (r0[idx] + r1[idx]) + (r2[idx] + r3[idx]);
    if (tid < G) {
        float mh = M[0];
#pragma unroll
        for (int q = 1; q < G; ++q)
            if (q == tid) mh = M[q];
        const float* l0 = reinterpret_cast<const float*>(vsf[0]);
        const float* l1 = reinterpret_cast<const float*>(vsf[1]);
        const float* l2 = reinterpret_cast<const float*>(vsf[2]);
        const float* l3 = reinterpret_cast<const float*>(vsf[3]);
        prow[tid * hstride + D] = mh;
        prow[tid * hstride + D + 1] = (l0[tid] + l1[tid]) + (l2[tid] + l3[tid]);
    }
}

// Merge the segments of one (sequence, query head): weights 2^(M_s - max M). Thread c
// owns channel c; the segments' maxima and weights are computed 128 at a time, one
// segment per thread, and shared through LDS; each channel's weighted sum then reads
// its partials 8 loads at a time.
template <int D>
__global__ __launch_bounds__(D) void k_decode_reduce(DecodeArgs a) {
    constexpr int SB = D, NL = 8;
    __shared__ float wl[2][SB];  // per segment of the pass: weight, exp-sum
    __shared__ float red[D / 64];
    const int c = threadIdx.x, hq = blockIdx.x, n = blockIdx.y;
    const int L = a.num_blocks > 0 ? min(a.lens[n], a.max_len) : 0;
    const int nseg = L > 0 ? (L + kSeg - 1) / kSeg : 0;
    const float* p = a.part + (static_cast<int64_t>(n) * a.Hq + hq) * a.segs * (D + 2);
    float mg = -__builtin_inff();
    for (int s = c; s < nseg; s += SB) mg = fmaxf(mg, p[s * (D + 2) + D]);
    mg = wave_max(mg);
    if ((c & 63) == 0) red[c >> 6] = mg;
    __syncthreads();
    // a sink joins as one more term of the denominator, at its logit in base 2
    const float sk = a.sinks ? a.sinks[hq] * 1.44269504f : -__builtin_inff();
    mg = fmaxf(fmaxf(red[0], red[D / 64 - 1]), sk);
    float tot = 0.0f, o = 0.0f;
    if (mg > -__builtin_inff()) {  // uniform over the workgroup
        if (sk > -__builtin_inff()) tot = __builtin_amdgcn_exp2f(sk - mg);
        for (int s0 = 0; s0 < nseg; s0 += SB) {
            const int s = s0 + c;
            float wgt = 0.0f, ls = 0.0f;
            if (s < nseg) {
                const float ms = p[s * (D + 2) + D];
                wgt = ms > -__builtin_inff() ? __builtin_amdgcn_exp2f(ms - mg) : 0.0f;
                ls = p[s * (D + 2) + D + 1];
            }
            __syncthreads();  // the previous pass has finished reading wl
            wl[0][c] = wgt;
            wl[1][c] = ls;
            __syncthreads();
            const int ns = min(SB, nseg - s0);
            for (int j0 = 0; j0 < ns; j0 += NL) {
                float v[NL];
#pragma unroll
                for (int j = 0; j < NL; ++j) v[j] = p[(s0 + min(j0 + j, ns - 1)) * (D + 2) + c];
#pragma unroll
                for (int j = 0; j < NL; ++j)
                    if (j0 + j < ns) {
                        tot = __builtin_fmaf(wl[0][j0 + j], wl[1][j0 + j], tot);
                        o = __builtin_fmaf(wl[0][j0 + j], v[j], o);
                    }
            }
        }
    }
    store_out(a.out, static_cast<int64_t>(n) * a.on + static_cast<int64_t>(hq) * a.oh + c, tot > 0.0f ? o / tot : 0.0f,
              a.out_bf16 != 0);
}

inline hipStream_t S(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address of scratch per device id (null: not looked up)
}  // namespace

int decode_scratch(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_paged_decode_noalloc: hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SQ_ERR_UNSUPPORTED, "sq_paged_decode_noalloc: device %d (at most %d devices)", dev, kMaxDevices);
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // with this device current: each GPU holds its own copy of the array at its own address
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(SQ_ERR_HIP, "sq_paged_decode_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
                        hipGetErrorString(e));
        g_scratch[dev].store(p, std::memory_order_release);   // racing first calls store the same address
    }
    *ptr = p;
    return SQ_OK;
}

namespace {
template <int D>
void launch_decode_d(const DecodeArgs& a, hipStream_t s) {
    const int64_t chunks = static_cast<int64_t>(a.segs) * a.N;      // (sequence, segment) pairs
    dim3 g1(static_cast<unsigned>((chunks + 7) / 8 * 8 * a.Hk));
    switch (a.Hq / a.Hk) {
    case 1: SQ_LAUNCH((k_decode_split<1, D>), g1, dim3(256), 0, s, a); break;
    case 2: SQ_LAUNCH((k_decode_split<2, D>), g1, dim3(256), 0, s, a); break;
    case 4: SQ_LAUNCH((k_decode_split<4, D>), g1, dim3(256), 0, s, a); break;
    default: SQ_LAUNCH((k_decode_split<8, D>), g1, dim3(256), 0, s, a); break;
    }
    SQ_LAUNCH(k_decode_reduce<D>, dim3(static_cast<unsigned>(a.Hq), static_cast<unsigned>(a.N)), dim3(D), 0, s,
                       a);
}
}  // namespace

int launch_decode(const DecodeArgs& a, void* stream) {
    if (a.N == 0) return SQ_OK;
    if (a.D == 128) launch_decode_d<128>(a, S(stream));
    else launch_decode_d<64>(a, S(stream));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_paged_decode: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
