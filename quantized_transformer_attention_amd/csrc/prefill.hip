// Paged causal prefill over a q8 KV cache on gfx950: varlen query chunks attend their
// sequence's cached keys (the context) and their own, causally, GQA heads stacked.
//
// Method: [impl] fastkernels L2/attention_impl.py _prefill_torch_from_cache (per sequence:
// _cache_seq gathers the keys through the block table, _sdpa_one masks k_pos <= key_offset +
// q_pos with key_offset = k_len - q_len), laid out as [tq] vLLM
// triton_turboquant_unified_attention.py kernel_tq_unified_attention_2d lays it out: q
// blocks of the packed tokens found by _find_seq_idx's binary search over query_start_len,
// the Hq / Hk query heads of a kv head stacked into one block of rows, context_len =
// seq_len - query_len, online softmax, sinks (USE_SINKS: M = sink logit, L = 1).
//
// Design (one workgroup = NW waves = 32 NW rows = 32 NW / G tokens x G heads of one kv head;
// 64-key tiles = 4 pages; head dim D = 64 or 128):
//  * K and V tiles are staged once per workgroup, key-major in LDS (2 D bytes per key, 16-byte
//    slots XOR-swizzled): K as its int8 codes widened exactly to f16, with its FP16 group
//    scales as FP32 beside them; V as an exact pair of f16 values per element, hi = f16(code
//    vs) and lo = code vs - hi (one fused multiply-add: the remainder fits in f16), so that
//    neither K nor V is rounded. The next tile's codes and scales are loaded into registers
//    while the current tile is processed; the block-table entries of the tile after it are
//    read (scalar) one step earlier still.
//  * q (bf16 or f16) is carried as f16 after an exact power-of-two rescale per row (its largest |q| in
//    [2^14, 2^15)), undone exactly in the row's score scale.
//  * S^T = K Q^T on v_mfma_f32_16x16x32_f16, one product per 32-channel q8 group (exact
//    f16 products, FP32 sums) meeting its key scale in FP32: s = sum_g dot_g ks_g. K rows are
//    permuted in LDS (key kappa = 16 G + 4 t + i to row 16 t + 4 G + i) so that lane group g
//    ends up holding the 16 consecutive keys [16 g, 16 g + 16) of one query row: those
//    registers, as f16, are the A operand of P.V, whose B operands (8 keys of one channel per
//    lane, hi and lo) are read from the key-major V tiles by transposing ds_read_b64_tr_b16.
//  * the softmax denominator is accumulated by the same matrix units from the same f16 P: one
//    more P.V product against a column of ones, so out = acc / l is a weighted mean whose
//    weights are exactly the P that multiplied the values (a one-key row returns its value).
//  * causal: a workgroup reads the tiles up to its last row's end; a wave masks only the
//    tiles that cross its rows' diagonal and skips those past its last row.
//  * the reference max of a row trails its running max by at most 8 (base 2): the
//    accumulator is rescaled only when a tile raises some row's max beyond that, so p <= 2^8
//    (the f16 P rounds relative to itself whatever the reference; l and acc are FP32).
// HBM: each (sequence, kv head) key/value row is read by every q block of the sequence
// that sees it; the q blocks of one kv head are dealt to one XCD in a row, so most of
// those reads hit its L2.
#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

constexpr int kBS = 16, kKT = 64;
constexpr float kLag = 8.0f;                // how far a row's reference max may trail its max
constexpr int kNQ = 2, kNT = kKT / 16;

// LDS tile geometry of head dim D: per key one f16 row of D channels (NS 16-byte slots) in each of
// K, V hi and V lo, then the keys' FP32 group scales.
template <int D>
struct PfTile {
    static constexpr int kNC = D / 32, kNCT = D / 16, NS = D / 8;
    static constexpr int kRowB = 2 * D;
    static constexpr int kTileB = kKT * kRowB;                                  // 16 KB at D = 128
    static constexpr int kVHi = kTileB, kVLo = 2 * kTileB, kKs = 3 * kTileB;   // K codes, V hi, V lo, K scales
    static constexpr int kBufB = 3 * kTileB + kKT * kNC * 4;
    static constexpr int KPW = kWave * 16 / D;                                  // keys a wave stages per pass
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lv4s_p;

// LDS row of key kappa in the K tile, and the 16-byte slot swizzles (NS slots per row): K is read as
// 16 rows x one slot per lane group (row mod NS spreads the rows over the banks); V as 16 keys
// 16 g + 8 u + 4 h + k (k, g = 0..3) x two slots, spread by k | g << 2 (D = 128) or k | (g & 1) << 2.
__device__ __forceinline__ int k_row(int kappa) { return 16 * ((kappa >> 2) & 3) + 4 * (kappa >> 4) + (kappa & 3); }
template <int D>
__device__ __forceinline__ int k_slot(int row, int slot) { return slot ^ (row & (D / 8 - 1)); }
template <int D>
__device__ __forceinline__ int v_slot(int key, int slot) { return slot ^ ((key & 3) | ((key >> 2) & (D / 8 - 4))); }

// x s as an exact pair: hi = f16(x s), lo = x s - hi (x an integer code, s an f16 scale: the product
// has at most 18 significant bits, so the remainder of its f16 rounding is an f16 number)
__device__ __forceinline__ void scale8_pair(v8h x, _Float16 s, v8h& hi, v8h& lo) {
    const v8h sv = {s, s, s, s, s, s, s, s};
    hi = x * sv;
    lo = __builtin_elementwise_fma(x, sv, -hi);
}

template <int G, int NW, int D>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_paged_prefill(PrefillArgs a) {
    using C = PfTile<D>;
    constexpr int kNC = C::kNC, kNCT = C::kNCT, kRowB = C::kRowB, kBufB = C::kBufB;
    constexpr int kVHi = C::kVHi, kVLo = C::kVLo, kKs = C::kKs;
    constexpr int kRows = 32 * NW;                      // rows per workgroup
    constexpr int BQ = kRows / G;                       // query tokens per workgroup
    // 16-byte K (and V) chunks per thread and tile; with more stagers than chunks the waves past
    // the tile's keys stage nothing
    constexpr int U = kKT / (NW * C::KPW) > 0 ? kKT / (NW * C::KPW) : 1;
    static_assert(U * NW * C::KPW >= kKT, "every key of a tile has a stager");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kBufB];
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, lq = l & 15, g = l >> 4;

    // ---- work item: (kv head, q block); the q blocks of a kv head run on one XCD, last first
    const int64_t items = a.nqb * a.Hk;
    const int64_t item = xcd_item(blockIdx.x, (items + 7) / 8);
    if (item >= items) return;  // uniform over the workgroup
    const int hk = static_cast<int>(item / a.nqb);
    const int qblk = static_cast<int>(a.nqb - 1 - item % a.nqb);
    // the sequence whose q blocks hold qblk: sequence n's first block is query_start[n] / BQ + n
    int lo = 0, hi = a.N;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a.qstart[mid] / BQ + mid <= qblk) lo = mid + 1;
        else hi = mid;
    }
    const int seq = lo - 1;
    if (seq < 0) return;
    const int qs0 = a.qstart[seq], qlen = a.qstart[seq + 1] - qs0;
    const int local = qblk - (qs0 / BQ + seq);
    if (local * BQ >= qlen) return;
    const int L = min(a.lens[seq], a.max_len);
    const int ctx = L - qlen;                           // keys before the first query
    const int j0 = local * BQ;                          // first query (in the sequence) of the block
    const int kv_end = min(L, ctx + min(qlen, j0 + BQ));
    const int ntiles = (kv_end + kKT - 1) / kKT;
    if (ntiles <= 0) return;
    // this wave's rows are tokens j0 + 32 w / G .. j0 + (32 w + 31) / G
    const int lo_end = min(L, ctx + j0 + (32 * w) / G + 1);
    const int hi_end = min(L, ctx + j0 + (32 * w + 31) / G + 1);
    // the block table is read through the constant address space: its wave-uniform reads become scalar
    // loads, whose counter is not the one the code loads are waited on with
    typedef __attribute__((address_space(4))) const int32_t cint32;
    const cint32* bt = reinterpret_cast<const cint32*>(reinterpret_cast<uintptr_t>(a.bt + static_cast<int64_t>(seq) * a.bt_stride));
    const int last_page = (L - 1) / kBS;

    // ---- q rows: row r = 32 w + 16 n + lq is token r / G, head r % G; per-row power-of-two rescale
    v8h qop[kNQ][kNC];
    float cr[kNQ], m_run[kNQ];
    v4f o[kNQ][kNCT], ol[kNQ];   // ol: the denominators of the rows o holds (P against a column of ones)
#pragma unroll
    for (int n = 0; n < kNQ; ++n) {
        const int r = 32 * w + 16 * n + lq;
        const int j = j0 + r / G, h = hk * G + r % G;
        const bool ok = j < qlen && qs0 + j >= 0 && qs0 + j < a.T;
        v4u raw[kNC];
        const uint16_t* qp = a.q + static_cast<int64_t>(qs0 + (ok ? j : 0)) * a.qt + static_cast<int64_t>(h) * a.qh;
#pragma unroll
        for (int c = 0; c < kNC; ++c)
            raw[c] = ok ? *reinterpret_cast<const v4u*>(qp + 32 * c + 8 * g) : v4u{0u, 0u, 0u, 0u};
        float f[kNC][8];
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < kNC; ++c) {
            const uint4 rc = make_uint4(raw[c][0], raw[c][1], raw[c][2], raw[c][3]);
            if (a.q_f16) unpack_f16x8(rc, f[c]);
            else unpack_bf16x8(rc, f[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[c][e]));
        }
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const int sh = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
        for (int c = 0; c < kNC; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) qop[n][c][e] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(f[c][e], sh));
        cr[n] = __builtin_amdgcn_ldexpf(a.scale, -sh);
        m_run[n] = a.sinks ? a.sinks[h] * 1.44269504f : -__builtin_inff();
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct) o[n][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        // a sink is one more term 2^(sink - m) = 1 of every row's denominator (its head is a.sinks' index of
        // row 4 g + i, whose sink starts its running max)
        const float l0 = a.sinks ? 1.0f : 0.0f;
        ol[n] = v4f{l0, l0, l0, l0};
    }

    // ---- staging: thread tid takes 16 channels (part) of keys kappa_u = tid / (D / 16) + NW KPW u of a
    // tile; the pages of those keys are wave-uniform: tile page (KPW w + NW KPW u) / 16
    constexpr int PARTS = D / 16;
    const int part = tid % PARTS, key0 = tid / PARTS;
    const bool stager = C::KPW * w < kKT;               // wave-uniform
    const int64_t rowstride = a.Hk;                     // cache rows per slot
    auto page_block = [&](int tile, int u) {
        const int tp = stager ? (C::KPW * w + NW * C::KPW * u) / kBS : 0;
        const int page = __builtin_amdgcn_readfirstlane(min(tile * (kKT / kBS) + tp, last_page));
        const int b = bt[page];
        return (b >= 0 && b < a.num_blocks) ? b : 0;    // a bad entry reads block 0 (no fault)
    };
    v4u kraw[U], vraw[U];
    uint32_t ksr[U], vsr[U];
    auto load_tile = [&](const int* blk) {
        if (!stager) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t row = (static_cast<int64_t>(blk[u]) * kBS + ((key0 + NW * C::KPW * u) & 15)) * rowstride + hk;
            kraw[u] = *reinterpret_cast<const v4u*>(a.kc + row * D + 16 * part);
            vraw[u] = *reinterpret_cast<const v4u*>(a.vc + row * D + 16 * part);
            ksr[u] = a.ks[row * kNC + (part >> 1)];
            vsr[u] = a.vs[row * kNC + (part >> 1)];
        }
    };
    // keys at or past L (unused slots, clamped pages) get zero scales: their scores are masked and their
    // values must not carry a NaN or inf of memory nobody wrote into the P.V sums
    auto store_tile = [&](uint8_t* buf, int kbase) {
        if (!stager) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kappa = key0 + NW * C::KPW * u;
            const bool live = kbase + kappa < L;
            const float ks = live ? f16_to_f32(static_cast<uint16_t>(ksr[u])) : 0.0f;
            const _Float16 vs = live ? __builtin_bit_cast(_Float16, static_cast<uint16_t>(vsr[u])) : static_cast<_Float16>(0.0f);
            const v4u kr4 = kraw[u], vr4 = vraw[u];
            const v8h k0 = i8x8_to_f16(kr4[0], kr4[1]), k1 = i8x8_to_f16(kr4[2], kr4[3]);
            v8h vh0, vl0, vh1, vl1;
            scale8_pair(i8x8_to_f16(vr4[0], vr4[1]), vs, vh0, vl0);
            scale8_pair(i8x8_to_f16(vr4[2], vr4[3]), vs, vh1, vl1);
            const int kr = k_row(kappa);
            *reinterpret_cast<v8h*>(buf + kr * kRowB + k_slot<D>(kr, 2 * part) * 16) = k0;
            *reinterpret_cast<v8h*>(buf + kr * kRowB + k_slot<D>(kr, 2 * part + 1) * 16) = k1;
            // the scale of group part / 2 of key kappa (both threads of the group hold it; the even one stores)
            if ((part & 1) == 0) reinterpret_cast<float*>(buf + kKs)[kappa * kNC + (part >> 1)] = ks;
            *reinterpret_cast<v8h*>(buf + kVHi + kappa * kRowB + v_slot<D>(kappa, 2 * part) * 16) = vh0;
            *reinterpret_cast<v8h*>(buf + kVHi + kappa * kRowB + v_slot<D>(kappa, 2 * part + 1) * 16) = vh1;
            *reinterpret_cast<v8h*>(buf + kVLo + kappa * kRowB + v_slot<D>(kappa, 2 * part) * 16) = vl0;
            *reinterpret_cast<v8h*>(buf + kVLo + kappa * kRowB + v_slot<D>(kappa, 2 * part + 1) * 16) = vl1;
        }
    };

    // one tile: S^T = K Q^T, online softmax (base 2), acc += P V
    auto tile_step = [&](const uint8_t* buf, int kbase, bool masked) {
        v8h pf[kNQ][2];
        int lane = l;
#pragma unroll
        for (int n = 0; n < kNQ; ++n) {
            // fresh lane offsets per n: the first tile's K reads are not kept in registers for the second
            asm volatile("" : "+v"(lane));
            const int klq = lane & 15, kg = lane >> 4;
            const float* ksc = reinterpret_cast<const float*>(buf + kKs);   // [key][kNC] group scales
            v4f s[kNT];
#pragma unroll
            for (int t = 0; t < kNT; ++t) {
                const int row = 16 * t + klq;
                v4f dg[kNC];
#pragma unroll
                for (int c = 0; c < kNC; ++c) {
                    const v8h kop = *reinterpret_cast<const v8h*>(buf + row * kRowB + k_slot<D>(row, 4 * c + kg) * 16);
                    dg[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[n][c], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                }
                // element i is key 16 kg + 4 t + i: its group dots meet its group scales in FP32
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float* kq = ksc + (16 * kg + 4 * t + i) * kNC;
                    float kv[kNC];
                    if constexpr (kNC == 4) {
                        const float4 k4 = *reinterpret_cast<const float4*>(kq);
                        kv[0] = k4.x; kv[1] = k4.y; kv[kNC - 2] = k4.z; kv[kNC - 1] = k4.w;
                    } else {
                        const float2 k2 = *reinterpret_cast<const float2*>(kq);
                        kv[0] = k2.x; kv[1] = k2.y;
                    }
                    float sv = dg[0][i] * kv[0];
#pragma unroll
                    for (int c = 1; c < kNC; ++c) sv = __builtin_fmaf(dg[c][i], kv[c], sv);
                    s[t][i] = sv;
                }
            }
            if (masked) {
                // keys of this lane group (16 g + 4 t + i) this row sees: below min(L, ctx + j + 1)
                const int r = 32 * w + 16 * n + lq;
                int nval = min(L, ctx + j0 + r / G + 1) - kbase - 16 * g;
                asm volatile("" : "+v"(nval));
#pragma unroll
                for (int t = 0; t < kNT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (4 * t + i >= nval) s[t][i] = -__builtin_inff();
            }
            float mt = -__builtin_inff();
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) mt = fmaxf(mt, s[t][i]);
            mt = fmaxf(mt, shfl_xor(mt, 16));
            mt = fmaxf(mt, shfl_xor(mt, 32));
            const float ms = mt * cr[n];
            // the reference max moves (and the accumulator rows with it) only when some row of the
            // wave would see p > 2^kLag against it
            if (__builtin_amdgcn_ballot_w64(ms > m_run[n] + kLag) != 0) {
                const float mo = m_run[n];
                const float mn = fmaxf(mo, ms);
                const float alpha = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
                m_run[n] = mn;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * g + i, kWave);
#pragma unroll
                    for (int ct = 0; ct < kNCT; ++ct) o[n][ct][i] *= ai;
                    ol[n][i] *= ai;
                }
            }
            // every row sees key 0 in the first tile, so mref is finite from there on and a masked
            // score (-inf) gives p = 2^-inf = 0 exactly
            const float mref = m_run[n];
#pragma unroll
            for (int t = 0; t < kNT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], cr[n], -mref));
                    pf[n][t >> 1][4 * (t & 1) + i] = static_cast<_Float16>(p);
                }
        }
        // acc += P V: B operand = keys 16 g + 8 u + 4 h + k (k = lq / 4) of channels 16 ct + 4 (lq % 4) ..
        // + 3, transposed so that lane lq receives channel 16 ct + lq of those 4 keys
        auto vop_of = [&](const uint8_t* vt, int ct, int u) {
            v4h half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int key = 16 * g + 8 * u + 4 * h + (lq >> 2), m = lq & 3;
                const uint8_t* p = vt + key * kRowB + v_slot<D>(key, 2 * ct + (m >> 1)) * 16 + 8 * (m & 1);
                half[h] = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s_p)(p)));
            }
            return v8h{half[0][0], half[0][1], half[0][2], half[0][3], half[1][0], half[1][1], half[1][2], half[1][3]};
        };
#pragma unroll
        for (int ct = 0; ct < kNCT; ++ct)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const v8h vhi = vop_of(buf + kVHi, ct, u), vlo = vop_of(buf + kVLo, ct, u);
#pragma unroll
                for (int n = 0; n < kNQ; ++n) {
                    o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[n][u], vhi, o[n][ct], 0, 0, 0);
                    o[n][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[n][u], vlo, o[n][ct], 0, 0, 0);
                }
            }
        const _Float16 one = static_cast<_Float16>(1.0f);
        const v8h ones = {one, one, one, one, one, one, one, one};
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int n = 0; n < kNQ; ++n) ol[n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[n][u], ones, ol[n], 0, 0, 0);
    };

    // ---- key loop: tile j is processed from buffer j % 2 while tile j + 1's codes are in flight;
    // the table entries of tile j + 2 are read meanwhile
    int nb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) nb[u] = page_block(0, u);
    load_tile(nb);
#pragma unroll
    for (int u = 0; u < U; ++u) nb[u] = page_block(min(1, ntiles - 1), u);
    store_tile(lds, 0);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        uint8_t* cur = lds + (j & 1) * kBufB;
        uint8_t* nxt = lds + ((j + 1) & 1) * kBufB;
        load_tile(nb);                                  // tile j + 1 (the last tile again past the end)
        const int t2 = min(j + 2, ntiles - 1);
#pragma unroll
        for (int u = 0; u < U; ++u) nb[u] = page_block(t2, u);
        __builtin_amdgcn_sched_barrier(0);              // the loads go out before the tile's arithmetic
        const int kbase = j * kKT;
        if (kbase < hi_end) tile_step(cur, kbase, kbase + kKT > lo_end);
        store_tile(nxt, (j + 1) * kKT);
        __syncthreads();
    }

    // ---- epilogue: out = acc / l (l of row 4 g + i is in every lane of group g)
#pragma unroll
    for (int n = 0; n < kNQ; ++n) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float inv = 1.0f / ol[n][i];
            const int r = 32 * w + 16 * n + 4 * g + i;
            const int j = j0 + r / G;
            if (j >= qlen || qs0 + j < 0 || qs0 + j >= a.T) continue;
            const int64_t orow = static_cast<int64_t>(qs0 + j) * a.ot + static_cast<int64_t>(hk * G + r % G) * a.oh;
#pragma unroll
            for (int ct = 0; ct < kNCT; ++ct) store_out(a.out, orow + 16 * ct + lq, o[n][ct][i] * inv, a.out_bf16 != 0);
        }
    }
}

}  // namespace

namespace {
template <int D>
void launch_prefill_d(const PrefillArgs& a, dim3 grid, hipStream_t s) {
    const dim3 block(64 * kPrefillWaves);
    switch (a.Hq / a.Hk) {
        case 1: SQ_LAUNCH((k_paged_prefill<1, kPrefillWaves, D>), grid, block, 0, s, a); break;
        case 2: SQ_LAUNCH((k_paged_prefill<2, kPrefillWaves, D>), grid, block, 0, s, a); break;
        case 4: SQ_LAUNCH((k_paged_prefill<4, kPrefillWaves, D>), grid, block, 0, s, a); break;
        default: SQ_LAUNCH((k_paged_prefill<8, kPrefillWaves, D>), grid, block, 0, s, a); break;
    }
}
}  // namespace

int launch_prefill(const PrefillArgs& a, void* stream) {
    const int64_t items = a.nqb * a.Hk;
    if (items == 0) return SQ_OK;
    dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (a.D == 128) launch_prefill_d<128>(a, grid, s);
    else launch_prefill_d<64>(a, grid, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "sq_paged_prefill: kernel launch failed: %s", hipGetErrorString(e));
    return SQ_OK;
}

}  // namespace sq
