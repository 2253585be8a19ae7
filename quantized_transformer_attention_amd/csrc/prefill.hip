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
//  * K and V tiles are staged once per workgroup, key-major in LDS (16-byte slots
//    XOR-swizzled), each element first split into an exact pair of f16 values: hi =
//    f16(code scale) and lo = code scale - hi (one fused multiply-add; an int8 code times an
//    FP16 scale is a multiple of 2^-24 with at most 18 significant bits, so the remainder is
//    an f16 number, subnormal or not). V keeps both halves (not rounded). K keeps hi as f16
//    and lo as e4m3 of lo 2^-E with one power-of-two block scale 2^E per key and 32 channels
//    (E = exponent of the FP16 scale - 13: lo 2^-E is a multiple of 4 of at most 256, normal
//    in e4m3), so a key is off by at most 2^-4 |lo| <= 2^-16 |code scale|. The next tile's
//    codes and scales are loaded into registers while the current tile is processed; the
//    block-table entries of the tile after it are read (scalar) one step earlier still.
//  * q (bf16 or f16) is carried as f16 after an exact power-of-two rescale per row (its
//    largest |q| in [2^14, 2^15)), undone exactly in the row's score scale.
//  * S^T = K Q^T into one FP32 accumulator: the hi products on v_mfma_f32_32x32x16_f16, the
//    lo products on v_mfma_scale_f32_32x32x64_f8f6f4 (one per 64 channels, the keys' block
//    scales applied by the matrix unit) against an e4m3 copy of the rescaled q (q 2^-7, block
//    scale 2^7): one query row per lane (lane % 32), 16 keys of each 32-key block per lane,
//    the wave halves holding different keys. K rows are permuted in LDS (the 32x32
//    attention core's key order) so that a lane's score registers are, in order, runs of 8
//    consecutive keys: as f16 they are the B operand P^T of O^T = V^T P^T, whose A operand
//    (8 keys of one channel per lane, hi and lo) is read from the key-major V tile by
//    transposing ds_read_b64_tr_b16. A row's output channels stay in its lane.
//  * the softmax denominator sums the same f16 P that multiplied the values (dot2 against
//    ones, FP32), so out = acc / l is a weighted mean whose weights are exactly those P (a
//    one-key row returns its value).
//  * causal: a workgroup reads the tiles up to its last row's end; the tiles below its first
//    row's diagonal run in a loop without masking code, and from there on a wave masks the
//    tiles it sees and skips those past its last row.
//  * the reference max of a row trails its running max by at most 8 (base 2): the
//    accumulator is rescaled only when a tile raises some row's max beyond that, so p <= 2^8
//    (the f16 P rounds relative to itself whatever the reference; l and acc are FP32).
// HBM: each (sequence, kv head) key/value row is read by every q block of the sequence
// that sees it; the q blocks of one kv head are dealt to one XCD in a row, so most of
// those reads hit its L2.
#include <type_traits>

#include "device.h"
#include "sq_internal.h"

namespace sq {
namespace {

constexpr int kBS = 16, kKT = 64;
constexpr float kLag = 8.0f;                // how far a row's reference max may trail its max

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s* lv4s_p;

// LDS tile geometry of head dim D: per key one f16 row of D channels (NS 16-byte slots) in each of
// K hi, V hi and V lo; per key one row of D FP8 bytes (K lo, D / 16 16-byte slots) and 8 bytes of K lo
// block scales.
template <int D>
struct PfTile {
    static constexpr int NS = D / 8, NCS = D / 16, NCB = D / 32;   // slots per row, 16-channel steps, 32-channel blocks
    static constexpr int NCC = D / 64;                             // 64-channel steps of the FP8 products
    static constexpr int kRowB = 2 * D;
    static constexpr int kTileB = kKT * kRowB;                     // 16 KB at D = 128
    static constexpr int kKLo8 = kTileB;                           // K lo as FP8: kKT rows of D bytes
    static constexpr int kKE = kKLo8 + kKT * D;                    // K lo block scales: 8 bytes per row
    static constexpr int kVHi = (kKE + kKT * 8 + 1023) / 1024 * 1024, kVLo = kVHi + kTileB;
    static constexpr int kBufB = kVLo + kTileB;
    static constexpr int KPW = kWave * 16 / D;                     // keys a wave stages per pass
};

// The E8M0 block scale of the FP8 products' q operand: q (largest |q| in [2^14, 2^15)) goes to FP8 as
// q 2^-7, so its scale is 2^7.
constexpr int kQ8Exp = 7;

// LDS row of key kappa in the K tile: the inverse of kappa_of_row<false> (32-key blocks; within a
// block, row 8 j + 4 h + i holds key 16 (j >> 1) + 8 h + 4 (j & 1) + i).
__host__ __device__ constexpr int k_row(int kappa) {
    const int r = kappa & 31;
    return (kappa & ~31) + 8 * (2 * ((r >> 4) & 1) + ((r >> 2) & 1)) + 4 * ((r >> 3) & 1) + (r & 3);
}
constexpr bool k_row_inverts() {
    for (int rho = 0; rho < kKT; ++rho)
        if (k_row(kappa_of_row<false>(rho)) != rho) return false;
    return true;
}
static_assert(k_row_inverts(), "k_row inverts the key permutation");

// V slot swizzle: the 4 keys of a transposing read (key mod 4 = 0..3) times 2 slots land on distinct
// slots, and so do those of two such 16-lane blocks side by side.
template <int D>
__device__ __forceinline__ int v_slot(int key, int slot) { return slot ^ ((key & 3) * (D / 32)); }

// x s as an exact pair: hi = f16(x s), lo = x s - hi (x an integer code, s an f16 scale).
__device__ __forceinline__ void scale8_pair(v8h x, _Float16 s, v8h& hi, v8h& lo) {
    const v8h sv = {s, s, s, s, s, s, s, s};
    hi = x * sv;
    lo = __builtin_elementwise_fma(x, sv, -hi);
}

// Per-wave state of the key loop: this lane's row (query ql of the wave), its half h of the keys.
template <int D>
struct PfState {
    v8h qop[PfTile<D>::NCS];     // B operand of S^T: channels 16 c + 8 h .. + 7 of the row
    v16f o[PfTile<D>::NCB];      // O^T: channels 32 cb + 8 j + 4 h + i of the row
    float cr, m_run, l;          // score scale (base 2), reference max, this half's denominator
};

// The instruction groups a scheduling region is laid out in (LLVM AMDGPU sched_group_barrier masks).
constexpr int kSgMfma = 0x008, kSgValu = 0x002 | 0x400, kSgDsRead = 0x100;

// One key tile: S^T = K Q^T, online softmax (base 2), O^T += V^T P^T. TAIL: the tile crosses some
// row's diagonal (or L), and key kappa of this row is kept iff kappa < lim - kbase.
//
// Operands come from LDS two steps ahead of their products (rings of three stages), and the
// exponentials of the next 16-key block are interleaved with the current block's P.V products, so
// the matrix unit and the vector unit of a wave overlap.
template <int D, bool TAIL, typename Mid>
__device__ __forceinline__ void pf_tile(PfState<D>& st, const uint8_t* buf, const uint8_t* q8w, int kbase, int lim,
                                        int ql, int h, int l, Mid mid) {
    using C = PfTile<D>;
    constexpr int RING = 3;
    // ---- S^T: step c takes channels 16 c .. 16 c + 15 of K hi for both 32-key blocks (f16 products),
    // step cc channels 64 cc .. 64 cc + 63 of K lo (FP8 products, the row's block scales applied by the
    // matrix unit)
    v16f s[2];
    v8h kop[RING][2];
    auto kread = [&](int c, v8h* dst) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int row = 32 * b + ql;
            dst[b] = *reinterpret_cast<const v8h*>(buf + row * C::kRowB + swz<C::NS>(row, 2 * c + h) * 16);
        }
    };
    // K lo of this lane's rows, in the scaled product's operand order: registers 0-3 hold channels
    // 64 cc + 16 h .. + 15 and registers 4-7 channels 64 cc + 32 + 16 h .. + 15 (16-byte slots 4 cc + h and
    // 4 cc + 2 + h of the D-byte row), while the block scale a lane supplies covers the 32 channels
    // 64 cc + 32 h .. + 31, half of them held by the other half-wave (group 2 cc + h, byte cc of the row's
    // scale word h); then this lane's FP8 q operand in the same order (the wave's LDS copy: 16-byte
    // pieces k of step cc at (2 cc + k) KB). Step cc is read two f16 steps before its products.
    v8i klo[2], q8;
    uint32_t kesc[2];
    auto loread = [&](int cc) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int row = 32 * b + ql;
            if (cc == 0) kesc[b] = *reinterpret_cast<const uint32_t*>(buf + C::kKE + row * 8 + 4 * h);
            const uint8_t* rb = buf + C::kKLo8 + row * D;
            const v4i lo0 = *reinterpret_cast<const v4i*>(rb + swz<D / 16>(row, 4 * cc + h) * 16);
            const v4i lo1 = *reinterpret_cast<const v4i*>(rb + swz<D / 16>(row, 4 * cc + 2 + h) * 16);
            klo[b] = v8i{lo0[0], lo0[1], lo0[2], lo0[3], lo1[0], lo1[1], lo1[2], lo1[3]};
        }
        const v4i a0 = *reinterpret_cast<const v4i*>(q8w + (2 * cc) * 1024 + 16 * l);
        const v4i a1 = *reinterpret_cast<const v4i*>(q8w + (2 * cc + 1) * 1024 + 16 * l);
        q8 = v8i{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    };
    // A operand of P.V step t (key block u = t / NCB, channel block cb = t % NCB): lane l gets channel
    // 32 cb + l % 32 of keys 16 u + 8 h .. + 7, two transposing reads of 4 keys x 16 channels per
    // 16-lane block
    const int blk = l >> 4, lj = l & 15;
    auto vop_of = [&](const uint8_t* vt, int cb, int u) {
        v4h half[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int key = 16 * u + 8 * (blk >> 1) + 4 * t + (lj >> 2);
            const int slot = 4 * cb + 2 * (blk & 1) + ((lj & 3) >> 1);
            const uint8_t* p = vt + key * C::kRowB + v_slot<D>(key, slot) * 16 + 8 * (lj & 1);
            half[t] = __builtin_bit_cast(v4h, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lv4s_p)(p)));
        }
        return v8h{half[0][0], half[0][1], half[0][2], half[0][3], half[1][0], half[1][1], half[1][2], half[1][3]};
    };
    constexpr int PV_STEPS = 4 * C::NCB;
    v8h vhi[RING], vlo[RING];
    auto vread = [&](int t) {
        vhi[t % RING] = vop_of(buf + C::kVHi, t % C::NCB, t / C::NCB);
        vlo[t % RING] = vop_of(buf + C::kVLo, t % C::NCB, t / C::NCB);
    };

    kread(0, kop[0]);
    kread(1, kop[1]);
#pragma unroll
    for (int c = 0; c < C::NCS; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        if (c + 2 < C::NCS) kread(c + 2, kop[(c + 2) % RING]);
        else if (c + 2 - C::NCS < 2) vread(c + 2 - C::NCS);     // the first P.V operands
        // the FP8 steps: step cc after f16 step (cc + 1) NCS / NCC - 1, its operands read two steps before
        constexpr int SPC = C::NCS / C::NCC;     // f16 steps per FP8 step
        if ((c + 3) % SPC == 0) loread((c + 3) / SPC - 1);
        const v8h* k = kop[c % RING];
#pragma unroll
        for (int b = 0; b < 2; ++b)
            s[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(k[b], st.qop[c], c == 0 ? v16f{} : s[b], 0, 0, 0);
        if ((c + 1) % SPC == 0) {
#pragma unroll
            for (int b = 0; b < 2; ++b)
                s[b] = (c + 1) / SPC == 1
                           ? __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(klo[b], q8, s[b], 0, 0, 0, kesc[b], 0, 127 + kQ8Exp)
                           : __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(klo[b], q8, s[b], 0, 0, 1, kesc[b], 0, 127 + kQ8Exp);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    mid();   // the next tile's code loads go out here, after the score products
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TAIL) {
        // a lane of half h holds the half-0 keys plus 8 h; opaque so that it is not hoisted
        int nval = lim - kbase - 8 * h;
        asm volatile("" : "+v"(nval));
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (kappa_of_row<false>(32 * b + 8 * (r >> 2) + (r & 3)) >= nval) s[b][r] = -__builtin_inff();
    }
    float mt = -__builtin_inff();
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[b][r]);
    {   // the other half's keys of the same row: lanes l and l ^ 32 swapped
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float ms = mt * st.cr;
    // the reference max moves (and the row's accumulator with it) only when some row of the wave
    // would see p > 2^kLag against it
    if (__builtin_amdgcn_ballot_w64(ms > st.m_run + kLag) != 0) {
        const float mo = st.m_run;
        const float mn = fmaxf(mo, ms);
        const float alpha = (mo == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mo - mn);
        st.m_run = mn;
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) st.o[cb][e] *= alpha;
        st.l *= alpha;
    }
    // every row sees key 0 in the first tile, so the reference is finite from there on and a masked
    // score (-inf) gives p = 2^-inf = 0 exactly. P^T operand of keys 16 u .. 16 u + 15: this half's
    // keys 16 u + 8 h + e, registers 4 (j & 1) + i of block u >> 1 with j >> 1 = u & 1.
    const float mref = st.m_run;
    auto p_of = [&](int u) {
        v8h p;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = s[u >> 1][4 * (2 * (u & 1) + (e >> 2)) + (e & 3)];
            p[e] = static_cast<_Float16>(__builtin_amdgcn_exp2f(__builtin_fmaf(x, st.cr, -mref)));
        }
        return p;
    };
    const v2h one2 = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
    v8h pf[4];
    pf[0] = p_of(0);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) {
            const int t = C::NCB * u + cb;
            if (t + 2 < PV_STEPS) vread(t + 2);
            st.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vhi[t % RING], pf[u], st.o[cb], 0, 0, 0);
            st.o[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vlo[t % RING], pf[u], st.o[cb], 0, 0, 0);
        }
        // the denominator (dot2 of the f16 P against ones) and the next block's P, between the products
        if (u + 1 < 4) pf[u + 1] = p_of(u + 1);
#pragma unroll
        for (int e = 0; e < 4; ++e) st.l = __builtin_amdgcn_fdot2(v2h{pf[u][2 * e], pf[u][2 * e + 1]}, one2, st.l, false);
#pragma unroll
        for (int m = 0; m < 2 * C::NCB; ++m) {
            __builtin_amdgcn_sched_group_barrier(kSgDsRead, 2, 0);
            __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSgValu, 3, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int G, int NW, int D>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_paged_prefill(PrefillArgs a) {
    using C = PfTile<D>;
    constexpr int kRowB = C::kRowB, kBufB = C::kBufB;
    constexpr int kRows = 32 * NW;                      // rows per workgroup
    constexpr int BQ = kRows / G;                       // query tokens per workgroup
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kBufB];
    __shared__ __attribute__((aligned(1024))) uint8_t q8s[NW * C::NCC * 2048];   // each wave's FP8 q operands
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63, ql = l & 31, h = l >> 5;

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
    // this wave's last row is token j0 + (32 w + 31) / G
    const int hi_end = min(L, ctx + j0 + (32 * w + 31) / G + 1);
    // the block table is read through the constant address space: its wave-uniform reads become scalar
    // loads, whose counter is not the one the code loads are waited on with
    typedef __attribute__((address_space(4))) const int32_t cint32;
    const cint32* bt = reinterpret_cast<const cint32*>(reinterpret_cast<uintptr_t>(a.bt + static_cast<int64_t>(seq) * a.bt_stride));
    const int last_page = (L - 1) / kBS;

    // ---- this lane's row r = 32 w + ql: token r / G, head r % G; per-row power-of-two rescale
    PfState<D> st;
    const int r = 32 * w + ql;
    const int jq = j0 + r / G, hq = hk * G + r % G;
    const int lim = min(L, ctx + jq + 1);               // keys this row sees
    {
        const bool ok = jq < qlen && qs0 + jq >= 0 && qs0 + jq < a.T;
        v4u raw[C::NCS];
        const uint16_t* qp = a.q + static_cast<int64_t>(qs0 + (ok ? jq : 0)) * a.qt + static_cast<int64_t>(hq) * a.qh;
#pragma unroll
        for (int c = 0; c < C::NCS; ++c)
            raw[c] = ok ? *reinterpret_cast<const v4u*>(qp + 16 * c + 8 * h) : v4u{0u, 0u, 0u, 0u};
        float f[C::NCS][8];
        float mx = 0.0f;
#pragma unroll
        for (int c = 0; c < C::NCS; ++c) {
            const uint4 rc = make_uint4(raw[c][0], raw[c][1], raw[c][2], raw[c][3]);
            if (a.q_f16) unpack_f16x8(rc, f[c]);
            else unpack_bf16x8(rc, f[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[c][e]));
        }
        mx = swap32_max(mx);
        const int sh = mx > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(mx) : 0;
#pragma unroll
        for (int c = 0; c < C::NCS; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.qop[c][e] = static_cast<_Float16>(__builtin_amdgcn_ldexpf(f[c][e], sh));
        // the FP8 products' operand, q 2^(sh - 7) as e4m3 in the scaled product's order: channels
        // 64 cc + 16 h .. + 15, then 64 cc + 32 + 16 h .. + 15 of the same row
#pragma unroll
        for (int cc = 0; cc < C::NCC; ++cc) {
            v4u r8[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                r8[k] = ok ? *reinterpret_cast<const v4u*>(qp + 64 * cc + 32 * (k >> 1) + 16 * h + 8 * (k & 1)) : v4u{0u, 0u, 0u, 0u};
            const float s8 = __builtin_amdgcn_ldexpf(1.0f, kQ8Exp - sh);   // the convert divides by it
            int q8v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float g[8];
                const uint4 rc = make_uint4(r8[k][0], r8[k][1], r8[k][2], r8[k][3]);
                if (a.q_f16) unpack_f16x8(rc, g);
                else unpack_bf16x8(rc, g);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    v2s w = {};
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, g[4 * e], g[4 * e + 1], s8, false);
                    w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, g[4 * e + 2], g[4 * e + 3], s8, true);
                    q8v[2 * k + e] = __builtin_bit_cast(int, w);
                }
            }
            uint8_t* q8w = q8s + w * C::NCC * 2048;
            *reinterpret_cast<v4i*>(q8w + (2 * cc) * 1024 + 16 * l) = v4i{q8v[0], q8v[1], q8v[2], q8v[3]};
            *reinterpret_cast<v4i*>(q8w + (2 * cc + 1) * 1024 + 16 * l) = v4i{q8v[4], q8v[5], q8v[6], q8v[7]};
        }
        st.cr = __builtin_amdgcn_ldexpf(a.scale, -sh);
        st.m_run = a.sinks ? a.sinks[hq] * 1.44269504f : -__builtin_inff();
        // a sink is one more term 2^(sink - m) = 1 of the row's denominator, counted in half 0
        st.l = (a.sinks && h == 0) ? 1.0f : 0.0f;
#pragma unroll
        for (int cb = 0; cb < C::NCB; ++cb) st.o[cb] = v16f{};
    }

    // ---- staging: thread tid takes 16 channels (part) of key kappa = tid / (D / 16) of a tile (K and V);
    // a wave's keys lie in one page, tile page KPW w / 16
    constexpr int PARTS = D / 16;
    static_assert(NW * C::KPW >= kKT, "one pass stages a tile");
    const int part = tid % PARTS, kappa = tid / PARTS;
    const bool stager = C::KPW * w < kKT;               // wave-uniform
    const int64_t rowstride = a.Hk;                     // cache rows per slot
    auto page_block = [&](int tile) {
        const int tp = stager ? (C::KPW * w) / kBS : 0;
        const int page = __builtin_amdgcn_readfirstlane(min(tile * (kKT / kBS) + tp, last_page));
        const int b = bt[page];
        return (b >= 0 && b < a.num_blocks) ? b : 0;    // a bad entry reads block 0 (no fault)
    };
    v4u kraw, vraw;
    uint32_t ksr, vsr;
    auto load_tile = [&](int blk) {
        if (!stager) return;
        const int64_t row = (static_cast<int64_t>(blk) * kBS + (kappa & 15)) * rowstride + hk;
        kraw = *reinterpret_cast<const v4u*>(a.kc + row * D + 16 * part);
        vraw = *reinterpret_cast<const v4u*>(a.vc + row * D + 16 * part);
        ksr = a.ks[row * C::NCB + (part >> 1)];
        vsr = a.vs[row * C::NCB + (part >> 1)];
    };
    // keys at or past L (unused slots, clamped pages) get zero scales: their scores are masked and their
    // values must not carry a NaN or inf of memory nobody wrote into the P.V sums
    auto store_tile = [&](uint8_t* buf, int kbase) {
        if (!stager) return;
        const bool live = kbase + kappa < L;
        const _Float16 zero = static_cast<_Float16>(0.0f);
        const _Float16 ks = live ? __builtin_bit_cast(_Float16, static_cast<uint16_t>(ksr)) : zero;
        const _Float16 vs = live ? __builtin_bit_cast(_Float16, static_cast<uint16_t>(vsr)) : zero;
        v8h kh0, kl0, kh1, kl1, vh0, vl0, vh1, vl1;
        scale8_pair(i8x8_to_f16(kraw[0], kraw[1]), ks, kh0, kl0);
        scale8_pair(i8x8_to_f16(kraw[2], kraw[3]), ks, kh1, kl1);
        scale8_pair(i8x8_to_f16(vraw[0], vraw[1]), vs, vh0, vl0);
        scale8_pair(i8x8_to_f16(vraw[2], vraw[3]), vs, vh1, vl1);
        const int kr = k_row(kappa);
        const int k0 = kr * kRowB + swz<C::NS>(kr, 2 * part) * 16, k1 = kr * kRowB + swz<C::NS>(kr, 2 * part + 1) * 16;
        *reinterpret_cast<v8h*>(buf + k0) = kh0;
        *reinterpret_cast<v8h*>(buf + k1) = kh1;
        // K lo to FP8 as lo 2^-E, E = (exponent of ks) - 13: |lo| <= 2^-12 |code ks| keeps lo 2^-E within
        // 256 (e4m3 holds 448), and its grain (a multiple of 2^-10 of the scale's leading bit) maps to
        // multiples of 4, so no e4m3 subnormal arises; the products apply 2^E through the block scale
        const int ee = __builtin_amdgcn_frexp_expf(static_cast<float>(ks)) - 13;
        const float e2 = __builtin_amdgcn_ldexpf(1.0f, ee);
        v4i lo8;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const v8h& src = q < 2 ? kl0 : kl1;
            v2s w = {};
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, v2h{src[4 * (q & 1)], src[4 * (q & 1) + 1]}, e2, false);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(w, v2h{src[4 * (q & 1) + 2], src[4 * (q & 1) + 3]}, e2, true);
            lo8[q] = __builtin_bit_cast(int, w);
        }
        *reinterpret_cast<v4i*>(buf + C::kKLo8 + kr * D + swz<D / 16>(kr, part) * 16) = lo8;
        // the block scale of group part / 2 (both threads of the group compute it; the even one stores):
        // byte 4 (g & 1) + (g >> 1) of the row's 8
        if ((part & 1) == 0) {
            const int g = part >> 1;
            buf[C::kKE + kr * 8 + 4 * (g & 1) + (g >> 1)] = static_cast<uint8_t>(127 + ee);
        }
        const int v0 = kappa * kRowB + v_slot<D>(kappa, 2 * part) * 16, v1 = kappa * kRowB + v_slot<D>(kappa, 2 * part + 1) * 16;
        *reinterpret_cast<v8h*>(buf + C::kVHi + v0) = vh0;
        *reinterpret_cast<v8h*>(buf + C::kVHi + v1) = vh1;
        *reinterpret_cast<v8h*>(buf + C::kVLo + v0) = vl0;
        *reinterpret_cast<v8h*>(buf + C::kVLo + v1) = vl1;
    };

    // ---- key loop: tile j is processed from buffer j % 2 while tile j + 1's codes are in flight;
    // the table entries of tile j + 2 are read meanwhile
    int nb = page_block(0);
    load_tile(nb);
    nb = page_block(min(1, ntiles - 1));
    store_tile(lds, 0);
    __syncthreads();
    // tiles every row of the workgroup sees whole run without masking code; from the first row's
    // diagonal on, a wave masks the tiles it sees and skips those past its last row
    const int j_whole = min(ntiles, min(L, ctx + j0 + 1) / kKT);
    auto step = [&](int j, auto tail) {
        uint8_t* cur = lds + (j & 1) * kBufB;
        uint8_t* nxt = lds + ((j + 1) & 1) * kBufB;
        // tile j + 1's codes (the last tile again past the end) are loaded once this tile's scores are in
        // flight, so their registers are not held through the score products
        auto mid = [&]() {
            load_tile(nb);
            nb = page_block(min(j + 2, ntiles - 1));
        };
        const int kbase = j * kKT;
        if (!decltype(tail)::value || kbase < hi_end)
            pf_tile<D, decltype(tail)::value>(st, cur, q8s + w * C::NCC * 2048, kbase, lim, ql, h, l, mid);
        else
            mid();
        store_tile(nxt, (j + 1) * kKT);
        __syncthreads();
    };
    for (int j = 0; j < j_whole; ++j) step(j, std::false_type{});
    for (int j = j_whole; j < ntiles; ++j) step(j, std::true_type{});

    // ---- epilogue: out = acc / l, the denominator summed over both halves
    const float lt = swap32_add(st.l);
    if (jq >= qlen || qs0 + jq < 0 || qs0 + jq >= a.T) return;
    const float inv = 1.0f / lt;
    const int64_t orow = static_cast<int64_t>(qs0 + jq) * a.ot + static_cast<int64_t>(hq) * a.oh;
#pragma unroll
    for (int cb = 0; cb < C::NCB; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
            store_out(a.out, orow + 32 * cb + 8 * (e >> 2) + 4 * h + (e & 3), st.o[cb][e] * inv, a.out_bf16 != 0);
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
