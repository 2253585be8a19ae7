"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test checks the oracle against something other than itself: a library routine
(torch / numpy format conversions), a closed form, an exact-arithmetic grid on which
quantized attention equals textbook FP64 attention, brute-force group enumeration from
the layout descriptions, or an invariant (power-of-two scaling, rotation norms,
permutations). A plausible slip in the oracle (a dropped term, a wrong sign, index or
operand) fails at least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

import gen
import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(bits):
    return gen.from_bf16_bits(bits)


# ----------------------------------------------------------------------------- number formats
def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(1)
    x = np.concatenate([g.standard_normal(4000).astype(np.float32) * 10.0 ** g.integers(-30, 30, 4000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.4e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    got = np.array([O.bf16_round(float(v)) for v in x], np.float32)
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_f16_matches_numpy():
    g = np.random.default_rng(2)
    x = np.concatenate([g.standard_normal(3000).astype(np.float32) * 10.0 ** g.integers(-9, 5, 3000),
                        np.array([65504.0, 65519.0, 65520.0, 1e-8, 2.0 ** -24, 3 * 2.0 ** -25], np.float32)])
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([O.f32_to_f16(float(v)) for v in x], np.uint16)
    np.testing.assert_array_equal(got, ref)
    for h in range(0, 65536, 97):
        want = np.array([h], np.uint16).view(np.float16).astype(np.float64)[0]
        v = O.f16_value(h)
        assert (math.isnan(v) and math.isnan(want)) or v == want


def test_e4m3_matches_torch_and_spec():
    g = np.random.default_rng(3)
    x = g.standard_normal(5000).astype(np.float32) * np.float32(2.0) ** g.integers(-12, 9, 5000).astype(np.float32)
    x = x[np.abs(x) < 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([O.f32_to_e4m3(float(v)) for v in x], np.uint8)
    np.testing.assert_array_equal(got, ref)
    for b in range(256):
        want = torch.tensor([b], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()
        v = O.e4m3_value(b)
        assert (math.isnan(v) and math.isnan(want)) or v == want
    # saturation at the largest normal (the quantizer divides by amax / 448)
    assert O.f32_to_e4m3(448.0 * (1 + 2 ** -20)) == 0x7E and O.f32_to_e4m3(-1000.0) == 0xFE
    with open(os.path.join(GOLDEN, "e4m3_encodings.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            val, byte = line.split()
            assert O.f32_to_e4m3(float(val)) == int(byte, 16), line


# ----------------------------------------------------------------------------- scale layouts
def _members(layout, T):
    """Row groups from the layout descriptions: per block, eight scales per 32 rows (rows r, r+8, r+16,
    r+24), four scales per 64 rows (row pairs repeating every 8 rows), four per 128 rows (32 consecutive
    rows each)."""
    groups = {}
    if layout == O.LAYOUT_THREAD_Q:
        for blk in range((T + 127) // 128 * 4):
            for r in range(8):
                groups[8 * blk + r] = [32 * blk + r + 8 * i for i in range(4)]
    elif layout == O.LAYOUT_THREAD_K:
        for blk in range((T + 63) // 64):
            for pair in range(4):
                groups[4 * blk + pair] = [64 * blk + 8 * m + 2 * pair + e for m in range(8) for e in range(2)]
    elif layout == O.LAYOUT_WARP_Q:
        for blk in range((T + 127) // 128):
            for w in range(4):
                groups[4 * blk + w] = list(range(128 * blk + 32 * w, 128 * blk + 32 * w + 32))
    return groups


@pytest.mark.parametrize("layout,block", [(O.LAYOUT_THREAD_Q, 32), (O.LAYOUT_THREAD_K, 64), (O.LAYOUT_WARP_Q, 128),
                                          (O.LAYOUT_PER_BLOCK, 64), (O.LAYOUT_PER_BLOCK, 128), (O.LAYOUT_PER_BLOCK, 32)])
def test_group_membership_by_enumeration(layout, block):
    T, D = 300, 64
    # row t holds the constant (t + 1) / 512 (exact in bf16 for t < 256 ... powers ok: compare in float)
    vals = (np.arange(T, dtype=np.float32) + 1) / 512.0
    x = gen.to_bf16_bits(np.broadcast_to(vals[None, :, None, None], (1, T, 1, D)))
    xv = f32(x)[0, :, 0, 0]
    codes, scales = O.quant_qk(x, O.Prologue(), layout, block, scale_eps=0.0)
    if layout == O.LAYOUT_PER_BLOCK:
        groups = {g: list(range(g * block, min(T, (g + 1) * block))) for g in range((T + block - 1) // block)}
    else:
        groups = _members(layout, T)
    assert scales.shape[-1] == len(groups) == O.scale_count(T, layout, block)
    for g, rows in groups.items():
        rows = [t for t in rows if t < T]
        amax = np.float32(max([xv[t] for t in rows], default=0.0))
        assert scales[0, 0, g] == np.float32(amax / np.float32(127.0)), (g, rows)
        for t in rows:
            assert O.scale_index(t, layout, block) == g


def test_thread_q_tail_groups_get_eps():
    T, D = 40, 64
    x = gen.normal_bf16((1, T, 2, D), gen.rng(7, 0))
    _, scales = O.quant_qk(x, O.Prologue(), O.LAYOUT_THREAD_Q, 32, scale_eps=1e-7)
    assert scales.shape[-1] == 32           # 40 tokens padded to 128 rows: 4 blocks x 8 scales
    np.testing.assert_array_equal(scales[:, :, 16:], np.float32(1e-7))
    assert np.all(scales[:, :, 8:16] > 1e-3) and np.all(scales[:, :, :8] > 1e-3)


# ----------------------------------------------------------------------------- quantizer arithmetic
@pytest.mark.parametrize("layout,block", [(0, 64), (1, 32), (2, 64), (3, 128)])
def test_absmax_int8_properties(layout, block):
    """Quantization-only mode is symmetric absmax INT8 of the bf16 rows times sm_scale."""
    x = gen.normal_bf16((2, 200, 3, 64), gen.rng(11, layout))
    sm = 0.3
    codes, scales = O.quant_qk(x, O.Prologue(), layout, block, sm_scale=sm, scale_eps=0.0)
    v = f32(x) * np.float32(sm)
    assert np.abs(codes.astype(np.int32)).max() <= 127
    idx = np.array([O.scale_index(t, layout, block) for t in range(200)])
    s = scales[:, :, idx].transpose(0, 2, 1)[..., None]             # (B, T, H, 1)
    err = np.abs(codes.astype(np.float64) * s - v)
    assert np.all(err <= s * (0.5 + 1e-5))
    # the largest element of every (nonempty) group reaches +-127
    for b in range(2):
        for h in range(3):
            for g in np.unique(idx):
                rows = np.nonzero(idx == g)[0]
                assert np.abs(codes[b, rows, h].astype(np.int32)).max() == 127


def test_half_away_from_zero_on_exact_ties():
    D = 64
    # scale 2^-4 exactly (amax 127 * 2^-4), values k/16 + 1/32: ties at k + 0.5
    k = np.arange(-126, 127, dtype=np.float32)
    vals = np.concatenate([[127 / 16.0], (k + 0.5) / 16.0])[:D * 3]
    vals = np.resize(vals, (3 * D,)).reshape(3, D).astype(np.float32)
    vals[0, 0] = 127 / 16.0
    x = gen.to_bf16_bits(vals[None, :, None, :])
    xv = f32(x)[0, :, 0, :]
    codes, scales = O.quant_qk(x, O.Prologue(), O.LAYOUT_PER_BLOCK, 64, scale_eps=0.0)
    assert scales[0, 0, 0] == np.float32(1 / 16.0)
    r = xv * 16.0
    want = np.sign(r) * np.floor(np.abs(r) + 0.5)
    np.testing.assert_array_equal(codes[0, :, 0, :], want.astype(np.int8))


def test_norm_matches_fp64_rmsnorm_and_power_of_two_invariance():
    B, T, H, D = 1, 64, 2, 128
    x = gen.normal_bf16((B, T, H, D), gen.rng(12, 0))
    w = gen.uniform_bf16((1, D), gen.rng(12, 1))
    pro = O.Prologue(norm=O.NORM_HEAD, weight=w, eps=1e-6)
    y = O.prologue_rows(x, pro)
    xv = f32(x).astype(np.float64)
    ref = xv / np.sqrt((xv ** 2).mean(-1, keepdims=True) + 1e-6) * f32(w)[0].astype(np.float64)
    np.testing.assert_allclose(y, ref, rtol=2 ** -8, atol=1e-6)    # bf16 output rounding
    # eps = 0: scaling the input by 2^k leaves the normalized rows (and codes) bit-identical
    pro0 = O.Prologue(norm=O.NORM_HEAD, weight=w, eps=0.0)
    x2 = gen.to_bf16_bits(f32(x) * np.float32(8.0))
    for layout, block in [(0, 64), (1, 32)]:
        c1, s1 = O.quant_qk(x, pro0, layout, block)
        c2, s2 = O.quant_qk(x2, pro0, layout, block)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(s1, s2)
    # unit weight: unit RMS up to bf16 rounding
    ones = gen.to_bf16_bits(np.ones((1, D), np.float32))
    y1 = O.prologue_rows(x, O.Prologue(norm=O.NORM_HEAD, weight=ones, eps=0.0))
    np.testing.assert_allclose(np.sqrt((y1.astype(np.float64) ** 2).mean(-1)), 1.0, rtol=3e-3)


def test_all_heads_mean_squares_and_norm():
    B, T, H, D = 2, 20, 5, 64
    x = gen.normal_bf16((B, T, H, D), gen.rng(13, 0))
    ms = O.mean_sq_all_heads(x)
    xv = f32(x).astype(np.float64)
    np.testing.assert_allclose(ms, (xv ** 2).mean(axis=(2, 3)), rtol=1e-6)
    w = gen.uniform_bf16((1, H * D), gen.rng(13, 1))
    y = O.prologue_rows(x, O.Prologue(norm=O.NORM_ALL_HEADS, weight=w, eps=1e-6))
    ref = xv / np.sqrt((xv ** 2).mean(axis=(2, 3), keepdims=True) + 1e-6) * f32(w)[0].reshape(H, D)
    np.testing.assert_allclose(y, ref, rtol=2 ** -8, atol=1e-6)


def test_segmented_weight_rows():
    B, T, H, D = 1, 16, 2, 64
    x = gen.normal_bf16((B, T, H, D), gen.rng(14, 0))
    w = gen.uniform_bf16((2, D), gen.rng(14, 1))
    rows = np.array([0] * 5 + [1] * 11, np.int32)
    y = O.prologue_rows(x, O.Prologue(norm=O.NORM_HEAD, weight=w, weight_rows=rows))
    for r, sl in ((0, slice(0, 5)), (1, slice(5, 16))):
        yr = O.prologue_rows(x[:, sl], O.Prologue(norm=O.NORM_HEAD, weight=w[r:r + 1]))
        np.testing.assert_array_equal(y[:, sl], yr)


def test_rope_is_complex_rotation():
    B, T, H, D = 1, 50, 2, 128
    x = gen.normal_bf16((B, T, H, D), gen.rng(15, 0))
    tb = gen.rope_table(T, D // 2, start=3)
    z = O.prologue_rows(x, O.Prologue(rope=O.ROPE_SPLIT_HALF, table=tb)).astype(np.float64)
    xv = f32(x).astype(np.float64)
    P = D // 2
    c = (xv[..., :P] + 1j * xv[..., P:]) * (tb[0, :, 0, :, 0] + 1j * tb[0, :, 0, :, 1])[None, :, None, :]
    np.testing.assert_allclose(z[..., :P], c.real, atol=1e-5)
    np.testing.assert_allclose(z[..., P:], c.imag, atol=1e-5)
    # interleaved pairs (2p, 2p+1): the same rotation under the channel permutation
    perm = np.stack([np.arange(P), np.arange(P) + P], -1).reshape(-1)
    xi = np.ascontiguousarray(x[..., perm])
    zi = O.prologue_rows(xi, O.Prologue(rope=O.ROPE_INTERLEAVED, table=tb))
    np.testing.assert_array_equal(zi, z.astype(np.float32)[..., perm])
    # the 2x2 matrix form of the table [[cos, -sin], [sin, cos]] reads the same cos / sin
    m = np.stack([np.stack([tb[..., 0], -tb[..., 1]], -1), np.stack([tb[..., 1], tb[..., 0]], -1)], -2)
    zm = O.prologue_rows(x, O.Prologue(rope=O.ROPE_SPLIT_HALF, table=np.ascontiguousarray(m)))
    np.testing.assert_array_equal(zm, z.astype(np.float32))
    # cos = 1, sin = 0 is the identity; partial rotation leaves channels >= 2 * pairs untouched
    ident = np.ascontiguousarray(np.stack([np.ones((1, T, 1, 16)), np.zeros((1, T, 1, 16))], -1).astype(np.float32))
    zid = O.prologue_rows(x, O.Prologue(rope=O.ROPE_SPLIT_HALF, table=ident))
    np.testing.assert_array_equal(zid, f32(x))
    zp = O.prologue_rows(x, O.Prologue(rope=O.ROPE_SPLIT_HALF, table=np.ascontiguousarray(tb[:, :, :, :16])))
    np.testing.assert_array_equal(zp[..., 32:], f32(x)[..., 32:])
    # split half over Pp < D/2 pairs rotates the leading 2 Pp channels as a row of its own: channel p
    # with p + Pp (not p + D/2), pair p of the table
    Pp = 21
    tp = gen.rope_table(T, Pp, start=7)
    zq = O.prologue_rows(x, O.Prologue(rope=O.ROPE_SPLIT_HALF, table=tp)).astype(np.float64)
    cq = (xv[..., :Pp] + 1j * xv[..., Pp:2 * Pp]) * (tp[0, :, 0, :, 0] + 1j * tp[0, :, 0, :, 1])[None, :, None, :]
    np.testing.assert_allclose(zq[..., :Pp], cq.real, atol=1e-5)
    np.testing.assert_allclose(zq[..., Pp:2 * Pp], cq.imag, atol=1e-5)
    np.testing.assert_array_equal(zq[..., 2 * Pp:], xv[..., 2 * Pp:])
    # rotation keeps pair norms
    n0 = xv[..., :P] ** 2 + xv[..., P:] ** 2
    n1 = z[..., :P] ** 2 + z[..., P:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-6, atol=1e-12)


def test_kmean_matches_fp64_mean():
    B, T, H, D = 2, 333, 3, 64
    x = gen.normal_bf16((B, T, H, D), gen.rng(16, 0))
    w = gen.uniform_bf16((1, D), gen.rng(16, 1))
    pro = O.Prologue(norm=O.NORM_HEAD, weight=w, rope=O.ROPE_SPLIT_HALF, table=gen.rope_table(T, D // 2))
    mu = O.kmean(x, pro)
    z = O.prologue_rows(x, pro).astype(np.float64)
    ref = z.mean(axis=1)
    # within 1e-6 of the FP64 mean, relative to the mean magnitude of the summed rows (a mean near zero has no
    # relative precision of its own), and within 1e-6 relative wherever the mean is not small
    scale = np.abs(z).mean(axis=1)
    assert (np.abs(mu - ref) <= 1e-6 * scale).all(), float((np.abs(mu - ref) / scale).max())
    big = np.abs(ref) >= 0.05 * scale
    assert big.sum() > 20
    np.testing.assert_allclose(mu[big], ref[big], rtol=1e-6, atol=0)
    # the mean subtracted by the quantizer: quantizing (x, mean) equals quantizing the centred rows
    codes, _ = O.quant_qk(x, pro, 0, 64, mean=mu, scale_eps=0.0)
    zc = O.prologue_rows(x, pro, mean=mu)
    np.testing.assert_array_equal(zc, (z.astype(np.float32) - mu[:, None]).astype(np.float32))


# ----------------------------------------------------------------------------- attention core
def _grid_qk(g, B, S, H, D, block, int_scale):
    """Codes with a power-of-two per-block scale: dequantized values are exact."""
    codes = g.integers(-6, 7, size=(B, S, H, D)).astype(np.int8)
    n = (S + block - 1) // block
    scales = np.full((B, H, n), int_scale, np.float32)
    return O.QK(codes, scales, O.LAYOUT_PER_BLOCK, block)


def _ref_attention_base2(q, k, v, G):
    """Textbook attention with base-2 scores s = qh . kh, FP64, GQA kv head h // G."""
    qh = q.codes.astype(np.float64) * np.repeat(q.scales, q.block, axis=2)[:, :, :q.codes.shape[1]].transpose(0, 2, 1)[..., None]
    kh = k.codes.astype(np.float64) * np.repeat(k.scales, k.block, axis=2)[:, :, :k.codes.shape[1]].transpose(0, 2, 1)[..., None]
    B, Sq, H, D = q.codes.shape
    out = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            s = qh[b, :, h] @ kh[b, :, h // G].T
            m = s.max(-1, keepdims=True)
            p = np.exp2(s - m)
            out[b, :, h] = (p @ v[b, :, h // G]) / p.sum(-1, keepdims=True)
            lse[b, h] = m[:, 0] + np.log2(p.sum(-1))
    return out, lse


@pytest.mark.parametrize("kv_tile", [64, 128])
def test_attention_exact_on_integer_score_grid_bf16(kv_tile):
    """Integer scores make every p a power of two (exact in bf16) and every P.V term exact:
    the quantized core must equal textbook FP64 attention."""
    g = np.random.default_rng(21)
    B, Sq, Sk, H, Hk, D = 1, 70, 200, 4, 2, 64
    q = _grid_qk(g, B, Sq, H, D, 64, 0.25)
    k = _grid_qk(g, B, Sk, Hk, D, 64, 0.25)          # c = 1/16, scores = dot / 16
    q.codes[..., :] = (q.codes // 2) * 2
    k.codes[..., :] = (k.codes // 2) * 2              # even codes: dot divisible by 4 ... scores in Z/4
    q.scales[:] = 0.5
    k.scales[:] = 0.5                                  # c = 1/4: s = dot/4, dot = 4 * integer
    vb = g.integers(-8, 9, size=(B, Sk, Hk, D)).astype(np.float32) / 4
    v = gen.to_bf16_bits(vb)
    out, lse, allow = O.attn(q, k, v, fp8=False, kv_tile=kv_tile)
    ref, rlse = _ref_attention_base2(q, k, f32(v).astype(np.float64), H // Hk)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=1e-12, atol=1e-12)


def test_attention_exact_on_grid_fp8():
    g = np.random.default_rng(22)
    B, Sq, Sk, H, D = 1, 40, 256, 2, 64
    q = _grid_qk(g, B, Sq, H, D, 64, 0.5)
    k = _grid_qk(g, B, Sk, H, D, 64, 0.5)
    # q codes +-2 on 4 channels, k codes in {-2, 0, 2}, c = 1/4: integer scores in [-4, 4]
    q.codes[:] = 0
    for i in range(Sq):
        for h in range(H):
            ch = g.choice(D, 4, replace=False)
            q.codes[0, i, h, ch] = g.choice([-2, 2], 4)
    k.codes[:] = g.integers(-1, 2, size=k.codes.shape) * 2
    v8 = g.integers(-7, 8, size=(B, Sk, H, D)).astype(np.float32)   # e4m3-exact integers
    codes = np.vectorize(O.f32_to_e4m3)(v8).astype(np.uint8)
    vs = np.full((B, H, D), 0.125, np.float32)
    out, lse, _ = O.attn(q, k, codes, fp8=True, vs=vs, kv_tile=128)
    ref, rlse = _ref_attention_base2(q, k, v8.astype(np.float64) * 0.125, 1)
    # p = 2^-n is e4m3-exact while 256 p >= 2^-9, i.e. n <= 17: scores span 8
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rlse, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- V to FP8
def test_v_fp8_scales_and_codes_by_brute_force():
    """Per (b, h, channel): vs = max(RN(amax over tokens / 448), 1e-8) in FP32, codes = e4m3fn(RN(v / vs)) as torch
    converts FP32 (round to nearest even); a zero channel, a channel of -0, a channel below the 1e-8 floor and a
    channel whose maximum reaches the largest code."""
    g = gen.rng(30, 0)
    B, T, H, D = 2, 53, 3, 64
    bits = gen.normal_bf16((B, T, H, D), g, outliers=3)
    bits[0, :, 0, 5] = 0x0000                                        # zeros
    bits[0, :, 1, 7] = 0x8000                                        # all -0: codes keep the sign
    tiny = (g.standard_normal(T) * 1e-7).astype(np.float32)
    bits[1, :, 2, 9] = gen.to_bf16_bits(tiny)                          # amax / 448 < 1e-8: the floor
    bits[1, 11, 0, 3] = gen.to_bf16_bits(np.array([-300.0], np.float32))[0]   # one large negative entry
    codes, vs = O.quant_v_fp8(bits)
    x = f32(bits)                                                    # FP32 values (B, T, H, D)
    amax = np.abs(x).max(axis=1)                                     # over tokens only
    want_vs = np.maximum(amax / np.float32(448.0), np.float32(1e-8)).astype(np.float32)
    np.testing.assert_array_equal(vs.view(np.uint32), want_vs.view(np.uint32))
    quot = (x / want_vs[:, None]).astype(np.float32)                 # IEEE FP32 division
    want = torch.from_numpy(quot).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes, want)
    assert (codes[0, :, 1, 7] == 0x80).all() and (codes[0, :, 0, 5] == 0).all()
    assert vs[1, 2, 9] == np.float32(1e-8) and codes[1, 11, 0, 3] == 0xFE   # -448: the channel's maximum
    # vs rounded down can put a quotient an ulp above 448: it still rounds to the largest code, never to NaN
    assert np.abs(quot).max() <= 448.0 * (1 + 2.0 ** -22)
    assert not np.isin(codes, (0x7F, 0xFF)).any()
    # the plausible slips fail: a 127 divisor, or the maximum over channels instead of tokens
    assert not np.array_equal(vs, np.maximum(amax / np.float32(127.0), np.float32(1e-8)))
    assert not np.array_equal(vs, np.broadcast_to(np.maximum(np.abs(x).max(axis=(1, 3)) / np.float32(448.0),
                                                             np.float32(1e-8))[..., None], vs.shape))


# ----------------------------------------------------------------------------- FP8 dot-product reading
def _run_on_grid(prod, rounding):
    """A run of exact products added on the grid of 2^(E - 13), E the exponent of its largest magnitude (numpy
    emulation of the reading the FP8 P.V allowance follows); rounding 'trunc' (toward zero) or 'nearest'."""
    prod = np.asarray(prod, np.float64)
    mx = np.abs(prod).max()
    if mx == 0.0:
        return 0.0
    _, e = np.frexp(mx)                       # mx = f 2^e, f in [0.5, 1): leading bit 2^(e - 1)
    u = 2.0 ** (int(e) - 1 - 13)
    q = np.trunc(prod / u) if rounding == "trunc" else np.rint(prod / u)
    return float((q * u).sum())


def _e4m3_values():
    return np.array([O.e4m3_value(b) for b in range(256) if b not in (0x7F, 0xFF)], np.float64)


def test_fp8_run_bound_covers_grid_emulation_and_is_tight():
    """run_truncation_bound >= what a run loses on the grid (either rounding), on random and adversarial runs of 8
    e4m3 x e4m3 products; for runs of one large product and seven below the grid it equals the loss."""
    g = np.random.default_rng(31)
    vals = _e4m3_values()
    ratios = []
    for it in range(3000):
        kind = it % 4
        if kind == 0:      # random codes
            prod = g.choice(vals, 8) * g.choice(vals, 8)
        elif kind == 1:    # one large product, seven small of random sign
            prod = np.concatenate([[448.0 * 448.0], g.choice(vals[np.abs(vals) < 2.0], 7) * g.choice([-1.0, 1.0], 7)])
        elif kind == 2:    # the products of P (~ 256 p) and V codes of one channel, p over two decades
            pt = np.array([O.e4m3_value(O.f32_to_e4m3(float(v))) for v in 256.0 * 2.0 ** -g.uniform(0, 7, 8)])
            prod = pt * g.choice(vals, 8)
        else:              # subnormal codes beside normal ones
            prod = g.choice(vals[np.abs(vals) < 2.0 ** -6], 8) * g.choice(vals, 8)
            prod[g.integers(0, 8)] = g.choice(vals) * 448.0
        g.shuffle(prod)
        exact = float(prod.sum())
        bound = O.run_truncation_bound(prod)
        for rnd in ("trunc", "nearest"):
            loss = abs(_run_on_grid(prod, rnd) - exact)
            assert loss <= bound * (1 + 1e-12), (it, rnd, prod, loss, bound)
        lt = abs(_run_on_grid(prod, "trunc") - exact)
        if lt > 0:
            ratios.append(bound / lt)
    ratios = np.array(ratios)
    assert ratios.size > 500
    assert np.median(ratios) <= 4.0, np.median(ratios)          # not slack by orders of magnitude
    # adversarial: seven products just below the grid step u beside the largest: loss == bound exactly
    big = 448.0 * 256.0                                          # 1.75 2^16: u = 2^3
    for small in (7.5, 7.0, 4.0, 1.0, -6.5, 2.0 ** -9):
        prod = np.array([big] + [small] * 7)
        loss = abs(_run_on_grid(prod, "trunc") - prod.sum())
        assert loss == O.run_truncation_bound(prod) == 7 * abs(small)
    # products on the grid lose nothing and the bound is zero
    prod = np.array([big, 8.0, -16.0, 24.0, 0.0, 8.0, 8.0, -8.0])
    assert _run_on_grid(prod, "trunc") == prod.sum() and O.run_truncation_bound(prod) == 0.0


def test_fp8_attention_allowance_covers_grid_emulation_end_to_end():
    """Through the attention oracle: with q = 0 every p is 1 and Pt = e4m3(256) = 256, so the FP8 P.V of channel c is
    a sum of 256 Vt over runs of 8 keys; the emulated grid sum lies within the oracle's allowance of its exact sum,
    and on channels built to lose the most the allowance is attained."""
    g = np.random.default_rng(32)
    B, Sq, Sk, H, D = 1, 3, 128, 1, 64
    q = O.QK(np.zeros((B, Sq, H, D), np.int8), np.full((B, H, 1), 0.01, np.float32), 0, 64)
    k = O.QK(g.integers(-127, 128, size=(B, Sk, H, D)).astype(np.int8), np.full((B, H, 2), 0.02, np.float32), 0, 64)
    vals = _e4m3_values()
    vt = g.choice(vals, size=(B, Sk, H, D))
    # channels 0..7: every run = one 448 and seven small values of one sign below its grid step (2^-5 at 448);
    # channels 8..15 the same with mixed signs (the truncations then partly cancel)
    small = vals[(vals > 0) & (vals < 2.0 ** -5)]
    for c in range(16):
        for r0 in range(0, Sk, 8):
            vt[0, r0, 0, c] = 448.0
            sign = (1.0 if c < 4 else -1.0) if c < 8 else g.choice([-1.0, 1.0], 7)
            vt[0, r0 + 1:r0 + 8, 0, c] = g.choice(small, 7) * sign
    codes = np.vectorize(O.f32_to_e4m3)(vt.astype(np.float32)).astype(np.uint8)
    assert np.array_equal(np.vectorize(O.e4m3_value)(codes), vt)
    vs = np.full((B, H, D), 0.5, np.float32)
    out, lse, allow = O.attn(q, k, codes, fp8=True, vs=vs, kv_tile=128, flip_rel=0.0)
    f = 0.5 / (256.0 * Sk)
    exact = vt[0, :, 0, :].sum(axis=0) * 256.0 * f
    np.testing.assert_allclose(out[0, 0, 0], exact, rtol=1e-13, atol=1e-15)
    emu = np.array([sum(_run_on_grid(256.0 * vt[0, r0:r0 + 8, 0, c], "trunc") for r0 in range(0, Sk, 8))
                    for c in range(D)]) * f
    err = np.abs(emu - out[0, 0, 0])
    assert (err <= allow[0, 0, 0] * (1 + 1e-12) + 1e-18).all()
    np.testing.assert_allclose(err[:8], allow[0, 0, 0, :8], rtol=1e-12)   # attained where built to be
    assert err[:8].min() > 0


def test_attention_special_cases():
    g = np.random.default_rng(23)
    B, S, H, D = 1, 1, 2, 64
    q = O.QK(g.integers(-127, 128, size=(B, 3, H, D)).astype(np.int8), np.full((B, H, 1), 0.01, np.float32), 0, 64)
    k = O.QK(g.integers(-127, 128, size=(B, S, H, D)).astype(np.int8), np.full((B, H, 1), 0.02, np.float32), 0, 64)
    v = gen.normal_bf16((B, S, H, D), g)
    out, lse, _ = O.attn(q, k, v, fp8=False)
    # one key: a one-element softmax is one up to the exponent's fused residual r = a*c - RN(a*c),
    # |r| <= ulp(s)/2, so p = 2^r, bf16(p) == 1 and out = v / p
    dots = np.einsum("bihd,bjhd->bhi", q.codes.astype(np.int64), k.codes.astype(np.int64))
    smax = np.abs(dots).max() * float(np.float32(0.01) * np.float32(0.02))
    np.testing.assert_allclose(out, np.broadcast_to(f32(v).astype(np.float64), out.shape), rtol=smax * 2.0 ** -24,
                               atol=0)
    np.testing.assert_allclose(lse, dots * float(np.float32(0.01) * np.float32(0.02)), rtol=1e-6)
    # q = 0: every score is 0 -> uniform weights, out = mean of v
    Sk = 96
    k = O.QK(g.integers(-127, 128, size=(B, Sk, H, D)).astype(np.int8), np.full((B, H, 2), 0.02, np.float32), 0, 64)
    v = gen.normal_bf16((B, Sk, H, D), g)
    q0 = O.QK(np.zeros((B, 5, H, D), np.int8), np.full((B, H, 1), 0.01, np.float32), 0, 64)
    out, lse, _ = O.attn(q0, k, v, fp8=False, kv_tile=64)
    np.testing.assert_allclose(out, np.broadcast_to(f32(v).astype(np.float64).mean(1, keepdims=True), out.shape),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, math.log2(Sk), rtol=1e-12)


def test_attention_close_to_dequantized_fp64_and_flip_allowance():
    """Off the grid the only quantized-mode deviation from FP64 attention over the dequantized q, k is the
    rounding of P to bf16: bounded by 2^-8 of the largest |v|; the flip allowance is 0 when p is exact."""
    g = np.random.default_rng(24)
    B, Sq, Sk, H, D = 1, 33, 300, 2, 64
    q = O.QK(g.integers(-127, 128, size=(B, Sq, H, D)).astype(np.int8), g.uniform(0.001, 0.003, (B, H, 1)).astype(np.float32), 0, 64)
    k = O.QK(g.integers(-127, 128, size=(B, Sk, H, D)).astype(np.int8), g.uniform(0.001, 0.003, (B, H, 5)).astype(np.float32), 0, 64)
    v = gen.normal_bf16((B, Sk, H, D), g)
    out, lse, allow = O.attn(q, k, v, fp8=False, kv_tile=64)
    vv = f32(v).astype(np.float64)
    qh = q.codes.astype(np.float64) * q.scales[:, :, 0][:, None, :, None]
    kh = k.codes.astype(np.float64) * np.repeat(k.scales, 64, axis=2)[:, :, :Sk].transpose(0, 2, 1)[..., None]
    for h in range(H):
        s = qh[0, :, h] @ kh[0, :, h].T
        p = np.exp2(s - s.max(-1, keepdims=True))
        ref = p @ vv[0, :, h] / p.sum(-1, keepdims=True)
        assert np.abs(out[0, :, h] - ref).max() <= 2 ** -8 * np.abs(vv).max()
        np.testing.assert_allclose(lse[0, h], np.log2(np.exp2(s).sum(-1)), rtol=1e-6)
    assert np.all(allow >= 0)
    _, _, allow0 = O.attn(q, k, v, fp8=False, kv_tile=64, flip_rel=0.0)
    assert np.all(allow0 == 0)


def test_gqa_head_mapping():
    g = np.random.default_rng(25)
    B, S, H, Hk, D = 1, 16, 6, 2, 64
    q = O.QK(g.integers(-127, 128, size=(B, 4, H, D)).astype(np.int8), np.full((B, H, 1), 0.01, np.float32), 0, 64)
    k = O.QK(g.integers(-127, 128, size=(B, S, Hk, D)).astype(np.int8), np.full((B, Hk, 1), 0.01, np.float32), 0, 64)
    vals = np.zeros((B, S, Hk, D), np.float32)
    vals[:, :, 0] = 3.0
    vals[:, :, 1] = -5.0
    out, _, _ = O.attn(q, k, gen.to_bf16_bits(vals), fp8=False)
    # kv head of q head h is h // (H / Hk): heads 0..2 -> 3, heads 3..5 -> -5
    # (sum of bf16(p) over sum of p: within a bf16 rounding of the constant)
    np.testing.assert_allclose(out[0, :, :3], 3.0, rtol=2.0 ** -8)
    np.testing.assert_allclose(out[0, :, 3:], -5.0, rtol=2.0 ** -8)


# ----------------------------------------------------------------------------- prefix pass + merge
def test_prefix_merge_equals_single_pass_over_joined_keys():
    """On an integer-score grid the two-pass merge equals one softmax over [prefix keys, projected keys],
    the projected keys having been smoothed by mu (their pass misses q . mu; the prefix pass subtracts it)."""
    g = np.random.default_rng(31)
    B, Sq, Sk, P, H, D = 1, 20, 64, 96, 2, 64
    q = O.QK(((g.integers(-3, 4, size=(B, Sq, H, D))) * 2).astype(np.int8), np.full((B, H, 1), 0.5, np.float32), 0, 64)
    k = O.QK(((g.integers(-3, 4, size=(B, Sk, H, D))) * 2).astype(np.int8), np.full((B, H, 1), 0.5, np.float32), 0, 64)
    mu = (g.integers(-1, 2, size=(B, H, D)) * 4).astype(np.float32)   # q . mu integer
    vb = gen.to_bf16_bits(g.integers(-8, 9, size=(B, Sk, H, D)).astype(np.float32) / 4)
    out_a, lse_a, _ = O.attn(q, k, vb, fp8=False, kv_tile=64)
    pk = ((g.integers(-3, 4, size=(1, P, H, D))) * 2).astype(np.int8)
    ks = gen.to_f16_bits(np.full((1, P, H, D // 32), 0.5, np.float32))
    pv = g.integers(-16, 17, size=(1, P, H, D)).astype(np.int8)
    vs = gen.to_f16_bits(np.full((1, P, H, D // 32), 0.25, np.float32))
    pf = O.Q8Prefix(pk, ks, pv, vs)
    out, lse, allow = O.prefix_merge(q, pf, mu, out_a.astype(np.float32), lse_a.astype(np.float32), kv_tile=64)
    # single pass in FP64: scores q_hat . key with key = prefix (raw) or projected (k_hat + mu)
    qh = q.codes.astype(np.float64) * 0.5
    kh = k.codes.astype(np.float64) * 0.5 + mu[:, None].astype(np.float64)
    keys = np.concatenate([pk.astype(np.float64) * 0.5, kh], axis=1)
    vals = np.concatenate([pv.astype(np.float64) * 0.25, f32(vb).astype(np.float64)], axis=1)
    for h in range(H):
        s = qh[0, :, h] @ keys[0, :, h].T
        p = np.exp2(s - s.max(-1, keepdims=True))
        ref = p @ vals[0, :, h] / p.sum(-1, keepdims=True)
        np.testing.assert_allclose(out[0, :, h], ref, rtol=1e-5, atol=1e-5)
        off = qh[0, :, h] @ mu[0, h].astype(np.float64)
        np.testing.assert_allclose(lse[0, h], np.log2(np.exp2(s - off[:, None]).sum(-1)), rtol=1e-5)
    assert np.all(allow == 0)          # all p are powers of two: no flip possible


def test_merge_is_symmetric_and_degenerate():
    g = np.random.default_rng(32)
    B, Sq, H, D = 1, 8, 2, 64
    q = O.QK(g.integers(-127, 128, size=(B, Sq, H, D)).astype(np.int8), np.full((B, H, 1), 0.004, np.float32), 0, 64)
    pk, ks = O.q8_quantize(g.standard_normal((1, 50, H, D)).astype(np.float32))
    pv, vs = O.q8_quantize(g.standard_normal((1, 50, H, D)).astype(np.float32))
    pf = O.Q8Prefix(pk, ks, pv, vs)
    other = g.standard_normal((B, Sq, H, D)).astype(np.float32)
    # an empty other pass (lse = -inf) leaves the prefix pass alone
    out, lse, _, po, pl = O.prefix_merge(q, pf, None, other, np.full((B, H, Sq), -np.inf, np.float32), want_parts=True)
    np.testing.assert_allclose(out, po, rtol=1e-12)
    np.testing.assert_allclose(lse, pl, rtol=1e-12)
    # merging with an equal-lse pass averages the two outputs
    out2, lse2, _ = O.prefix_merge(q, pf, None, po.astype(np.float32), pl.astype(np.float32))
    np.testing.assert_allclose(out2, po.astype(np.float32).astype(np.float64) * 0.5 + po * 0.5, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(lse2, pl + 1.0, atol=1e-6)


# ----------------------------------------------------------------------------- q8 format
def test_q8_quantizer():
    g = np.random.default_rng(41)
    x = g.standard_normal((100, 128)).astype(np.float32) * 3
    x[0, :32] = 0.0
    codes, sc = O.q8_quantize(x)
    s32 = np.maximum(np.abs(x.reshape(100, 4, 32)).max(-1) / np.float32(127.0), np.float32(1e-8)).astype(np.float32)
    np.testing.assert_array_equal(sc, s32.astype(np.float16).view(np.uint16))
    assert np.abs(codes.astype(np.int32)).max() <= 127
    err = np.abs(codes.reshape(100, 4, 32) * s32[..., None].astype(np.float64) - x.reshape(100, 4, 32))
    assert np.all(err <= s32[..., None] * 0.5 * (1 + 1e-6))
    assert np.all(np.abs(codes.reshape(100, 4, 32)).max(-1)[1:] == 127)
    # ties round half to even: scale 1 (amax 127), values k + 0.5
    t = np.zeros((1, 32), np.float32)
    t[0, 0] = 127.0
    t[0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 10.5, 11.5]
    c, _ = O.q8_quantize(t)
    assert c[0, :9].tolist() == [127, 0, 2, 2, 0, -2, -2, 10, 12]


def _textbook_attention(q, k, v):
    """Binary64 softmax(q k^T) v per (b, h) with its base-2 log-sum-exp; q (B, S, H, D), k, v (B, T, H, D)."""
    s = np.einsum("bshd,bthd->bhst", q, k) * np.log2(np.e)          # base-2 scores
    m = s.max(-1, keepdims=True)
    p = np.exp2(s - m)
    l = p.sum(-1, keepdims=True)
    out = np.einsum("bhst,bthd->bshd", p / l, v)
    return out, (m + np.log2(l))[..., 0]


def test_lse_merge_equals_attention_over_joined_keys():
    """[kit] _merge_lse_: attention over key set A merged with attention over a disjoint set B equals attention
    over A and B joined (binary64, to rounding); an empty side (lse -inf) leaves the other; both empty give 0."""
    g = np.random.default_rng(44)
    B, S, H, D = 2, 5, 3, 16
    q = g.standard_normal((B, S, H, D)) * 0.4
    ka, va = g.standard_normal((B, 7, H, D)), g.standard_normal((B, 7, H, D))
    kb, vb = g.standard_normal((B, 11, H, D)) + 0.5, g.standard_normal((B, 11, H, D))
    oa, la = _textbook_attention(q, ka, va)
    ob, lb = _textbook_attention(q, kb, vb)
    oj, lj = _textbook_attention(q, np.concatenate([ka, kb], 1), np.concatenate([va, vb], 1))
    om, lm = O.lse_merge(oa, la, ob, lb)
    np.testing.assert_allclose(om, oj, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lm, lj, rtol=0, atol=1e-12)
    empty = np.full_like(lb, -np.inf)
    om, lm = O.lse_merge(oa, la, ob * 0 + 123.0, empty)
    np.testing.assert_array_equal(om, oa)
    np.testing.assert_array_equal(lm, la)
    om, lm = O.lse_merge(oa, empty, ob, empty)
    assert (om == 0).all() and (lm == -np.inf).all()


def test_q8_cache_writer_placement():
    """[impl] _store_kvcache_nhd placement written out by hand for a tiny cache (block 4, 3 blocks): slot 5 is
    block 1 row 1, slot 0 block 0 row 0, slot 11 block 2 row 3; slot -1 and slot 12 (past the cache) write nothing;
    every other row keeps its fill. The rows placed are the q8 rows of the tokens ([kit] quantize_q8)."""
    g = np.random.default_rng(43)
    n, Hk, D, NB, bs = 5, 2, 64, 3, 4
    k = g.standard_normal((n, Hk, D)).astype(np.float32)
    v = g.standard_normal((n, Hk, D)).astype(np.float32)
    slots = np.array([5, -1, 0, 11, 12], np.int64)
    kc = np.full((NB, bs, Hk, D), 99, np.int8)
    vc = np.full((NB, bs, Hk, D), -99, np.int8)
    ks = np.full((NB, bs, Hk, D // 32), 0x1234, np.uint16)
    vs = np.full((NB, bs, Hk, D // 32), 0x4321, np.uint16)
    O.q8_cache_write(k, v, slots, kc, ks, vc, vs)
    qk, qks = O.q8_quantize(k)
    qv, qvs = O.q8_quantize(v)
    placed = {(1, 1): 0, (0, 0): 2, (2, 3): 3}
    for b in range(NB):
        for r in range(bs):
            if (b, r) in placed:
                t = placed[(b, r)]
                assert (kc[b, r] == qk[t]).all() and (vc[b, r] == qv[t]).all()
                assert (ks[b, r] == qks[t]).all() and (vs[b, r] == qvs[t]).all()
            else:
                assert (kc[b, r] == 99).all() and (vc[b, r] == -99).all()
                assert (ks[b, r] == 0x1234).all() and (vs[b, r] == 0x4321).all()


# ----------------------------------------------------------------------------- paged decode
def _paged_case(g, N=3, Hq=8, Hk=2, D=64, bs=16, lens=(1, 17, 40)):
    pages = [(L + bs - 1) // bs for L in lens]
    NB = sum(pages) + 2
    kc, ks = O.q8_quantize(g.standard_normal((NB, bs, Hk, D)).astype(np.float32))
    vc, vs = O.q8_quantize(g.standard_normal((NB, bs, Hk, D)).astype(np.float32))
    perm = g.permutation(NB)
    bt = np.full((N, 8), -1, np.int32)
    o = 0
    for n, p in enumerate(pages):
        bt[n, :p] = perm[o:o + p]
        o += p
    q = gen.normal_bf16((N, 1, Hq, D), g).reshape(N, Hq, D)
    return q, kc, ks, vc, vs, bt, np.array(lens, np.int32)


def test_paged_decode_equals_contiguous_attention():
    """The paged decode over a block table equals unpaged attention over the gathered keys (a different
    path of the oracle), with the q8 values exact in bf16 (power-of-two scales)."""
    g = np.random.default_rng(51)
    q, kc, ks, vc, vs, bt, lens = _paged_case(g)
    ks[:] = gen.to_f16_bits(np.full(ks.shape, 2.0 ** -5, np.float32))
    vs[:] = gen.to_f16_bits(np.full(vs.shape, 2.0 ** -4, np.float32))
    scale = 1 / math.sqrt(64)
    out = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale)
    for n, L in enumerate(lens):
        pages = bt[n, :(L + 15) // 16]
        kseq = (kc[pages].reshape(-1, 2, 64)[:L].astype(np.float32) * 2.0 ** -5)[None]
        vseq = (vc[pages].reshape(-1, 2, 64)[:L].astype(np.float32) * 2.0 ** -4)[None]
        ref = O.attn_exact(q[n][None, None], O.Prologue(), gen.to_bf16_bits(kseq), O.Prologue(), gen.to_bf16_bits(vseq))
        np.testing.assert_allclose(out[n], ref[0, 0], rtol=1e-12, atol=1e-12)
    # one key (L = 1): out = v
    np.testing.assert_allclose(out[0], np.repeat(vc[bt[0, 0], 0].astype(np.float64) * 2.0 ** -4, 4, axis=0),
                               rtol=1e-15)


def test_paged_q_in_binary16_by_brute_force():
    """q given as IEEE binary16 (the f16 query dtype) is read as binary16, not as bf16 bits: the decode equals a
    numpy softmax over the gathered exact q8 keys and values, and the prefill's last rows equal that decode."""
    g = np.random.default_rng(56)
    q, kc, ks, vc, vs, bt, lens = _paged_case(g, D=128)
    q16 = (g.standard_normal(q.shape) * 3).astype(np.float16)
    scale = 0.0884
    out = O.paged_decode(q16, kc, ks, vc, vs, bt, lens, scale)
    kf = kc.astype(np.float64) * np.repeat(ks.view(np.float16).astype(np.float64), 32, axis=-1)
    vf = vc.astype(np.float64) * np.repeat(vs.view(np.float16).astype(np.float64), 32, axis=-1)
    for n, L in enumerate(lens):
        pages = bt[n, :(L + 15) // 16]
        kseq = kf[pages].reshape(-1, 2, 128)[:L]
        vseq = vf[pages].reshape(-1, 2, 128)[:L]
        for h in range(8):
            s_ = kseq[:, h // 4] @ q16[n, h].astype(np.float64) * scale
            p_ = np.exp(s_ - s_.max())
            ref = (p_ / p_.sum()) @ vseq[:, h // 4]
            np.testing.assert_allclose(out[n, h], ref, rtol=1e-12, atol=1e-12)
    # one query per sequence as a prefill: each row is that sequence's decode
    qs = np.arange(len(lens) + 1, dtype=np.int32)
    np.testing.assert_array_equal(O.paged_prefill(q16, kc, ks, vc, vs, bt, lens, qs, scale), out)


def test_paged_decode_block_permutation_invariance_and_dominant_key():
    g = np.random.default_rng(52)
    q, kc, ks, vc, vs, bt, lens = _paged_case(g)
    out = O.paged_decode(q, kc, ks, vc, vs, bt, lens, 0.125)
    NB = kc.shape[0]
    perm = g.permutation(NB)
    inv = np.argsort(perm)
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    out2 = O.paged_decode(q, kc[perm], ks[perm], vc[perm], vs[perm], bt2, lens, 0.125)
    np.testing.assert_array_equal(out, out2)
    # a key far above the rest takes all the weight: out equals its value exactly
    n, pos = 2, 29
    phys, slot = bt[n, pos // 16], pos % 16
    q = q.copy()
    q[n, 1:4] = q[n, 0]                # the q heads of a kv head share one query here
    q[n, 5:8] = q[n, 4]
    kc2 = kc.copy()
    qv = gen.from_bf16_bits(q[n])
    kc2[phys, slot, 0] = (np.sign(qv[0]) * 127).astype(np.int8)
    kc2[phys, slot, 1] = (np.sign(qv[4]) * 127).astype(np.int8)
    ks2 = ks.copy()
    ks2[phys, slot] = gen.to_f16_bits(np.full((2, 2), 60.0, np.float32))
    out3 = O.paged_decode(q, kc2, ks2, vc, vs, bt, lens, 0.125)
    vexact = vc[phys, slot].astype(np.float64) * np.repeat(
        np.array([O.f16_value(int(h)) for h in vs[phys, slot].reshape(-1)]).reshape(2, 2), 32, axis=1)
    np.testing.assert_allclose(out3[n, :4], np.broadcast_to(vexact[0], (4, 64)), rtol=1e-12)
    np.testing.assert_allclose(out3[n, 4:], np.broadcast_to(vexact[1], (4, 64)), rtol=1e-12)


def test_exact_attention_shift_invariance_of_k():
    """Subtracting a per-head constant from every key leaves attention unchanged (why k may be smoothed)."""
    g = np.random.default_rng(53)
    B, S, H, D = 1, 40, 2, 64
    q = gen.normal_bf16((B, S, H, D), g)
    kx = g.standard_normal((B, S, H, D)).astype(np.float32)
    mu = np.round(g.standard_normal((1, 1, H, D)) * 4).astype(np.float32)
    v = gen.normal_bf16((B, S, H, D), g)
    k1 = gen.to_bf16_bits(np.round(kx * 8) / 8)
    k2 = gen.to_bf16_bits(np.round(kx * 8) / 8 - mu)
    o1 = O.attn_exact(q, O.Prologue(), k1, O.Prologue(), v)
    o2 = O.attn_exact(q, O.Prologue(), k2, O.Prologue(), v)
    np.testing.assert_allclose(o1, o2, rtol=1e-9, atol=1e-12)


def test_exact_attention_matches_numpy_textbook():
    """Binary64 attention with RMSNorm and complex-rotation RoPE written with numpy routines."""
    g = np.random.default_rng(54)
    B, S, H, D = 1, 48, 2, 64
    q, k, v = (gen.normal_bf16((B, S, H, D), g) for _ in range(3))
    w = gen.uniform_bf16((1, D), g)
    tb = gen.rope_table(S, D // 2)
    pro = O.Prologue(norm=O.NORM_HEAD, weight=w, eps=1e-6, rope=O.ROPE_SPLIT_HALF, table=tb)
    out = O.attn_exact(q, pro, k, pro, v)

    def prep(x):
        xv = f32(x).astype(np.float64)
        y = xv / np.sqrt((xv ** 2).mean(-1, keepdims=True) + 1e-6) * f32(w)[0]
        z = (y[..., :D // 2] + 1j * y[..., D // 2:]) * (tb[0, :, 0, :, 0] + 1j * tb[0, :, 0, :, 1])[None, :, None]
        return np.concatenate([z.real, z.imag], -1)

    qx, kx, vx = prep(q), prep(k), f32(v).astype(np.float64)
    for h in range(H):
        s = qx[0, :, h] @ kx[0, :, h].T / math.sqrt(D)
        p = np.exp(s - s.max(-1, keepdims=True))
        np.testing.assert_allclose(out[0, :, h], p @ vx[0, :, h] / p.sum(-1, keepdims=True), rtol=1e-9, atol=1e-12)


def test_quantized_pipeline_tracks_exact_attention_tiny():
    """Norm + RoPE + k mean + INT8 q/k + bf16 P.V on the tiny workload stays within cos 0.999 of the
    unquantized FP64 attention (the method is an approximation of it)."""
    c = gen.CFG1
    inp = gen.attn_inputs(c)
    pq = O.Prologue(norm=O.NORM_HEAD, weight=inp.wq, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=inp.table)
    pk = O.Prologue(norm=O.NORM_HEAD, weight=inp.wk, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=inp.table)
    mu = O.kmean(inp.k, pk)
    qc, qs = O.quant_qk(inp.q, pq, 0, 64, sm_scale=gen.sm_scale_q(c.D))
    kc, ks = O.quant_qk(inp.k, pk, 0, 64, mean=mu)
    out, lse, _ = O.attn(O.QK(qc, qs, 0, 64), O.QK(kc, ks, 0, 64), inp.v, fp8=False, kv_tile=64)
    ref = O.attn_exact(inp.q, pq, inp.k, pk, inp.v)
    cos = (out * ref).sum() / np.sqrt((out ** 2).sum() * (ref ** 2).sum())
    assert cos > 0.999, cos


# ----------------------------------------------------------------------------- causal mask and sinks
def _core_inputs(g, B=1, Sq=70, Sk=200, H=2, D=64, fp8=True):
    qc = g.integers(-127, 128, size=(B, Sq, H, D)).astype(np.int8)
    kc = g.integers(-127, 128, size=(B, Sk, H, D)).astype(np.int8)
    qs = g.uniform(1e-3, 4e-3, size=(B, H, O.scale_count(Sq, 0, 64))).astype(np.float32)
    ks = g.uniform(1e-3, 4e-3, size=(B, H, O.scale_count(Sk, 2, 64))).astype(np.float32)
    if fp8:
        v = (g.integers(0, 0x7f, size=(B, Sk, H, D)) | (g.integers(0, 2, size=(B, Sk, H, D)) << 7)).astype(np.uint8)
        vs = np.full((B, H, D), 0.01, np.float32)
    else:
        v, vs = gen.normal_bf16((B, Sk, H, D), g), None
    return qc, qs, kc, ks, v, vs


def test_causal_row_equals_attention_over_its_visible_keys():
    """[tq] causal rows (query i at position context + i sees keys 0 .. context + i, context = Sk - Sq): each causal
    row equals the non-causal core run over those keys alone (same tiles from key 0), bit for bit."""
    g = np.random.default_rng(61)
    for fp8 in (True, False):
        qc, qs, kc, ks, v, vs = _core_inputs(g, fp8=fp8)
        Sq, Sk = qc.shape[1], kc.shape[1]
        kv_tile = 128 if fp8 else 64
        q = O.QK(qc, qs, 0, 64)
        out, lse, allow = O.attn(q, O.QK(kc, ks, 2, 64), v, fp8, vs, kv_tile=kv_tile, causal=True)
        for i in (0, 1, 37, Sq - 1):
            kend = i + Sk - Sq + 1
            nk = O.scale_count(kend, 2, 64)
            kt = O.QK(np.ascontiguousarray(kc[:, :kend]), np.ascontiguousarray(ks[:, :, :nk]), 2, 64)
            o1, l1, a1 = O.attn(q, kt, np.ascontiguousarray(v[:, :kend]), fp8, vs, kv_tile=kv_tile,
                                rows=np.array([i], np.int64))
            np.testing.assert_array_equal(out[:, i], o1[:, 0])
            np.testing.assert_array_equal(lse[:, :, i], l1[:, :, 0])
            np.testing.assert_array_equal(allow[:, i], a1[:, 0])


def test_sinks_join_the_denominator_only():
    """[tq] USE_SINKS: out = sum exp(s_i) v_i / (exp(s_h) + sum exp(s_i)). A sink of -inf changes nothing; the
    log-sum-exp with a sink is log2(2^lse + 2^(s_h log2 e)); out shrinks by 2^lse / (2^lse + 2^(s_h log2 e)) up
    to the P rounding (bf16: relative 2^-8)."""
    g = np.random.default_rng(62)
    qc, qs, kc, ks, v, vs = _core_inputs(g, fp8=False)
    q, k = O.QK(qc, qs, 0, 64), O.QK(kc, ks, 2, 64)
    out, lse, _ = O.attn(q, k, v, False, None, kv_tile=64)
    o2, l2, _ = O.attn(q, k, v, False, None, kv_tile=64, sinks=np.full(2, -np.inf, np.float32))
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)
    sinks = np.array([float(lse.mean()) * np.log(2.0), float(lse.max()) * np.log(2.0) + 1.0], np.float32)
    o3, l3, _ = O.attn(q, k, v, False, None, kv_tile=64, sinks=sinks)
    sb = (sinks.astype(np.float32) * np.float32(1.44269504)).astype(np.float64)[None, :, None]
    np.testing.assert_allclose(l3, np.log2(np.exp2(lse) + np.exp2(sb)), rtol=0, atol=2e-6)
    f = (np.exp2(lse) / (np.exp2(lse) + np.exp2(sb))).transpose(0, 2, 1)[..., None]
    assert np.abs(o3 - out * f).max() <= 2.0 ** -8 * np.abs(out).max()


def test_paged_decode_sinks():
    """Decode with per-head sinks against a softmax with the extra logit written out with numpy on the gathered
    q8 values; a sink of -inf changes nothing."""
    g = np.random.default_rng(63)
    q, kc, ks, vc, vs, bt, lens = _paged_case(g)
    scale = 0.125
    sinks = g.standard_normal(8).astype(np.float32) * 2
    out = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale, sinks=sinks)
    assert np.array_equal(O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale, sinks=np.full(8, -np.inf, np.float32)),
                          O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale))
    f16 = lambda a: a.view(np.float16).astype(np.float64)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for n, L in enumerate(lens):
        pages = bt[n, :(L + 15) // 16]
        kv = (kc[pages].astype(np.float64) * np.repeat(f16(ks[pages]), 32, -1)).reshape(-1, 2, 64)[:L]
        vv = (vc[pages].astype(np.float64) * np.repeat(f16(vs[pages]), 32, -1)).reshape(-1, 2, 64)[:L]
        for h in range(8):
            s = kv[:, h // 4] @ qf[n, h] * scale
            m = max(s.max(), float(sinks[h]))
            p = np.exp(s - m)
            ref = p @ vv[:, h // 4] / (p.sum() + np.exp(float(sinks[h]) - m))
            np.testing.assert_allclose(out[n, h], ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- paged prefill
def _prefill_case(g, ctx=(0, 23, 40), qlen=(5, 17, 1), Hq=8, Hk=2, D=64, bs=16, extra=2):
    """A varlen batch over a paged q8 cache: sequence n has ctx[n] cached keys before its qlen[n] queries, whose
    own keys are in the cache too (seq_lens = ctx + qlen), pages dealt from a seeded permutation."""
    lens = np.array(ctx, np.int32) + np.array(qlen, np.int32)
    pages = [(int(L) + bs - 1) // bs for L in lens]
    NB = sum(pages) + extra
    kc, ks = O.q8_quantize(g.standard_normal((NB, bs, Hk, D)).astype(np.float32))
    vc, vs = O.q8_quantize(g.standard_normal((NB, bs, Hk, D)).astype(np.float32))
    perm = g.permutation(NB)
    bt = np.full((len(lens), max(pages) + 1), -1, np.int32)
    o = 0
    for n, p in enumerate(pages):
        bt[n, :p] = perm[o:o + p]
        o += p
    qs = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = gen.normal_bf16((int(qs[-1]), 1, Hq, D), g).reshape(-1, Hq, D)
    return q, kc, ks, vc, vs, bt, lens, qs


def _gather(c, s, bt_row, L, Hk, D):
    """Dense (L, Hk, D) binary64 q8 values of one sequence gathered through its block-table row."""
    f16 = s.view(np.float16).astype(np.float64)
    pages = bt_row[:(L + 15) // 16]
    return (c[pages].astype(np.float64) * np.repeat(f16[pages], 32, -1)).reshape(-1, Hk, D)[:L]


def test_paged_prefill_matches_torch_sdpa_with_the_pages_mask():
    """Against torch's own scaled_dot_product_attention in float64 on the CPU, called as [impl] _sdpa_one calls it:
    GQA by repeat_interleave, the boolean mask k_pos <= key_offset + q_pos, key_offset = k_len - q_len."""
    import torch
    import torch.nn.functional as F
    g = np.random.default_rng(71)
    Hq, Hk, D = 8, 2, 64
    q, kc, ks, vc, vs, bt, lens, qs = _prefill_case(g, Hq=Hq, Hk=Hk, D=D)
    scale = 1 / math.sqrt(D)
    out = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for n in range(len(lens)):
        L, a, b = int(lens[n]), int(qs[n]), int(qs[n + 1])
        kseq = torch.from_numpy(_gather(kc, ks, bt[n], L, Hk, D)).repeat_interleave(Hq // Hk, dim=1)
        vseq = torch.from_numpy(_gather(vc, vs, bt[n], L, Hk, D)).repeat_interleave(Hq // Hk, dim=1)
        qseq = torch.from_numpy(qf[a:b])
        qpos = (L - (b - a)) + torch.arange(b - a)
        mask = torch.arange(L)[None, :] <= qpos[:, None]
        ref = F.scaled_dot_product_attention(qseq.transpose(0, 1)[None], kseq.transpose(0, 1)[None],
                                             vseq.transpose(0, 1)[None], attn_mask=mask, scale=scale)
        np.testing.assert_allclose(out[a:b], ref[0].transpose(0, 1).numpy(), rtol=1e-11, atol=1e-12)


def test_paged_prefill_rows_are_decode_and_chunking_invariant():
    """A query's row depends only on the keys it sees: the last query of a sequence equals the paged decode over
    the whole sequence, a one-query sequence is a decode, and splitting a sequence's queries into a cached context
    and a later chunk leaves every later row unchanged, bit for bit."""
    g = np.random.default_rng(72)
    q, kc, ks, vc, vs, bt, lens, qs = _prefill_case(g)
    scale = 0.125
    out = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
    last = qs[1:] - 1
    dec = O.paged_decode(q[last], kc, ks, vc, vs, bt, lens, scale)
    np.testing.assert_array_equal(out[last], dec)
    # sequence 1 (23 cached + 17 queries) as 30 cached + the last 10 queries: those rows are unchanged
    qs2 = np.array([0, 10], np.int32)
    out2 = O.paged_prefill(q[qs[1] + 7:qs[2]], kc, ks, vc, vs, bt[1:2], lens[1:2], qs2, scale)
    np.testing.assert_array_equal(out2, out[qs[1] + 7:qs[2]])
    # rows= computes the same rows alone
    rows = np.array([0, 4, 6, 21], np.int64)
    np.testing.assert_array_equal(O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale, rows=rows), out[rows])
    # physical blocks relabelled with the table: bit-identical
    NB = kc.shape[0]
    perm = g.permutation(NB)
    inv = np.argsort(perm)
    bt2 = np.where(bt >= 0, inv[np.maximum(bt, 0)], -1).astype(np.int32)
    np.testing.assert_array_equal(O.paged_prefill(q, kc[perm], ks[perm], vc[perm], vs[perm], bt2, lens, qs, scale), out)


def test_paged_prefill_equal_keys_give_running_means():
    """With every key equal all visible scores tie, so query j of a sequence with key_offset o returns the mean of
    the values at positions 0..o + j (a running mean, written with numpy's cumsum); a sink of logit z adds
    exp(z - s0) to the count, s0 the common score."""
    g = np.random.default_rng(73)
    Hq, Hk, D = 4, 2, 64
    q, kc, ks, vc, vs, bt, lens, qs = _prefill_case(g, Hq=Hq, Hk=Hk, D=D)
    kc[:] = 3
    ks[:] = gen.to_f16_bits(np.full(ks.shape, 0.5, np.float32))
    scale = 0.1
    sinks = np.array([0.5, -1.0, 2.0, -np.inf], np.float32)
    out = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
    outs = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale, sinks=sinks)
    qf = (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for n in range(len(lens)):
        L, a, b = int(lens[n]), int(qs[n]), int(qs[n + 1])
        vseq = _gather(vc, vs, bt[n], L, Hk, D)
        csum = np.cumsum(vseq, axis=0)
        for j in range(b - a):
            last = L - (b - a) + j
            for h in range(Hq):
                ref = csum[last, h // 2] / (last + 1)
                np.testing.assert_allclose(out[a + j, h], ref, rtol=1e-12, atol=1e-14)
                s0 = float(qf[a + j, h].sum() * 1.5) * scale
                cnt = (last + 1) + np.exp(float(sinks[h]) - s0)
                np.testing.assert_allclose(outs[a + j, h], csum[last, h // 2] / cnt, rtol=1e-10, atol=1e-14)
