"""GPU parity of the q8 prefix pass + log-sum-exp merge and of the paged GQA decode against the CPU
oracle, with the decode's bit-exact block-table indexing probe."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import DEV, check_float, cosine, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _rand_codes(g, B, S, H, D, layout, block, lo=0.001, hi=0.004):
    codes = g.integers(-127, 128, size=(B, S, H, D)).astype(np.int8)
    scales = g.uniform(lo, hi, size=(B, H, O.scale_count(S, layout, block))).astype(np.float32)
    return codes, scales


def _q8(x):
    c, s = O.q8_quantize(x)
    return c, s


def _dev_prefix(kc, ks, vc, vs):
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    return sq.Q8Prefix(dev(kc), f16(ks), dev(vc), f16(vs))


PREFIX_CASES = [
    # D, B, PB, H, Hk, Sq, P, q layout, kv_tile, with mu
    (128, 1, 1, 4, 2, 200, 333, (0, 128), 64, True),
    (128, 2, 1, 2, 2, 129, 64, (1, 32), 128, True),
    (128, 2, 2, 3, 1, 70, 257, (3, 128), 64, False),
    (64, 1, 1, 4, 4, 130, 100, (0, 32), 128, True),
    (64, 1, 1, 2, 2, 1, 1, (0, 64), 64, True),
    (128, 1, 1, 2, 2, 300, 128, (0, 64), 64, True),     # whole tiles only: no masked key
    (64, 2, 1, 2, 1, 97, 192, (3, 128), 64, False),
    (128, 1, 1, 2, 1, 140, 640, (1, 32), 128, True),
]


@pytest.mark.parametrize("case", PREFIX_CASES, ids=[str(i) for i in range(len(PREFIX_CASES))])
def test_prefix_merge_parity_ragged(case):
    D, B, PB, H, Hk, Sq, P, (ql, qb), kvt, with_mu = case
    print("prefix case", case, flush=True)
    g = np.random.default_rng(2000 + D + Sq + P)
    qc, qs = _rand_codes(g, B, Sq, H, D, ql, qb, 0.01, 0.02)
    kx = g.standard_normal(size=(PB, P, Hk, D), dtype=np.float32)
    vx = g.standard_normal(size=(PB, P, Hk, D), dtype=np.float32)
    kc, ks = _q8(kx)
    vc, vs = _q8(vx)
    mu = (g.standard_normal(size=(B, Hk, D)) * 0.3).astype(np.float32) if with_mu else None
    out_in = g.standard_normal(size=(B, Sq, H, D)).astype(np.float32)
    lse_in = (g.standard_normal(size=(B, H, Sq)) * 3 + 5).astype(np.float32)
    ref, rlse, allow = O.prefix_merge(O.QK(qc, qs, ql, qb), O.Q8Prefix(kc, ks, vc, vs), mu, out_in, lse_in,
                                      kv_tile=kvt)
    out, lse = dev(out_in.copy()), dev(lse_in.copy())
    sq.sq_attn_prefix_lse_merge(sq.QK(dev(qc), dev(qs), ql, qb), _dev_prefix(kc, ks, vc, vs),
                                dev(mu) if mu is not None else None, out, lse, 1.0, kvt)
    torch.cuda.synchronize()
    check_float(host(out), ref, allow, what="merged out")
    np.testing.assert_allclose(host(lse), rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("D", [64, 128])
def test_prefix_merge_scale_exponents_spread(D):
    """Prefix keys and values whose FP16 group scales differ by up to 2^8 across the groups of a token and across
    tokens: each group's integer dot meets its own key scale and each value its own group scale, so a scale read
    from the wrong group or token shows far above the bound."""
    g = np.random.default_rng(2400 + D)
    B, H, Hk, Sq, P, (ql, qb), kvt = 1, 4, 2, 150, 300, (0, 64), 64
    qc, qs = _rand_codes(g, B, Sq, H, D, ql, qb, 0.01, 0.02)
    spread = lambda: np.repeat(np.exp2(g.integers(-4, 5, size=(1, P, Hk, D // 32))), 32, axis=-1).astype(np.float32)
    kc, ks = _q8(g.standard_normal(size=(1, P, Hk, D), dtype=np.float32) * spread())
    vc, vs = _q8(g.standard_normal(size=(1, P, Hk, D), dtype=np.float32) * spread())
    mu = (g.standard_normal(size=(B, Hk, D)) * 0.3).astype(np.float32)
    out_in = g.standard_normal(size=(B, Sq, H, D)).astype(np.float32)
    lse_in = (g.standard_normal(size=(B, H, Sq)) * 3 + 5).astype(np.float32)
    ref, rlse, allow = O.prefix_merge(O.QK(qc, qs, ql, qb), O.Q8Prefix(kc, ks, vc, vs), mu, out_in, lse_in,
                                      kv_tile=kvt)
    out, lse = dev(out_in.copy()), dev(lse_in.copy())
    sq.sq_attn_prefix_lse_merge(sq.QK(dev(qc), dev(qs), ql, qb), _dev_prefix(kc, ks, vc, vs), dev(mu), out, lse, 1.0,
                                kvt)
    torch.cuda.synchronize()
    check_float(host(out), ref, allow, what="merged out, spread D %d" % D)
    np.testing.assert_allclose(host(lse), rlse, rtol=0, atol=1e-4)


def test_prefix_merge_empty_prefix_keeps_projected_pass():
    g = np.random.default_rng(7)
    qc, qs = _rand_codes(g, 1, 40, 2, 128, 0, 64)
    out_in = g.standard_normal(size=(1, 40, 2, 128)).astype(np.float32)
    lse_in = g.standard_normal(size=(1, 2, 40)).astype(np.float32)
    e8 = np.zeros((1, 0, 2, 128), np.int8)
    e16 = np.zeros((1, 0, 2, 4), np.uint16)
    out, lse = dev(out_in.copy()), dev(lse_in.copy())
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    sq.sq_attn_prefix_lse_merge(sq.QK(dev(qc), dev(qs), 0, 64), sq.Q8Prefix(dev(e8), f16(e16), dev(e8), f16(e16)),
                                None, out, lse)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), out_in)
    np.testing.assert_array_equal(host(lse), lse_in)


def _sample_rows(S, n, seed, tile=128):
    g = np.random.default_rng(seed)
    last_tile = np.arange((S - 1) // tile * tile, S)
    rows = np.unique(np.concatenate([[0, S - 1], last_tile[:: max(1, len(last_tile) // 8)],
                                     g.choice(S, n, replace=False)]))
    return rows.astype(np.int64)


def test_cfg3_joint_with_q8_prefix_full_size():
    """Joint text+image workload at full size (512 + 8192 projected tokens, H=24, d=128, segmented norm
    weights) with a 4096-token q8 prefix: projected pass, prefix pass, merge; checked on sampled rows."""
    c = gen.CFG3
    inp = gen.attn_inputs(c)
    pk_x, pv_x = gen.prefix_fp32(c)
    kc, ks = _q8(pk_x)
    vc, vs = _q8(pv_x)
    print("cfg3 inputs ready", flush=True)
    wr = dev(inp.weight_rows)
    nq = sq.Norm(sq.NORM_HEAD, dev_bf16(inp.wq), wr, None, c.eps)
    nk = sq.Norm(sq.NORM_HEAD, dev_bf16(inp.wk), wr, None, c.eps)
    r = sq.Rope(sq.ROPE_SPLIT_HALF, dev(inp.table))
    kd = dev_bf16(inp.k)
    mu = sq.sq_kmean(kd, nk, r)
    q = sq.sq_quant_qk(dev_bf16(inp.q), nq, r, None, gen.sm_scale_q(c.D), 1e-7, 0, c.q_block)
    k = sq.sq_quant_qk(kd, nk, r, mu, 1.0, 1e-7, 0, c.k_block)
    out, lse = sq.sq_attn(q, k, dev_bf16(inp.v), None, 1.0, c.kv_tile)
    sq.sq_attn_prefix_lse_merge(q, _dev_prefix(kc, ks, vc, vs), mu, out, lse, 1.0, c.kv_tile)
    torch.cuda.synchronize()
    rows = _sample_rows(c.Sq, 24, c.seed)
    print("gpu done; oracle on %d rows" % rows.size, flush=True)
    pq = O.Prologue(norm=O.NORM_HEAD, weight=inp.wq, weight_rows=inp.weight_rows, eps=c.eps, rope=O.ROPE_SPLIT_HALF,
                    table=inp.table)
    pk = O.Prologue(norm=O.NORM_HEAD, weight=inp.wk, weight_rows=inp.weight_rows, eps=c.eps, rope=O.ROPE_SPLIT_HALF,
                    table=inp.table)
    mu_o = O.kmean(inp.k, pk)
    np.testing.assert_array_equal(host(mu).view(np.uint32), mu_o.view(np.uint32))
    qc, qs = O.quant_qk(inp.q, pq, 0, c.q_block, sm_scale=gen.sm_scale_q(c.D))
    kcc, kss = O.quant_qk(inp.k, pk, 0, c.k_block, mean=mu_o)
    np.testing.assert_array_equal(host(q.codes), qc)
    np.testing.assert_array_equal(host(k.codes), kcc)
    po, pl, pa = O.attn(O.QK(qc, qs, 0, c.q_block), O.QK(kcc, kss, 0, c.k_block), inp.v, False, kv_tile=c.kv_tile,
                        rows=rows)
    full_o = np.zeros((1, c.Sq, c.H, c.D), np.float32)
    full_l = np.zeros((1, c.H, c.Sq), np.float32)
    full_o[:, rows] = po
    full_l[:, :, rows] = pl
    ref, rlse, allow = O.prefix_merge(O.QK(qc, qs, 0, c.q_block), O.Q8Prefix(kc, ks, vc, vs), mu_o, full_o, full_l,
                                      kv_tile=c.kv_tile, rows=rows)
    o = host(out)[:, rows]
    err = check_float(o, ref, allow + pa, what="cfg3 merged out")
    np.testing.assert_allclose(host(lse)[:, :, rows], rlse, rtol=0, atol=1e-4)
    exact = O.attn_exact(inp.q, pq, inp.k, pk, inp.v, prefix=O.Q8Prefix(kc, ks, vc, vs), rows=rows)
    cs = cosine(o, exact)
    print("cfg3 max err/rms %.3g cos %.6f" % (err, cs))
    assert cs >= 0.995


# ------------------------------------------------------------------------------------------------ paged decode
def _decode_case(lens, Hq, Hk, seed, D=128, bs=16, extra_blocks=3, v_sigma=1.0, q_f16=False, k_spread=0, v_spread=0):
    g = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    pages = (lens + bs - 1) // bs
    NB = int(pages.sum()) + extra_blocks
    perm = g.permutation(NB).astype(np.int32)
    maxb = int(pages.max()) + 2
    bt = np.full((len(lens), maxb), -1, np.int32)
    o = 0
    for n, p in enumerate(pages):
        bt[n, :p] = perm[o:o + p]
        o += p
    kx = g.standard_normal(size=(NB, bs, Hk, D), dtype=np.float32)
    vx = g.standard_normal(size=(NB, bs, Hk, D), dtype=np.float32) * np.float32(v_sigma)
    if k_spread or v_spread:   # a power of two per (slot, head, 32-channel group)
        kx *= np.repeat(np.exp2(g.integers(-k_spread, k_spread + 1, size=(NB, bs, Hk, D // 32))), 32, axis=-1).astype(np.float32)
        vx *= np.repeat(np.exp2(g.integers(-v_spread, v_spread + 1, size=(NB, bs, Hk, D // 32))), 32, axis=-1).astype(np.float32)
    kc, ks = _q8(kx)
    vc, vs = _q8(vx)
    if q_f16:   # binary16 queries, spread over f16's range
        q = (g.standard_normal(size=(len(lens), Hq, D)) * 4).astype(np.float16)
    else:
        q = gen.normal_bf16((len(lens), 1, Hq, D), g).reshape(len(lens), Hq, D)
    return q, kc, ks, vc, vs, bt, lens


def _dev_q(q):
    return dev(q) if q.dtype == np.float16 else dev_bf16(q)


def _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale, max_len=None):
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    out = sq.sq_paged_decode(_dev_q(q), dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens),
                             int(lens.max()) if max_len is None else max_len, scale)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("Hq,Hk", [(8, 2), (4, 4), (8, 4), (16, 2)])
def test_paged_decode_parity(Hq, Hk):
    lens = [1, 16, 17, 511, 512, 513, 1100, 37]
    print("decode Hq %d Hk %d" % (Hq, Hk), flush=True)
    q, kc, ks, vc, vs, bt, lens = _decode_case(lens, Hq, Hk, 3000 + Hq + Hk)
    scale = 1.0 / np.sqrt(128.0)
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale)
    got = _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale)
    check_float(got, ref, None, what="decode out")
    assert cosine(got, ref) >= 0.999999


@pytest.mark.parametrize("D,q_f16,Hq,Hk", [(64, False, 8, 2), (64, True, 16, 2), (128, True, 8, 2), (64, False, 4, 4)])
def test_paged_decode_head_dims_and_q_dtypes(D, q_f16, Hq, Hk):
    """Head dim 64 (two q8 groups per row) and binary16 queries, against the oracle's binary64 decode."""
    lens = [1, 17, 255, 256, 257, 700]
    print("decode D %d q_f16 %d Hq %d Hk %d" % (D, q_f16, Hq, Hk), flush=True)
    q, kc, ks, vc, vs, bt, lens = _decode_case(lens, Hq, Hk, 3100 + D + Hq + q_f16, D=D, q_f16=q_f16)
    scale = 1.0 / np.sqrt(float(D))
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale)
    got = _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale)
    check_float(got, ref, None, what="decode D %d out" % D)
    assert cosine(got, ref) >= 0.999999


@pytest.mark.parametrize("v_sigma", [0.01, 0.003, 1e-4])
def test_paged_decode_small_values(v_sigma):
    """Values ~N(0, sigma^2): their FP16 scales are small, and the P.V weights p * vs would fall into f16's subnormal
    range without the per-wave power-of-two rescale of the scales; held to the same bound."""
    lens = [1, 17, 300, 1100, 4096]
    print("decode small values sigma %g" % v_sigma, flush=True)
    q, kc, ks, vc, vs, bt, lens = _decode_case(lens, 8, 2, 3100, v_sigma=v_sigma)
    scale = 1.0 / np.sqrt(128.0)
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale)
    got = _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale)
    check_float(got, ref, None, what="decode out sigma %g" % v_sigma)


@pytest.mark.parametrize("D", [64, 128])
def test_paged_decode_scale_exponents_spread(D):
    """Group scales whose exponents differ across the groups of a slot and across slots (keys by up to 2^12, values
    by up to 2^4): each group's dot meets its own key scale and each value group its own weight, so a scale taken
    from the wrong group or slot shows far above the bound."""
    lens = [1, 17, 300, 1100]
    print("decode spread D %d" % D, flush=True)
    q, kc, ks, vc, vs, bt, lens = _decode_case(lens, 8, 2, 3200 + D, D=D, k_spread=6, v_spread=2)
    q = gen.to_bf16_bits(gen.from_bf16_bits(q) * 0.125)   # moderate scores against the spread keys
    scale = 1.0 / np.sqrt(float(D))
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale)
    got = _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale)
    check_float(got, ref, None, what="decode spread D %d out" % D)


def test_paged_decode_block_permutation_is_bit_identical():
    q, kc, ks, vc, vs, bt, lens = _decode_case([300, 1000, 45], 8, 2, 31)
    scale = 1.0 / np.sqrt(128.0)
    a = _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale)
    g = np.random.default_rng(5)
    NB = kc.shape[0]
    perm = g.permutation(NB)                       # new physical id of each old block
    inv = np.argsort(perm)
    kc2, ks2, vc2, vs2 = kc[inv], ks[inv], vc[inv], vs[inv]
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    b = _gpu_decode(q, kc2, ks2, vc2, vs2, bt2, lens, scale)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_paged_decode_dominant_key_indexing_bit_exact():
    """One key per sequence dominates by > 2000 log2 units (every other p is exactly 0 in FP32); the
    values are powers of two that spell the physical slot id, so the output must equal that slot's
    dequantized value bit for bit. The dominant position sweeps every page of every sequence."""
    Hq, Hk, D, bs = 8, 2, 128, 16
    lens = np.asarray([1, 17, 600, 1300], np.int32)
    q, kc, ks, vc, vs, bt, lens = _decode_case(lens, Hq, Hk, 77)
    NB = kc.shape[0]
    q = np.full_like(q, 0x3f80)                    # bf16 1.0
    one, sixteenth = 0x3c00, 0x2c00                # FP16 1.0 and 2^-4
    slots = np.arange(NB * bs).reshape(NB, bs)
    digits = [(slots // 64 ** i) % 64 + 1 for i in range(3)]    # 1..64
    vc = np.zeros((NB, bs, Hk, D), np.int8)
    for i in range(3):
        vc[:, :, :, i] = digits[i][:, :, None]
    vc[:, :, :, 3:] = ((np.arange(D - 3) % 64) + 1)[None, None, None, :]
    vc[:, :, 1, :] *= -1                           # kv head 1 negated
    vs = np.full((NB, bs, Hk, D // 32), sixteenth, np.uint16)
    ks = np.full((NB, bs, Hk, D // 32), one, np.uint16)
    scale = 1.0 / np.sqrt(128.0)
    pages = (lens + bs - 1) // bs
    for k in range(int(pages.max())):
        kc = np.zeros((NB, bs, Hk, D), np.int8)
        want = []
        for n, L in enumerate(lens):
            pos = min(k * bs + (k * 7) % bs, int(L) - 1)
            phys, slot = bt[n, pos // bs], pos % bs
            kc[phys, slot] = 127
            want.append((n, phys, slot))
        got = _gpu_decode(q, kc, ks, vc, vs, bt, lens, scale)
        for n, phys, slot in want:
            for h in range(Hq):
                hk = h // (Hq // Hk)
                exp = vc[phys, slot, hk].astype(np.float32) * np.float32(2.0 ** -4)
                np.testing.assert_array_equal(got[n, h].view(np.uint32), exp.view(np.uint32),
                                              err_msg="seq %d page sweep %d head %d" % (n, k, h))


def test_cfg5_paged_decode_full_size():
    """64 sequences, lengths ~U(512, 16384), 32 query / 8 kv heads, block 16, permuted block table,
    q8 cache from N(0,1) keys and values: every sequence against the binary64 oracle."""
    c = gen.CFG5
    lens, bt, NB = gen.decode_layout(c)
    kx, vx = gen.decode_fp32(c, NB)
    kc, ks = _q8(kx)
    del kx
    vc, vs = _q8(vx)
    del vx
    q = gen.decode_query(c)
    print("cfg5 inputs ready: %d blocks" % NB, flush=True)
    got = _gpu_decode(q, kc, ks, vc, vs, bt, lens, c.scale, max_len=c.lmax)
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, c.scale)
    err = check_float(got, ref, None, what="cfg5 out")
    cs = cosine(got, ref)
    print("cfg5 max err/rms %.3g cos %.8f" % (err, cs))
    assert cs >= 0.995
