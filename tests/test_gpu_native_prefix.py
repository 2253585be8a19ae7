"""GPU parity of the log-sum-exp merge (sq_lse_merge) and of a native cached prefix built from the library's
entry points ([kit] cache_prefix native, _attend_with_prefix): the prefix's k mean, prefix keys quantized with it,
prefix values in FP8, the projected keys quantized with the same mean, one core pass per key set, then the merge."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import check_float, cosine, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,S,H,D", [(1, 300, 4, 128), (2, 77, 3, 64), (1, 1, 1, 128)])
def test_lse_merge_parity(B, S, H, D):
    g = gen.rng(3000 + S, 0)
    out = g.standard_normal((B, S, H, D)).astype(np.float32)
    other = g.standard_normal((B, S, H, D)).astype(np.float32) * 3
    lse = (g.standard_normal((B, H, S)) * 8).astype(np.float32)
    olse = (g.standard_normal((B, H, S)) * 8).astype(np.float32)
    if S > 4:
        olse[:, :, 0] = -np.inf           # the other set is empty for query 0
        lse[:, :, 1] = -np.inf            # this one for query 1
        lse[:, :, 2] = olse[:, :, 2] = -np.inf   # both for query 2
    ref, rlse = O.lse_merge(out, lse, other, olse)
    d_out, d_lse = dev(out), dev(lse)
    print("merge B %d S %d H %d D %d" % (B, S, H, D), flush=True)
    sq.sq_lse_merge(d_out, d_lse, dev(other), dev(olse))
    torch.cuda.synchronize()
    o, l = host(d_out), host(d_lse)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-5 * float(np.abs(ref).max()))
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(l[fin], rlse[fin], rtol=0, atol=1e-5)
    assert (l[~fin] == -np.inf).all()


def test_lse_merge_at_size_sampled_rows():
    """The benchmarked shape (two video-size outputs, B=1 Sq=32760 H=40 d=128, FP32), with empty sets on some
    queries; 1024 sampled queries (all heads) against the oracle, every other query checked to be a convex
    combination of its two inputs."""
    B, S, H, D = 1, 32760, 40, 128
    g = gen.rng(3100, 0)
    out = g.standard_normal((B, S, H, D), dtype=np.float32)
    other = g.standard_normal((B, S, H, D), dtype=np.float32) * np.float32(3)
    lse = (g.standard_normal((B, H, S), dtype=np.float32) * np.float32(8))
    olse = (g.standard_normal((B, H, S), dtype=np.float32) * np.float32(8))
    olse[:, :, 5::997] = -np.inf
    lse[:, :, 7::991] = -np.inf
    rows = np.unique(np.concatenate([g.integers(0, S, size=1000), [0, 5, 7, S - 1]]))
    ref, rlse = O.lse_merge(out[:, rows], lse[:, :, rows], other[:, rows], olse[:, :, rows])
    d_out, d_lse = dev(out), dev(lse)
    print("merge at size B %d S %d H %d D %d" % (B, S, H, D), flush=True)
    sq.sq_lse_merge(d_out, d_lse, dev(other), dev(olse))
    torch.cuda.synchronize()
    o = host(d_out)
    l = host(d_lse)
    np.testing.assert_allclose(o[:, rows], ref, rtol=0, atol=1e-5 * float(np.abs(ref).max()))
    fin = np.isfinite(rlse)
    np.testing.assert_allclose(l[:, :, rows][fin], rlse[fin], rtol=0, atol=1e-5)
    # every query: each channel lies between its two inputs (a convex combination), within rounding
    lo = np.minimum(out, other) - 1e-5
    hi = np.maximum(out, other) + 1e-5
    assert ((o >= lo) & (o <= hi)).all()


def test_native_prefix_attention():
    c = gen.CFG1
    inp = gen.attn_inputs(c)
    B, S, H, D = inp.q.shape
    P = 300
    g = gen.rng(3100, 0)
    pk = gen.normal_bf16((B, P, H, D), g)       # prefix keys, already normalized and rotated
    pv = gen.normal_bf16((B, P, H, D), g)
    pq_pro = O.Prologue(norm=O.NORM_HEAD, weight=inp.wq, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=inp.table)
    pk_pro = O.Prologue(norm=O.NORM_HEAD, weight=inp.wk, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=inp.table)
    none = O.Prologue()
    smq = gen.sm_scale_q(D)

    # oracle: the prefix mean, both key sets quantized with it, FP8 values per set, two passes, merge
    mu = O.kmean(pk, none)
    qc, qs = O.quant_qk(inp.q, pq_pro, 0, 64, sm_scale=smq)
    kc, ks = O.quant_qk(inp.k, pk_pro, 0, 64, mean=mu)
    pkc, pks = O.quant_qk(pk, none, 0, 64, mean=mu)
    v8, vs = O.quant_v_fp8(inp.v)
    pv8, pvs = O.quant_v_fp8(pv)
    oa, la, aa = O.attn(O.QK(qc, qs, 0, 64), O.QK(kc, ks, 0, 64), v8, True, vs, kv_tile=128)
    ob, lb, ab = O.attn(O.QK(qc, qs, 0, 64), O.QK(pkc, pks, 0, 64), pv8, True, pvs, kv_tile=128)
    ref, rlse = O.lse_merge(oa, la, ob, lb)
    allow = np.maximum(aa, ab)

    # GPU: the same steps through the library
    nq = sq.Norm(sq.NORM_HEAD, dev_bf16(inp.wq), None, None, c.eps)
    nk = sq.Norm(sq.NORM_HEAD, dev_bf16(inp.wk), None, None, c.eps)
    r = sq.Rope(sq.ROPE_SPLIT_HALF, dev(inp.table))
    dpk = dev_bf16(pk)
    dmu = sq.sq_kmean(dpk)
    q = sq.sq_quant_qk(dev_bf16(inp.q), nq, r, None, smq, 1e-7, 0, 64)
    k = sq.sq_quant_qk(dev_bf16(inp.k), nk, r, dmu, 1.0, 1e-7, 0, 64)
    pkq = sq.sq_quant_qk(dpk, None, None, dmu, 1.0, 1e-7, 0, 64)
    dv8, dvs = sq.sq_quant_v_fp8(dev_bf16(inp.v))
    dpv8, dpvs = sq.sq_quant_v_fp8(dev_bf16(pv))
    out, lse = sq.sq_attn(q, k, dv8, dvs, 1.0, 128)
    pout, plse = sq.sq_attn(q, pkq, dpv8, dpvs, 1.0, 128)
    sq.sq_lse_merge(out, lse, pout, plse)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dmu).view(np.uint32), mu.view(np.uint32))
    np.testing.assert_array_equal(host(pkq.codes), pkc)
    np.testing.assert_array_equal(host(k.codes), kc)
    o = host(out)
    err = check_float(o, ref, allow, what="native prefix out")
    np.testing.assert_allclose(host(lse), rlse, atol=1e-4)
    # against unquantized binary64 attention over the joined keys (prefix first, as joint attention joins them)
    qr = O.prologue_rows(inp.q, pq_pro).astype(np.float64) / np.sqrt(D)
    kr = np.concatenate([(pk.astype(np.uint32) << 16).view(np.float32), O.prologue_rows(inp.k, pk_pro)], 1)
    vr = np.concatenate([(pv.astype(np.uint32) << 16).view(np.float32), (inp.v.astype(np.uint32) << 16).view(np.float32)], 1)
    s = np.einsum("bshd,bthd->bhst", qr, kr.astype(np.float64))
    p = np.exp(s - s.max(-1, keepdims=True))
    exact = np.einsum("bhst,bthd->bshd", p / p.sum(-1, keepdims=True), vr.astype(np.float64))
    cs = cosine(o, exact)
    print("native prefix max err/rms %.3g cos %.6f" % (err, cs))
    assert cs >= 0.995
