"""GPU parity of the quantized attention core against the CPU oracle (quantized mode, with the flip
allowance) and accuracy against unquantized binary64 attention (cosine >= 0.995)."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import DEV, check_float, cosine, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _qk_from_oracle(codes, scales, layout, block):
    return sq.QK(dev(codes), dev(scales), layout, block)


def _run_core(qc, qs, ql, qb, kc, ks, kl, kb, v, fp8, vs=None, kv_tile=64, score_scale=1.0, v_token_major=None):
    q = _qk_from_oracle(qc, qs, ql, qb)
    k = _qk_from_oracle(kc, ks, kl, kb)
    if fp8:
        # channel-major FP8 codes, as the V quantizer writes them
        B, S, H, D = v.shape
        tp = (S + 127) // 128 * 128
        cm = np.zeros((B, H, D, tp), np.uint8)
        cm[..., :S] = v.transpose(0, 2, 3, 1)
        out, lse = sq.sq_attn(q, k, dev(cm), dev(vs), score_scale, kv_tile)
    else:
        out, lse = sq.sq_attn(q, k, dev_bf16(v), None, score_scale, kv_tile)
    torch.cuda.synchronize()
    return host(out), host(lse)


def _rand_codes(g, B, S, H, D, layout, block, lo=0.001, hi=0.004):
    codes = g.integers(-127, 128, size=(B, S, H, D)).astype(np.int8)
    n = O.scale_count(S, layout, block)
    scales = g.uniform(lo, hi, size=(B, H, n)).astype(np.float32)
    return codes, scales


CASES = [
    # D, H, Hk, Sq, Sk, q layout, k layout, pv, kv_tile
    (128, 4, 2, 200, 333, (1, 32), (2, 64), "fp8", 128),
    (128, 2, 2, 129, 257, (3, 128), (0, 64), "fp8", 128),
    (64, 4, 4, 130, 300, (0, 32), (0, 32), "fp8", 128),
    (128, 4, 1, 70, 333, (0, 64), (0, 64), "bf16", 64),
    (128, 2, 2, 257, 129, (1, 32), (2, 64), "bf16", 128),
    (64, 6, 3, 100, 200, (0, 128), (2, 64), "bf16", 64),
    (64, 2, 2, 1, 1, (0, 64), (0, 64), "bf16", 64),
    (128, 2, 2, 5, 1, (0, 64), (0, 64), "fp8", 128),
    (128, 4, 2, 200, 333, (1, 32), (2, 64), "fp8", 64),
    (64, 4, 4, 130, 300, (0, 32), (0, 32), "fp8", 64),
    (128, 2, 1, 129, 65, (3, 128), (0, 128), "fp8", 64),
    (128, 2, 2, 3, 1, (0, 64), (2, 64), "fp8", 64),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_core_parity_ragged(case):
    D, H, Hk, Sq, Sk, (ql, qb), (kl, kb), pv, kvt = case
    print("core case", case, flush=True)
    g = np.random.default_rng(1000 + D + Sq + Sk)
    qc, qs = _rand_codes(g, 1, Sq, H, D, ql, qb)
    kc, ks = _rand_codes(g, 1, Sk, Hk, D, kl, kb)
    v = gen.normal_bf16((1, Sk, Hk, D), g, outliers=3)
    fp8 = pv == "fp8"
    run = None
    if fp8:
        v8, vs = O.quant_v_fp8(v)
        ref, rlse, allow, run = O.attn(O.QK(qc, qs, ql, qb), O.QK(kc, ks, kl, kb), v8, True, vs, kv_tile=kvt,
                                       want_run_allow=True)
        out, lse = _run_core(qc, qs, ql, qb, kc, ks, kl, kb, v8, True, vs, kvt)
    else:
        ref, rlse, allow = O.attn(O.QK(qc, qs, ql, qb), O.QK(kc, ks, kl, kb), v, False, kv_tile=kvt)
        out, lse = _run_core(qc, qs, ql, qb, kc, ks, kl, kb, v, False, None, kvt)
    check_float(out, ref, allow, what="out", run=run)
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)


def test_core_score_scale():
    g = np.random.default_rng(5)
    D, H, S = 128, 2, 150
    qc, qs = _rand_codes(g, 1, S, H, D, 0, 64)
    kc, ks = _rand_codes(g, 1, S, H, D, 0, 64)
    v = gen.normal_bf16((1, S, H, D), g)
    ref, rlse, allow = O.attn(O.QK(qc, qs, 0, 64), O.QK(kc, ks, 0, 64), v, False, score_scale=0.7, kv_tile=64)
    out, lse = _run_core(qc, qs, 0, 64, kc, ks, 0, 64, v, False, None, 64, score_scale=0.7)
    check_float(out, ref, allow, what="out")
    np.testing.assert_allclose(lse, rlse, atol=1e-4)


def _pipeline_gpu(c, inp, mu_from_gpu=True):
    """GPU: norm stats / k mean / quantize q, k / V to FP8 / core."""
    norm_mode = O.NORM_ALL_HEADS if c.norm == "all_heads" else O.NORM_HEAD
    wr = dev(inp.weight_rows) if inp.weight_rows is not None else None
    nq = sq.Norm(norm_mode, dev_bf16(inp.wq), wr, None, c.eps)
    nk = sq.Norm(norm_mode, dev_bf16(inp.wk), wr, None, c.eps)
    r = sq.Rope(O.ROPE_SPLIT_HALF, dev(inp.table))
    qd, kd, vd = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    ql, qb = gen.LAYOUT[c.q_layout], c.q_block
    kl, kb = gen.LAYOUT[c.k_layout], c.k_block
    mu = sq.sq_kmean(kd, nk, r)
    q = sq.sq_quant_qk(qd, nq, r, None, gen.sm_scale_q(c.D), 1e-7, ql, qb)
    k = sq.sq_quant_qk(kd, nk, r, mu, 1.0, 1e-7, kl, kb)
    if c.pv == "fp8":
        v8, vs = sq.sq_quant_v_fp8(vd)
        out, lse = sq.sq_attn(q, k, v8, vs, 1.0, c.kv_tile)
    else:
        out, lse = sq.sq_attn(q, k, vd, None, 1.0, c.kv_tile)
    torch.cuda.synchronize()
    return out, lse, q, k, mu


def _pipeline_oracle(c, inp, rows):
    norm_mode = O.NORM_ALL_HEADS if c.norm == "all_heads" else O.NORM_HEAD
    pq = O.Prologue(norm=norm_mode, weight=inp.wq, weight_rows=inp.weight_rows, eps=c.eps, rope=O.ROPE_SPLIT_HALF,
                    table=inp.table)
    pk = O.Prologue(norm=norm_mode, weight=inp.wk, weight_rows=inp.weight_rows, eps=c.eps, rope=O.ROPE_SPLIT_HALF,
                    table=inp.table)
    ql, qb = gen.LAYOUT[c.q_layout], c.q_block
    kl, kb = gen.LAYOUT[c.k_layout], c.k_block
    mu = O.kmean(inp.k, pk)
    qc, qs = O.quant_qk(inp.q, pq, ql, qb, sm_scale=gen.sm_scale_q(c.D))
    kc, ks = O.quant_qk(inp.k, pk, kl, kb, mean=mu)
    run = None
    if c.pv == "fp8":
        v8, vs = O.quant_v_fp8(inp.v)
        out, lse, allow, run = O.attn(O.QK(qc, qs, ql, qb), O.QK(kc, ks, kl, kb), v8, True, vs, kv_tile=c.kv_tile,
                                      rows=rows, want_run_allow=True)
    else:
        out, lse, allow = O.attn(O.QK(qc, qs, ql, qb), O.QK(kc, ks, kl, kb), inp.v, False, kv_tile=c.kv_tile,
                                 rows=rows)
    exact = O.attn_exact(inp.q, pq, inp.k, pk, inp.v, rows=rows)
    return out, lse, (allow, run), exact, (qc, qs, kc, ks, mu)


def _sample_rows(S, n, seed, tile=128):
    g = np.random.default_rng(seed)
    last_tile = np.arange((S - 1) // tile * tile, S)
    rows = np.unique(np.concatenate([[0, S - 1], last_tile[:: max(1, len(last_tile) // 8)],
                                     g.choice(S, n, replace=False)]))
    return rows.astype(np.int64)


def test_cfg1_tiny_end_to_end():
    c = gen.CFG1
    inp = gen.attn_inputs(c)
    out, lse, q, k, mu = _pipeline_gpu(c, inp)
    ref, rlse, (allow, run), exact, (qc, qs, kc, ks, mu_o) = _pipeline_oracle(c, inp, None)
    np.testing.assert_array_equal(host(q.codes), qc)
    np.testing.assert_array_equal(host(k.codes), kc)
    o = host(out)
    err = check_float(o, ref, allow, what="cfg1 out", run=run)
    np.testing.assert_allclose(host(lse), rlse, atol=1e-4)
    cs = cosine(o, exact)
    print("cfg1 max err/rms %.3g cos %.6f" % (err, cs))
    assert cs >= 0.995


@pytest.mark.parametrize("c", [gen.CFG2, gen.CFG3], ids=["video", "joint"])
def test_full_size_sampled_rows(c):
    """The video and joint workloads at full size in the benchmark's launch configuration, checked on sampled
    query rows (first, last, the last partial tile, and random rows) of every head."""
    inp = gen.attn_inputs(c)
    print("inputs ready", c.name, flush=True)
    out, lse, q, k, mu = _pipeline_gpu(c, inp)
    rows = _sample_rows(c.Sq, 24, c.seed)
    print("gpu done; oracle on %d rows" % rows.size, flush=True)
    ref, rlse, (allow, run), exact, (qc, qs, kc, ks, mu_o) = _pipeline_oracle(c, inp, rows)
    np.testing.assert_array_equal(host(mu).view(np.uint32), mu_o.view(np.uint32))
    np.testing.assert_array_equal(host(k.codes), kc)
    np.testing.assert_array_equal(host(q.codes)[:, rows], qc[:, rows])
    np.testing.assert_array_equal(host(q.scales).view(np.uint32), qs.view(np.uint32))
    o = host(out)[:, rows]
    # the video workload (FP8 P.V) is accepted partly through the FP8 run allowance: the count is printed
    err = check_float(o, ref, allow, what="%s out" % c.name, run=run)
    np.testing.assert_allclose(host(lse)[:, :, rows], rlse, atol=1e-4)
    cs = cosine(o, exact)
    print("%s max err/rms %.3g cos %.6f" % (c.name, err, cs))
    assert cs >= 0.995
