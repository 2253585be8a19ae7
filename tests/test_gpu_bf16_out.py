"""bf16 outputs (out_dtype) of the attention core, the paged decode and the paged prefill. Each is checked against
the oracle with the FP32 output's tolerance plus bf16's rounding (at most 2^-9 relative, taken as 2^-8 |ref|), and
against the same call's FP32 output rounded to nearest even on the host, bit for bit (the kernels round their FP32
result once, at the store)."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu

BF16_REL = 2.0 ** -8


def _rne_bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().to(torch.bfloat16).view(torch.int16).numpy()


def _bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().view(torch.int16).numpy()


def _as_f32(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().float().numpy()


@pytest.mark.parametrize("fp8,causal", [(False, False), (True, False), (True, True)])
def test_core_bf16_out(fp8, causal):
    c = gen.CFG1
    inp = gen.attn_inputs(c)
    pq = O.Prologue(norm=O.NORM_HEAD, weight=inp.wq, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=inp.table)
    pk = O.Prologue(norm=O.NORM_HEAD, weight=inp.wk, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=inp.table)
    nq = sq.Norm(sq.NORM_HEAD, dev_bf16(inp.wq), None, None, c.eps)
    nk = sq.Norm(sq.NORM_HEAD, dev_bf16(inp.wk), None, None, c.eps)
    r = sq.Rope(sq.ROPE_SPLIT_HALF, dev(inp.table))
    kd = dev_bf16(inp.k)
    mu = sq.sq_kmean(kd, nk, r)
    q = sq.sq_quant_qk(dev_bf16(inp.q), nq, r, None, gen.sm_scale_q(c.D), 1e-7, sq.LAYOUT_PER_BLOCK, 64)
    k = sq.sq_quant_qk(kd, nk, r, mu, 1.0, 1e-7, sq.LAYOUT_PER_BLOCK, 64)
    sinks = np.array([0.5, -1.0], np.float32) if causal else None
    sd = dev(sinks) if causal else None
    if fp8:
        v8, vs = sq.sq_quant_v_fp8(dev_bf16(inp.v))
        args = (q, k, v8, vs, 1.0, 128)
    else:
        args = (q, k, dev_bf16(inp.v), None, 1.0, 64)
    print("core bf16 out fp8 %s causal %s" % (fp8, causal), flush=True)
    o32, l32 = sq.sq_attn(*args, causal=causal, sinks=sd)
    o16, l16 = sq.sq_attn(*args, causal=causal, sinks=sd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert o16.dtype == torch.bfloat16
    np.testing.assert_array_equal(_bits(o16), _rne_bits(o32))
    np.testing.assert_array_equal(host(l16).view(np.uint32), host(l32).view(np.uint32))
    mu_o = O.kmean(inp.k, pk)
    qc, qs = O.quant_qk(inp.q, pq, 0, 64, sm_scale=gen.sm_scale_q(c.D))
    kc, ks = O.quant_qk(inp.k, pk, 0, 64, mean=mu_o)
    if fp8:
        vc_o, vs_o = O.quant_v_fp8(inp.v)
        ref, _, allow = O.attn(O.QK(qc, qs, 0, 64), O.QK(kc, ks, 0, 64), vc_o, True, vs_o, kv_tile=128,
                               causal=causal, sinks=sinks)
    else:
        ref, _, allow = O.attn(O.QK(qc, qs, 0, 64), O.QK(kc, ks, 0, 64), inp.v, False, kv_tile=64, causal=causal,
                               sinks=sinks)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(_as_f32(o16) - ref)
    assert np.all(err <= 2e-3 * rms + allow + BF16_REL * np.abs(ref)), "bf16 core output outside tolerance"


def _paged_case(seed, ctx, qlen, Hq=8, Hk=2, D=128, bs=16):
    g = np.random.default_rng(seed)
    lens = np.array(ctx, np.int32) + np.array(qlen, np.int32)
    pages = [(int(L) + bs - 1) // bs for L in lens]
    NB = sum(pages) + 2
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


def test_paged_decode_and_prefill_bf16_out():
    q, kc, ks, vc, vs, bt, lens, qs = _paged_case(6200, (0, 100, 300), (90, 33, 1))
    scale = 1 / math.sqrt(128)
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    dkc, dks, dvc, dvs, dbt, dl = dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens)
    ml = int(lens.max())
    print("prefill / decode bf16 out", flush=True)
    p32 = sq.sq_paged_prefill(dev_bf16(q), dkc, dks, dvc, dvs, dbt, dl, dev(qs), ml, scale)
    p16 = sq.sq_paged_prefill(dev_bf16(q), dkc, dks, dvc, dvs, dbt, dl, dev(qs), ml, scale, out_dtype=torch.bfloat16)
    last = qs[1:] - 1
    qd = dev_bf16(q[last])
    d32 = sq.sq_paged_decode(qd, dkc, dks, dvc, dvs, dbt, dl, ml, scale)
    d16 = sq.sq_paged_decode(qd, dkc, dks, dvc, dvs, dbt, dl, ml, scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_bits(p16), _rne_bits(p32))
    np.testing.assert_array_equal(_bits(d16), _rne_bits(d32))
    pref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
    dref = O.paged_decode(q[last], kc, ks, vc, vs, bt, lens, scale)
    for got, ref, tol, what in ((p16, pref, 2e-3, "prefill"), (d16, dref, 2e-3, "decode")):
        ref = ref.astype(np.float64)
        rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        err = np.abs(_as_f32(got) - ref)
        assert np.all(err <= tol * rms + BF16_REL * np.abs(ref)), "%s bf16 output outside tolerance" % what
