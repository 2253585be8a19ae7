"""GPU parity of the causal mask and the per-head attention sinks ([tq] unified attention: causal mask, USE_SINKS)
in the quantized core (sq_attn) and the paged decode (sq_paged_decode), against the oracle, plus properties that hold
without it: the last causal row of a square problem is the non-causal row bit for bit, and a -inf sink is no sink."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import check_float, dev, dev_bf16, host
from tests.test_gpu_prefix_decode import _decode_case

pytestmark = pytest.mark.gpu


def _codes(g, S, H, D, layout, block):
    codes = g.integers(-127, 128, size=(1, S, H, D)).astype(np.int8)
    scales = g.uniform(0.001, 0.004, size=(1, H, O.scale_count(S, layout, block))).astype(np.float32)
    return codes, scales


def _inputs(D, H, Hk, Sq, Sk, ql, qb, kl, kb, fp8, seed):
    g = np.random.default_rng(seed)
    qc, qs = _codes(g, Sq, H, D, ql, qb)
    kc, ks = _codes(g, Sk, Hk, D, kl, kb)
    v = gen.normal_bf16((1, Sk, Hk, D), g, outliers=3)
    if fp8:
        v8, vs = O.quant_v_fp8(v)
        return qc, qs, kc, ks, v8, vs
    return qc, qs, kc, ks, v, None


def _gpu(qc, qs, ql, qb, kc, ks, kl, kb, v, vs, kv_tile, causal, sinks):
    q, k = sq.QK(dev(qc), dev(qs), ql, qb), sq.QK(dev(kc), dev(ks), kl, kb)
    sk = dev(sinks) if sinks is not None else None
    if vs is not None:
        B, S, H, D = v.shape
        cm = np.zeros((B, H, D, (S + 127) // 128 * 128), np.uint8)   # channel-major FP8 codes
        cm[..., :S] = v.transpose(0, 2, 3, 1)
        out, lse = sq.sq_attn(q, k, dev(cm), dev(vs), 1.0, kv_tile, causal=causal, sinks=sk)
    else:
        out, lse = sq.sq_attn(q, k, dev_bf16(v), None, 1.0, kv_tile, causal=causal, sinks=sk)
    torch.cuda.synchronize()
    return host(out), host(lse)


CASES = [
    # D, H, Hk, Sq, Sk, q layout, k layout, pv, kv_tile, causal, sinks
    (128, 4, 2, 300, 300, (1, 32), (2, 64), "fp8", 128, True, False),     # square: query i sees keys 0 .. i
    (128, 2, 2, 200, 457, (3, 128), (0, 64), "fp8", 128, True, True),     # 257 keys of context before the queries
    (64, 4, 4, 130, 130, (0, 32), (0, 32), "fp8", 128, True, True),
    (128, 4, 1, 333, 333, (0, 64), (0, 64), "bf16", 64, True, False),
    (128, 2, 2, 129, 1000, (1, 32), (2, 64), "bf16", 128, True, True),
    (64, 6, 3, 257, 300, (0, 128), (2, 64), "bf16", 64, True, True),
    (128, 4, 2, 200, 333, (1, 32), (2, 64), "fp8", 128, False, True),     # sinks alone
    (64, 2, 2, 100, 77, (0, 64), (0, 64), "bf16", 64, False, True),
    (128, 2, 2, 1, 1, (0, 64), (0, 64), "fp8", 128, True, True),          # one query, one key
    (64, 2, 1, 1, 190, (0, 64), (0, 64), "bf16", 64, True, False),        # one query after 189 keys
    (128, 4, 2, 300, 300, (1, 32), (2, 64), "fp8", 64, True, True),       # FP8 P.V over 64-key tiles
    (128, 2, 2, 200, 457, (3, 128), (0, 32), "fp8", 64, True, False),
    (64, 2, 2, 33, 97, (0, 64), (2, 64), "fp8", 64, True, True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_causal_sinks_parity(case):
    D, H, Hk, Sq, Sk, (ql, qb), (kl, kb), pv, kvt, causal, use_sinks = case
    print("causal/sinks case", case, flush=True)
    seed = 4000 + D + Sq + Sk + H
    qc, qs, kc, ks, v, vs = _inputs(D, H, Hk, Sq, Sk, ql, qb, kl, kb, pv == "fp8", seed)
    sinks = None
    if use_sinks:
        # logits around the scores' range; one head's sink dominates every score, one is -inf (no sink)
        sinks = np.random.default_rng(seed + 1).uniform(-1.0, 2.0, size=H).astype(np.float32)
        sinks[0] = 6.0
        if H > 2:
            sinks[1] = -np.inf
    ref, rlse, allow = O.attn(O.QK(qc, qs, ql, qb), O.QK(kc, ks, kl, kb), v, vs is not None, vs, kv_tile=kvt,
                              causal=causal, sinks=sinks)
    out, lse = _gpu(qc, qs, ql, qb, kc, ks, kl, kb, v, vs, kvt, causal, sinks)
    check_float(out, ref, allow, what="out")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("pv,kvt", [("fp8", 128), ("fp8", 64), ("bf16", 64), ("bf16", 128)])
def test_last_causal_row_is_the_full_row(pv, kvt):
    """With Sq == Sk the last query sees every key: its causal row equals the non-causal row bit for bit (masked
    keys add exact zeros), and so does its lse."""
    D, H, S = 128, 2, 517
    qc, qs, kc, ks, v, vs = _inputs(D, H, H, S, S, 0, 64, 2, 64, pv == "fp8", 77)
    oc, lc = _gpu(qc, qs, 0, 64, kc, ks, 2, 64, v, vs, kvt, True, None)
    on, ln = _gpu(qc, qs, 0, 64, kc, ks, 2, 64, v, vs, kvt, False, None)
    np.testing.assert_array_equal(oc[:, -1].view(np.uint32), on[:, -1].view(np.uint32))
    np.testing.assert_array_equal(lc[:, :, -1].view(np.uint32), ln[:, :, -1].view(np.uint32))
    assert not np.array_equal(oc[:, :-1], on[:, :-1])


def test_minus_inf_sinks_are_no_sinks():
    D, H, S = 128, 4, 300
    qc, qs, kc, ks, v, vs = _inputs(D, H, 2, S, S, 1, 32, 2, 64, True, 78)
    a = _gpu(qc, qs, 1, 32, kc, ks, 2, 64, v, vs, 128, True, None)
    b = _gpu(qc, qs, 1, 32, kc, ks, 2, 64, v, vs, 128, True, np.full(H, -np.inf, np.float32))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x.view(np.uint32), y.view(np.uint32))


def test_causal_at_size_sampled_rows():
    """A square causal problem of 4096 tokens (32 query blocks per head, the diagonal crossing every wave), checked
    on sampled rows the oracle computes one by one."""
    D, H, Hk, S = 128, 4, 2, 4096
    qc, qs, kc, ks, v, vs = _inputs(D, H, Hk, S, S, 1, 32, 2, 64, True, 79)
    sinks = np.array([0.5, -1.0, 2.0, 1.0], np.float32)
    g = np.random.default_rng(80)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 129, S - 1], g.choice(S, 40, replace=False)])).astype(np.int64)
    ref, rlse, allow, run = O.attn(O.QK(qc, qs, 1, 32), O.QK(kc, ks, 2, 64), v, True, vs, kv_tile=64, rows=rows,
                                   causal=True, sinks=sinks, want_run_allow=True)
    out, lse = _gpu(qc, qs, 1, 32, kc, ks, 2, 64, v, vs, 64, True, sinks)
    check_float(out[:, rows], ref, allow, what="out", run=run)
    np.testing.assert_allclose(lse[:, :, rows], rlse, rtol=0, atol=1e-4)


@pytest.mark.parametrize("Hq,Hk", [(8, 2), (4, 4), (16, 2)])
def test_paged_decode_sinks(Hq, Hk):
    lens = [1, 16, 17, 511, 513, 1100, 37]
    print("decode sinks Hq %d Hk %d" % (Hq, Hk), flush=True)
    q, kc, ks, vc, vs, bt, lens = _decode_case(lens, Hq, Hk, 5000 + Hq + Hk)
    scale = 1.0 / np.sqrt(128.0)
    sinks = np.random.default_rng(Hq).uniform(-1.0, 3.0, size=Hq).astype(np.float32)
    sinks[0] = 8.0            # dominates: the outputs of head 0 shrink well below the others
    sinks[-1] = -np.inf       # no sink
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale, sinks=sinks)
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    out = sq.sq_paged_decode(dev_bf16(q), dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens), int(lens.max()),
                             scale, sinks=dev(sinks))
    torch.cuda.synchronize()
    got = host(out)
    # same bound as the decode without sinks, per head, so the shrunken head is held to its own scale
    for h in range(Hq):
        check_float(got[:, h], ref[:, h], None, what="decode head %d" % h)
    base = sq.sq_paged_decode(dev_bf16(q), dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens), int(lens.max()),
                              scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got[:, -1].view(np.uint32), host(base)[:, -1].view(np.uint32))
