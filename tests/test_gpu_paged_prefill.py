"""GPU parity of the paged causal prefill over a q8 cache (sq_paged_prefill) against the oracle's binary64
[impl] _prefill_torch_from_cache.

Tolerance: every element within 2e-3 rms(row) and ||gpu - ref|| <= 2e-3 ||ref|| per (token, head) row, the row
being that query's own attention output (the rows of a batch attend 1 to thousands of keys, so their output RMS
differs by orders of magnitude). The kernel's arithmetic: values exact (code scale as two f16 halves), keys as
f16(code scale) plus the remainder rounded to e4m3 with a power-of-two block scale (a key off by at most 2^-16 of
itself), q as f16 after a power-of-two rescale with an e4m3 copy for the remainder products, P rounded once to f16
(relative <= 2^-11), its denominator summed from the same rounded P; a CPU emulation of that arithmetic gives at
most 1.1e-3 rms(row) per element on these inputs."""
import math

import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import dev, dev_bf16, host

pytestmark = pytest.mark.gpu

ROW_REL, ELEM_REL = 2e-3, 2e-3


def check_rows(got, ref, what=""):
    got = got.astype(np.float64)
    err = got - ref
    nrm = np.sqrt(np.sum(ref * ref, axis=-1))
    rel = np.sqrt(np.sum(err * err, axis=-1)) / nrm
    rms = nrm[..., None] / math.sqrt(ref.shape[-1])
    bad = np.abs(err) > ELEM_REL * rms
    assert rel.max() <= ROW_REL, "%s: row relative error %.3g (row %s)" % (what, rel.max(), np.unravel_index(rel.argmax(), rel.shape))
    assert not bad.any(), "%s: %d elements beyond %.0e rms(row)" % (what, int(bad.sum()), ELEM_REL)
    print("%s: row error %.3g, element error %.3g rms(row)" % (what, rel.max(), float((np.abs(err) / rms).max())),
          flush=True)
    return float(rel.max())


def _case(seed, ctx, qlen, Hq, Hk, D=128, bs=16, extra=3, q_f16=False):
    """Varlen batch over a paged q8 cache: sequence n has ctx[n] cached keys before its qlen[n] queries (their
    keys in the cache as well), pages dealt from a seeded permutation, table rows padded with -1."""
    g = np.random.default_rng(seed)
    lens = np.array(ctx, np.int32) + np.array(qlen, np.int32)
    pages = [(int(L) + bs - 1) // bs for L in lens]
    NB = sum(pages) + extra
    kc, ks = O.q8_quantize(g.standard_normal((NB, bs, Hk, D)).astype(np.float32))
    vc, vs = O.q8_quantize(g.standard_normal((NB, bs, Hk, D)).astype(np.float32))
    perm = g.permutation(NB)
    bt = np.full((len(lens), max(pages) + 2), -1, np.int32)
    o = 0
    for n, p in enumerate(pages):
        bt[n, :p] = perm[o:o + p]
        o += p
    qs = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    if q_f16:   # binary16 queries
        q = (g.standard_normal(size=(int(qs[-1]), Hq, D)) * 4).astype(np.float16)
    else:
        q = gen.normal_bf16((int(qs[-1]), 1, Hq, D), g).reshape(-1, Hq, D)
    return q, kc, ks, vc, vs, bt, lens, qs


def _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale, sinks=None, max_len=None):
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    out = sq.sq_paged_prefill(dev(q) if q.dtype == np.float16 else dev_bf16(q), dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens), dev(qs),
                              int(lens.max()) if max_len is None else max_len, scale,
                              sinks=dev(sinks) if sinks is not None else None)
    torch.cuda.synchronize()
    return host(out)


CASES = [
    # contexts, query lengths, Hq, Hk
    ((0, 100, 300), (90, 33, 1), 8, 2),            # a fresh prompt, a chunk after 100 keys, a decode-like row
    ((0, 7), (200, 150), 4, 4),                    # G = 1: 128-token q blocks
    ((500, 0, 64), (64, 17, 129), 16, 2),          # G = 8: 16-token q blocks
    ((31, 0, 1000, 5), (40, 0, 77, 300), 8, 4),    # an empty sequence in the middle; G = 2
    ((2048,), (1,), 32, 8),                        # one query after a long context
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_paged_prefill_parity(case):
    ctx, qlen, Hq, Hk = case
    print("prefill case", case, flush=True)
    q, kc, ks, vc, vs, bt, lens, qs = _case(6000 + sum(ctx) + sum(qlen) + Hq, ctx, qlen, Hq, Hk)
    scale = 1 / math.sqrt(128)
    ref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
    got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale)
    rel = check_rows(got, ref, "prefill")
    print("max row rel %.3g" % rel)


@pytest.mark.parametrize("D,q_f16", [(64, False), (64, True), (128, True)])
def test_paged_prefill_head_dims_and_q_dtypes(D, q_f16):
    """Head dim 64 and binary16 queries, ragged varlen batch with G = 1, 2 and 8 launches."""
    for ctx, qlen, Hq, Hk in (((0, 100, 300), (90, 33, 1), 8, 4), ((0, 7), (200, 150), 4, 4), ((64,), (129,), 16, 2)):
        print("prefill D %d q_f16 %d" % (D, q_f16), ctx, qlen, Hq, Hk, flush=True)
        q, kc, ks, vc, vs, bt, lens, qs = _case(6200 + D + sum(ctx) + Hq, ctx, qlen, Hq, Hk, D=D, q_f16=q_f16)
        scale = 1 / math.sqrt(D)
        ref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
        got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale)
        check_rows(got, ref, "prefill D %d" % D)


def _case_spread(seed, ctx, qlen, Hq, Hk, D=128, bs=16, extra=3, k_spread=6, v_spread=2):
    """Varlen batch whose cached rows carry a power of two per (key, 32-channel group): 2^U{-k_spread..k_spread}
    for keys, 2^U{-v_spread..v_spread} for values, so the FP16 group scales of a key (and of neighbouring keys)
    differ by up to 2^(2 spread); q ~ N(0, 1/64) keeps the scores moderate."""
    g = np.random.default_rng(seed)
    lens = np.array(ctx, np.int32) + np.array(qlen, np.int32)
    pages = [(int(L) + bs - 1) // bs for L in lens]
    NB = sum(pages) + extra

    def rows(spread):
        x = g.standard_normal((NB, bs, Hk, D // 32, 32))
        x *= np.exp2(g.integers(-spread, spread + 1, size=(NB, bs, Hk, D // 32, 1)))
        return O.q8_quantize(x.reshape(NB, bs, Hk, D).astype(np.float32))

    kc, ks = rows(k_spread)
    vc, vs = rows(v_spread)
    perm = g.permutation(NB)
    bt = np.full((len(lens), max(pages) + 2), -1, np.int32)
    o = 0
    for n, p in enumerate(pages):
        bt[n, :p] = perm[o:o + p]
        o += p
    qs = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    q = gen.normal_bf16((int(qs[-1]), 1, Hq, D), g).reshape(-1, Hq, D)
    q = gen.to_bf16_bits(gen.from_bf16_bits(q) * 0.125)
    return q, kc, ks, vc, vs, bt, lens, qs


@pytest.mark.parametrize("D", [64, 128])
def test_paged_prefill_scale_exponents_spread(D):
    """Group scales whose exponents differ across the groups of a key and across keys (keys by up to 2^12, values
    by up to 2^4): the keys' FP8 remainders take one power-of-two block scale per (key, group), so a scale applied
    to the wrong group or key shows here as errors far above the bound. (Values spread much wider would test the
    f16 rounding of P against the per-element bound rather than the scales.)"""
    for ctx, qlen, Hq, Hk in (((0, 300), (130, 70), 8, 2), ((77,), (200,), 4, 4)):
        print("prefill spread D %d" % D, ctx, qlen, Hq, Hk, flush=True)
        q, kc, ks, vc, vs, bt, lens, qs = _case_spread(6300 + D + sum(ctx) + Hq, ctx, qlen, Hq, Hk, D=D)
        scale = 1 / math.sqrt(D)
        ref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
        got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale)
        check_rows(got, ref, "prefill spread D %d" % D)


def test_paged_prefill_sinks_and_max_len_bound():
    """Per-head sinks (one dominant, one -inf), and a max_seq_len host bound above every length."""
    Hq, Hk = 8, 2
    q, kc, ks, vc, vs, bt, lens, qs = _case(6101, (0, 200), (150, 70), Hq, Hk, extra=8)
    scale = 1 / math.sqrt(128)
    sinks = np.array([0.5, 4.0, -1.0, -np.inf, 2.0, 0.0, 1.0, -3.0], np.float32)
    ref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale, sinks=sinks)
    max_len = bt.shape[1] * 16                     # the table's whole reach: above every length
    assert max_len > lens.max()
    got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale, sinks=sinks, max_len=max_len)
    check_rows(got, ref, "prefill sinks")
    base = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale)
    np.testing.assert_array_equal(got[:, 3].view(np.uint32), base[:, 3].view(np.uint32))   # -inf sink: no sink


def test_paged_prefill_garbage_in_unused_slots_and_pages():
    """Slots past a sequence's length and blocks it does not own hold NaN scales and random codes: no row may
    see them (the kernel zeroes the scales of keys past the length before they reach the products)."""
    Hq, Hk = 8, 2
    q, kc, ks, vc, vs, bt, lens, qs = _case(6102, (10, 45), (20, 30), Hq, Hk, extra=4)
    scale = 1 / math.sqrt(128)
    ref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, scale)
    nan16 = np.uint16(0x7e00)
    used = set()
    for n, L in enumerate(lens):
        for pos in range(int(L)):
            used.add((int(bt[n, pos // 16]), pos % 16))
    for b in range(kc.shape[0]):
        for s in range(16):
            if (b, s) not in used:
                ks[b, s] = nan16
                vs[b, s] = nan16
    got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale)
    assert np.isfinite(got).all()
    check_rows(got, ref, "prefill with garbage")


def test_paged_prefill_last_rows_match_decode():
    """The last query of each sequence sees its whole sequence: it is the paged decode's row (both within the
    float tolerance of the same oracle row, and close to each other)."""
    Hq, Hk = 8, 2
    q, kc, ks, vc, vs, bt, lens, qs = _case(6103, (0, 300, 17), (64, 1, 200), Hq, Hk)
    scale = 1 / math.sqrt(128)
    got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, scale)
    last = qs[1:] - 1
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    dec = sq.sq_paged_decode(dev_bf16(q[last]), dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens),
                             int(lens.max()), scale)
    torch.cuda.synchronize()
    ref = O.paged_decode(q[last], kc, ks, vc, vs, bt, lens, scale)
    check_rows(got[last], ref, "prefill last rows")
    check_rows(host(dec), ref, "decode rows")


def test_chunked_prefill_through_the_cache_writer():
    """Chunked prefill as an engine runs it: each chunk's keys and values are quantized into the paged cache by
    sq_q8_cache_write, then the chunk attends the cache; the outputs of all chunks equal a one-shot prefill of
    the whole prompt over the same cache (row for row, bit for bit: a row depends only on the keys it sees) and
    the oracle."""
    Hq, Hk, D, bs = 8, 2, 128, 16
    g = np.random.default_rng(6104)
    S = 700
    pages = (S + bs - 1) // bs
    NB = pages + 5
    bt = np.full((1, pages + 1), -1, np.int32)
    bt[0, :pages] = g.permutation(NB)[:pages]
    k = gen.to_bf16_bits(g.standard_normal((S, Hk, D)).astype(np.float32))
    v = gen.to_bf16_bits(g.standard_normal((S, Hk, D)).astype(np.float32))
    q = gen.normal_bf16((S, 1, Hq, D), g).reshape(S, Hq, D)
    slots = np.array([bt[0, p // bs] * bs + p % bs for p in range(S)], np.int64)
    kc, vc = dev(np.zeros((NB, bs, Hk, D), np.int8)), dev(np.zeros((NB, bs, Hk, D), np.int8))
    ksd = dev(np.zeros((NB, bs, Hk, D // 32), np.int16)).view(torch.float16)
    vsd = dev(np.zeros((NB, bs, Hk, D // 32), np.int16)).view(torch.float16)
    kd = dev(k.view(np.int16)).view(torch.bfloat16)
    vd = dev(v.view(np.int16)).view(torch.bfloat16)
    qd = dev_bf16(q)
    btd = dev(bt)
    scale = 1 / math.sqrt(D)
    chunks = [(0, 256), (256, 300), (300, 640), (640, 700)]
    outs = []
    for a, b in chunks:
        sq.sq_q8_cache_write(kd[a:b], vd[a:b], dev(slots[a:b]), kc, ksd, vc, vsd)
        outs.append(sq.sq_paged_prefill(qd[a:b], kc, ksd, vc, vsd, btd, dev(np.array([b], np.int32)),
                                        dev(np.array([0, b - a], np.int32)), S, scale))
    whole = sq.sq_paged_prefill(qd, kc, ksd, vc, vsd, btd, dev(np.array([S], np.int32)),
                                dev(np.array([0, S], np.int32)), S, scale)
    torch.cuda.synchronize()
    chunked = np.concatenate([host(o) for o in outs])
    np.testing.assert_array_equal(chunked.view(np.uint32), host(whole).view(np.uint32))
    kch = host(kc)
    ksh = host(ksd.view(torch.int16)).view(np.uint16)
    vch = host(vc)
    vsh = host(vsd.view(torch.int16)).view(np.uint16)
    rows = np.array([0, 1, 255, 256, 299, 300, 450, 639, 640, 699], np.int64)
    ref = O.paged_prefill(q, kch, ksh, vch, vsh, bt, np.array([S], np.int32), np.array([0, S], np.int32), scale,
                          rows=rows)
    check_rows(chunked[rows], ref, "chunked prefill")


def test_paged_prefill_at_size_sampled_rows():
    """The benchmarked shape: 16 sequences with contexts ~U(0, 8192) and 1024-token chunks, Hq 32 / Hk 8, checked
    on sampled rows (first, last and random tokens of every sequence)."""
    c = gen.PREFILL
    q, kc, ks, vc, vs, bt, lens, qs = gen.prefill_case(c)
    g = np.random.default_rng(7)
    rows = []
    for n in range(c.N):
        a, b = int(qs[n]), int(qs[n + 1])
        rows += [a, b - 1] + list(g.integers(a, b, size=2))
    rows = np.unique(np.array(rows, np.int64))
    ref = O.paged_prefill(q, kc, ks, vc, vs, bt, lens, qs, c.scale, rows=rows)
    got = _gpu(q, kc, ks, vc, vs, bt, lens, qs, c.scale, max_len=c.max_len)
    check_rows(got[rows], ref, "prefill at size")
