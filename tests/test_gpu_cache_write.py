"""GPU parity of the q8 paged-cache writer (sq_q8_cache_write) against the oracle's quantize-and-scatter:
codes, FP16 scales and every untouched cache row compared bit for bit."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import DEV, dev, host

pytestmark = pytest.mark.gpu


def _bf16_rows(shape, g, scale=1.0):
    """bf16 bits of N(0, scale^2) and the same values as FP32 (exact widening)."""
    bits = gen.to_bf16_bits(g.standard_normal(shape).astype(np.float32) * np.float32(scale))
    return bits, (bits.astype(np.uint32) << 16).view(np.float32)


def _run(k_host, v_host, kf, vf, slots, NB, bs, fp32, seed):
    n, Hk, D = kf.shape
    g = np.random.default_rng(seed)
    # caches start from a seeded fill, so rows the writer must not touch are checked too
    kc0 = g.integers(-128, 128, size=(NB, bs, Hk, D)).astype(np.int8)
    vc0 = g.integers(-128, 128, size=(NB, bs, Hk, D)).astype(np.int8)
    ks0 = g.integers(0, 1 << 16, size=(NB, bs, Hk, D // 32)).astype(np.uint16)
    vs0 = g.integers(0, 1 << 16, size=(NB, bs, Hk, D // 32)).astype(np.uint16)
    kc, vc, ks, vs = kc0.copy(), vc0.copy(), ks0.copy(), vs0.copy()
    O.q8_cache_write(kf, vf, slots, kc, ks, vc, vs)

    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    dkc, dvc, dks, dvs = dev(kc0), dev(vc0), f16(ks0), f16(vs0)
    if fp32:
        dk, dv = dev(kf), dev(vf)
    else:
        dk = dev(k_host.view(np.int16)).view(torch.bfloat16)
        dv = dev(v_host.view(np.int16)).view(torch.bfloat16)
    sq.sq_q8_cache_write(dk, dv, dev(slots), dkc, dks, dvc, dvs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dkc), kc, err_msg="k codes")
    np.testing.assert_array_equal(host(dvc), vc, err_msg="v codes")
    np.testing.assert_array_equal(host(dks.view(torch.int16)).view(np.uint16), ks, err_msg="k scales")
    np.testing.assert_array_equal(host(dvs.view(torch.int16)).view(np.uint16), vs, err_msg="v scales")


CASES = [
    # n tokens, Hk, D, NB, bs, fp32 rows, seed
    (300, 8, 128, 40, 16, False, 1),
    (257, 2, 64, 20, 16, False, 2),
    (129, 4, 128, 12, 16, True, 3),
    (1, 1, 64, 1, 16, True, 4),
    (33, 8, 128, 4, 16, False, 5),
]


@pytest.mark.parametrize("n,Hk,D,NB,bs,fp32,seed", CASES)
def test_cache_write_parity(n, Hk, D, NB, bs, fp32, seed):
    g = gen.rng(2000 + seed, 0)
    kb, kf = _bf16_rows((n, Hk, D), g, 2.0)
    vb, vf = _bf16_rows((n, Hk, D), g, 0.5)
    # a permutation of slots with a few skipped tokens (-1) and one past the cache
    nslots = NB * bs
    slots = g.permutation(nslots)[:n].astype(np.int64) if n <= nslots else g.integers(0, nslots, size=n)
    slots = np.asarray(slots, np.int64)
    if n > 3:
        slots[1] = -1
        slots[n // 2] = nslots + 7
    print("cache write n %d Hk %d D %d NB %d fp32 %s" % (n, Hk, D, NB, fp32), flush=True)
    _run(kb, vb, kf, vf, slots, NB, bs, fp32, seed)


def test_cache_write_ties_and_zero_rows():
    """Group with amax 127 (scale exactly 1): codes of k + 0.5 round half to even; an all-zero group gets
    scale max(0, 1e-8) (FP16 0) and codes 0; a tiny group keeps its own scale."""
    Hk, D = 2, 128
    kf = np.zeros((3, Hk, D), np.float32)
    kf[0, 0, 0] = 127.0
    kf[0, 0, 1:9] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 10.5, 11.5]
    kf[0, 0, 32:64] = 1e-3                       # its own group, scale 1e-3 / 127
    kf[1, 1, 64:96] = np.linspace(-3, 3, 32)
    kb = gen.to_bf16_bits(kf)
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    vb, vf = kb.copy(), kf.copy()
    slots = np.array([3, 0, 17], np.int64)
    _run(kb, vb, kf, vf, slots, 2, 16, False, 9)
    _run(kb, vb, kf, vf, slots, 2, 16, True, 10)


def test_cache_write_then_decode():
    """Rows written by the writer are the q8 cache the decode reads: a decode over a cache filled token by token
    through a block table equals the oracle's decode over the oracle-written cache."""
    N, Hq, Hk, D, bs = 3, 8, 2, 128, 16
    lens = np.array([5, 40, 33], np.int32)
    g = gen.rng(2100, 0)
    pages = [(L + bs - 1) // bs for L in lens]
    NB = sum(pages) + 1
    perm = g.permutation(NB)
    bt = np.full((N, 4), -1, np.int32)
    o = 0
    slots = []
    for n, p in enumerate(pages):
        bt[n, :p] = perm[o:o + p]
        o += p
        slots += [bt[n, pos // bs] * bs + pos % bs for pos in range(lens[n])]
    slots = np.array(slots, np.int64)
    ntok = len(slots)
    kb, kf = _bf16_rows((ntok, Hk, D), g)
    vb, vf = _bf16_rows((ntok, Hk, D), g)
    kc = np.zeros((NB, bs, Hk, D), np.int8)
    vc = np.zeros((NB, bs, Hk, D), np.int8)
    ks = np.zeros((NB, bs, Hk, D // 32), np.uint16)
    vs = np.zeros((NB, bs, Hk, D // 32), np.uint16)
    O.q8_cache_write(kf, vf, slots, kc, ks, vc, vs)
    q = gen.normal_bf16((N, 1, Hq, D), g).reshape(N, Hq, D)
    scale = 1.0 / np.sqrt(D)
    ref = O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale)

    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    dkc, dvc = dev(np.zeros_like(kc)), dev(np.zeros_like(vc))
    dks, dvs = f16(np.zeros_like(ks)), f16(np.zeros_like(vs))
    sq.sq_q8_cache_write(dev(kb.view(np.int16)).view(torch.bfloat16), dev(vb.view(np.int16)).view(torch.bfloat16),
                         dev(slots), dkc, dks, dvc, dvs)
    out = sq.sq_paged_decode(dev(q.view(np.int16)).view(torch.bfloat16), dkc, dks, dvc, dvs, dev(bt), dev(lens),
                             int(lens.max()), scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(dkc), kc)
    got = host(out).astype(np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    assert np.abs(got - ref).max() <= 2e-3 * rms


def test_cache_write_at_size():
    """The benchmarked shape: 131072 new bf16 tokens (Hk 8, d 128) scattered to a random permutation of the slots
    of an 8192 x 16 block cache; every code, scale and untouched row compared bit for bit."""
    n, Hk, D, NB, bs = 131072, 8, 128, 8192, 16
    g = gen.rng(2500, 1)
    kb, kf = _bf16_rows((n, Hk, D), g, 1.0)
    vb, vf = _bf16_rows((n, Hk, D), g, 1.0)
    slots = g.permutation(NB * bs)[:n].astype(np.int64)
    print("cache write at size n %d" % n, flush=True)
    _run(kb, vb, kf, vf, slots, NB, bs, False, 9)
