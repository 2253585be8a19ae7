"""The whole path captured in one HIP graph (torch.cuda.CUDAGraph over the library's stream) and replayed: the
calls only enqueue work (no host synchronisation, no device reads on the host, no allocation or memset inside the
library), so a serving loop can record a step once. Every replay, with eager work and synchronisations between
them, must reproduce the eager results bit for bit."""
import numpy as np
import pytest
import torch

import gen
import quantized_transformer_attention_amd as sq
from tests._util import dev, dev_bf16

pytestmark = pytest.mark.gpu


def _inputs():
    c = gen.CFG1
    inp = gen.attn_inputs(c)
    g = gen.rng(2900, 0)
    N, Hq, Hk, D, bs = 2, 8, 2, 128, 16
    lens = np.array([20, 37], np.int32)
    bt = np.array([[2, 0, -1], [1, 3, 4]], np.int32)
    slots = np.array([bt[n, p // bs] * bs + p % bs for n in range(N) for p in range(lens[n])], np.int64)
    kn = gen.to_bf16_bits(g.standard_normal((len(slots), Hk, D)).astype(np.float32))
    vn = gen.to_bf16_bits(g.standard_normal((len(slots), Hk, D)).astype(np.float32))
    qd = gen.normal_bf16((N, 1, Hq, D), g).reshape(N, Hq, D)
    qp = gen.normal_bf16((12, 1, Hq, D), g).reshape(12, Hq, D)
    t = dict(q=dev_bf16(inp.q), k=dev_bf16(inp.k), v=dev_bf16(inp.v), wq=dev_bf16(inp.wq), wk=dev_bf16(inp.wk),
             table=dev(inp.table), sinks=dev(np.array([0.5, -1.0], np.float32)),
             kn=dev_bf16(kn), vn=dev_bf16(vn), slots=dev(slots), bt=dev(bt), lens=dev(lens), qd=dev_bf16(qd),
             qp=dev_bf16(qp), qs=dev(np.array([0, 5, 12], np.int32)),
             kc=torch.zeros((5, bs, Hk, D), dtype=torch.int8, device="cuda"),
             vc=torch.zeros((5, bs, Hk, D), dtype=torch.int8, device="cuda"),
             ks=torch.zeros((5, bs, Hk, D // 32), dtype=torch.float16, device="cuda"),
             vs=torch.zeros((5, bs, Hk, D // 32), dtype=torch.float16, device="cuda"))
    return c, t


def _step(c, t):
    """One pass of every stage; returns the tensors it produced."""
    nq = sq.Norm(sq.NORM_HEAD, t["wq"], None, None, c.eps)
    nk = sq.Norm(sq.NORM_HEAD, t["wk"], None, None, c.eps)
    r = sq.Rope(sq.ROPE_SPLIT_HALF, t["table"])
    ms = sq.sq_norm_stats(t["k"])
    mu = sq.sq_kmean(t["k"], nk, r)
    q = sq.sq_quant_qk(t["q"], nq, r, None, gen.sm_scale_q(c.D), 1e-7, sq.LAYOUT_PER_BLOCK, 64)
    k = sq.sq_quant_qk(t["k"], nk, r, mu, 1.0, 1e-7, sq.LAYOUT_PER_BLOCK, 64)
    v8, vs = sq.sq_quant_v_fp8(t["v"])
    o1, l1 = sq.sq_attn(q, k, t["v"], None, 1.0, 64)
    o2, l2 = sq.sq_attn(q, k, v8, vs, 1.0, 128, causal=True, sinks=t["sinks"])
    om = o1.clone()
    lm = l1.clone()
    sq.sq_lse_merge(om, lm, o2, l2)
    sq.sq_q8_cache_write(t["kn"], t["vn"], t["slots"], t["kc"], t["ks"], t["vc"], t["vs"])
    od = sq.sq_paged_decode(t["qd"], t["kc"], t["ks"], t["vc"], t["vs"], t["bt"], t["lens"], 37, 1.0 / np.sqrt(128))
    op = sq.sq_paged_prefill(t["qp"], t["kc"], t["ks"], t["vc"], t["vs"], t["bt"], t["lens"], t["qs"], 37,
                             1.0 / np.sqrt(128))
    return [ms, mu, q.codes, q.scales, k.codes, k.scales, v8, vs, o1, l1, o2, l2, om, lm, t["kc"], t["ks"], od, op]


def _bits(x):
    return x.detach().cpu().contiguous().view(torch.uint8).numpy()


def test_whole_path_replays_in_a_hip_graph():
    c, t = _inputs()
    eager = [_bits(x) for x in _step(c, t)]
    torch.cuda.synchronize()
    # warm-up on a side stream (default priority), as graph capture asks, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(c, t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = _step(c, t)
    scratch = torch.empty(1 << 22, dtype=torch.float32, device="cuda")
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(eager, outs)):
            assert np.array_equal(a, _bits(b)), "replay %d differs from eager in output %d" % (rep, i)
        # eager work between replays: other kernels on the same stream, and a synchronisation
        scratch.normal_()
        sq.sq_quant_v_fp8(t["v"])
        torch.cuda.synchronize()
