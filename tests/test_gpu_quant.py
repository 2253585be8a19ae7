"""GPU parity of the prologue and quantizers against the CPU oracle: bit-exact INT8 codes, FP32 scales,
all-heads mean squares, k means and FP8 V codes, on ragged small cases and at the workloads' full sizes."""
import numpy as np
import pytest
import torch

import gen
import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import DEV, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def _pro(norm, rope, w, table, wrows=None, eps=1e-6):
    return O.Prologue(norm=norm, weight=w, weight_rows=wrows, eps=eps, rope=rope, table=table)


def _gpu_specs(norm, rope, w, table, wrows=None, eps=1e-6):
    n = sq.Norm(norm, dev_bf16(w), dev(wrows) if wrows is not None else None, None, eps) if norm else None
    r = sq.Rope(rope, dev(table)) if rope else None
    return n, r


def _case(B, T, H, D, seed, outliers=0):
    g = gen.rng(seed, 0)
    x = gen.normal_bf16((B, T, H, D), g, outliers)
    return x


LAYOUTS = [(0, 32), (0, 64), (0, 128), (1, 32), (2, 64), (3, 128)]


# (mode, pairs): all D/2 pairs, fewer (split half over a pair count that is no multiple of
# a lane's 4 channels, so partners sit in other lanes; interleaved over D/2 - 3)
ROPES = {"none": (O.ROPE_NONE, 0), "split": (O.ROPE_SPLIT_HALF, None), "interleaved_part": (O.ROPE_INTERLEAVED, -3),
         "split_part": (O.ROPE_SPLIT_HALF, 5)}


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("norm", [O.NORM_NONE, O.NORM_HEAD, O.NORM_ALL_HEADS])
@pytest.mark.parametrize("rope_name", list(ROPES))
def test_quant_bit_exact_ragged(D, norm, rope_name):
    B, T, H = 2, 333, 3
    rope, pp = ROPES[rope_name]
    pairs = D // 2 if pp is None else (D // 2 + pp if pp < 0 else D // 4 + pp)
    print("quant D=%d norm=%d rope=%s pairs=%d" % (D, norm, rope_name, pairs), flush=True)
    x = _case(B, T, H, D, 100 + D + 10 * norm + list(ROPES).index(rope_name))
    wd = H * D if norm == O.NORM_ALL_HEADS else D
    w = gen.uniform_bf16((2, wd), gen.rng(7, 1))
    wrows = (np.arange(T) >= 100).astype(np.int32)
    table = gen.rope_table(T, pairs, start=5)
    pro = _pro(norm, rope, w, table, wrows)
    mu = O.kmean(x, pro)
    n, r = _gpu_specs(norm, rope, w, table, wrows)
    xd = dev_bf16(x)
    mu_gpu = sq.sq_kmean(xd, n, r)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(mu_gpu).view(np.uint32), mu.view(np.uint32))
    for layout, block in LAYOUTS:
        for mean, sm in ((None, 0.1275), (mu, 1.0)):
            codes, scales = O.quant_qk(x, pro, layout, block, mean=mean, sm_scale=sm, scale_eps=1e-7)
            res = sq.sq_quant_qk(xd, n, r, dev(mean) if mean is not None else None, sm, 1e-7, layout, block)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(res.scales).view(np.uint32), scales.view(np.uint32),
                                          err_msg="scales layout %d block %d" % (layout, block))
            np.testing.assert_array_equal(host(res.codes), codes, err_msg="codes layout %d block %d" % (layout, block))


def test_norm_stats_bit_exact():
    for D, H in ((128, 40), (64, 7)):
        x = _case(2, 77, H, D, 200 + D, outliers=9)
        ms = O.mean_sq_all_heads(x)
        got = sq.sq_norm_stats(dev_bf16(x))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(got).view(np.uint32), ms.view(np.uint32))


def test_quant_edge_cases():
    D = 128
    # one token; all-zero rows with scale_eps = 0 (scale 0 -> codes 0); strided input (a head slice)
    x = _case(1, 1, 2, D, 300)
    for layout, block in LAYOUTS:
        codes, scales = O.quant_qk(x, O.Prologue(), layout, block)
        res = sq.sq_quant_qk(dev_bf16(x), layout=layout, block=block)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(res.codes), codes)
        np.testing.assert_array_equal(host(res.scales).view(np.uint32), scales.view(np.uint32))
    z = np.zeros((1, 70, 2, D), np.uint16)
    codes, scales = O.quant_qk(z, O.Prologue(), 0, 64, scale_eps=0.0)
    res = sq.sq_quant_qk(dev_bf16(z), layout=0, block=64, scale_eps=0.0)
    torch.cuda.synchronize()
    assert np.all(host(res.codes) == 0) and np.all(codes == 0)
    np.testing.assert_array_equal(host(res.scales), scales)
    big = _case(1, 130, 6, D, 301)
    xd = dev_bf16(big)[:, :, 1:5]            # strided view: heads 1..4 of 6
    codes, scales = O.quant_qk(np.ascontiguousarray(big[:, :, 1:5]), O.Prologue(), 1, 32)
    res = sq.sq_quant_qk(xd, layout=1, block=32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(res.codes), codes)
    np.testing.assert_array_equal(host(res.scales).view(np.uint32), scales.view(np.uint32))


def test_v_fp8_bit_exact():
    for D, T in ((128, 300), (64, 129), (128, 1)):
        v = _case(1, T, 3, D, 400 + T, outliers=5)
        codes, vs = O.quant_v_fp8(v)
        c_gpu, vs_gpu = sq.sq_quant_v_fp8(dev_bf16(v))
        torch.cuda.synchronize()
        cg = host(c_gpu)                                   # (B, H, D, Tpad)
        np.testing.assert_array_equal(host(vs_gpu).view(np.uint32), vs.view(np.uint32))
        np.testing.assert_array_equal(cg[..., :T], codes.transpose(0, 2, 3, 1))
        assert np.all(cg[..., T:] == 0)


def test_cfg2_video_quantizers_full_size():
    """Video workload at full size (1 x 32760 x 40 x 128, 1% outlier channels): all-heads norm + RoPE,
    THREAD_Q q, k mean + THREAD_K k, V to FP8, bit-exact on every element."""
    c = gen.CFG2
    inp = gen.attn_inputs(c)
    print("cfg2 inputs ready", flush=True)
    pq = _pro(O.NORM_ALL_HEADS, O.ROPE_SPLIT_HALF, inp.wq, inp.table, eps=c.eps)
    pk = _pro(O.NORM_ALL_HEADS, O.ROPE_SPLIT_HALF, inp.wk, inp.table, eps=c.eps)
    nq, r = _gpu_specs(O.NORM_ALL_HEADS, O.ROPE_SPLIT_HALF, inp.wq, inp.table, eps=c.eps)
    nk, _ = _gpu_specs(O.NORM_ALL_HEADS, O.ROPE_SPLIT_HALF, inp.wk, inp.table, eps=c.eps)
    qd, kd, vd = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    ms = sq.sq_norm_stats(kd)
    mu_gpu = sq.sq_kmean(kd, nk, r)
    qq = sq.sq_quant_qk(qd, nq, r, None, gen.sm_scale_q(c.D), 1e-7, O.LAYOUT_THREAD_Q, 32)
    kq = sq.sq_quant_qk(kd, nk, r, mu_gpu, 1.0, 1e-7, O.LAYOUT_THREAD_K, 64)
    v8, vs = sq.sq_quant_v_fp8(vd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(ms).view(np.uint32), O.mean_sq_all_heads(inp.k).view(np.uint32))
    mu = O.kmean(inp.k, pk)
    np.testing.assert_array_equal(host(mu_gpu).view(np.uint32), mu.view(np.uint32))
    print("cfg2 k mean ok", flush=True)
    codes, scales = O.quant_qk(inp.q, pq, O.LAYOUT_THREAD_Q, 32, sm_scale=gen.sm_scale_q(c.D))
    np.testing.assert_array_equal(host(qq.scales).view(np.uint32), scales.view(np.uint32))
    np.testing.assert_array_equal(host(qq.codes), codes)
    codes, scales = O.quant_qk(inp.k, pk, O.LAYOUT_THREAD_K, 64, mean=mu)
    np.testing.assert_array_equal(host(kq.scales).view(np.uint32), scales.view(np.uint32))
    np.testing.assert_array_equal(host(kq.codes), codes)
    vc, vsc = O.quant_v_fp8(inp.v)
    np.testing.assert_array_equal(host(vs).view(np.uint32), vsc.view(np.uint32))
    np.testing.assert_array_equal(host(v8)[..., :c.Sk], vc.transpose(0, 2, 3, 1))


def test_cfg4_quantizer_full_size_sampled_heads():
    """Quantizer workload at full size (2 x 75600 x 40 x 128), every layout, checked on sampled heads
    (the per-head norm makes heads independent; the oracle runs on the sampled head slices)."""
    c = gen.CFG4
    x, w, table = gen.quant_inputs(c)
    print("cfg4 inputs ready", flush=True)
    pro = _pro(O.NORM_HEAD, O.ROPE_SPLIT_HALF, w, table, eps=c.eps)
    n, r = _gpu_specs(O.NORM_HEAD, O.ROPE_SPLIT_HALF, w, table, eps=c.eps)
    xd = dev_bf16(x)
    heads = [0, 17, 39]
    xs = np.ascontiguousarray(x[:, :, heads])
    mu_gpu = sq.sq_kmean(xd, n, r)
    torch.cuda.synchronize()
    mu = O.kmean(xs, pro)
    np.testing.assert_array_equal(host(mu_gpu)[:, heads].view(np.uint32), mu.view(np.uint32))
    smq = gen.sm_scale_q(c.D)
    for layout, block, mean, sm in ((0, 128, None, smq), (1, 32, None, smq), (3, 128, None, smq), (0, 64, mu, 1.0),
                                    (2, 64, mu, 1.0)):
        res = sq.sq_quant_qk(xd, n, r, mu_gpu if mean is not None else None, sm, 1e-7, layout, block)
        torch.cuda.synchronize()
        codes, scales = O.quant_qk(xs, pro, layout, block, mean=mean, sm_scale=sm)
        np.testing.assert_array_equal(host(res.scales)[:, heads].view(np.uint32), scales.view(np.uint32))
        np.testing.assert_array_equal(host(res.codes)[:, :, heads], codes)
        print("cfg4 layout %d ok" % layout, flush=True)


def test_results_do_not_depend_on_the_grid():
    """The same rows launched as different grids: the whole (B, H) batch, one batch item at a time, and single heads
    of a strided view (the grids of the norm statistics, k mean, quantizer and V quantizer all scale with B and H).
    Every result is bit-identical: no kernel's arithmetic depends on which workgroup or XCD ran an item."""
    B, T, H, D = 2, 333, 6, 128
    x = _case(B, T, H, D, 777, outliers=3)
    w_all = gen.uniform_bf16((1, H * D), gen.rng(8, 1))
    w_head = gen.uniform_bf16((1, D), gen.rng(8, 2))
    table = gen.rope_table(T, D // 2, start=2)
    xd = dev_bf16(x)
    # all-heads norm: full batch against one batch item at a time
    na, r = _gpu_specs(O.NORM_ALL_HEADS, O.ROPE_SPLIT_HALF, w_all, table)
    ms = sq.sq_norm_stats(xd)
    mu = sq.sq_kmean(xd, na, r)
    res = sq.sq_quant_qk(xd, na, r, mu, 1.0, 1e-7, O.LAYOUT_THREAD_K, 64)
    v8, vs = sq.sq_quant_v_fp8(xd)
    torch.cuda.synchronize()
    for b in range(B):
        xb = xd[b:b + 1]
        ms_b = sq.sq_norm_stats(xb)
        mu_b = sq.sq_kmean(xb, na, r)
        res_b = sq.sq_quant_qk(xb, na, r, mu_b, 1.0, 1e-7, O.LAYOUT_THREAD_K, 64)
        v8_b, vs_b = sq.sq_quant_v_fp8(xb)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(ms_b).view(np.uint32), host(ms)[b:b + 1].view(np.uint32))
        np.testing.assert_array_equal(host(mu_b).view(np.uint32), host(mu)[b:b + 1].view(np.uint32))
        np.testing.assert_array_equal(host(res_b.codes), host(res.codes)[b:b + 1])
        np.testing.assert_array_equal(host(res_b.scales).view(np.uint32), host(res.scales)[b:b + 1].view(np.uint32))
        np.testing.assert_array_equal(host(v8_b), host(v8)[b:b + 1])
        np.testing.assert_array_equal(host(vs_b).view(np.uint32), host(vs)[b:b + 1].view(np.uint32))
    # per-head norm: all heads against single heads of a strided view
    nh, _ = _gpu_specs(O.NORM_HEAD, O.ROPE_SPLIT_HALF, w_head, table)
    mu = sq.sq_kmean(xd, nh, r)
    res = sq.sq_quant_qk(xd, nh, r, mu, 1.0, 1e-7, O.LAYOUT_THREAD_Q, 32)
    torch.cuda.synchronize()
    for h in (0, 3, 5):
        xh = xd[:, :, h:h + 1]
        mu_h = sq.sq_kmean(xh, nh, r)
        res_h = sq.sq_quant_qk(xh, nh, r, mu_h, 1.0, 1e-7, O.LAYOUT_THREAD_Q, 32)
        v8_h, vs_h = sq.sq_quant_v_fp8(xh)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(mu_h).view(np.uint32), host(mu)[:, h:h + 1].view(np.uint32))
        np.testing.assert_array_equal(host(res_h.codes), host(res.codes)[:, :, h:h + 1])
        np.testing.assert_array_equal(host(res_h.scales).view(np.uint32), host(res.scales)[:, h:h + 1].view(np.uint32))
        np.testing.assert_array_equal(host(v8_h), host(v8)[:, h:h + 1])
        np.testing.assert_array_equal(host(vs_h).view(np.uint32), host(vs)[:, h:h + 1].view(np.uint32))


TRACE_SCRIPT = r"""
import numpy as np, torch
import quantized_transformer_attention_amd as sq
x = torch.zeros((1, 300, 3, 128), dtype=torch.bfloat16, device="cuda:0")
res = sq.sq_quant_qk(x, layout=sq.LAYOUT_PER_BLOCK, block=64)
torch.cuda.synchronize()
print("done", flush=True)
"""


def test_launch_trace_names_every_launch():
    """SQ_TRACE=1 logs each launch (kernel, grid, block) to stderr: the quantizer of 300 tokens x 3 heads is
    ceil(300 / 128) x 3 = 9 items on a grid rounded up to a multiple of the 8 XCDs."""
    import os
    import subprocess
    import sys
    env = dict(os.environ, SQ_TRACE="1")
    r = subprocess.run([sys.executable, "-c", TRACE_SCRIPT], capture_output=True, text=True, env=env, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    print(r.stderr[-2000:])
    assert r.returncode == 0 and "done" in r.stdout
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("sq_trace: ")]
    assert len(lines) == 1, lines
    assert "k_quant_qk" in lines[0] and "grid=(16,1,1)" in lines[0] and "block=256" in lines[0]
