#!/usr/bin/env python3
"""Throughput of the quantized attention path on one MI355X (gfx950).

A step is one pass of the whole path over one batch of seeded synthetic input, every
stage in the library's HIP kernels:
  video (default; the workload the TFLOPS metric is quoted on): B=1, H=40, D=128,
    Sq=Sk=32760, 1% outlier channels x20 -> all-heads mean squares of q and k, k mean,
    fused norm + RoPE + INT8 quantization of q (THREAD_Q) and k (THREAD_K, k mean
    subtracted), V to FP8 per channel, attention core with FP8 P.V;
  causal: the video pipeline with a causal mask and per-head sinks in the core;
  joint: the video recipe's projected pass at H=24, 8704 tokens (PER_BLOCK q 128 / k 64,
    bf16 P.V) plus the 4096-token q8 prefix pass merged by log-sum-exp;
  quantizer: k mean + the five quantizer runs of a 2 x 75600 x 40 x 128 tensor;
  decode: paged GQA decode of 64 sequences over a q8 cache;
  prefill: paged causal chunked prefill of 16 sequences (1024-token chunks) over a q8 cache.
value = the workload's algorithmic work / the step time (TFLOPS = 4 B H Sq Sk D for the
attention workloads; GB/s of algorithmic bytes for the quantizer and decode).

Prints ONE JSON line. roofline: the dominant kernel's algorithmic rate, from HIP events
around its launches on the stream it runs on, against MI355X's published peak; traffic
from the committed rocprofv3 counter summary when it was taken on the current kernel
source. cpu_baseline (video, quantizer and decode workloads): the CPU oracle timed on this
host on the same seeded inputs, in full where it finishes in seconds, else on sampled
query rows with the full-size time extrapolated (the sample is named in the line).

`python bench.py traffic ...` (see traffic_main) turns rocprofv3 FETCH_SIZE / WRITE_SIZE
counter runs into the HBM bytes per launch stored in profiles/traffic.json.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS_INT8 = 5000.0        # dense INT8 (and FP8) MFMA, POP/s -> TFLOP/s units
PEAK_TFLOPS_BF16 = 2500.0        # dense bf16 and f16 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "quantized_transformer_attention_amd", "csrc")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video",
                    choices=["video", "causal", "joint", "quantizer", "decode", "prefill", "cachewrite", "merge",
                             "copy"],
                    help="copy: a plain 1 GiB device copy, the reference for scaling HBM byte counters")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time for the baseline")
    return ap.parse_args()


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, files, units_per_launch: float):
    """HBM bytes per launch from the committed counter summary, or None when absent or stale."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_sha") != source_sha(files) or e.get("units") != units_per_launch:
        return None
    return e.get("bytes_per_launch")


class Timer:
    """HIP events on torch's current stream, which is the stream every library call enqueues on."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def __call__(self, name, fn):
        t = self.torch
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        r = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return r

    def avg_ms(self, name):
        p = self.pairs.get(name, [])
        return sum(s.elapsed_time(e) for s, e in p) / len(p) if p else float("nan")

    def reset(self):
        self.pairs = {}


# ---------------------------------------------------------------------------------------------- workloads
def video_like(args, torch, sq, gen, c, timer, causal=False, sinks=None):
    """Build the video-style pipeline (also the joint workload's projected pass and the causal variant)."""
    import numpy as np

    dev = torch.device("cuda:0")
    inp = gen.attn_inputs(c)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kd, vd = bf(inp.q), bf(inp.k), bf(inp.v)
    table = torch.from_numpy(inp.table).to(dev)
    wr = torch.from_numpy(inp.weight_rows).to(dev) if inp.weight_rows is not None else None
    all_heads = c.norm == "all_heads"
    mode = sq.NORM_ALL_HEADS if all_heads else sq.NORM_HEAD
    wq, wk = bf(inp.wq), bf(inp.wk)
    rope = sq.Rope(sq.ROPE_SPLIT_HALF, table)
    ql, qb = gen.LAYOUT[c.q_layout], c.q_block
    kl, kb = gen.LAYOUT[c.k_layout], c.k_block
    smq = gen.sm_scale_q(c.D)
    wsp = {n: sq.Workspace(dev) for n in ("kmean", "q", "k", "v", "attn")}
    elems = c.B * c.Sq * c.H * c.D

    def step():
        if all_heads:
            msq = timer("norm_stats_q", lambda: sq.sq_norm_stats(qd))
            msk = timer("norm_stats_k", lambda: sq.sq_norm_stats(kd))
        else:
            msq = msk = None
        nq = sq.Norm(mode, wq, wr, msq, c.eps)
        nk = sq.Norm(mode, wk, wr, msk, c.eps)
        mu = timer("kmean", lambda: sq.sq_kmean(kd, nk, rope, workspace=wsp["kmean"]))
        q = timer("quant_q", lambda: sq.sq_quant_qk(qd, nq, rope, None, smq, 1e-7, ql, qb, workspace=wsp["q"]))
        k = timer("quant_k", lambda: sq.sq_quant_qk(kd, nk, rope, mu, 1.0, 1e-7, kl, kb, workspace=wsp["k"]))
        if c.pv == "fp8":
            v8, vs = timer("quant_v", lambda: sq.sq_quant_v_fp8(vd, workspace=wsp["v"]))
            out, lse = timer("attn", lambda: sq.sq_attn(q, k, v8, vs, 1.0, c.kv_tile, workspace=wsp["attn"],
                                                        causal=causal, sinks=sinks))
        else:
            out, lse = timer("attn", lambda: sq.sq_attn(q, k, vd, None, 1.0, c.kv_tile, workspace=wsp["attn"],
                                                        causal=causal, sinks=sinks))
        return q, mu, out, lse

    bytes_ = {
        "norm_stats_q": elems * 2 + c.B * c.Sq * 4, "norm_stats_k": elems * 2 + c.B * c.Sk * 4,
        "kmean": elems * 2, "quant_q": elems * 3, "quant_k": elems * 3, "quant_v": elems * 5,
    }
    return step, bytes_, inp


def run_video(args, torch, sq, gen, timer):
    c = gen.CFG2
    step, bytes_, inp = video_like(args, torch, sq, gen, c, timer)
    flops = c.flops()
    res = time_steps(args, torch, step, timer)
    attn_ms = timer.avg_ms("attn")
    achieved = flops / (attn_ms * 1e-3) / 1e12
    files = ["attn.hip", "device.h", "sq_internal.h"]
    line = {
        "metric": "quantized-attention TFLOPS (4*B*H*Sq*Sk*d) and % of gfx950 INT8 MFMA peak",
        "value": flops / (res["ms"] * 1e-3) / 1e12, "unit": "TFLOPS",
        "dtype": "i8",
        "config": {"workload": "video self-attention B=1 H=40 Sq=Sk=32760 d=128, THREAD_Q/THREAD_K INT8, FP8 P.V",
                   "B": c.B, "H": c.H, "Sq": c.Sq, "Sk": c.Sk, "head_dim": c.D, "kv_tile": c.kv_tile},
        "roofline": {"bound": "mfma", "kernel": "k_attn", "achieved": achieved, "peak": PEAK_TFLOPS_INT8,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS_INT8,
                     "traffic": traffic_for("k_attn_video", files, flops),
                     "avg_launch_ms": attn_ms, "flops_per_launch": flops},
        "stages_ms": {n: timer.avg_ms(n) for n in timer.pairs},
        "stages_gbs": {n: b / (timer.avg_ms(n) * 1e-3) / 1e9 for n, b in bytes_.items()},
        "core_pct_of_int8_peak": 100.0 * achieved / PEAK_TFLOPS_INT8,
    }
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_video(args, c, inp)
    return res, line


def run_causal(args, torch, sq, gen, timer):
    """The video pipeline with a causal mask and per-head sinks in the core: query i sees keys 0 .. i, so the
    work is 4 B H d S (S + 1) / 2 (the visible query-key pairs)."""
    import numpy as np

    c = gen.CFG2
    sinks = torch.from_numpy(gen.rng(c.seed, gen.S_EXTRA).uniform(-1.0, 2.0, size=c.H).astype(np.float32)).cuda()
    step, bytes_, _ = video_like(args, torch, sq, gen, c, timer, causal=True, sinks=sinks)
    flops = 4.0 * c.B * c.H * c.D * c.Sq * (c.Sq + 1) / 2
    res = time_steps(args, torch, step, timer)
    attn_ms = timer.avg_ms("attn")
    achieved = flops / (attn_ms * 1e-3) / 1e12
    files = ["attn.hip", "device.h", "sq_internal.h"]
    line = {
        "metric": "causal quantized-attention TFLOPS (4*B*H*d*S*(S+1)/2 visible pairs) and % of INT8 MFMA peak",
        "value": flops / (res["ms"] * 1e-3) / 1e12, "unit": "TFLOPS", "dtype": "i8",
        "config": {"workload": "causal self-attention with per-head sinks, B=1 H=40 Sq=Sk=32760 d=128, "
                               "THREAD_Q/THREAD_K INT8, FP8 P.V", "B": c.B, "H": c.H, "Sq": c.Sq, "Sk": c.Sk,
                   "head_dim": c.D, "kv_tile": c.kv_tile, "causal": True, "sinks": True},
        "roofline": {"bound": "mfma", "kernel": "k_attn", "achieved": achieved, "peak": PEAK_TFLOPS_INT8,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS_INT8,
                     "traffic": traffic_for("k_attn_causal", files, flops),
                     "avg_launch_ms": attn_ms, "flops_per_launch": flops},
        "stages_ms": {n: timer.avg_ms(n) for n in timer.pairs},
    }
    return res, line


def run_joint(args, torch, sq, gen, timer):
    import numpy as np

    c = gen.CFG3
    step_proj, bytes_, _ = video_like(args, torch, sq, gen, c, timer)
    dev = torch.device("cuda:0")
    g = gen.rng(c.seed, gen.S_EXTRA)
    kc, ks = gen.q8_like((1, c.prefix, c.Hk, c.D), g)
    vc, vs = gen.q8_like((1, c.prefix, c.Hk, c.D), g)
    f16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.float16).to(dev)
    pre = sq.Q8Prefix(torch.from_numpy(kc).to(dev), f16(ks), torch.from_numpy(vc).to(dev), f16(vs))

    def step():
        q, mu, out, lse = step_proj()
        timer("prefix", lambda: sq.sq_attn_prefix_lse_merge(q, pre, mu, out, lse, 1.0, c.kv_tile))

    f_proj = c.flops()
    f_pre = 4.0 * c.B * c.H * c.Sq * c.prefix * c.D
    res = time_steps(args, torch, step, timer)
    attn_ms, pre_ms = timer.avg_ms("attn"), timer.avg_ms("prefix")
    achieved = f_proj / (attn_ms * 1e-3) / 1e12
    line = {
        "metric": "quantized-attention TFLOPS (4*B*H*Sq*Sk*d) and % of gfx950 INT8 MFMA peak",
        "value": (f_proj + f_pre) / (res["ms"] * 1e-3) / 1e12, "unit": "TFLOPS", "dtype": "i8",
        "config": {"workload": "joint text+image attention, 512 + 8192 projected tokens + 4096-token q8 prefix, "
                               "H=24 d=128, bf16 P.V", "B": c.B, "H": c.H, "Sq": c.Sq, "Sk": c.Sk, "prefix": c.prefix,
                   "head_dim": c.D, "kv_tile": c.kv_tile},
        "roofline": {"bound": "mfma", "kernel": "k_attn", "achieved": achieved, "peak": PEAK_TFLOPS_INT8,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS_INT8,
                     "traffic": traffic_for("k_attn_joint", ["attn.hip", "device.h", "sq_internal.h"], f_proj),
                     "avg_launch_ms": attn_ms, "flops_per_launch": f_proj},
        "prefix_pass": {"avg_ms": pre_ms, "tflops": f_pre / (pre_ms * 1e-3) / 1e12,
                        "frac": f_pre / (pre_ms * 1e-3) / 1e12 / PEAK_TFLOPS_INT8,
                        "traffic": traffic_for("k_prefix_joint", ["prefix.hip", "device.h", "sq_internal.h"], f_pre)},
        "stages_ms": {n: timer.avg_ms(n) for n in timer.pairs},
    }
    return res, line


def run_quantizer(args, torch, sq, gen, timer):
    import numpy as np
    c = gen.CFG4
    dev = torch.device("cuda:0")
    x, w, table = gen.quant_inputs(c)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    norm = sq.Norm(sq.NORM_HEAD, torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev), None, None, c.eps)
    rope = sq.Rope(sq.ROPE_SPLIT_HALF, torch.from_numpy(table).to(dev))
    smq = gen.sm_scale_q(c.D)
    ws = sq.Workspace(dev)
    runs = [("quant_q_per_block128", None, smq, 0, 128), ("quant_q_thread_q", None, smq, 1, 32),
            ("quant_q_warp_q", None, smq, 3, 128), ("quant_k_per_block64", "mu", 1.0, 0, 64),
            ("quant_k_thread_k", "mu", 1.0, 2, 64)]

    def step():
        mu = timer("kmean", lambda: sq.sq_kmean(xd, norm, rope, workspace=ws))
        for name, m, sm, lay, blk in runs:
            timer(name, lambda: sq.sq_quant_qk(xd, norm, rope, mu if m else None, sm, 1e-7, lay, blk))

    elems = c.B * c.T * c.H * c.D
    table_bytes = table.nbytes
    bytes_ = {"kmean": elems * 2}
    for name, *_ in runs:
        bytes_[name] = elems * 3 + table_bytes
    total = sum(bytes_.values())
    res = time_steps(args, torch, step, timer)
    qn = "quant_q_per_block128"
    q_ms = timer.avg_ms(qn)
    achieved = bytes_[qn] / (q_ms * 1e-3) / 1e9
    line = {
        "metric": "fused q/k quantizer GB/s (algorithmic bytes) and % of HBM peak",
        "value": total / (res["ms"] * 1e-3) / 1e9, "unit": "GB/s", "dtype": "bf16->i8",
        "config": {"workload": "quantizer B=2 T=75600 H=40 d=128: k mean + q PER_BLOCK(128), THREAD_Q, WARP_Q + "
                               "k PER_BLOCK(64), THREAD_K", "B": c.B, "T": c.T, "H": c.H, "head_dim": c.D},
        "roofline": {"bound": "hbm", "kernel": "k_quant_qk", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_for("k_quant_qk_quantizer", ["quant.hip", "device.h", "sq_internal.h"],
                                            float(bytes_[qn])),
                     "avg_launch_ms": q_ms,
                     "bytes_per_launch": bytes_[qn]},
        "stages_ms": {n: timer.avg_ms(n) for n in timer.pairs},
        "stages_gbs": {n: b / (timer.avg_ms(n) * 1e-3) / 1e9 for n, b in bytes_.items()},
    }
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_quantizer(args, c, x, w, table, runs, total)
    return res, line


def run_decode(args, torch, sq, gen, timer):
    import numpy as np
    c = gen.CFG5
    dev = torch.device("cuda:0")
    lens, bt, NB = gen.decode_layout(c)
    g = gen.rng(c.seed, gen.S_EXTRA)
    kc, ks = gen.q8_like((NB, c.bs, c.Hk, c.D), g)
    vc, vs = gen.q8_like((NB, c.bs, c.Hk, c.D), g)
    f16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.float16).to(dev)
    kd, ksd, vd, vsd = torch.from_numpy(kc).to(dev), f16(ks), torch.from_numpy(vc).to(dev), f16(vs)
    qh = gen.decode_query(c)
    q = torch.from_numpy(qh.view(np.int16)).view(torch.bfloat16).to(dev)
    btd, ld = torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev)
    ws = sq.Workspace(dev)
    out = torch.empty((c.N, c.Hq, c.D), dtype=torch.float32, device=dev)

    def step():
        timer("decode", lambda: sq.sq_paged_decode(q, kd, ksd, vd, vsd, btd, ld, c.lmax, c.scale, out=out,
                                                   workspace=ws))

    nbytes = int(lens.sum()) * c.Hk * (2 * c.D + 2 * 2 * (c.D // 32)) + q.numel() * 2 + out.numel() * 4
    res = time_steps(args, torch, step, timer)
    d_ms = timer.avg_ms("decode")
    achieved = nbytes / (d_ms * 1e-3) / 1e9
    line = {
        "metric": "paged q8 decode GB/s (algorithmic bytes) and % of HBM peak",
        "value": nbytes / (res["ms"] * 1e-3) / 1e9, "unit": "GB/s", "dtype": "i8",
        "config": {"workload": "paged GQA decode, 64 sequences L~U(512,16384), 32 q / 8 kv heads, d=128, block 16, "
                               "q8 cache", "num_seqs": c.N, "Hq": c.Hq, "Hk": c.Hk, "head_dim": c.D,
                   "sum_len": int(lens.sum())},
        "roofline": {"bound": "hbm", "kernel": "k_decode_split+k_decode_reduce", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_for("k_decode_split_decode", ["decode.hip", "device.h", "sq_internal.h"],
                                            float(nbytes)),
                     "avg_launch_ms": d_ms, "bytes_per_launch": nbytes},
    }
    if not args.no_cpu_baseline:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_decode(args, c, qh, kc, ks, vc, vs, bt, lens, nbytes)
    return res, line


def run_prefill(args, torch, sq, gen, timer):
    """Paged causal chunked prefill: 16 sequences with cached contexts ~U{0..8192} and 1024-token chunks each,
    Hq 32 / Hk 8, d 128, block 16, q8 cache. Work = 4 Hq d x the visible (query, key) pairs."""
    import numpy as np

    c = gen.PREFILL
    dev = torch.device("cuda:0")
    q, kc, ks, vc, vs, bt, lens, qs = gen.prefill_case(c)
    f16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.float16).to(dev)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).to(dev)
    kd, vd = torch.from_numpy(kc).to(dev), torch.from_numpy(vc).to(dev)
    ksd, vsd = f16(ks), f16(vs)
    btd, ld, qsd = torch.from_numpy(bt).to(dev), torch.from_numpy(lens).to(dev), torch.from_numpy(qs).to(dev)
    out = torch.empty((q.shape[0], c.Hq, c.D), dtype=torch.float32, device=dev)

    def step():
        timer("prefill", lambda: sq.sq_paged_prefill(qd, kd, ksd, vd, vsd, btd, ld, qsd, c.max_len, c.scale, out=out))

    ctx = lens.astype(np.float64) - c.chunk
    pairs = float(np.sum(c.chunk * ctx + c.chunk * (c.chunk + 1) / 2))
    flops = 4.0 * c.Hq * c.D * pairs
    res = time_steps(args, torch, step, timer)
    ms = timer.avg_ms("prefill")
    achieved = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "paged causal prefill TFLOPS (4*Hq*d x visible query-key pairs) and % of f16 MFMA peak",
        "value": flops / (res["ms"] * 1e-3) / 1e12, "unit": "TFLOPS", "dtype": "f16",
        "config": {"workload": "paged chunked prefill, 16 sequences, contexts ~U(0,8192) + 1024-token chunks, "
                               "32 q / 8 kv heads, d=128, block 16, q8 cache", "num_seqs": c.N, "chunk": c.chunk,
                   "Hq": c.Hq, "Hk": c.Hk, "head_dim": c.D, "sum_len": int(lens.sum())},
        "roofline": {"bound": "mfma", "kernel": "k_paged_prefill", "achieved": achieved, "peak": PEAK_TFLOPS_BF16,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS_BF16,
                     "traffic": traffic_for("k_paged_prefill_prefill", ["prefill.hip", "device.h", "sq_internal.h"],
                                            flops),
                     "avg_launch_ms": ms, "flops_per_launch": flops},
    }
    return res, line


def run_cachewrite(args, torch, sq, gen, timer):
    """q8 paged-cache writer: a 131072-token prefill chunk of new K/V rows (Hk 8, d 128, bf16; 537 MB read, more
    than the 256 MiB MALL, so the rows come from HBM) quantized and scattered to a random permutation of the slots of
    an 8192-block cache (block 16)."""
    import numpy as np
    dev = torch.device("cuda:0")
    n, Hk, D, NB, bs = 131072, 8, 128, 8192, 16
    g = gen.rng(2500, 0)
    k = torch.from_numpy(gen.to_bf16_bits(g.standard_normal((n, Hk, D), dtype=np.float32)).view(np.int16)).view(
        torch.bfloat16).to(dev)
    v = torch.from_numpy(gen.to_bf16_bits(g.standard_normal((n, Hk, D), dtype=np.float32)).view(np.int16)).view(
        torch.bfloat16).to(dev)
    slots = torch.from_numpy(g.permutation(NB * bs)[:n].astype(np.int64)).to(dev)
    kc = torch.zeros((NB, bs, Hk, D), dtype=torch.int8, device=dev)
    vc = torch.zeros_like(kc)
    ks = torch.zeros((NB, bs, Hk, D // 32), dtype=torch.float16, device=dev)
    vs = torch.zeros_like(ks)

    def step():
        timer("cachewrite", lambda: sq.sq_q8_cache_write(k, v, slots, kc, ks, vc, vs))

    nbytes = 2 * n * Hk * D * 2 + n * 8 + 2 * n * Hk * D + 2 * n * Hk * (D // 32) * 2
    res = time_steps(args, torch, step, timer)
    ms = timer.avg_ms("cachewrite")
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "q8 paged-cache writer GB/s (algorithmic bytes) and % of HBM peak",
        "value": nbytes / (res["ms"] * 1e-3) / 1e9, "unit": "GB/s", "dtype": "bf16->i8",
        "config": {"workload": "q8 cache write: 131072 new tokens, Hk 8, d 128, bf16 rows, random slots of an "
                               "8192 x 16 block cache", "n_tokens": n, "Hk": Hk, "head_dim": D},
        "roofline": {"bound": "hbm", "kernel": "k_q8_cache_write", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_for("k_q8_cache_write_cachewrite", ["cache.hip", "device.h", "sq_internal.h"],
                                            float(nbytes)),
                     "avg_launch_ms": ms,
                     "bytes_per_launch": nbytes},
    }
    return res, line


def run_merge(args, torch, sq, gen, timer):
    """Log-sum-exp merge of two attention outputs of the video shape (B=1, Sq=32760, H=40, d=128, FP32: 671 MB
    each, beyond the 256 MiB MALL), as a native cached prefix's second pass is merged."""
    dev = torch.device("cuda:0")
    B, S, H, D = 1, 32760, 40, 128
    gt = torch.Generator(device=dev)
    gt.manual_seed(2700)
    out = torch.randn((B, S, H, D), generator=gt, device=dev)
    other = torch.randn((B, S, H, D), generator=gt, device=dev)
    lse = torch.randn((B, H, S), generator=gt, device=dev) * 8
    olse = torch.randn((B, H, S), generator=gt, device=dev) * 8

    def step():
        timer("merge", lambda: sq.sq_lse_merge(out, lse, other, olse))

    nbytes = 3 * B * S * H * D * 4 + 3 * B * H * S * 4
    res = time_steps(args, torch, step, timer)
    ms = timer.avg_ms("merge")
    achieved = nbytes / (ms * 1e-3) / 1e9
    line = {
        "metric": "log-sum-exp merge GB/s (algorithmic bytes) and % of HBM peak",
        "value": nbytes / (res["ms"] * 1e-3) / 1e9, "unit": "GB/s", "dtype": "f32",
        "config": {"workload": "merge of two attention outputs B=1 Sq=32760 H=40 d=128 FP32", "B": B, "Sq": S, "H": H,
                   "head_dim": D},
        "roofline": {"bound": "hbm", "kernel": "k_lse_merge", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic_for("k_lse_merge_merge", ["merge.hip", "device.h", "sq_internal.h"], nbytes),
                     "avg_launch_ms": ms, "bytes_per_launch": nbytes},
    }
    return res, line


def run_copy(args, torch, sq, gen, timer):
    """A plain device-to-device copy of 1 GiB: the known-size kernel that calibrates FETCH_SIZE / WRITE_SIZE."""
    dev = torch.device("cuda:0")
    x = torch.ones(1 << 29, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    res = time_steps(args, torch, lambda: timer("copy", lambda: y.copy_(x)), timer)
    nbytes = 2 * x.numel() * 2
    ms = timer.avg_ms("copy")
    line = {"metric": "device copy GB/s (read + write)", "value": nbytes / (res["ms"] * 1e-3) / 1e9, "unit": "GB/s",
            "dtype": "bf16", "config": {"workload": "copy 1 GiB", "bytes_read": nbytes // 2, "bytes_written": nbytes // 2},
            "roofline": {"bound": "hbm", "kernel": "copy", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                         "avg_launch_ms": ms}}
    return res, line


def time_steps(args, torch, step, timer):
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer.reset()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return {"ms": (t1 - t0) * 1e3 / args.steps}


# ---------------------------------------------------------------------------------------------- CPU baseline
def _timed(fn):
    t0 = time.perf_counter()
    r = fn()
    return r, time.perf_counter() - t0


def cpu_baseline_video(args, c, inp):
    """The oracle on the benchmark's own seeded video inputs: the prologue stages (all-heads mean squares, k mean,
    fused q and k quantization, V to FP8) in full, then the quantized attention core on sampled query rows (every
    head, every key), as many as fit in --cpu-seconds. Its full-size step time is the prologue's plus the core's per
    row times Sq (the core's work is linear in the rows); value is the workload's TFLOPS at that step time."""
    import numpy as np

    import gen
    import oracle as O
    pq = O.Prologue(norm=O.NORM_ALL_HEADS, weight=inp.wq, weight_rows=inp.weight_rows, eps=c.eps,
                    rope=O.ROPE_SPLIT_HALF, table=inp.table)
    pk = O.Prologue(norm=O.NORM_ALL_HEADS, weight=inp.wk, weight_rows=inp.weight_rows, eps=c.eps,
                    rope=O.ROPE_SPLIT_HALF, table=inp.table)
    ql, qb = gen.LAYOUT[c.q_layout], c.q_block
    kl, kb = gen.LAYOUT[c.k_layout], c.k_block
    t_pro = 0.0
    _, t = _timed(lambda: (O.mean_sq_all_heads(inp.q), O.mean_sq_all_heads(inp.k)))
    t_pro += t
    mu, t = _timed(lambda: O.kmean(inp.k, pk))
    t_pro += t
    (qc, qs), t = _timed(lambda: O.quant_qk(inp.q, pq, ql, qb, sm_scale=gen.sm_scale_q(c.D)))
    t_pro += t
    (kc, ks), t = _timed(lambda: O.quant_qk(inp.k, pk, kl, kb, mean=mu))
    t_pro += t
    (v8, vs), t = _timed(lambda: O.quant_v_fp8(inp.v))
    t_pro += t
    q, k = O.QK(qc, qs, ql, qb), O.QK(kc, ks, kl, kb)
    rows = np.random.default_rng(c.seed + 1).permutation(c.Sq).astype(np.int64)
    done, t_core, chunk = 0, 0.0, 2 * O.num_threads()
    while t_core < args.cpu_seconds and done < c.Sq:
        sel = np.sort(rows[done:done + chunk])
        _, t = _timed(lambda: O.attn(q, k, v8, True, vs, kv_tile=c.kv_tile, rows=sel, want_allow=False))
        t_core += t
        done += sel.size
    step_s = t_pro + t_core / done * c.Sq
    return {"value": c.flops() / step_s / 1e12, "unit": "TFLOPS", "cores": O.num_threads(), "kind": "oracle",
            "sample": "the benchmark's seeded inputs: norm statistics, k mean, q/k quantization and V to FP8 in full "
                      "(%.1f s), the attention core on %d random query rows x 40 heads x 32760 keys (%.1f s); full "
                      "step extrapolated linearly in query rows: %.0f s" % (t_pro, done, t_core, step_s),
            "step_s_extrapolated": step_s, "prologue_s": t_pro, "core_s_per_row": t_core / done}


def cpu_baseline_quantizer(args, c, x, w, table, runs, total_bytes):
    """The oracle's k mean and five quantizer runs on the benchmark's own seeded tensor, in full."""
    import gen
    import oracle as O
    pro = O.Prologue(norm=O.NORM_HEAD, weight=w, eps=c.eps, rope=O.ROPE_SPLIT_HALF, table=table)
    mu, t_all = _timed(lambda: O.kmean(x, pro))
    for _, m, sm, lay, blk in runs:
        _, t = _timed(lambda: O.quant_qk(x, pro, lay, blk, mean=mu if m else None, sm_scale=sm, scale_eps=1e-7))
        t_all += t
    return {"value": total_bytes / t_all / 1e9, "unit": "GB/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": "the whole step on the benchmark's seeded %d x %d x %d x %d tensor (k mean + 5 quantizer runs), "
                      "%.1f s" % (c.B, c.T, c.H, c.D, t_all)}


def cpu_baseline_decode(args, c, q, kc, ks, vc, vs, bt, lens, nbytes):
    """The oracle's binary64 paged decode on the benchmark's own seeded cache and queries, all 64 sequences."""
    import oracle as O
    _, t = _timed(lambda: O.paged_decode(q, kc, ks, vc, vs, bt, lens, c.scale))
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": "the whole step (%d sequences, %d cached positions, %d query heads) on the benchmark's seeded "
                      "cache, %.1f s" % (c.N, int(lens.sum()), c.Hq, t)}


# ---------------------------------------------------------------------------------------------- traffic
COPY_BYTES = 1 << 30  # the copy workload: 1 GiB read and 1 GiB written


def _per_dispatch_kib(d, counter, regex):
    """Mean counter value (KiB) over the dispatches of kernels matching regex in a rocprofv3 -d directory."""
    import csv
    import re
    with open(os.path.join(d, "run_counter_collection.csv")) as fh:
        rows = list(csv.DictReader(fh))
    vals = {}
    for r in rows:
        if r["Counter_Name"] != counter or not re.search(regex, r["Kernel_Name"]):
            continue
        vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        sys.exit("no %s values for /%s/ in %s" % (counter, regex, d))
    return sum(vals.values()) / len(vals)


def traffic_main(argv):
    """bench.py traffic KEY KERNEL_REGEX UNITS SOURCES FETCH_DIR WRITE_DIR COPY_FETCH_DIR COPY_WRITE_DIR

    HBM bytes per launch of a benchmarked kernel from two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE: KiB per
    dispatch), each scaled by what the same counter reads for the copy workload (1 GiB read, 1 GiB written), since on
    this GPU the counters see only part of the memory channels. Stored in profiles/traffic.json under KEY with UNITS
    (the algorithmic flops or bytes per launch the bench line uses) and a hash of SOURCES (comma-separated names under
    csrc/): the bench reports the figure only while those sources are unchanged."""
    if len(argv) != 8:
        sys.exit(traffic_main.__doc__)
    key, regex, units, sources, fd, wd, cfd, cwd = argv
    fetch = _per_dispatch_kib(fd, "FETCH_SIZE", regex)
    write = _per_dispatch_kib(wd, "WRITE_SIZE", regex)
    copy_regex = "copyBuffer|elementwise|copy"
    f_fac = COPY_BYTES / (_per_dispatch_kib(cfd, "FETCH_SIZE", copy_regex) * 1024.0)
    w_fac = COPY_BYTES / (_per_dispatch_kib(cwd, "WRITE_SIZE", copy_regex) * 1024.0)
    fetch_b, write_b = fetch * 1024.0 * f_fac, write * 1024.0 * w_fac
    files = sources.split(",")
    entry = {"source_sha": source_sha(files), "sources": files, "units": float(units),
             "bytes_per_launch": fetch_b + write_b, "fetch_bytes": fetch_b, "write_bytes": write_b,
             "fetch_kib_raw": fetch, "write_kib_raw": write, "fetch_scale": f_fac, "write_scale": w_fac}
    try:
        with open(TRAFFIC_FILE) as fh:
            table = json.load(fh)
    except (OSError, ValueError):
        table = {}
    table[key] = entry
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print("%s: fetch %.4g GB + write %.4g GB per launch (raw %.0f / %.0f KiB, scales %.3f / %.3f)"
          % (key, fetch_b / 1e9, write_b / 1e9, fetch, write, f_fac, w_fac))


# ---------------------------------------------------------------------------------------------- main
def main():
    if len(sys.argv) > 1 and sys.argv[1] == "traffic":
        traffic_main(sys.argv[2:])
        return
    args = parse()
    if args.gpus != 1:
        sys.exit("bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus %d)" % args.gpus)
    import torch

    import gen
    import quantized_transformer_attention_amd as sq
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    sq.lib()
    timer = Timer(torch)
    runners = {"video": run_video, "causal": run_causal, "joint": run_joint, "quantizer": run_quantizer, "decode": run_decode,
               "prefill": run_prefill,
               "cachewrite": run_cachewrite, "merge": run_merge, "copy": run_copy}
    if args.workload not in runners:
        sys.exit("workload %s is not benchmarked yet" % args.workload)
    print("bench: workload %s, warmup %d, steps %d" % (args.workload, args.warmup, args.steps), file=sys.stderr,
          flush=True)
    res, line = runners[args.workload](args, torch, sq, gen, timer)
    out = {"metric": line.pop("metric"), "value": line.pop("value"), "unit": line.pop("unit"), "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": line.pop("dtype"), "data": "synthetic (seeded)",
           "config": line.pop("config")}
    out.update(line)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
