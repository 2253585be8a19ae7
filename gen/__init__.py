"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random tensors and states the workload shapes; it holds
none of the quantized-attention arithmetic. Both the HIP path and the CPU oracle
consume the same host arrays produced here.

Recipe: ``numpy.random.Generator(PCG64(SeedSequence([1000 + cfg, stream])))``, one
stream per tensor. Normal values are drawn in FP32 and rounded to bf16 (round to
nearest even, by torch's dtype conversion). Tensors are returned as numpy arrays:
bf16 as ``uint16`` bit patterns, FP16 as ``uint16``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

# stream ids: fixed order of the tensors of a workload
S_Q, S_K, S_V, S_WQ, S_WK, S_OUTQ, S_OUTK, S_OUTV, S_PK, S_PV, S_LENS, S_PERM, S_KC, S_VC, S_DQ, S_EXTRA = range(16)


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_bf16(shape, g: np.random.Generator, outliers: int = 0, factor: float = 20.0) -> np.ndarray:
    """bf16 N(0,1) of shape (B, T, H, D); ``outliers`` seeded channel indices of the flattened
    H*D channels are scaled by ``factor`` for every token (outlier channels)."""
    x = g.standard_normal(size=shape, dtype=np.float32)
    if outliers:
        B, T, H, D = shape
        idx = g.choice(H * D, size=outliers, replace=False)
        x = x.reshape(B, T, H * D)
        x[:, :, idx] *= np.float32(factor)
        x = x.reshape(shape)
    return to_bf16_bits(x)


def uniform_bf16(shape, g, lo=0.5, hi=1.5) -> np.ndarray:
    return to_bf16_bits(g.uniform(lo, hi, size=shape).astype(np.float32))


def rope_table(T: int, pairs: int, theta: float = 10000.0, start: int = 0) -> np.ndarray:
    """FP32 (1, T, 1, pairs, 2) table of (cos, sin) of pos * theta^(-p / pairs), pos = start + t,
    computed in binary64 and rounded once."""
    pos = np.arange(start, start + T, dtype=np.float64)[:, None]
    inv = theta ** (-np.arange(pairs, dtype=np.float64) / pairs)[None, :]
    ang = pos * inv
    tb = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    return np.ascontiguousarray(tb.reshape(1, T, 1, pairs, 2))


def sm_scale_q(D: int) -> float:
    """log2(e) / sqrt(D) rounded to FP32: q rows carry the softmax scale in log2 units."""
    return float(np.float32(math.log2(math.e) / math.sqrt(D)))


# ----------------------------------------------------------------------------- workloads
LAYOUT = {"per_block": 0, "thread_q": 1, "thread_k": 2, "warp_q": 3}
NORM = {"none": 0, "head": 1, "all_heads": 2}
ROPE = {"none": 0, "split_half": 1, "interleaved": 2}


@dataclass
class AttnConfig:
    name: str
    cfg: int
    B: int
    H: int
    Hk: int
    Sq: int
    Sk: int
    D: int
    norm: str
    q_layout: str
    q_block: int
    k_layout: str
    k_block: int
    pv: str                      # "bf16" | "fp8"
    kv_tile: int
    outliers: int = 0            # outlier channels per tensor
    weight_rows: Optional[list] = None   # [(rows of text tokens, weight row)...] segmented weights
    prefix: int = 0              # q8 prefix tokens
    eps: float = 1e-6

    @property
    def seed(self) -> int:
        return 1000 + self.cfg

    def flops(self) -> float:
        """4 * B * H * Sq * Sk * D: the algorithmic work of the core (Q.K^T and P.V)."""
        return 4.0 * self.B * self.H * self.Sq * self.Sk * self.D


CFG1 = AttnConfig("tiny", 1, B=1, H=2, Hk=2, Sq=256, Sk=256, D=64, norm="head", q_layout="per_block", q_block=64,
                  k_layout="per_block", k_block=64, pv="bf16", kv_tile=64)
CFG2 = AttnConfig("video", 2, B=1, H=40, Hk=40, Sq=32760, Sk=32760, D=128, norm="all_heads", q_layout="thread_q",
                  q_block=32, k_layout="thread_k", k_block=64, pv="fp8", kv_tile=64, outliers=51)
CFG3 = AttnConfig("joint_prefix", 3, B=1, H=24, Hk=24, Sq=8704, Sk=8704, D=128, norm="head", q_layout="per_block",
                  q_block=128, k_layout="per_block", k_block=64, pv="bf16", kv_tile=64, weight_rows=[512, 8192],
                  prefix=4096)


@dataclass
class AttnInputs:
    cfg: AttnConfig
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    weight_rows: Optional[np.ndarray]
    table: np.ndarray
    extra: dict = field(default_factory=dict)


def attn_inputs(c: AttnConfig, Sq: Optional[int] = None, Sk: Optional[int] = None) -> AttnInputs:
    """q, k, v (B, S, H|Hk, D) bf16, norm weights, RoPE table for a workload; Sq/Sk override the token
    counts (smaller cases of the same recipe)."""
    Sq = c.Sq if Sq is None else Sq
    Sk = c.Sk if Sk is None else Sk
    s = c.seed
    q = normal_bf16((c.B, Sq, c.H, c.D), rng(s, S_Q), c.outliers)
    k = normal_bf16((c.B, Sk, c.Hk, c.D), rng(s, S_K), c.outliers)
    v = normal_bf16((c.B, Sk, c.Hk, c.D), rng(s, S_V), c.outliers)
    wd = c.H * c.D if c.norm == "all_heads" else c.D
    wkd = c.Hk * c.D if c.norm == "all_heads" else c.D
    nrows = len(c.weight_rows) if c.weight_rows else 1
    wq = uniform_bf16((nrows, wd), rng(s, S_WQ))
    wk = uniform_bf16((nrows, wkd), rng(s, S_WK))
    wr = None
    if c.weight_rows:
        seg = []
        for row, n in enumerate(c.weight_rows):
            seg += [row] * n
        wr = np.asarray(seg, dtype=np.int32)
        T = max(Sq, Sk)
        if wr.size < T:
            wr = np.concatenate([wr, np.full(T - wr.size, nrows - 1, np.int32)])
        wr = np.ascontiguousarray(wr[:T])
    table = rope_table(max(Sq, Sk), c.D // 2)
    return AttnInputs(c, q, k, v, wq, wk, wr, table)


def prefix_fp32(c: AttnConfig, P: Optional[int] = None):
    """FP32 N(0,1) prefix keys and values (1, P, Hk, D), to be put in the q8 format."""
    P = c.prefix if P is None else P
    k = rng(c.seed, S_PK).standard_normal(size=(1, P, c.Hk, c.D), dtype=np.float32)
    v = rng(c.seed, S_PV).standard_normal(size=(1, P, c.Hk, c.D), dtype=np.float32)
    return k, v


def q8_like(shape, g: np.random.Generator):
    """Random q8-format data for throughput runs: int8 codes in [-127, 127] spread like a normal
    sample at full scale, and FP16 scales near those of N(0,1) groups (no quantizer involved)."""
    codes = np.clip(np.rint(g.standard_normal(size=shape, dtype=np.float32) * 42.0), -127, 127).astype(np.int8)
    scales = to_f16_bits(g.uniform(0.02, 0.03, size=shape[:-1] + (shape[-1] // 32,)).astype(np.float32))
    return codes, scales


# ----------------------------------------------------------------------------- quantizer workload
@dataclass
class QuantConfig:
    name: str = "quantizer"
    cfg: int = 4
    B: int = 2
    T: int = 75600
    H: int = 40
    D: int = 128
    eps: float = 1e-6

    @property
    def seed(self) -> int:
        return 1000 + self.cfg


CFG4 = QuantConfig()


def quant_inputs(c: QuantConfig, T: Optional[int] = None):
    T = c.T if T is None else T
    x = normal_bf16((c.B, T, c.H, c.D), rng(c.seed, S_Q))
    w = uniform_bf16((1, c.D), rng(c.seed, S_WQ))
    return x, w, rope_table(T, c.D // 2)


# ----------------------------------------------------------------------------- paged decode workload
@dataclass
class DecodeConfig:
    name: str = "paged_decode"
    cfg: int = 5
    N: int = 64
    Hq: int = 32
    Hk: int = 8
    D: int = 128
    bs: int = 16
    lmin: int = 512
    lmax: int = 16384
    max_blocks: int = 1024

    @property
    def seed(self) -> int:
        return 1000 + self.cfg

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


CFG5 = DecodeConfig()


def decode_layout(c: DecodeConfig, N: Optional[int] = None, lmin=None, lmax=None):
    """Sequence lengths ~U{lmin..lmax}, and a block table (N, max_blocks) int32 whose used entries are
    a seeded random permutation of the NB = sum ceil(L/bs) physical blocks; unused entries -1."""
    N = c.N if N is None else N
    lmin = c.lmin if lmin is None else lmin
    lmax = c.lmax if lmax is None else lmax
    lens = rng(c.seed, S_LENS).integers(lmin, lmax + 1, size=N).astype(np.int32)
    pages = (lens + c.bs - 1) // c.bs
    NB = int(pages.sum())
    perm = rng(c.seed, S_PERM).permutation(NB).astype(np.int32)
    maxb = max(c.max_blocks, int(pages.max()))
    bt = np.full((N, maxb), -1, np.int32)
    o = 0
    for n in range(N):
        bt[n, :pages[n]] = perm[o:o + pages[n]]
        o += pages[n]
    return lens, bt, NB


def decode_fp32(c: DecodeConfig, NB: int):
    """FP32 N(0,1) K and V for every slot of the paged cache [NB, bs, Hk, D]."""
    k = rng(c.seed, S_KC).standard_normal(size=(NB, c.bs, c.Hk, c.D), dtype=np.float32)
    v = rng(c.seed, S_VC).standard_normal(size=(NB, c.bs, c.Hk, c.D), dtype=np.float32)
    return k, v


def decode_query(c: DecodeConfig, N: Optional[int] = None):
    N = c.N if N is None else N
    return normal_bf16((N, 1, c.Hq, c.D), rng(c.seed, S_DQ)).reshape(N, c.Hq, c.D)


# ----------------------------------------------------------------------------- paged prefill workload
@dataclass
class PrefillConfig:
    """Chunked prefill over the decode workload's cache shape: N sequences, each with a cached context of
    ~U{0..ctx_max} keys and a chunk of `chunk` new queries whose keys and values are in the cache too."""
    name: str = "paged_prefill"
    cfg: int = 6
    N: int = 16
    chunk: int = 1024
    ctx_max: int = 8192
    Hq: int = 32
    Hk: int = 8
    D: int = 128
    bs: int = 16

    @property
    def seed(self) -> int:
        return 1000 + self.cfg

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_len(self) -> int:
        return self.ctx_max + self.chunk


PREFILL = PrefillConfig()


def prefill_case(c: PrefillConfig):
    """q bf16 (N * chunk, Hq, D); q8-format caches (random codes and scales, q8_like) for every slot; block table
    (N, ceil(max_len / bs)) whose used entries are a seeded permutation of the NB physical blocks (-1 elsewhere);
    seq_lens = context + chunk; query_start = 0, chunk, 2 chunk, ..."""
    ctx = rng(c.seed, S_LENS).integers(0, c.ctx_max + 1, size=c.N).astype(np.int32)
    lens = (ctx + c.chunk).astype(np.int32)
    pages = (lens + c.bs - 1) // c.bs
    NB = int(pages.sum())
    perm = rng(c.seed, S_PERM).permutation(NB).astype(np.int32)
    bt = np.full((c.N, (c.max_len + c.bs - 1) // c.bs), -1, np.int32)
    o = 0
    for n in range(c.N):
        bt[n, :pages[n]] = perm[o:o + pages[n]]
        o += pages[n]
    kc, ks = q8_like((NB, c.bs, c.Hk, c.D), rng(c.seed, S_KC))
    vc, vs = q8_like((NB, c.bs, c.Hk, c.D), rng(c.seed, S_VC))
    q = normal_bf16((c.N * c.chunk, 1, c.Hq, c.D), rng(c.seed, S_DQ)).reshape(-1, c.Hq, c.D)
    qs = (np.arange(c.N + 1) * c.chunk).astype(np.int32)
    return q, kc, ks, vc, vs, bt, lens, qs
