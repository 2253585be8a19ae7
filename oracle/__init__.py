"""CPU oracle for quantized attention -- TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper over ``oracle.c``, a plain, slow C implementation of what the
quantized attention path computes. Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the HIP library and
its Python binding never do, and share no code with it.

Every array is a contiguous numpy array: bf16 tensors are ``uint16`` bit patterns,
FP16 scales ``uint16``, FP8 codes ``uint8``. Functions return numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

NORM_NONE, NORM_HEAD, NORM_ALL_HEADS = 0, 1, 2
ROPE_NONE, ROPE_SPLIT_HALF, ROPE_INTERLEAVED = 0, 1, 2
LAYOUT_PER_BLOCK, LAYOUT_THREAD_Q, LAYOUT_THREAD_K, LAYOUT_WARP_Q = 0, 1, 2, 3


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (plain IEEE arithmetic, OpenMP over rows). SQ_ORACLE_LIBRARY names another build
    of it to load instead (e.g. an instrumented one in tests)."""
    if os.environ.get("SQ_ORACLE_LIBRARY"):
        return os.environ["SQ_ORACLE_LIBRARY"]
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
                               "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        _declare(_lib)
    return _lib


_i64, _f32, _f64, _vp, _int = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p, ctypes.c_int


class _Rows(ctypes.Structure):
    _fields_ = [("B", _i64), ("T", _i64), ("H", _i64), ("D", _i64), ("x", _vp), ("norm", _int), ("w", _vp),
                ("wrows", _vp), ("eps", _f32), ("rope", _int), ("table", _vp), ("pairs", _i64), ("rb", _i64),
                ("rs", _i64), ("rp", _i64), ("rc", _i64), ("mean", _vp), ("sm_scale", _f32)]


class _QK(ctypes.Structure):
    _fields_ = [("B", _i64), ("S", _i64), ("H", _i64), ("D", _i64), ("codes", _vp), ("scales", _vp),
                ("layout", _int), ("block", _int)]


class _Prefix(ctypes.Structure):
    _fields_ = [("B", _i64), ("P", _i64), ("H", _i64), ("D", _i64), ("k", _vp), ("ks", _vp), ("v", _vp), ("vs", _vp)]


def _declare(L):
    P = ctypes.POINTER
    L.orc_bf16_round.argtypes, L.orc_bf16_round.restype = [_f32], _f32
    L.orc_f32_to_f16.argtypes, L.orc_f32_to_f16.restype = [_f32], ctypes.c_uint16
    L.orc_f16_value.argtypes, L.orc_f16_value.restype = [ctypes.c_uint16], _f64
    L.orc_f32_to_e4m3.argtypes, L.orc_f32_to_e4m3.restype = [_f32], ctypes.c_uint8
    L.orc_e4m3_value.argtypes, L.orc_e4m3_value.restype = [ctypes.c_uint8], _f64
    L.orc_num_threads.restype = _int
    L.orc_set_num_threads.argtypes = [_int]
    L.orc_mean_sq_all_heads.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp]
    L.orc_prologue_rows.argtypes = [P(_Rows), _vp]
    L.orc_kmean.argtypes = [P(_Rows), _vp]
    L.orc_scale_count.argtypes, L.orc_scale_count.restype = [_i64, _int, _int], _i64
    L.orc_scale_index.argtypes, L.orc_scale_index.restype = [_i64, _int, _int], _i64
    L.orc_quant_qk.argtypes = [P(_Rows), _int, _int, _f32, _vp, _vp]
    L.orc_quant_v_fp8.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _vp]
    L.orc_run_truncation_bound.argtypes, L.orc_run_truncation_bound.restype = [_vp, _i64], _f64
    L.orc_attn.argtypes = [P(_QK), P(_QK), _vp, _int, _vp, _f32, _int, _f64, _int, _vp, _vp, _i64, _vp, _vp, _vp,
                           _vp]
    L.orc_prefix_merge.argtypes = [P(_QK), P(_Prefix), _vp, _f32, _int, _f64, _vp, _vp, _vp, _i64, _vp, _vp, _vp,
                                   _vp, _vp]
    L.orc_q8_quantize.argtypes = [_vp, _i64, _i64, _vp, _vp]
    L.orc_paged_decode.argtypes = [_vp, _int, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _f64, _vp,
                                   _vp]
    L.orc_attn_exact.argtypes = [P(_Rows), P(_Rows), _vp, P(_Prefix), _vp, _i64, _vp]
    L.orc_paged_prefill.argtypes = [_vp, _int, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _i64, _i64,
                                    _f64, _vp, _vp, _i64, _vp]


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ----------------------------------------------------------------------------- formats
def bf16_round(f: float) -> float:
    return float(lib().orc_bf16_round(f))


def f32_to_f16(f: float) -> int:
    return int(lib().orc_f32_to_f16(f))


def f16_value(h: int) -> float:
    return float(lib().orc_f16_value(h))


def f32_to_e4m3(f: float) -> int:
    return int(lib().orc_f32_to_e4m3(f))


def e4m3_value(b: int) -> float:
    return float(lib().orc_e4m3_value(b))


# ----------------------------------------------------------------------------- prologue
@dataclass
class Prologue:
    """What the q/k row prologue applies: norm mode and weight, RoPE mode and table."""
    norm: int = NORM_NONE
    weight: Optional[np.ndarray] = None       # bf16 bits, (rows, D) or (rows, H*D)
    weight_rows: Optional[np.ndarray] = None  # int32 (T,)
    eps: float = 1e-6
    rope: int = ROPE_NONE
    table: Optional[np.ndarray] = None        # FP32 (1|B, T, 1, pairs, 2) or (..., pairs, 2, 2)


def _rows_struct(x, pro: Prologue, mean=None, sm_scale=1.0):
    B, T, H, D = x.shape
    keep = [x]
    r = _Rows(B=B, T=T, H=H, D=D, x=_p(x), norm=pro.norm, eps=pro.eps, rope=pro.rope, sm_scale=sm_scale)
    if pro.norm != NORM_NONE:
        w = _c(pro.weight, np.uint16)
        keep.append(w)
        r.w = _p(w)
        if pro.weight_rows is not None:
            wr = _c(pro.weight_rows, np.int32)
            keep.append(wr)
            r.wrows = _p(wr)
    if pro.rope != ROPE_NONE:
        tb = np.asarray(pro.table, dtype=np.float32)
        assert tb.flags.c_contiguous
        keep.append(tb)
        st = [s // 4 for s in tb.strides]
        r.table = _p(tb)
        r.pairs = tb.shape[3]
        r.rb = 0 if tb.shape[0] == 1 else st[0]
        r.rs, r.rp, r.rc = st[1], st[3], st[4]
    if mean is not None:
        mu = _c(mean, np.float32)
        keep.append(mu)
        r.mean = _p(mu)
    return r, keep


def mean_sq_all_heads(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    B, T, H, D = x.shape
    out = np.empty((B, T), np.float32)
    lib().orc_mean_sq_all_heads(_p(x), B, T, H, D, _p(out))
    return out


def prologue_rows(x: np.ndarray, pro: Prologue, mean=None, sm_scale=1.0) -> np.ndarray:
    x = _c(x, np.uint16)
    r, keep = _rows_struct(x, pro, mean, sm_scale)
    out = np.empty(x.shape, np.float32)
    lib().orc_prologue_rows(ctypes.byref(r), _p(out))
    return out


def kmean(x: np.ndarray, pro: Prologue) -> np.ndarray:
    x = _c(x, np.uint16)
    B, T, H, D = x.shape
    r, keep = _rows_struct(x, pro)
    out = np.empty((B, H, D), np.float32)
    lib().orc_kmean(ctypes.byref(r), _p(out))
    return out


def scale_count(T: int, layout: int, block: int) -> int:
    return int(lib().orc_scale_count(T, layout, block))


def scale_index(t: int, layout: int, block: int) -> int:
    return int(lib().orc_scale_index(t, layout, block))


def quant_qk(x: np.ndarray, pro: Prologue, layout: int, block: int, mean=None, sm_scale=1.0, scale_eps=1e-7):
    """INT8 codes (B, T, H, D) and FP32 scales (B, H, n) of the prologue's rows."""
    x = _c(x, np.uint16)
    B, T, H, D = x.shape
    r, keep = _rows_struct(x, pro, mean, sm_scale)
    codes = np.empty((B, T, H, D), np.int8)
    scales = np.empty((B, H, scale_count(T, layout, block)), np.float32)
    lib().orc_quant_qk(ctypes.byref(r), layout, block, scale_eps, _p(codes), _p(scales))
    return codes, scales


def quant_v_fp8(v: np.ndarray):
    """e4m3fn codes (B, T, H, D) (token-major) and FP32 per-channel scales (B, H, D)."""
    v = _c(v, np.uint16)
    B, T, H, D = v.shape
    codes = np.empty((B, T, H, D), np.uint8)
    vs = np.empty((B, H, D), np.float32)
    lib().orc_quant_v_fp8(_p(v), B, T, H, D, _p(codes), _p(vs))
    return codes, vs


def run_truncation_bound(prod: np.ndarray) -> float:
    """What the FP8 P.V allowance admits for one run of exact products (the reading of an FP8 dot product that
    adds a run of 8 products on a grid of 2^(E - 13), E the exponent of the run's largest magnitude)."""
    prod = _c(prod, np.float64)
    return float(lib().orc_run_truncation_bound(_p(prod), prod.size))


# ----------------------------------------------------------------------------- attention
@dataclass
class QK:
    codes: np.ndarray   # int8 (B, S, H, D)
    scales: np.ndarray  # FP32 (B, H, n)
    layout: int
    block: int


def _qk_struct(t: QK):
    c, s = _c(t.codes, np.int8), _c(t.scales, np.float32)
    B, S, H, D = c.shape
    return _QK(B=B, S=S, H=H, D=D, codes=_p(c), scales=_p(s), layout=t.layout, block=t.block), [c, s]


def attn(q: QK, k: QK, v: np.ndarray, fp8: bool, vs=None, score_scale=1.0, kv_tile=64, rows=None,
         flip_rel=2.0 ** -22, want_allow=True, causal=False, sinks=None, want_run_allow=False):
    """Quantized-mode attention core: out (B, rows, H, D), lse (B, H, rows), allow. causal: query i attends keys
    0 .. i + Sk - Sq; sinks: FP32 (H,) per-head sink logits ([tq] USE_SINKS) or None. want_run_allow: also return
    the part of allow that the FP8 dot-product reading adds (zero for bf16 P.V) as a fourth result."""
    qs, kq = _qk_struct(q)
    ks, kk = _qk_struct(k)
    v = _c(v, np.uint8 if fp8 else np.uint16)
    vs_ = _c(vs, np.float32) if fp8 else None
    B, Sq, H, D = q.codes.shape
    rows = np.arange(Sq, dtype=np.int64) if rows is None else _c(rows, np.int64)
    n = rows.size
    out = np.empty((B, n, H, D), np.float64)
    lse = np.empty((B, H, n), np.float64)
    allow = np.empty((B, n, H, D), np.float64) if want_allow else None
    run = np.empty((B, n, H, D), np.float64) if (want_allow and want_run_allow) else None
    sk_ = _c(sinks, np.float32) if sinks is not None else None
    lib().orc_attn(ctypes.byref(qs), ctypes.byref(ks), _p(v), int(fp8), _p(vs_), score_scale, kv_tile, flip_rel,
                   int(causal), _p(sk_), _p(rows), n, _p(out), _p(lse), _p(allow), _p(run))
    if want_run_allow:
        return out, lse, allow, run
    return out, lse, allow


@dataclass
class Q8Prefix:
    k: np.ndarray    # int8 (1|B, P, Hk, D)
    ks: np.ndarray   # FP16 bits (1|B, P, Hk, D/32)
    v: np.ndarray
    vs: np.ndarray


def _prefix_struct(pf: Q8Prefix):
    k, ks, v, vs = _c(pf.k, np.int8), _c(pf.ks, np.uint16), _c(pf.v, np.int8), _c(pf.vs, np.uint16)
    B, P, H, D = k.shape
    return _Prefix(B=B, P=P, H=H, D=D, k=_p(k), ks=_p(ks), v=_p(v), vs=_p(vs)), [k, ks, v, vs]


def prefix_merge(q: QK, pf: Q8Prefix, mu, out_in, lse_in, score_scale=1.0, kv_tile=64, rows=None,
                 flip_rel=2.0 ** -16, want_parts=False):
    """q8 prefix pass merged by base-2 log-sum-exp with (out_in, lse_in)."""
    qs, kq = _qk_struct(q)
    ps, kp = _prefix_struct(pf)
    mu_ = _c(mu, np.float32) if mu is not None else None
    oi, li = _c(out_in, np.float32), _c(lse_in, np.float32)
    B, Sq, H, D = q.codes.shape
    rows = np.arange(Sq, dtype=np.int64) if rows is None else _c(rows, np.int64)
    n = rows.size
    out = np.empty((B, n, H, D), np.float64)
    lse = np.empty((B, H, n), np.float64)
    allow = np.empty((B, n, H, D), np.float64)
    po = np.empty((B, n, H, D), np.float64) if want_parts else None
    pl = np.empty((B, H, n), np.float64) if want_parts else None
    lib().orc_prefix_merge(ctypes.byref(qs), ctypes.byref(ps), _p(mu_), score_scale, kv_tile, flip_rel, _p(oi),
                           _p(li), _p(rows), n, _p(out), _p(lse), _p(allow), _p(po), _p(pl))
    if want_parts:
        return out, lse, allow, po, pl
    return out, lse, allow


def q8_quantize(x: np.ndarray):
    """q8 codes (..., D) int8 and FP16 scales (..., D/32) of FP32 x."""
    x = _c(x, np.float32)
    D = x.shape[-1]
    rows = x.size // D
    codes = np.empty(x.shape, np.int8)
    scales = np.empty(x.shape[:-1] + (D // 32,), np.uint16)
    lib().orc_q8_quantize(_p(x), rows, D, _p(codes), _p(scales))
    return codes, scales


def lse_merge(out, lse, other, other_lse):
    """[kit] _merge_lse_ in binary64: out (B, S, H, D) and lse (B, H, S) over one key set, other / other_lse over
    a disjoint one; top = max of the base-2 log-sum-exps, weights 2^(lse - top) over their sum. Returns the merged
    out and the merged lse = top + log2(sum of weights); both -inf gives out 0 and lse -inf."""
    a = np.asarray(lse, np.float64)
    b = np.asarray(other_lse, np.float64)
    top = np.maximum(a, b)
    live = top > -np.inf
    ts = np.where(live, top, 0.0)
    wa = np.where(live, np.exp2(a - ts), 0.0)
    wb = np.where(live, np.exp2(b - ts), 0.0)
    tot = wa + wb
    fa = np.where(live, wa / np.where(live, tot, 1.0), 0.0).transpose(0, 2, 1)[..., None]
    fb = np.where(live, wb / np.where(live, tot, 1.0), 0.0).transpose(0, 2, 1)[..., None]
    o = np.asarray(out, np.float64) * fa + np.asarray(other, np.float64) * fb
    l = np.where(live, ts + np.log2(np.where(live, tot, 1.0)), -np.inf)
    return o, l


def q8_cache_write(k, v, slot_mapping, k_cache, k_scale, v_cache, v_scale):
    """[kit] quantize_q8 of each new row, then [impl] _store_kvcache_nhd: token t's rows (Hk, D) go to cache block
    slot // block_size, row slot % block_size of k_cache / v_cache [NB, bs, Hk, D] (codes) and k_scale / v_scale
    [NB, bs, Hk, D/32] (FP16 bits); a negative slot skips the token (as does one past NB * bs). k, v (n, Hk, D) FP32
    (bf16 inputs widened exactly). Updates the four cache arrays in place, tokens in order."""
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    kc, ksc = q8_quantize(k)
    vc, vsc = q8_quantize(v)
    for t, s in enumerate(np.asarray(slot_mapping, np.int64)):
        if s < 0 or s >= NB * bs:
            continue
        k_cache[s // bs, s % bs] = kc[t]
        k_scale[s // bs, s % bs] = ksc[t]
        v_cache[s // bs, s % bs] = vc[t]
        v_scale[s // bs, s % bs] = vsc[t]


def paged_decode(q, k_cache, k_scale, v_cache, v_scale, block_table, seq_lens, scale, sinks=None):
    """Binary64 paged decode over a q8 cache: out (N, Hq, D). q: bf16 bits (uint16) or float16 values.
    sinks: FP32 (Hq,) per-head sink logits or None."""
    q_f16 = int(np.asarray(q).dtype == np.float16)
    q = _c(np.asarray(q).view(np.uint16), np.uint16)
    kc, ks, vc, vsc = _c(k_cache, np.int8), _c(k_scale, np.uint16), _c(v_cache, np.int8), _c(v_scale, np.uint16)
    bt, sl = _c(block_table, np.int32), _c(seq_lens, np.int32)
    N, Hq, D = q.shape
    bs, Hk = kc.shape[1], kc.shape[2]
    out = np.empty((N, Hq, D), np.float64)
    sk_ = _c(sinks, np.float32) if sinks is not None else None
    lib().orc_paged_decode(_p(q), q_f16, _p(kc), _p(ks), _p(vc), _p(vsc), bs, Hk, _p(bt), bt.shape[1], _p(sl), N, Hq, D,
                           float(scale), _p(sk_), _p(out))
    return out


def paged_prefill(q, k_cache, k_scale, v_cache, v_scale, block_table, seq_lens, query_start, scale, sinks=None,
                  rows=None):
    """Binary64 paged causal prefill over a q8 cache ([impl] _prefill_torch_from_cache): q bf16 (T, Hq, D) packed
    by query_start (N + 1,); seq_lens (N,) keys per sequence (context + its queries). out (len(rows) or T, Hq, D).
    q: bf16 bits (uint16) or float16 values."""
    q_f16 = int(np.asarray(q).dtype == np.float16)
    q = _c(np.asarray(q).view(np.uint16), np.uint16)
    kc, ks, vc, vsc = _c(k_cache, np.int8), _c(k_scale, np.uint16), _c(v_cache, np.int8), _c(v_scale, np.uint16)
    bt, sl, qsl = _c(block_table, np.int32), _c(seq_lens, np.int32), _c(query_start, np.int32)
    T, Hq, D = q.shape
    bs, Hk = kc.shape[1], kc.shape[2]
    rows_ = _c(rows, np.int64) if rows is not None else None
    n = rows_.size if rows_ is not None else T
    out = np.empty((n, Hq, D), np.float64)
    sk_ = _c(sinks, np.float32) if sinks is not None else None
    lib().orc_paged_prefill(_p(q), q_f16, _p(kc), _p(ks), _p(vc), _p(vsc), bs, Hk, _p(bt), bt.shape[1], _p(sl), _p(qsl),
                            sl.size, Hq, D, float(scale), _p(sk_), _p(rows_), n, _p(out))
    return out


def attn_exact(q: np.ndarray, qpro: Prologue, k: np.ndarray, kpro: Prologue, v: np.ndarray,
               prefix: Optional[Q8Prefix] = None, rows=None):
    """Unquantized binary64 attention of the bf16 inputs (natural-base softmax, 1/sqrt(D))."""
    q, k, v = _c(q, np.uint16), _c(k, np.uint16), _c(v, np.uint16)
    qr, kq = _rows_struct(q, qpro)
    kr, kk = _rows_struct(k, kpro)
    B, Sq, H, D = q.shape
    rows = np.arange(Sq, dtype=np.int64) if rows is None else _c(rows, np.int64)
    n = rows.size
    out = np.empty((B, n, H, D), np.float64)
    if prefix is not None:
        ps, kp = _prefix_struct(prefix)
        pref = ctypes.byref(ps)
    else:
        pref = None
    lib().orc_attn_exact(ctypes.byref(qr), ctypes.byref(kr), _p(v), pref, _p(rows), n, _p(out))
    return out
