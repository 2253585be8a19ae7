"""Quantized scaled-dot-product attention on AMD Instinct MI355X (gfx950).

Thin Python binding of ``libsq.so`` (see ``include/sq.h``): argument marshalling only.
Every step of the path runs in the library's HIP kernels; PyTorch provides device
memory (output and workspace allocation) and the current HIP stream. There is no
fallback: if the library is missing the import of any entry point raises.

Functions carry the C names: ``sq_norm_stats``, ``sq_kmean``, ``sq_quant_qk``,
``sq_quant_v_fp8``, ``sq_attn``, ``sq_attn_prefix_lse_merge``, ``sq_paged_decode``, ``sq_paged_prefill``.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SQ_LIBRARY: load another build of the same library (e.g. an instrumented host build in tests)
LIB_PATH = os.environ.get("SQ_LIBRARY") or os.path.join(_HERE, "libsq.so")

SQ_OK = 0
SQ_BF16, SQ_F16, SQ_F32, SQ_I8, SQ_FP8E4M3 = range(5)
LAYOUT_PER_BLOCK, LAYOUT_THREAD_Q, LAYOUT_THREAD_K, LAYOUT_WARP_Q = range(4)
NORM_NONE, NORM_HEAD, NORM_ALL_HEADS = range(3)
ROPE_NONE, ROPE_SPLIT_HALF, ROPE_INTERLEAVED = range(3)

_i64, _f32, _vp, _int = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_int


class SqError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__("%s (%d): %s" % (name, status, detail))
        self.status = status


class sq_rows(ctypes.Structure):
    _fields_ = [("data", _vp), ("B", _i64), ("T", _i64), ("H", _i64), ("D", _i64), ("sb", _i64), ("st", _i64),
                ("sh", _i64)]


class sq_norm(ctypes.Structure):
    _fields_ = [("mode", _int), ("weight", _vp), ("weight_rows", _vp), ("mean_sq", _vp), ("msb", _i64), ("mst", _i64),
                ("eps", _f32)]


class sq_rope(ctypes.Structure):
    _fields_ = [("mode", _int), ("table", _vp), ("pairs", _i64), ("rb", _i64), ("rs", _i64), ("rp", _i64),
                ("rc", _i64)]


class sq_qk(ctypes.Structure):
    _fields_ = [("codes", _vp), ("B", _i64), ("S", _i64), ("H", _i64), ("D", _i64), ("sb", _i64), ("st", _i64),
                ("sh", _i64), ("scales", _vp), ("ssb", _i64), ("ssh", _i64), ("layout", _int), ("block", _int)]


class sq_values(ctypes.Structure):
    _fields_ = [("data", _vp), ("dtype", _int), ("sb", _i64), ("st", _i64), ("sh", _i64), ("sd", _i64),
                ("scale", _vp), ("vsb", _i64), ("vsh", _i64)]


class sq_q8prefix(ctypes.Structure):
    _fields_ = [("B", _i64), ("P", _i64), ("Hk", _i64), ("D", _i64), ("k", _vp), ("kb", _i64), ("kt", _i64),
                ("kh", _i64), ("k_scale", _vp), ("ksb", _i64), ("kst", _i64), ("ksh", _i64), ("v", _vp),
                ("vb", _i64), ("vt", _i64), ("vh", _i64), ("v_scale", _vp), ("vsb", _i64), ("vst", _i64),
                ("vsh", _i64)]


_lib = None
ABI_VERSION = 4  # SQ_ABI_VERSION of the sq.h these argument lists follow

EXPORTS = ["sq_scale_count", "sq_norm_stats", "sq_kmean_workspace_bytes", "sq_kmean", "sq_quant_qk_workspace_bytes",
           "sq_quant_qk", "sq_quant_v_fp8_workspace_bytes", "sq_quant_v_fp8", "sq_attn_workspace_bytes", "sq_attn",
           "sq_attn_prefix_lse_merge_workspace_bytes", "sq_attn_prefix_lse_merge", "sq_paged_decode_workspace_bytes",
           "sq_paged_decode", "sq_paged_decode_noalloc", "sq_paged_prefill", "sq_q8_cache_write", "sq_lse_merge", "sq_status_string", "sq_last_error", "sq_abi_version"]


def lib():
    """The loaded libsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libsq.so is not built: run quantized_transformer_attention_amd/_build.py "
                              "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        _sz = ctypes.c_size_t
        L.sq_scale_count.argtypes, L.sq_scale_count.restype = [_i64, _int, _int], _i64
        L.sq_norm_stats.argtypes = [P(sq_rows), _vp, _i64, _i64, _vp]
        L.sq_kmean_workspace_bytes.argtypes, L.sq_kmean_workspace_bytes.restype = [P(sq_rows), P(sq_norm)], _sz
        L.sq_kmean.argtypes = [P(sq_rows), P(sq_norm), P(sq_rope), _vp, _i64, _i64, _vp, _sz, _vp]
        L.sq_quant_qk_workspace_bytes.argtypes, L.sq_quant_qk_workspace_bytes.restype = [P(sq_rows), P(sq_norm)], _sz
        L.sq_quant_qk.argtypes = [P(sq_rows), P(sq_norm), P(sq_rope), _vp, _i64, _i64, _f32, _f32, _int, _int, _vp,
                                  _i64, _i64, _i64, _vp, _i64, _i64, _vp, _sz, _vp]
        L.sq_quant_v_fp8_workspace_bytes.argtypes, L.sq_quant_v_fp8_workspace_bytes.restype = [P(sq_rows)], _sz
        L.sq_quant_v_fp8.argtypes = [P(sq_rows), _vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _sz, _vp]
        L.sq_attn_workspace_bytes.argtypes = [P(sq_qk), P(sq_qk), P(sq_values)]
        L.sq_attn_workspace_bytes.restype = _sz
        L.sq_attn.argtypes = [P(sq_qk), P(sq_qk), P(sq_values), _f32, _int, _int, _vp, _vp, _int, _i64, _i64, _i64,
                              _vp, _i64, _i64, _vp, _sz, _vp]
        L.sq_attn_prefix_lse_merge_workspace_bytes.argtypes = [P(sq_qk), P(sq_q8prefix)]
        L.sq_attn_prefix_lse_merge_workspace_bytes.restype = _sz
        L.sq_attn_prefix_lse_merge.argtypes = [P(sq_qk), P(sq_q8prefix), _vp, _i64, _i64, _f32, _int, _vp, _i64, _i64,
                                               _i64, _vp, _i64, _i64, _vp, _sz, _vp]
        L.sq_paged_decode_workspace_bytes.argtypes = [_int, _int, _int, _int]
        L.sq_paged_decode_workspace_bytes.restype = _sz
        L.sq_paged_decode.argtypes = [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _int, _int, _vp, _i64, _vp, _int,
                                      _int, _int, _int, _f32, _vp, _vp, _int, _i64, _i64, _vp, _sz, _vp]
        L.sq_paged_decode_noalloc.argtypes = [_vp, _int, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _int, _int, _vp, _i64, _vp,
                                              _int, _int, _int, _int, _f32, _vp, _vp, _int, _i64, _i64, _vp]
        L.sq_paged_prefill.argtypes = [_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _i64, _int, _int, _vp, _i64, _vp,
                                       _vp, _int, _int, _int, _int, _f32, _vp, _vp, _int, _i64, _i64, _vp]
        L.sq_lse_merge.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                   _i64, _i64, _i64, _vp]
        L.sq_q8_cache_write.argtypes = [_vp, _vp, _int, _i64, _int, _int, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp,
                                        _vp, _i64, _int, _vp]
        L.sq_status_string.argtypes, L.sq_status_string.restype = [_int], ctypes.c_char_p
        L.sq_last_error.argtypes, L.sq_last_error.restype = [], ctypes.c_char_p
        L.sq_abi_version.restype = _int
        if L.sq_abi_version() != ABI_VERSION:
            raise ImportError("libsq.so has ABI version %d, this binding needs %d: rebuild it"
                              % (L.sq_abi_version(), ABI_VERSION))
        _lib = L
    return _lib


def _check(status: int):
    if status != SQ_OK:
        L = lib()
        raise SqError(status, L.sq_status_string(status).decode(), L.sq_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ws(nbytes: int, device):
    if nbytes == 0:
        return None, 0
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


class Workspace:
    """A reusable device workspace (grown on demand) for repeated calls, e.g. timing loops."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf, self.buf.numel()


def _rows(x: torch.Tensor) -> sq_rows:
    assert x.dtype == torch.bfloat16 and x.dim() == 4 and x.stride(3) == 1, "rows: bf16 (B, T, H, D), channels contiguous"
    B, T, H, D = x.shape
    return sq_rows(x.data_ptr(), B, T, H, D, x.stride(0), x.stride(1), x.stride(2))


@dataclass
class Norm:
    """Weighted RMSNorm: mode NORM_HEAD (weight (rows, D)) or NORM_ALL_HEADS (weight (rows, H*D))."""
    mode: int
    weight: torch.Tensor
    weight_rows: Optional[torch.Tensor] = None
    mean_sq: Optional[torch.Tensor] = None
    eps: float = 1e-6

    def c(self) -> sq_norm:
        n = sq_norm(self.mode, self.weight.data_ptr(), None, None, 0, 0, self.eps)
        if self.weight_rows is not None:
            assert self.weight_rows.dtype == torch.int32
            n.weight_rows = self.weight_rows.data_ptr()
        if self.mean_sq is not None:
            n.mean_sq = self.mean_sq.data_ptr()
            n.msb, n.mst = self.mean_sq.stride(0), self.mean_sq.stride(1)
        return n


@dataclass
class Rope:
    """RoPE table FP32 (1|B, T, 1, pairs, 2) or (1|B, T, 1, pairs, 2, 2); mode ROPE_SPLIT_HALF or ROPE_INTERLEAVED."""
    mode: int
    table: torch.Tensor

    def c(self) -> sq_rope:
        t = self.table
        assert t.dtype == torch.float32
        return sq_rope(self.mode, t.data_ptr(), t.shape[3], 0 if t.shape[0] == 1 else t.stride(0), t.stride(1),
                       t.stride(3), t.stride(4))


def _norm_c(norm):
    return ctypes.byref(norm.c()) if norm is not None else None


def sq_scale_count(T: int, layout: int, block: int) -> int:
    return int(lib().sq_scale_count(T, layout, block))


def sq_norm_stats(x: torch.Tensor) -> torch.Tensor:
    """Per-token mean of squares over all heads, FP32 (B, T)."""
    out = torch.empty(x.shape[:2], dtype=torch.float32, device=x.device)
    r = _rows(x)
    _check(lib().sq_norm_stats(ctypes.byref(r), _ptr(out), out.stride(0), out.stride(1), _stream(x.device)))
    return out


def sq_kmean(k: torch.Tensor, norm: Optional[Norm] = None, rope: Optional[Rope] = None,
             workspace: Optional[Workspace] = None) -> torch.Tensor:
    """Mean over tokens of the normalized, rotated k rows, FP32 (B, H, D)."""
    B, T, H, D = k.shape
    out = torch.empty((B, H, D), dtype=torch.float32, device=k.device)
    r = _rows(k)
    nc = norm.c() if norm is not None else None
    rc = rope.c() if rope is not None else None
    L = lib()
    need = L.sq_kmean_workspace_bytes(ctypes.byref(r), ctypes.byref(nc) if nc else None)
    ws, nb = workspace.get(need) if workspace is not None else _ws(need, k.device)
    _check(L.sq_kmean(ctypes.byref(r), ctypes.byref(nc) if nc else None, ctypes.byref(rc) if rc else None, _ptr(out),
                      out.stride(0), out.stride(1), _ptr(ws), nb, _stream(k.device)))
    return out


@dataclass
class QK:
    """INT8 codes (B, S, H, D) and their FP32 scales (B, H, n) in a layout."""
    codes: torch.Tensor
    scales: torch.Tensor
    layout: int
    block: int

    def c(self) -> sq_qk:
        c, s = self.codes, self.scales
        B, S, H, D = c.shape
        return sq_qk(c.data_ptr(), B, S, H, D, c.stride(0), c.stride(1), c.stride(2), s.data_ptr(), s.stride(0),
                     s.stride(1), self.layout, self.block)


def sq_quant_qk(x: torch.Tensor, norm: Optional[Norm] = None, rope: Optional[Rope] = None,
                mean: Optional[torch.Tensor] = None, sm_scale: float = 1.0, scale_eps: float = 1e-7,
                layout: int = LAYOUT_PER_BLOCK, block: int = 64, workspace: Optional[Workspace] = None) -> QK:
    """Fused norm + RoPE + mean + INT8 quantization of bf16 rows (B, T, H, D)."""
    B, T, H, D = x.shape
    n = sq_scale_count(T, layout, block)
    if n < 0:
        raise SqError(-5, "SQ_ERR_UNSUPPORTED", "layout %d with block %d" % (layout, block))
    codes = torch.empty((B, T, H, D), dtype=torch.int8, device=x.device)
    scales = torch.empty((B, H, n), dtype=torch.float32, device=x.device)
    r = _rows(x)
    nc = norm.c() if norm is not None else None
    rc = rope.c() if rope is not None else None
    L = lib()
    need = L.sq_quant_qk_workspace_bytes(ctypes.byref(r), ctypes.byref(nc) if nc else None)
    ws, nb = workspace.get(need) if workspace is not None else _ws(need, x.device)
    _check(L.sq_quant_qk(ctypes.byref(r), ctypes.byref(nc) if nc else None, ctypes.byref(rc) if rc else None,
                         _ptr(mean), mean.stride(0) if mean is not None else 0,
                         mean.stride(1) if mean is not None else 0, sm_scale, scale_eps, layout, block, _ptr(codes),
                         codes.stride(0), codes.stride(1), codes.stride(2), _ptr(scales), scales.stride(0),
                         scales.stride(1), _ptr(ws), nb, _stream(x.device)))
    return QK(codes, scales, layout, block)


def sq_quant_v_fp8(v: torch.Tensor, token_stride: Optional[int] = None, workspace: Optional[Workspace] = None):
    """bf16 V (B, T, H, D) -> FP8 e4m3fn codes channel-major (B, H, D, Tpad) as uint8, FP32 scales (B, H, D)."""
    B, T, H, D = v.shape
    tp = token_stride if token_stride is not None else (T + 127) // 128 * 128
    codes = torch.empty((B, H, D, tp), dtype=torch.uint8, device=v.device)
    vs = torch.empty((B, H, D), dtype=torch.float32, device=v.device)
    r = _rows(v)
    L = lib()
    need = L.sq_quant_v_fp8_workspace_bytes(ctypes.byref(r))
    ws, nb = workspace.get(need) if workspace is not None else _ws(need, v.device)
    _check(L.sq_quant_v_fp8(ctypes.byref(r), _ptr(codes), codes.stride(0), codes.stride(1), codes.stride(2), _ptr(vs),
                            vs.stride(0), vs.stride(1), _ptr(ws), nb, _stream(v.device)))
    return codes, vs


def _values(v: torch.Tensor, v_scale: Optional[torch.Tensor]) -> sq_values:
    if v.dtype == torch.bfloat16:
        B, S, H, D = v.shape
        return sq_values(v.data_ptr(), SQ_BF16, v.stride(0), v.stride(1), v.stride(2), v.stride(3), None, 0, 0)
    assert v.dtype == torch.uint8 and v_scale is not None, "FP8 values: uint8 channel-major (B, H, D, Tpad) + scales"
    # channel-major (B, H, D, Tpad): element (b, s, h, c) at b*sb + h*sh + c*sd + s
    return sq_values(v.data_ptr(), SQ_FP8E4M3, v.stride(0), 1, v.stride(1), v.stride(2), v_scale.data_ptr(),
                     v_scale.stride(0), v_scale.stride(1))


def _out_dtype(out: torch.Tensor) -> int:
    """The sq_dtype of an attention output tensor: FP32 or bf16."""
    dt = {torch.float32: SQ_F32, torch.bfloat16: SQ_BF16}.get(out.dtype)
    assert dt is not None, "out: torch.float32 or torch.bfloat16, got %s" % out.dtype
    return dt


def sq_attn(q: QK, k: QK, v: torch.Tensor, v_scale: Optional[torch.Tensor] = None, score_scale: float = 1.0,
            kv_tile: int = 64, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            want_lse: bool = True, workspace: Optional[Workspace] = None, causal: bool = False,
            sinks: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32):
    """Quantized attention core. v: bf16 (B, Sk, Hk, D) token-major, or FP8 codes from sq_quant_v_fp8 with v_scale.
    causal: query i sees keys 0 .. i + Sk - Sq; sinks: FP32 (H,) per-head sink logits (natural log) or None.
    out_dtype: torch.float32 or torch.bfloat16 (rounded to nearest even; a given out sets it).
    Returns (out (B, Sq, H, D), lse FP32 (B, H, Sq) base 2 or None)."""
    B, Sq, H, D = q.codes.shape
    dev = q.codes.device
    if out is None:
        out = torch.empty((B, Sq, H, D), dtype=out_dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=dev)
    qc, kc, vc = q.c(), k.c(), _values(v, v_scale)
    L = lib()
    need = L.sq_attn_workspace_bytes(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc))
    ws, nb = workspace.get(need) if workspace is not None else _ws(need, dev)
    if sinks is not None:
        assert sinks.dtype == torch.float32 and sinks.is_contiguous() and sinks.numel() == H, "sinks: FP32 (H,)"
    _check(L.sq_attn(ctypes.byref(qc), ctypes.byref(kc), ctypes.byref(vc), score_scale, kv_tile, int(causal),
                     _ptr(sinks), _ptr(out), _out_dtype(out),
                     out.stride(0), out.stride(1), out.stride(2), _ptr(lse), lse.stride(0) if lse is not None else 0,
                     lse.stride(1) if lse is not None else 0, _ptr(ws), nb, _stream(dev)))
    return out, lse


@dataclass
class Q8Prefix:
    """A cached q8 prefix: int8 k, v (1|B, P, Hk, D) with FP16 scales (1|B, P, Hk, D/32) (torch.float16)."""
    k: torch.Tensor
    k_scale: torch.Tensor
    v: torch.Tensor
    v_scale: torch.Tensor

    def c(self) -> sq_q8prefix:
        k, ks, v, vs = self.k, self.k_scale, self.v, self.v_scale
        B, P, Hk, D = k.shape
        return sq_q8prefix(B, P, Hk, D, k.data_ptr(), k.stride(0), k.stride(1), k.stride(2), ks.data_ptr(),
                           ks.stride(0), ks.stride(1), ks.stride(2), v.data_ptr(), v.stride(0), v.stride(1),
                           v.stride(2), vs.data_ptr(), vs.stride(0), vs.stride(1), vs.stride(2))


def sq_attn_prefix_lse_merge(q: QK, prefix: Q8Prefix, k_mean: Optional[torch.Tensor], out: torch.Tensor,
                             lse: torch.Tensor, score_scale: float = 1.0, kv_tile: int = 64,
                             workspace: Optional[Workspace] = None):
    """The q8 prefix pass merged in place into (out, lse) of the projected-key pass: out FP32 (B, Sq, H, D) and lse
    FP32 (B, H, Sq), both read and written (the merge keeps FP32); k_mean FP32 (B, Hk, D) or None."""
    B, Sq, H, D = q.codes.shape
    def _inner(t, d):   # contiguous along dim d (an empty tensor has no strides to speak of)
        return t.numel() == 0 or t.stride(d) == 1

    if out.dtype != torch.float32 or out.dim() != 4 or tuple(out.shape) != (B, Sq, H, D) or not _inner(out, 3):
        raise ValueError("out: FP32 (B, Sq, H, D) of the queries, channels contiguous (the merge reads and writes FP32)")
    if lse.dtype != torch.float32 or lse.dim() != 3 or tuple(lse.shape) != (B, H, Sq) or not _inner(lse, 2):
        raise ValueError("lse: FP32 (B, H, Sq), queries contiguous")
    Bp, P, Hk, Dp = prefix.k.shape
    if Dp != D or H % Hk != 0 or Bp not in (1, B):
        raise ValueError("prefix: (1|B, P, Hk, D) with the queries' D and H a multiple of Hk")
    for t, name in ((prefix.k, "k"), (prefix.v, "v")):
        if t.dtype != torch.int8 or tuple(t.shape) != (Bp, P, Hk, D) or not _inner(t, 3):
            raise ValueError("prefix %s: int8 (1|B, P, Hk, D), channels contiguous" % name)
    for t, name in ((prefix.k_scale, "k_scale"), (prefix.v_scale, "v_scale")):
        if t.dtype != torch.float16 or tuple(t.shape) != (Bp, P, Hk, D // 32) or not _inner(t, 3):
            raise ValueError("prefix %s: FP16 (1|B, P, Hk, D/32), groups contiguous" % name)
    if k_mean is not None and (k_mean.dtype != torch.float32 or tuple(k_mean.shape) != (B, Hk, D) or
                               not _inner(k_mean, 2)):
        raise ValueError("k_mean: FP32 (B, Hk, D), channels contiguous")
    dev = q.codes.device
    qc, pc = q.c(), prefix.c()
    L = lib()
    need = L.sq_attn_prefix_lse_merge_workspace_bytes(ctypes.byref(qc), ctypes.byref(pc))
    ws, nb = workspace.get(need) if workspace is not None else _ws(need, dev)
    _check(L.sq_attn_prefix_lse_merge(ctypes.byref(qc), ctypes.byref(pc), _ptr(k_mean),
                                      k_mean.stride(0) if k_mean is not None else 0,
                                      k_mean.stride(1) if k_mean is not None else 0, score_scale, kv_tile, _ptr(out),
                                      out.stride(0), out.stride(1), out.stride(2), _ptr(lse), lse.stride(0),
                                      lse.stride(1), _ptr(ws), nb, _stream(dev)))
    return out, lse



def _q_dtype(q: torch.Tensor) -> int:
    return SQ_F16 if q.dtype == torch.float16 else SQ_BF16


def _check_paged(q, k_cache, k_scale, v_cache, v_scale, block_table, seq_lens, query_start=None):
    """Host-side dtype and layout checks of the paged entry points' tensors (the C ABI takes raw pointers)."""
    assert q.dtype in (torch.bfloat16, torch.float16) and q.dim() == 3 and q.stride(2) == 1, \
        "q: bf16 or f16 (tokens, Hq, D), channels contiguous"
    for c in (k_cache, v_cache):
        assert c.dtype == torch.int8 and c.dim() == 4 and c.is_contiguous(), "caches: contiguous int8 [NB, bs, Hk, D]"
    for sc in (k_scale, v_scale):
        assert sc.dtype == torch.float16 and sc.dim() == 4 and sc.is_contiguous(), \
            "cache scales: contiguous FP16 [NB, bs, Hk, D/32]"
    assert v_cache.shape == k_cache.shape and k_scale.shape == v_scale.shape == k_cache.shape[:3] + (k_cache.shape[3] // 32,)
    assert block_table.dtype == torch.int32 and block_table.dim() == 2 and block_table.stride(1) == 1, \
        "block_table: int32 (num_seqs, max_blocks), rows contiguous"
    assert seq_lens.dtype == torch.int32 and seq_lens.is_contiguous(), "seq_lens: contiguous int32 (num_seqs,)"
    if query_start is not None:
        assert query_start.dtype == torch.int32 and query_start.is_contiguous() and \
            query_start.numel() == seq_lens.numel() + 1, "query_start: contiguous int32 (num_seqs + 1,)"


def sq_paged_decode(q: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor, v_cache: torch.Tensor,
                    v_scale: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                    softmax_scale: float, out: Optional[torch.Tensor] = None,
                    workspace: Optional[Workspace] = None, sinks: Optional[torch.Tensor] = None,
                    out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Paged GQA decode over a q8 cache. q bf16 or f16 (N, Hq, D), D 64 or 128; caches int8 [NB, bs, Hk, D] with FP16 scales
    [NB, bs, Hk, D/32]; block_table int32 (N, max_blocks); seq_lens int32 (N,); sinks FP32 (Hq,) per-head sink
    logits (natural log) or None. Returns (N, Hq, D) in out_dtype (FP32 or bf16)."""
    _check_paged(q, k_cache, k_scale, v_cache, v_scale, block_table, seq_lens)
    N, Hq, D = q.shape
    NB, bs, Hk, _ = k_cache.shape
    dev = q.device
    if sinks is not None:
        assert sinks.dtype == torch.float32 and sinks.is_contiguous() and sinks.numel() == Hq, "sinks: FP32 (Hq,)"

    if out is None:
        out = torch.empty((N, Hq, D), dtype=out_dtype, device=dev)
    L = lib()
    need = L.sq_paged_decode_workspace_bytes(N, Hq, D, max_seq_len)
    ws, nb = workspace.get(need) if workspace is not None else _ws(need, dev)
    _check(L.sq_paged_decode(_ptr(q), _q_dtype(q), q.stride(0), q.stride(1), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                             _ptr(v_scale), NB, bs, Hk, _ptr(block_table), block_table.stride(0), _ptr(seq_lens), N,
                             max_seq_len, Hq, D, softmax_scale, _ptr(sinks), _ptr(out), _out_dtype(out),
                             out.stride(0), out.stride(1),
                             _ptr(ws), nb,
                             _stream(dev)))
    return out


DECODE_SCRATCH_BYTES = 64 << 20   # SQ_DECODE_SCRATCH_BYTES


def sq_paged_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor, v_cache: torch.Tensor,
                            v_scale: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                            softmax_scale: float, out: torch.Tensor, sinks: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sq_paged_decode without allocation (for callers that cannot allocate: graph capture, serving loops): the
    segment partials live in the library's own scratch array on the GPU; out (N, Hq, D), FP32 or bf16, is given by
    the caller and nothing is allocated here either. Calls that overlap on one GPU share that array and race."""
    _check_paged(q, k_cache, k_scale, v_cache, v_scale, block_table, seq_lens)
    N, Hq, D = q.shape
    NB, bs, Hk, _ = k_cache.shape
    if sinks is not None:
        assert sinks.dtype == torch.float32 and sinks.is_contiguous() and sinks.numel() == Hq, "sinks: FP32 (Hq,)"
    assert out.dim() == 3 and tuple(out.shape) == (N, Hq, D) and out.stride(2) == 1, "out: (N, Hq, D), channels contiguous"
    L = lib()
    _check(L.sq_paged_decode_noalloc(_ptr(q), _q_dtype(q), q.stride(0), q.stride(1), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                                     _ptr(v_scale), NB, bs, Hk, _ptr(block_table), block_table.stride(0),
                                     _ptr(seq_lens), N, max_seq_len, Hq, D, softmax_scale, _ptr(sinks), _ptr(out),
                                     _out_dtype(out), out.stride(0), out.stride(1), _stream(q.device)))
    return out


def sq_paged_prefill(q: torch.Tensor, k_cache: torch.Tensor, k_scale: torch.Tensor, v_cache: torch.Tensor,
                     v_scale: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor,
                     query_start: torch.Tensor, max_seq_len: int, softmax_scale: float,
                     out: Optional[torch.Tensor] = None, sinks: Optional[torch.Tensor] = None,
                     out_dtype: torch.dtype = torch.float32) -> torch.Tensor:
    """Paged causal (chunked) prefill over a q8 cache. q bf16 or f16 (num_tokens, Hq, D), D 64 or 128, packed by query_start int32
    (N + 1,); seq_lens int32 (N,) keys per sequence (context + its queries, already in the cache); caches and
    block_table as sq_paged_decode; sinks FP32 (Hq,) or None. Returns (num_tokens, Hq, D) in out_dtype (FP32 or
    bf16)."""
    _check_paged(q, k_cache, k_scale, v_cache, v_scale, block_table, seq_lens, query_start)
    T, Hq, D = q.shape
    NB, bs, Hk, _ = k_cache.shape
    dev = q.device
    if out is None:
        out = torch.empty((T, Hq, D), dtype=out_dtype, device=dev)
    if sinks is not None:
        assert sinks.dtype == torch.float32 and sinks.is_contiguous() and sinks.numel() == Hq, "sinks: FP32 (Hq,)"
    L = lib()
    _check(L.sq_paged_prefill(_ptr(q), _q_dtype(q), q.stride(0), q.stride(1), T, _ptr(k_cache), _ptr(k_scale), _ptr(v_cache),
                              _ptr(v_scale), NB, bs, Hk, _ptr(block_table), block_table.stride(0), _ptr(seq_lens),
                              _ptr(query_start), seq_lens.numel(), max_seq_len, Hq, D, softmax_scale, _ptr(sinks),
                              _ptr(out), _out_dtype(out), out.stride(0), out.stride(1), _stream(dev)))
    return out


def sq_q8_cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                      k_scale: torch.Tensor, v_cache: torch.Tensor, v_scale: torch.Tensor) -> None:
    """Quantize new rows k, v (n_tokens, Hk, D), bf16 or FP32, to q8 and write them into the paged caches
    (int8 [NB, bs, Hk, D], FP16 scales [NB, bs, Hk, D/32]) at the slots slot_mapping (int64 (n_tokens,));
    negative slots are skipped."""
    n, Hk, D = k.shape
    NB, bs = k_cache.shape[0], k_cache.shape[1]
    if k.dtype != v.dtype or k.shape != v.shape:
        raise ValueError("k and v must have one shape and dtype")
    dt = {torch.bfloat16: SQ_BF16, torch.float32: SQ_F32}.get(k.dtype)
    if dt is None:
        raise ValueError("k and v must be bf16 or float32")
    if slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64")
    if k.stride(2) != 1 or v.stride(2) != 1:
        raise ValueError("k and v need contiguous channels")
    L = lib()
    _check(L.sq_q8_cache_write(_ptr(k), _ptr(v), dt, n, Hk, D, k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                               _ptr(slot_mapping), _ptr(k_cache), _ptr(k_scale), _ptr(v_cache), _ptr(v_scale), NB, bs,
                               _stream(k.device)))


def sq_lse_merge(out: torch.Tensor, lse: torch.Tensor, other: torch.Tensor, other_lse: torch.Tensor) -> None:
    """In place: (out, lse) becomes the attention of the same queries over both key sets, from (out, lse) over one
    and (other, other_lse) over the other. out, other FP32 (B, S, H, D); lse, other_lse FP32 (B, H, S), base 2."""
    B, S, H, D = out.shape
    for t in (out, lse, other, other_lse):
        if t.dtype != torch.float32:
            raise ValueError("sq_lse_merge takes FP32 tensors")
    if out.stride(3) != 1 or other.stride(3) != 1 or lse.stride(2) != 1 or other_lse.stride(2) != 1:
        raise ValueError("channels and tokens of the log-sum-exps must be contiguous")
    L = lib()
    _check(L.sq_lse_merge(_ptr(out), out.stride(0), out.stride(1), out.stride(2), _ptr(lse), lse.stride(0),
                          lse.stride(1), _ptr(other), other.stride(0), other.stride(1), other.stride(2), _ptr(other_lse),
                          other_lse.stride(0), other_lse.stride(1), B, S, H, D, _stream(out.device)))
