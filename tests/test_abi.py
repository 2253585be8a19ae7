"""The C-ABI library (no GPU): it loads, exports every symbol include/sq.h declares, and rejects invalid
arguments on the host before anything is enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import quantized_transformer_attention_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "sq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = sq.lib()
    names = declared_symbols()
    assert len(names) >= 17
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(sq.EXPORTS)
    assert L.sq_abi_version() == sq.ABI_VERSION == 4


def test_status_strings():
    L = sq.lib()
    assert L.sq_status_string(0) == b"SQ_OK"
    assert L.sq_status_string(-5) == b"SQ_ERR_UNSUPPORTED"
    assert L.sq_status_string(-99) == b"SQ_ERR_UNKNOWN"


def test_scale_counts():
    assert sq.sq_scale_count(32760, sq.LAYOUT_THREAD_Q, 32) == 8192
    assert sq.sq_scale_count(32760, sq.LAYOUT_THREAD_K, 64) == 2048
    assert sq.sq_scale_count(75600, sq.LAYOUT_WARP_Q, 128) == 2364
    assert sq.sq_scale_count(75600, sq.LAYOUT_PER_BLOCK, 64) == 1182
    assert sq.sq_scale_count(8704, sq.LAYOUT_PER_BLOCK, 128) == 68
    assert sq.sq_scale_count(100, sq.LAYOUT_THREAD_Q, 64) == -1
    assert sq.sq_scale_count(100, sq.LAYOUT_PER_BLOCK, 48) == -1


def _rows(D=128, T=10, data=0x1000, st=None):
    return sq.sq_rows(data, 1, T, 2, D, 2 * T * D, st if st is not None else 2 * D, D)


def _call_quant(rows, layout=0, block=64, codes=0x2000, scales=0x3000, norm=None, rope=None, sm=1.0, eps=1e-7):
    L = sq.lib()
    return L.sq_quant_qk(ctypes.byref(rows), ctypes.byref(norm) if norm else None,
                         ctypes.byref(rope) if rope else None, None, 0, 0, sm, eps, layout, block, codes, 2 * 10 * 128,
                         256, 128, scales, 2, 1, None, 0, None)


def test_quant_validation_errors():
    L = sq.lib()
    assert _call_quant(_rows(D=96)) == -5
    assert _call_quant(_rows(data=0)) == -1
    assert _call_quant(_rows(data=0x1008)) == -4          # misaligned row base
    assert _call_quant(_rows(st=260)) == -4               # stride not a multiple of 8 elements
    assert _call_quant(_rows(), layout=1, block=64) == -5  # THREAD_Q needs block 32
    assert _call_quant(_rows(), codes=0) == -1
    assert _call_quant(_rows(), codes=0x2004) == -4
    assert _call_quant(_rows(), eps=-1.0) == -2
    bad_norm = sq.sq_norm(sq.NORM_HEAD, 0, None, None, 0, 0, 1e-6)
    assert _call_quant(_rows(), norm=bad_norm) == -1
    rope = sq.sq_rope(sq.ROPE_SPLIT_HALF, 0x4000, 0, 0, 128, 2, 1)   # no pairs
    assert _call_quant(_rows(), rope=rope) == -2
    rope = sq.sq_rope(3, 0x4000, 12, 0, 128, 2, 1)                   # no such mode
    assert _call_quant(_rows(), rope=rope) == -5
    rope = sq.sq_rope(sq.ROPE_SPLIT_HALF, 0x4000, 80, 0, 128, 2, 1)  # pairs > D / 2
    assert _call_quant(_rows(), rope=rope) == -2
    # an all-heads norm without precomputed statistics needs a workspace
    norm = sq.sq_norm(sq.NORM_ALL_HEADS, 0x5000, None, None, 0, 0, 1e-6)
    assert _call_quant(_rows(), norm=norm) == -6
    assert b"workspace" in L.sq_last_error()
    # empty input is a valid no-op
    assert _call_quant(_rows(T=0)) == 0


def _qk(layout=0, block=64, S=10, H=2, D=128, codes=0x1000):
    return sq.sq_qk(codes, 1, S, H, D, S * H * D, H * D, D, 0x2000, H * 4, 4, layout, block)


def test_attn_validation_errors():
    L = sq.lib()
    v = sq.sq_values(0x3000, sq.SQ_BF16, 10 * 2 * 128, 2 * 128, 128, 1, None, 0, 0)

    def call(q, k, vv=v, tile=64, out=0x4000, scale=1.0, ws=None, wsb=0, causal=0, odt=sq.SQ_F32):
        return L.sq_attn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(vv), scale, tile, causal, None, out, odt, 0, 0,
                         0, None, 0, 0, ws, wsb, None)

    assert call(_qk(layout=2), _qk()) == -5                # THREAD_K is a key layout
    assert call(_qk(), _qk(layout=1, block=32)) == -5      # THREAD_Q is a query layout
    assert call(_qk(H=3), _qk(H=2)) == -2                  # heads not a multiple of kv heads
    assert call(_qk(D=64), _qk()) == -2                   # head dims differ
    assert call(_qk(), _qk(), tile=32) == -5
    assert call(_qk(), _qk(), out=0) == -1
    assert call(_qk(), _qk(), odt=sq.SQ_F16) == -5          # out FP32 or bf16
    assert call(_qk(), _qk(), out=0x4002) == -4             # FP32 out on 4-byte boundaries
    assert call(_qk(), _qk(), out=0x4001, odt=sq.SQ_BF16) == -4
    assert call(_qk(), _qk(), scale=0.0) == -2
    assert call(_qk(), _qk(S=0)) == -2                     # no keys
    assert call(_qk(), _qk()) == -6                        # bf16 values are staged in a workspace
    v8 = sq.sq_values(0x3000, sq.SQ_FP8E4M3, 0, 1, 0, 16, None, 0, 0)
    assert call(_qk(), _qk(), vv=v8, tile=128) == -1       # FP8 needs its scales
    v8 = sq.sq_values(0x3000, sq.SQ_FP8E4M3, 0, 1, 0, 16, 0x5000, 0, 0)
    assert call(_qk(), _qk(), vv=v8, tile=96) == -5        # kv_tile 64 or 128
    v8 = sq.sq_values(0x3000, sq.SQ_FP8E4M3, 0, 1, 0, 8, 0x5000, 0, 0)
    assert call(_qk(), _qk(), vv=v8, tile=128) == -3       # channel stride below the key count
    assert call(_qk(S=0), _qk()) == 0                      # no queries: no-op
    assert call(_qk(), _qk(), causal=2) == -2              # causal is 0 or 1
    assert call(_qk(S=11), _qk(S=10), causal=1) == -2      # causal needs Sk >= Sq
    assert call(_qk(S=11), _qk(S=10), causal=0) == -6      # (non-causal: any Sk; then the workspace check)


def _call_cache_write(dtype=0, n=4, Hk=2, D=128, k=0x1000, v=0x2000, kn=256, kh=128, slots=0x3000, kc=0x4000,
                      ks=0x5000, vc=0x6000, vs=0x7000, NB=4, bs=16):
    L = sq.lib()
    return L.sq_q8_cache_write(k, v, dtype, n, Hk, D, kn, kh, kn, kh, slots, kc, ks, vc, vs, NB, bs, None)


def test_cache_write_validation_errors():
    assert _call_cache_write(dtype=sq.SQ_F16) == -5          # only bf16 and FP32 rows
    assert _call_cache_write(D=96) == -5
    assert _call_cache_write(Hk=0) == -2
    assert _call_cache_write(bs=0) == -2
    assert _call_cache_write(n=0, k=None) == 0               # nothing to write: no pointer is read
    assert _call_cache_write(k=None) == -1
    assert _call_cache_write(slots=None) == -1
    assert _call_cache_write(kn=-256) == -3
    assert _call_cache_write(k=0x1008) == -4                 # rows 16-byte aligned
    assert _call_cache_write(kh=132) == -4                   # bf16 strides in multiples of 8 elements
    assert _call_cache_write(dtype=sq.SQ_F32, kh=130) == -4  # FP32 strides in multiples of 4 elements
    assert _call_cache_write(kc=0x4008) == -4                # caches 16-byte aligned
    assert _call_cache_write(ks=0x5001) == -4                # scales 2-byte aligned
    assert b"16-byte" in sq.lib().sq_last_error()


def _call_merge(out=0x1000, lse=0x2000, other=0x3000, olse=0x4000, D=128, ob=128 * 4 * 10, ot=128 * 4, oh=128,
                lh=10, B=1, S=10, H=4):
    L = sq.lib()
    return L.sq_lse_merge(out, ob, ot, oh, lse, 4 * 10, lh, other, ob, ot, oh, olse, 4 * 10, lh, B, S, H, D, None)


def test_lse_merge_validation_errors():
    assert _call_merge(D=96) == -5
    assert _call_merge(S=-1) == -2
    assert _call_merge(S=0, out=None) == 0                  # nothing to merge
    assert _call_merge(lse=None) == -1
    assert _call_merge(lh=-1) == -3
    assert _call_merge(out=0x1004) == -4                    # rows 16-byte aligned
    assert _call_merge(oh=130) == -4


def _call_prefill(T=10, NB=4, bs=16, Hk=2, Hq=8, D=128, q=0x1000, qt=1024, qh=128, kc=0x2000, ks=0x3000, vc=0x4000,
                  vs=0x5000, bt=0x6000, bts=4, lens=0x7000, qs=0x8000, N=2, max_len=64, scale=0.125, out=0x9000,
                  odt=sq.SQ_F32, qdt=sq.SQ_BF16):
    L = sq.lib()
    return L.sq_paged_prefill(q, qdt, qt, qh, T, kc, ks, vc, vs, NB, bs, Hk, bt, bts, lens, qs, N, max_len, Hq, D, scale,
                              None, out, odt, Hq * D, D, None)


def test_paged_prefill_validation_errors():
    assert _call_prefill(D=96) == -5                       # head dim 64 or 128
    assert _call_prefill(qdt=sq.SQ_F32) == -5              # q bf16 or f16
    assert _call_prefill(bs=32) == -5                      # block size 16 only
    assert _call_prefill(Hq=6, Hk=4) == -2                 # heads not a multiple
    assert _call_prefill(Hq=32, Hk=2) == -5                # Hq / Hk = 16
    assert _call_prefill(T=0, q=None) == 0                 # no tokens: nothing read
    assert _call_prefill(N=0, q=None) == 0
    assert _call_prefill(NB=0) == -2                       # the queries' keys live in the cache
    assert _call_prefill(max_len=0) == -2
    assert _call_prefill(qs=None) == -1
    assert _call_prefill(bts=3) == -3                      # table rows shorter than max_len needs
    assert _call_prefill(q=0x1008) == -4
    assert _call_prefill(qh=132) == -4
    assert _call_prefill(ks=0x3001) == -4                  # FP16 scales
    assert _call_prefill(scale=0.0) == -2
    assert _call_prefill(odt=sq.SQ_I8) == -5               # out FP32 or bf16
    assert _call_prefill(out=0x9002) == -4


def _call_decode(N=2, NB=4, bs=16, Hk=2, Hq=8, D=128, q=0x1000, qn=1024, qh=128, kc=0x2000, ks=0x3000, vc=0x4000,
                 vs=0x5000, bt=0x6000, bts=4, lens=0x7000, max_len=64, scale=0.125, out=0x9000, odt=sq.SQ_F32,
                 ws=0x10000, wsb=1 << 20, qdt=sq.SQ_BF16):
    L = sq.lib()
    return L.sq_paged_decode(q, qdt, qn, qh, kc, ks, vc, vs, NB, bs, Hk, bt, bts, lens, N, max_len, Hq, D, scale, None,
                             out, odt, Hq * D, D, ws, wsb, None)


def test_paged_decode_validation_errors():
    assert _call_decode(D=96) == -5                        # head dim 64 or 128
    assert _call_decode(qdt=sq.SQ_I8) == -5                # q bf16 or f16
    assert _call_decode(bs=32) == -5                       # block size 16 only
    assert _call_decode(Hq=6, Hk=4) == -2
    assert _call_decode(Hq=32, Hk=2) == -5                 # Hq / Hk = 16
    assert _call_decode(N=0, q=None) == 0                  # no sequences: nothing read
    assert _call_decode(max_len=0) == -2
    assert _call_decode(lens=None) == -1
    assert _call_decode(bts=3) == -3                       # table rows shorter than max_len needs
    assert _call_decode(q=0x1008) == -4
    assert _call_decode(vs=0x5004) == -4                   # a row of 4 FP16 scales (D 128): 8-byte aligned
    assert _call_decode(D=64, qh=64, vs=0x5002) == -4       # 2 scales (D 64): 4-byte aligned
    assert _call_decode(scale=float("inf")) == -2
    assert _call_decode(odt=sq.SQ_FP8E4M3) == -5           # out FP32 or bf16
    assert _call_decode(out=0x9001, odt=sq.SQ_BF16) == -4
    assert _call_decode(ws=None) == -6                     # the segment partials need a workspace


def test_paged_decode_noalloc_rejects_oversize_before_any_device_call():
    """The no-allocation decode refuses, on the host and before any HIP call, work whose segment partials exceed its
    fixed scratch array (64 sequences x 32 heads x 16,384 positions needs 65 MiB)."""
    L = sq.lib()
    assert sq.DECODE_SCRATCH_BYTES == 64 << 20
    need = L.sq_paged_decode_workspace_bytes(64, 32, 128, 16384)
    assert need > sq.DECODE_SCRATCH_BYTES >= L.sq_paged_decode_workspace_bytes(64, 32, 128, 16128)
    st = L.sq_paged_decode_noalloc(0x1000, sq.SQ_BF16, 32 * 128, 128, 0x2000, 0x3000, 0x4000, 0x5000, 100, 16, 8,
                                   0x6000, 1024, 0x7000, 64, 16384, 32, 128, 0.088, None, 0x8000, sq.SQ_F32, 32 * 128, 128, None)
    assert st == -6
    assert b"scratch" in L.sq_last_error()
    # a bad argument inside the limit is rejected by the decode's own validation (still no device call)
    st = L.sq_paged_decode_noalloc(0x1000, sq.SQ_BF16, 32 * 128, 128, 0x2000, 0x3000, 0x4000, 0x5000, 100, 16, 8,
                                   0x6000, 1024, 0x7000, 4, 1000, 32, 96, 0.088, None, 0x8000, sq.SQ_F32, 32 * 128, 128, None)
    assert st == -5


def test_paged_bindings_reject_wrong_dtypes():
    """The Python binding checks the paged entry points' tensors before any library call (CPU tensors suffice):
    int64 lengths or a float32 q would otherwise be read as int32 / bf16 by the kernels."""
    import torch
    q = torch.zeros((3, 8, 128), dtype=torch.bfloat16)
    kc = torch.zeros((4, 16, 2, 128), dtype=torch.int8)
    ks = torch.zeros((4, 16, 2, 4), dtype=torch.float16)
    bt = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.tensor([5, 9], dtype=torch.int32)
    qs = torch.tensor([0, 1, 3], dtype=torch.int32)
    cases = [
        dict(q=q.float()), dict(kc=kc.to(torch.int16)), dict(ks=ks.float()), dict(bt=bt.long()),
        dict(lens=lens.long()), dict(qs=qs.long()), dict(qs=qs[:2]),
    ]
    for bad in cases:
        a = dict(q=q, kc=kc, ks=ks, bt=bt, lens=lens, qs=qs)
        a.update(bad)
        with pytest.raises(AssertionError):
            sq.sq_paged_prefill(a["q"], a["kc"], a["ks"], a["kc"], a["ks"], a["bt"], a["lens"], a["qs"], 64, 0.125)
        if "qs" not in bad:
            with pytest.raises(AssertionError):
                sq.sq_paged_decode(a["q"], a["kc"], a["ks"], a["kc"], a["ks"], a["bt"], a["lens"], 64, 0.125)


def test_paged_bindings_reject_wrong_out_dtype():
    """A given output tensor sets out_dtype: only FP32 and bf16 reach the library."""
    import torch
    q = torch.zeros((3, 8, 128), dtype=torch.bfloat16)
    kc = torch.zeros((4, 16, 2, 128), dtype=torch.int8)
    ks = torch.zeros((4, 16, 2, 4), dtype=torch.float16)
    bt = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.tensor([5, 9], dtype=torch.int32)
    qs = torch.tensor([0, 1, 3], dtype=torch.int32)
    with pytest.raises(AssertionError):
        sq.sq_paged_prefill(q, kc, ks, kc, ks, bt, lens, qs, 64, 0.125, out=torch.zeros((3, 8, 128), dtype=torch.float16))
    with pytest.raises(AssertionError):
        sq.sq_paged_decode(q[:2], kc, ks, kc, ks, bt, lens, 64, 0.125, out=torch.zeros((2, 8, 128), dtype=torch.float64))


def test_prefix_merge_binding_rejects_wrong_tensors():
    """The q8 prefix merge reads and writes FP32 (out, lse): a bf16 out (the core's bf16 output mode) or a mis-shaped
    lse, mean or scale tensor is rejected by the binding before any library call (CPU tensors suffice)."""
    import torch
    B, S, H, Hk, D, P = 1, 10, 4, 2, 128, 32
    q = sq.QK(torch.zeros((B, S, H, D), dtype=torch.int8), torch.zeros((B, H, 1), dtype=torch.float32), 0, 64)
    pf = sq.Q8Prefix(torch.zeros((1, P, Hk, D), dtype=torch.int8), torch.zeros((1, P, Hk, D // 32), dtype=torch.float16),
                     torch.zeros((1, P, Hk, D), dtype=torch.int8), torch.zeros((1, P, Hk, D // 32), dtype=torch.float16))
    out = torch.zeros((B, S, H, D), dtype=torch.float32)
    lse = torch.zeros((B, H, S), dtype=torch.float32)
    mu = torch.zeros((B, Hk, D), dtype=torch.float32)
    bad = [
        dict(out=out.to(torch.bfloat16)), dict(out=out[:, :5]), dict(lse=lse.to(torch.float16)), dict(lse=lse[:, :2]),
        dict(mu=mu.double()), dict(mu=mu[:, :1]),
        dict(pf=sq.Q8Prefix(pf.k, pf.k_scale.float(), pf.v, pf.v_scale)),
        dict(pf=sq.Q8Prefix(pf.k, pf.k_scale, pf.v.to(torch.uint8), pf.v_scale)),
        dict(pf=sq.Q8Prefix(pf.k[:, :, :1], pf.k_scale, pf.v, pf.v_scale)),
    ]
    for b in bad:
        a = dict(out=out, lse=lse, mu=mu, pf=pf)
        a.update(b)
        with pytest.raises(ValueError):
            sq.sq_attn_prefix_lse_merge(q, a["pf"], a["mu"], a["out"], a["lse"])
    # an empty prefix (zero strides) passes the binding's checks and reaches the library, which needs a GPU stream:
    # only the binding's own checks are exercised here
    import numpy as np
    e8 = torch.from_numpy(np.zeros((1, 0, Hk, D), np.int8))
    e16 = torch.from_numpy(np.zeros((1, 0, Hk, D // 32), np.float16))
    assert e8.stride() == (0, 0, 0, 0)
    try:
        sq.sq_attn_prefix_lse_merge(q, sq.Q8Prefix(e8, e16, e8, e16), None, out, lse)
    except ValueError as e:
        raise AssertionError("an empty prefix is valid: %s" % e)
    except Exception:
        pass   # past the binding: the CPU has no HIP stream


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libsq.so every entry point raises: there is no CPU fallback."""
    monkeypatch.setattr(sq, "LIB_PATH", str(tmp_path / "libsq.so"))
    monkeypatch.setattr(sq, "_lib", None)
    with pytest.raises(ImportError):
        sq.lib()
    with pytest.raises(ImportError):
        sq.sq_scale_count(100, sq.LAYOUT_PER_BLOCK, 64)
