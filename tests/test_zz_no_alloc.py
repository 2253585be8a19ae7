"""sq_paged_decode_noalloc (the decode without allocation, for callers that cannot allocate) against
sq_paged_decode with a caller workspace: the same kernels on the same inputs give the same bits, on two calls in a
row, the second with a smaller input; both within the decode's tolerance of the binary64 oracle."""
import numpy as np
import pytest
import torch

import oracle as O
import quantized_transformer_attention_amd as sq
from tests._util import check_float, dev, dev_bf16, host
from tests.test_gpu_prefix_decode import _decode_case

pytestmark = pytest.mark.gpu


def _both(q, kc, ks, vc, vs, bt, lens, scale, sinks=None, out_dtype=torch.float32):
    f16 = lambda a: dev(a.view(np.int16)).view(torch.float16)
    args = (dev_bf16(q), dev(kc), f16(ks), dev(vc), f16(vs), dev(bt), dev(lens), int(lens.max()), scale)
    sk = dev(sinks) if sinks is not None else None
    with_ws = sq.sq_paged_decode(*args, sinks=sk, out_dtype=out_dtype)
    out = torch.empty(with_ws.shape, dtype=out_dtype, device=with_ws.device)
    out.fill_(float("nan"))                      # every element must be written
    sq.sq_paged_decode_noalloc(*args, out=out, sinks=sk)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:       # numpy has no bf16: compare the bit patterns
        return host(with_ws.view(torch.int16)), host(out.view(torch.int16))
    return host(with_ws), host(out)


def test_noalloc_decode_equals_workspace_decode_twice_then_smaller():
    scale = 1.0 / np.sqrt(128.0)
    # first call: 6 sequences up to 4096 positions, 8 q / 2 kv heads
    print("no-alloc decode: first call", flush=True)
    case = _decode_case([1, 17, 300, 1100, 4096, 257], 8, 2, 4100)
    a_ws, a_na = _both(*case, scale)
    np.testing.assert_array_equal(a_na.view(np.uint32), a_ws.view(np.uint32))
    q, kc, ks, vc, vs, bt, lens = case
    check_float(a_na, O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale), None, what="no-alloc decode (first)")
    # second call, smaller: 2 sequences, 4 q / 4 kv heads, with sinks; the scratch keeps the first call's partials
    print("no-alloc decode: second, smaller call", flush=True)
    case = _decode_case([5, 40], 4, 4, 4101)
    sinks = np.array([0.5, -1.0, 2.0, -np.inf], np.float32)
    b_ws, b_na = _both(*case, scale, sinks=sinks)
    np.testing.assert_array_equal(b_na.view(np.uint32), b_ws.view(np.uint32))
    q, kc, ks, vc, vs, bt, lens = case
    check_float(b_na, O.paged_decode(q, kc, ks, vc, vs, bt, lens, scale, sinks=sinks), None,
                what="no-alloc decode (second)")
    # bf16 output, the first case again
    print("no-alloc decode: bf16 output", flush=True)
    case = _decode_case([1, 17, 300, 1100, 4096, 257], 8, 2, 4100)
    c_ws, c_na = _both(*case, scale, out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(c_na.view(np.uint16), c_ws.view(np.uint16))


def test_noalloc_decode_rejects_work_beyond_its_scratch():
    """More segment partials than the scratch array holds: an error before anything is enqueued."""
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 16, 8, 128), dtype=torch.int8, device="cuda")
    ks = torch.zeros((4, 16, 8, 4), dtype=torch.float16, device="cuda")
    bt = torch.zeros((64, 1024), dtype=torch.int32, device="cuda")
    lens = torch.full((64,), 16, dtype=torch.int32, device="cuda")
    out = torch.zeros((64, 32, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(sq.SqError) as e:
        sq.sq_paged_decode_noalloc(q, kc, ks, kc, ks, bt, lens, 16384, 0.088, out=out)
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert float(out.abs().sum()) == 0.0          # nothing ran
