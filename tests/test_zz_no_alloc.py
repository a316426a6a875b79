"""The routed linear for callers that cannot allocate (mbq_linear_static, a library-held
device buffer instead of a caller workspace) against mbq_linear on the same inputs.

Same kernels, so the outputs must be identical bit for bit.  Two calls in a row, the
second on a smaller input, so that the shared buffer's leftover partials from the first
call cannot leak into the second.  The calls go through the C ABI (ctypes).
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from token_adaptive_bit_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_adaptive_bit_amd import api
    return api


def to_dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def static_call(mbq, p, x, perm, off, y):
    from token_adaptive_bit_amd import _lib
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = _lib.LIB.mbq_linear_static(ctypes.byref(p.desc), ctypes.c_void_p(p.blob.data_ptr()), x.shape[0],
                                    ctypes.c_void_p(x.data_ptr()), _lib.MBQ_BF16,
                                    ctypes.c_void_p(perm.data_ptr()), ctypes.c_void_p(off.data_ptr()),
                                    ctypes.c_void_p(y.data_ptr()), _lib.MBQ_BF16, None, s)
    assert st == 0, _lib.STATUS.get(st, st)


# N, K, T: K split over workgroups (partials in the buffer), first call larger than the second
CASES = [((2048, 8192, 64), (1024, 8192, 20)),
         ((18944, 3584, 64), (18944, 3584, 40)),
         ((5120, 13824, 64), (5120, 13824, 9))]


@pytest.mark.parametrize("first,second", CASES)
def test_linear_static_matches_linear(mbq, first, second):
    for i, (N, K, T) in enumerate((first, second)):
        print(f"static linear call {i}: N={N} K={K} T={T}", flush=True)
        d = inputs.make_linear(N + T, N, K, T)
        p = mbq.pack(to_dev(d["W"], torch.bfloat16), 128, 3)
        x = to_dev(d["X"], torch.bfloat16)
        _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
        assert mbq.linear_workspace(p, T) > 0          # the split-K partials are in play
        want = mbq.linear(p, x, perm, off)
        y = torch.empty_like(want)
        static_call(mbq, p, x, perm, off, y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"call {i} differs"
        del p
