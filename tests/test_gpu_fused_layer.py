"""GPU parity of the fused decoder-layer linears: weights that read the same activations
(q/k/v, gate/up) packed into one blob by row ranges (mbq_pack_rows) and run as one routed
linear.  Quantization groups lie within a row, so the fused blob must equal the oracle's
blob of the row-concatenated weight byte for byte, and each weight's output columns must
meet the usual per-token bar against the oracle.
"""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mbq_oracle as O
from token_adaptive_bit_amd import inputs
from parity import TOL, budget_from_perm, oracle_blob, oracle_linear_rows, say, token_errors

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


def parts(seed, ns, K, dtype="bf16"):
    rng = np.random.default_rng(seed)
    out = []
    for n in ns:
        W = rng.standard_normal((n, K), dtype=np.float32) * np.float32(0.02)
        out.append(inputs.round_bf16(W) if dtype == "bf16" else W)
    return out


@pytest.mark.parametrize("ns,K,G,S,dtype", [
    ([64, 32, 48], 512, 128, 3, "bf16"),
    ([320, 320, 320], 640, 64, 4, "f32"),
    ([48, 37], 768, 256, 2, "bf16"),      # the last part ends mid row block
    ([16], 256, 64, 1, "f32"),
])
def test_pack_concat_bitexact(mbq, ns, K, G, S, dtype):
    say(f"pack concat {ns} K={K} G={G} S={S} {dtype}")
    Ws = parts(sum(ns) + K, ns, K, dtype)
    want, _ = oracle_blob(np.concatenate(Ws), G, S)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    p, starts = mbq.pack_concat([to_dev(W, tdt) for W in Ws], G, S, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert starts == [int(v) for v in np.cumsum([0] + ns[:-1])]
    got = p.blob.cpu().numpy()
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} bytes differ"


def test_pack_rows_any_order(mbq):
    """Parts write disjoint bytes: packing them last-first gives the same blob."""
    from token_adaptive_bit_amd import _lib
    ns, K = [32, 64, 21], 512
    Ws = parts(5, ns, K)
    want, _ = oracle_blob(np.concatenate(Ws), 128, 3)
    d = _lib.describe(sum(ns), K, 128, 3)
    blob = torch.full((int(d.total_bytes),), 0xAB, dtype=torch.uint8, device=DEV)
    starts = np.cumsum([0] + ns[:-1])
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = [to_dev(W, torch.bfloat16) for W in Ws]
    for i in reversed(range(len(ns))):
        _lib.check(_lib.LIB.mbq_pack_rows(ctypes.byref(d), int(starts[i]), ns[i],
                                          ctypes.c_void_p(ws[i].data_ptr()), _lib.MBQ_BF16,
                                          ctypes.c_void_p(blob.data_ptr()), None, s), "pack_rows")
    torch.cuda.synchronize()
    assert np.array_equal(blob.cpu().numpy(), want)


@pytest.mark.parametrize("T", [16, 50, 100, 300])
def test_fused_linear_parity(mbq, T):
    """q/k/v-like parts fused: each part's columns of the fused output against the oracle."""
    ns, K = [320, 160, 160], 1280
    say(f"fused linear T={T}")
    Ws = parts(9, ns, K)
    d = inputs.make_linear(10, 8, K, T)
    x = to_dev(d["X"], torch.bfloat16)
    _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    p, starts = mbq.pack_concat([to_dev(W, torch.bfloat16) for W in Ws], 128, 3)
    y = mbq.linear(p, x, perm, off)
    torch.cuda.synchronize()
    b = budget_from_perm(perm.cpu().numpy(), off.cpu().numpy())
    yg = y.float().cpu().numpy()
    for W, s0 in zip(Ws, starts):
        yref = oracle_linear_rows(W, d["X"], b, 128, 3)
        err = token_errors(yg[:, s0:s0 + W.shape[0]], yref)
        assert err.max() <= TOL

# (the 14B-like layer at full size, fused and separate, every output row:
# tests/test_gpu_full_size.py)
