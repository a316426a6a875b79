"""GPU parity of the bit-plane pack (mbq_pack_bitplane) against the oracle, and of the
routed linear on bit-plane blobs.

Bars: the blob bit-exact (codes, float16 params, padding); the routed linear within the
per-token bar of 1e-2 against the float64 oracle on the same slices (the linear kernels
do not know how the slices were made).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mbq_oracle as O
from token_adaptive_bit_amd import inputs
from parity import TOL, budget_from_perm, say, token_errors

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


def tdt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def oracle_bp_blob(W, G, S):
    p = O.pack_bitplane(W, G, S)
    return O.to_blob_fast(p["codes"], p["scale"], p["zero"], G), p


def gpu_bp(mbq, W, G, S, dtype):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = mbq.pack_bitplane(to_dev(W, tdt(dtype)), group=G, slices=S, status=st)
    torch.cuda.synchronize()
    return p, int(st.item())


@pytest.mark.parametrize("N,K,G,S,dtype,seed,outl", [
    (512, 256, 64, 3, "f32", 1, 4),
    (200, 640, 128, 3, "bf16", 2, 3),
    (33, 512, 256, 4, "bf16", 3, 0),
    (48, 768, 128, 2, "f32", 5, 1),
    (17, 320, 64, 1, "f32", 6, 0),
    (64, 512, 64, 4, "f32", 7, 2),
])
def test_pack_bitplane_bitexact(mbq, N, K, G, S, dtype, seed, outl):
    say(f"bitplane pack N={N} K={K} G={G} S={S} {dtype}")
    d = inputs.make_linear(seed, N, K, 1, group=G, slices=S, dtype=dtype, n_outliers=outl,
                           outlier_scale=20.0)
    want, pk = oracle_bp_blob(d["W"], G, S)
    p, st = gpu_bp(mbq, d["W"], G, S, dtype)
    assert st == pk["flags"] == 0
    got = p.blob.cpu().numpy()
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_pack_bitplane_edge_groups(mbq):
    rng = np.random.default_rng(9)
    W = rng.standard_normal((32, 512)).astype(np.float32) * np.float32(0.02)
    W[0, :64] = 0.125                                        # constant group
    W[1, :64] = (np.arange(64) % 64) / np.float32(64)        # exact 6-bit grid
    W[2, :64] = rng.standard_normal(64).astype(np.float32) * np.float32(1e-6)   # tiny step
    W[3, :64] = 0.0
    W[3, 64:128] = -0.0                                      # signed-zero minimum
    W[3, 70] = 1.0
    W[4, :64] = rng.standard_normal(64).astype(np.float32) * np.float32(3e3)   # large
    for S in (1, 3):
        want, pk = oracle_bp_blob(W, 64, S)
        p, st = gpu_bp(mbq, W, 64, S, "f32")
        assert st == pk["flags"]
        got = p.blob.cpu().numpy()
        assert np.array_equal(got, want), f"S={S}: {np.count_nonzero(got != want)} bytes differ"


def test_pack_bitplane_status_flags(mbq):
    W = np.zeros((16, 256), np.float32)
    W[3, 7] = np.inf
    _, st = gpu_bp(mbq, W, 64, 2, "f32")
    assert st & 1
    W = np.zeros((16, 256), np.float32)
    W[1, 1] = 3.0e5                    # step * 16 overflows half at 3 slices
    _, st = gpu_bp(mbq, W, 64, 3, "f32")
    assert st & 2 and O.pack_bitplane(W, 64, 3)["flags"] & 2


def test_pack_bitplane_full_decode_weight(mbq):
    say("bitplane pack full 18944x3584")
    d = inputs.make_workload("decode_18944x3584")
    want, _ = oracle_bp_blob(d["W"], 128, 3)
    p, st = gpu_bp(mbq, d["W"], 128, 3, "bf16")
    assert st == 0
    got = p.blob.cpu().numpy()
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} bytes differ"


@pytest.mark.parametrize("N,K,G,S,T,dtype", [
    (200, 640, 128, 3, 16, "bf16"), (150, 2304, 64, 4, 48, "f32"), (300, 1024, 128, 3, 300, "bf16"),
    (96, 512, 256, 2, 7, "f32"), (200, 768, 64, 3, 130, "f32"),
])
def test_linear_on_bitplane_blob(mbq, N, K, G, S, T, dtype):
    say(f"linear on bitplane N={N} K={K} G={G} S={S} T={T} {dtype}")
    d = inputs.make_linear(N + T, N, K, T, group=G, slices=S, dtype=dtype)
    x = to_dev(d["X"], tdt(dtype))
    _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    p, st = gpu_bp(mbq, d["W"], G, S, dtype)
    y = mbq.linear(p, x, perm, off, out_dtype=torch.float32)
    torch.cuda.synchronize()
    b = budget_from_perm(perm.cpu().numpy(), off.cpu().numpy())
    pk = O.pack_bitplane(d["W"], G, S)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    err = token_errors(y.cpu().numpy(), O.linear(d["X"], deq, b))
    assert err.max() <= TOL
