"""GPU parity of the MLP router with threshold delta (mbq_route_mlp) against the oracle.

Bars:
  * scores: max |s - s_ref| <= SCORE_TOL * max(1, max |s_ref|) against the float64 oracle.
    The hidden layer multiplies bfloat16 x (or the bf16 hi + lo pair of float32 x, about
    16 mantissa bits) by bfloat16 W1 with float32 accumulation over K <= 5120 inputs; the
    worst-case float32 sum error there is ~1e-4 of the absolute sum, and the output layer
    adds a 256-term float32 dot product.  1e-3 is above every such bound and far below the
    O(0.1) change a dropped term, a wrong sign or a transposed operand would cause.
  * budgets, perm, offsets: bit-exact against the oracle's gate and regroup applied to
    the GPU's own float32 scores; against the float64 scores a budget may differ only
    where the deciding score lies within SCORE_TOL of the threshold.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mbq_oracle as O
from token_adaptive_bit_amd import inputs
from parity import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCORE_TOL = 1e-3


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


def dev_router(mbq, r):
    return mbq.MlpRouter(w1=to_dev(r["W1"], torch.bfloat16), b1=to_dev(r["b1"], torch.float32),
                         w2=to_dev(r["W2"], torch.float32), b2=to_dev(r["b2"], torch.float32))


def make_x(seed, T, K, dtype):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, K), dtype=np.float32)
    return inputs.round_bf16(X) if dtype == "bf16" else X


def check_gate(scores_gpu, b, perm, off, delta, S):
    th = O.gate_threshold(delta)
    wb = O.budgets_from_scores(scores_gpu, th)
    wp, wo = O.regroup(wb, S)
    assert np.array_equal(b, wb)
    assert np.array_equal(perm, wp)
    assert np.array_equal(off, wo)
    return wb


def check_route_mlp(mbq, X, x_dev, r, delta):
    S = r["slices"]
    T = X.shape[0]
    sc, b, perm, off = mbq.route_mlp(x_dev, dev_router(mbq, r), delta)
    torch.cuda.synchronize()
    sc, b, perm, off = (a.cpu().numpy() for a in (sc, b, perm, off))
    ref = O.mlp_router_scores(X, r["W1"], r["b1"], r["W2"], r["b2"])
    assert sc.shape == (T, S - 1)
    if S > 1 and T:
        err = np.abs(sc - ref).max()
        say(f"  max score error {err:.3e} (scale {np.abs(ref).max():.3f})")
        assert err <= SCORE_TOL * max(1.0, np.abs(ref).max())
    wb = check_gate(sc, b, perm, off, delta, S)
    # against the float64 scores: a budget may move only at a near tie with the threshold
    th = float(O.gate_threshold(delta))
    b64 = O.budgets_from_scores(ref, O.gate_threshold(delta))
    for t in np.nonzero(b64 != wb)[0]:
        j = min(b64[t], wb[t]) - 1            # the first residual slice the two disagree on
        assert abs(ref[t, j] - th) <= SCORE_TOL * max(1.0, np.abs(ref).max())
    return sc, wb


# dtype, T, K, hidden, S, delta
CASES = [
    ("bf16", 16, 3584, 256, 3, 0.5),    # decode batch on the 18944x3584 layer's input
    ("bf16", 2048, 4096, 256, 3, 0.5),  # prefill batch on the 11008x4096 layer's input
    ("f32", 16, 256, 64, 3, 0.3),       # the tiny float32 layer
    ("bf16", 64, 5120, 256, 3, 0.6),    # the 14B-like layer input, largest one-workgroup gate
    ("bf16", 65, 5120, 128, 4, 0.5),    # first batch past it: 64-token tiles, separate regroup
    ("f32", 300, 1000, 128, 2, 0.4),    # K % 32 != 0: a partial last k step
    ("bf16", 5, 100, 64, 3, 0.5),       # K % 8 != 0: element loads
    ("bf16", 33, 3584, 512, 4, 0.7),
    ("bf16", 1, 3584, 256, 3, 0.4),     # one token: one gate workgroup
    ("bf16", 63, 1024, 128, 3, 0.5),    # the last gate workgroup one wave short
    ("f32", 1, 64, 64, 3, 0.5),
    ("bf16", 16, 3584, 256, 1, 0.5),    # one slice: no scores, every budget 1
    ("bf16", 200, 13824, 64, 3, 0.45),  # long K (the down projection's input)
    ("bf16", 130, 2048, 192, 3, 0.5),   # a full and a half 128-unit tile, a ragged token tile
    ("f32", 1000, 4096, 256, 3, 0.5),
]


@pytest.mark.parametrize("dtype,T,K,H,S,delta", CASES)
def test_route_mlp_parity(mbq, dtype, T, K, H, S, delta):
    say(f"route_mlp {dtype} T={T} K={K} H={H} S={S} delta={delta}")
    r = inputs.make_mlp_router(100 + T, K, slices=S, hidden=H)
    X = make_x(200 + T, T, K, dtype)
    check_route_mlp(mbq, X, to_dev(X, tdt(dtype)), r, delta)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_route_mlp_unaligned_x(mbq, dtype):
    """x that is only element-aligned takes the element loads; same contract."""
    T, K = 20, 512
    say(f"route_mlp unaligned {dtype}")
    r = inputs.make_mlp_router(7, K, slices=3, hidden=128)
    X = make_x(8, T, K, dtype)
    buf = torch.zeros(T * K + 1, dtype=tdt(dtype), device=DEV)
    x = buf[1:].view(T, K)
    x.copy_(to_dev(X, tdt(dtype)))
    assert x.data_ptr() % 16 != 0
    check_route_mlp(mbq, X, x, r, 0.5)


def test_route_mlp_repeats_exactly(mbq):
    T, K = 48, 3584
    r = dev_router(mbq, inputs.make_mlp_router(3, K))
    x = to_dev(make_x(4, T, K, "bf16"), torch.bfloat16)
    a = [t.cpu() for t in mbq.route_mlp(x, r, 0.5)]
    b = [t.cpu() for t in mbq.route_mlp(x, r, 0.5)]
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("T,S", [(16, 3), (64, 4), (65, 2), (2048, 3), (1000, 1)])
def test_route_mlp_scores_in_bitexact(mbq, T, S):
    say(f"route_mlp scores-in T={T} S={S}")
    rng = np.random.default_rng(T * 7 + S)
    sc = (np.round(rng.standard_normal((T, S - 1)) * 4) / 4).astype(np.float32)  # many exact ties
    for delta in (0.5, 0.0, 1.0, 0.3, 0.75, -2.0, 3.0):
        b, perm, off = mbq.route_mlp_from_scores(to_dev(sc, torch.float32), delta)
        torch.cuda.synchronize()
        check_gate(sc, b.cpu().numpy(), perm.cpu().numpy(), off.cpu().numpy(), delta, S)


def test_route_mlp_empty(mbq):
    r = dev_router(mbq, inputs.make_mlp_router(1, 256))
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    sc, b, perm, off = mbq.route_mlp(x, r, 0.5)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("T", [16, 2048])
def test_route_mlp_delta_sweep(mbq, T):
    """Raising delta never adds a slice; delta 0 and 1 give every slice and the base only."""
    K, S = 3584, 3
    say(f"route_mlp delta sweep T={T}")
    r = dev_router(mbq, inputs.make_mlp_router(11, K, slices=S))
    x = to_dev(make_x(12, T, K, "bf16"), torch.bfloat16)
    prev, bits = None, []
    for delta in np.linspace(0.0, 1.0, 21):
        _, b, _, off = mbq.route_mlp(x, r, float(delta))
        b = b.cpu().numpy()
        if prev is not None:
            assert np.all(b <= prev)
        prev = b
        bits.append(O.average_bits(b))
        assert off.cpu().numpy()[-1] == T
    assert bits[0] == 2.0 * S and bits[-1] == 2.0
    assert len(set(bits)) >= 8
