"""GPU parity of the one-call decode step (mbq_route_linear): MoBiRoute's linear-argmax
router, the stable regroup and the routed linear, against the oracle.

Bars (as for mbq_route and mbq_linear called apart):
  * logits within 1e-5 of the largest |logit| against the float64 oracle;
  * budget, perm, offsets bit-exact against the oracle's argmax and regroup applied to the
    logits this call wrote (the routes must follow the logits it reports), and against
    the float64 logits a budget may differ only at a near tie;
  * y within the per-token bar of 1e-2 against the float64 oracle on those budgets.
Where budgets agree with the two-call path (mbq_route, then mbq_linear), y must equal its
y bit for bit (the in-kernel routing changes where budgets come from, not the products),
except on the fp8 x fp4 multiply (MBQ_DECODE_F4, chosen by the plan from 4 row blocks per
workgroup), a different summation whose y must stay within 1e-3 per token of it.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mbq_oracle as O
from token_adaptive_bit_amd import inputs
from parity import TOL, say, token_errors

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


def run_case(mbq, N, K, G, S, T, dtype, seed, rows=None, f4=False):
    d = inputs.make_linear(seed, N, K, T, group=G, slices=S, dtype=dtype)
    x = to_dev(d["X"], tdt(dtype))
    wr = to_dev(d["Wr"], torch.float32)
    p = mbq.pack(to_dev(d["W"], tdt(dtype)), group=G, slices=S)
    y, lg, b, perm, off = mbq.route_linear(p, x, wr, out_dtype=torch.float32)
    # the two-call path on the same inputs
    lg2, b2, perm2, off2 = mbq.route(x, wr)
    y2 = mbq.linear(p, x, perm2, off2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Lg, bg, pg, og = (a.cpu().numpy() for a in (lg, b, perm, off))
    Lref = O.router_logits(d["X"], d["Wr"])
    assert np.abs(Lg - Lref).max() <= 1e-5 * max(np.abs(Lref).max(), 1e-30)
    wb = O.route_from_logits(Lg)
    wp, wo = O.regroup(wb, S)
    assert np.array_equal(bg, wb)
    assert np.array_equal(pg, wp)
    assert np.array_equal(og, wo)
    b64 = O.route_from_logits(Lref)
    for t in np.nonzero(b64 != wb)[0]:
        top2 = np.sort(Lref[t])[-2:]
        assert top2[1] - top2[0] < 1e-4 * np.abs(Lref[t]).max()
    W = d["W"] if rows is None else d["W"][rows]
    pk = O.pack(W, G, S)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    yref = O.linear(d["X"], deq, wb)
    yg, y2g = y.cpu().numpy(), y2.cpu().numpy()
    if rows is not None:
        yg, y2g = yg[:, rows], y2g[:, rows]
    err = token_errors(yg, yref)
    say(f"  max token error {err.max():.3e}")
    assert err.max() <= TOL
    if np.array_equal(b2.cpu().numpy(), bg):
        if f4:
            assert token_errors(yg, y2g.astype(np.float64)).max() <= 1e-3
        else:
            assert np.array_equal(yg, y2g), "same budgets, different y"
    return bg


# N, K, G, S, T, dtype: the first group takes the one-launch path, the rest fall back
FUSED = [
    (200, 640, 128, 3, 16, "bf16"),
    (150, 2304, 64, 4, 5, "bf16"),
    (300, 1024, 256, 2, 1, "bf16"),
    (96, 512, 128, 1, 8, "bf16"),
    (64, 4096, 128, 3, 16, "bf16"),     # 16 k tiles: the most one workgroup holds
    (257, 768, 64, 3, 11, "bf16"),      # ragged N and T
    (130, 1280, 256, 4, 16, "bf16"),
]
FALLBACK = [
    (64, 8192, 128, 3, 16, "bf16"),     # K split over workgroups
    (100, 640, 128, 3, 16, "f32"),      # float32 activations
    (100, 640, 128, 3, 20, "bf16"),     # more than one token block
    (100, 640, 128, 3, 200, "bf16"),    # prefill
]


@pytest.fixture
def bf16_mul(monkeypatch):
    monkeypatch.setenv("MBQ_DECODE_F4", "0")


@pytest.mark.parametrize("N,K,G,S,T,dtype", FUSED + FALLBACK)
def test_route_linear_parity(mbq, bf16_mul, N, K, G, S, T, dtype):
    say(f"route_linear N={N} K={K} G={G} S={S} T={T} {dtype}")
    run_case(mbq, N, K, G, S, T, dtype, seed=N + 7 * T)


@pytest.mark.parametrize("N,K,G,S,T,dtype", FUSED)
def test_route_linear_parity_f4(mbq, monkeypatch, N, K, G, S, T, dtype):
    """The same cases on the fp8 x fp4 multiply (forced on)."""
    monkeypatch.setenv("MBQ_DECODE_F4", "1")
    say(f"route_linear f4 N={N} K={K} G={G} S={S} T={T}")
    run_case(mbq, N, K, G, S, T, dtype, seed=N + 7 * T, f4=True)


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("f4", [False, True])
def test_route_linear_every_variant(mbq, monkeypatch, G, S, f4):
    """Every group / slice count of the in-kernel routing, with two k tiles per wave
    (K = 2560: 10 tiles over 8 waves) and a router that mixes budgets, on either multiply."""
    monkeypatch.setenv("MBQ_DECODE_F4", "1" if f4 else "0")
    say(f"route_linear variant G={G} S={S} f4={f4}")
    run_case(mbq, 80, 2560, G, S, 16, "bf16", seed=G + S, f4=f4)


@pytest.mark.parametrize("f4", [False, True])
def test_route_linear_one_tile_per_wave(mbq, monkeypatch, f4):
    """K of 8 tiles: one tile per wave."""
    monkeypatch.setenv("MBQ_DECODE_F4", "1" if f4 else "0")
    run_case(mbq, 120, 2048, 128, 3, 16, "bf16", seed=3, f4=f4)


def test_route_linear_uniform_budgets(mbq):
    """A router that sends every token to one budget: slices past it are never used."""
    d = inputs.make_linear(9, 160, 1024, 16, group=128, slices=3, dtype="bf16")
    x = to_dev(d["X"], torch.bfloat16)
    p = mbq.pack(to_dev(d["W"], torch.bfloat16), group=128, slices=3)
    xin = d["X"].copy()
    xin[:, 0] = 64.0                      # logit `top` = 64, the others 0
    x = to_dev(xin, torch.bfloat16)
    for top in range(3):
        Wr = np.zeros((1024, 3), np.float32)
        Wr[0, top] = 1.0
        y, lg, b, perm, off = mbq.route_linear(p, x, to_dev(Wr, torch.float32), out_dtype=torch.float32)
        torch.cuda.synchronize()
        bg = b.cpu().numpy()
        assert np.all(bg == top + 1)
        assert off.cpu().tolist() == [0] + [0 if v < top + 1 else 16 for v in range(1, 4)]
        pk = O.pack(d["W"], 128, 3)
        deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], 128)
        err = token_errors(y.cpu().numpy(), O.linear(xin, deq, bg))
        assert err.max() <= TOL


def test_route_linear_repeats_exactly(mbq):
    d = inputs.make_linear(21, 512, 3584, 16, group=128, slices=3, dtype="bf16")
    x = to_dev(d["X"], torch.bfloat16)
    wr = to_dev(d["Wr"], torch.float32)
    p = mbq.pack(to_dev(d["W"], torch.bfloat16), group=128, slices=3)
    a = [t.cpu() for t in mbq.route_linear(p, x, wr)]
    b = [t.cpu() for t in mbq.route_linear(p, x, wr)]
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_route_linear_empty(mbq):
    p = mbq.pack(torch.zeros((32, 256), dtype=torch.bfloat16, device=DEV), group=128, slices=3)
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    wr = torch.zeros((256, 3), dtype=torch.float32, device=DEV)
    y, lg, b, perm, off = mbq.route_linear(p, x, wr)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == [0, 0, 0, 0]
    assert y.shape == (0, 32)


@pytest.mark.parametrize("f4", [None, False])
def test_route_linear_full_decode_workload(mbq, monkeypatch, f4):
    """18944 x 3584, G128, S3, T = 16 (the one-launch path: 4.6 row blocks per workgroup,
    so the plan takes the fp4 multiply; then forced off); sampled rows against the oracle."""
    if f4 is not None:
        monkeypatch.setenv("MBQ_DECODE_F4", "0")
    else:
        monkeypatch.delenv("MBQ_DECODE_F4", raising=False)
    rows = np.unique(np.concatenate([[0, 18943], np.random.default_rng(5).choice(18944, 40, replace=False)]))
    say(f"route_linear full decode 18944x3584 T=16 f4={f4}")
    b = run_case(mbq, 18944, 3584, 128, 3, 16, "bf16", seed=2, rows=rows, f4=f4 is None)
    assert len(set(b.tolist())) >= 2   # the router mixes budgets here
