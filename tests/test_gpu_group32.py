"""Groups of 32 inputs on the GPU, against the oracle.

A group of 32 is half of a lane's 64-input code vector (word i of lanes c = 2h, 2h + 1),
so the streaming decode and the MFMA prefill do not take it; the pack kernels, the
generic decode (one MFMA pass per half of each code word, the other half's activations
zeroed) and the generic prefill (the lane's group looked up per 16-input word) do.  The
shapes include K with K % 64 == 32 (the last group ends half way through a 64-input
step) and K % 256 != 0 (a padded k tile), ragged N, every slice count and both
activation types; the plan picks the generic kernels by itself.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mbq_oracle as O
from token_adaptive_bit_amd import inputs
from parity import TOL, budget_from_perm, say, token_errors

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
G = 32


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


@pytest.mark.parametrize("N,K,S,dtype,seed,outl", [
    (40, 96, 3, "f32", 1, 2),        # K = 96: three groups in one padded tile
    (130, 544, 4, "bf16", 2, 3),     # K % 256 = 32
    (17, 352, 1, "f32", 3, 0),
    (200, 640, 2, "bf16", 4, 1),
])
@pytest.mark.parametrize("kind", ["residual", "bitplane"])
def test_pack_group32_bitexact(mbq, N, K, S, dtype, seed, outl, kind):
    say(f"G=32 {kind} pack N={N} K={K} S={S} {dtype}")
    d = inputs.make_linear(seed, N, K, 1, group=G, slices=S, dtype=dtype, n_outliers=outl,
                           outlier_scale=20.0)
    pk = O.pack(d["W"], G, S) if kind == "residual" else O.pack_bitplane(d["W"], G, S)
    want = O.to_blob_fast(pk["codes"], pk["scale"], pk["zero"], G)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    packer = mbq.pack if kind == "residual" else mbq.pack_bitplane
    p = packer(to_dev(d["W"], tdt(dtype)), group=G, slices=S, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = p.blob.cpu().numpy()
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def run(mbq, N, K, S, T, dtype, seed, budget=None, options=None):
    d = inputs.make_linear(seed, N, K, T, group=G, slices=S, dtype=dtype, n_outliers=2,
                           outlier_scale=10.0)
    x = to_dev(d["X"], tdt(dtype))
    if budget is None:
        _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    else:
        perm, off = mbq.regroup(to_dev(budget, torch.int32), S)
    p = mbq.pack(to_dev(d["W"], tdt(dtype)), group=G, slices=S)
    y = mbq.linear(p, x, perm, off, out_dtype=torch.float32, options=options)
    torch.cuda.synchronize()
    b = budget_from_perm(perm.cpu().numpy(), off.cpu().numpy())
    pk = O.pack(d["W"], G, S)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    return y.cpu().numpy(), O.linear(d["X"], deq, b), d, p, b


@pytest.mark.parametrize("N,K,S,T,dtype", [
    (200, 352, 3, 1, "bf16"),
    (200, 352, 3, 16, "bf16"),
    (150, 544, 4, 17, "f32"),
    (96, 2304, 2, 48, "bf16"),       # nine k tiles over the waves
    (77, 96, 3, 64, "f32"),          # one padded tile, four 16-token blocks
    (300, 1024, 3, 65, "bf16"),      # prefill
    (130, 352, 4, 300, "bf16"),
    (200, 544, 2, 200, "f32"),
])
def test_linear_group32(mbq, N, K, S, T, dtype):
    say(f"G=32 linear N={N} K={K} S={S} T={T} {dtype}")
    yg, yref, *_ = run(mbq, N, K, S, T, dtype, seed=N + T)
    err = token_errors(yg, yref)
    say(f"  max token error {err.max():.3e}")
    assert err.max() <= TOL
    if dtype == "f32" and T <= 64:
        assert err.max() <= 1e-4     # exact codes, split activations, float32 accumulate


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [24, 300])
def test_group32_every_variant(mbq, S, dtype, T):
    """Every slice count and activation type, decode (two 16-token blocks) and prefill,
    budgets mixed over every slice count."""
    say(f"G=32 variant S={S} {dtype} T={T}")
    budget = np.random.default_rng(S + T).integers(1, S + 1, T).astype(np.int32)
    yg, yref, *_ = run(mbq, 96, 352, S, T, dtype, seed=S + T, budget=budget)
    assert token_errors(yg, yref).max() <= TOL


def test_route_linear_group32(mbq):
    """The decode step in one call takes route + linear for groups of 32."""
    d = inputs.make_linear(9, 160, 544, 16, group=G, slices=3, dtype="bf16")
    x = to_dev(d["X"], torch.bfloat16)
    p = mbq.pack(to_dev(d["W"], torch.bfloat16), group=G, slices=3)
    y, lg, b, perm, off = mbq.route_linear(p, x, to_dev(d["Wr"], torch.float32))
    torch.cuda.synchronize()
    wb = O.route_from_logits(lg.cpu().numpy())
    assert np.array_equal(b.cpu().numpy(), wb)
    pk = O.pack(d["W"], G, 3)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    assert token_errors(y.float().cpu().numpy(), O.linear(d["X"], deq, wb)).max() <= TOL


@pytest.mark.parametrize("T", [16, 100])
def test_lowrank_group32(mbq, T):
    """The side path on the generic kernels (added to y afterwards)."""
    yg0, yref, d, p, b = run(mbq, 160, 352, 3, T, "bf16", seed=T)
    lr = inputs.make_lowrank(T + 1, 160, 352, rank=16, b_scale=0.1)
    x = to_dev(d["X"], torch.bfloat16)
    perm, off = mbq.regroup(to_dev(b, torch.int32), 3)
    y = mbq.linear_lowrank(p, x, perm, off, to_dev(lr["A"], torch.bfloat16), to_dev(lr["B"], torch.bfloat16),
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    term = O.lowrank_term(d["X"], lr["A"], lr["B"])
    assert token_errors(y.cpu().numpy(), yref + term).max() <= TOL
