"""GPU parity of the routed linear with the low-rank side path (mbq_linear_lowrank)
against the oracle: y_t = x_t . W^(b(t))^T + (x_t . A^T) . B^T.

The factors are drawn with B ~ N(0, 0.1^2) here, so the side path is a sizeable part of
every output (about half the routed term's spread): a dropped, doubled or mis-indexed
side path breaks the per-token bar of 1e-2 by far.  Each case also checks the side path
on its own: (y_lowrank - y_plain) against the oracle's (x A^T) B^T, to 2e-2 of its
largest value per token (both GPU outputs are rounded once to their dtype).
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


def run(mbq, N, K, G, S, T, dtype, rank, seed, rows=None):
    d = inputs.make_linear(seed, N, K, T, group=G, slices=S, dtype=dtype)
    lr = inputs.make_lowrank(seed + 1, N, K, rank=rank, b_scale=0.1)
    x = to_dev(d["X"], tdt(dtype))
    _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    p = mbq.pack(to_dev(d["W"], tdt(dtype)), group=G, slices=S)
    a, b = to_dev(lr["A"], torch.bfloat16), to_dev(lr["B"], torch.bfloat16)
    y = mbq.linear_lowrank(p, x, perm, off, a, b, out_dtype=torch.float32)
    y0 = mbq.linear(p, x, perm, off, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bud = budget_from_perm(perm.cpu().numpy(), off.cpu().numpy())
    W = d["W"] if rows is None else d["W"][rows]
    Bm = lr["B"] if rows is None else lr["B"][rows]
    pk = O.pack(W, G, S)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    term = O.lowrank_term(d["X"], lr["A"], Bm)
    yref = O.linear(d["X"], deq, bud) + term
    yg, y0g = y.cpu().numpy(), y0.cpu().numpy()
    if rows is not None:
        yg, y0g = yg[:, rows], y0g[:, rows]
    return yg, y0g, yref, term


def check(yg, y0g, yref, term):
    err = token_errors(yg, yref)
    say(f"  max token error {err.max():.3e}")
    assert err.max() <= TOL
    side = token_errors(yg - y0g, term)
    assert side.max() <= 2e-2


CASES = [
    # N, K, G, S, T, dtype, rank
    (200, 640, 128, 3, 1, "bf16", 16),
    (200, 640, 128, 3, 16, "bf16", 16),
    (130, 768, 256, 4, 33, "bf16", 32),
    (96, 512, 64, 2, 64, "bf16", 8),
    (150, 2304, 64, 3, 48, "f32", 24),     # split K (two chunks), float32 activations
    (100, 4096, 128, 3, 64, "bf16", 16),   # split K in two chunks
    (77, 1280, 256, 1, 20, "f32", 16),
    (300, 1024, 128, 3, 65, "bf16", 16),   # prefill
    (257, 640, 64, 4, 300, "bf16", 32),
    (200, 512, 128, 2, 200, "f32", 8),     # prefill with float32 activations
]


@pytest.mark.parametrize("N,K,G,S,T,dtype,rank", CASES)
def test_lowrank_parity(mbq, N, K, G, S, T, dtype, rank):
    say(f"lowrank N={N} K={K} G={G} S={S} T={T} {dtype} r={rank}")
    check(*run(mbq, N, K, G, S, T, dtype, rank, seed=N + T))


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lowrank_every_decode_variant(mbq, G, S, dtype):
    """Every group / slice count / activation type of the decode with the side path
    (two 16-token blocks, router-mixed budgets, two k tiles)."""
    say(f"lowrank variant G={G} S={S} {dtype}")
    check(*run(mbq, 96, 512, G, S, 24, dtype, 16, seed=G + 10 * S))


@pytest.mark.parametrize("env,T", [("MBQ_GENERIC_DECODE", 16), ("MBQ_GENERIC_PREFILL", 100)])
def test_lowrank_generic_kernels(mbq, monkeypatch, env, T):
    """The generic kernels add the side path to y afterwards; same contract."""
    monkeypatch.setenv(env, "1")
    say(f"lowrank generic {env} T={T}")
    check(*run(mbq, 160, 768, 128, 3, T, "bf16", 16, seed=7))


def test_lowrank_generic_decode_g64_s4_f32(mbq):
    """Group 64, 4 slices, float32 activations: only the generic decode takes it."""
    check(*run(mbq, 64, 512, 64, 4, 16, "f32", 16, seed=8))


def test_lowrank_full_decode_workload(mbq):
    """18944 x 3584, G128, S3, T = 16, rank 16; sampled rows against the oracle."""
    rows = np.unique(np.concatenate([[0, 18943], np.random.default_rng(3).choice(18944, 40, replace=False)]))
    say("lowrank full decode 18944x3584 T=16")
    check(*run(mbq, 18944, 3584, 128, 3, 16, "bf16", 16, seed=2, rows=rows))


def test_lowrank_full_prefill_workload(mbq):
    """11008 x 4096, G128, S3, T = 2048, rank 16; sampled rows against the oracle."""
    rows = np.unique(np.concatenate([[0, 11007], np.random.default_rng(4).choice(11008, 24, replace=False)]))
    say("lowrank full prefill 11008x4096 T=2048")
    check(*run(mbq, 11008, 4096, 128, 3, 2048, "bf16", 16, seed=3, rows=rows))
