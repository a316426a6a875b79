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


def run(mbq, N, K, G, S, T, dtype, rank, seed, rows=None, options=None):
    d = inputs.make_linear(seed, N, K, T, group=G, slices=S, dtype=dtype)
    lr = inputs.make_lowrank(seed + 1, N, K, rank=rank, b_scale=0.1)
    x = to_dev(d["X"], tdt(dtype))
    _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    p = mbq.pack(to_dev(d["W"], tdt(dtype)), group=G, slices=S)
    a, b = to_dev(lr["A"], torch.bfloat16), to_dev(lr["B"], torch.bfloat16)
    y = mbq.linear_lowrank(p, x, perm, off, a, b, out_dtype=torch.float32, options=options)
    y0 = mbq.linear(p, x, perm, off, out_dtype=torch.float32, options=options)
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


@pytest.mark.parametrize("T", [16, 100])
def test_lowrank_generic_kernels(mbq, T):
    """The generic kernels (decode at 16 tokens, prefill at 100) add the side path to y
    afterwards; same contract."""
    say(f"lowrank generic T={T}")
    check(*run(mbq, 160, 768, 128, 3, T, "bf16", 16, seed=7, options=mbq.opts(path="generic")))


def test_lowrank_generic_decode_g64_s4_f32(mbq):
    """Group 64, 4 slices, float32 activations: only the generic decode takes it."""
    check(*run(mbq, 64, 512, 64, 4, 16, "f32", 16, seed=8))


@pytest.mark.parametrize("K,dtype,rank", [(2304, "bf16", 8), (2304, "bf16", 16), (2304, "f32", 16),
                                          (1280, "f32", 8), (4096, "bf16", 16), (8192, "bf16", 16),
                                          (2304, "bf16", 32), (2304, "bf16", 24)])
def test_lowrank_decode_tiles_chunks_ranks(mbq, K, dtype, rank):
    """The decode side path across one and two k tiles per wave, K within one workgroup
    and split over workgroups (8192), both activation types and ranks 8, 16 and 32."""
    say(f"lowrank u placement K={K} {dtype} r={rank}")
    check(*run(mbq, 130, K, 128, 3, 16, dtype, rank, seed=K + rank))


def test_lowrank_inline_u_call_state(mbq):
    """Where the streaming decode computes u inside its own launch, the workspace carries
    call state from one call to the next.  Calls on one workspace with different
    activations, HIP-graph replays of one captured call with the activations changed
    between replays, eager calls in between and a call with fewer tokens on the same
    workspace all match the oracle; afterwards the state words read: launch count = calls
    made, an unused word 0, no error flag.  293 row blocks over 255 streaming workgroups:
    some stream two row blocks, most one."""
    N, K, G, S, T, rank = 4688, 3584, 128, 3, 16, 16
    d = inputs.make_linear(31, N, K, T, group=G, slices=S, dtype="bf16")
    lr = inputs.make_lowrank(32, N, K, rank=rank, b_scale=0.1)
    p = mbq.pack(to_dev(d["W"], torch.bfloat16), group=G, slices=S)
    pk = O.pack(d["W"], G, S)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    a, b = to_dev(lr["A"], torch.bfloat16), to_dev(lr["B"], torch.bfloat16)
    wr = to_dev(d["Wr"], torch.float32)
    xs = [d["X"]] + [inputs.make_linear(40 + i, 16, K, T, group=G, slices=S, dtype="bf16")["X"] for i in range(3)]
    ws = torch.zeros(mbq.linear_lowrank_workspace(p, T, rank), dtype=torch.uint8, device=DEV)
    xb = torch.empty((T, K), dtype=torch.bfloat16, device=DEV)
    perm = torch.empty(T, dtype=torch.int32, device=DEV)
    off = torch.empty(S + 1, dtype=torch.int32, device=DEV)
    y = torch.empty((T, N), dtype=torch.float32, device=DEV)

    def load(i):
        xb.copy_(to_dev(xs[i], torch.bfloat16))
        _, _, pm, of = mbq.route(xb, wr)
        perm.copy_(pm)
        off.copy_(of)
        y.zero_()

    def call():
        mbq.linear_lowrank(p, xb, perm, off, a, b, y=y, workspace=ws)

    def check(X, yy, pm, of):
        torch.cuda.synchronize()
        bud = budget_from_perm(pm.cpu().numpy(), of.cpu().numpy())
        yref = O.linear(X, deq, bud) + O.lowrank_term(X, lr["A"], lr["B"])
        err = token_errors(yy.cpu().numpy(), yref)
        say(f"  max token error {err.max():.3e}")
        assert err.max() <= TOL

    calls = 0
    for i in range(3):
        load(i)
        call()
        calls += 1
        check(xs[i], y, perm, off)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    calls += 1
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in (3, 0, 2, 1):
        load(i)
        g.replay()
        calls += 1
        check(xs[i], y, perm, off)
        y.zero_()
        call()                       # an eager call between replays
        calls += 1
        check(xs[i], y, perm, off)
    x5 = to_dev(xs[3][:5], torch.bfloat16)
    _, _, pm5, of5 = mbq.route(x5, wr)
    y5 = mbq.linear_lowrank(p, x5, pm5, of5, a, b, out_dtype=torch.float32, workspace=ws)
    calls += 1
    check(xs[3][:5], y5, pm5, of5)
    state = ws[:12].view(torch.int32).cpu().numpy().tolist()
    assert state == [calls, 0, 0]


def test_lowrank_inline_u_four_token_rows(mbq):
    """u computed inside the launch for four 16-token rows (64 tokens, one producing
    workgroup per row) with several row blocks parked per streaming workgroup."""
    say("lowrank inline u, 64 tokens, 293 row blocks")
    check(*run(mbq, 4688, 2304, 128, 3, 64, "bf16", 16, seed=77))
