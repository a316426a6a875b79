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
except on the fp8 x fp4 multiply (mbq_opts decode_mul, chosen by the plan from 2 tokens and
4 row blocks per workgroup), a different summation whose y must stay within 1e-3 per token
of it.
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


def run_case(mbq, N, K, G, S, T, dtype, seed, rows=None, f4=False, mul="bf16", d=None, launches=0):
    """mul: the routed step's multiply (decode_mul; None lets the plan choose); f4: the
    call is expected to take the fp8 x fp4 multiply; launches: decode_launches (0 lets the
    plan choose, 2 prepares the fp8 operands once in a first launch)."""
    if d is None:
        d = inputs.make_linear(seed, N, K, T, group=G, slices=S, dtype=dtype)
    x = to_dev(d["X"][:T], tdt(dtype))
    wr = to_dev(d["Wr"], torch.float32)
    p = mbq.pack(to_dev(d["W"], tdt(dtype)), group=G, slices=S)
    y, lg, b, perm, off = mbq.route_linear(p, x, wr, out_dtype=torch.float32,
                                           options=mbq.opts(decode_mul=mul, decode_launches=launches))
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


@pytest.mark.parametrize("N,K,G,S,T,dtype", FUSED + FALLBACK)
def test_route_linear_parity(mbq, N, K, G, S, T, dtype):
    say(f"route_linear N={N} K={K} G={G} S={S} T={T} {dtype}")
    run_case(mbq, N, K, G, S, T, dtype, seed=N + 7 * T)


@pytest.mark.parametrize("launches", [1, 2])
@pytest.mark.parametrize("N,K,G,S,T,dtype", FUSED)
def test_route_linear_parity_f4(mbq, N, K, G, S, T, dtype, launches):
    """The same cases on the fp8 x fp4 multiply (forced on; one slice keeps bf16), in one
    launch and in two (operands prepared once)."""
    say(f"route_linear f4 N={N} K={K} G={G} S={S} T={T} launches={launches}")
    run_case(mbq, N, K, G, S, T, dtype, seed=N + 7 * T, f4=S > 1, mul="fp8fp4", launches=launches)


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("mode", ["bf16", "f4_one", "f4_two"])
def test_route_linear_every_variant(mbq, G, S, mode):
    """Every group / slice count of the routed step, with two k tiles per wave (K = 2560:
    10 tiles over 8 waves) and a router that mixes budgets, on the bf16 multiply and on the
    fp8 x fp4 one in one launch and in two."""
    say(f"route_linear variant G={G} S={S} {mode}")
    f4 = mode != "bf16"
    run_case(mbq, 80, 2560, G, S, 16, "bf16", seed=G + S, f4=f4 and S > 1, mul="fp8fp4" if f4 else "bf16",
             launches={"bf16": 1, "f4_one": 1, "f4_two": 2}[mode])


@pytest.mark.parametrize("f4", [False, True])
def test_route_linear_one_tile_per_wave(mbq, f4):
    """K of 8 tiles: one tile per wave (the fp8 x fp4 multiply in two launches)."""
    run_case(mbq, 120, 2048, 128, 3, 16, "bf16", seed=3, f4=f4, mul="fp8fp4" if f4 else "bf16",
             launches=2 if f4 else 1)


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


@pytest.mark.parametrize("G,S,K,T", [(128, 3, 3584, 16), (64, 2, 1536, 9), (256, 4, 1280, 13)])
def test_route_prepare_then_prepared(mbq, G, S, K, T):
    """The two calls apart give exactly what mbq_route_linear does in two launches, and
    one prepared buffer serves two weights with the same inputs (q / k -like)."""
    say(f"route prepare G={G} S={S} K={K} T={T}")
    d = inputs.make_linear(G + S + T, 144, K, T, group=G, slices=S)
    d2 = inputs.make_linear(G + S + T + 1, 80, K, T, group=G, slices=S)
    x, wr = to_dev(d["X"], torch.bfloat16), to_dev(d["Wr"], torch.float32)
    p = mbq.pack(to_dev(d["W"], torch.bfloat16), group=G, slices=S)
    p2 = mbq.pack(to_dev(d2["W"], torch.bfloat16), group=G, slices=S)
    want = mbq.route_linear(p, x, wr, out_dtype=torch.float32,
                            options=mbq.opts(decode_mul="fp8fp4", decode_launches=2))
    prep = mbq.route_prepare(p, x, wr)
    got = mbq.route_linear_prepared(p, T, prep, out_dtype=torch.float32)
    got2 = mbq.route_linear_prepared(p2, T, prep, out_dtype=torch.float32)
    torch.cuda.synchronize()
    for a, b in zip(want, got):
        assert torch.equal(a, b)
    b2 = got2[2].cpu().numpy()
    assert np.array_equal(b2, got[2].cpu().numpy())        # same routes for the second weight
    pk = O.pack(d2["W"], G, S)
    deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], G)
    assert token_errors(got2[0].cpu().numpy(), O.linear(d["X"], deq, b2)).max() <= TOL



@pytest.mark.parametrize("T,mul,launches", [(1, None, 0), (4, None, 0), (16, None, 0), (16, "bf16", 0),
                                            (16, "fp8fp4", 1)])
def test_route_linear_single_slice(mbq, T, mul, launches):
    """Router columns all equal: every logit ties, every token takes budget 1 (the first
    argmax), and the step streams one slice after routing in the kernel (one launch) or
    on prepared operands (two launches).  2307 row blocks; every row."""
    say(f"route_linear single slice T={T} mul={mul} launches={launches}")
    d = inputs.make_linear(500 + T, 36904, 1024, T, group=128, slices=3, dtype="bf16")
    d["Wr"] = np.repeat(d["Wr"][:, :1], 3, axis=1)
    run_case(mbq, 36904, 1024, 128, 3, T, "bf16", 0, mul=mul, d=d, launches=launches,
             f4=(mul == "fp8fp4" or (mul is None and T >= 2)))


@pytest.mark.parametrize("mul", [None, "fp8fp4"])
@pytest.mark.parametrize("b", [2, 3])
def test_route_linear_one_token_deep_budget(mbq, b, mul):
    """One token whose router picks 2 or 3 slices on 1184 row blocks (4-5 per workgroup):
    the one-token step issues row block 1 only after routing, with the slices the budget
    reads; y must equal the two-call path's bit for bit (the plan's bf16 multiply; within
    1e-3 per token on the fp8 x fp4 one) and the oracle's within the bar.  Router column
    b - 1 dominates, so the budget is b."""
    say(f"route_linear one token, budget {b}, mul {mul}")
    d = inputs.make_linear(600 + b, 18944, 1024, 1, group=128, slices=3, dtype="bf16")
    wr = np.zeros_like(d["Wr"])
    wr[:, b - 1] = np.abs(d["Wr"][:, b - 1]) * np.sign(d["X"][0]).astype(wr.dtype)
    d["Wr"] = wr
    bg = run_case(mbq, 18944, 1024, 128, 3, 1, "bf16", 0, mul=mul, d=d, f4=mul is not None)
    assert list(bg) == [b]


@pytest.mark.parametrize("T", [4, 16])
def test_route_linear_graph_replays_match_eager(mbq, T):
    """The routed step captured in a HIP graph (one launch at 4 tokens, two at 16: the
    operands prepared in the workspace first) and replayed several times, with eager work
    in between, writes exactly the eager outputs: y, logits, budget, perm and offsets."""
    say(f"route_linear graph replays T={T}")
    d = inputs.make_linear(70 + T, 16400, 1280, T, group=128, slices=3, dtype="bf16")
    x = to_dev(d["X"], torch.bfloat16)
    wr = to_dev(d["Wr"], torch.float32)
    p = mbq.pack(to_dev(d["W"], torch.bfloat16), group=128, slices=3)
    outs = dict(y=torch.empty((T, 16400), dtype=torch.bfloat16, device=DEV),
                logits=torch.empty((T, 3), dtype=torch.float32, device=DEV),
                budget=torch.empty(T, dtype=torch.int32, device=DEV),
                perm=torch.empty(T, dtype=torch.int32, device=DEV),
                offsets=torch.empty(4, dtype=torch.int32, device=DEV))
    ws = torch.empty(max(1, mbq.route_linear_workspace(p, T)), dtype=torch.uint8, device=DEV)

    def step():
        mbq.route_linear(p, x, wr, workspace=ws, **outs)

    step()
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in outs.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        for v in outs.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], want[k]), k
        step()                       # eager work between replays
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k], want[k]), k


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_route_linear_small_every_variant(mbq, G, S, T):
    """The plan's routed step for 1 to 4 tokens (one launch; the fp8 x fp4 multiply from 2
    tokens where a workgroup streams 4 row blocks): every group / slice count / token count,
    ragged N, K over 9 k tiles, router-mixed budgets."""
    say(f"route_linear small G={G} S={S} T={T}")
    run_case(mbq, 300, 2304, G, S, T, "bf16", seed=G + 10 * S + T, mul=None, f4=True)


@pytest.mark.parametrize("N,K,G,S,T", [(64, 13824, 128, 3, 1), (40, 256, 64, 2, 3), (17, 768, 256, 4, 4),
                                       (2048, 4096, 128, 3, 4)])
def test_route_linear_small_shapes(mbq, N, K, G, S, T):
    """The routed step for 1 to 4 tokens on a long K (54 k tiles: split over workgroups, so
    route then linear), a single tile, a row block that is mostly padding, and 128 row
    blocks."""
    say(f"route_linear small N={N} K={K} G={G} S={S} T={T}")
    run_case(mbq, N, K, G, S, T, "bf16", seed=N + K + T, mul=None, f4=True)
