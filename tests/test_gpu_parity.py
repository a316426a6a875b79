"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: packed codes and params bit-exact; routes bit-exact given identical logits;
regroup bit-exact; outputs within max_n |y - yref| / max_n |yref| <= 1e-2 per token
(bf16 I/O, fp32 accumulate), and a tighter bar where the arithmetic allows it.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import mbq_oracle as O
from token_adaptive_bit_amd import inputs
from parity import (TOL, budget_from_perm, oracle_blob, oracle_linear_rows, say,
                    token_errors)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mbq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from token_adaptive_bit_amd import api
    return api


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device=DEV, dtype=dtype)


def tdt(name):
    return torch.bfloat16 if name == "bf16" else torch.float32


def gpu_pack(mbq, W, group, slices, dtype):
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    p = mbq.pack(to_dev(W, tdt(dtype)), group=group, slices=slices, status=st)
    torch.cuda.synchronize()
    return p, int(st.item())


# ------------------------------------------------------------------------------ pack
PACK_CASES = [
    # N, K, G, S, dtype, seed, outliers
    (512, 256, 64, 3, "f32", 1, 4),       # the tiny workload's shape
    (200, 640, 128, 3, "bf16", 2, 3),     # ragged rows (not /16) and inputs (not /256)
    (33, 512, 256, 4, "bf16", 3, 0),
    (64, 256, 64, 1, "f32", 4, 2),
    (48, 768, 128, 2, "bf16", 5, 1),
    (17, 320, 64, 3, "f32", 6, 0),        # K = 320: 5 groups, one padded tile
]


@pytest.mark.parametrize("N,K,G,S,dtype,seed,outl", PACK_CASES)
def test_pack_bitexact(mbq, N, K, G, S, dtype, seed, outl):
    say(f"pack N={N} K={K} G={G} S={S} {dtype}")
    d = inputs.make_linear(seed, N, K, 1, group=G, slices=S, dtype=dtype, n_outliers=outl,
                           outlier_scale=20.0)
    want, _ = oracle_blob(d["W"], G, S)
    p, st = gpu_pack(mbq, d["W"], G, S, dtype)
    assert st == 0
    got = p.blob.cpu().numpy()
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


def test_pack_edge_groups(mbq):
    """Constant groups, exact grids, f16-subnormal steps, signed zeros, huge dynamic range."""
    rng = np.random.default_rng(7)
    W = (rng.standard_normal((32, 512)).astype(np.float32) * np.float32(0.02))
    W[0, :64] = 0.125                                       # constant
    W[1, :64] = np.float32(-0.375) + np.float32(0.125) * (np.arange(64) % 4)  # exact grid
    W[2, :64] = rng.standard_normal(64).astype(np.float32) * np.float32(1e-6)  # subnormal step
    W[3, :64] = 0.0
    W[3, 5] = -0.0
    W[3, 64:128] = -0.0                                     # signed-zero minimum
    W[3, 70] = 1.0
    W[4, :64] = rng.standard_normal(64).astype(np.float32) * np.float32(3e3)  # large
    W[5, 64:128] = np.float32(1e-30)                        # float32 tiny, half zero
    want, _ = oracle_blob(W, 64, 3)
    p, st = gpu_pack(mbq, W, 64, 3, "f32")
    assert st == 0
    got = p.blob.cpu().numpy()
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} bytes differ"


def test_pack_status_flags(mbq):
    W = np.zeros((16, 256), np.float32)
    W[3, 7] = np.inf
    _, st = gpu_pack(mbq, W, 64, 2, "f32")
    assert st & 1
    W = np.zeros((16, 256), np.float32)
    W[1, 1] = 3.0e5
    _, st = gpu_pack(mbq, W, 64, 1, "f32")
    assert st & 2
    assert O.pack(W, 64, 1)["flags"] & 2


def test_pack_full_decode_workload(mbq):
    """The 18944 x 3584 bf16 decode weight with outlier columns, all three slices."""
    say("pack full 18944x3584")
    d = inputs.make_workload("decode_18944x3584")
    want, _ = oracle_blob(d["W"], 128, 3)
    p, st = gpu_pack(mbq, d["W"], 128, 3, "bf16")
    assert st == 0
    got = p.blob.cpu().numpy()
    assert np.array_equal(got, want), f"{np.count_nonzero(got != want)} bytes differ"


# ------------------------------------------------------------------------------ route
@pytest.mark.parametrize("T,S", [(2048, 3), (1, 3), (37, 4), (5000, 2), (1025, 1)])
def test_route_from_logits_bitexact(mbq, T, S):
    say(f"route logits-in T={T} S={S}")
    rng = np.random.default_rng(T + S)
    L = np.round(rng.standard_normal((T, S)) * 2).astype(np.float32)   # many exact ties
    b, perm, off = mbq.route_from_logits(to_dev(L, torch.float32))
    torch.cuda.synchronize()
    wb = O.route_from_logits(L)
    wp, wo = O.regroup(wb, S)
    assert np.array_equal(b.cpu().numpy(), wb)
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(off.cpu().numpy(), wo)


def test_route_empty(mbq):
    L = torch.zeros((0, 3), dtype=torch.float32, device=DEV)
    b, perm, off = mbq.route_from_logits(L)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == [0, 0, 0, 0]


def check_route(mbq, d, x, S):
    logits, b, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    torch.cuda.synchronize()
    Lg = logits.cpu().numpy()
    Lref = O.router_logits(d["X"], d["Wr"])
    assert np.abs(Lg - Lref).max() <= 1e-5 * np.abs(Lref).max()
    # bit-exact given identical logits
    wb = O.route_from_logits(Lg)
    wp, wo = O.regroup(wb, S)
    assert np.array_equal(b.cpu().numpy(), wb)
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(off.cpu().numpy(), wo)
    # against float64 logits: a flip is allowed only at a near tie
    b64 = O.route_from_logits(Lref)
    flips = np.nonzero(b64 != wb)[0]
    for t in flips:
        top2 = np.sort(Lref[t])[-2:]
        assert top2[1] - top2[0] < 1e-4 * np.abs(Lref[t]).max()


# 16-byte aligned x and Wr with K % 8 == 0 take the vector logits loads, K = 100 (and the
# unaligned case below) the scalar loop; T <= 64 sorts in one wave, larger T in a workgroup
@pytest.mark.parametrize("cfg_dtype,T,K,S", [("f32", 16, 256, 3), ("bf16", 64, 5120, 3),
                                             ("bf16", 300, 4096, 3), ("bf16", 1, 3584, 3),
                                             ("bf16", 16, 3584, 1), ("f32", 33, 512, 2),
                                             ("bf16", 7, 13824, 4), ("bf16", 5, 100, 3)])
def test_route_with_router(mbq, cfg_dtype, T, K, S):
    say(f"route x T={T} K={K} S={S} {cfg_dtype}")
    d = inputs.make_linear(31, 8, K if K % 64 == 0 else 128, T, slices=S, dtype=cfg_dtype)
    if K % 64:  # a K no group divides: only the router is used here
        rng = np.random.default_rng(5)
        d = dict(d, X=rng.standard_normal((T, K)).astype(np.float32),
                 Wr=(rng.standard_normal((K, S)) * 0.1).astype(np.float32))
        if cfg_dtype == "bf16":
            d["X"] = torch.from_numpy(d["X"]).to(torch.bfloat16).float().numpy()
    check_route(mbq, d, to_dev(d["X"], tdt(cfg_dtype)), S)


@pytest.mark.parametrize("cfg_dtype", ["bf16", "f32"])
def test_route_unaligned_x(mbq, cfg_dtype):
    """x that is only element-aligned takes the scalar logits loop; same contract."""
    T, K, S = 16, 512, 3
    d = inputs.make_linear(32, 8, K, T, slices=S, dtype=cfg_dtype)
    buf = torch.zeros(T * K + 1, dtype=tdt(cfg_dtype), device=DEV)
    x = buf[1:].view(T, K)
    x.copy_(to_dev(d["X"], tdt(cfg_dtype)))
    assert x.data_ptr() % 16 != 0
    check_route(mbq, d, x, S)


def test_regroup_forced_mix(mbq):
    d = inputs.make_linear(3, 4, 64, 2048, forced_counts=inputs.forced_mix(2048, [0.3, 0.5, 0.2]))
    perm, off = mbq.regroup(to_dev(d["budget"], torch.int32), 3)
    torch.cuda.synchronize()
    wp, wo = O.regroup(d["budget"], 3)
    assert wo.tolist() == [0, 614, 1638, 2048]
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(off.cpu().numpy(), wo)


# ------------------------------------------------------------------------------ linear
def run_linear(mbq, d, budget=None, out_dtype=None, rows=None, options=None):
    """GPU pack + route/regroup + linear; returns (y_gpu, y_ref [T, rows], budget)."""
    G, S, dt = d["group"], d["slices"], d["dtype"]
    p, st = gpu_pack(mbq, d["W"], G, S, dt)
    assert st == 0
    x = to_dev(d["X"], tdt(dt))
    if budget is None:
        _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    else:
        perm, off = mbq.regroup(to_dev(budget, torch.int32), S)
    y = mbq.linear(p, x, perm, off, out_dtype=out_dtype or tdt(dt), options=options)
    torch.cuda.synchronize()
    b = budget_from_perm(perm.cpu().numpy(), off.cpu().numpy())
    if budget is not None:
        assert np.array_equal(b, budget)
    yref = oracle_linear_rows(d["W"], d["X"], b, G, S, rows)
    yg = y.float().cpu().numpy()
    if rows is not None:
        yg = yg[:, rows]
    return yg, yref, b


LINEAR_CASES = [
    # N, K, G, S, T, dtype, budget mode
    (512, 256, 64, 3, 16, "f32", "router"),     # the tiny workload
    (200, 640, 128, 3, 1, "bf16", "router"),
    (200, 640, 128, 3, 5, "bf16", "mix"),
    (200, 640, 128, 3, 17, "bf16", "mix"),
    (130, 768, 256, 4, 33, "bf16", "mix"),
    (96, 512, 64, 2, 64, "bf16", "mix"),
    (96, 512, 64, 3, 64, "bf16", "all1"),
    (96, 512, 64, 3, 40, "bf16", "allS"),
    (77, 384, 128, 1, 9, "f32", "allS"),
    # streaming decode with several 16-token blocks: 16 k tiles (two per wave), float32
    # activations (split into two bf16 operands), four slices at group 64
    (100, 4096, 128, 3, 64, "bf16", "mix"),
    (200, 640, 128, 3, 50, "f32", "mix"),
    (150, 2304, 64, 4, 48, "f32", "mix"),
    # two 16-token blocks per workgroup: group 64 with one slice, a partial second group
    (150, 2304, 64, 1, 48, "bf16", "mix"),
    (77, 1280, 256, 2, 63, "bf16", "mix"),
    # decode with K split over several workgroups (float32 partials in the workspace)
    (100, 5120, 128, 3, 64, "bf16", "mix"),
    (60, 13824, 128, 3, 20, "bf16", "mix"),
    (70, 2560, 64, 3, 7, "bf16", "allS"),
    (200, 640, 128, 3, 65, "bf16", "mix"),      # smallest prefill
    (200, 640, 128, 3, 300, "bf16", "mix"),
    (300, 1024, 128, 3, 257, "bf16", "router"),
    (130, 768, 256, 4, 200, "bf16", "mix"),
    (96, 512, 64, 2, 129, "f32", "mix"),
    (64, 256, 64, 3, 100, "bf16", "all1"),
    # MFMA prefill edges: one chunk of 64 inputs, odd chunk counts, several token tiles
    # per budget group, four slices at group 64, float32 activations over several tiles
    (40, 64, 64, 2, 70, "bf16", "mix"),
    (300, 192, 64, 3, 90, "bf16", "mix"),
    (272, 320, 64, 4, 700, "bf16", "mix"),
    (17, 448, 64, 1, 600, "bf16", "allS"),
    (520, 512, 128, 3, 530, "bf16", "all1"),
    (130, 640, 128, 4, 333, "f32", "mix"),
]


def budgets_for(mode, T, S, seed):
    rng = np.random.default_rng(seed)
    if mode == "mix":
        return rng.integers(1, S + 1, T).astype(np.int32)
    if mode == "all1":
        return np.ones(T, np.int32)
    if mode == "allS":
        return np.full(T, S, np.int32)
    return None


@pytest.mark.parametrize("N,K,G,S,T,dtype,mode", LINEAR_CASES)
def test_linear_parity(mbq, N, K, G, S, T, dtype, mode):
    say(f"linear N={N} K={K} G={G} S={S} T={T} {dtype} {mode}")
    d = inputs.make_linear(100 + T, N, K, T, group=G, slices=S, dtype=dtype, n_outliers=2,
                           outlier_scale=10.0)
    yg, yref, _ = run_linear(mbq, d, budgets_for(mode, T, S, T))
    err = token_errors(yg, yref)
    say(f"  max token error {err.max():.3e}")
    assert err.max() <= TOL
    if dtype == "f32" and T <= 64:
        assert err.max() <= 1e-4     # exact codes, split activations, float32 accumulate


def test_linear_fp32_output_from_bf16(mbq):
    d = inputs.make_linear(5, 160, 512, 12, dtype="bf16")
    yg, yref, _ = run_linear(mbq, d, budgets_for("mix", 12, 3, 1), out_dtype=torch.float32)
    assert token_errors(yg, yref).max() <= 1e-4


def test_prefill_fp32_output(mbq):
    d = inputs.make_linear(6, 300, 512, 150, dtype="bf16")
    yg, yref, _ = run_linear(mbq, d, budgets_for("mix", 150, 3, 2), out_dtype=torch.float32)
    assert token_errors(yg, yref).max() <= TOL


def test_prefill_generic_kernel(mbq):
    """The plain LDS prefill kernel (kept for activations or slices of 4 GiB and more)."""
    d = inputs.make_linear(7, 200, 640, 300, dtype="bf16", n_outliers=2, outlier_scale=10.0)
    yg, yref, _ = run_linear(mbq, d, budgets_for("mix", 300, 3, 3), options=mbq.opts(path="generic"))
    assert token_errors(yg, yref).max() <= TOL


@pytest.mark.parametrize("slots", [9, 10, 11, 12])
def test_prefill_halved_tail_tiles(mbq, slots):
    """Full tiles past the first round of workgroups halved into 128-token tiles.  With
    budget groups of 300 / 600 / 200 tokens and 600 outputs (3 column tiles) there are 12
    full tiles and 6 half tiles: 10 or 11 workgroup slots halve the last 2 or 1 (the last
    one holding 200 tokens: parts of 128 and 72), 9 and 12 halve none.  Against the oracle,
    and against the launch on the real CU count (no halving) within float32 rounding."""
    d = inputs.make_linear(8, 600, 512, 1100, group=128, slices=3, dtype="bf16", n_outliers=2,
                           outlier_scale=10.0)
    b = np.repeat(np.arange(1, 4, dtype=np.int32), [300, 600, 200])
    b = b[np.random.default_rng(8).permutation(1100)]
    base, _, _ = run_linear(mbq, d, b, out_dtype=torch.float32)
    say(f"prefill halved tail tiles, {slots} slots")
    yg, yref, _ = run_linear(mbq, d, b, out_dtype=torch.float32, options=mbq.opts(prefill_slots=slots))
    assert token_errors(yg, yref).max() <= TOL
    assert token_errors(yg, base.astype(np.float64)).max() <= 1e-6


@pytest.mark.parametrize("T,K,dtype", [(16, 640, "bf16"), (40, 5120, "bf16"), (9, 2304, "f32")])
def test_decode_generic_kernel(mbq, T, K, dtype):
    """The generic decode kernel (kept for slices of 4 GiB and more) against the oracle."""
    say(f"generic decode N=120 K={K} T={T} {dtype}")
    d = inputs.make_linear(7 + T, 120, K, T, group=128, slices=3, dtype=dtype)
    yg, yref, _ = run_linear(mbq, d, budgets_for("mix", T, 3, T), options=mbq.opts(path="generic"))
    assert token_errors(yg, yref).max() <= TOL


@pytest.mark.parametrize("T", [16, 200])
def test_linear_subnormal_scales(mbq, T):
    """Weights ~1e-5: the residual slices' float16 scales are subnormal and must count."""
    d = inputs.make_linear(8, 128, 512, T, dtype="bf16")
    d = dict(d, W=inputs.round_bf16(d["W"] * np.float32(1e-3)))
    p, _ = gpu_pack(mbq, d["W"], 128, 3, "bf16")
    s = O.pack(d["W"], 128, 3)["scale"]
    assert np.any((s[2] > 0) & (s[2] < np.float32(6.1e-5)))   # subnormal scales present
    yg, yref, _ = run_linear(mbq, d, budgets_for("allS", T, 3, 0), out_dtype=torch.float32)
    err = token_errors(yg, yref)
    say(f"  subnormal scales T={T}: max token error {err.max():.3e}")
    assert err.max() <= TOL


def test_linear_deterministic(mbq):
    for T in (16, 200):
        d = inputs.make_linear(9, 256, 1024, T)
        p, _ = gpu_pack(mbq, d["W"], 128, 3, "bf16")
        x = to_dev(d["X"], torch.bfloat16)
        _, _, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
        y1 = mbq.linear(p, x, perm, off).clone()
        y2 = mbq.linear(p, x, perm, off)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_linear_empty_batch(mbq):
    d = inputs.make_linear(9, 64, 256, 1)
    p, _ = gpu_pack(mbq, d["W"], 128, 3, "bf16")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=DEV)
    perm = torch.zeros(0, dtype=torch.int32, device=DEV)
    off = torch.zeros(4, dtype=torch.int32, device=DEV)
    y = mbq.linear(p, x, perm, off)
    torch.cuda.synchronize()
    assert y.shape == (0, 64)


# ------------------------------------------------------------------------------ variants
# (the five workloads at full size, every output row: tests/test_gpu_full_size.py)
@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K,T", [(512, 24), (2304, 40)])
def test_decode_every_variant(mbq, G, S, dtype, K, T):
    """Every group / slice count / activation type of the decode, with one or two k tiles
    per wave (K = 2304 is 9 tiles) and one or two 16-token blocks per workgroup."""
    say(f"decode variant G={G} S={S} {dtype} K={K} T={T}")
    d = inputs.make_linear(G + S + K, 96, K, T, group=G, slices=S, dtype=dtype)
    yg, yref, _ = run_linear(mbq, d)
    assert token_errors(yg, yref).max() <= TOL


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_generic_decode_every_variant(mbq, G, S, dtype):
    """The generic decode kernel over every group / slice count / activation type."""
    say(f"generic decode variant G={G} S={S} {dtype}")
    d = inputs.make_linear(G + S + 7, 96, 512, 24, group=G, slices=S, dtype=dtype)
    yg, yref, _ = run_linear(mbq, d, options=mbq.opts(path="generic"))
    assert token_errors(yg, yref).max() <= TOL


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("generic", [False, True])
def test_prefill_every_variant(mbq, G, S, dtype, generic):
    """The MFMA prefill (and the generic one) over every group / slice count / activation
    type, router-mixed budgets over 300 tokens (full and half tiles, ragged rows)."""
    say(f"prefill variant G={G} S={S} {dtype} generic={generic}")
    d = inputs.make_linear(G + S + 11, 200, 768, 300, group=G, slices=S, dtype=dtype)
    yg, yref, _ = run_linear(mbq, d, options=mbq.opts(path="generic" if generic else None))
    assert token_errors(yg, yref).max() <= TOL


@pytest.mark.parametrize("G,S", [(64, 2), (64, 3), (128, 3), (128, 4), (256, 2), (256, 4)])
@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (40, "bf16"), (16, "f32")])
def test_decode_single_slice(mbq, G, S, T, dtype):
    """Every token at budget 1 (the one-slice instantiation of the streaming loop, the
    other slices' loads out of range).  2307 row blocks (ragged N) give every workgroup
    about nine, so every buffer rotation and a ragged last round are crossed; every
    output row is compared."""
    say(f"single-slice decode G={G} S={S} T={T} {dtype}")
    d = inputs.make_linear(G + S + T, 36904, 512, T, group=G, slices=S, dtype=dtype)
    yg, yref, _ = run_linear(mbq, d, np.ones(T, np.int32))
    err = token_errors(yg, yref)
    say(f"  max token error {err.max():.3e}")
    assert err.max() <= TOL


def test_decode_step_graph_replays_match_eager(mbq):
    """The decode step (route + routed linear) captured in a HIP graph and replayed
    several times, with eager work in between, gives exactly the eager outputs."""
    d = inputs.make_linear(61, 300, 1280, 16, group=128, slices=3, dtype="bf16")
    x = to_dev(d["X"], torch.bfloat16)
    wr = to_dev(d["Wr"], torch.float32)
    p, _ = gpu_pack(mbq, d["W"], 128, 3, "bf16")
    logits = torch.empty((16, 3), dtype=torch.float32, device=DEV)
    b = torch.empty(16, dtype=torch.int32, device=DEV)
    perm = torch.empty(16, dtype=torch.int32, device=DEV)
    off = torch.empty(4, dtype=torch.int32, device=DEV)
    y = torch.empty((16, 300), dtype=torch.bfloat16, device=DEV)
    ws = torch.empty(max(1, mbq.linear_workspace(p, 16)), dtype=torch.uint8, device=DEV)

    def step():
        mbq.route(x, wr, logits, b, perm, off)
        mbq.linear(p, x, perm, off, y=y, workspace=ws)

    step()
    torch.cuda.synchronize()
    want = y.clone()
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
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want)
        step()                       # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, want)


@pytest.mark.parametrize("G", [64, 128, 256])
@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [1, 3, 4])
def test_linear_small_every_variant(mbq, G, S, T):
    """mbq_linear for 1 to 4 tokens: every group / slice count, budgets mixed over all
    slices, ragged N, 9 k tiles."""
    say(f"linear small G={G} S={S} T={T}")
    d = inputs.make_linear(G + S + T + 900, 300, 2304, T, group=G, slices=S, dtype="bf16")
    budget = (np.arange(T) % S + 1).astype(np.int32)[::-1].copy()
    yg, yref, _ = run_linear(mbq, d, budget)
    assert token_errors(yg, yref).max() <= TOL
