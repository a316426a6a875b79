"""GPU parity at the five workloads' own sizes and inputs, every output compared.

Each workload's weight is packed on the GPU and the blob compared byte for byte with the
oracle's; the routed linear's y is compared with the oracle's float64 y on every output
row of every token, at the per-token bar (max_n |y - yref| / max_n |yref| <= 1e-2).
Routes come from the GPU (their own bit-exact contract is tested on identical logits),
or are the workloads' forced budget mixes.

The oracle products of one weight are computed once per module and reused by the cases
that share it; nothing here reads a result of the HIP path except to compare it.
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


class Packed:
    """One weight, packed by the oracle and by the GPU, with the oracle's dequantized slices."""

    def __init__(self, mbq, W, group=128, slices=3):
        self.W, self.group, self.slices = W, group, slices
        self.pk = O.pack(W, group, slices)
        self.deq = O.dequant_slices(self.pk["codes"], self.pk["scale"], self.pk["zero"], group)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        self.p = mbq.pack(to_dev(W, torch.bfloat16), group=group, slices=slices, status=st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0

    def check_blob(self):
        want = O.to_blob_fast(self.pk["codes"], self.pk["scale"], self.pk["zero"], self.group)
        got = self.p.blob.cpu().numpy()
        assert got.shape == want.shape
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"{bad.size} blob bytes differ, first at {bad[:8]}"

    def yref(self, X, budget):
        return O.linear(X, self.deq, budget)


def compare(y, yref, bar=TOL, what=""):
    err = token_errors(y.float().cpu().numpy(), yref)
    say(f"  {what} every row: max token error {err.max():.3e}")
    assert err.max() <= bar
    return err


def check_routes(logits, budget, perm, off, X, Wr, S):
    """Routing outputs of a call: logits within 1e-5 of the float64 oracle, budgets and the
    regroup exactly the oracle's argmax and stable sort of the logits the call wrote."""
    Lg = logits.cpu().numpy()
    Lref = O.router_logits(X, Wr)
    assert np.abs(Lg - Lref).max() <= 1e-5 * np.abs(Lref).max()
    wb = O.route_from_logits(Lg)
    wp, wo = O.regroup(wb, S)
    assert np.array_equal(budget.cpu().numpy(), wb)
    assert np.array_equal(perm.cpu().numpy(), wp)
    assert np.array_equal(off.cpu().numpy(), wo)
    return wb


# ---------------------------------------------------------------- decode GEMV 18944 x 3584
@pytest.fixture(scope="module")
def decode_w(mbq):
    say("packing the 18944 x 3584 decode weight (oracle and GPU)")
    d = inputs.make_workload("decode_18944x3584")
    pw = Packed(mbq, d["W"])
    yield d, pw
    del pw


def test_decode_18944x3584_blob_bitexact(decode_w):
    decode_w[1].check_blob()


@pytest.mark.parametrize("T", [1, 4, 16])
@pytest.mark.parametrize("mul,launches", [(None, 0), ("bf16", 1), ("fp8fp4", 1), ("fp8fp4", 2)])
def test_decode_18944x3584_route_linear_every_row(mbq, decode_w, T, mul, launches):
    """The decode step in one call (the benchmark's step) on the workload's own inputs, on
    the plan's choices and on each multiply and launch count forced."""
    d, pw = decode_w
    say(f"decode 18944x3584 route_linear T={T} decode_mul={mul} launches={launches}")
    X = d["X"][:T]
    y, lg, b, perm, off = mbq.route_linear(pw.p, to_dev(X, torch.bfloat16), to_dev(d["Wr"], torch.float32),
                                           options=mbq.opts(decode_mul=mul, decode_launches=launches))
    torch.cuda.synchronize()
    wb = check_routes(lg, b, perm, off, X, d["Wr"], 3)
    compare(y, pw.yref(X, wb), what=f"T={T} {mul}")


@pytest.mark.parametrize("T", [1, 4, 16, 17, 33, 64])
def test_decode_18944x3584_two_call_every_row(mbq, decode_w, T):
    """mbq_route then mbq_linear for every decode batch size (two 16-token blocks per
    workgroup above 32 tokens)."""
    d, pw = decode_w
    say(f"decode 18944x3584 route + linear T={T}")
    X = d["X"][:T] if T <= 16 else inputs.make_linear(2, 8, 3584, T)["X"]
    x = to_dev(X, torch.bfloat16)
    lg, b, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
    y = mbq.linear(pw.p, x, perm, off)
    torch.cuda.synchronize()
    wb = check_routes(lg, b, perm, off, X, d["Wr"], 3)
    compare(y, pw.yref(X, wb), what=f"T={T}")


# ---------------------------------------------------------------- prefill 11008 x 4096
def test_prefill_11008x4096_every_row(mbq):
    say("prefill 11008 x 4096, T = 2048, forced 614 / 1024 / 410")
    d = inputs.make_workload("prefill_11008x4096")
    pw = Packed(mbq, d["W"])
    pw.check_blob()
    perm, off = mbq.regroup(to_dev(d["budget"], torch.int32), 3)
    y = mbq.linear(pw.p, to_dev(d["X"], torch.bfloat16), perm, off)
    torch.cuda.synchronize()
    assert off.cpu().tolist() == [0, 614, 1638, 2048]
    assert np.array_equal(budget_from_perm(perm.cpu().numpy(), off.cpu().numpy()), d["budget"])
    compare(y, pw.yref(d["X"], d["budget"]), what="prefill_w")


# ---------------------------------------------------------------- elasticity sweep 14336 x 4096
@pytest.fixture(scope="module")
def sweep_w(mbq):
    say("packing the 14336 x 4096 sweep weight (oracle and GPU)")
    d = inputs.make_workload("sweep_14336x4096")
    pw = Packed(mbq, d["W"])
    yield d, pw
    del pw


def test_sweep_14336x4096_blob_bitexact(sweep_w):
    sweep_w[1].check_blob()


@pytest.mark.parametrize("T", [32, 1024])
@pytest.mark.parametrize("mode", ["b1", "b2", "b3", "router"])
def test_sweep_14336x4096_every_row(mbq, sweep_w, T, mode):
    d, pw = sweep_w
    say(f"sweep 14336x4096 T={T} {mode}")
    X = d["X"][:T]
    x = to_dev(X, torch.bfloat16)
    if mode == "router":
        lg, b, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
        torch.cuda.synchronize()
        budget = check_routes(lg, b, perm, off, X, d["Wr"], 3)
    else:
        budget = np.full(T, int(mode[1]), np.int32)
        perm, off = mbq.regroup(to_dev(budget, torch.int32), 3)
    y = mbq.linear(pw.p, x, perm, off)
    torch.cuda.synchronize()
    compare(y, pw.yref(X, budget), what=f"T={T} {mode}")


# ---------------------------------------------------------------- 14B-like layer, T = 64
@pytest.fixture(scope="module")
def layer_w(mbq):
    lay = inputs.make_workload("layer14b_t64")
    x0 = to_dev(lay["X_layer"], torch.bfloat16)
    lg, b, perm, off = mbq.route(x0, to_dev(lay["Wr"], torch.float32))
    torch.cuda.synchronize()
    budget = check_routes(lg, b, perm, off, lay["X_layer"], lay["Wr"], 3)
    return lay, perm, off, budget


def test_layer14b_every_row(mbq, layer_w):
    """The seven linears one by one: blob bytes and every output row."""
    lay, perm, off, budget = layer_w
    for lin in lay["linears"]:
        say(f"layer14b {lin['name']} {lin['W'].shape}")
        pw = Packed(mbq, lin["W"])
        pw.check_blob()
        y = mbq.linear(pw.p, to_dev(lin["X"], torch.bfloat16), perm, off)
        torch.cuda.synchronize()
        compare(y, pw.yref(lin["X"], budget), what=lin["name"])
        del pw


def test_layer14b_fused_every_row(mbq, layer_w):
    """q/k/v and gate/up packed as one blob each (row concatenation) and run as one
    launch each: the fused blob is the oracle's pack of the stacked rows, and every
    output column of the fused y is compared."""
    lay, perm, off, budget = layer_w
    lin = {l["name"]: l for l in lay["linears"]}
    for names, xname in ((["q", "k", "v"], "q"), (["gate", "up"], "gate")):
        say(f"layer14b fused {'/'.join(names)}")
        Ws = [lin[n]["W"] for n in names]
        p, starts = mbq.pack_concat([to_dev(W, torch.bfloat16) for W in Ws], 128, 3)
        X = lin[xname]["X"]
        y = mbq.linear(p, to_dev(X, torch.bfloat16), perm, off)
        torch.cuda.synchronize()
        Wcat = np.concatenate(Ws, axis=0)
        pk = O.pack(Wcat, 128, 3)
        want = O.to_blob_fast(pk["codes"], pk["scale"], pk["zero"], 128)
        assert np.array_equal(p.blob.cpu().numpy(), want)
        deq = O.dequant_slices(pk["codes"], pk["scale"], pk["zero"], 128)
        compare(y, O.linear(X, deq, budget), what="/".join(names))
        assert starts == list(np.cumsum([0] + [W.shape[0] for W in Ws[:-1]]))
        del p, deq, pk


# ---------------------------------------------------------------- low-rank side path, full sizes
@pytest.mark.parametrize("name,T,seed", [("decode_18944x3584", 16, 202), ("prefill_11008x4096", 2048, 203)])
def test_lowrank_full_every_row(mbq, name, T, seed):
    """Rank-16 side path on the decode and prefill workloads' weights (B ~ N(0, 0.1^2),
    so the side path is a large part of every output)."""
    d = inputs.make_workload(name)
    say(f"lowrank full {name} T={T}")
    lr = inputs.make_lowrank(seed, d["N"], d["K"], rank=16, b_scale=0.1)
    X = d["X"][:T]
    x = to_dev(X, torch.bfloat16)
    if d["budget"] is not None:
        budget = d["budget"]
        perm, off = mbq.regroup(to_dev(budget, torch.int32), 3)
    else:
        lg, b, perm, off = mbq.route(x, to_dev(d["Wr"], torch.float32))
        torch.cuda.synchronize()
        budget = check_routes(lg, b, perm, off, X, d["Wr"], 3)
    pw = Packed(mbq, d["W"])
    y = mbq.linear_lowrank(pw.p, x, perm, off, to_dev(lr["A"], torch.bfloat16), to_dev(lr["B"], torch.bfloat16))
    torch.cuda.synchronize()
    compare(y, pw.yref(X, budget) + O.lowrank_term(X, lr["A"], lr["B"]), what=f"lowrank {name}")
