"""Host-only checks of the C ABI: the library loads, exports what include/mbq.h declares,
reports the blob geometry of the format, and rejects bad arguments before any launch.

No test here touches a GPU: every call either fails validation (and so launches nothing)
or is a host-only call (mbq_describe, mbq_linear_workspace, a t == 0 linear).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbq.h")

lib_mod = pytest.importorskip("token_adaptive_bit_amd._lib",
                              reason="libmbq.so not built (run __graft_entry__.build())")
L = lib_mod.LIB
OK, ARG, SHAPE, RANGE, WS, DEV, UNSUP = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
FAKE = 0x7F0000000000          # a 256-byte aligned address that is never dereferenced
P = ctypes.c_void_p


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mbq_status|const char\*|int32_t)\s+(mbq_\w+)\(", text, re.M)))


def test_exports_match_header():
    names = declared_functions()
    assert set(names) == set(lib_mod.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.mbq_abi_version() == 3


def test_status_strings():
    for code in (OK, ARG, SHAPE, RANGE, WS, DEV, UNSUP):
        assert L.mbq_status_str(code)
    assert L.mbq_status_str(123) == b"unknown status"


def desc(n, k, g, s):
    d = lib_mod.MbqDesc()
    st = L.mbq_describe(n, k, g, s, ctypes.byref(d))
    return st, d


def test_describe_geometry_matches_format():
    from oracle import mbq_oracle as O   # the format description, written independently
    for (n, k, g, s) in [(512, 256, 64, 3), (18944, 3584, 128, 3), (11008, 4096, 128, 3),
                         (200, 640, 128, 2), (5120, 13824, 128, 3), (17, 768, 256, 4),
                         (40, 96, 32, 3), (130, 544, 32, 4)]:
        st, d = desc(n, k, g, s)
        assert st == OK
        geo = O.blob_geometry(n, k, g, s)
        assert d.total_bytes == geo["total_bytes"]
        assert d.slice_stride == geo["slice_stride"]
        assert d.params_offset == geo["params_offset"]
        assert d.codes_bytes == geo["codes_bytes"] and d.params_bytes == geo["params_bytes"]
        assert (d.row_blocks, d.k_tiles, d.groups_padded) == (geo["NB"], geo["KB"], geo["NG"])


@pytest.mark.parametrize("n,k,g,s,want", [
    (16, 256, 16, 3, UNSUP), (16, 256, 96, 3, UNSUP), (16, 256, 64, 0, UNSUP),
    (16, 48, 32, 3, SHAPE),
    (16, 256, 64, 5, UNSUP), (0, 256, 64, 3, SHAPE), (16, 100, 64, 3, SHAPE),
    (16, 32, 64, 1, SHAPE), (-3, 256, 64, 1, SHAPE)])
def test_describe_rejects(n, k, g, s, want):
    st, _ = desc(n, k, g, s)
    assert st == want
    assert L.mbq_describe(16, 256, 64, 1, None) == ARG


def test_pack_validation():
    st, d = desc(64, 256, 64, 3)
    assert st == OK
    dp = ctypes.byref(d)
    assert L.mbq_pack(None, P(FAKE), F32, P(FAKE), None, None) == ARG
    assert L.mbq_pack(dp, None, F32, P(FAKE), None, None) == ARG
    assert L.mbq_pack(dp, P(FAKE), F32, None, None, None) == ARG
    assert L.mbq_pack(dp, P(FAKE), 7, P(FAKE), None, None) == ARG
    assert L.mbq_pack(dp, P(FAKE), F32, P(FAKE + 16), None, None) == ARG     # blob alignment
    assert L.mbq_pack(dp, P(FAKE + 2), F32, P(FAKE), None, None) == ARG      # f32 alignment
    assert L.mbq_pack(dp, P(FAKE), F32, P(FAKE), P(FAKE + 2), None) == ARG   # status alignment
    bad = lib_mod.MbqDesc.from_buffer_copy(d)
    bad.abi = 99
    assert L.mbq_pack(ctypes.byref(bad), P(FAKE), F32, P(FAKE), None, None) == UNSUP
    bad = lib_mod.MbqDesc.from_buffer_copy(d)
    bad.total_bytes += 256
    assert L.mbq_pack(ctypes.byref(bad), P(FAKE), F32, P(FAKE), None, None) == SHAPE


def test_pack_bitplane_validation():
    st, d = desc(100, 512, 128, 3)
    dp, f = ctypes.byref(d), P(FAKE)
    assert L.mbq_pack_bitplane(dp, None, F32, f, None, None) == ARG
    assert L.mbq_pack_bitplane(dp, f, 7, f, None, None) == ARG
    assert L.mbq_pack_bitplane(dp, f, F32, P(FAKE + 16), None, None) == ARG
    assert L.mbq_pack_bitplane(dp, f, F32, f, P(FAKE + 2), None) == ARG
    assert L.mbq_pack_bitplane(None, f, F32, f, None, None) == ARG


def test_pack_rows_validation():
    st, d = desc(100, 512, 128, 3)
    dp, f = ctypes.byref(d), P(FAKE)
    assert L.mbq_pack_rows(dp, 8, 16, f, F32, f, None, None) == SHAPE      # row0 not on a block
    assert L.mbq_pack_rows(dp, 0, 0, f, F32, f, None, None) == SHAPE       # no rows
    assert L.mbq_pack_rows(dp, -16, 16, f, F32, f, None, None) == SHAPE
    assert L.mbq_pack_rows(dp, 96, 16, f, F32, f, None, None) == SHAPE     # past n
    assert L.mbq_pack_rows(dp, 0, 40, f, F32, f, None, None) == SHAPE      # partial block mid-blob
    assert L.mbq_pack_rows(dp, 0, 16, None, F32, f, None, None) == ARG
    assert L.mbq_pack_rows(dp, 0, 16, f, 5, f, None, None) == ARG
    assert L.mbq_pack_rows(dp, 0, 16, f, F32, P(FAKE + 16), None, None) == ARG
    assert L.mbq_pack_rows(None, 0, 16, f, F32, f, None, None) == ARG


@pytest.mark.parametrize("N,K,G,S,t,rank,uchunks,chunks", [
    (18944, 3584, 128, 3, 16, 16, 7, 1),    # 14 k tiles: two per wave, no split
    (5120, 5120, 128, 3, 64, 16, 8, 2),     # one 16-token block per workgroup, K in 2 chunks
    (150, 2304, 64, 2, 48, 32, 4, 2),       # one tile per wave (group 64): K in 2 chunks
    (512, 256, 64, 3, 16, 8, 1, 1),         # K fits one workgroup: u only
    (11008, 4096, 128, 3, 2048, 16, 1, 1),  # prefill: u only
])
def test_linear_lowrank_workspace(N, K, G, S, t, rank, uchunks, chunks):
    """The side path's call state (256 bytes, 512 check-in lines of 128 bytes, then u of
    every 16-token block as 8-byte pairs rounded up to 256 bytes), u as uchunks float32
    partials [uchunks x t x rank] (rounded up to 256 bytes), then the decode's split-K
    partials under the side path's plan (one 16-token block per workgroup)."""
    st, d = desc(N, K, G, S)
    n = ctypes.c_size_t(123)
    assert L.mbq_linear_lowrank_workspace(ctypes.byref(d), t, BF16, rank, ctypes.byref(n)) == OK
    fb = 256 + 512 * 128 + ((t + 15) // 16 * 16 * rank * 8 + 255) // 256 * 256
    ub = (uchunks * t * rank * 4 + 255) // 256 * 256
    assert n.value == fb + ub + (chunks * t * N * 4 if chunks > 1 else 0)
    assert L.mbq_linear_lowrank_workspace(ctypes.byref(d), 0, BF16, rank, ctypes.byref(n)) == OK
    assert n.value == 0
    f = P(FAKE)
    need = fb + ub + (chunks * t * N * 4 if chunks > 1 else 0)
    for ws, wsb in ((None, 0), (f, need - 1), (P(FAKE + 8), need)):
        assert L.mbq_linear_lowrank(ctypes.byref(d), f, t, f, BF16, f, f, f, f, rank, f, BF16, ws, wsb,
                                    None, None) == WS


def test_linear_lowrank_validation():
    st, d = desc(200, 640, 128, 3)
    dp, f = ctypes.byref(d), P(FAKE)
    n = ctypes.c_size_t(0)
    for r in (0, 4, 12, 40, -8):
        assert L.mbq_linear_lowrank_workspace(dp, 16, BF16, r, ctypes.byref(n)) == UNSUP
        assert L.mbq_linear_lowrank(dp, f, 16, f, BF16, f, f, f, f, r, f, BF16, f, 1 << 30, None, None) == UNSUP

    def call(a=f, b=f, t=16):
        return L.mbq_linear_lowrank(dp, f, t, f, BF16, f, f, a, b, 16, f, BF16, f, 1 << 30, None, None)

    assert call(a=None) == ARG and call(b=None) == ARG
    assert call(a=P(FAKE + 8)) == ARG and call(b=P(FAKE + 2)) == ARG
    assert call(t=-1) == SHAPE
    assert call(t=0) == OK          # nothing to compute, nothing launched


def test_route_and_regroup_validation():
    f = P(FAKE)
    assert L.mbq_route(4, 16, 0, f, F32, f, f, f, f, f, None) == UNSUP
    assert L.mbq_route(4, 16, 5, f, F32, f, f, f, f, f, None) == UNSUP
    assert L.mbq_route(-1, 16, 3, f, F32, f, f, f, f, f, None) == SHAPE
    assert L.mbq_route(4, 0, 3, f, F32, f, f, f, f, f, None) == SHAPE
    assert L.mbq_route(4, 16, 3, f, 9, f, f, f, f, f, None) == ARG
    assert L.mbq_route(4, 16, 3, f, F32, None, f, f, f, f, None) == ARG
    assert L.mbq_route(4, 16, 3, f, F32, f, None, f, f, f, None) == ARG
    assert L.mbq_route(4, 16, 3, f, F32, f, f, f, P(FAKE + 1), f, None) == ARG
    assert L.mbq_regroup(4, 3, None, f, f, None) == ARG
    assert L.mbq_regroup(4, 0, f, f, f, None) == UNSUP
    assert L.mbq_regroup(-2, 3, f, f, f, None) == SHAPE


def test_route_linear_validation():
    """Errors of the one-call decode step, all caught before any launch (the shape here,
    16 bf16 tokens on a 200 x 640 weight, takes the one-launch path, which checks
    alignment itself)."""
    st, d = desc(200, 640, 128, 3)
    dp, f = ctypes.byref(d), P(FAKE)

    def call(**kw):
        a = dict(desc=dp, packed=f, t=16, x=f, xd=BF16, wr=f, lg=f, b=f, perm=f, off=f, y=f, yd=BF16)
        a.update(kw)
        return L.mbq_route_linear(a["desc"], a["packed"], a["t"], a["x"], a["xd"], a["wr"], a["lg"], a["b"],
                                  a["perm"], a["off"], a["y"], a["yd"], None, 0, a.get("o"), None)

    assert call(desc=None) == ARG
    assert call(t=-1) == SHAPE and call(t=1 << 25) == SHAPE
    assert call(xd=7) == ARG and call(yd=7) == ARG
    assert call(off=None) == ARG
    assert call(o=ctypes.byref(lib_mod.MbqOpts(0, 5, 0, 0))) == ARG
    assert call(o=ctypes.byref(lib_mod.MbqOpts(3, 0, 0, 0))) == ARG
    # two launches need the prepared operands' workspace (mbq_route_linear_workspace)
    n = ctypes.c_size_t(0)
    assert L.mbq_route_linear_workspace(dp, 16, BF16, ctypes.byref(n)) == OK
    assert n.value == 3 * (8192 + 512 + 2 * 64 + 256)     # 3 k tiles of 256 inputs, group 128
    assert call(o=ctypes.byref(lib_mod.MbqOpts(0, 2, 0, 2))) == WS
    assert L.mbq_route_linear_workspace(dp, 16, F32, ctypes.byref(n)) == OK and n.value == 0
    for k in ("packed", "x", "wr", "lg", "b", "perm", "y"):
        assert call(**{k: None}) == ARG, k
    assert call(packed=P(FAKE + 64)) == ARG
    assert call(x=P(FAKE + 8)) == ARG
    assert call(y=P(FAKE + 8)) == ARG
    assert call(perm=P(FAKE + 2)) == ARG and call(lg=P(FAKE + 2)) == ARG
    bad = lib_mod.MbqDesc.from_buffer_copy(d)
    bad.groups_padded += 1
    assert call(desc=ctypes.byref(bad)) == SHAPE


def mlp_ws(t, k, h):
    n = ctypes.c_size_t(123)
    st = L.mbq_route_mlp_workspace(t, k, h, ctypes.byref(n))
    return st, n.value


def test_route_mlp_validation():
    f = P(FAKE)
    st, need = mlp_ws(16, 3584, 256)
    assert st == OK and need > 0
    ws = ctypes.c_size_t(need)

    def call(t=16, k=3584, s=3, h=256, x=f, xd=BF16, w1=f, b1=f, w2=f, b2=f, delta=0.5,
             scores=f, budget=f, perm=f, offsets=f, ws_p=f, ws_b=None):
        return L.mbq_route_mlp(t, k, s, h, x, xd, w1, b1, w2, b2, delta, scores, budget, perm,
                               offsets, ws_p, need if ws_b is None else ws_b, None)

    assert call(s=0) == UNSUP and call(s=5) == UNSUP
    assert call(t=-1) == SHAPE and call(t=(1 << 24) + 1) == SHAPE
    assert call(delta=float("nan")) == RANGE
    assert call(offsets=None) == ARG
    assert call(budget=None) == ARG and call(perm=None) == ARG and call(scores=None) == ARG
    assert call(h=0) == SHAPE and call(h=96) == SHAPE and call(h=4160) == SHAPE
    assert call(k=0) == SHAPE
    assert call(xd=7) == ARG
    for name in ("w1", "b1", "w2", "b2"):
        assert call(**{name: None}) == ARG
    assert call(b1=P(FAKE + 4)) == ARG           # b1 is read as float4
    assert call(x=P(FAKE + 1)) == ARG and call(w1=P(FAKE + 1)) == ARG
    assert call(ws_p=None) == WS and call(ws_b=need - 1) == WS and call(ws_p=P(FAKE + 4)) == WS
    assert call(t=1 << 20, k=1 << 10, xd=F32, ws_b=1 << 40) == SHAPE   # x of 4 GiB
    assert call(h=4096, k=1 << 18, ws_b=1 << 40) == SHAPE              # W1 of 2 GiB
    # scores-in mode needs no weights and no workspace; s == 1 needs no scores
    # (these would launch, so only their argument checks are exercised by a bad stream-free
    #  field: a misaligned perm)
    assert call(x=None, w1=None, b1=None, w2=None, b2=None, ws_p=None, perm=P(FAKE + 2)) == ARG
    assert call(s=1, scores=None, ws_p=None, perm=P(FAKE + 2)) == ARG


@pytest.mark.parametrize("t,k,h,chunks", [
    (16, 3584, 256, 14), (1, 3584, 256, 14), (64, 5120, 256, 16), (65, 5120, 256, 16),
    (2048, 3584, 256, 8), (2048, 4096, 512, 4), (17, 100, 64, 1), (5, 256, 128, 1),
    (300, 64, 64, 1), (1024, 13824, 192, 16)])
def test_route_mlp_workspace(t, k, h, chunks):
    st, n = mlp_ws(t, k, h)
    assert st == OK and n == chunks * t * h * 4 + (256 if t <= 64 else 0)  # (+ per-token budget words)
    assert mlp_ws(0, k, h) == (OK, 0)
    assert mlp_ws(t, k, 100)[0] == SHAPE


def test_linear_validation_and_workspace():
    st, d = desc(200, 640, 128, 3)
    dp = ctypes.byref(d)
    f = P(FAKE)
    n = ctypes.c_size_t(123)
    # K = 640 fits one workgroup (3 k tiles): no k split, no scratch; prefill needs none
    for t, dt in ((16, BF16), (16, F32), (64, BF16), (1000, BF16), (0, F32)):
        assert L.mbq_linear_workspace(dp, t, dt, ctypes.byref(n)) == OK and n.value == 0
    assert L.mbq_linear_workspace(dp, -1, BF16, ctypes.byref(n)) == SHAPE
    assert L.mbq_linear_workspace(dp, 1, BF16, None) == ARG
    assert L.mbq_linear_workspace(dp, 1, 5, ctypes.byref(n)) == ARG
    args = lambda **kw: dict(dict(desc=dp, packed=f, t=16, x=f, xd=BF16, perm=f, off=f, y=f,
                                  yd=BF16, ws=None, wsb=0, o=None, s=None), **kw)
    call = lambda a: L.mbq_linear(a["desc"], a["packed"], a["t"], a["x"], a["xd"], a["perm"],
                                  a["off"], a["y"], a["yd"], a["ws"], a["wsb"], a["o"], a["s"])
    assert call(args(desc=None)) == ARG
    assert call(args(packed=None)) == ARG
    assert call(args(packed=P(FAKE + 64))) == ARG
    assert call(args(x=P(FAKE + 8))) == ARG
    assert call(args(y=None)) == ARG
    assert call(args(perm=P(FAKE + 2))) == ARG
    assert call(args(yd=3)) == ARG
    assert call(args(xd=3)) == ARG
    assert call(args(t=-1)) == SHAPE
    assert call(args(t=1 << 25)) == SHAPE
    bad = lib_mod.MbqDesc.from_buffer_copy(d)
    bad.groups_padded += 1
    assert call(args(desc=ctypes.byref(bad))) == SHAPE
    # nothing to do: every t-sized pointer may be NULL and nothing is launched
    assert call(args(t=0, x=None, perm=None, off=None, y=None, packed=None)) == OK
    # kernel choices: a field out of range is an argument error, found before any launch
    Opts = lib_mod.MbqOpts
    for o in (Opts(2, 0, 0, 0), Opts(-1, 0, 0, 0), Opts(0, 3, 0, 0), Opts(0, -1, 0, 0),
              Opts(0, 0, -1, 0), Opts(0, 0, 0, 3), Opts(0, 0, 0, -1)):
        assert call(args(o=ctypes.byref(o))) == ARG
        assert call(args(o=ctypes.byref(o), t=0, x=None, perm=None, off=None, y=None, packed=None)) == ARG
    assert call(args(o=ctypes.byref(Opts(1, 2, 300, 0)), t=0, x=None, perm=None, off=None, y=None,
                     packed=None)) == OK


def test_route_prepare_validation():
    """The two calls of the prepared decode step refuse bad arguments before any launch."""
    f = P(FAKE)
    st, d = desc(200, 640, 128, 3)
    dp = ctypes.byref(d)
    n = ctypes.c_size_t(0)
    assert L.mbq_route_prepare_workspace(dp, 16, ctypes.byref(n)) == OK
    need = n.value
    assert need == 3 * (8192 + 512 + 2 * 64 + 256)
    assert L.mbq_route_prepare_workspace(dp, 17, ctypes.byref(n)) == OK and n.value == 0
    assert L.mbq_route_prepare(dp, 16, f, f, f, need - 1, None) == WS
    assert L.mbq_route_prepare(dp, 16, f, f, None, need, None) == WS
    assert L.mbq_route_prepare(dp, 16, P(FAKE + 8), f, f, need, None) == ARG
    assert L.mbq_route_prepare(dp, 16, f, None, f, need, None) == ARG
    assert L.mbq_route_prepare(dp, 17, f, f, f, need, None) == UNSUP
    assert L.mbq_route_prepare(dp, 0, None, None, None, 0, None) == OK
    call = lambda **kw: L.mbq_route_linear_prepared(*[kw.get(k, v) for k, v in (
        ("desc", dp), ("packed", f), ("t", 16), ("prep", f), ("pb", need), ("lg", f), ("b", f), ("perm", f),
        ("off", f), ("y", f), ("yd", BF16), ("s", None))])
    assert call(pb=need - 1) == WS
    assert call(y=None) == ARG and call(off=None) == ARG and call(yd=5) == ARG
    assert call(packed=P(FAKE + 64)) == ARG
    assert call(t=17) == UNSUP
    assert call(t=0, packed=None, prep=None, lg=None, b=None, perm=None, y=None) == OK
    st1, d1 = desc(200, 640, 128, 1)            # one slice: no fp8 x fp4 step
    assert L.mbq_route_prepare_workspace(ctypes.byref(d1), 16, ctypes.byref(n)) == OK and n.value == 0
    assert L.mbq_route_prepare(ctypes.byref(d1), 16, f, f, f, need, None) == UNSUP
    st2, d2 = desc(200, 640, 32, 3)             # groups of 32: the generic kernels only
    assert st2 == OK
    assert L.mbq_route_prepare_workspace(ctypes.byref(d2), 16, ctypes.byref(n)) == OK and n.value == 0
    assert L.mbq_route_prepare(ctypes.byref(d2), 16, f, f, f, need, None) == UNSUP
    assert L.mbq_linear_workspace(ctypes.byref(d2), 16, BF16, ctypes.byref(n)) == OK and n.value == 0


def test_linear_static_limits():
    """The no-allocation linear refuses, before touching a device, any call whose split-K
    partials exceed the library's static buffer; an empty batch needs none."""
    assert lib_mod.STATIC_SCRATCH_BYTES == 16 << 20
    f = P(FAKE)
    st, d = desc(18944, 13824, 128, 3)     # 64 tokens: 7 chunks x 64 x 18944 x 4 bytes
    n = ctypes.c_size_t(0)
    assert L.mbq_linear_workspace(ctypes.byref(d), 64, BF16, ctypes.byref(n)) == OK
    assert n.value > lib_mod.STATIC_SCRATCH_BYTES
    assert L.mbq_linear_static(ctypes.byref(d), f, 64, f, BF16, f, f, f, BF16, None, None) == WS
    assert L.mbq_linear_static(ctypes.byref(d), f, 0, None, BF16, None, None, None, BF16, None, None) == OK
    assert L.mbq_linear_static(None, f, 16, f, BF16, f, f, f, BF16, None, None) == ARG
    assert L.mbq_linear_static(ctypes.byref(d), f, -1, f, BF16, f, f, f, BF16, None, None) == SHAPE
    bad = lib_mod.MbqOpts(0, 0, 0, 7)      # decode_launches out of range
    assert L.mbq_linear_static(ctypes.byref(d), f, 16, f, BF16, f, f, f, BF16, ctypes.byref(bad), None) == ARG


@pytest.mark.parametrize("N,K,G,S,t,dt,chunks", [
    (18944, 3584, 128, 3, 16, BF16, 1),   # 14 k tiles: two per wave, one workgroup
    (18944, 3584, 128, 3, 16, F32, 2),    # float32 activations: one tile per wave, 7 + 7
    (5120, 5120, 128, 3, 16, BF16, 2),    # 20 tiles, two per wave: 10 + 10
    (5120, 5120, 128, 3, 32, BF16, 2),    # up to 32 tokens: one 16-token block per workgroup
    (5120, 5120, 128, 3, 33, BF16, 3),    # two 16-token blocks per workgroup: one tile per wave, 7 + 7 + 6
    (5120, 5120, 128, 3, 64, BF16, 3),
    (5120, 13824, 128, 3, 64, BF16, 7),   # 54 tiles: 8 x 6 + 6
    (5120, 13824, 128, 4, 64, BF16, 7),   # group 128 with 4 slices: one block, one tile per wave
    (150, 2304, 64, 3, 48, F32, 2),       # 9 tiles, one per wave: 5 + 4
    (150, 2304, 64, 4, 48, F32, 0),       # group 64, 4 slices, float32: generic kernel
    (150, 2304, 64, 1, 48, BF16, 2),      # two blocks, one tile per wave: 5 + 4
    (150, 2304, 64, 1, 32, BF16, 1),      # one block: 9 tiles, two per wave
    (150, 2304, 64, 2, 48, BF16, 2),      # group 64, 2 slices: one block, one tile per wave
    (5120, 13824, 128, 3, 65, BF16, 0),   # prefill: no workspace
])
def test_decode_split_k_workspace(N, K, G, S, t, dt, chunks):
    """Decode over more k tiles than one workgroup holds (8 waves x 1 or 2 tiles; 1 when two
    16-token blocks share a workgroup, t > 32) splits K into equal chunks whose float32
    partials [chunks, t, N] live in the workspace."""
    st, d = desc(N, K, G, S)
    assert st == OK
    n = ctypes.c_size_t(123)
    assert L.mbq_linear_workspace(ctypes.byref(d), t, dt, ctypes.byref(n)) == OK
    assert n.value == (chunks * t * N * 4 if chunks > 1 else 0)
    if chunks > 1:  # a missing or short workspace is refused before any launch
        f = P(FAKE)
        for ws, wsb in ((None, 0), (f, n.value - 1)):
            assert L.mbq_linear(ctypes.byref(d), f, t, f, dt, f, f, f, BF16, ws, wsb, None, None) == WS
