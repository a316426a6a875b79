"""Host-only checks of the Python binding's argument validation.

The C ABI carries pointers, not sizes, so the binding must refuse a tensor of the wrong
shape, dtype or device before any call reaches the library.  Here the library's compute
entry points are replaced by a recorder (its host-only calls -- describe, workspace
sizes -- stay real) and CPU tensors stand in for device tensors: every mismatch must
raise without a compute call being made, and a well-formed call must make exactly one.
"""
import pytest

torch = pytest.importorskip("torch")

from token_adaptive_bit_amd import _lib, api   # noqa: E402


class Recorder:
    HOST = {"mbq_describe", "mbq_linear_workspace", "mbq_linear_lowrank_workspace", "mbq_route_linear_workspace",
            "mbq_route_mlp_workspace", "mbq_status_str", "mbq_abi_version"}

    def __init__(self, lib):
        self.lib = lib
        self.calls = []

    def __getattr__(self, name):
        if name in self.HOST:
            return getattr(self.lib, name)

        def call(*args):
            self.calls.append(name)
            return 0
        return call


@pytest.fixture
def rec(monkeypatch):
    r = Recorder(_lib.LIB)
    monkeypatch.setattr(_lib, "LIB", r)
    monkeypatch.setattr(api, "_stream", lambda: None)

    def dev(t, name):            # everything but the device check
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    monkeypatch.setattr(api, "_dev", dev)
    return r


N, K, T = 64, 256, 8
bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32


def packed():
    d = api.describe(N, K, 128, 3)
    return api.PackedLinear(d, torch.zeros(int(d.total_bytes), dtype=torch.uint8))


def good():
    return dict(x=torch.zeros((T, K), dtype=bf), perm=torch.zeros(T, dtype=i32),
                off=torch.zeros(4, dtype=i32), y=torch.zeros((T, N), dtype=bf))


def test_linear_accepts_and_forwards(rec):
    g = good()
    api.linear(packed(), g["x"], g["perm"], g["off"], y=g["y"])
    assert rec.calls == ["mbq_linear"]


@pytest.mark.parametrize("field,bad,exc", [
    ("x", torch.zeros((T, K + 64), dtype=bf), ValueError),      # wrong K
    ("x", torch.zeros((T, K), dtype=torch.float16), TypeError),
    ("x", torch.zeros((T, K * 2), dtype=bf)[:, ::2], ValueError),  # not contiguous
    ("perm", torch.zeros(T - 1, dtype=i32), ValueError),
    ("perm", torch.zeros(T, dtype=torch.int64), TypeError),
    ("off", torch.zeros(3, dtype=i32), ValueError),
    ("y", torch.zeros((T, N - 1), dtype=bf), ValueError),
    ("y", torch.zeros((T + 1, N), dtype=bf), ValueError),
    ("y", torch.zeros((T, N), dtype=torch.int32), TypeError),
])
def test_linear_refuses_mismatch(rec, field, bad, exc):
    g = good()
    g[field] = bad
    with pytest.raises(exc):
        api.linear(packed(), g["x"], g["perm"], g["off"], y=g["y"])
    with pytest.raises(exc):
        api.linear_static(packed(), g["x"], g["perm"], g["off"], y=g["y"])
    assert rec.calls == []


def test_linear_refuses_short_blob_and_workspace(rec):
    g = good()
    p = packed()
    short = api.PackedLinear(p.desc, p.blob[:-1])
    with pytest.raises(ValueError):
        api.linear(short, g["x"], g["perm"], g["off"], y=g["y"])
    big = api.describe(N, 8192, 128, 3)          # 32 k tiles: the decode splits K
    pb = api.PackedLinear(big, torch.zeros(int(big.total_bytes), dtype=torch.uint8))
    need = api.linear_workspace(pb, T)
    assert need > 0
    with pytest.raises(ValueError):
        api.linear(pb, torch.zeros((T, 8192), dtype=bf), g["perm"], g["off"], y=g["y"],
                   workspace=torch.zeros(need - 1, dtype=torch.uint8))
    assert rec.calls == []


def test_route_and_route_linear_refuse_mismatch(rec):
    g = good()
    with pytest.raises(ValueError):
        api.route(g["x"], torch.zeros((K - 1, 3), dtype=f32))
    with pytest.raises(TypeError):
        api.route(g["x"], torch.zeros((K, 3), dtype=bf))
    with pytest.raises(ValueError):
        api.route(g["x"], torch.zeros((K, 3), dtype=f32), logits=torch.zeros((T, 2), dtype=f32))
    with pytest.raises(ValueError):
        api.route_linear(packed(), g["x"], torch.zeros((K, 2), dtype=f32))   # slices differ
    with pytest.raises(ValueError):
        api.route_linear(packed(), g["x"], torch.zeros((K, 3), dtype=f32), budget=torch.zeros(T + 1, dtype=i32))
    with pytest.raises(TypeError):
        api.regroup(torch.zeros(T, dtype=torch.int64), 3)
    assert rec.calls == []
    api.route_linear(packed(), g["x"], torch.zeros((K, 3), dtype=f32))
    assert rec.calls == ["mbq_route_linear"]


def test_lowrank_and_mlp_refuse_mismatch(rec):
    g = good()
    a, b = torch.zeros((16, K), dtype=bf), torch.zeros((N, 16), dtype=bf)
    for bad in ((torch.zeros((16, K - 64), dtype=bf), b), (a, torch.zeros((N, 8), dtype=bf)),
                (a.float(), b), (a, b.float())):
        with pytest.raises((ValueError, TypeError)):
            api.linear_lowrank(packed(), g["x"], g["perm"], g["off"], *bad, y=g["y"])
    r = api.MlpRouter(torch.zeros((64, K), dtype=bf), torch.zeros(64, dtype=f32),
                      torch.zeros((64, 2), dtype=f32), torch.zeros(2, dtype=f32))
    for field, bad in (("w1", torch.zeros((64, K + 64), dtype=bf)), ("b1", torch.zeros(63, dtype=f32)),
                       ("w2", torch.zeros((63, 2), dtype=f32)), ("b2", torch.zeros(3, dtype=f32)),
                       ("w1", torch.zeros((64, K), dtype=f32))):
        rb = api.MlpRouter(**{**r.__dict__, field: bad})
        with pytest.raises((ValueError, TypeError)):
            api.route_mlp(g["x"], rb, 0.5)
    assert rec.calls == []
    api.route_mlp(g["x"], r, 0.5)
    assert rec.calls == ["mbq_route_mlp"]


def test_pack_refuses_bad_weights(rec):
    with pytest.raises(TypeError):
        api.pack(torch.zeros((N, K), dtype=torch.float16))
    with pytest.raises(ValueError):
        api.pack(torch.zeros((N, K), dtype=bf), out=torch.zeros(10, dtype=torch.uint8))
    with pytest.raises(ValueError):
        api.pack(torch.zeros((N, K), dtype=bf), status=torch.zeros(2, dtype=i32))
    assert rec.calls == []


def test_opts_values():
    o = api.opts(path="generic", decode_mul="fp8fp4", prefill_slots=12, decode_launches=2)
    assert (o.path, o.decode_mul, o.prefill_slots, o.decode_launches) == (1, 2, 12, 2)
    for kw in (dict(path="fast"), dict(decode_mul="fp8"), dict(prefill_slots=-1), dict(decode_launches=3)):
        with pytest.raises(ValueError):
            api.opts(**kw)
