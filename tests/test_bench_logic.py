"""Host-only checks of bench.py's bookkeeping: the algorithmic byte counts behind the
roofline, the rotation rule, the reading of committed traffic summaries, and the refusal
of more than one GPU.  No GPU, no library calls beyond mbq_describe."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

torch = pytest.importorskip("torch")
from token_adaptive_bit_amd import api  # noqa: E402


def packed(n, k, g=128, s=3):
    d = api.describe(n, k, g, s)
    return api.PackedLinear(d, torch.zeros(1, dtype=torch.uint8))


def test_decode_bytes_by_hand():
    """The decode workload at 16 tokens, 3 slices read, on prepared operands: the slices,
    the prepared operands, y and the routing outputs, counted by hand from the blob
    layout (1184 row blocks x 14 k tiles x 1 KiB codes, 1184 x 28 groups x 64 B params)."""
    p = packed(18944, 3584)
    slice_bytes = 1184 * 14 * 1024 + 1184 * 28 * 64          # both multiples of 256
    assert int(p.desc.slice_stride) == slice_bytes
    prep = 14 * (8192 + 512 + 2 * 64 + 256)
    y = 16 * 18944 * 2
    routing = 16 * 3 * 4 + 2 * 16 * 4 + 4 * 4               # logits, budget + perm, offsets
    assert bench.decode_bytes(p, 16, 3, router=True, prep_bytes=prep) == 3 * slice_bytes + prep + y + routing
    assert bench.decode_bytes(p, 16, 3, router=True, prep_bytes=prep) == 58020432
    # one launch (activations and Wr read instead of the prepared operands)
    x = 16 * 3584 * 2
    wr = 3584 * 3 * 4
    assert bench.decode_bytes(p, 16, 3, router=True) == 3 * slice_bytes + x + y + wr + routing
    # the plain linear: perm and offsets read
    assert bench.decode_bytes(p, 16, 1) == slice_bytes + x + y + 16 * 4 + 4 * 4
    assert bench.weight_bytes(p, 2) == 2 * slice_bytes


def test_rotation_covers_512_mib():
    for nbytes in (1 << 20, 57286656, 38043648, 300 << 20, 1 << 30):
        n = bench.copies_for(nbytes)
        assert n >= 2 and n * nbytes >= 512 << 20


def test_traffic_summary_needs_the_measured_source(tmp_path, monkeypatch):
    """A committed traffic summary counts only while its kernel source is the one that was
    measured (its SHA-256 is stored)."""
    csrc = tmp_path / "token_adaptive_bit_amd" / "csrc"
    prof = tmp_path / "profiles"
    csrc.mkdir(parents=True)
    prof.mkdir()
    (csrc / "k.hip").write_bytes(b"kernel source")
    sha = hashlib.sha256(b"kernel source").hexdigest()
    (prof / "k_traffic.txt").write_text(f"# title\nhbm_bytes_per_launch: 123456\nsource_sha256: {sha}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.traffic_from_profile("k.hip", "k_traffic.txt") == 123456.0
    (csrc / "k.hip").write_bytes(b"kernel source, changed")
    assert bench.traffic_from_profile("k.hip", "k_traffic.txt") is None
    assert bench.traffic_from_profile("k.hip", "missing.txt") is None


def test_committed_decode_traffic_matches_its_source():
    """The committed decode traffic summary was measured on the kernel source as it stands."""
    v = bench.traffic_from_profile("decode_stream.hip", "decode_stream_18944x3584_t16_traffic.txt")
    assert v is not None and 0.95 * 58020432 < v < 1.1 * 58020432


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
