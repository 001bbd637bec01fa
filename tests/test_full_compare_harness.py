"""The full-size comparison harness (tests/full_compare.py), run on the CPU
with "GPU outputs" made by the oracle itself: it accepts them, and it
reports a single changed byte in any output of each kind of path.  The
shared files it writes are removed afterwards."""
import glob

import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests import full_compare as fc


def _site(rows=96, cols=2048, seed=3):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    xr = F.f32_to_bf16_rne(v.reshape(-1))
    xt = F.f32_to_bf16_rne((v * (1 + 0.05 * rng.standard_normal(v.shape))).astype(np.float32).reshape(-1))
    g = F.f32_to_bf16_rne(rng.standard_normal(v.size).astype(np.float32))
    return xr, xt, g


@pytest.fixture(autouse=True)
def small_chunks(monkeypatch):
    monkeypatch.setattr(fc, "CHUNK_ELEMS", 1 << 14)   # several chunks on a small site


def test_nvfp4_harness_accepts_and_detects():
    xr, xt, g = _site()
    with fc.Shared({"xr": xr, "xt": xt, "g": g}) as sh:
        ts = fc.tensor_scale_of(sh)
        assert ts.view(np.uint32) == np.float32(oracle.tensor_scale(xr)).view(np.uint32)
        want = fc._oracle_nvfp4(xr, xt, g, ts)
        assert fc.compare_every_element("ok", sh, want, ts) == xr.size
        for key in ("bits", "y_f", "gin", "q_r"):
            bad = dict(want)
            bad[key] = want[key].copy()
            bad[key][bad[key].size // 2 + 1] ^= 1
            with pytest.raises(AssertionError, match=key):
                fc.compare_every_element("planted", sh, bad, ts)
        d = sh.dir
    assert not glob.glob(d)


@pytest.mark.parametrize("kind", ["mx", "mx8"])
def test_variant_harness_accepts_and_detects(kind):
    xr, xt, g = _site(seed=4)
    want = fc._oracle_variant(kind, xr, xt, g, "with_rne")
    assert fc.compare_variant_every_element("ok", kind, xr, xt, want, extra="with_rne", g=g) == xr.size
    bad = dict(want)
    bad["m_r"] = want["m_r"].copy()
    bad["m_r"][-1] ^= 0x80
    with pytest.raises(AssertionError, match="m_r"):
        fc.compare_variant_every_element("planted", kind, xr, xt, bad, extra="with_rne", g=g)


def test_lowbits_harness_checks_every_plane():
    xr, xt, _ = _site(seed=5)
    ts = np.float32(oracle.tensor_scale(xr))
    want = fc._oracle_variant("lowbits", xr, xt, None, (ts, 3))
    assert fc.compare_variant_every_element("ok", "lowbits", xr, xt, want, extra=(ts, 3)) == xr.size
    bad = dict(want)
    bad["planes"] = want["planes"].copy()
    bad["planes"][2 * (xr.size // 8) + 5] ^= 4          # plane 2
    with pytest.raises(AssertionError, match="planes"):
        fc.compare_variant_every_element("planted", "lowbits", xr, xt, bad, extra=(ts, 3))


def test_grouped_harness_keeps_each_rows_group():
    rows, cols = 96, 512
    xr, xt, _ = _site(rows, cols, seed=6)
    off = np.array([0, 10, 10, 50, 96], dtype=np.int64)
    ts = oracle.grouped_tensor_scale(xr, rows, cols, off)
    want = fc._oracle_grouped(xr, xt, rows, cols, off, ts)
    assert fc.compare_grouped_every_element("ok", xr, xt, rows, cols, off, ts, want) == rows * cols
    bad = dict(want)
    bad["scales"] = want["scales"].copy()
    bad["scales"][(50 * cols) // 16] ^= 1              # first block of the last group
    with pytest.raises(AssertionError, match="scales"):
        fc.compare_grouped_every_element("planted", xr, xt, rows, cols, off, ts, bad)


def test_shared_files_hold_tensor_bytes():
    import torch
    x = torch.randn(64, 32).to(torch.bfloat16)
    b = torch.randint(0, 256, (777,), dtype=torch.uint8)
    with fc.Shared({"x": x, "b": b, "h": np.arange(5, dtype=np.uint16)}) as sh:
        assert np.array_equal(fc._read(sh.specs["x"], 0, x.numel()), x.view(torch.int16).numpy().view(np.uint16).reshape(-1))
        assert np.array_equal(fc._read(sh.specs["b"], 0, 777), b.numpy())
        assert fc._read(sh.specs["h"], 1, 4).tolist() == [1, 2, 3]


@pytest.mark.parametrize("grouped", [False, True])
def test_gathered_harness_rebuilds_each_chunks_records(grouped):
    """The per-chunk record of the referenced source rows (and the index
    remapping into it) reproduces the whole-site oracle: gathered_fwd on the
    full source record."""
    src_rows, cols = 80, 512
    xr, _, _ = _site(src_rows, cols, seed=7)
    rng = np.random.default_rng(8)
    idx = np.r_[rng.permutation(src_rows), rng.integers(0, src_rows, 30), [-1, src_rows, 5]].astype(np.int64)
    xt = F.f32_to_bf16_rne(rng.standard_normal(idx.size * cols).astype(np.float32))
    off = np.array([0, 0, 17, 17, 60, 80], dtype=np.int64) if grouped else None
    if grouped:
        ts = oracle.grouped_tensor_scale(xr, src_rows, cols, off)
        rec = oracle.grouped_capture(xr, src_rows, cols, off, ts, with_codes=True)
    else:
        ts = np.float32(oracle.tensor_scale(xr))
        rec = oracle.capture(xr, ts, with_codes=True)
    want = {}
    for mode, tag in (("guided", "g"), ("full", "f"), ("rne", "r")):
        r = oracle.gathered_fwd(mode, xt, cols, rec, src_rows, idx, ts, off)
        want.update({f"y_{tag}": r["y"], f"mask_{tag}": r["mask"], f"q_{tag}": r["codes"]})
    assert fc.compare_gathered_every_element("ok", xr, src_rows, xt, idx, cols, off, ts, want) == idx.size * cols
    bad = dict(want)
    bad["q_f"] = want["q_f"].copy()
    bad["q_f"][(idx.size - 2) * cols // 2] ^= 0x10     # the row whose index is out of range
    with pytest.raises(AssertionError, match="q_f"):
        fc.compare_gathered_every_element("planted", xr, src_rows, xt, idx, cols, off, ts, bad)
