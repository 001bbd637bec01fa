"""Pin the oracle's vectorized capture / guided / RNE / full-information /
STE code against an independent scalar twin written with exact rational
arithmetic (CPU only).

The twin follows the same definitions element by element but shares no code
with the oracle: every binary32 operation is an exact Fraction rounded by
``tests.exact.round_f32``, and every grid rounding is an exact comparison
against the enumerated grid.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import formats as F
from tests.exact import round_bf16, round_f32

GRID = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]
E4M3 = [Fraction(float(v)) for v in F.E4M3FN_VALUES[:0x7F]]


def _f(v):
    return Fraction(float(v))


def _is_nan(v):
    return v != v


def twin_tensor_scale(xs):
    m = max([abs(x) for x in xs if not _is_nan(x)], default=0.0)
    if np.isinf(m):
        return float("inf")
    return round_f32(_f(m) / 2688)


def twin_e4m3(v):
    if _is_nan(v):
        return 0
    v = min(_f(v), Fraction(448))
    d = [abs(v - e) for e in E4M3]
    best = min(d)
    cands = [i for i, di in enumerate(d) if di == best]
    return cands[0] if len(cands) == 1 or cands[0] % 2 == 0 else cands[1]


def twin_block_byte(block, ts):
    if not (np.isfinite(ts) and ts > 0):
        return 0
    m = max([abs(x) for x in block if not _is_nan(x)], default=0.0)
    v = round_f32(round_f32(_f(m) / 6) / _f(ts))
    return twin_e4m3(v)


def twin_scale(byte, ts):
    dec = F.E4M3FN_VALUES[byte]
    if _is_nan(dec):
        return float("nan")
    return round_f32(_f(dec) * _f(ts)) if np.isfinite(ts) else float("nan")


def twin_rne_idx(a):
    fa = _f(a)
    d = [abs(fa - g) for g in GRID]
    best = min(d)
    c = [i for i, di in enumerate(d) if di == best]
    return c[0] if len(c) == 1 or c[0] % 2 == 0 else c[1]


def twin_bracket(a):
    fa = _f(a)
    lo = max(i for i, g in enumerate(GRID) if g <= fa)
    hi = min(i for i, g in enumerate(GRID) if g >= fa)
    return lo, hi


def twin_element(x, s, rule, c=None, roll_code=None):
    """Return (code, mask, y_value) for one element; y_value is a float."""
    neg_x = np.signbit(x)
    valid = np.isfinite(s) and s > 0
    if _is_nan(x):
        return 0, 0, 0.0
    if not valid:
        return (8 if neg_x else 0), 0, (-0.0 if neg_x else 0.0)
    if np.isinf(x):
        zr = x
    else:
        zr = round_f32(_f(x) / _f(s))
    mask = 1 if abs(zr) <= 6 else 0
    neg = np.signbit(zr) if zr != 0 else neg_x
    a = min(abs(zr), 6.0)
    if rule == "rne":
        m = twin_rne_idx(a)
    else:
        lo, hi = twin_bracket(a)
        if lo == hi:
            m = lo
        elif rule == "guided":
            m = lo if (lo & 1) == c else hi
        else:  # full information
            rv = -GRID[roll_code & 7] if roll_code & 8 else GRID[roll_code & 7]
            sg = -1 if neg else 1
            m = lo if abs(sg * GRID[lo] - rv) < abs(sg * GRID[hi] - rv) else hi
    q = -float(GRID[m]) if neg else float(GRID[m])
    if q == 0:
        q = -0.0 if neg else 0.0
    prod = round_f32(_f(s) * _f(q)) if q != 0 else q
    y = round_bf16(_f(prod)) if not np.isinf(prod) else prod
    if y == 0:
        y = -0.0 if np.signbit(q) else 0.0
    return (8 if neg else 0) | m, mask, y


def _bf16(vals):
    return F.f32_to_bf16_rne(np.asarray(vals, np.float32))


def _tiny_tensor(rng):
    blocks = [
        rng.standard_normal(16),
        rng.standard_normal(16) * 50,
        rng.standard_t(4, 16),
        rng.laplace(size=16) * 1e-3,
        np.zeros(16),
        np.r_[np.zeros(15), -0.0],
        rng.standard_normal(16) * 2.0 ** -130,   # subnormal magnitudes
        rng.standard_normal(16) * 1e-30,
        np.r_[rng.standard_normal(14), np.nan, 3.0],
        np.r_[rng.standard_normal(15), -3e38],
        rng.uniform(-6, 6, 16),
        np.r_[rng.standard_normal(15), 2688.0],
    ]
    return _bf16(np.concatenate(blocks))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_capture_matches_exact_twin(seed):
    rng = np.random.default_rng(seed)
    xb = _tiny_tensor(rng)
    x = F.bf16_to_f32(xb)
    ts = oracle.tensor_scale(xb)
    assert float(ts) == twin_tensor_scale(list(x))
    cap = oracle.capture(xb, ts, with_codes=True)
    codes = oracle.unpack_nibbles(cap["codes"], x.size)
    bits = oracle.unpack_bits(cap["bits"], x.size)
    for b in range(x.size // 16):
        blk = list(x[16 * b:16 * b + 16])
        byte = twin_block_byte(blk, ts)
        assert cap["scales"][b] == byte, (b, blk)
        s = twin_scale(byte, ts)
        for k, xv in enumerate(blk):
            code, _, _ = twin_element(xv, s, "rne")
            assert codes[16 * b + k] == code, (b, k, xv, s)
            assert bits[16 * b + k] == (code & 1)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_training_side_matches_exact_twin(seed):
    rng = np.random.default_rng(100 + seed)
    xr = _tiny_tensor(rng)
    xr32 = F.bf16_to_f32(xr)
    xt32 = np.where(np.isfinite(xr32), xr32 * (1 + 0.05 * rng.standard_normal(xr32.size)), xr32)
    xt32[[5, 40, 77]] = [np.inf, -np.inf, 1e38]
    xt = _bf16(xt32)
    # also some random scale bytes, including zero and NaN bytes
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts, with_codes=True)
    scales = cap["scales"].copy()
    scales[2] = 0x7F
    scales[3] = 0x00
    scales[4] = 0x01
    n = xt.size
    g = oracle.guided_fwd(xt, scales, ts, cap["bits"])
    r = oracle.rne_fwd(xt, scales, ts)
    fi = oracle.full_info_fwd(xt, scales, ts, cap["codes"])
    c_bits = oracle.unpack_bits(cap["bits"], n)
    rcodes = oracle.unpack_nibbles(cap["codes"], n)
    xt32 = F.bf16_to_f32(xt)
    for name, out, rule in (("guided", g, "guided"), ("rne", r, "rne"), ("full", fi, "full")):
        codes = oracle.unpack_nibbles(out["codes"], n)
        mask = oracle.unpack_bits(out["mask"], n)
        y = F.bf16_to_f32(out["y"])
        for i in range(n):
            s = twin_scale(scales[i // 16], ts)
            code, m, yv = twin_element(xt32[i], s, rule, c=int(c_bits[i]), roll_code=int(rcodes[i]))
            assert codes[i] == code, (name, i, xt32[i], s)
            assert mask[i] == m, (name, i)
            assert (y[i] == yv and np.signbit(y[i]) == np.signbit(yv)) or (np.isinf(yv) and y[i] == yv), (name, i, y[i], yv)


def test_capture_with_infinite_tensor_scale_is_all_zero_scale():
    x = _bf16(np.r_[np.arange(31, dtype=np.float32) - 15.0, -np.inf])
    ts = oracle.tensor_scale(x)
    assert np.isinf(ts)
    cap = oracle.capture(x, ts, with_codes=True)
    assert np.all(cap["scales"] == 0) and np.all(cap["bits"] == 0)
    codes = oracle.unpack_nibbles(cap["codes"], x.size)
    assert np.array_equal(codes, np.where(np.signbit(F.bf16_to_f32(x)), 8, 0))


def test_ste_bwd_against_mask_definition():
    rng = np.random.default_rng(7)
    n = 4096
    g = rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16)
    m = rng.integers(0, 2, size=n).astype(np.uint8)
    out = oracle.ste_bwd(g, np.packbits(m, bitorder="little"), n)
    for i in range(n):
        assert out[i] == (g[i] if m[i] else 0)


def test_gather_records_against_row_loop():
    """Pinned against a plain per-row, per-byte loop over the definition."""
    rng = np.random.default_rng(12)
    src_rows, cols, dst_rows = 9, 64, 13
    rec = {"bits": rng.integers(0, 256, src_rows * cols // 8, dtype=np.uint8),
           "scales": rng.integers(0, 127, src_rows * cols // 16, dtype=np.uint8),
           "codes": rng.integers(0, 256, src_rows * cols // 2, dtype=np.uint8)}
    idx = rng.integers(-3, src_rows + 3, dst_rows)
    out = oracle.gather_records(rec, idx, src_rows, cols)
    for name, per in (("bits", cols // 8), ("scales", cols // 16), ("codes", cols // 2)):
        for r in range(dst_rows):
            for k in range(per):
                want = rec[name][idx[r] * per + k] if 0 <= idx[r] < src_rows else 0
                assert out[name][r * per + k] == want
    # a gathered record drives the trainer exactly like the rows it came from
    xr = F.f32_to_bf16_rne(rng.standard_normal(src_rows * cols).astype(np.float32))
    ts = oracle.tensor_scale(xr)
    cap = oracle.capture(xr, ts)
    perm = rng.permutation(src_rows)
    g = oracle.gather_records({"bits": cap["bits"], "scales": cap["scales"]}, perm, src_rows, cols)
    xt = xr.reshape(src_rows, cols)[perm].reshape(-1)
    a = oracle.guided_fwd(xt, g["scales"], ts, g["bits"])
    b = oracle.guided_fwd(xr, cap["scales"], ts, cap["bits"])
    assert np.array_equal(a["y"], b["y"].reshape(src_rows, cols)[perm].reshape(-1))


def test_grouped_path_matches_exact_twin():
    """Per-expert tensor scales: every group of rows (one empty) gets its own
    amax and tensor scale; capture and all three forwards of each row use its
    group's scale.  Checked element by element against the exact twin."""
    rng = np.random.default_rng(21)
    rows, cols = 7, 32
    offsets = [0, 2, 2, 5, 7]
    mags = [1.0, 40.0, 1e-3, 7.0]  # a different range per group
    vals = np.zeros((rows, cols))
    for g, (a, b) in enumerate(zip(offsets, offsets[1:])):
        vals[a:b] = rng.standard_t(4, (b - a, cols)) * mags[g]
    vals[3, 5] = np.nan
    xr = _bf16(vals.reshape(-1))
    xt = _bf16(F.bf16_to_f32(xr) * (1 + 0.05 * rng.standard_normal(xr.size)))
    ts = oracle.grouped_tensor_scale(xr, rows, cols, offsets)
    cap = oracle.grouped_capture(xr, rows, cols, offsets, ts, with_codes=True)
    gd = oracle.grouped_guided_fwd(xt, rows, cols, offsets, cap["scales"], ts, cap["bits"])
    rn = oracle.grouped_rne_fwd(xt, rows, cols, offsets, cap["scales"], ts)
    fi = oracle.grouped_full_info_fwd(xt, rows, cols, offsets, cap["scales"], ts, cap["codes"])

    fr, ft = F.bf16_to_f32(xr), F.bf16_to_f32(xt)
    roll = oracle.unpack_nibbles(cap["codes"], xr.size)
    bits = oracle.unpack_bits(cap["bits"], xr.size)
    for g, (a, b) in enumerate(zip(offsets, offsets[1:])):
        want_ts = twin_tensor_scale(list(fr[a * cols:b * cols])) if b > a else 0.0
        assert np.float32(ts[g]) == np.float32(want_ts), (g, ts[g], want_ts)
        for r in range(a, b):
            for blk in range(cols // 16):
                i0 = r * cols + blk * 16
                byte = twin_block_byte(list(fr[i0:i0 + 16]), np.float32(want_ts))
                assert cap["scales"][i0 // 16] == byte, (r, blk)
                s = twin_scale(byte, np.float32(want_ts))
                for i in range(i0, i0 + 16):
                    code, _, _ = twin_element(fr[i], s, "rne")
                    assert roll[i] == code and bits[i] == (code & 1), i
                    for out, rule, kw in ((gd, "guided", {"c": int(bits[i])}), (rn, "rne", {}),
                                          (fi, "full", {"roll_code": int(roll[i])})):
                        c2, m2, y2 = twin_element(ft[i], s, rule, **kw)
                        assert oracle.unpack_nibbles(out["codes"], xr.size)[i] == c2, (rule, i)
                        assert oracle.unpack_bits(out["mask"], xr.size)[i] == m2, (rule, i)
                        assert out["y"][i] == _bf16([y2])[0], (rule, i)


def test_grouped_offsets_are_validated():
    x = np.zeros(64, np.uint16)
    for bad in ([0, 3, 2, 4], [1, 4], [0, 3], [0]):
        with pytest.raises(ValueError):
            oracle.grouped_tensor_scale(x, 4, 16, bad)
