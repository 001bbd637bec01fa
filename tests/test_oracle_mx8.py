"""Pins of the FP8 activation-grid oracle (``oracle.mx8``, MXFP8 E4M3), CPU only.

* the E4M3 magnitude table against torch's ``float8_e4m3fn`` decode;
* round-to-nearest-even onto E4M3 against torch's float32 -> float8_e4m3fn
  cast for every bf16 value up to 448 and for random float32 values
  (subnormal ones and those one ulp around every midpoint included), and
  against the textbook binary rounding of ``tests.exact``;
* the bracket against brute force over exact rationals;
* block scale bytes against closed forms of the OCP MX definition with
  E4M3's largest-normal exponent 8, and the property that a block maximum
  lands in [256, 512) after scaling wherever the clamp is not reached;
* capture and the three forwards element by element against an exact
  rational twin that takes its grid from torch's decode;
* the rule's guarantees swept over every bf16 z up to 448 under a unit
  scale, with rollout codewords up to three steps from z's RNE codeword:
  identical inputs give the rollout code, straddling rollout codes are
  recovered, full information is never farther from the rollout than RNE,
  and the 1-bit rule's violations are exactly the set the parity argument
  allows;
* a constructed example worked by hand on the E4M3 grid.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests.exact import round_bf16, round_f32, round_to_binary

TORCH_E4M3 = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
GRID = [Fraction(float(v)) for v in TORCH_E4M3]


def _bf16(v):
    return F.f32_to_bf16_rne(np.asarray(v, np.float32))


def _torch_e4m3_code(a):
    """torch's float32 -> float8_e4m3fn cast (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_magnitudes_match_torch_decode():
    assert np.array_equal(oracle.E4M3_MAGNITUDES, TORCH_E4M3)
    assert np.all(np.diff(oracle.E4M3_MAGNITUDES) > 0)
    assert oracle.E4M3_MAGNITUDES[0x7E] == 448 and oracle.E4M3_MAGNITUDES[1] == 2.0 ** -9
    assert oracle.E4M3_MAGNITUDES[0x08] == 2.0 ** -6


def test_rne_every_bf16_up_to_448_matches_torch_cast():
    b = np.arange(0x8000, dtype=np.uint16)
    v = F.bf16_to_f32(b)
    a = v[np.isfinite(v) & (v <= 448)]
    assert np.array_equal(oracle.e4m3_rne_code(a), _torch_e4m3_code(a).astype(np.int64))


def test_rne_random_f32_and_midpoints_match_torch_cast():
    rng = np.random.default_rng(3)
    u = rng.integers(0, 0x43E00001, size=1 << 20, dtype=np.uint32)          # [0, 448] incl. subnormals
    a = u.view(np.float32)
    mids = ((oracle.E4M3_MAGNITUDES[:-1] + oracle.E4M3_MAGNITUDES[1:]) / 2).astype(np.float32)
    mb = mids.view(np.uint32)
    near = np.concatenate([mb - 1, mb, mb + 1]).view(np.float32)
    a = np.concatenate([a, near, oracle.E4M3_MAGNITUDES.astype(np.float32)])
    assert np.array_equal(oracle.e4m3_rne_code(a), _torch_e4m3_code(a).astype(np.int64))


def test_rne_matches_textbook_binary_rounding():
    rng = np.random.default_rng(4)
    a = np.concatenate([rng.uniform(0, 448, 3000), 2.0 ** rng.uniform(-14, 8.8, 3000)]).astype(np.float32)
    a = np.minimum(a, np.float32(448))
    got = oracle.E4M3_MAGNITUDES[oracle.e4m3_rne_code(a)]
    for ai, gi in zip(a, got):
        assert Fraction(float(gi)) == round_to_binary(Fraction(float(ai)), 3, -6, 8), ai


def test_bracket_brute_force():
    rng = np.random.default_rng(5)
    a = np.concatenate([rng.uniform(0, 448, 1500), 2.0 ** rng.uniform(-16, 8.8, 1500),
                        oracle.E4M3_MAGNITUDES[::5], [0.0, 448.0]]).astype(np.float32)
    a = np.minimum(a, np.float32(448))
    lo, hi = oracle.e4m3_bracket(a)
    for ai, l, h in zip(a, lo, hi):
        fa = Fraction(float(ai))
        assert l == max(i for i, g in enumerate(GRID) if g <= fa)
        assert h == min(i for i, g in enumerate(GRID) if g >= fa)


def _block(values):
    v = np.zeros(32, np.float32)
    v[: len(values)] = values
    return _bf16(v)


@pytest.mark.parametrize("amax,byte", [
    (448.0, 127),          # 448 = 1.75 * 2^8: scale 1, the plain E4M3 grid
    (256.0, 127),
    (255.0, 126),          # floor(log2 255) = 7 -> scale 1/2
    (480.0, 127),          # still scale 1; 480 saturates to 448
    (512.0, 128),
    (1.0, 119),            # 2^(0 - 8)
    (0.0, 0),              # all-zero block: smallest scale
    (2.0 ** -130, 0),      # clamps at the bottom of E8M0
    (2.0 ** 127, 246),     # 127 - 8 + 127
    (float("inf"), 247),   # reading: infinity counts as exponent 128
])
def test_block_scale_closed_forms(amax, byte):
    assert oracle.mx8_block_scales(_block([amax, -amax / 3, amax / 7]))[0] == byte


def test_scaled_block_maximum_lands_in_the_top_binade():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((4000, 32)) * 2.0 ** rng.uniform(-100, 100, (4000, 1))
    xb = _bf16(v.reshape(-1))
    sb = oracle.mx8_block_scales(xb).astype(np.int64)
    amax = np.abs(F.bf16_to_f32(xb)).reshape(-1, 32).max(axis=1).astype(np.float64)
    scaled = amax / np.ldexp(1.0, sb - 127)
    assert np.all((scaled >= 256) & (scaled < 512))


# ---------------------------------------------------------------------------
# exact twin (grid from torch's decode, Fractions, textbook fp32 / bf16 rounding)
# ---------------------------------------------------------------------------

def _twin_byte(block):
    vals = [abs(Fraction(float(v))) for v in block if v == v and np.isfinite(v)]
    if any(np.isinf(v) for v in block):
        return 247
    a = max(vals, default=Fraction(0))
    if a == 0:
        return 0
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    return 127 + min(max(e - 8, -127), 127)


def _twin_nearest(fa):
    d = [abs(fa - g) for g in GRID]
    best = min(d)
    c = [i for i, di in enumerate(d) if di == best]
    return c[0] if len(c) == 1 or c[0] % 2 == 0 else c[1]


def _twin_element(x, byte, rule, c=0, roll=0):
    """(code byte, mask, y) for one element under E8M0 byte ``byte``."""
    if x != x:
        return 0, 0, 0.0
    if byte == 0xFF:
        neg = np.signbit(x)
        return (0x80 if neg else 0), 0, (-0.0 if neg else 0.0)
    s = Fraction(2) ** (int(byte) - 127)
    zr = x if np.isinf(x) else round_f32(Fraction(float(x)) / s)
    neg = np.signbit(zr) if zr != 0 else np.signbit(x)
    mask = 1 if abs(zr) <= 448 else 0
    fa = min(abs(Fraction(zr)) if not np.isinf(zr) else Fraction(448), Fraction(448))
    lo = max(i for i, g in enumerate(GRID) if g <= fa)
    hi = min(i for i, g in enumerate(GRID) if g >= fa)
    if rule == "rne":
        m = _twin_nearest(fa)
    elif lo == hi:
        m = lo
    elif rule == "guided":
        m = lo if (lo & 1) == c else hi
    else:
        rmag = Fraction(480) if (roll & 0x7F) == 0x7F else GRID[roll & 0x7F]
        rv = -rmag if roll & 0x80 else rmag
        sg = -1 if neg else 1
        m = lo if abs(sg * GRID[lo] - rv) < abs(sg * GRID[hi] - rv) else hi
    q = -GRID[m] if neg else GRID[m]
    prod = round_f32(s * q)
    y = prod if np.isinf(prod) else round_bf16(Fraction(prod))
    if y == 0:
        y = -0.0 if neg else 0.0
    return (0x80 if neg else 0) | m, mask, y


def _tiny_tensor(rng):
    blocks = [
        rng.standard_normal(32),
        rng.standard_normal(32) * 300,
        rng.standard_t(4, 32) * 1e-3,
        rng.laplace(size=32) * 2.0 ** -120,   # scales near the bottom of E8M0
        np.zeros(32),
        np.r_[np.zeros(31), -0.0],
        np.r_[rng.standard_normal(30), np.nan, 3.0],
        np.r_[rng.standard_normal(31), -3e38],
        np.r_[rng.standard_normal(31) * 1e-6, 1.0],  # tiny elements beside a large one
        rng.uniform(-448, 448, 32),
        np.r_[rng.standard_normal(31), np.inf],
    ]
    return _bf16(np.concatenate(blocks))


@pytest.mark.parametrize("seed", [0, 1])
def test_capture_matches_exact_twin(seed):
    xb = _tiny_tensor(np.random.default_rng(seed))
    x = F.bf16_to_f32(xb)
    cap = oracle.mx8_capture(xb, with_codes=True)
    bits = oracle.unpack_bits(cap["bits"], x.size)
    for b in range(x.size // 32):
        blk = x[32 * b:32 * b + 32]
        assert cap["scales"][b] == _twin_byte(blk), b
        for k in range(32):
            code, _, _ = _twin_element(blk[k], cap["scales"][b], "rne")
            assert cap["codes"][32 * b + k] == code, (b, k, blk[k])
            assert bits[32 * b + k] == code & 1


@pytest.mark.parametrize("seed", [0, 1])
def test_forwards_match_exact_twin(seed):
    rng = np.random.default_rng(50 + seed)
    xr = _tiny_tensor(rng)
    xr32 = F.bf16_to_f32(xr)
    xt32 = np.where(np.isfinite(xr32), xr32 * (1 + 0.05 * rng.standard_normal(xr32.size)), xr32)
    xt = _bf16(xt32)
    cap = oracle.mx8_capture(xr, with_codes=True)
    scales = cap["scales"].copy()
    scales[[2, 3, 4]] = [0xFF, 0x00, 0xFE]     # zero-scale, smallest and largest scales
    roll = cap["codes"].copy()
    roll[[7, 8, 70]] = [0x7F, 0xFF, 0x80]
    n = xt.size
    c = oracle.unpack_bits(cap["bits"], n)
    outs = {"guided": oracle.mx8_guided_fwd(xt, scales, cap["bits"]), "rne": oracle.mx8_rne_fwd(xt, scales),
            "full": oracle.mx8_full_info_fwd(xt, scales, roll)}
    xt32 = F.bf16_to_f32(xt)
    for rule, out in outs.items():
        mask = oracle.unpack_bits(out["mask"], n)
        y = F.bf16_to_f32(out["y"])
        for i in range(n):
            code, m, yv = _twin_element(xt32[i], scales[i // 32], rule, c=int(c[i]), roll=int(roll[i]))
            assert out["codes"][i] == code, (rule, i, xt32[i])
            assert mask[i] == m, (rule, i)
            assert y[i] == yv and np.signbit(y[i]) == np.signbit(yv), (rule, i, y[i], yv)


# ---------------------------------------------------------------------------
# the rule's guarantees, swept over every bf16 z up to 448 (unit scale)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def sweep():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(b)
    x = b[np.isfinite(v) & (np.abs(v) <= 448)]
    x = np.concatenate([x, np.zeros((-x.size) % 32, np.uint16)])
    n = x.size
    scales = np.full(n // 32, 127, np.uint8)                 # s = 1: z = x
    z = F.bf16_to_f32(x).astype(np.float64)
    sg = np.where(np.signbit(z), -1, 1)
    lo, hi = oracle.e4m3_bracket(np.abs(z))
    rne_out = oracle.mx8_rne_fwd(x, scales)
    rne_mag = rne_out["codes"].astype(np.int64) & 0x7F
    # signed bracket: [lo, hi] for z >= 0, [-hi, -lo] below zero
    L, H = np.where(sg < 0, -hi, lo), np.where(sg < 0, -lo, hi)
    return {"x": x, "n": n, "scales": scales, "sg": sg, "L": L, "H": H, "rne": sg * rne_mag,
            "rne_codes": rne_out["codes"]}


def _signed(codes):
    c = codes.astype(np.int64)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def _val(si):
    return np.where(si < 0, -1.0, 1.0) * oracle.E4M3_MAGNITUDES[np.abs(si)]


def _code_of(si):
    return (np.where(si < 0, 0x80, 0) | np.abs(si)).astype(np.uint8)


def test_identical_inputs_give_the_rollout_code(sweep):
    cap = oracle.mx8_capture(sweep["x"], with_codes=True)
    assert np.array_equal(cap["scales"], oracle.mx8_block_scales(sweep["x"]))
    g = oracle.mx8_guided_fwd(sweep["x"], cap["scales"], cap["bits"])
    r = oracle.mx8_rne_fwd(sweep["x"], cap["scales"])
    assert np.array_equal(g["codes"], cap["codes"]) and np.array_equal(r["codes"], cap["codes"])
    assert np.array_equal(g["y"], r["y"])


@pytest.mark.parametrize("step", [-3, -2, -1, 1, 2, 3])
def test_guarantees_against_nearby_rollout_codes(sweep, step):
    x, scales, n = sweep["x"], sweep["scales"], sweep["n"]
    L, H, rne = sweep["L"], sweep["H"], sweep["rne"]
    r = np.clip(rne + step, -126, 126)
    roll = _code_of(r)
    bits = oracle.pack_bits((np.abs(r) & 1).astype(np.uint8))
    g = _signed(oracle.mx8_guided_fwd(x, scales, bits)["codes"])
    f = _signed(oracle.mx8_full_info_fwd(x, scales, roll)["codes"])
    vr = _val(r)
    d_rne = np.abs(_val(rne) - vr)
    # full information: never farther from the rollout value than RNE; the
    # rollout codeword itself whenever it is an endpoint of z's bracket
    assert np.all(np.abs(_val(f) - vr) <= d_rne)
    ends = (r == L) | (r == H)
    assert np.array_equal(f[ends], r[ends])
    # guided: an endpoint of the bracket with the cached parity (z itself on a codeword)
    strict = L != H
    assert np.all((g == L) | (g == H))
    assert np.all((np.abs(g[strict]) & 1) == (np.abs(r[strict]) & 1))
    # straddling rollout codes are recovered
    assert np.array_equal(g[ends & strict], r[ends & strict])
    # violations of |q* - r| <= |q_RNE - r| are exactly the parity set: r
    # outside the bracket, an odd number of steps beyond q_RNE on its side
    viol = np.abs(_val(g) - vr) > d_rne
    odd = ((np.abs(r) - np.abs(rne)) & 1) == 1
    beyond = ((rne == H) & (r > H)) | ((rne == L) & (r < L))
    in_v = strict & ~ends & odd & beyond
    assert np.array_equal(viol, in_v)
    assert n == x.size


def test_mismatch_counts_on_a_straddle():
    """Constructed example on the E4M3 grid, worked by hand.  A block whose
    maximum is 448 gets byte 127 (s = 1).  x_roll = 17 is the midpoint of the
    codewords 16 (0x58) and 18 (0x59): the tie goes to the even code 0x58,
    cached bit 0.  x_train = 17.125 rounds to 18 under RNE, but the guided
    rule keeps the bracket [16, 18]'s even endpoint, 16, the rollout's."""
    xr = _block([448.0, 17.0])
    xt = _block([448.0, 17.125])
    cap = oracle.mx8_capture(xr, with_codes=True)
    assert cap["scales"][0] == 127 and cap["codes"][1] == 0x58 and cap["codes"][0] == 0x7E
    assert oracle.unpack_bits(cap["bits"], 32)[1] == 0
    r = oracle.mx8_rne_fwd(xt, cap["scales"])
    g = oracle.mx8_guided_fwd(xt, cap["scales"], cap["bits"])
    assert r["codes"][1] == 0x59 and F.bf16_to_f32(r["y"])[1] == 18.0
    assert g["codes"][1] == 0x58 and F.bf16_to_f32(g["y"])[1] == 16.0
    st = oracle.mx8_mismatch_counts(xt, cap["scales"], cap["codes"], cap["bits"])
    assert st == {"n": 32, "mismatched": 1, "straddle": 1, "recovered": 1}


def test_mask_boundary_and_specials():
    """|x / s| <= 448 keeps the gradient: 448 does, the next bf16 value 450
    does not (and rounds to 448); NaN gives +0 with mask 0; infinities clip
    to +-448 with mask 0; a zero-scale byte gives signed zeros, mask 0."""
    xb = _block([448.0, 450.0, -450.0, np.nan, np.inf, -np.inf, -0.0, 2.0 ** -10, 2.0 ** -10 * 3])
    scales = np.array([127], np.uint8)
    out = oracle.mx8_rne_fwd(xb, scales)
    mask = oracle.unpack_bits(out["mask"], 32)
    assert list(mask[:9]) == [1, 0, 0, 0, 0, 0, 1, 1, 1]
    assert list(out["codes"][:9]) == [0x7E, 0x7E, 0xFE, 0x00, 0x7E, 0xFE, 0x80, 0x00, 0x02]
    zs = oracle.mx8_guided_fwd(xb, np.array([0xFF], np.uint8), np.zeros(4, np.uint8))
    assert not zs["mask"].any()
    assert list(zs["codes"][:7]) == [0, 0, 0x80, 0, 0, 0x80, 0x80]
