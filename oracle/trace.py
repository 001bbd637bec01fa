"""Oracle for capture, guided fake-quant, RNE fake-quant and STE backward.

Test infrastructure only (see ``oracle/__init__.py``).  All sources cited
are the rcap.io post "TRACE: Rollout-Guided Quantization-Aware Training for
FP4" unless stated otherwise.

Tensors are flat arrays of bf16 bit patterns (``uint16``) whose length is a
multiple of 16; a block is 16 consecutive elements.  Record layouts:

* scale bytes: one E4M3FN byte per block, in block order;
* bit-plane / mask: bit k of byte j belongs to element 8*j + k;
* 4-bit codes: element 2*j in the low nibble of byte j, 2*j+1 in the high
  nibble; a code is sign << 3 | magnitude index.

Readings of points the pages leave open:

* the single low bit kept per site is bit 0 of the E2M1 code, which is
  the parity of the codeword's signed grid index: adjacent codewords,
  including the pair around zero, always differ in it;
* ``reconstruct_from_mantissa(c, z)`` is the endpoint of z's bracket whose
  parity is c, so the listing's argmin picks it; when z is itself a
  codeword the bracket is that single codeword;
* the block scale is ``E4M3FN_RNE_sat(fl32(fl32(amax_b / 6) / ts))`` and
  the decoded scale is ``s = fl32(dec(byte) * ts)``;
* a block whose decoded scale is not a positive finite number is a
  zero-scale block: every element quantizes to a zero with the input's
  sign and its clip mask is 0;
* NaN inputs quantize to +0 with mask 0; the tensor and block maxima
  ignore NaN;
* the clip mask is ``|x / s| <= 6`` on the unclipped quotient (inclusive);
* the training output is ``bf16_RNE(fl32(s * q*))``.
"""

import numpy as np

from .formats import (
    E2M1_MAGNITUDES,
    bf16_to_f32,
    e2m1_bracket,
    e2m1_rne_index,
    e4m3fn_decode,
    e4m3fn_encode_rne_sat,
    f32_to_bf16_rne,
)

BLOCK = 16
# Largest E2M1 magnitude times largest E4M3FN value: the NVFP4 tensor scale
# maps the tensor's amax onto the top of the two-level range.
TENSOR_SCALE_DIVISOR = 6 * 448
_F32 = np.float32


# --------------------------------------------------------------------------
# bit and nibble packing (record layout)
# --------------------------------------------------------------------------

def pack_bits(flags) -> np.ndarray:
    """bool/0-1 per element -> bytes, bit k of byte j = element 8j+k."""
    return np.packbits(np.asarray(flags, dtype=np.uint8).reshape(-1), bitorder="little")


def unpack_bits(packed, n: int) -> np.ndarray:
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), bitorder="little")[:n]


def pack_nibbles(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return (c[0::2] & 0xF) | ((c[1::2] & 0xF) << 4)


def unpack_nibbles(packed, n: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(2 * p.size, dtype=np.uint8)
    out[0::2] = p & 0xF
    out[1::2] = p >> 4
    return out[:n]


# --------------------------------------------------------------------------
# scales (NVFP4 two-level scaling; "scale metadata" in the bandwidth
# paragraph, scale_roll in the listing)
# --------------------------------------------------------------------------

def _abs_max_ignoring_nan(f32_rows: np.ndarray) -> np.ndarray:
    a = np.abs(f32_rows)
    a = np.where(np.isnan(a), _F32(0), a)
    return a.max(axis=-1)


def tensor_scale(x_bits) -> np.float32:
    """FP32 tensor scale ``fl32(amax / 2688)``, amax = max |x| over the whole
    site tensor, NaN ignored (0 for an empty or all-NaN tensor)."""
    x = bf16_to_f32(np.asarray(x_bits).reshape(-1))
    if x.size == 0:
        return _F32(0)
    amax = _abs_max_ignoring_nan(x)
    with np.errstate(over="ignore"):
        return _F32(amax) / _F32(TENSOR_SCALE_DIVISOR)


def _block_view(x_bits) -> np.ndarray:
    x = np.asarray(x_bits, dtype=np.uint16).reshape(-1)
    if x.size % BLOCK:
        raise ValueError("tensor length must be a multiple of 16")
    return x.reshape(-1, BLOCK)


def block_scales(x_bits, ts) -> np.ndarray:
    """One E4M3FN scale byte per 16-element block:
    ``E4M3FN_RNE_sat(fl32(fl32(amax_b / 6) / ts))``; 0 when ts is zero or
    not finite."""
    xb = _block_view(x_bits)
    amax_b = _abs_max_ignoring_nan(bf16_to_f32(xb))
    ts = _F32(ts)
    if not (np.isfinite(ts) and ts > 0):
        return np.zeros(xb.shape[0], dtype=np.uint8)
    with np.errstate(over="ignore", under="ignore"):
        v = (amax_b / _F32(6)) / ts
    return e4m3fn_encode_rne_sat(v)


def decode_scales(scale_bytes, ts):
    """Decoded block scales ``s = fl32(dec(byte) * ts)`` and the mask of
    blocks whose s is a positive finite number (all others are zero-scale
    blocks).  ts is one tensor scale, or one per block."""
    dec = e4m3fn_decode(scale_bytes).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", under="ignore"):
        s = dec * _F32(ts)
        valid = np.isfinite(s) & (s > 0)
    return s, valid


def _quotients(x_bits, scale_bytes, ts):
    """Per element: x as float32, the unclipped quotient ``fl32(x / s)``
    (meaningful in valid blocks only), the per-element decoded scale, and
    the valid-block mask broadcast to elements."""
    xb = _block_view(x_bits)
    x = bf16_to_f32(xb)
    s, valid = decode_scales(np.asarray(scale_bytes, dtype=np.uint8), ts)
    if s.shape[0] != xb.shape[0]:
        raise ValueError("one scale byte per 16-element block is required")
    s_safe = np.where(valid, s, _F32(1))[:, None]
    with np.errstate(over="ignore", under="ignore", invalid="ignore", divide="ignore"):
        zr = x / s_safe
    return x.reshape(-1), zr.reshape(-1), np.repeat(s, BLOCK), np.repeat(valid, BLOCK)


def _sign_and_clipped(x, zr, valid):
    """Sign bit of z and |z| clipped to [0, 6]; NaN -> +0, zero-scale block
    -> zero with the input's sign."""
    nan = np.isnan(x)
    z = np.where(valid, zr, np.copysign(_F32(0), x))
    z = np.where(nan, _F32(0), z)
    sign = np.signbit(z)
    a = np.minimum(np.abs(z), _F32(6))
    return sign, a


# --------------------------------------------------------------------------
# rollout side: capture (fp4_quantize + low_bits(q_roll, b=1) in the listing)
# --------------------------------------------------------------------------

def capture(x_bits, ts, with_codes: bool = False) -> dict:
    """Quantize a rollout site tensor to NVFP4 and keep the compact record.

    Per block: the scale byte.  Per element: ``z = fl32(x / s)``, the E2M1
    index of ``min(|z|, 6)`` by round-to-nearest-even, code
    ``sign(z) << 3 | idx``, and the cached bit ``idx & 1``.
    Returns ``scales`` (u8[n/16]), ``bits`` (u8[n/8]) and, on request, the
    full 4-bit ``codes`` (u8[n/2]).
    """
    scales = block_scales(x_bits, ts)
    x, zr, _, valid = _quotients(x_bits, scales, ts)
    return {"scales": scales, **capture_record(x, zr, valid, with_codes)}


def capture_record(x, zr, valid, with_codes: bool) -> dict:
    """The per-element half of the capture, given the quotients ``zr`` and
    the per-element valid-scale flags: parity bit-plane and optional codes."""
    sign, a = _sign_and_clipped(x, zr, valid)
    idx = np.where(valid & ~np.isnan(x), e2m1_rne_index(a), 0).astype(np.uint8)
    out = {"bits": pack_bits(idx & 1)}
    if with_codes:
        out["codes"] = pack_nibbles((sign.astype(np.uint8) << 3) | idx)
    return out


# --------------------------------------------------------------------------
# training side (the QAT half of the listing)
# --------------------------------------------------------------------------

def _finish(x, zr, s, valid, sign, m_idx, m_val):
    """Common tail: clip mask, q* = copysign(m, z), y = bf16(fl32(s * q*))."""
    nan = np.isnan(x)
    with np.errstate(invalid="ignore"):
        mask = valid & ~nan & (np.abs(zr) <= _F32(6))
    q = np.where(sign, -m_val, m_val).astype(np.float32)
    q = np.where(valid & ~nan, q, np.where(sign, _F32(-0.0), _F32(0.0)))
    with np.errstate(over="ignore", invalid="ignore"):
        prod = np.where(valid & ~nan, s * q, q).astype(np.float32)
    codes = (sign.astype(np.uint8) << 3) | np.where(valid & ~nan, m_idx, 0).astype(np.uint8)
    return {
        "y": f32_to_bf16_rne(prod),
        "mask": pack_bits(mask),
        "codes": pack_nibbles(codes),
    }


def guided_fwd(x_bits, scale_bytes, ts, bits) -> dict:
    """Rollout-guided fake-quant forward.

    ``z = clip(fl32(x_train / s), -6, 6)`` with the cached rollout scale;
    ``lo, hi`` = the E2M1 magnitudes around |z|; if they coincide the result
    is |z| itself, otherwise the endpoint whose index parity equals the
    cached bit c.  ``q* = copysign(m, z)``; ``y = bf16(fl32(s * q*))``;
    ``mask = |x_train / s| <= 6``.  Returns ``y`` (u16[n]), ``mask``
    (u8[n/8]) and the codes of q* (u8[n/2]).
    """
    x, zr, s, valid = _quotients(x_bits, scale_bytes, ts)
    return guided_rule(x, zr, s, valid, unpack_bits(bits, x.size))


def guided_rule(x, zr, s, valid, c) -> dict:
    """The guided rule on given quotients (per-element x, zr, s, valid) and
    cached bits c (one 0/1 per element)."""
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e2m1_bracket(a)
    pick_lo = (lo & 1) == c
    m_idx = np.where(lo == hi, lo, np.where(pick_lo, lo, hi))
    m_val = E2M1_MAGNITUDES[m_idx].astype(np.float32)
    # lo == hi means |z| is the grid value itself, so m_val == a there.
    return _finish(x, zr, s, valid, sign, m_idx, m_val)


def rne_fwd(x_bits, scale_bytes, ts) -> dict:
    """Plain round-to-nearest-even fake-quant forward (the usual rounding,
    the vanilla-QAT baseline the post compares against): as ``guided_fwd`` but
    ``m`` = the E2M1 value nearest to |z|, ties to the even index."""
    x, zr, s, valid = _quotients(x_bits, scale_bytes, ts)
    return rne_rule(x, zr, s, valid)


def rne_rule(x, zr, s, valid) -> dict:
    """Round-to-nearest-even on given quotients."""
    sign, a = _sign_and_clipped(x, zr, valid)
    m_idx = e2m1_rne_index(a)
    m_val = E2M1_MAGNITUDES[m_idx].astype(np.float32)
    return _finish(x, zr, s, valid, sign, m_idx, m_val)


def _signed_values(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where(c & 8, -mag, mag)


def full_info_fwd(x_bits, scale_bytes, ts, roll_codes) -> dict:
    """Full-information guidance (the ablation reference that caches the
    whole 4-bit rollout code): the endpoint of z's bracket nearest to the
    rollout's signed codeword; |z| itself when z is a codeword."""
    x, zr, s, valid = _quotients(x_bits, scale_bytes, ts)
    return full_info_rule(x, zr, s, valid, unpack_nibbles(roll_codes, x.size))


def full_info_rule(x, zr, s, valid, roll) -> dict:
    """Full-information guidance on given quotients and rollout codes (one
    code per element)."""
    q_roll = _signed_values(roll)
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e2m1_bracket(a)
    sgn = np.where(sign, -1.0, 1.0)
    d_lo = np.abs(sgn * E2M1_MAGNITUDES[lo] - q_roll)
    d_hi = np.abs(sgn * E2M1_MAGNITUDES[hi] - q_roll)
    m_idx = np.where((lo == hi) | (d_lo < d_hi), lo, hi)
    m_val = E2M1_MAGNITUDES[m_idx].astype(np.float32)
    return _finish(x, zr, s, valid, sign, m_idx, m_val)


def ste_bwd(grad_bits, mask_bytes, n: int) -> np.ndarray:
    """Straight-through estimator backward: the incoming gradient where the
    clip mask is set, +0.0 (bf16 0x0000) elsewhere."""
    g = np.asarray(grad_bits, dtype=np.uint16).reshape(-1)[:n]
    m = unpack_bits(mask_bytes, n).astype(bool)
    return np.where(m, g, np.uint16(0)).astype(np.uint16)


# --------------------------------------------------------------------------
# b > 1 cached low bits (low_bits(q_roll, b) in the listing, which the post
# runs with b = 1).  Reading: the b low bits of the codeword's signed grid
# index in two's complement (for b = 1 the E2M1 mantissa bit); stored as b
# bit-planes of the b = 1 layout, plane k holding bit k.  The training side
# reconstructs the rollout codeword as the signed index with that residue
# modulo 2^b nearest to the middle of z's bracket (within the grid's 15
# signed indices), then takes the bracket endpoint nearest to it.  For b = 1
# this is the guided rule, for b = 4 the full-information rule.  A residue
# no index has (8 for b = 4, which no capture writes) takes the endpoint
# nearer zero.
# --------------------------------------------------------------------------

SIGNED_INDEX_MAX = 7


def signed_index(codes) -> np.ndarray:
    """Signed grid index of each E2M1 code (sign << 3 | index): -7 .. 7, with
    both zeros at 0."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = (c & 7).astype(np.int64)
    return np.where(c & 8, -mag, mag)


def capture_lowbits(x_bits, ts, b: int) -> dict:
    """Capture keeping b low bits per element: ``scales`` as ``capture`` and
    ``planes`` (u8[b * n/8]): plane k is bit k of each element's signed grid
    index modulo 2^b, in the bit-plane layout."""
    if not 1 <= b <= 4:
        raise ValueError("b must be 1..4")
    cap = capture(x_bits, ts, with_codes=True)
    n = np.asarray(x_bits).size
    r = np.mod(signed_index(unpack_nibbles(cap["codes"], n)), 1 << b)
    planes = np.concatenate([pack_bits((r >> k) & 1) for k in range(b)])
    return {"scales": cap["scales"], "planes": planes}


def lowbits_reconstruct(r, lo_signed, b: int) -> np.ndarray:
    """Signed index with residue r (mod 2^b) nearest to lo_signed + 1/2, among
    -7 .. 7 (candidates are 2^b apart, so there are no ties); 99 where no
    index has residue r (r = 8 for b = 4)."""
    m = 1 << b
    best = np.full(np.shape(r), 99, dtype=np.int64)
    for cand in range(-SIGNED_INDEX_MAX, SIGNED_INDEX_MAX + 1):
        ok = np.mod(cand, m) == r
        closer = ok & (np.abs(2 * cand - (2 * lo_signed + 1)) < np.abs(2 * best - (2 * lo_signed + 1)))
        best = np.where(closer, cand, best)
    return best


def lowbits_fwd(x_bits, scale_bytes, ts, planes, b: int) -> dict:
    """Guided fake-quant forward from b cached low bits: z's bracket
    (q-, q+) in signed indices (a, a + 1); the reconstructed rollout index t
    (``lowbits_reconstruct``); q* = q+ if t >= a + 1 else q-; z itself when it
    is a codeword.  Outputs as ``guided_fwd``."""
    x, zr, s, valid = _quotients(x_bits, scale_bytes, ts)
    n = x.size
    pl = np.asarray(planes, dtype=np.uint8).reshape(b, -1)
    r = np.zeros(n, dtype=np.int64)
    for k in range(b):
        r |= unpack_bits(pl[k], n).astype(np.int64) << k
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e2m1_bracket(a)
    # signed bracket: z >= 0: (lo, hi); z < 0: (-hi, -lo)
    lo_signed = np.where(sign, -hi.astype(np.int64), lo.astype(np.int64))
    t = lowbits_reconstruct(r, lo_signed, b)
    upper = t >= lo_signed + 1
    # magnitude of the chosen endpoint: the signed upper endpoint is hi for z >= 0, lo for z < 0;
    # a residue no grid index has (8 when b = 4; no capture produces it) takes the endpoint nearer zero
    none = t == 99
    m_idx = np.where((lo == hi) | none, lo, np.where(upper != sign, hi, lo)).astype(np.uint8)
    m_val = E2M1_MAGNITUDES[m_idx].astype(np.float32)
    return _finish(x, zr, s, valid, sign, m_idx, m_val)


# --------------------------------------------------------------------------
# trainer-side readback (the post's remark that the training engine must
# read the rollout records back): records in the trainer's row order
# --------------------------------------------------------------------------

def gather_records(record, row_index, src_rows: int, cols: int) -> dict:
    """Row gather of a compact record: destination row r is source row
    ``row_index[r]`` of every plane (bits: cols/8 bytes per row, scales:
    cols/16, codes: cols/2).  An index outside [0, src_rows) gives an
    all-zero row, i.e. zero-scale blocks."""
    per_row = {"bits": cols // 8, "scales": cols // BLOCK, "codes": cols // 2}
    idx = np.asarray(row_index, dtype=np.int64).reshape(-1)
    ok = (idx >= 0) & (idx < src_rows)
    out = {}
    for name, plane in record.items():
        if plane is None:
            continue
        src = np.asarray(plane, dtype=np.uint8).reshape(src_rows, per_row[name])
        dst = np.zeros((idx.size, per_row[name]), dtype=np.uint8)
        dst[ok] = src[idx[ok]]
        out[name] = dst.reshape(-1)
    return out


def gathered_fwd(mode, x_bits, cols: int, record, src_rows: int, row_index, ts, offsets=None) -> dict:
    """The training side's forward on records read back in its own row order
    (the trainer reads the rollout's records back): destination row r takes
    its record from source row ``row_index[r]`` (``gather_records``: an index
    outside [0, src_rows) gives an all-zero row, i.e. zero-scale blocks) and
    the tensor scale of that source row -- ``ts[0]`` for one tensor scale, or,
    with ``offsets`` describing groups of source rows (per-expert scales),
    ``ts[g]`` of the group holding it.  mode "guided" reads the record's
    bits, "full" its codes, "rne" only its scale bytes (the vanilla-QAT
    baseline on the same records).  Outputs as ``guided_fwd``."""
    rec = gather_records(record, row_index, src_rows, cols)
    idx = np.asarray(row_index, dtype=np.int64).reshape(-1)
    tsv = np.asarray(ts, dtype=np.float32).reshape(-1)
    row_ts = np.full(idx.size, tsv[0], dtype=np.float32)   # rows outside every group keep ts[0]: zero-scale anyway
    if offsets is not None:
        for g, (a, b) in enumerate(_group_slices(offsets, src_rows)):
            row_ts[(idx >= a) & (idx < b)] = tsv[g]
    block_ts = np.repeat(row_ts, cols // BLOCK)             # one tensor scale per block of the destination
    if mode == "guided":
        return guided_fwd(x_bits, rec["scales"], block_ts, rec["bits"])
    if mode == "full":
        return full_info_fwd(x_bits, rec["scales"], block_ts, rec["codes"])
    if mode == "rne":
        return rne_fwd(x_bits, rec["scales"], block_ts)
    raise ValueError("mode must be 'guided', 'full' or 'rne'")


# --------------------------------------------------------------------------
# per-expert tensor scales for packed MoE rows: the routed-expert sites hold
# the rows of every expert back to back, and each expert's rows form their
# own tensor (its own amax and tensor scale)
# --------------------------------------------------------------------------

def _group_slices(offsets, rows: int):
    """Row ranges of the groups: group g is rows [offsets[g], offsets[g+1]).
    The offsets must start at 0, end at ``rows`` and never decrease."""
    off = [int(v) for v in np.asarray(offsets, dtype=np.int64).reshape(-1)]
    if len(off) < 2 or off[0] != 0 or off[-1] != rows or any(b < a for a, b in zip(off, off[1:])):
        raise ValueError("group offsets must run from 0 to rows without decreasing")
    return [(off[g], off[g + 1]) for g in range(len(off) - 1)]


def grouped_tensor_scale(x_bits, rows: int, cols: int, offsets) -> np.ndarray:
    """One tensor scale per group of rows (fp32[groups]): the tensor scale
    of the group's rows taken as a tensor of their own (0 for an empty
    group)."""
    x = np.asarray(x_bits, dtype=np.uint16).reshape(rows, cols)
    return np.array([tensor_scale(x[a:b]) for a, b in _group_slices(offsets, rows)], dtype=np.float32)


def _per_group(fn, rows, cols, offsets, ts, planes):
    """Apply ``fn(group's planes..., ts[g])`` to each group's rows and join
    the results in row order.  ``planes`` maps a name to (array, bytes per
    row)."""
    parts = []
    ts = np.asarray(ts, dtype=np.float32).reshape(-1)
    for g, (a, b) in enumerate(_group_slices(offsets, rows)):
        args = [np.asarray(arr).reshape(rows, per_row)[a:b].reshape(-1) for arr, per_row in planes]
        parts.append(fn(*args, ts[g]))
    keys = [k for k in parts[0] if parts[0][k] is not None] if parts else []
    return {k: np.concatenate([p[k] for p in parts]) for k in keys}


def grouped_capture(x_bits, rows: int, cols: int, offsets, ts, with_codes: bool = False) -> dict:
    """``capture`` of each group's rows with that group's tensor scale."""
    return _per_group(lambda x, t: capture(x, t, with_codes), rows, cols, offsets, ts, [(x_bits, cols)])


def grouped_guided_fwd(x_bits, rows: int, cols: int, offsets, scale_bytes, ts, bits) -> dict:
    """``guided_fwd`` of each group's rows with that group's tensor scale."""
    return _per_group(lambda x, sb, c, t: guided_fwd(x, sb, t, c), rows, cols, offsets, ts,
                      [(x_bits, cols), (scale_bytes, cols // BLOCK), (bits, cols // 8)])


def grouped_rne_fwd(x_bits, rows: int, cols: int, offsets, scale_bytes, ts) -> dict:
    """``rne_fwd`` of each group's rows with that group's tensor scale."""
    return _per_group(rne_fwd, rows, cols, offsets, ts, [(x_bits, cols), (scale_bytes, cols // BLOCK)])


def grouped_full_info_fwd(x_bits, rows: int, cols: int, offsets, scale_bytes, ts, roll_codes) -> dict:
    """``full_info_fwd`` of each group's rows with that group's tensor scale."""
    return _per_group(lambda x, sb, rc, t: full_info_fwd(x, sb, t, rc), rows, cols, offsets, ts,
                      [(x_bits, cols), (scale_bytes, cols // BLOCK), (roll_codes, cols // 2)])


# --------------------------------------------------------------------------
# diagnostics and accounting
# --------------------------------------------------------------------------

def _signed_index(codes) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    mag = (c & 7).astype(np.int16)
    return np.where(c & 8, -mag, mag)


def mismatch_stats(x_train_bits, scale_bytes, ts, roll_codes, bits) -> dict:
    """Rollout/training agreement statistics on one site tensor.

    * ``hist[k]``: sites whose rollout code and the training-side RNE code
      are k signed grid steps apart (the bandwidth paragraph's ">99% of
      mismatched sites differ by one adjacent codeword");
    * ``straddle``: mismatched sites whose rollout codeword is an endpoint
      of the training value's bracket (the 0.48 -> 24 example);
    * ``crossed``: one-step mismatches that are not straddles;
    * ``recovered``: mismatched sites where guided rounding returns the
      rollout codeword;
    * ``violations``: sites where the guided value is farther from the
      rollout value than the RNE value (the local guarantee).
    """
    n = np.asarray(x_train_bits).size
    roll = unpack_nibbles(roll_codes, n)
    rne = unpack_nibbles(rne_fwd(x_train_bits, scale_bytes, ts)["codes"], n)
    gd = unpack_nibbles(guided_fwd(x_train_bits, scale_bytes, ts, bits)["codes"], n)
    si_roll, si_rne, si_gd = _signed_index(roll), _signed_index(rne), _signed_index(gd)
    steps = np.abs(si_roll - si_rne)
    mism = steps > 0
    x, zr, _, valid = _quotients(x_train_bits, scale_bytes, ts)
    sign, a = _sign_and_clipped(x, zr, valid)
    lo, hi = e2m1_bracket(a)
    sg = np.where(sign, -1, 1)
    lo_s, hi_s = sg * lo.astype(np.int16), sg * hi.astype(np.int16)
    straddle = mism & ((si_roll == lo_s) | (si_roll == hi_s))
    v_roll, v_rne, v_gd = _signed_values(roll), _signed_values(rne), _signed_values(gd)
    violations = np.abs(v_gd - v_roll) > np.abs(v_rne - v_roll)
    return {
        "n": int(n),
        "hist": np.bincount(steps, minlength=15).tolist(),
        "mismatched": int(mism.sum()),
        "straddle": int(straddle.sum()),
        "crossed": int((mism & (steps == 1) & ~straddle).sum()),
        "recovered": int((mism & (si_gd == si_roll)).sum()),
        "violations": int(violations.sum()),
        "violation_mask": violations,
        "straddle_mask": straddle,
        "steps": steps,
    }


def compact_cache_bytes(n_per_layer: int, captured_layers: int, total_layers: int) -> dict:
    """Bytes of the compact record (1 bit + one scale byte per 16 elements +
    a 4-byte tensor scale per captured site) against full NVFP4 codes
    (4 bits + the same scale metadata) for every layer, as in the bandwidth
    paragraph ("one mantissa bit plus scale metadata, and only for the
    deeper half of the layers")."""
    if n_per_layer % BLOCK:
        raise ValueError("site size must be a multiple of 16")
    compact = n_per_layer // 8 + n_per_layer // BLOCK
    full = n_per_layer // 2 + n_per_layer // BLOCK
    return {
        "compact_bytes": captured_layers * compact,
        "full_nvfp4_bytes": total_layers * full,
        "compact_with_ts": captured_layers * (compact + 4),
        "full_with_ts": total_layers * (full + 4),
        "ratio_per_layer": full / compact,
        "ratio": (total_layers * full) / (captured_layers * compact),
        "bits_per_elem_compact": 8.0 * compact / n_per_layer,
        "bits_per_elem_full": 8.0 * full / n_per_layer,
    }
