"""Whole-tensor checks of the NVFP4 path's outputs at any size, with plain
torch operations on the device (no oracle, no libtrace code).  They hold for
every element by the definitions of the rule, so they cover the full
workload sizes where the oracle runs on sampled rows only:

* y = bf16_RNE(fl32(s * q)) for the codes q each forward reports, with
  s = fl32(E4M3FN(scale byte) * ts) (the decode step; torch's float8 decode,
  float32 multiply and bfloat16 cast are exact / IEEE round to nearest even),
  ts being the tensor scale or, with per-expert scales, the row's group's;
* the clip mask does not depend on the rounding rule (guided, RNE and full
  information report the same mask), and the STE backward passes exactly the
  masked gradient (+0 elsewhere);
* capture's cached bit is the parity of its code;
* guided vs RNE: both have z's sign; where RNE's code already has the cached
  parity the guided code equals it; where they differ, the guided code has
  the cached parity and is one grid step from RNE's (the other endpoint of
  the bracket);
* full information: one step at most from RNE, z's sign, and the rollout's
  own code wherever that code is RNE's or the guided one (both are bracket
  endpoints);
* where x_train == x_roll bit for bit, RNE, guided and full information all
  return the rollout's code.
"""
import torch

E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _nibbles(packed, lo, hi):
    """Codes of elements [lo, hi) (even element = low nibble), as uint8."""
    p = packed[lo // 2: hi // 2]
    return torch.stack((p & 15, p >> 4), dim=-1).reshape(-1)


def _bits(packed, lo, hi):
    p = packed[lo // 8: hi // 8]
    sh = torch.arange(8, dtype=torch.uint8, device=p.device)
    return ((p.unsqueeze(-1) >> sh) & 1).reshape(-1)


def _signed(c):
    m = (c & 7).to(torch.int16)
    return torch.where((c & 8) != 0, -m, m)


def _bf16_bits(t):
    return t.contiguous().view(torch.int16)


def check_nvfp4_outputs(ctx, x_roll, x_train, grad, ts, out, chunk=1 << 26):
    """``out``: device tensors scales, bits, codes, y_g, mask_g, q_g, y_r,
    mask_r, q_r, y_f, mask_f, q_f, gin (the latter three groups from the
    guided, RNE and full-information forwards; gin = STE backward of the
    guided mask).  ``ts``: the tensor scale (one element), or one per row
    (per-expert scales: the scale of each row's group).  Raises
    AssertionError naming the first failing property."""
    n = x_roll.numel()
    cols = x_roll.shape[-1]
    dev = x_roll.device
    per_row = ts.numel() > 1
    table = torch.tensor(E2M1, dtype=torch.float32, device=dev)
    xr = x_roll.reshape(-1).view(torch.int16)
    xt = x_train.reshape(-1).view(torch.int16)
    g = grad.reshape(-1).view(torch.int16)
    ts32 = ts.reshape(-1).float()
    for lo in range(0, n, chunk):
        hi = min(n, lo + chunk)
        sb = out["scales"][lo // 16: hi // 16]
        if per_row:
            blk = torch.arange(lo // 16, hi // 16, device=dev)
            tsb = ts32[(blk * 16) // cols]
        else:
            tsb = ts32
        s = sb.view(torch.float8_e4m3fn).float() * tsb                   # fl32(E4M3FN(sb) * ts)
        valid = (sb < 0x7F) & (s > 0) & torch.isfinite(s)
        s_el = torch.where(valid, s, torch.ones_like(s)).repeat_interleave(16)
        codes = {k: _nibbles(out[f"q_{k}"], lo, hi) for k in ("g", "r", "f")}
        for k, c in codes.items():
            q = table[(c & 7).long()]
            q = torch.where((c & 8) != 0, -q, q)
            want = (s_el * q).to(torch.bfloat16)
            got = out[f"y_{k}"].reshape(-1)[lo:hi]
            bad = _bf16_bits(want) != _bf16_bits(got)
            assert not bool(bad.any()), f"{ctx}: y_{k} != bf16(s * q) at {int(bad.nonzero()[0]) + lo}"
        mg, mr, mf = (out[f"mask_{k}"][lo // 8: hi // 8] for k in ("g", "r", "f"))
        assert torch.equal(mg, mr) and torch.equal(mg, mf), f"{ctx}: masks differ between rules"
        m = _bits(out["mask_g"], lo, hi).bool()
        want_gin = torch.where(m, g[lo:hi], torch.zeros_like(g[lo:hi]))
        assert torch.equal(out["gin"].reshape(-1).view(torch.int16)[lo:hi], want_gin), f"{ctx}: STE backward"
        cap = _nibbles(out["codes"], lo, hi)
        c_bit = _bits(out["bits"], lo, hi)
        assert torch.equal(c_bit, cap & 1), f"{ctx}: cached bit != parity of the capture code"
        cg, cr, cf = codes["g"], codes["r"], codes["f"]
        assert torch.equal(cg & 8, cr & 8) and torch.equal(cf & 8, cr & 8), f"{ctx}: sign differs between rules"
        sg, sr, sf = _signed(cg), _signed(cr), _signed(cf)
        same_par = (cr & 1) == c_bit
        assert bool((cg[same_par] == cr[same_par]).all()), f"{ctx}: guided left an RNE code of the cached parity"
        moved = cg != cr
        assert bool(((cg[moved] & 1) == c_bit[moved]).all()), f"{ctx}: guided code without the cached parity"
        assert bool(((sg[moved] - sr[moved]).abs() == 1).all()), f"{ctx}: guided code not adjacent to RNE's"
        assert bool(((sf - sr).abs() <= 1).all()), f"{ctx}: full-information code not adjacent to RNE's"
        hit = (cap == cr) | (cap == cg)
        assert bool((cf[hit] == cap[hit]).all()), f"{ctx}: full information missed an endpoint rollout code"
        same_x = xt[lo:hi] == xr[lo:hi]
        for k, c in codes.items():
            assert bool((c[same_x] == cap[same_x]).all()), f"{ctx}: {k} differs from the rollout on x_train == x_roll"
