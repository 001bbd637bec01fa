"""CPU oracle for TRACE's rollout-guided rounding path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, table or constant generator with
the HIP library in ``fp4_rollout_guided_amd``.

What it computes is taken from the rcap.io post "TRACE: Rollout-Guided
Quantization-Aware Training for FP4" (2026-10-06):

* the rollout side records, per quantization site, the FP4 codeword the
  rollout produced, compacted to one mantissa bit plus the scale metadata
  (the bandwidth paragraph and the pseudo-code listing);
* the training side recomputes ``z = clip(x_train / s, -6, 6)`` with the
  cached rollout scale, brackets z between two adjacent FP4 codewords and
  keeps the one the cached bit points at, with a straight-through estimator
  around ``s * q*`` (the rollout-guided rounding paragraph and the listing);
* the same path on MXFP4 scales (``oracle.mx``) and on the FP8 activation
  grid of the W4A8 setting (``oracle.mx8``), both from the Ablations bullet.

The pages name NVFP4 and the E2M1 grid but not the format's parameters; the
oracle uses the NVFP4 definition: 16-element blocks along the last dimension,
an OCP E4M3FN block scale, and an FP32 tensor scale ``amax / (6 * 448)``.

Every floating-point step is IEEE binary32 with round-to-nearest-even
(NumPy float32 arithmetic, no fused multiply-add, subnormals kept); every
rounding onto a small grid (bf16, E4M3, E2M1) is a nearest-value search over
the enumerated grid with an explicit tie rule.  Readings the pages leave open
are stated where they are used.

Pins (``tests/test_oracle_*.py``) tie each function to something other than
itself: exact rational arithmetic, PyTorch's CPU casts, exhaustive sweeps,
closed forms, the page's worked example and invariants of the rule.
"""

from .formats import (
    E2M1_MAGNITUDES,
    E4M3FN_MAX,
    bf16_to_f32,
    e2m1_bracket,
    e2m1_rne_index,
    e4m3fn_decode,
    e4m3fn_encode_rne_sat,
    f32_to_bf16_rne,
)
from .mx import (
    MX_BLOCK,
    e8m0_decode,
    floor_log2,
    mx_block_scales,
    mx_capture,
    mx_full_info_fwd,
    mx_guided_fwd,
    mx_rne_fwd,
)
from .mx8 import (
    E4M3_MAGNITUDES,
    e4m3_bracket,
    e4m3_rne_code,
    e4m3_signed_values,
    mx8_block_scales,
    mx8_capture,
    mx8_full_info_fwd,
    mx8_guided_fwd,
    mx8_mismatch_counts,
    mx8_rne_fwd,
)
from .trace import (
    BLOCK,
    TENSOR_SCALE_DIVISOR,
    block_scales,
    capture,
    capture_lowbits,
    compact_cache_bytes,
    decode_scales,
    full_info_fwd,
    gather_records,
    gathered_fwd,
    grouped_capture,
    grouped_full_info_fwd,
    grouped_guided_fwd,
    grouped_rne_fwd,
    grouped_tensor_scale,
    guided_fwd,
    lowbits_fwd,
    lowbits_reconstruct,
    mismatch_stats,
    pack_bits,
    pack_nibbles,
    rne_fwd,
    signed_index,
    ste_bwd,
    tensor_scale,
    unpack_bits,
    unpack_nibbles,
)

__all__ = [
    "E2M1_MAGNITUDES", "E4M3FN_MAX", "bf16_to_f32", "e2m1_bracket",
    "e2m1_rne_index", "e4m3fn_decode", "e4m3fn_encode_rne_sat",
    "f32_to_bf16_rne", "BLOCK", "TENSOR_SCALE_DIVISOR", "block_scales",
    "capture", "compact_cache_bytes", "decode_scales", "full_info_fwd", "gather_records", "gathered_fwd",
    "grouped_capture", "grouped_full_info_fwd", "grouped_guided_fwd", "grouped_rne_fwd",
    "grouped_tensor_scale", "MX_BLOCK", "e8m0_decode", "floor_log2", "mx_block_scales", "mx_capture",
    "mx_full_info_fwd", "mx_guided_fwd", "mx_rne_fwd", "capture_lowbits", "lowbits_fwd", "lowbits_reconstruct",
    "signed_index", "E4M3_MAGNITUDES", "e4m3_bracket", "e4m3_rne_code", "e4m3_signed_values",
    "mx8_block_scales", "mx8_capture", "mx8_full_info_fwd", "mx8_guided_fwd", "mx8_mismatch_counts",
    "mx8_rne_fwd",
    "guided_fwd", "mismatch_stats", "pack_bits", "pack_nibbles", "rne_fwd",
    "ste_bwd", "tensor_scale", "unpack_bits", "unpack_nibbles",
]
