"""Oracle: rotary position embedding ahead of quantization (the fused
producer of [QK-MMAC] §4: rotary embedding, query quantization and the
KV-cache write in one pass).

Test infrastructure only (see the package docstring).

The pages name the fusion but give no rotary parameters. Readings taken:

* The table is an input, [max_position, rot_dim] fp32, cos(p w_i) in
  columns [0, rot_dim/2) and sin(p w_i) in [rot_dim/2, rot_dim).
* Channel pairs: "neox" rotates (i, i + rot_dim/2), otherwise adjacent pairs
  (2i, 2i + 1); pair i uses frequency i. Channels from rot_dim on pass
  through unchanged (partial rotary).
* Arithmetic in fp32 from the exactly widened 16-bit inputs, one rounding
  per operation and no fused multiply-add:
      a' = fl32(fl32(a cos) - fl32(b sin)),  b' = fl32(fl32(b cos) + fl32(a sin)).
* The rotated fp32 values are quantized directly (no rounding back to the
  16-bit type: that round trip is what the fusion removes). V is not rotated.
"""
from __future__ import annotations

import numpy as np

from .quant import quant_rows, widen, write_kv_values


def _pairs(rot_dim: int, neox: bool):
    half = rot_dim // 2
    if neox:
        return np.arange(half), np.arange(half, rot_dim)
    return np.arange(0, rot_dim, 2), np.arange(1, rot_dim, 2)


def apply_rope(x_bits, dtype, positions, cos_sin, rot_dim, neox=True):
    """Rotate [T, H, d] 16-bit inputs by the table rows of their tokens'
    positions; returns fp32 [T, H, d]."""
    x = widen(x_bits, dtype)
    half = rot_dim // 2
    cs = np.asarray(cos_sin, np.float32)[np.asarray(positions, np.int64)]   # [T, rot_dim]
    c, s = cs[:, None, :half], cs[:, None, half:rot_dim]
    ia, ib = _pairs(rot_dim, neox)
    a, b = x[..., ia], x[..., ib]
    out = x.copy()
    out[..., ia] = (a * c).astype(np.float32) - (b * s).astype(np.float32)
    out[..., ib] = (b * c).astype(np.float32) + (a * s).astype(np.float32)
    return out.astype(np.float32)


def rope_quantize_q(q_bits, dtype, positions, cos_sin, rot_dim, neox=True):
    """Per-(token, head) INT8 of the rotated query (the rule of quant_rows).
    Returns (q_i8 [T, Hq, d], q_scale [T, Hq])."""
    return quant_rows(apply_rope(q_bits, dtype, positions, cos_sin, rot_dim, neox))


def rope_write_kv_cache(k_bits, v_bits, dtype, slot_mapping, num_blocks, positions, cos_sin, rot_dim,
                        neox=True, v_int8=False, caches=None):
    """write_kv_cache with K rotated first (V as given)."""
    k_rot = apply_rope(k_bits, dtype, positions, cos_sin, rot_dim, neox)
    return write_kv_values(k_rot, v_bits, dtype, slot_mapping, num_blocks, v_int8=v_int8, caches=caches)
