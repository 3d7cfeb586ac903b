"""Oracle: FP8 E4M3 (OCP "e4m3fn") encoding and the dense attention with an
FP8 P.V product.

Test infrastructure only (see the package docstring).

Format (OCP 8-bit floating point, E4M3): sign bit, 4 exponent bits with bias
7, 3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the code
S.1111.111 is NaN and there is no infinity, so the largest finite value is
1.75 * 2^8 = 448. Encoding rounds to the nearest value, ties to the code
with an even mantissa; inputs here never exceed 448 by more than rounding.
"""
from __future__ import annotations

import numpy as np

from .attention import _int_dot, _scale
from .quant import widen

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_POS_CODES = np.arange(0x7F, dtype=np.uint8)            # 0 .. 448, increasing
_POS_VALUES = e4m3_decode(_POS_CODES)


def e4m3_encode(x) -> np.ndarray:
    """float values -> uint8 codes: nearest finite E4M3 value, ties to the
    even code (its mantissa's last bit), magnitudes above 448 to 448."""
    x = np.asarray(x, np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")           # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS_VALUES[lo]
    dhi = _POS_VALUES[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)     # the sign is kept, also of zero


def e4m3_round(x) -> np.ndarray:
    """The E4M3 value nearest to x (as float64)."""
    return e4m3_decode(e4m3_encode(x))


def v_fp8_per_channel(v_vals):
    """Per-(batch, KV head, channel) FP8 quantization of V over all its tokens
    ([SAGE-MACA]'s next versions quantize V per channel for an FP8 P.V):
    s_c = fl32(max_t |V[t, c]| / 448), codes = E4M3(fl32(V / s_c)) (0 where
    s_c = 0). v_vals: fp32 [B, N, H, d]. Returns (values fp64 of the codes,
    scales fp32 [B, H, d])."""
    v = np.asarray(v_vals, np.float32)
    amax = np.max(np.abs(v), axis=1) if v.shape[1] else np.zeros((v.shape[0],) + v.shape[2:], np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)                 # [B, H, d]
    live = s > 0
    r = (v / np.where(live, s, np.float32(1.0))[:, None]).astype(np.float32)
    vals = np.where(live[:, None], e4m3_round(r), 0.0)
    return vals, s


def dense_sage_attention_fp8pv(quant, v_bits, dtype="f16", causal=False, scale=None, smooth_v=False,
                               tile=64, slack=3.0, rows=None, heads=None, return_lse=False):
    """Dense attention with the P.V product in FP8 (the pages' next step for
    P.V: [SAGE-MACA] lists FP8 P.V of later SageAttention versions as not
    portable to its hardware; gfx950 has it natively).

    Scores as dense_sage_attention. Readings (the pages fix none of this):
    online softmax over tiles of `tile` keys in order with a reference m_t
    per row: m_t = m_{t-1} unless the tile's largest score exceeds it by more
    than `slack` in base-2 units (slack * ln 2 in scores), then m_t is the
    running maximum (slack 0: the exact running maximum); each probability of
    tile t is P8 = E4M3(448 * 2^-slack * exp(s - m_t)), so the largest
    possible is 448; V per channel in FP8 (v_fp8_per_channel, of V - mu_v
    with smooth_v); the row sum l and the output accumulate the rounded P8
    exactly, rescaled by exp(m_{t-1} - m_t) when the reference moves;
    out = (O / l) * s_V (+ mu_v with smooth_v, on rows that see a key).
    Products and sums in fp64. With return_lse: the natural log of
    l / (448 * 2^-slack) * exp(m) (the sum of the rounded probabilities).
    Returns fp64 [B, Nq, Hq, d] (and lse [B, Hq, Nq])."""
    q_i8, k_i8 = quant["q_i8"], quant["k_i8"]
    B, Nq, Hq, d = q_i8.shape
    Nk, Hkv = k_i8.shape[1], k_i8.shape[2]
    G = Hq // Hkv
    sc = _scale(scale, d)
    v = widen(v_bits, dtype)
    mu = None
    if smooth_v:
        mu = (v.astype(np.float64).sum(axis=1) / np.float64(max(Nk, 1))).astype(np.float32)
        v = (v - mu[:, None]).astype(np.float32)
    v8, sv = v_fp8_per_channel(v)
    out = np.zeros((B, Nq, Hq, d), np.float64)
    lse = np.full((B, Hq, Nq), -np.inf)
    qr = np.arange(Nq) if rows is None else np.asarray(rows)
    qblk = qr // 128
    kblk = np.arange(Nk) // 64
    vis = np.arange(Nk)[None, :] <= (qr[:, None] + (Nk - Nq)) if causal else np.ones((len(qr), Nk), bool)
    for b in range(B):
        for h in range(Hq):
            if heads is not None and h not in heads:
                continue
            kvh = h // G
            acc = _int_dot(q_i8[b, qr, h], k_i8[b, :, kvh])
            s = (acc * quant["q_scale"][b, h, qblk].astype(np.float64)[:, None]
                 * quant["k_scale"][b, kvh, kblk].astype(np.float64)[None, :] * sc)
            s = np.where(vis, s, -np.inf)
            m = np.full(len(qr), -np.inf)
            l = np.zeros(len(qr))
            o = np.zeros((len(qr), d))
            top = E4M3_MAX * 2.0 ** -slack
            for t0 in range(0, Nk, tile):
                st = s[:, t0:t0 + tile]
                mt = st.max(axis=1)
                move = mt > m + slack * np.log(2.0)
                m_new = np.where(move, np.maximum(m, mt), m)
                live = np.isfinite(m_new)
                alpha = np.where(np.isfinite(m), np.exp(m - np.where(live, m_new, 0.0)), 0.0)
                p8 = np.where(live[:, None], e4m3_round(top * np.exp(st - np.where(live, m_new, 0.0)[:, None])), 0.0)
                l = l * alpha + p8.sum(axis=1)
                o = o * alpha[:, None] + p8 @ v8[b, t0:t0 + tile, kvh]
                m = m_new
            ok = l > 0
            res = np.where(ok[:, None], o / np.where(ok, l, 1.0)[:, None], 0.0) * sv[b, kvh].astype(np.float64)
            if smooth_v:
                res = res + np.where(ok[:, None], mu[b, kvh].astype(np.float64), 0.0)
            out[b, qr, h] = res
            lse[b, h, qr] = np.where(ok, m + np.log(np.where(ok, l, 1.0) / top), -np.inf)
    return (out, lse) if return_lse else out
