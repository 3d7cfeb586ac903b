"""Oracle: symmetric INT8 quantization and the paged cache layout.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np

BLOCK = 16  # tokens per cache block


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """16-bit storage pattern -> float32, exactly.

    bf16 is the top half of an IEEE binary32, so shifting the pattern left by
    16 bits gives the same value. fp16 widens exactly through numpy's half type.
    """
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float32)
    raise ValueError(f"unknown 16-bit dtype {dtype!r}")


def quant_rows(x: np.ndarray):
    """Symmetric dynamic INT8 quantization of each row (last axis) of x.

    [QK-MMAC] §1 writes Q ~= Qq * sQ and K ~= Kq * sK; §4 gives the row rule
    as scale = max|x| / 127 and Qq = round(x / scale); §2.1 fixes the code
    range to [-127, 127]. [SAGE-MACA] "quantization kernels" table names the
    rounding as round-to-nearest-even. Arithmetic, step by step, in fp32:

      amax = max_i |x_i|                 (exact)
      s    = fl32(amax / 127)            (one IEEE division)
      q_i  = clamp(rne(fl32(x_i / s)), -127, 127)

    A row with amax == 0 gets s = 0 and all-zero codes (the pages leave this
    case open; this is the reading that keeps scores finite).

    Returns (codes int8 with x's shape, scales float32 with x.shape[:-1]).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    live = s > 0
    denom = np.where(live, s, np.float32(1.0))[..., None]
    r = (x / denom).astype(np.float32)
    q = np.clip(np.rint(r), -127, 127)
    q = np.where(live[..., None], q, 0).astype(np.int8)
    return q, s


def quantize_q(q_bits: np.ndarray, dtype: str = "bf16"):
    """Per-(token, query head) quantization of Q [T, Hq, d] over head_dim.

    [QK-MMAC] §1: the query scale depends on the query token and query head;
    §4: Q is quantized once, before attention, and reused by every split.
    Returns (q_i8 [T, Hq, d], q_scale [T, Hq]).
    """
    return quant_rows(widen(q_bits, dtype))


def write_kv_cache(k_bits, v_bits, dtype, slot_mapping, num_blocks, v_int8=False,
                   caches=None):
    """Quantize K (and V if v_int8) per (token, KV head) and scatter into pages.

    Layouts ([QK-MMAC] §3 fixes K's; the scale and V layouts are this
    library's choice, since the pages do not give them):

      k_cache [NB, Hkv, d/16, 16, 16] int8  : k_cache[b][h][c][o][j] = Kq[t][h][16c + j]
      k_scale [NB, Hkv, 16]          fp32  : k_scale[b][h][o] = sK[t][h]
      v_cache [NB, Hkv, d, 16]  bf16 bits or int8 : v_cache[b][h][i][o] = V[t][h][i]
      v_scale [NB, Hkv, 16]          fp32  (INT8 V only)

    with b = slot // 16 and o = slot % 16. Tokens whose slot is negative are
    skipped. Slots must be distinct. ``caches`` (a dict returned by an earlier
    call) is updated in place; otherwise zero-filled caches are created.
    """
    return write_kv_values(widen(np.asarray(k_bits, np.uint16), dtype), v_bits, dtype, slot_mapping, num_blocks,
                           v_int8=v_int8, caches=caches)


def write_kv_values(k_vals, v_bits, dtype, slot_mapping, num_blocks, v_int8=False, caches=None):
    """write_kv_cache from fp32 K values (the 16-bit inputs widened, or
    values computed from them, such as rotated keys)."""
    k_vals = np.asarray(k_vals, np.float32)
    T, H, d = k_vals.shape
    assert d % 16 == 0
    if caches is None:
        caches = {
            "k_cache": np.zeros((num_blocks, H, d // 16, BLOCK, 16), np.int8),
            "k_scale": np.zeros((num_blocks, H, BLOCK), np.float32),
            "v_cache": np.zeros((num_blocks, H, d, BLOCK), np.int8 if v_int8 else np.uint16),
            "v_scale": np.zeros((num_blocks, H, BLOCK), np.float32) if v_int8 else None,
        }
    slots = np.asarray(slot_mapping, np.int64)
    keep = slots >= 0
    blk, off = slots[keep] // BLOCK, slots[keep] % BLOCK
    kq, ks = quant_rows(k_vals[keep])                               # [T', H, d], [T', H]
    caches["k_cache"][blk, :, :, off, :] = kq.reshape(-1, H, d // 16, 16)
    caches["k_scale"][blk, :, off] = ks
    v_sel = np.asarray(v_bits, np.uint16)[keep]
    if v_int8:
        vq, vs = quant_rows(widen(v_sel, dtype))
        caches["v_cache"][blk, :, :, off] = vq
        caches["v_scale"][blk, :, off] = vs
    else:
        caches["v_cache"][blk, :, :, off] = v_sel
    return caches


def gather_kv(caches, table_row, ctx, kv_head, v_dtype="bf16"):
    """Read one sequence's first ``ctx`` tokens of one KV head back through
    its block table ([QK-MMAC] §3: logical token -> block table -> physical
    block -> slot in the page -> head_dim chunk).

    Returns (Kq [ctx, d] int8, sK [ctx] fp32, V [ctx, d] fp64 dequantized).
    """
    k_cache = caches["k_cache"]
    d = k_cache.shape[2] * 16
    nblk = -(-ctx // BLOCK)
    blocks = np.asarray(table_row[:nblk], np.int64)
    kb = k_cache[blocks, kv_head]                                  # [nblk, d/16, 16 tok, 16]
    kq = kb.transpose(0, 2, 1, 3).reshape(nblk * BLOCK, d)[:ctx]  # token-major
    sk = caches["k_scale"][blocks, kv_head].reshape(-1)[:ctx]
    vb = caches["v_cache"][blocks, kv_head]                        # [nblk, d, 16 tok]
    vt = vb.transpose(0, 2, 1).reshape(nblk * BLOCK, d)[:ctx]
    if caches.get("v_scale") is not None:
        sv = caches["v_scale"][blocks, kv_head].reshape(-1)[:ctx]
        v = vt.astype(np.float64) * sv.astype(np.float64)[:, None]
    else:
        v = widen(vt, v_dtype).astype(np.float64)
    return kq, sk, v


def sage_quantize(q_bits, k_bits, dtype="f16", smooth_k=True, q_block=128, k_block=64):
    """SageAttention-style preprocessing of dense NHD Q [B, Nq, Hq, d] and
    K [B, Nk, Hkv, d].

    [SAGE-MACA] (feature matrix, "smooth_k"; advanced options): smoothing
    subtracts the mean of K over tokens, per channel, before quantization.
    [SAGE-MACA] ("quantization kernels" table; "per_block" granularity):
    one scale per block of 128 query rows or 64 key rows, computed over all
    rows x head_dim values of the block; the last block of a head takes the
    remaining rows.

    Mean precision is not on the pages. Reading taken: the per-(b, h, c) sum
    over all Nk tokens is accumulated in fp64 (exact for fp16 inputs and
    Nk <= 8192 in any order), divided by Nk in fp64 and rounded to fp32:
      mu = fl32(S / Nk);  K' = fl32(K - mu).

    Returns dict: q_i8 [B,Nq,Hq,d], q_scale [B,Hq,ceil(Nq/qb)],
    k_i8 [B,Nk,Hkv,d], k_scale [B,Hkv,ceil(Nk/kb)], k_mean [B,Hkv,d] fp32.
    """
    q = widen(q_bits, dtype)
    k = widen(k_bits, dtype)
    B, Nk, Hkv, d = k.shape
    if smooth_k and Nk > 0:
        total = k.astype(np.float64).sum(axis=1)                  # [B, Hkv, d]
        mu = (total / np.float64(Nk)).astype(np.float32)
    else:
        mu = np.zeros((B, Hkv, d), np.float32)
    ks = (k - mu[:, None, :, :]).astype(np.float32)

    def per_block(x, blk):
        b_, n, h, dd = x.shape
        nb = -(-n // blk)
        codes = np.zeros(x.shape, np.int8)
        scales = np.zeros((b_, h, nb), np.float32)
        for j in range(nb):
            rows = x[:, j * blk:min((j + 1) * blk, n)]              # [B, r, H, d]
            flat = rows.transpose(0, 2, 1, 3).reshape(b_, h, -1)    # one row per (b, h) block
            c, s = quant_rows(flat)
            codes[:, j * blk:min((j + 1) * blk, n)] = c.reshape(b_, h, -1, dd).transpose(0, 2, 1, 3)
            scales[:, :, j] = s
        return codes, scales

    q_i8, q_scale = per_block(q, q_block)
    k_i8, k_scale = per_block(ks, k_block)
    return {"q_i8": q_i8, "q_scale": q_scale, "k_i8": k_i8, "k_scale": k_scale, "k_mean": mu}
